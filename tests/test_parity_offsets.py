"""Prefill and decode calls whose tensors hold more than 2^31 elements
(dn_chunk_fwd, dn_decode_step, through the C ABI): every offset past that
point must be formed in 64 bits.

Eight seeded base heads (``synthetic.make``, Gated DeltaNet, bf16, d = 128)
are tiled over B x H heads on the GPU, so head i carries base head i % 8. The
heads are independent and the kernels deterministic, so:

  * the head that holds element 2^31 of q, the one after it and the last head
    equal their copies among the first eight heads, bit for bit, in o and in
    the end state (a wrapped 32-bit offset would read or write another head's
    rows, or fault);
  * the last head matches the fp64 oracle's token-by-token recurrence on its
    base head (bound 2e-2, bf16).

Two sizes: T = 4096 (64 chunks: the prep + scan launches) and T = 8192 (128
chunks with more than 16 heads: the one-launch form). About 35 GB of device
memory each (q, k, v, o and the prefill's workspace).

The decode step likewise on a state of 2.15G fp32 elements (8200 sequences x
16 heads of 128 x 128): the heads that hold element 2^31 and the last head
equal their copies, and the last one matches one step of the oracle.

KDA's chunked prefill (dn_kda_chunk_fwd, per-channel decay g [B,H,T,dk]) the
same way at 2 x 1040 heads x 8192 tokens (two launches; the last head also
against the oracle) and 2 x 16 heads x 540672 tokens (the one-launch form,
which KDA takes at 32 heads or fewer).

The gated layer's two one-call forms (dn_layer_prefill, dn_layer_decode_step)
on seeded base sequences (``synthetic.make_layer``) tiled along the batch:
the prefill with 2.42G elements of qkv (48 sequences x 8192 tokens, 16 + 16
heads of 128), the decode step with a state of 2.15G fp32 elements (8200
sequences x 16 heads). The sequences that hold element 2^31 and the last one
equal their copies among the base sequences, bit for bit, in out, the end
state and the new convolution history; the base sequences themselves are the
layer parity tests' cases.
"""
import pytest
import torch

import oracle
import synthetic
from gpu_util import TOL, rel_err, say

pytestmark = pytest.mark.gpu

NB = 8   # base heads


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import delta_rule_recurrent_amd as dn  # noqa: F401  (loads libdeltanet.so)


@pytest.mark.parametrize("T,H", [(4096, 2056), (8192, 1040)])
def test_chunk_offsets_past_2_31(T, H):
    import delta_rule_recurrent_amd as dn
    B, d = 2, 128
    BH = B * H
    assert BH * T * d > 2 ** 31
    say("chunk prefill past 2^31 elements: B=%d H=%d T=%d d=%d (%.2fG elements per tensor)"
        % (B, H, T, d, BH * T * d / 1e9))
    x = synthetic.make("gated", 1, NB, T, d, d, "bf16", seed=4200 + T, decay_scale=0.1)
    idx = torch.arange(BH, device="cuda") % NB

    def tile(t):
        return t[0].cuda()[idx].view(B, H, *t.shape[2:]).contiguous()

    q, k, v, beta, g = (tile(x[n]) for n in ("q", "k", "v", "beta", "g"))
    o, S = dn.chunk_fwd(q, k, v, beta, g)
    torch.cuda.synchronize()
    del q, k, v, beta, g
    o, S = o.view(BH, T, d), S.view(BH, d, d)
    h_wrap = 2 ** 31 // (T * d)
    for h in (h_wrap, h_wrap + 1, BH - 1):
        assert torch.equal(o[h], o[h % NB]), h
        assert torch.equal(S[h], S[h % NB]), h
    last = (BH - 1) % NB
    sl = lambda n: x[n][:, last:last + 1].double().numpy()   # noqa: E731
    o_ref, S_ref = oracle.recurrent(sl("q"), sl("k"), sl("v"), sl("beta"), sl("g"), None, kind=oracle.GATED)
    e = rel_err(o[BH - 1].unsqueeze(0).unsqueeze(0), o_ref)
    eS = rel_err(S[BH - 1].unsqueeze(0).unsqueeze(0), S_ref)
    say("  heads %d, %d, %d equal their copies; last head vs oracle: out %.3g, state %.3g"
        % (h_wrap, h_wrap + 1, BH - 1, e, eS))
    assert e <= TOL["bf16"], e
    assert eS <= TOL["bf16"], eS
    del o, S
    torch.cuda.empty_cache()


def test_decode_offsets_past_2_31():
    import delta_rule_recurrent_amd as dn
    B, H, d = 8200, 16, 128
    BH = B * H
    assert BH * d * d > 2 ** 31
    say("decode step past 2^31 state elements: B=%d H=%d d=%d (%.2fG fp32 elements)"
        % (B, H, d, BH * d * d / 1e9))
    x = synthetic.make("gated", 1, NB, 1, d, d, "bf16", seed=4300, steps=1, s0_std=0.05)
    idx = torch.arange(BH, device="cuda") % NB

    def tile(t):   # [1, 1, NB, ...] per-step inputs, or S0 [1, NB, d, d]
        t = t[0, 0] if t.dim() >= 3 and t.shape[1] == 1 else t[0]
        return t.cuda()[idx].view(B, H, *t.shape[1:]).contiguous()

    q, k, v, beta, g = (tile(x[n]) for n in ("q", "k", "v", "beta", "g"))
    S = tile(x["S0"])
    o = dn.decode_step(q, k, v, beta, g, S)
    torch.cuda.synchronize()
    o, S = o.view(BH, d), S.view(BH, d, d)
    h_wrap = 2 ** 31 // (d * d)
    for h in (h_wrap, h_wrap + 1, BH - 1):
        assert torch.equal(o[h], o[h % NB]), h
        assert torch.equal(S[h], S[h % NB]), h
    last = (BH - 1) % NB
    sl = lambda n: x[n][0][:, last:last + 1].unsqueeze(2).double().numpy()   # noqa: E731  ([1,1,1,...])
    o_ref, S_ref = oracle.recurrent(sl("q"), sl("k"), sl("v"), sl("beta"), sl("g"),
                                    x["S0"][:, last:last + 1].double().numpy(), kind=oracle.GATED)
    e = rel_err(o[BH - 1].view(1, 1, 1, d), o_ref)
    eS = rel_err(S[BH - 1].view(1, 1, d, d), S_ref)
    say("  heads %d, %d, %d equal their copies; last head vs oracle: out %.3g, state %.3g"
        % (h_wrap, h_wrap + 1, BH - 1, e, eS))
    assert e <= TOL["bf16"], e
    assert eS <= TOL["bf16"], eS
    del o, S
    torch.cuda.empty_cache()


def _tile_layer(x, B, nb):
    """The base sequences of ``make_layer`` repeated along the batch on the GPU
    (sequence s carries base sequence s % nb); shared weights moved as they are."""
    idx = torch.arange(B, device="cuda") % nb
    out = {}
    for n, t in x.items():
        if n in ("qkv", "z", "b", "a", "conv_state"):
            out[n] = t.cuda()[idx].contiguous()
        elif isinstance(t, torch.Tensor):
            out[n] = t.cuda()
    return out


def _same_as_copies(seqs, nb, *tensors):
    for s in seqs:
        for t in tensors:
            assert torch.equal(t[s], t[s % nb]), s


def test_layer_prefill_offsets_past_2_31():
    import delta_rule_recurrent_amd as dn
    B, T, H, d, nb = 48, 8192, 16, 128, 4
    C = 3 * H * d
    assert B * T * C > 2 ** 31
    say("layer prefill past 2^31 qkv elements: B=%d T=%d H=%d+%d d=%d (%.2fG elements)"
        % (B, T, H, H, d, B * T * C / 1e9))
    x = _tile_layer(synthetic.make_layer(nb, T, H, H, d, "bf16", seed=4400, conv_state=True), B, nb)
    out, cst, S = dn.layer_prefill(x["qkv"], x["z"], x["b"], x["a"], x["conv_w"], x["A_log"], x["dt_bias"],
                                   x["norm_w"], H, H, conv_state=x["conv_state"])
    torch.cuda.synchronize()
    seqs = (2 ** 31 // (T * C), 2 ** 31 // (T * C) + 1, B - 1)
    _same_as_copies(seqs, nb, out, cst, S)
    say("  sequences %s equal their copies" % (seqs,))
    del x, out, cst, S
    torch.cuda.empty_cache()


def test_layer_decode_offsets_past_2_31():
    import delta_rule_recurrent_amd as dn
    B, H, d, nb = 8200, 16, 128, 8
    assert B * H * d * d > 2 ** 31
    say("layer decode step past 2^31 state elements: B=%d H=%d+%d d=%d" % (B, H, H, d))
    x = _tile_layer(synthetic.make_layer(nb, 1, H, H, d, "bf16", seed=4500, conv_state=True), B, nb)
    gen = torch.Generator().manual_seed(4501)
    S = (torch.randn(nb, H, d, d, generator=gen) * 0.02).cuda()[torch.arange(B, device="cuda") % nb]
    out, cst = dn.layer_decode_step(x["qkv"], x["z"], x["b"], x["a"], x["conv_w"], x["A_log"], x["dt_bias"],
                                    x["norm_w"], H, H, S, conv_state=x["conv_state"])
    torch.cuda.synchronize()
    seqs = (2 ** 31 // (H * d * d), 2 ** 31 // (H * d * d) + 1, B - 1)
    _same_as_copies(seqs, nb, out, cst, S)
    say("  sequences %s equal their copies" % (seqs,))
    del x, out, cst, S
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T,H,nb", [(8192, 1040, 8), (540672, 16, 2)])
def test_kda_offsets_past_2_31(T, H, nb):
    import delta_rule_recurrent_amd as dn
    B, d = 2, 128
    BH = B * H
    assert BH * T * d > 2 ** 31
    say("KDA prefill past 2^31 elements: B=%d H=%d T=%d d=%d (%.2fG elements per tensor)"
        % (B, H, T, d, BH * T * d / 1e9))
    x = synthetic.make("kda", 1, nb, T, d, d, "bf16", seed=4600 + nb, decay_scale=0.1)
    idx = torch.arange(BH, device="cuda") % nb

    def tile(t):
        return t[0].cuda()[idx].view(B, H, *t.shape[2:]).contiguous()

    q, k, v, beta, g = (tile(x[n]) for n in ("q", "k", "v", "beta", "g"))
    o, S = dn.kda_chunk_fwd(q, k, v, beta, g)
    torch.cuda.synchronize()
    del q, k, v, beta, g
    o, S = o.view(BH, T, d), S.view(BH, d, d)
    h_wrap = 2 ** 31 // (T * d)
    heads = sorted({h_wrap, min(h_wrap + 1, BH - 1), BH - 1})
    for h in heads:
        assert torch.equal(o[h], o[h % nb]), h
        assert torch.equal(S[h], S[h % nb]), h
    msg = "  heads %s equal their copies" % heads
    if T <= 8192:
        last = (BH - 1) % nb
        sl = lambda n: x[n][:, last:last + 1].double().numpy()   # noqa: E731
        o_ref, S_ref = oracle.recurrent(sl("q"), sl("k"), sl("v"), sl("beta"), sl("g"), None, kind=oracle.KDA)
        e = rel_err(o[BH - 1].unsqueeze(0).unsqueeze(0), o_ref)
        eS = rel_err(S[BH - 1].unsqueeze(0).unsqueeze(0), S_ref)
        msg += "; last head vs oracle: out %.3g, state %.3g" % (e, eS)
        assert e <= TOL["bf16"], e
        assert eS <= TOL["bf16"], eS
    say(msg)
    del o, S
    torch.cuda.empty_cache()

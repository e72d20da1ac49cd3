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

"""GPU parity of the serving forms at the sizes bench.py times them, in the same
launch configuration, against the fp64 oracle on sampled (sequence, head)
pairs (the heads are independent recurrences, so the oracle runs each sampled
head alone):

  * chunk-boundary states at B=4, H=8, T=2048, d=128, bf16 Gated DeltaNet: the
    state after every 8th chunk of 4 sampled heads (the oracle run up to that
    token), and o, S_final bitwise equal to the plain prefill's;
  * 4 key heads for 8 value heads at the same size: o and S_final of 4 sampled
    value heads against the oracle with the shared key head;
  * 8 packed sequences of 63 .. 3008 tokens, 8 heads: o and the final state of
    every sequence for 2 sampled heads;
  * 4-token decode with snapshots for 256 x 16 states: every output and
    snapshot of 6 sampled states.
Bound 2e-2 (bf16).
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_util import TOL, rel_err, say, to_dev

pytestmark = pytest.mark.gpu
TOLB = TOL["bf16"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _dn():
    import delta_rule_recurrent_amd as dn
    return dn


def _head(inp, b, h, a=0, e=None):
    """Inputs of one (sequence, head) over tokens a .. e as [1,1,...] arrays."""
    return {n: (None if inp[n] is None else inp[n][b:b + 1, h:h + 1, a:e])
            for n in ("q", "k", "v", "beta", "g")}


def test_boundary_states_full_size():
    dn = _dn()
    name = "gdn_prefill_b4_h8_t2048_d128"
    say("boundary states full size")
    inp = synthetic.make_config(name)
    d = to_dev(inp)
    o, S, Sc = dn.chunk_fwd_states(d["q"], d["k"], d["v"], d["beta"], d["g"], None)
    o2, S2 = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], None)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(S, S2) and torch.equal(Sc[:, :, -1], S)
    for b, h in ((0, 0), (1, 5), (2, 3), (3, 7)):
        for c in (0, 7, 15, 23, 31):
            x = _head(inp, b, h, 0, 64 * (c + 1))
            _, Sref = oracle.recurrent(x["q"], x["k"], x["v"], x["beta"], x["g"], None,
                                       kind=oracle.GATED)
            e = rel_err(Sc[b:b + 1, h:h + 1, c], Sref)
            assert e <= TOLB, (b, h, c, e)
    say("  ok")


def test_shared_key_heads_full_size():
    dn = _dn()
    B, Hk, Hv, T, dd = 4, 4, 8, 2048, 128
    say("shared key heads full size")
    x = synthetic.make_config("gdn_prefill_b4_h8_t2048_d128")
    qk = synthetic.make("gated", B, Hk, T, dd, dd, dtype="bf16", seed=2001)
    dx, dq = to_dev(x), to_dev(qk)
    o, S = dn.chunk_fwd_gqa(dq["q"], dq["k"], dx["v"], dx["beta"], dx["g"], None)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (1, 3), (2, 6), (3, 7)):
        kh = h // (Hv // Hk)
        o_ref, S_ref = oracle.recurrent(qk["q"][b:b + 1, kh:kh + 1], qk["k"][b:b + 1, kh:kh + 1],
                                        x["v"][b:b + 1, h:h + 1], x["beta"][b:b + 1, h:h + 1],
                                        x["g"][b:b + 1, h:h + 1], None, kind=oracle.GATED)
        eo, es = rel_err(o[b:b + 1, h:h + 1], o_ref), rel_err(S[b:b + 1, h:h + 1], S_ref)
        assert eo <= TOLB and es <= TOLB, (b, h, eo, es)
    say("  ok")


def test_packed_sequences_full_size():
    dn = _dn()
    lens = [3008, 64, 1536, 520, 1024, 77, 1900, 63]
    H, dd = 8, 128
    Tp = sum(lens)
    say("packed sequences full size")
    xp = synthetic.make("gated", 1, H, Tp, dd, dd, dtype="bf16", seed=2002)
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    dx = to_dev(xp)
    o, S = dn.chunk_fwd_varlen(dx["q"], dx["k"], dx["v"], dx["beta"], dx["g"],
                               torch.tensor(cu, dtype=torch.int32, device="cuda"), None)
    torch.cuda.synchronize()
    for h in (2, 6):
        for n in range(len(lens)):
            x = _head(xp, 0, h, cu[n], cu[n + 1])
            o_ref, S_ref = oracle.recurrent(x["q"], x["k"], x["v"], x["beta"], x["g"], None,
                                            kind=oracle.GATED)
            eo = rel_err(o[0:1, h:h + 1, cu[n]:cu[n + 1]], o_ref)
            es = rel_err(S[n:n + 1, h:h + 1], S_ref)
            assert eo <= TOLB and es <= TOLB, (h, n, eo, es)
    say("  ok")


def test_decode_tokens_full_size():
    dn = _dn()
    B, H, K, dd = 256, 16, 4, 128
    say("decode tokens full size")
    x = synthetic.make("gated", B, H, K, dd, dd, dtype="bf16", seed=2003, s0_std=0.02)
    dx = to_dev(x)
    S = dx["S0"].clone()
    o, snap = dn.decode_tokens(dx["q"], dx["k"], dx["v"], dx["beta"], dx["g"], S)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (17, 4), (100, 9), (128, 15), (200, 1), (255, 12)):
        for j in range(K):
            xx = _head(x, b, h, 0, j + 1)
            o_ref, S_ref = oracle.recurrent(xx["q"], xx["k"], xx["v"], xx["beta"], xx["g"],
                                            x["S0"][b:b + 1, h:h + 1], kind=oracle.GATED)
            assert rel_err(snap[b:b + 1, h:h + 1, j], S_ref) <= TOLB, (b, h, j)
            assert rel_err(o[b:b + 1, h:h + 1, j], o_ref[:, :, j]) <= TOLB, (b, h, j)
    assert torch.equal(snap[:, :, -1], S)
    say("  ok")

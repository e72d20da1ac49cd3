"""GPU parity of the chunked prefill at chunk lengths 32, 64 and 128
(dn_chunk_fwd_len, through the C ABI) against the fp64 oracle's token-by-token
recurrence: the chunk length changes only the rounding (page "28. Linear
attention and Gated DeltaNet", section "Stretch exercises", item 2).

  * DeltaNet and Gated DeltaNet, bf16, d in {64, 128}, T in {1, 31, 100, 300}
    (ragged last chunks at every length), with a start state: o and S_final
    within 2e-2.
  * Decays eight times stronger (sums over a 128-token chunk far below the
    fp32 exponent range): finite and within the bound.
  * Chunk 64 bitwise equal to dn_chunk_fwd's two launches.
  * The sweep's size (16 heads of 4096 tokens, d = 128) at every length, on
    sampled heads against the oracle run on those heads alone.
"""
import pytest
import torch

import oracle
import synthetic
from gpu_util import TOL, oracle_prefill, rel_err, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import delta_rule_recurrent_amd as dn  # noqa: F401  (loads libdeltanet.so)


def _dn():
    import delta_rule_recurrent_amd as dn
    return dn


CASES = [(c, d) for c in (32, 64, 128) for d in (64, 128) if not (c == 128 and d == 64)]


@pytest.mark.parametrize("kind", ["deltanet", "gated"])
@pytest.mark.parametrize("chunk,d", CASES)
@pytest.mark.parametrize("T", [1, 31, 100, 300])
def test_chunk_len_matches_oracle(kind, chunk, d, T):
    dn = _dn()
    say("chunk len", kind, chunk, d, T)
    inp = synthetic.make(kind, 2, 3, T, d, d, dtype="bf16", seed=900 + T + d + chunk, s0_std=0.5)
    x = to_dev(inp)
    o, S = dn.chunk_fwd_len(x["q"], x["k"], x["v"], x["beta"], x["g"], x["S0"], chunk=chunk)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_prefill(inp)
    eo, eS = rel_err(o, o_ref), rel_err(S, S_ref)
    say("  o err %.3g, S err %.3g" % (eo, eS))
    assert eo <= TOL["bf16"] and eS <= TOL["bf16"], (eo, eS)


@pytest.mark.parametrize("chunk", [32, 64, 128])
def test_chunk_len_strong_decay(chunk):
    dn = _dn()
    inp = synthetic.make("gated", 1, 4, 2 * chunk + 9, 128, 128, dtype="bf16", seed=950 + chunk,
                         s0_std=0.5, decay_scale=8.0)
    x = to_dev(inp)
    o, S = dn.chunk_fwd_len(x["q"], x["k"], x["v"], x["beta"], x["g"], x["S0"], chunk=chunk)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    o_ref, S_ref = oracle_prefill(inp)
    assert rel_err(o, o_ref) <= TOL["bf16"] and rel_err(S, S_ref) <= TOL["bf16"]


@pytest.mark.parametrize("d", [64, 128])
def test_chunk_len_64_is_two_phase_chunk_fwd(d):
    """Chunk 64 runs the same kernels as dn_chunk_fwd's two launches."""
    dn = _dn()
    inp = to_dev(synthetic.make("gated", 2, 3, 333, d, d, dtype="bf16", seed=970 + d, s0_std=0.5))
    B, H, T = 2, 3, 333
    ws = torch.empty(dn.workspace_bytes(B, H, T, d, d, torch.bfloat16), dtype=torch.uint8, device="cuda")
    o1 = torch.empty(B, H, T, d, dtype=torch.bfloat16, device="cuda")
    S1 = torch.empty(B, H, d, d, dtype=torch.float32, device="cuda")
    dn.chunk_prep(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], ws)
    dn.chunk_scan(inp["q"], o1, ws, inp["S0"], S1)
    o2, S2 = dn.chunk_fwd_len(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], inp["S0"], chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


# (sequence, head) pairs of the 1 x 16 x 4096 sweep size replayed by the oracle
SWEEP_HEADS = [0, 5, 11, 15]


@pytest.mark.parametrize("chunk", [32, 64, 128])
def test_chunk_len_sweep_size(chunk):
    """The size the chunk lengths are timed at (16 heads x 4096 tokens, d = 128,
    bf16 Gated DeltaNet): four sampled heads against the oracle run on those
    heads alone."""
    dn = _dn()
    say("chunk len sweep size", chunk)
    inp = synthetic.make("gated", 1, 16, 4096, 128, 128, dtype="bf16", seed=2007)
    x = to_dev(inp)
    o, S = dn.chunk_fwd_len(x["q"], x["k"], x["v"], x["beta"], x["g"], None, chunk=chunk)
    torch.cuda.synchronize()
    hi = SWEEP_HEADS
    sub = {n: inp[n][:, hi] for n in ("q", "k", "v", "beta", "g")}
    o_ref, S_ref = oracle.recurrent(sub["q"], sub["k"], sub["v"], sub["beta"], sub["g"], None,
                                    kind=oracle.GATED)
    eo, eS = rel_err(o[:, hi], o_ref), rel_err(S[:, hi], S_ref)
    say("  o err %.3g, S err %.3g" % (eo, eS))
    assert eo <= TOL["bf16"] and eS <= TOL["bf16"], (eo, eS)

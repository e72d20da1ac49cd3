"""GPU generalized delta rule (through the C ABI) versus its fp64 oracle.

S_t = (diag(exp g_t) - (a_t * kr_t) kr_t^T) S_{t-1} + kw_t v_t^T, o_t = S_t^T q_t
(oracle/gdr.py), token by token and as single-token decode steps, on seeded
inputs (``synthetic.make_gdr``) with T in {1, 5, 64, 130}, both head sizes,
both dtypes and a non-zero start state; the tie to DeltaNet against the GPU
DeltaNet recurrence; the in-place state update. Bound: max|gpu - ref| /
max|ref| <= 1e-4 (fp32), 2e-2 (bf16).
"""
import pytest
import torch

import synthetic
from gpu_util import TOL, rel_err, say, to_dev
from oracle import gdr as ogdr

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import delta_rule_recurrent_amd as dn  # noqa: F401  (loads libdeltanet.so)


def _dn():
    import delta_rule_recurrent_amd as dn
    return dn


NAMES = ("q", "kw", "v", "kr", "a", "g")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T", [1, 5, 64, 130])
def test_gdr_matches_oracle(dtype, d, T):
    dn = _dn()
    say("gdr", dtype, d, T)
    x = synthetic.make_gdr(2, 3, T, d, dtype, seed=700 + T + d, s0_std=0.5)
    dx = to_dev(x)
    o, S = dn.gdr_recurrent_fwd(*(dx[n] for n in NAMES), dx["S0"])
    torch.cuda.synchronize()
    o_ref, S_ref = ogdr.recurrent(*(x[n] for n in NAMES), x["S0"])
    eo, eS = rel_err(o, o_ref), rel_err(S, S_ref)
    say("  o err %.3g, S err %.3g" % (eo, eS))
    assert eo <= TOL[dtype] and eS <= TOL[dtype], (eo, eS)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_gdr_decode_steps_in_place(dtype, d):
    """Four single-token steps on one state buffer, against the oracle over
    the four tokens."""
    dn = _dn()
    say("gdr decode", dtype, d)
    x = synthetic.make_gdr(3, 2, 4, d, dtype, seed=760 + d, s0_std=0.5)
    dx = to_dev(x)
    S = dx["S0"].clone()
    outs = [dn.gdr_decode_step(*(dx[n][:, :, t].contiguous() for n in NAMES), S) for t in range(4)]
    torch.cuda.synchronize()
    o_ref, S_ref = ogdr.recurrent(*(x[n] for n in NAMES), x["S0"])
    assert rel_err(torch.stack(outs, dim=2), o_ref) <= TOL[dtype]
    assert rel_err(S, S_ref) <= TOL[dtype]


def test_gdr_tied_equals_deltanet_on_gpu():
    """kr = k, kw = beta k, a = beta, g = 0 is DeltaNet: the two GPU paths agree
    to fp32 rounding (fp32 inputs)."""
    dn = _dn()
    inp = synthetic.make("deltanet", 2, 2, 90, 64, 64, dtype="f32", seed=81, s0_std=0.5)
    d = to_dev(inp)
    k, beta = d["k"], d["beta"]
    o1, S1 = dn.gdr_recurrent_fwd(d["q"], (beta[..., None] * k).contiguous(), d["v"], k,
                                  (beta[..., None] * torch.ones_like(k)).contiguous(),
                                  torch.zeros_like(k), d["S0"])
    o2, S2 = dn.recurrent_fwd(d["q"], k, d["v"], beta, None, d["S0"])
    torch.cuda.synchronize()
    assert rel_err(o1, o2.double().cpu().numpy()) <= 1e-5
    assert rel_err(S1, S2.double().cpu().numpy()) <= 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gdr_decode_strong_decay(dtype):
    """Decays that underflow to zero in some channels (g = -200): those rows of
    the state drop out, nothing becomes NaN."""
    dn = _dn()
    x = synthetic.make_gdr(4, 2, 1, 128, dtype, seed=91, s0_std=0.5)
    x["g"][..., ::3] = -200.0
    dx = to_dev(x)
    S = dx["S0"].clone()
    o = dn.gdr_decode_step(*(dx[n][:, :, 0].contiguous() for n in NAMES), S)
    torch.cuda.synchronize()
    o_ref, S_ref = ogdr.recurrent(*(x[n] for n in NAMES), x["S0"])
    assert rel_err(o, o_ref[:, :, 0]) <= TOL[dtype]
    assert rel_err(S, S_ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T", [1, 37, 64, 65, 200])
def test_gdr_chunk_matches_oracle(dtype, d, T):
    """The chunked form (64-token chunks as affine maps, ragged last chunk)
    against the oracle's recurrence; fp32 inputs within 1e-4, bf16 within 2e-2."""
    dn = _dn()
    say("gdr chunk", dtype, d, T)
    x = synthetic.make_gdr(2, 3, T, d, dtype, seed=800 + T + d, s0_std=0.5)
    dx = to_dev(x)
    o, S = dn.gdr_chunk_fwd(*(dx[n] for n in NAMES), dx["S0"])
    torch.cuda.synchronize()
    o_ref, S_ref = ogdr.recurrent(*(x[n] for n in NAMES), x["S0"])
    eo, eS = rel_err(o, o_ref), rel_err(S, S_ref)
    say("  o err %.3g, S err %.3g" % (eo, eS))
    assert eo <= TOL[dtype] and eS <= TOL[dtype], (eo, eS)


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_gdr_chunk_strong_decay_and_in_place(chunk):
    """Decays of -30 per token in a third of the channels (sums far below the
    fp32 exponent range inside a chunk, and across its 16-token sub-blocks)
    stay finite; S_final == S0 in place."""
    dn = _dn()
    say("gdr chunk strong decay", chunk)
    x = synthetic.make_gdr(1, 2, 150, 64, "f32", seed=812, s0_std=0.5)
    x["g"][..., ::3] = -30.0
    dx = to_dev(x)
    S = dx["S0"].clone()
    o, S2 = dn.gdr_chunk_fwd(*(dx[n] for n in NAMES), S, S_final=S, chunk=chunk)
    torch.cuda.synchronize()
    assert S2 is S
    o_ref, S_ref = ogdr.recurrent(*(x[n] for n in NAMES), x["S0"])
    assert rel_err(o, o_ref) <= TOL["f32"]
    assert rel_err(S, S_ref) <= TOL["f32"]


def test_gdr_chunk_long_sequence():
    """70 chunks and a ragged tail (4489 tokens) at d = 128, bf16, with a start
    state: the chunk maps chained 70 times stay within the bound of the
    oracle's recurrence."""
    dn = _dn()
    say("gdr chunk long")
    x = synthetic.make_gdr(1, 2, 64 * 70 + 9, 128, "bf16", seed=820, s0_std=0.5)
    dx = to_dev(x)
    o, S = dn.gdr_chunk_fwd(*(dx[n] for n in NAMES), dx["S0"])
    torch.cuda.synchronize()
    o_ref, S_ref = ogdr.recurrent(*(x[n] for n in NAMES), x["S0"])
    eo, eS = rel_err(o, o_ref), rel_err(S, S_ref)
    say("  o err %.3g, S err %.3g" % (eo, eS))
    assert eo <= TOL["bf16"] and eS <= TOL["bf16"], (eo, eS)


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_gdr_chunk_many_heads(chunk):
    """40 (sequence, head) rows (a multiple of 8: the scan groups a head's
    column tiles on one XCD) of a ragged 150 tokens: the grid and workspace
    indexing over many heads, every head against the oracle's recurrence
    (fp32, 1e-4)."""
    dn = _dn()
    say("gdr chunk many heads", chunk)
    x = synthetic.make_gdr(5, 8, 150, 64, "f32", seed=830, s0_std=0.5)
    dx = to_dev(x)
    o, S = dn.gdr_chunk_fwd(*(dx[n] for n in NAMES), dx["S0"], chunk=chunk)
    torch.cuda.synchronize()
    o_ref, S_ref = ogdr.recurrent(*(x[n] for n in NAMES), x["S0"])
    eo, eS = rel_err(o, o_ref), rel_err(S, S_ref)
    say("  o err %.3g, S err %.3g" % (eo, eS))
    assert eo <= TOL["f32"] and eS <= TOL["f32"], (eo, eS)


# (sequence, head) pairs of the 4 x 8 timed size replayed by the oracle: both
# ends of the grid and heads on different XCD groups (h mod 8)
TIMED_SAMPLE = [(0, 0), (0, 7), (1, 3), (2, 5), (3, 1), (3, 6)]


def test_gdr_chunk_timed_size():
    """The size the chunked form is timed at (4 x 8 x 2048 tokens, d = 128,
    bf16 inputs; 32 heads: the scan's XCD grouping), six sampled heads
    against the oracle's recurrence run on those heads alone: read-outs and
    final states within the bf16 bound."""
    dn = _dn()
    say("gdr chunk timed size")
    x = synthetic.make_gdr(4, 8, 2048, 128, "bf16", seed=2005)
    dx = to_dev(x)
    o, S = dn.gdr_chunk_fwd(*(dx[n] for n in NAMES), None)
    torch.cuda.synchronize()
    bi = [b for b, _ in TIMED_SAMPLE]
    hi = [h for _, h in TIMED_SAMPLE]
    sub = {n: x[n][bi, hi][None] for n in NAMES}      # [1, 6, T, d]
    o_ref, S_ref = ogdr.recurrent(*(sub[n] for n in NAMES), None)
    eo = rel_err(o[bi, hi][None], o_ref)
    eS = rel_err(S[bi, hi][None], S_ref)
    say("  o err %.3g, S err %.3g" % (eo, eS))
    assert eo <= TOL["bf16"] and eS <= TOL["bf16"], (eo, eS)


@pytest.mark.parametrize("chunk", [16, 32])
@pytest.mark.parametrize("dtype,d,T", [("f32", 64, 37), ("bf16", 128, 130), ("f32", 128, 100)])
def test_gdr_chunk_lengths(chunk, dtype, d, T):
    """Chunks of 16 and 32 tokens (ragged last chunk) against the oracle's
    recurrence; the chunk length changes only the rounding."""
    dn = _dn()
    say("gdr chunk length", chunk, dtype, d, T)
    x = synthetic.make_gdr(2, 2, T, d, dtype, seed=840 + chunk + T, s0_std=0.5)
    dx = to_dev(x)
    o, S = dn.gdr_chunk_fwd(*(dx[n] for n in NAMES), dx["S0"], chunk=chunk)
    torch.cuda.synchronize()
    o_ref, S_ref = ogdr.recurrent(*(x[n] for n in NAMES), x["S0"])
    assert rel_err(o, o_ref) <= TOL[dtype] and rel_err(S, S_ref) <= TOL[dtype]

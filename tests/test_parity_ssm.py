"""GPU selective state-space recurrence (through the C ABI) versus its fp64 oracle.

S_t = exp(g_t) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t (oracle/ssm.py): the
chunked form (the chunk machinery with the UT solve reduced to the identity),
the token-by-token form and the single-token decode step, on seeded inputs
spanning several 64-token chunks and ragged tails, both head sizes, both
dtypes, a non-zero start state, no decay (plain causal linear attention) and
a strong decay. Bound: max|gpu - ref| / max|ref| <= 1e-4 (fp32), 2e-2 (bf16).
"""
import numpy as np
import pytest
import torch

from gpu_util import TOL, make, rel_err, say, to_dev
from oracle import ssm as ossm

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import delta_rule_recurrent_amd as dn  # noqa: F401  (loads libdeltanet.so)


def _dn():
    import delta_rule_recurrent_amd as dn
    return dn


def _inputs(T, d, dtype, seed, decay=1.0):
    # the gated draw supplies q, k, v, g and S0; beta is not used by this kind
    return make("gated", 2, 3, T, d, dtype, seed=seed, s0_std=0.5, decay_scale=decay)


@pytest.mark.parametrize("form", ["chunk", "recurrent"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T", [1, 37, 64, 65, 200])
def test_ssm_matches_oracle(form, dtype, d, T):
    dn = _dn()
    say("ssm", form, dtype, d, T)
    x = _inputs(T, d, dtype, seed=300 + T + d)
    dx = to_dev(x)
    fn = dn.ssm_chunk_fwd if form == "chunk" else dn.ssm_recurrent_fwd
    o, S = fn(dx["q"], dx["k"], dx["v"], dx["g"], dx["S0"])
    torch.cuda.synchronize()
    o_ref, S_ref = ossm.recurrent(x["q"], x["k"], x["v"], x["g"], x["S0"])
    eo, eS = rel_err(o, o_ref), rel_err(S, S_ref)
    say("  o err %.3g, S err %.3g" % (eo, eS))
    assert eo <= TOL[dtype] and eS <= TOL[dtype], (eo, eS)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ssm_no_decay_and_strong_decay(dtype):
    """g = 0: plain causal linear attention (the state only grows); g scaled
    by 8: only the last few tokens matter. Chunked form against the oracle."""
    dn = _dn()
    for name, scale in (("no decay", 0.0), ("strong decay", 8.0)):
        say("ssm", dtype, name)
        x = _inputs(150, 64, dtype, seed=17, decay=scale)
        dx = to_dev(x)
        o, S = dn.ssm_chunk_fwd(dx["q"], dx["k"], dx["v"], dx["g"], dx["S0"])
        torch.cuda.synchronize()
        o_ref, S_ref = ossm.recurrent(x["q"], x["k"], x["v"], x["g"], x["S0"])
        assert rel_err(o, o_ref) <= TOL[dtype]
        assert rel_err(S, S_ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_ssm_decode_steps(dtype, d):
    """Five decode steps from a start state, each against the oracle run over
    the tokens so far."""
    dn = _dn()
    say("ssm decode", dtype, d)
    x = _inputs(5, d, dtype, seed=90 + d)
    dx = to_dev(x)
    S = dx["S0"].clone()
    outs = []
    for t in range(5):
        outs.append(dn.ssm_decode_step(dx["q"][:, :, t].contiguous(), dx["k"][:, :, t].contiguous(),
                                       dx["v"][:, :, t].contiguous(), dx["g"][:, :, t].contiguous(),
                                       S))
    torch.cuda.synchronize()
    o_ref, S_ref = ossm.recurrent(x["q"], x["k"], x["v"], x["g"], x["S0"])
    o = torch.stack(outs, dim=2)
    assert rel_err(o, o_ref) <= TOL[dtype]
    assert rel_err(S, S_ref) <= TOL[dtype]


def test_ssm_chunk_long_bf16():
    """A long bf16 sequence (70 chunks, ragged tail) through the chunked form."""
    dn = _dn()
    say("ssm long")
    x = make("gated", 1, 2, 64 * 70 + 9, 128, "bf16", seed=5, s0_std=0.5)
    dx = to_dev(x)
    o, S = dn.ssm_chunk_fwd(dx["q"], dx["k"], dx["v"], dx["g"], dx["S0"])
    torch.cuda.synchronize()
    o_ref, S_ref = ossm.recurrent(x["q"], x["k"], x["v"], x["g"], x["S0"])
    assert rel_err(o, o_ref) <= TOL["bf16"]
    assert rel_err(S, S_ref) <= TOL["bf16"]

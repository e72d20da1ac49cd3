"""dn_chunk_fwd_noalloc (the library's built-in scratch; nothing allocated)
against dn_chunk_fwd with a caller workspace, through the C ABI: two calls in
a row on the same scratch, the second smaller than the first. The first has
67 chunks per sequence, so dn_chunk_fwd takes the one-launch form; the second
runs the two phases. Outputs and final states must be bitwise equal to the
workspace form (same kernels, same order), and within the bf16 bound of the
fp64 oracle.
"""
import pytest
import torch

from gpu_util import TOL, make, oracle_prefill, rel_err, say, to_dev

pytestmark = pytest.mark.gpu

CASES = [("gated", 2, 4, 66 * 64 + 7, 701),   # larger first: one-launch form
         ("deltanet", 1, 3, 300, 702)]        # smaller second: two phases


def test_noalloc_matches_workspace_form():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import delta_rule_recurrent_amd as dn

    for kind, B, H, T, seed in CASES:
        say("noalloc", kind, B, H, T)
        inp = make(kind, B, H, T, 128, "bf16", seed=seed, s0_std=0.5)
        x = to_dev(inp)
        o1, S1 = dn.chunk_fwd_noalloc(x["q"], x["k"], x["v"], x["beta"], x["g"], x["S0"])
        o2, S2 = dn.chunk_fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["S0"])
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(S1, S2)
        o_ref, S_ref = oracle_prefill(inp)
        eo, es = rel_err(o1, o_ref), rel_err(S1, S_ref)
        say("  err o %.3e  S %.3e" % (eo, es))
        assert eo <= TOL["bf16"] and es <= TOL["bf16"]

"""GPU parity of the layer kernels and the selective state-space form at the
sizes bench.py measures them, in the same launch configuration, against the
fp64 oracles:

  * layer prologue and epilogue at B=4, T=2048, 8 key + 8 value heads of 128,
    bf16, with carried conv state (the bench's prefill layer): every output;
  * the single-token prologue and the epilogue at 256 sequences x 16 + 16
    heads (the bench's decode layer): every output;
  * the state-space chunked form on the Gated DeltaNet prefill inputs (B=4,
    H=8, T=2048, d=128, bf16): outputs and final states of 6 sampled
    (sequence, head) pairs against the oracle run on those heads alone (the
    heads are independent).
Bound 2e-2 (bf16) as everywhere; the new conv state is compared bit for bit.
"""
import numpy as np
import pytest
import torch

import synthetic
from gpu_util import TOL, rel_err, say, to_dev
from oracle import layer as ol
from oracle import ssm as ossm

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("B,T,Hk,Hv", [(4, 2048, 8, 8), (256, 1, 16, 16)])
def test_layer_full_size(B, T, Hk, Hv):
    import delta_rule_recurrent_amd as dn

    d = 128
    say("layer full size", B, T, Hk, Hv)
    x = synthetic.make_layer(B, T, Hk, Hv, d, "bf16", seed=3001)
    dx = to_dev(x)
    cst = dx["conv_state"].clone()
    q, k, v, beta, g, _ = dn.layer_prologue(dx["qkv"], dx["conv_w"], dx["b"], dx["a"], dx["A_log"],
                                            dx["dt_bias"], Hk, Hv, conv_state=dx["conv_state"],
                                            conv_state_out=cst)
    gen = torch.Generator().manual_seed(3002)
    o = (torch.randn(B, Hv, T, d, generator=gen) * 0.3).to(torch.bfloat16)
    y = dn.layer_epilogue(o.cuda(), dx["z"], dx["norm_w"], 1e-6)
    torch.cuda.synchronize()
    say("  oracle")
    rq, rk, rv, rbeta, rg, rst = ol.prologue(x["qkv"], x["conv_w"], x["conv_state"], x["b"], x["a"],
                                             x["A_log"], x["dt_bias"], Hk, Hv, d, d)
    for name, gpu, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv), ("beta", beta, rbeta),
                           ("g", g, rg)):
        e = rel_err(gpu, ref)
        say("  %s err %.3g" % (name, e))
        assert e <= TOL["bf16"], (name, e)
    assert np.array_equal(cst.float().cpu().double().numpy(), rst)
    ref = ol.rmsnorm_gated(o, x["z"], x["norm_w"], 1e-6)
    e = rel_err(y, ref)
    say("  epilogue err %.3g" % e)
    assert e <= TOL["bf16"], e


def test_ssm_chunk_full_size():
    import delta_rule_recurrent_amd as dn

    name = "gdn_prefill_b4_h8_t2048_d128"
    c = synthetic.CONFIGS[name]
    B, H, T, dk = c["B"], c["H"], c["T"], c["dk"]
    say("ssm full size", name)
    inp = synthetic.make_config(name)
    dd = to_dev(inp)
    o = torch.empty(B, H, T, dk, dtype=torch.bfloat16, device="cuda")
    S = torch.empty(B, H, dk, dk, dtype=torch.float32, device="cuda")
    ws = torch.empty(dn.workspace_bytes(B, H, T, dk, dk, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    dn.ssm_chunk_fwd(dd["q"], dd["k"], dd["v"], dd["g"], None, o=o, S_final=S, workspace=ws)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (0, 5), (1, 3), (2, 7), (3, 1), (3, 6)):
        sl = lambda t: t[b:b + 1, h:h + 1]   # noqa: E731
        o_ref, S_ref = ossm.recurrent(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["g"]), None)
        eo, es = rel_err(o[b:b + 1, h:h + 1], o_ref), rel_err(S[b:b + 1, h:h + 1], S_ref)
        say("  head (%d,%d): err o %.3g S %.3g" % (b, h, eo, es))
        assert eo <= TOL["bf16"] and es <= TOL["bf16"], (b, h, eo, es)

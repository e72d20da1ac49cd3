"""GPU (HIP, through the C ABI) versus the fp64 oracle on small seeded inputs.

Sizes span several 64-token chunks and ragged tails (T = 1, 16, 37, 64, 65,
200), both head sizes, both dtypes, non-zero start states, and stress inputs:
weak decay (long carries through the state) and beta in (0, 2) (the
reflection range, which the kernels must not clamp). Bound per output tensor:
max|gpu - ref| / max|ref| <= 1e-4 for fp32 inputs and <= 2e-2 for bf16.
"""
import numpy as np
import pytest
import torch

from gpu_util import TOL, make, oracle_prefill, rel_err, say, to_dev

pytestmark = pytest.mark.gpu

KINDS = ["deltanet", "gated", "kda"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import delta_rule_recurrent_amd as dn  # noqa: F401  (loads libdeltanet.so)


def _dn():
    import delta_rule_recurrent_amd as dn
    return dn


def _prefill(form, kind, inp):
    dn = _dn()
    d = to_dev(inp)
    args = (d["q"], d["k"], d["v"], d["beta"], d["g"], d["S0"])
    if form == "chunk":
        fn = dn.kda_chunk_fwd if kind == "kda" else dn.chunk_fwd
    else:
        fn = dn.kda_recurrent_fwd if kind == "kda" else dn.recurrent_fwd
    o, S = fn(*args)
    torch.cuda.synchronize()
    return o, S


@pytest.mark.parametrize("form", ["chunk", "recurrent"])
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T", [1, 16, 37, 64, 65, 200])
def test_prefill_matches_oracle(form, kind, dtype, d, T):
    say("case", form, kind, dtype, d, T)
    inp = make(kind, 2, 3, T, d, dtype, seed=T * 7 + d, s0_std=0.5)
    o, S = _prefill(form, kind, inp)
    o_ref, S_ref = oracle_prefill(inp)
    eo, es = rel_err(o, o_ref), rel_err(S, S_ref)
    say("  err o %.3e  S %.3e" % (eo, es))
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("variant", ["weak_decay", "reflection_beta", "zero_state"])
def test_prefill_stress(kind, dtype, variant):
    d, T = (128, 300) if dtype == "bf16" else (64, 300)
    kw = {}
    s0 = 0.5
    if variant == "weak_decay":
        kw["decay_scale"] = 0.01
    elif variant == "reflection_beta":
        kw["beta_scale"] = 2.0
    else:
        s0 = None
    inp = make(kind, 1, 4, T, d, dtype, seed=99, s0_std=s0, **kw)
    o_ref, S_ref = oracle_prefill(inp)
    for form in ("chunk", "recurrent"):
        say("case", form, kind, dtype, variant)
        o, S = _prefill(form, kind, inp)
        eo, es = rel_err(o, o_ref), rel_err(S, S_ref)
        say("  err o %.3e  S %.3e" % (eo, es))
        assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("f32", 64), ("bf16", 128)])
@pytest.mark.parametrize("T", [37, 300])
def test_kda_strong_decay(dtype, d, T):
    """KDA with per-channel log-decay g = -16 softplus(N(0,1)) (the scale the
    full layer's gate -exp(A_log) softplus(a + dt_bias) reaches with A_log up
    to log 16): the decay summed over a few tokens is far below the fp32
    exponent range, so every decay factor of the chunked form must stay a
    decay (no overflow, no inf * 0). Chunked and recurrent forms against the
    oracle, with a start state."""
    inp = make("kda", 1, 3, T, d, dtype, seed=500 + T + d, s0_std=0.5, decay_scale=16.0)
    g = inp["g"].float()
    assert float(g.min()) < -40.0          # several tokens' worth exceeds exp's range
    o_ref, S_ref = oracle_prefill(inp)
    for form in ("chunk", "recurrent"):
        say("case kda strong decay", form, dtype, d, T)
        o, S = _prefill(form, "kda", inp)
        eo, es = rel_err(o, o_ref), rel_err(S, S_ref)
        say("  err o %.3e  S %.3e" % (eo, es))
        assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_matches_oracle(kind, dtype, d):
    import oracle
    dn = _dn()
    say("case decode", kind, dtype, d)
    steps = 5
    inp = make(kind, 3, 5, 1, d, dtype, seed=d + 3, s0_std=0.3, steps=steps)
    dev = to_dev(inp)
    S = dev["S0"].clone()
    outs = []
    fn = dn.kda_decode_step if kind == "kda" else dn.decode_step
    for s in range(steps):
        g = None if dev["g"] is None else dev["g"][s]
        outs.append(fn(dev["q"][s], dev["k"][s], dev["v"][s], dev["beta"][s], g, S))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.decode_steps(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"],
                                       inp["S0"], kind={"deltanet": 0, "gated": 1, "kda": 2}[kind])
    eo = rel_err(torch.stack(outs), o_ref)
    es = rel_err(S, S_ref)
    say("  err o %.3e  S %.3e" % (eo, es))
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_empty_sequence_copies_state():
    dn = _dn()
    for kind in KINDS:
        inp = to_dev(make(kind, 2, 2, 0, 64, "bf16", seed=1, s0_std=1.0))
        fn = dn.kda_chunk_fwd if kind == "kda" else dn.chunk_fwd
        o, S = fn(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], inp["S0"])
        torch.cuda.synchronize()
        assert o.numel() == 0 and torch.equal(S, inp["S0"])
        o, S = fn(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], None)
        torch.cuda.synchronize()
        assert torch.count_nonzero(S).item() == 0


def test_in_place_state_and_determinism():
    dn = _dn()
    inp = to_dev(make("gated", 2, 4, 150, 128, "bf16", seed=5, s0_std=0.5))
    o1, S1 = dn.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], inp["S0"])
    o2, S2 = dn.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], inp["S0"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)   # no atomics: bitwise reproducible
    S = inp["S0"].clone()
    o3, S3 = dn.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], S, S_final=S)
    torch.cuda.synchronize()
    assert S3.data_ptr() == S.data_ptr()
    assert torch.equal(o3, o1) and torch.equal(S, S1)


@pytest.mark.parametrize("kind", KINDS)
def test_state_handoff(kind):
    """prefill(T1) then prefill(T2, S0 = S) equals prefill(T1 + T2)."""
    dn = _dn()
    T1, T2 = 100, 77
    inp = make(kind, 1, 3, T1 + T2, 128, "bf16", seed=11, s0_std=0.5)
    d = to_dev(inp)
    fn = dn.kda_chunk_fwd if kind == "kda" else dn.chunk_fwd
    sl = lambda x, a, b: None if x is None else x[:, :, a:b].contiguous()
    o1, S1 = fn(sl(d["q"], 0, T1), sl(d["k"], 0, T1), sl(d["v"], 0, T1), sl(d["beta"], 0, T1),
                sl(d["g"], 0, T1), d["S0"])
    o2, S2 = fn(sl(d["q"], T1, None), sl(d["k"], T1, None), sl(d["v"], T1, None),
                sl(d["beta"], T1, None), sl(d["g"], T1, None), S1)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_prefill(inp)
    assert rel_err(torch.cat([o1, o2], dim=2), o_ref) <= TOL["bf16"]
    assert rel_err(S2, S_ref) <= TOL["bf16"]


@pytest.mark.parametrize("kind", KINDS)
def test_decode_equals_one_token_prefill(kind):
    dn = _dn()
    inp = to_dev(make(kind, 4, 4, 1, 128, "f32", seed=21, s0_std=0.5))
    fn = dn.kda_chunk_fwd if kind == "kda" else dn.chunk_fwd
    o_p, S_p = fn(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], inp["S0"])
    S = inp["S0"].clone()
    dec = dn.kda_decode_step if kind == "kda" else dn.decode_step
    g = None if inp["g"] is None else inp["g"][:, :, 0].contiguous()
    o_d = dec(inp["q"][:, :, 0].contiguous(), inp["k"][:, :, 0].contiguous(),
              inp["v"][:, :, 0].contiguous(), inp["beta"][:, :, 0].contiguous(), g, S)
    torch.cuda.synchronize()
    assert torch.allclose(o_d, o_p[:, :, 0], rtol=1e-5, atol=1e-5)
    assert torch.allclose(S, S_p, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T", [32 * 64 + 37, 48 * 64, 64 * 64 + 5])
def test_long_prefill(kind, dtype, T):
    """Sequences of 32 chunks and more, with a ragged last chunk: same results as
    the oracle with a start state, bitwise the same with the state updated in
    place, and bitwise equal to calling the two phases one after the other
    (kda_chunk_fwd runs bf16 inputs of 64 chunks and more as one launch)."""
    dn = _dn()
    say("long prefill", kind, dtype, T)
    inp = make(kind, 1, 2, T, 128, dtype, seed=23, s0_std=0.5)
    d = to_dev(inp)
    fn = dn.kda_chunk_fwd if kind == "kda" else dn.chunk_fwd
    o, S = fn(d["q"], d["k"], d["v"], d["beta"], d["g"], d["S0"])
    Sip = d["S0"].clone()
    o2, _ = fn(d["q"], d["k"], d["v"], d["beta"], d["g"], Sip, S_final=Sip)
    # the two phases called one after the other
    ws = torch.empty(dn.workspace_bytes(1, 2, T, 128, 128, d["q"].dtype), dtype=torch.uint8,
                     device="cuda")
    o3 = torch.empty_like(o)
    S3 = torch.empty_like(S)
    dn.chunk_prep(d["q"], d["k"], d["v"], d["beta"], d["g"], ws, kda=kind == "kda")
    dn.chunk_scan(d["q"], o3, ws, d["S0"], S3, kda=kind == "kda")
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_prefill(inp)
    tol = TOL[dtype]
    eo, es = rel_err(o, o_ref), rel_err(S, S_ref)
    say("  err o %.3e  S %.3e" % (eo, es))
    assert eo <= tol and es <= tol
    assert torch.equal(o2, o) and torch.equal(Sip, S)
    assert torch.equal(o3, o) and torch.equal(S3, S)


@pytest.mark.parametrize("kind", ["deltanet", "gated"])
@pytest.mark.parametrize("BH", [(1, 2), (3, 5), (4, 8)])
def test_fused_handoff(kind, BH):
    """The one-launch prefill (prep and scan workgroups handing chunk blocks
    over through tags in the workspace) on short sequences: bitwise equal to
    the two phases, and
    the tags show every block published by both of its wavefronts, from the
    XCD its consumers run on (workgroup b on XCD b % 8, head h served by XCD
    h % 8), with a new epoch per launch and the error word untouched."""
    dn = _dn()
    B, H = BH
    T = 5 * 64 + 9
    nch = (T + 63) // 64
    say("fused hand-off", kind, B, H, T)
    inp = make(kind, B, H, T, 128, "bf16", seed=29, s0_std=0.5)
    d = to_dev(inp)
    dt = d["q"].dtype
    nbytes = dn.workspace_bytes(B, H, T, 128, 128, dt)
    block = dn.workspace_bytes(1, 1, 128, 128, 128, dt) - dn.workspace_bytes(1, 1, 64, 128, 128, dt)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    o, S = dn.chunk_fwd_fused(d["q"], d["k"], d["v"], d["beta"], d["g"], d["S0"], workspace=ws)
    torch.cuda.synchronize()
    tail = ws[B * H * nch * block:].cpu()
    tags1 = tail[:B * H * nch * 16].view(torch.int64).view(B * H, nch, 2).clone()
    err, last = (int(x) for x in tail[B * H * nch * 16:B * H * nch * 16 + 16].view(torch.int64))
    assert err == 0 and last != 0
    assert dn.chunk_fwd_handoff_status(ws, B, H, T, 128, 128, dt) == 0
    assert torch.equal(tags1[:, :, 0], tags1[:, :, 1])
    t = tags1[:, :, 0].numpy().astype(np.uint64)
    low = t & np.uint64((1 << 56) - 1)
    assert (low == low[0, 0]).all() and low[0, 0] != 0
    # the XCD number sits XORed into bits 56..59 of the tag (over the epoch's
    # own bits there), so tags of heads h and 0 differ there by h % 8
    xcc = ((t >> np.uint64(56)) & np.uint64(15)) ^ ((t[0, 0] >> np.uint64(56)) & np.uint64(15))
    for h in range(B * H):
        assert (xcc[h] == np.uint64(h % 8)).all(), (h, xcc[h])
    # the latest-epoch word is the epoch the tags carry (below the XCD bits)
    assert np.uint64(last & ((1 << 56) - 1)) == low[0, 0]

    ws2 = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    o3, S3 = torch.empty_like(o), torch.empty_like(S)
    dn.chunk_prep(d["q"], d["k"], d["v"], d["beta"], d["g"], ws2)
    dn.chunk_scan(d["q"], o3, ws2, d["S0"], S3)
    o4, S4 = dn.chunk_fwd_fused(d["q"], d["k"], d["v"], d["beta"], d["g"], d["S0"], workspace=ws)
    torch.cuda.synchronize()
    tags2 = ws[B * H * nch * block:].cpu()[:B * H * nch * 16].view(torch.int64).view(B * H, nch, 2)
    assert not (tags2 == tags1).any()
    assert torch.equal(o3, o) and torch.equal(S3, S)
    assert torch.equal(o4, o) and torch.equal(S4, S)
    o_ref, S_ref = oracle_prefill(inp)
    eo, es = rel_err(o, o_ref), rel_err(S, S_ref)
    say("  err o %.3e  S %.3e" % (eo, es))
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("in_place", [False, True])
def test_fused_handoff_failure_recomputed(in_place, monkeypatch):
    """The one-launch form with its hand-off waits cut to zero polls (set from
    the host through DN_HANDOFF_SPIN_LIMIT; every kernel still ends normally):
    waits give up on blocks not yet published, the launch marks itself
    failed, and the two phases enqueued behind it recompute the call. The
    status query reports DN_EHANDOFF, and o and S_final are bitwise the
    two-phase prefill's, also when S_final is S0 (updated in place). A
    following call with the default limit reports DN_OK."""
    dn = _dn()
    B, H, T = 1, 4, 80 * 64 + 11
    nch = (T + 63) // 64
    say("fused hand-off failure", in_place, B, H, T)
    inp = make("gated", B, H, T, 128, "bf16", seed=31, s0_std=0.5)
    d = to_dev(inp)
    dt = d["q"].dtype
    ws = torch.empty(dn.workspace_bytes(B, H, T, 128, 128, dt), dtype=torch.uint8, device="cuda")
    # the reference: the two phases on their own workspace
    ws2 = torch.empty_like(ws)
    o2, S2 = torch.empty(B, H, T, 128, dtype=dt, device="cuda"), torch.empty_like(d["S0"])
    dn.chunk_prep(d["q"], d["k"], d["v"], d["beta"], d["g"], ws2)
    dn.chunk_scan(d["q"], o2, ws2, d["S0"], S2)
    monkeypatch.setenv("DN_HANDOFF_SPIN_LIMIT", "0")
    if in_place:
        S = d["S0"].clone()
        o, S1 = dn.chunk_fwd_fused(d["q"], d["k"], d["v"], d["beta"], d["g"], S, S_final=S,
                                   workspace=ws)
        assert S1 is S
    else:
        o, S1 = dn.chunk_fwd_fused(d["q"], d["k"], d["v"], d["beta"], d["g"], d["S0"], workspace=ws)
    st = dn.chunk_fwd_handoff_status(ws, B, H, T, 128, 128, dt)
    assert st == _lib_status("DN_EHANDOFF"), st
    assert torch.equal(o, o2) and torch.equal(S1, S2)
    monkeypatch.delenv("DN_HANDOFF_SPIN_LIMIT")
    o3, S3 = dn.chunk_fwd_fused(d["q"], d["k"], d["v"], d["beta"], d["g"], d["S0"], workspace=ws)
    assert dn.chunk_fwd_handoff_status(ws, B, H, T, 128, 128, dt) == 0
    assert torch.equal(o3, o2) and torch.equal(S3, S2)
    assert nch >= 64


@pytest.mark.parametrize("BH", [(1, 2), (3, 5)])
def test_kda_fused_handoff(BH):
    """KDA's one-launch prefill (kda_chunk_fwd from 64 chunks on; four-wavefront prep
    workgroups publish each block once all four wavefronts' stores are done):
    bitwise equal to the two phases, every block's two tags carry the launch
    epoch and the XCD of the head (h % 8), the error word is untouched, and the
    results match the oracle."""
    dn = _dn()
    B, H = BH
    T = 64 * 64 + 9
    nch = (T + 63) // 64
    say("kda fused hand-off", B, H, T)
    inp = make("kda", B, H, T, 128, "bf16", seed=37, s0_std=0.5)
    d = to_dev(inp)
    dt = d["q"].dtype
    nbytes = dn.workspace_bytes(B, H, T, 128, 128, dt)
    block = dn.workspace_bytes(1, 1, 128, 128, 128, dt) - dn.workspace_bytes(1, 1, 64, 128, 128, dt)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    o, S = dn.kda_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["S0"], workspace=ws)
    torch.cuda.synchronize()
    tail = ws[B * H * nch * block:].cpu()
    tags = tail[:B * H * nch * 16].view(torch.int64).view(B * H, nch, 2).clone()
    err, last = (int(x) for x in tail[B * H * nch * 16:B * H * nch * 16 + 16].view(torch.int64))
    assert err == 0 and last != 0
    assert dn.chunk_fwd_handoff_status(ws, B, H, T, 128, 128, dt) == 0
    assert torch.equal(tags[:, :, 0], tags[:, :, 1])
    t = tags[:, :, 0].numpy().astype(np.uint64)
    low = t & np.uint64((1 << 56) - 1)
    assert (low == low[0, 0]).all() and low[0, 0] != 0
    assert np.uint64(last & ((1 << 56) - 1)) == low[0, 0]
    xcc = ((t >> np.uint64(56)) & np.uint64(15)) ^ ((t[0, 0] >> np.uint64(56)) & np.uint64(15))
    for h in range(B * H):
        assert (xcc[h] == np.uint64(h % 8)).all(), (h, xcc[h])
    ws2 = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    o2, S2 = torch.empty_like(o), torch.empty_like(S)
    dn.chunk_prep(d["q"], d["k"], d["v"], d["beta"], d["g"], ws2, kda=True)
    dn.chunk_scan(d["q"], o2, ws2, d["S0"], S2, kda=True)
    torch.cuda.synchronize()
    assert torch.equal(o2, o) and torch.equal(S2, S)
    o_ref, S_ref = oracle_prefill(inp)
    eo, es = rel_err(o, o_ref), rel_err(S, S_ref)
    say("  err o %.3e  S %.3e" % (eo, es))
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("in_place", [False, True])
def test_kda_fused_handoff_failure_recomputed(in_place, monkeypatch):
    """KDA's one-launch form with its hand-off waits cut to zero polls (from
    the host; every kernel still ends normally): the launch marks itself
    failed, the guarded two phases behind it recompute the call (bitwise the
    two-phase results, also with the state updated in place), the status
    query reports DN_EHANDOFF, and the next call with the default limit DN_OK."""
    dn = _dn()
    B, H, T = 1, 4, 66 * 64 + 21
    say("kda fused hand-off failure", in_place, B, H, T)
    inp = make("kda", B, H, T, 128, "bf16", seed=41, s0_std=0.5)
    d = to_dev(inp)
    dt = d["q"].dtype
    ws = torch.empty(dn.workspace_bytes(B, H, T, 128, 128, dt), dtype=torch.uint8, device="cuda")
    ws2 = torch.empty_like(ws)
    o2, S2 = torch.empty(B, H, T, 128, dtype=dt, device="cuda"), torch.empty_like(d["S0"])
    dn.chunk_prep(d["q"], d["k"], d["v"], d["beta"], d["g"], ws2, kda=True)
    dn.chunk_scan(d["q"], o2, ws2, d["S0"], S2, kda=True)
    monkeypatch.setenv("DN_HANDOFF_SPIN_LIMIT", "0")
    if in_place:
        S = d["S0"].clone()
        o, S1 = dn.kda_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], S, S_final=S, workspace=ws)
        assert S1 is S
    else:
        o, S1 = dn.kda_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["S0"], workspace=ws)
    st = dn.chunk_fwd_handoff_status(ws, B, H, T, 128, 128, dt)
    assert st == _lib_status("DN_EHANDOFF"), st
    assert torch.equal(o, o2) and torch.equal(S1, S2)
    monkeypatch.delenv("DN_HANDOFF_SPIN_LIMIT")
    o3, S3 = dn.kda_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["S0"], workspace=ws)
    assert dn.chunk_fwd_handoff_status(ws, B, H, T, 128, 128, dt) == 0
    assert torch.equal(o3, o2) and torch.equal(S3, S2)


def _lib_status(name):
    from delta_rule_recurrent_amd import _lib
    return getattr(_lib, name)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_boundary_states(kind, dtype, d):
    """dn_chunk_fwd_states: the state after every chunk against the oracle run
    chunk by chunk (each segment started from the oracle's state at the end of
    the one before), on a ragged last chunk; o and S_final bitwise equal to the
    plain prefill's, and the last boundary state equal to S_final."""
    dn = _dn()
    B, H, T = 2, 3, 5 * 64 + 9
    n = (T + 63) // 64
    say("boundary states", kind, dtype, d, T)
    inp = make(kind, B, H, T, d, dtype, seed=41, s0_std=0.5)
    dv = to_dev(inp)
    args = (dv["q"], dv["k"], dv["v"], dv["beta"], dv["g"], dv["S0"])
    o, S, Sc = dn.chunk_fwd_states(*args, kda=(kind == "kda"))
    ref_fn = dn.kda_chunk_fwd if kind == "kda" else dn.chunk_fwd
    o2, S2 = ref_fn(*args)
    torch.cuda.synchronize()
    assert Sc.shape == (B, H, n, d, d)
    assert torch.equal(o, o2) and torch.equal(S, S2)
    assert torch.equal(Sc[:, :, -1], S)
    state = inp["S0"]
    worst = 0.0
    for c in range(n):
        a, b = 64 * c, min(64 * (c + 1), T)
        seg = {key: (inp[key][:, :, a:b] if inp[key] is not None else None)
               for key in ("q", "k", "v", "beta", "g")}
        seg["kind"] = inp["kind"]
        _, state = oracle_prefill(seg, S0=state)
        e = rel_err(Sc[:, :, c], state)
        worst = max(worst, e)
        assert e <= TOL[dtype], (c, e)
    say("  worst boundary-state err %.3e" % worst)


def _gqa_inputs(kind, B, Hk, Hv, T, d, dtype, seed):
    """q, k drawn for Hk key heads; v, beta, g and S0 for Hv value heads."""
    kv = make(kind, B, Hk, T, d, dtype, seed=seed)
    vv = make(kind, B, Hv, T, d, dtype, seed=seed + 1, s0_std=0.5)
    inp = dict(vv)
    inp["q"], inp["k"] = kv["q"], kv["k"]
    rep = dict(inp)
    rep["q"] = inp["q"].repeat_interleave(Hv // Hk, dim=1).contiguous()
    rep["k"] = inp["k"].repeat_interleave(Hv // Hk, dim=1).contiguous()
    return inp, rep


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dtype,d,T,Hk,Hv", [("bf16", 128, 200, 2, 6), ("f32", 64, 137, 1, 3),
                                             ("bf16", 128, 128 * 64 + 5, 4, 16)])
def test_gqa_prefill(kind, dtype, d, T, Hk, Hv):
    """Key heads shared by value heads: bitwise equal to the plain prefill on
    q, k repeated over heads (the pages' repeat_interleave), and within the
    bound of the oracle run on that repetition. 16 value heads of 129 chunks
    take the one-launch form (every kind has it at bf16)."""
    dn = _dn()
    say("gqa prefill", kind, dtype, d, T, Hk, Hv)
    inp, rep = _gqa_inputs(kind, 1 if T > 1000 else 2, Hk, Hv, T, d, dtype, seed=51)
    di, dr = to_dev(inp), to_dev(rep)
    o, S = dn.chunk_fwd_gqa(di["q"], di["k"], di["v"], di["beta"], di["g"], di["S0"],
                            kda=(kind == "kda"))
    fn = dn.kda_chunk_fwd if kind == "kda" else dn.chunk_fwd
    o2, S2 = fn(dr["q"], dr["k"], dr["v"], dr["beta"], dr["g"], dr["S0"])
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(S, S2)
    o_ref, S_ref = oracle_prefill(rep)
    eo, es = rel_err(o, o_ref), rel_err(S, S_ref)
    say("  err o %.3e  S %.3e" % (eo, es))
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("kind", KINDS)
def test_gqa_decode(kind):
    """One decode step with shared key heads equals the plain step on the
    repetition, bitwise, and the oracle within the bound."""
    dn = _dn()
    B, Hk, Hv, d = 3, 2, 8, 128
    inp, rep = _gqa_inputs(kind, B, Hk, Hv, 1, d, "bf16", seed=61)
    di, dr = to_dev(inp), to_dev(rep)
    one = lambda x: None if x is None else x[:, :, 0].contiguous()   # noqa: E731
    S1, S2 = di["S0"].clone(), di["S0"].clone()
    o1 = dn.decode_step_gqa(one(di["q"]), one(di["k"]), one(di["v"]), one(di["beta"]), one(di["g"]),
                            S1, kda=(kind == "kda"))
    fn = dn.kda_decode_step if kind == "kda" else dn.decode_step
    o2 = fn(one(dr["q"]), one(dr["k"]), one(dr["v"]), one(dr["beta"]), one(dr["g"]), S2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    o_ref, S_ref = oracle_prefill(rep)
    eo, es = rel_err(o1, o_ref[:, :, 0]), rel_err(S1, S_ref)
    say("gqa decode", kind, "err o %.3e  S %.3e" % (eo, es))
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_varlen_prefill(kind, dtype, d):
    """Packed sequences of different lengths (one empty, ragged tails, one
    shorter than a chunk) in one call: each sequence bitwise equal to the plain
    prefill of that sequence alone, and within the bound of the oracle; the
    empty one passes its start state through."""
    dn = _dn()
    lens = [1, 64, 65, 200, 0, 37, 130]
    N, H, T = len(lens), 3, sum(lens)
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    say("varlen", kind, dtype, d, lens)
    inp = make(kind, 1, H, T, d, dtype, seed=71)
    S0 = make(kind, N, H, 1, d, dtype, seed=72, s0_std=0.5)["S0"]
    di = to_dev(inp)
    S0d = S0.cuda()
    cud = torch.tensor(cu, dtype=torch.int32, device="cuda")
    o, S = dn.chunk_fwd_varlen(di["q"], di["k"], di["v"], di["beta"], di["g"], cud, S0d,
                               kda=(kind == "kda"))
    torch.cuda.synchronize()
    fn = dn.kda_chunk_fwd if kind == "kda" else dn.chunk_fwd
    worst = 0.0
    for n in range(N):
        a, b = cu[n], cu[n + 1]
        if a == b:
            assert torch.equal(S[n], S0d[n])
            continue
        sl = lambda x: None if x is None else x[:, :, a:b].contiguous()   # noqa: E731
        seg = {key: sl(inp[key]) for key in ("q", "k", "v", "beta", "g")}
        seg["kind"] = inp["kind"]
        sd = to_dev(seg)
        o1, S1 = fn(sd["q"], sd["k"], sd["v"], sd["beta"], sd["g"], S0d[n:n + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(o[:, :, a:b], o1), n
        assert torch.equal(S[n:n + 1], S1), n
        o_ref, S_ref = oracle_prefill(seg, S0=S0[n:n + 1])
        eo, es = rel_err(o[:, :, a:b], o_ref), rel_err(S[n:n + 1], S_ref)
        worst = max(worst, eo, es)
        assert eo <= TOL[dtype] and es <= TOL[dtype], (n, eo, es)
    say("  worst err %.3e" % worst)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_decode_tokens_snapshots(kind, dtype, d):
    """K tokens per sequence in one call: the snapshot after token j against the
    oracle run over the first j + 1 tokens; o and the updated state bitwise
    equal to the token-by-token prefill from the same start state."""
    dn = _dn()
    B, H, K = 3, 4, 5
    say("decode tokens", kind, dtype, d, K)
    inp = make(kind, B, H, K, d, dtype, seed=81, s0_std=0.5)
    di = to_dev(inp)
    S = di["S0"].clone()
    o, snap = dn.decode_tokens(di["q"], di["k"], di["v"], di["beta"], di["g"], S,
                               kda=(kind == "kda"))
    fn = dn.kda_recurrent_fwd if kind == "kda" else dn.recurrent_fwd
    o2, S2 = fn(di["q"], di["k"], di["v"], di["beta"], di["g"], di["S0"])
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(S, S2)
    assert torch.equal(snap[:, :, -1], S)
    for j in range(K):
        seg = {key: (inp[key][:, :, :j + 1] if inp[key] is not None else None)
               for key in ("q", "k", "v", "beta", "g")}
        seg["kind"] = inp["kind"]
        _, S_ref = oracle_prefill(seg, S0=inp["S0"])
        e = rel_err(snap[:, :, j], S_ref)
        assert e <= TOL[dtype], (j, e)
    o_ref, _ = oracle_prefill(inp)
    assert rel_err(o, o_ref) <= TOL[dtype]

"""The C-ABI library loads, exports every declared symbol, and validates its
arguments synchronously before any HIP call (so these run without a GPU).

No test here passes a complete set of valid arguments: that would enqueue
work. Fake device pointers are plain aligned integers and are never touched.
"""
import ctypes
import os
import re

import pytest

from delta_rule_recurrent_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "deltanet.h")

P = 0x10000          # aligned fake device pointer
MIS = 0x10008        # 8-byte aligned only
ODD = 0x10001        # not even element-aligned
WS = 0x100000        # 256-aligned fake workspace


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dn_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = _lib.lib()
    names = declared_functions()
    assert len(names) == 34, names
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(_lib.SIGNATURES)


def test_version_and_strerror():
    lib = _lib.lib()
    assert lib.dn_version() >= 3   # workspace holds the start-state copy since 3
    for code in (0, -1, -2, -3, -4, -5, -6, 7):
        s = lib.dn_strerror(code)
        assert isinstance(s, bytes) and len(s) > 0


def test_workspace_size_function():
    lib = _lib.lib()
    ws = lib.dn_chunk_fwd_workspace
    assert ws(1, 1, 0, 64, 64, 0) == 0
    assert ws(1, 1, 64, 64, 64, 0) > 0
    # one block per (head, chunk), then two 64-bit hand-off tags per block, an
    # error word and the latest epoch (padded to 256 bytes), then a copy of
    # the fp32 start state per head
    state = 128 * 128 * 4
    block = ws(1, 1, 128, 128, 128, 1) - ws(1, 1, 64, 128, 128, 1)
    assert block > 0 and block % 256 == 0
    assert ws(1, 1, 64, 128, 128, 1) == block + 256 + state
    a = ws(4, 8, 2048, 128, 128, 1)
    assert a == 32 * 32 * block + (32 * 32 * 16 + 16 + 255) // 256 * 256 + 32 * state
    assert ws(1, 1, 65, 128, 128, 1) == ws(1, 1, 128, 128, 128, 1)
    assert ws(1, 1, 64, 96, 96, 1) == 0     # unsupported head size
    assert ws(0, 1, 64, 64, 64, 1) == 0
    assert ws(1, 1, 64, 64, 64, 5) == 0     # unknown dtype


def _chunk(fn, **kw):
    args = dict(q=P, k=P, v=P, beta=P, g=P, S0=P, o=P, S_final=P, B=1, H=1, T=64, dk=64, dv=64,
                dtype=1, ws=WS, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return getattr(_lib.lib(), fn)(args["q"], args["k"], args["v"], args["beta"], args["g"],
                                    args["S0"], args["o"], args["S_final"], args["B"], args["H"],
                                    args["T"], args["dk"], args["dv"], args["dtype"], args["ws"],
                                    args["ws_bytes"], args["stream"])


@pytest.mark.parametrize("fn", ["dn_chunk_fwd", "dn_chunk_fwd_fused", "dn_kda_chunk_fwd"])
def test_chunk_validation(fn):
    E, N, W = _lib.DN_EINVAL, _lib.DN_ENOTSUP, _lib.DN_EWORKSPACE
    for name in ("q", "k", "v", "beta", "o"):
        assert _chunk(fn, **{name: None}) == E, name
    assert _chunk(fn, B=0) == E
    assert _chunk(fn, H=-1) == E
    assert _chunk(fn, T=-5) == E
    assert _chunk(fn, dtype=2) == E
    assert _chunk(fn, q=MIS) == E
    assert _chunk(fn, S_final=MIS) == E
    assert _chunk(fn, g=ODD) == E
    assert _chunk(fn, dk=96, dv=96) == N
    assert _chunk(fn, dk=64, dv=128) == N
    assert _chunk(fn, dk=256, dv=256) == N
    assert _chunk(fn, ws=None) == W
    assert _chunk(fn, ws_bytes=16) == W
    assert _chunk(fn, ws=WS + 16) == W
    assert _chunk(fn, B=1 << 20, H=1 << 10) == E   # heads beyond the grid limit
    if fn == "dn_kda_chunk_fwd":
        assert _chunk(fn, g=None) == E               # KDA needs its per-channel decay
    if fn == "dn_chunk_fwd_fused":
        assert _chunk(fn, dtype=0) == N              # the one-launch form is bf16 only
        assert _chunk(fn, dtype=0, q=None) == E      # argument errors still come first


def _states(**kw):
    args = dict(kda=0, q=P, k=P, v=P, beta=P, g=P, S0=P, o=P, S_final=P, S_chunks=P, B=1, H=1,
                T=64, dk=64, dv=64, dtype=1, ws=WS, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return _lib.lib().dn_chunk_fwd_states(*[args[n] for n in (
        "kda", "q", "k", "v", "beta", "g", "S0", "o", "S_final", "S_chunks", "B", "H", "T", "dk",
        "dv", "dtype", "ws", "ws_bytes", "stream")])


def test_boundary_states_validation():
    E, N, W = _lib.DN_EINVAL, _lib.DN_ENOTSUP, _lib.DN_EWORKSPACE
    assert _states(S_chunks=None) == E           # required whenever there is a chunk
    assert _states(S_chunks=MIS) == E
    assert _states(q=None) == E
    assert _states(B=0) == E
    assert _states(kda=1, g=None) == E           # KDA needs its per-channel decay
    assert _states(dk=96, dv=96) == N
    assert _states(ws=None) == W
    assert _states(ws_bytes=16) == W
    # T == 0 with no S_final: nothing to do, no launch
    assert _states(T=0, S_chunks=None, S_final=None) == _lib.DN_OK


def _gqa(**kw):
    args = dict(kda=0, q=P, k=P, v=P, beta=P, g=P, S0=P, o=P, S_final=P, B=1, Hk=2, Hv=6, T=64,
                dk=64, dv=64, dtype=1, ws=WS, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return _lib.lib().dn_chunk_fwd_gqa(*[args[n] for n in (
        "kda", "q", "k", "v", "beta", "g", "S0", "o", "S_final", "B", "Hk", "Hv", "T", "dk", "dv",
        "dtype", "ws", "ws_bytes", "stream")])


def _gqa_dec(**kw):
    args = dict(kda=0, q=P, k=P, v=P, beta=P, g=P, S=P, o=P, B=1, Hk=2, Hv=6, dk=128, dv=128,
                dtype=1, stream=None)
    args.update(kw)
    return _lib.lib().dn_decode_step_gqa(*[args[n] for n in (
        "kda", "q", "k", "v", "beta", "g", "S", "o", "B", "Hk", "Hv", "dk", "dv", "dtype",
        "stream")])


def test_shared_key_heads_validation():
    E, N, W = _lib.DN_EINVAL, _lib.DN_ENOTSUP, _lib.DN_EWORKSPACE
    for fn in (_gqa, _gqa_dec):
        assert fn(Hk=0) == E
        assert fn(Hv=0) == E
        assert fn(Hk=4, Hv=6) == E                 # value heads not a multiple of key heads
        assert fn(Hk=3, Hv=2) == E
        assert fn(q=None) == E
        assert fn(B=0) == E
        assert fn(kda=1, g=None) == E
        assert fn(dk=96, dv=96) == N
    assert _gqa(ws=None) == W
    assert _gqa(ws_bytes=16) == W
    assert _gqa_dec(S=None) == E


def _varlen(**kw):
    args = dict(kda=0, q=P, k=P, v=P, beta=P, g=P, S0=P, o=P, S_final=P, cu=P, N=3, H=2, T=300,
                dk=64, dv=64, dtype=1, ws=WS, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return _lib.lib().dn_chunk_fwd_varlen(*[args[n] for n in (
        "kda", "q", "k", "v", "beta", "g", "S0", "o", "S_final", "cu", "N", "H", "T", "dk", "dv",
        "dtype", "ws", "ws_bytes", "stream")])


def test_varlen_workspace_and_validation():
    lib = _lib.lib()
    ws = lib.dn_chunk_fwd_varlen_workspace
    block = lib.dn_chunk_fwd_workspace(1, 1, 128, 128, 128, 1) - lib.dn_chunk_fwd_workspace(1, 1, 64, 128, 128, 1)
    # blocks for H x (ceil(T/64) + N) chunks, then N+1 chunk offsets and a
    # table of 8 bytes per chunk, each padded to 256 bytes
    assert ws(2, 1, 64, 128, 128, 1) == 3 * block + 256 + 256
    assert ws(5, 4, 1000, 128, 128, 1) == 4 * 21 * block + 256 + 256
    assert ws(0, 1, 64, 128, 128, 1) == 0 and ws(1, 1, 0, 128, 128, 1) == 0
    E, N, W = _lib.DN_EINVAL, _lib.DN_ENOTSUP, _lib.DN_EWORKSPACE
    assert _varlen(N=0) == E
    assert _varlen(cu=None) == E
    assert _varlen(cu=P + 2) == E              # int array: 4-byte alignment
    assert _varlen(q=None) == E
    assert _varlen(kda=1, g=None) == E
    assert _varlen(dk=96, dv=96) == N
    assert _varlen(ws=None) == W
    assert _varlen(ws_bytes=16) == W
    assert _varlen(N=1 << 23, H=4) == E         # more than 2^24 (sequence, head) rows
    assert _varlen(T=0, S_final=None) == _lib.DN_OK


def _tokens(**kw):
    args = dict(kda=0, q=P, k=P, v=P, beta=P, g=P, S=P, o=P, S_snap=P, B=1, H=1, K=4, dk=128,
                dv=128, dtype=1, stream=None)
    args.update(kw)
    return _lib.lib().dn_decode_tokens(*[args[n] for n in (
        "kda", "q", "k", "v", "beta", "g", "S", "o", "S_snap", "B", "H", "K", "dk", "dv", "dtype",
        "stream")])


def test_decode_tokens_validation():
    E, N = _lib.DN_EINVAL, _lib.DN_ENOTSUP
    assert _tokens(S=None) == E
    assert _tokens(K=0) == E
    assert _tokens(S_snap=MIS) == E
    assert _tokens(q=None) == E
    assert _tokens(kda=1, g=None) == E
    assert _tokens(dk=96, dv=96) == N
    assert _tokens(B=0) == E


def _rec(fn, **kw):
    args = dict(q=P, k=P, v=P, beta=P, g=P, S0=P, o=P, S_final=P, B=1, H=1, T=64, dk=64, dv=64,
                dtype=1, stream=None)
    args.update(kw)
    return getattr(_lib.lib(), fn)(*[args[n] for n in ("q", "k", "v", "beta", "g", "S0", "o",
                                                        "S_final", "B", "H", "T", "dk", "dv",
                                                        "dtype", "stream")])


@pytest.mark.parametrize("fn", ["dn_recurrent_fwd", "dn_kda_recurrent_fwd"])
def test_recurrent_validation(fn):
    E, N = _lib.DN_EINVAL, _lib.DN_ENOTSUP
    assert _rec(fn, q=None) == E
    assert _rec(fn, o=None) == E
    assert _rec(fn, B=0) == E
    assert _rec(fn, dk=32, dv=32) == N
    assert _rec(fn, beta=ODD) == E
    assert _rec(fn, v=MIS) == E
    if fn == "dn_kda_recurrent_fwd":
        assert _rec(fn, g=None) == E


def _dec(fn, **kw):
    args = dict(q=P, k=P, v=P, beta=P, g=P, S=P, o=P, B=1, H=1, dk=128, dv=128, dtype=1,
                stream=None)
    args.update(kw)
    return getattr(_lib.lib(), fn)(*[args[n] for n in ("q", "k", "v", "beta", "g", "S", "o", "B",
                                                        "H", "dk", "dv", "dtype", "stream")])


@pytest.mark.parametrize("fn", ["dn_decode_step", "dn_kda_decode_step"])
def test_decode_validation(fn):
    E, N = _lib.DN_EINVAL, _lib.DN_ENOTSUP
    assert _dec(fn, S=None) == E
    assert _dec(fn, o=None) == E
    assert _dec(fn, k=None) == E
    assert _dec(fn, S=MIS) == E
    assert _dec(fn, B=0) == E
    assert _dec(fn, dk=64, dv=128) == N
    assert _dec(fn, dtype=-1) == E
    if fn == "dn_kda_decode_step":
        assert _dec(fn, g=None) == E


def test_python_binding_rejects_cpu_tensors():
    import torch
    import delta_rule_recurrent_amd as dn

    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        dn.chunk_fwd(q, q, q, torch.zeros(1, 1, 4, dtype=torch.bfloat16))


def _prep(**kw):
    a = dict(kda=0, q=P, k=P, v=P, beta=P, g=P, B=1, H=1, T=64, dk=64, dv=64, dtype=1, ws=WS,
             wsb=1 << 30, stream=None)
    a.update(kw)
    return _lib.lib().dn_chunk_prep(*[a[n] for n in ("kda", "q", "k", "v", "beta", "g", "B", "H",
                                                     "T", "dk", "dv", "dtype", "ws", "wsb",
                                                     "stream")])


def _scan(**kw):
    a = dict(kda=0, q=P, S0=P, o=P, S_final=P, B=1, H=1, T=64, dk=64, dv=64, dtype=1, ws=WS,
             wsb=1 << 30, stream=None)
    a.update(kw)
    return _lib.lib().dn_chunk_scan(*[a[n] for n in ("kda", "q", "S0", "o", "S_final", "B", "H",
                                                     "T", "dk", "dv", "dtype", "ws", "wsb",
                                                     "stream")])


def test_phase_validation():
    E, W = _lib.DN_EINVAL, _lib.DN_EWORKSPACE
    assert _prep(q=None) == E
    assert _prep(kda=1, g=None) == E
    assert _prep(ws=None) == W
    assert _prep(wsb=8) == W
    assert _scan(o=None) == E
    assert _scan(q=None) == E
    assert _scan(q=ODD) == E
    assert _scan(S0=MIS) == E
    assert _scan(ws=None) == W
    assert _scan(dk=96, dv=96) == _lib.DN_ENOTSUP


def _prologue(**kw):
    args = dict(qkv=P, conv_w=P, conv_state=P, conv_state_out=P, b=P, a=P, A_log=P, dt_bias=P,
                q=P, k=P, v=P, beta=P, g=P, neg=0, B=1, T=64, Hk=1, Hv=2, dk=64, dv=64, dtype=1,
                stream=None)
    args.update(kw)
    return _lib.lib().dn_layer_prologue(*[args[n] for n in (
        "qkv", "conv_w", "conv_state", "conv_state_out", "b", "a", "A_log", "dt_bias", "q", "k",
        "v", "beta", "g", "neg", "B", "T", "Hk", "Hv", "dk", "dv", "dtype", "stream")])


def test_layer_prologue_validation():
    E, N = _lib.DN_EINVAL, _lib.DN_ENOTSUP
    assert _prologue(Hv=3, Hk=2) == E          # value heads not a multiple of key heads
    assert _prologue(Hk=0) == E
    assert _prologue(B=0) == E
    assert _prologue(B=70000) == E
    assert _prologue(T=-1) == E
    assert _prologue(dtype=5) == E
    assert _prologue(conv_w=None) == E
    assert _prologue(qkv=None) == E
    assert _prologue(beta=None) == E
    assert _prologue(a=None) == E              # a decay gate needs a, A_log, dt_bias
    assert _prologue(A_log=None) == E
    assert _prologue(dt_bias=None) == E
    assert _prologue(qkv=MIS) == E
    assert _prologue(conv_w=MIS) == E
    assert _prologue(conv_state_out=MIS) == E
    assert _prologue(q=MIS) == E
    assert _prologue(b=ODD) == E
    assert _prologue(A_log=P + 2) == E
    assert _prologue(dk=96, dv=96) == N
    assert _prologue(dk=64, dv=128) == N


def _epilogue(**kw):
    args = dict(o=P, z=P, norm_w=P, out=P, B=1, Hv=2, T=64, dv=64, eps=1e-6, dtype=1, stream=None)
    args.update(kw)
    return _lib.lib().dn_layer_epilogue(*[args[n] for n in (
        "o", "z", "norm_w", "out", "B", "Hv", "T", "dv", "eps", "dtype", "stream")])


def test_layer_epilogue_validation():
    E, N = _lib.DN_EINVAL, _lib.DN_ENOTSUP
    assert _epilogue(o=None) == E
    assert _epilogue(z=None) == E
    assert _epilogue(norm_w=None) == E
    assert _epilogue(out=MIS) == E
    assert _epilogue(B=0) == E
    assert _epilogue(T=-1) == E
    assert _epilogue(eps=-1.0) == E
    assert _epilogue(eps=float("nan")) == E
    assert _epilogue(eps=float("inf")) == E
    assert _epilogue(dtype=7) == E
    assert _epilogue(dv=96) == N


def _layer_decode(**kw):
    args = dict(qkv=P, conv_w=P, conv_state=P, conv_state_out=P + 0x100000, b=P, a=P, A_log=P,
                dt_bias=P, z=P, norm_w=P, eps=1e-6, S=P, out=P, neg=0, B=2, Hk=1, Hv=2, d=128,
                dtype=1, stream=None)
    args.update(kw)
    return _lib.lib().dn_layer_decode_step(*[args[n] for n in (
        "qkv", "conv_w", "conv_state", "conv_state_out", "b", "a", "A_log", "dt_bias", "z", "norm_w",
        "eps", "S", "out", "neg", "B", "Hk", "Hv", "d", "dtype", "stream")])


def test_layer_decode_validation():
    E, N = _lib.DN_EINVAL, _lib.DN_ENOTSUP
    assert _layer_decode(Hv=3, Hk=2) == E      # value heads not a multiple of key heads
    assert _layer_decode(B=0) == E
    assert _layer_decode(Hk=0) == E
    assert _layer_decode(dtype=4) == E
    assert _layer_decode(eps=-1.0) == E
    assert _layer_decode(eps=float("nan")) == E
    for name in ("qkv", "conv_w", "b", "z", "norm_w", "S", "out"):
        assert _layer_decode(**{name: None}) == E, name
    assert _layer_decode(A_log=None) == E      # a decay gate needs A_log and dt_bias
    assert _layer_decode(dt_bias=None) == E
    for name in ("qkv", "conv_w", "conv_state", "conv_state_out", "z", "norm_w", "S", "out"):
        assert _layer_decode(**{name: MIS}) == E, name
    assert _layer_decode(b=ODD) == E
    assert _layer_decode(A_log=P + 2) == E
    assert _layer_decode(d=96) == N
    # the history in place only with one value head per key head; no partial overlap
    assert _layer_decode(conv_state_out=P) == E
    assert _layer_decode(conv_state_out=P + 16) == E
    assert _layer_decode(Hk=2, Hv=2, conv_state_out=P + 16) == E


def _layer_prefill(**kw):
    args = dict(qkv=P, conv_w=P, conv_state=P, conv_state_out=P + 0x100000, b=P, a=P, A_log=P,
                dt_bias=P, z=P, norm_w=P, eps=1e-6, S0=P, S_final=P, out=P, neg=0, B=2, T=100, Hk=1,
                Hv=2, d=128, dtype=1, ws=WS, wsb=1 << 30, stream=None)
    args.update(kw)
    return _lib.lib().dn_layer_prefill(*[args[n] for n in (
        "qkv", "conv_w", "conv_state", "conv_state_out", "b", "a", "A_log", "dt_bias", "z", "norm_w",
        "eps", "S0", "S_final", "out", "neg", "B", "T", "Hk", "Hv", "d", "dtype", "ws", "wsb",
        "stream")])


def test_layer_prefill_validation():
    E, N, W = _lib.DN_EINVAL, _lib.DN_ENOTSUP, _lib.DN_EWORKSPACE
    lib = _lib.lib()
    need = lib.dn_layer_prefill_workspace(2, 100, 1, 2, 128, 1)
    assert need > 0 and need % 256 == 0
    assert lib.dn_layer_prefill_workspace(2, 100, 1, 2, 64, 1) == 0      # bf16, d = 128 only
    assert lib.dn_layer_prefill_workspace(2, 100, 1, 2, 128, 0) == 0
    assert _layer_prefill(Hv=3, Hk=2) == E
    assert _layer_prefill(B=0) == E
    assert _layer_prefill(T=-1) == E
    assert _layer_prefill(dtype=4) == E
    assert _layer_prefill(eps=float("nan")) == E
    for name in ("qkv", "conv_w", "b", "z", "norm_w", "S_final", "out"):
        assert _layer_prefill(**{name: None}) == E, name
    assert _layer_prefill(A_log=None) == E
    for name in ("qkv", "conv_w", "conv_state", "conv_state_out", "z", "norm_w", "out", "S0",
                 "S_final"):
        assert _layer_prefill(**{name: MIS}) == E, name
    assert _layer_prefill(b=ODD) == E
    assert _layer_prefill(d=64) == N
    assert _layer_prefill(dtype=0) == N
    assert _layer_prefill(conv_state_out=P) == E          # no in-place history
    assert _layer_prefill(conv_state_out=P + 16) == E
    assert _layer_prefill(ws=None) == W
    assert _layer_prefill(ws=WS + 16) == W
    assert _layer_prefill(wsb=need - 1) == W


def _ssm(fn, **kw):
    args = dict(q=P, k=P, v=P, g=P, S0=P, o=P, S_final=P, S=P, B=1, H=1, T=64, dk=64, dv=64,
                dtype=1, ws=WS, wsb=1 << 30, stream=None)
    args.update(kw)
    names = {"dn_ssm_chunk_fwd": ("q", "k", "v", "g", "S0", "o", "S_final", "B", "H", "T", "dk",
                                  "dv", "dtype", "ws", "wsb", "stream"),
             "dn_ssm_recurrent_fwd": ("q", "k", "v", "g", "S0", "o", "S_final", "B", "H", "T",
                                      "dk", "dv", "dtype", "stream"),
             "dn_ssm_decode_step": ("q", "k", "v", "g", "S", "o", "B", "H", "dk", "dv", "dtype",
                                    "stream")}[fn]
    return getattr(_lib.lib(), fn)(*[args[n] for n in names])


@pytest.mark.parametrize("fn", ["dn_ssm_chunk_fwd", "dn_ssm_recurrent_fwd", "dn_ssm_decode_step"])
def test_ssm_validation(fn):
    E, N = _lib.DN_EINVAL, _lib.DN_ENOTSUP
    assert _ssm(fn, g=None) == E          # the decay is required
    assert _ssm(fn, q=None) == E
    assert _ssm(fn, o=None) == E
    assert _ssm(fn, B=0) == E
    assert _ssm(fn, v=MIS) == E
    assert _ssm(fn, g=ODD) == E
    assert _ssm(fn, dk=96, dv=96) == N
    assert _ssm(fn, dtype=3) == E
    if fn == "dn_ssm_chunk_fwd":
        assert _ssm(fn, ws=None) == _lib.DN_EWORKSPACE
        assert _ssm(fn, wsb=16) == _lib.DN_EWORKSPACE
    if fn == "dn_ssm_decode_step":
        assert _ssm(fn, S=None) == E


def _gdr(fn, **kw):
    args = dict(q=P, kw=P, v=P, kr=P, a=P, g=P, S0=P, o=P, S_final=P, S=P, B=1, H=1, T=64, dk=64,
                dv=64, dtype=1, stream=None)
    args.update(kw)
    names = {"dn_gdr_recurrent_fwd": ("q", "kw", "v", "kr", "a", "g", "S0", "o", "S_final", "B",
                                      "H", "T", "dk", "dv", "dtype", "stream"),
             "dn_gdr_decode_step": ("q", "kw", "v", "kr", "a", "g", "S", "o", "B", "H", "dk", "dv",
                                    "dtype", "stream")}[fn]
    return getattr(_lib.lib(), fn)(*[args[n] for n in names])


@pytest.mark.parametrize("fn", ["dn_gdr_recurrent_fwd", "dn_gdr_decode_step"])
def test_gdr_validation(fn):
    E, N = _lib.DN_EINVAL, _lib.DN_ENOTSUP
    for name in ("q", "kw", "v", "kr", "a", "g", "o"):
        assert _gdr(fn, **{name: None}) == E, name
    assert _gdr(fn, kr=ODD) == E
    assert _gdr(fn, v=MIS) == E      # v, o and the states are read as 16-byte vectors
    assert _gdr(fn, o=MIS) == E
    assert _gdr(fn, B=0) == E
    assert _gdr(fn, dtype=2) == E
    assert _gdr(fn, dk=96, dv=96) == N
    assert _gdr(fn, dk=64, dv=128) == N
    if fn == "dn_gdr_decode_step":
        assert _gdr(fn, S=None) == E
        assert _gdr(fn, S=MIS) == E
    else:
        assert _gdr(fn, T=-1) == E
        assert _gdr(fn, S0=MIS) == E


def test_gdr_chunk_workspace_and_validation():
    lib = _lib.lib()
    ws = lib.dn_gdr_chunk_workspace
    assert ws(1, 1, 0, 64, 64, 1, 64) == 0
    assert ws(1, 1, 64, 96, 96, 1, 64) == 0
    assert ws(1, 1, 64, 128, 128, 1, 48) == 0                # chunk lengths 16, 32, 64 only
    one = ws(1, 1, 64, 128, 128, 1, 64)
    assert one > 0 and one % 256 == 0
    assert ws(2, 3, 65, 128, 128, 1, 64) == 2 * 3 * 2 * one  # per (head, chunk)
    assert ws(1, 1, 64, 128, 128, 1, 16) % 256 == 0
    assert ws(1, 1, 65, 128, 128, 1, 16) == 5 * ws(1, 1, 16, 128, 128, 1, 16)
    args = dict(q=P, kw=P, v=P, kr=P, a=P, g=P, S0=P, o=P, S_final=P, B=1, H=1, T=64, dk=64,
                dv=64, dtype=1, chunk=64, ws=WS, wsb=1 << 30, stream=None)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return lib.dn_gdr_chunk_fwd(*[a[n] for n in ("q", "kw", "v", "kr", "a", "g", "S0", "o",
                                                       "S_final", "B", "H", "T", "dk", "dv",
                                                       "dtype", "chunk", "ws", "wsb", "stream")])
    E, W = _lib.DN_EINVAL, _lib.DN_EWORKSPACE
    assert call(kr=None) == E
    assert call(v=MIS) == E
    assert call(dk=96, dv=96) == _lib.DN_ENOTSUP
    assert call(chunk=128) == _lib.DN_ENOTSUP
    assert call(ws=None) == W
    assert call(wsb=16) == W
    assert call(ws=WS + 128) == W
    # the chunked form reads q, kw, kr, a and g as 4-element vectors: 8-byte
    # alignment for bf16, 16-byte for fp32 (an element-aligned pointer is not enough)
    for name in ("q", "kw", "kr", "a", "g"):
        assert call(**{name: P + 2}) == E, name               # bf16: 2-byte aligned only
        assert call(**{name: P + 4, "dtype": 0}) == E, name   # fp32: 4-byte aligned only
        assert call(**{name: MIS, "dtype": 0}) == E, name     # fp32: 8-byte aligned only


def test_handoff_status_validation():
    """The status query of the one-launch form validates like the prefill
    (no GPU is touched on these paths)."""
    lib = _lib.lib()
    fn = lib.dn_chunk_fwd_handoff_status
    need = lib.dn_chunk_fwd_workspace(1, 2, 4096, 128, 128, 1)
    E, N, W = _lib.DN_EINVAL, _lib.DN_ENOTSUP, _lib.DN_EWORKSPACE
    assert fn(WS, need, 0, 2, 4096, 128, 128, 1, None) == E
    assert fn(WS, need, 1, 2, -1, 128, 128, 1, None) == E
    assert fn(WS, need, 1, 2, 4096, 128, 128, 7, None) == E
    assert fn(WS, need, 1, 2, 4096, 96, 96, 1, None) == N
    assert fn(None, need, 1, 2, 4096, 128, 128, 1, None) == W
    assert fn(WS, need - 1, 1, 2, 4096, 128, 128, 1, None) == W
    assert fn(WS + 128, need, 1, 2, 4096, 128, 128, 1, None) == W
    assert fn(None, 0, 1, 2, 0, 128, 128, 1, None) == _lib.DN_OK   # T == 0: nothing ran


def test_noalloc_validation():
    """dn_chunk_fwd_noalloc checks its arguments like dn_chunk_fwd, and rejects
    sizes beyond its built-in scratch, all before any HIP call."""
    lib = _lib.lib()
    fn = lib.dn_chunk_fwd_noalloc

    def call(**kw):
        a = dict(q=P, k=P, v=P, beta=P, g=P, S0=P, o=P, S_final=P, B=1, H=1, T=64, dk=128, dv=128,
                 dtype=1, stream=None)
        a.update(kw)
        return fn(*[a[n] for n in ("q", "k", "v", "beta", "g", "S0", "o", "S_final", "B", "H", "T",
                                   "dk", "dv", "dtype", "stream")])
    assert call(q=None) == _lib.DN_EINVAL
    assert call(o=MIS) == _lib.DN_EINVAL
    assert call(B=0) == _lib.DN_EINVAL
    assert call(dk=96, dv=96) == _lib.DN_ENOTSUP
    # 128 MiB of scratch: 4 x 8 heads of 2048 tokens fit (about 75 MiB at
    # bf16, d = 128), 4 x 32 heads of 8192 tokens do not
    assert lib.dn_chunk_fwd_workspace(4, 8, 2048, 128, 128, 1) <= 128 << 20
    assert call(B=4, H=32, T=8192) == _lib.DN_ESCRATCH
    assert call(B=1, H=1, T=1 << 20, dtype=0) == _lib.DN_ESCRATCH


def test_chunk_len_validation():
    """dn_chunk_fwd_len: chunk lengths 32, 64, 128 (128 only at d = 128), bf16
    only; the workspace size is one block per (head, chunk) of the length;
    every check before any HIP call."""
    lib = _lib.lib()
    wsf = lib.dn_chunk_fwd_len_workspace
    fn = lib.dn_chunk_fwd_len

    def call(**kw):
        a = dict(q=P, k=P, v=P, beta=P, g=P, S0=P, o=P, S_final=P, B=1, H=1, T=64, dk=128, dv=128,
                 dtype=1, chunk=32, ws=WS, wsb=1 << 30, stream=None)
        a.update(kw)
        return fn(*[a[n] for n in ("q", "k", "v", "beta", "g", "S0", "o", "S_final", "B", "H", "T",
                                   "dk", "dv", "dtype", "chunk", "ws", "wsb", "stream")])
    # the block of a chunk length, through the size function
    for chunk in (32, 64, 128):
        one = wsf(1, 1, chunk, 128, 128, 1, chunk)
        assert one > 0 and one % 256 == 0
        assert wsf(2, 3, 5 * chunk + 1, 128, 128, 1, chunk) == 2 * 3 * 6 * one
    # at 64 the block is the one dn_chunk_fwd uses (its tail aside)
    state = 128 * 128 * 4
    assert wsf(1, 1, 64, 128, 128, 1, 64) == lib.dn_chunk_fwd_workspace(1, 1, 64, 128, 128, 1) - 256 - state
    assert wsf(1, 1, 64, 64, 64, 1, 128) == 0       # 128-token chunks need d = 128
    assert wsf(1, 1, 64, 128, 128, 0, 64) == 0      # bf16 only
    assert wsf(1, 1, 64, 128, 128, 1, 48) == 0
    assert wsf(1, 1, 0, 128, 128, 1, 64) == 0
    N, E, W = _lib.DN_ENOTSUP, _lib.DN_EINVAL, _lib.DN_EWORKSPACE
    assert call(chunk=48) == N
    assert call(chunk=128, dk=64, dv=64) == N
    assert call(dtype=0) == N
    assert call(q=None) == E
    assert call(o=MIS) == E
    assert call(B=0) == E
    assert call(dk=96, dv=96) == N
    assert call(ws=None) == W
    assert call(wsb=16) == W
    assert call(ws=WS + 16) == W

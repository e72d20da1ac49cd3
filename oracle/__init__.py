"""fp64 CPU oracle for the delta-rule family (DeltaNet, Gated DeltaNet, KDA).

TEST INFRASTRUCTURE ONLY. The test-suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers. The product package
never imports this module, and this module never imports the product package:
the two share no code.

The arithmetic lives in ``oracle.c`` (plain fp64 loops); this file only
compiles it with gcc, loads it and marshals numpy arrays. Inputs of any dtype
(torch bf16/fp32 tensors or numpy arrays) are widened to float64, which is
exact for bf16 and fp32 values.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DELTANET, GATED, KDA = 0, 1, 2

_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so (gcc, -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        L = ctypes.c_long
        for name in ("orc_recurrent", "orc_recurrent_matrix"):
            f = getattr(lib, name)
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.c_int] + [dp] * 8 + [L] * 5 + [ctypes.c_int]
        lib.orc_chunk.restype = ctypes.c_int
        lib.orc_chunk.argtypes = [ctypes.c_int] + [dp] * 8 + [L] * 6 + [ctypes.c_int]
        lib.orc_max_threads.restype = ctypes.c_int
        lib.orc_max_threads.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().to("cpu")
        import torch  # local: only when a tensor is passed in

        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _kind_of(g, kind):
    if kind is not None:
        return kind
    if g is None:
        return DELTANET
    return GATED


def _run(fname, q, k, v, beta, g=None, S0=None, kind=None, C=None, nthreads=0):
    lib = _load()
    kind = _kind_of(g, kind)
    q, k, v, beta, g, S0 = (_f64(x) for x in (q, k, v, beta, g, S0))
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    assert q.shape == (B, H, T, dk) and v.shape == (B, H, T, dv) and beta.shape == (B, H, T)
    if kind == GATED:
        assert g is not None and g.shape == (B, H, T)
    elif kind == KDA:
        assert g is not None and g.shape == (B, H, T, dk)
    else:
        g = None
    if S0 is not None:
        assert S0.shape == (B, H, dk, dv)
    o = np.zeros((B, H, T, dv), dtype=np.float64)
    S = np.zeros((B, H, dk, dv), dtype=np.float64)
    args = [kind, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(S0), _ptr(o), _ptr(S),
            B, H, T, dk, dv]
    if C is not None:
        args.append(C)
    args.append(nthreads)
    rc = getattr(lib, fname)(*args)
    if rc != 0:
        raise ValueError("%s rejected its arguments" % fname)
    return o, S


def recurrent(q, k, v, beta, g=None, S0=None, kind=None, nthreads=0):
    """Token-by-token error form. Returns (o [B,H,T,dv], S_T [B,H,dk,dv]) in fp64.

    kind: DELTANET (g ignored), GATED (g [B,H,T]) or KDA (g [B,H,T,dk]); by
    default GATED when g is given, DELTANET otherwise.
    """
    return _run("orc_recurrent", q, k, v, beta, g, S0, kind, None, nthreads)


def recurrent_matrix(q, k, v, beta, g=None, S0=None, kind=None, nthreads=0):
    """Transition-then-write form with an explicit d_k x d_k transition."""
    return _run("orc_recurrent_matrix", q, k, v, beta, g, S0, kind, None, nthreads)


def chunk(q, k, v, beta, g=None, S0=None, kind=None, C=64, nthreads=0):
    """fp64 chunkwise (UT / WY) form with chunk size C; cross-check only."""
    return _run("orc_chunk", q, k, v, beta, g, S0, kind, int(C), nthreads)


def decode_steps(q, k, v, beta, g, S0, kind=None, nthreads=0):
    """Apply N successive single-token steps to S0.

    q, k [N,B,H,dk]; v [N,B,H,dv]; beta [N,B,H]; g [N,B,H] (Gated), [N,B,H,dk]
    (KDA) or None. Returns (o [N,B,H,dv], S_N). Token n of the step sequence
    is token n of the recurrence, so this is the recurrence over N tokens.
    """
    def step_axis_to_time(x):
        # [N,B,H,...] -> [B,H,N,...]
        if x is None:
            return None
        return np.ascontiguousarray(np.moveaxis(_f64(x), 0, 2))

    qq, kk, vv, bb, gg = (step_axis_to_time(x) for x in (q, k, v, beta, g))
    o, S = recurrent(qq, kk, vv, bb, gg, S0, kind=kind, nthreads=nthreads)
    return np.ascontiguousarray(np.moveaxis(o, 2, 0)), S


def max_threads(nthreads: int = 0) -> int:
    """Threads an oracle call with this ``nthreads`` argument runs on."""
    return int(_load().orc_max_threads(int(nthreads)))

"""Shared helpers of the GPU parity tests (not a test module)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synthetic

KIND_CODE = {"deltanet": oracle.DELTANET, "gated": oracle.GATED, "kda": oracle.KDA}
# Parity bound per output tensor: max|gpu - ref| / max|ref| (fp32 inputs, bf16 inputs).
TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(gpu, ref) -> float:
    g = gpu.detach().float().cpu().double().numpy() if hasattr(gpu, "detach") else np.asarray(gpu)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.isfinite(g).all(), "non-finite GPU output"
    denom = max(np.abs(r).max(), 1e-30)
    return float(np.abs(g - r).max() / denom)


def to_dev(d: dict, dev="cuda") -> dict:
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def oracle_prefill(inp: dict, S0=None):
    kind = KIND_CODE[inp["kind"]]
    return oracle.recurrent(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"],
                            S0 if S0 is not None else inp.get("S0"), kind=kind)


def make(kind, B, H, T, d, dtype, seed, s0_std=None, **kw):
    return synthetic.make(kind, B, H, T, d, d, dtype=dtype, seed=seed, s0_std=s0_std, **kw)

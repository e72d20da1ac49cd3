"""MI355X (gfx950) delta-rule linear attention: DeltaNet, Gated DeltaNet, KDA.

Thin binding over the C ABI of ``include/deltanet.h``: it checks shapes and
dtypes, allocates outputs with PyTorch (device memory and streams only), and
calls the HIP library on the current stream. Every step of the operator runs
in the library's kernels; there is no CPU or PyTorch fallback, and a missing
library or GPU raises.

Tensor contract (page "28. Linear attention and Gated DeltaNet", section "The
recurrent form"): q, k [B,H,T,dk]; v [B,H,T,dv]; beta, g [B,H,T] (KDA: g
[B,H,T,dk]); states fp32 [B,H,dk,dv]. q and k are expected L2-normalised with
q already scaled by dk^-1/2 (the kernels apply no scale). Inputs are bf16 or
fp32; outputs o have the input dtype.
"""
from __future__ import annotations

import torch

from . import _lib
from ._lib import DeltaNetError, lib

__all__ = ["chunk_fwd", "chunk_fwd_fused", "chunk_fwd_len", "chunk_fwd_noalloc", "chunk_fwd_handoff_status", "kda_chunk_fwd", "chunk_fwd_states", "chunk_fwd_gqa",
           "decode_step_gqa", "chunk_fwd_varlen", "decode_tokens", "layer_prologue",
           "layer_epilogue", "gated_deltanet_layer", "ssm_chunk_fwd", "ssm_recurrent_fwd",
           "ssm_decode_step", "gdr_recurrent_fwd", "gdr_chunk_fwd", "gdr_decode_step", "chunk_prep", "chunk_scan",
           "recurrent_fwd",
           "kda_recurrent_fwd", "decode_step", "kda_decode_step", "workspace_bytes",
           "DeltaNetError", "lib", "library_path"]

_DT = {torch.float32: _lib.DN_F32, torch.bfloat16: _lib.DN_BF16}


def library_path() -> str:
    return _lib.LIB_PATH


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _check_tensor(name, t, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device or t.device.type != "cuda":
        raise ValueError("%s must be on %s (got %s)" % (name, device, t.device))
    if t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s (got %s)" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _prefill_args(q, k, v, beta, g, S0, kda):
    if q.dim() != 4:
        raise ValueError("q must be [B,H,T,dk]")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    if dt not in _DT:
        raise TypeError("inputs must be float32 or bfloat16")
    _check_tensor("q", q, (B, H, T, dk), dt, dev)
    _check_tensor("k", k, (B, H, T, dk), dt, dev)
    _check_tensor("v", v, (B, H, T, dv), dt, dev)
    _check_tensor("beta", beta, (B, H, T), dt, dev)
    if kda:
        if g is None:
            raise ValueError("KDA needs g [B,H,T,dk]")
        _check_tensor("g", g, (B, H, T, dk), dt, dev)
    elif g is not None:
        _check_tensor("g", g, (B, H, T), dt, dev)
    if S0 is not None:
        _check_tensor("S0", S0, (B, H, dk, dv), torch.float32, dev)
    return B, H, T, dk, dv, dev, dt


def workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, dtype: torch.dtype) -> int:
    """Bytes of device workspace chunk_fwd / kda_chunk_fwd need at these sizes."""
    return int(lib().dn_chunk_fwd_workspace(B, H, T, dk, dv, _DT[dtype]))


def _alloc_workspace(nbytes, dev):
    # 256-byte alignment is guaranteed by the caching allocator's block granularity
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)


def _chunk(fn_name, q, k, v, beta, g, S0, output_final_state, o, S_final, workspace, stream,
           kda):
    B, H, T, dk, dv, dev, dt = _prefill_args(q, k, v, beta, g, S0, kda)
    if o is None:
        o = torch.empty(B, H, T, dv, dtype=dt, device=dev)
    else:
        _check_tensor("o", o, (B, H, T, dv), dt, dev)
    if S_final is None and output_final_state:
        S_final = torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev)
    elif S_final is not None:
        _check_tensor("S_final", S_final, (B, H, dk, dv), torch.float32, dev)
    need = int(lib().dn_chunk_fwd_workspace(B, H, T, dk, dv, _DT[dt]))
    if workspace is None:
        workspace = _alloc_workspace(need, dev)
    fn = getattr(lib(), fn_name)
    st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(S0), _ptr(o), _ptr(S_final),
            B, H, T, dk, dv, _DT[dt], _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream(stream))
    _lib.check(fn_name, st)
    return o, S_final


def chunk_fwd(q, k, v, beta, g=None, S0=None, *, output_final_state=True, o=None, S_final=None,
              workspace=None, stream=None):
    """Chunkwise (C=64) prefill of DeltaNet (g=None) or Gated DeltaNet (g [B,H,T]).

    Returns (o [B,H,T,dv] in the input dtype, S_final fp32 [B,H,dk,dv] or None).
    S_final may be S0 for an in-place state update.
    """
    return _chunk("dn_chunk_fwd", q, k, v, beta, g, S0, output_final_state, o, S_final,
                  workspace, stream, kda=False)


def chunk_fwd_fused(q, k, v, beta, g=None, S0=None, *, output_final_state=True, o=None,
                    S_final=None, workspace=None, stream=None):
    """chunk_fwd as one kernel launch (prep and scan concurrently); bf16 only.

    Results are bitwise equal to chunk_fwd. Raises DeltaNetError (DN_ENOTSUP)
    where no one-launch form exists."""
    return _chunk("dn_chunk_fwd_fused", q, k, v, beta, g, S0, output_final_state, o, S_final,
                  workspace, stream, kda=False)


def chunk_fwd_len(q, k, v, beta, g=None, S0=None, *, chunk=64, o=None, S_final=None,
                  workspace=None, stream=None):
    """chunk_fwd in its two-launch form with chunks of `chunk` tokens (32, 64 or
    128; bf16; 128 needs d = 128). chunk=64 is bitwise chunk_fwd's two
    launches. Returns (o, S_final)."""
    B, H, T, dk, dv, dev, dt = _prefill_args(q, k, v, beta, g, S0, False)
    if o is None:
        o = torch.empty(B, H, T, dv, dtype=dt, device=dev)
    else:
        _check_tensor("o", o, (B, H, T, dv), dt, dev)
    if S_final is None:
        S_final = torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev)
    else:
        _check_tensor("S_final", S_final, (B, H, dk, dv), torch.float32, dev)
    if workspace is None:
        need = int(lib().dn_chunk_fwd_len_workspace(B, H, T, dk, dv, _DT[dt], chunk))
        workspace = _alloc_workspace(need, dev)
    st = lib().dn_chunk_fwd_len(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(S0), _ptr(o),
                                _ptr(S_final), B, H, T, dk, dv, _DT[dt], chunk, _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream))
    _lib.check("dn_chunk_fwd_len", st)
    return o, S_final


def chunk_fwd_noalloc(q, k, v, beta, g=None, S0=None, *, o=None, S_final=None, stream=None):
    """chunk_fwd without a workspace (dn_chunk_fwd_noalloc: the library's
    built-in 128 MiB scratch per GPU). o and S_final are allocated here unless
    given; pass them to keep the whole call allocation-free. Calls that
    overlap in time on one GPU race."""
    B, H, T, dk, dv, dev, dt = _prefill_args(q, k, v, beta, g, S0, False)
    if o is None:
        o = torch.empty(B, H, T, dv, dtype=dt, device=dev)
    else:
        _check_tensor("o", o, (B, H, T, dv), dt, dev)
    if S_final is None:
        S_final = torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev)
    else:
        _check_tensor("S_final", S_final, (B, H, dk, dv), torch.float32, dev)
    st = lib().dn_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(S0), _ptr(o),
                                    _ptr(S_final), B, H, T, dk, dv, _DT[dt], _stream(stream))
    _lib.check("dn_chunk_fwd_noalloc", st)
    return o, S_final


def chunk_fwd_handoff_status(workspace, B, H, T, dk, dv, dtype, stream=None):
    """Status of the latest one-launch prefill that used `workspace` with these
    sizes: DN_OK, or DN_EHANDOFF when a hand-off wait gave up and the call's
    results were recomputed by the two phases (correct either way).
    Synchronizes the stream."""
    return int(lib().dn_chunk_fwd_handoff_status(_ptr(workspace),
                                                 workspace.numel() * workspace.element_size(),
                                                 B, H, T, dk, dv, _DT[dtype], _stream(stream)))


def kda_chunk_fwd(q, k, v, beta, g, S0=None, *, output_final_state=True, o=None, S_final=None,
                  workspace=None, stream=None):
    """Chunkwise (C=64) KDA prefill; g [B,H,T,dk] per-key-channel log-decay."""
    return _chunk("dn_kda_chunk_fwd", q, k, v, beta, g, S0, output_final_state, o, S_final,
                  workspace, stream, kda=True)


def chunk_fwd_states(q, k, v, beta, g=None, S0=None, *, kda=False, o=None, S_final=None,
                     S_chunks=None, workspace=None, stream=None):
    """Chunkwise prefill that also returns the state at every chunk boundary.

    kda=False: DeltaNet / Gated DeltaNet as chunk_fwd; kda=True: as
    kda_chunk_fwd. Returns (o, S_final, S_chunks) with S_chunks fp32
    [B,H,ceil(T/64),dk,dv]: entry c is the state after the first
    min(64(c+1), T) tokens (the last equals S_final).
    """
    B, H, T, dk, dv, dev, dt = _prefill_args(q, k, v, beta, g, S0, kda)
    n = (T + 63) // 64
    if o is None:
        o = torch.empty(B, H, T, dv, dtype=dt, device=dev)
    else:
        _check_tensor("o", o, (B, H, T, dv), dt, dev)
    if S_final is None:
        S_final = torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev)
    else:
        _check_tensor("S_final", S_final, (B, H, dk, dv), torch.float32, dev)
    if S_chunks is None:
        S_chunks = torch.empty(B, H, n, dk, dv, dtype=torch.float32, device=dev)
    else:
        _check_tensor("S_chunks", S_chunks, (B, H, n, dk, dv), torch.float32, dev)
    need = int(lib().dn_chunk_fwd_workspace(B, H, T, dk, dv, _DT[dt]))
    if workspace is None:
        workspace = _alloc_workspace(need, dev)
    st = lib().dn_chunk_fwd_states(int(kda), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                                   _ptr(S0), _ptr(o), _ptr(S_final),
                                   _ptr(S_chunks) if n > 0 else None, B, H, T, dk, dv, _DT[dt],
                                   _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream))
    _lib.check("dn_chunk_fwd_states", st)
    return o, S_final, S_chunks


def chunk_fwd_gqa(q, k, v, beta, g=None, S0=None, *, kda=False, output_final_state=True, o=None,
                  S_final=None, workspace=None, stream=None):
    """Chunkwise prefill with key heads shared by value heads.

    q, k [B,Hk,T,dk]; v [B,Hv,T,dv] with Hv a multiple of Hk (key head j serves
    value heads j*Hv/Hk .. (j+1)*Hv/Hk - 1); beta, g, S0 per value head. Equal
    to chunk_fwd (kda_chunk_fwd) on q, k repeated over heads. Returns (o, S_final).
    """
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q must be [B,Hk,T,dk] and v [B,Hv,T,dv]")
    B, Hk, T, dk = q.shape
    Hv, dv = v.shape[1], v.shape[3]
    dev, dt = q.device, q.dtype
    if dt not in _DT:
        raise TypeError("q must be bfloat16 or float32")
    _check_tensor("k", k, (B, Hk, T, dk), dt, dev)
    _check_tensor("v", v, (B, Hv, T, dv), dt, dev)
    _check_tensor("beta", beta, (B, Hv, T), dt, dev)
    if kda:
        _check_tensor("g", g, (B, Hv, T, dk), dt, dev)
    elif g is not None:
        _check_tensor("g", g, (B, Hv, T), dt, dev)
    if S0 is not None:
        _check_tensor("S0", S0, (B, Hv, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty(B, Hv, T, dv, dtype=dt, device=dev)
    else:
        _check_tensor("o", o, (B, Hv, T, dv), dt, dev)
    if S_final is None and output_final_state:
        S_final = torch.empty(B, Hv, dk, dv, dtype=torch.float32, device=dev)
    elif S_final is not None:
        _check_tensor("S_final", S_final, (B, Hv, dk, dv), torch.float32, dev)
    if workspace is None:
        workspace = _alloc_workspace(int(lib().dn_chunk_fwd_workspace(B, Hv, T, dk, dv, _DT[dt])), dev)
    st = lib().dn_chunk_fwd_gqa(int(kda), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                                _ptr(S0), _ptr(o), _ptr(S_final), B, Hk, Hv, T, dk, dv, _DT[dt],
                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(stream))
    _lib.check("dn_chunk_fwd_gqa", st)
    return o, S_final


def decode_step_gqa(q, k, v, beta, g, S, *, kda=False, o=None, stream=None):
    """One decode step with key heads shared by value heads: q, k [B,Hk,dk];
    v [B,Hv,dv]; beta [B,Hv]; g [B,Hv] (gated), [B,Hv,dk] (KDA) or None;
    S [B,Hv,dk,dv] fp32 updated in place. Returns o [B,Hv,dv]."""
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q must be [B,Hk,dk] and v [B,Hv,dv]")
    B, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    dev, dt = q.device, q.dtype
    if dt not in _DT:
        raise TypeError("q must be bfloat16 or float32")
    _check_tensor("k", k, (B, Hk, dk), dt, dev)
    _check_tensor("v", v, (B, Hv, dv), dt, dev)
    _check_tensor("beta", beta, (B, Hv), dt, dev)
    if kda:
        _check_tensor("g", g, (B, Hv, dk), dt, dev)
    elif g is not None:
        _check_tensor("g", g, (B, Hv), dt, dev)
    _check_tensor("S", S, (B, Hv, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty(B, Hv, dv, dtype=dt, device=dev)
    else:
        _check_tensor("o", o, (B, Hv, dv), dt, dev)
    st = lib().dn_decode_step_gqa(int(kda), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                                  _ptr(S), _ptr(o), B, Hk, Hv, dk, dv, _DT[dt], _stream(stream))
    _lib.check("dn_decode_step_gqa", st)
    return o


def chunk_fwd_varlen(q, k, v, beta, g, cu_seqlens, S0=None, *, kda=False, output_final_state=True,
                     o=None, S_final=None, workspace=None, stream=None):
    """Chunkwise prefill over packed sequences of different lengths.

    q, k [1,H,T,dk], v [1,H,T,dv], beta [1,H,T], g [1,H,T] / [1,H,T,dk] (KDA) /
    None: the sequences back to back; cu_seqlens int32 [N+1] on the device
    (sequence n = tokens cu_seqlens[n] .. cu_seqlens[n+1]-1); S0 [N,H,dk,dv].
    Returns (o [1,H,T,dv], S_final [N,H,dk,dv] fp32 or None).
    """
    B, H, T, dk, dv, dev, dt = _prefill_args(q, k, v, beta, g, None, kda)
    if B != 1:
        raise ValueError("packed sequences take B = 1 (q [1,H,T,dk])")
    if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dim() != 1 or \
            cu_seqlens.dtype != torch.int32 or cu_seqlens.device != dev:
        raise ValueError("cu_seqlens must be an int32 [N+1] tensor on %s" % dev)
    N = cu_seqlens.numel() - 1
    if N < 1:
        raise ValueError("cu_seqlens needs at least two entries")
    cu_seqlens = cu_seqlens.contiguous()
    if S0 is not None:
        _check_tensor("S0", S0, (N, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty(1, H, T, dv, dtype=dt, device=dev)
    else:
        _check_tensor("o", o, (1, H, T, dv), dt, dev)
    if S_final is None and output_final_state:
        S_final = torch.empty(N, H, dk, dv, dtype=torch.float32, device=dev)
    elif S_final is not None:
        _check_tensor("S_final", S_final, (N, H, dk, dv), torch.float32, dev)
    if workspace is None:
        need = int(lib().dn_chunk_fwd_varlen_workspace(N, H, T, dk, dv, _DT[dt]))
        workspace = _alloc_workspace(need, dev)
    st = lib().dn_chunk_fwd_varlen(int(kda), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                                   _ptr(S0), _ptr(o), _ptr(S_final), _ptr(cu_seqlens), N, H, T, dk,
                                   dv, _DT[dt], _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream))
    _lib.check("dn_chunk_fwd_varlen", st)
    return o, S_final


def decode_tokens(q, k, v, beta, g, S, *, kda=False, snapshots=True, o=None, S_snap=None,
                  stream=None):
    """K decode tokens per sequence in one call (speculative decoding).

    q, k [B,H,K,dk]; v [B,H,K,dv]; beta [B,H,K]; g [B,H,K] / [B,H,K,dk] (KDA) /
    None; S [B,H,dk,dv] fp32 updated in place. Returns (o [B,H,K,dv], S_snap
    [B,H,K,dk,dv] with the state after each token, or None if not requested).
    """
    B, H, K, dk, dv, dev, dt = _prefill_args(q, k, v, beta, g, None, kda)
    _check_tensor("S", S, (B, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty(B, H, K, dv, dtype=dt, device=dev)
    else:
        _check_tensor("o", o, (B, H, K, dv), dt, dev)
    if S_snap is None and snapshots:
        S_snap = torch.empty(B, H, K, dk, dv, dtype=torch.float32, device=dev)
    elif S_snap is not None:
        _check_tensor("S_snap", S_snap, (B, H, K, dk, dv), torch.float32, dev)
    st = lib().dn_decode_tokens(int(kda), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(S),
                                _ptr(o), _ptr(S_snap), B, H, K, dk, dv, _DT[dt], _stream(stream))
    _lib.check("dn_decode_tokens", st)
    return o, S_snap


def layer_prologue(qkv, conv_w, b, a, A_log, dt_bias, Hk, Hv, *, conv_state=None,
                   conv_state_out=None, update_conv_state=True, allow_neg_eigval=False, out=None,
                   stream=None):
    """The gated layer's work before the rule, from the projected rows.

    qkv [B,T,2*Hk*d + Hv*d] (q, k, v channels per token); conv_w [C,4];
    b, a [B,T,Hv]; A_log, dt_bias [Hv] fp32 (a, A_log, dt_bias all None: no
    decay gate, g is None). conv_state [B,C,3] or None (zeros). The new
    convolution state goes to conv_state_out (default: a new tensor, or None
    when update_conv_state is False); pass conv_state_out=conv_state to update
    in place. allow_neg_eigval: beta = 2 sigmoid(b) in (0, 2) (the reflection
    range). ``out`` optionally gives (q, k, v, beta, g) to write into.
    Returns (q [B,Hk,T,d], k, v [B,Hv,T,d], beta [B,Hv,T], g [B,Hv,T] or None,
    new conv state or None).
    """
    if qkv.dim() != 3:
        raise ValueError("qkv must be [B,T,C]")
    B, T, C = qkv.shape
    dev, dt = qkv.device, qkv.dtype
    if dt not in _DT:
        raise TypeError("qkv must be bfloat16 or float32")
    if Hk < 1 or Hv < 1 or C % (2 * Hk + Hv):
        raise ValueError("C = %d is not (2*Hk + Hv) * d for Hk=%d, Hv=%d" % (C, Hk, Hv))
    d = C // (2 * Hk + Hv)
    _check_tensor("qkv", qkv, (B, T, C), dt, dev)
    _check_tensor("conv_w", conv_w, (C, 4), dt, dev)
    _check_tensor("b", b, (B, T, Hv), dt, dev)
    gated = a is not None
    if gated:
        _check_tensor("a", a, (B, T, Hv), dt, dev)
        _check_tensor("A_log", A_log, (Hv,), torch.float32, dev)
        _check_tensor("dt_bias", dt_bias, (Hv,), torch.float32, dev)
    if conv_state is not None:
        _check_tensor("conv_state", conv_state, (B, C, 3), dt, dev)
    if conv_state_out is None and update_conv_state:
        conv_state_out = torch.empty(B, C, 3, dtype=dt, device=dev)
    elif conv_state_out is not None:
        _check_tensor("conv_state_out", conv_state_out, (B, C, 3), dt, dev)
    if out is None:
        q = torch.empty(B, Hk, T, d, dtype=dt, device=dev)
        k = torch.empty(B, Hk, T, d, dtype=dt, device=dev)
        v = torch.empty(B, Hv, T, d, dtype=dt, device=dev)
        beta = torch.empty(B, Hv, T, dtype=dt, device=dev)
        g = torch.empty(B, Hv, T, dtype=dt, device=dev) if gated else None
    else:
        q, k, v, beta, g = out
        _check_tensor("q", q, (B, Hk, T, d), dt, dev)
        _check_tensor("k", k, (B, Hk, T, d), dt, dev)
        _check_tensor("v", v, (B, Hv, T, d), dt, dev)
        _check_tensor("beta", beta, (B, Hv, T), dt, dev)
        if gated:
            _check_tensor("g", g, (B, Hv, T), dt, dev)
        else:
            g = None
    st = lib().dn_layer_prologue(_ptr(qkv), _ptr(conv_w), _ptr(conv_state), _ptr(conv_state_out),
                                 _ptr(b), _ptr(a), _ptr(A_log), _ptr(dt_bias), _ptr(q), _ptr(k),
                                 _ptr(v), _ptr(beta), _ptr(g), int(bool(allow_neg_eigval)), B, T,
                                 Hk, Hv, d, d, _DT[dt], _stream(stream))
    _lib.check("dn_layer_prologue", st)
    return q, k, v, beta, g, conv_state_out


def layer_epilogue(o, z, norm_w, eps=1e-6, *, out=None, stream=None):
    """Gated RMSNorm after the rule: o [B,Hv,T,dv] (head-major read-out),
    z [B,T,Hv*dv], norm_w [dv] -> out [B,T,Hv*dv] (token-major, ready for the
    output projection)."""
    if o.dim() != 4:
        raise ValueError("o must be [B,Hv,T,dv]")
    B, Hv, T, dv = o.shape
    dev, dt = o.device, o.dtype
    if dt not in _DT:
        raise TypeError("o must be bfloat16 or float32")
    _check_tensor("o", o, (B, Hv, T, dv), dt, dev)
    _check_tensor("z", z, (B, T, Hv * dv), dt, dev)
    _check_tensor("norm_w", norm_w, (dv,), dt, dev)
    if out is None:
        out = torch.empty(B, T, Hv * dv, dtype=dt, device=dev)
    else:
        _check_tensor("out", out, (B, T, Hv * dv), dt, dev)
    st = lib().dn_layer_epilogue(_ptr(o), _ptr(z), _ptr(norm_w), _ptr(out), B, Hv, T, dv,
                                 float(eps), _DT[dt], _stream(stream))
    _lib.check("dn_layer_epilogue", st)
    return out


def layer_decode_step(qkv, z, b, a, conv_w, A_log, dt_bias, norm_w, Hk, Hv, S, *, conv_state=None,
                      conv_state_out=None, eps=1e-6, allow_neg_eigval=False, out=None,
                      stream=None):
    """The whole gated layer for one token per sequence in one kernel:
    prologue, decode step (S [B,Hv,d,d] fp32 updated in place) and epilogue.

    qkv [B,1,C], z [B,1,Hv*d], b, a [B,1,Hv] (a, A_log, dt_bias None: no decay
    gate); conv_state [B,C,3] or None (zeros). The new convolution state goes
    to conv_state_out (default: a new tensor; conv_state itself is allowed when
    Hk == Hv). Returns (out [B,1,Hv*d], new conv state).
    """
    if qkv.dim() != 3 or qkv.shape[1] != 1:
        raise ValueError("qkv must be [B,1,C]")
    B, _, C = qkv.shape
    dev, dt = qkv.device, qkv.dtype
    if dt not in _DT:
        raise TypeError("qkv must be bfloat16 or float32")
    if Hk < 1 or Hv < 1 or C % (2 * Hk + Hv):
        raise ValueError("C = %d is not (2*Hk + Hv) * d for Hk=%d, Hv=%d" % (C, Hk, Hv))
    d = C // (2 * Hk + Hv)
    _check_tensor("conv_w", conv_w, (C, 4), dt, dev)
    _check_tensor("b", b, (B, 1, Hv), dt, dev)
    if a is not None:
        _check_tensor("a", a, (B, 1, Hv), dt, dev)
        _check_tensor("A_log", A_log, (Hv,), torch.float32, dev)
        _check_tensor("dt_bias", dt_bias, (Hv,), torch.float32, dev)
    _check_tensor("z", z, (B, 1, Hv * d), dt, dev)
    _check_tensor("norm_w", norm_w, (d,), dt, dev)
    _check_tensor("S", S, (B, Hv, d, d), torch.float32, dev)
    if conv_state is not None:
        _check_tensor("conv_state", conv_state, (B, C, 3), dt, dev)
    if conv_state_out is None:
        conv_state_out = torch.empty(B, C, 3, dtype=dt, device=dev)
    else:
        _check_tensor("conv_state_out", conv_state_out, (B, C, 3), dt, dev)
    if out is None:
        out = torch.empty(B, 1, Hv * d, dtype=dt, device=dev)
    else:
        _check_tensor("out", out, (B, 1, Hv * d), dt, dev)
    st = lib().dn_layer_decode_step(_ptr(qkv), _ptr(conv_w), _ptr(conv_state), _ptr(conv_state_out),
                                    _ptr(b), _ptr(a), _ptr(A_log), _ptr(dt_bias), _ptr(z),
                                    _ptr(norm_w), float(eps), _ptr(S), _ptr(out),
                                    int(bool(allow_neg_eigval)), B, Hk, Hv, d, _DT[dt], _stream(stream))
    _lib.check("dn_layer_decode_step", st)
    return out, conv_state_out


def layer_prefill_workspace(B, T, Hk, Hv, d, dtype, device):
    """Workspace of layer_prefill (uninitialised device bytes)."""
    n = lib().dn_layer_prefill_workspace(B, T, Hk, Hv, d, _DT[dtype])
    if n == 0 and T > 0:
        raise ValueError("layer_prefill supports bfloat16 with d = 128 only")
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def layer_prefill(qkv, z, b, a, conv_w, A_log, dt_bias, norm_w, Hk, Hv, *, conv_state=None,
                  conv_state_out=None, update_conv_state=True, S0=None, S_final=None, eps=1e-6,
                  allow_neg_eigval=False, out=None, workspace=None, stream=None):
    """The gated layer between its projections for a prefill (bf16, d = 128):
    the prologue formed in the prefill's chunk-parallel phase, the scan, the
    gated RMSNorm; bitwise the result of layer_prologue, chunk_fwd_gqa and
    layer_epilogue.

    qkv [B,T,C], z [B,T,Hv*d], b, a [B,T,Hv] (a, A_log, dt_bias None: no decay
    gate); conv_state [B,C,3] or None (zeros); S0 [B,Hv,d,d] fp32 or None. The
    new conv state goes to conv_state_out (default: a new tensor, or None when
    update_conv_state is False; it must not overlap conv_state). Returns
    (out [B,T,Hv*d], new conv state, S_final).
    """
    if qkv.dim() != 3:
        raise ValueError("qkv must be [B,T,C]")
    B, T, C = qkv.shape
    dev, dt = qkv.device, qkv.dtype
    if dt not in _DT:
        raise TypeError("qkv must be bfloat16 or float32")
    if Hk < 1 or Hv < 1 or C % (2 * Hk + Hv):
        raise ValueError("C = %d is not (2*Hk + Hv) * d for Hk=%d, Hv=%d" % (C, Hk, Hv))
    d = C // (2 * Hk + Hv)
    _check_tensor("conv_w", conv_w, (C, 4), dt, dev)
    _check_tensor("b", b, (B, T, Hv), dt, dev)
    if a is not None:
        _check_tensor("a", a, (B, T, Hv), dt, dev)
        _check_tensor("A_log", A_log, (Hv,), torch.float32, dev)
        _check_tensor("dt_bias", dt_bias, (Hv,), torch.float32, dev)
    _check_tensor("z", z, (B, T, Hv * d), dt, dev)
    _check_tensor("norm_w", norm_w, (d,), dt, dev)
    if conv_state is not None:
        _check_tensor("conv_state", conv_state, (B, C, 3), dt, dev)
    if conv_state_out is None and update_conv_state:
        conv_state_out = torch.empty(B, C, 3, dtype=dt, device=dev)
    elif conv_state_out is not None:
        _check_tensor("conv_state_out", conv_state_out, (B, C, 3), dt, dev)
    if S0 is not None:
        _check_tensor("S0", S0, (B, Hv, d, d), torch.float32, dev)
    if S_final is None:
        S_final = torch.empty(B, Hv, d, d, dtype=torch.float32, device=dev)
    else:
        _check_tensor("S_final", S_final, (B, Hv, d, d), torch.float32, dev)
    if out is None:
        out = torch.empty(B, T, Hv * d, dtype=dt, device=dev)
    else:
        _check_tensor("out", out, (B, T, Hv * d), dt, dev)
    if workspace is None:
        workspace = layer_prefill_workspace(B, T, Hk, Hv, d, dt, dev)
    st = lib().dn_layer_prefill(_ptr(qkv), _ptr(conv_w), _ptr(conv_state), _ptr(conv_state_out),
                                _ptr(b), _ptr(a), _ptr(A_log), _ptr(dt_bias), _ptr(z), _ptr(norm_w),
                                float(eps), _ptr(S0), _ptr(S_final), _ptr(out),
                                int(bool(allow_neg_eigval)), B, T, Hk, Hv, d, _DT[dt], _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream))
    _lib.check("dn_layer_prefill", st)
    return out, conv_state_out, S_final


def gated_deltanet_layer(qkv, z, b, a, conv_w, A_log, dt_bias, norm_w, Hk, Hv, *,
                         conv_state=None, S=None, eps=1e-6, allow_neg_eigval=False,
                         workspace=None, stream=None):
    """The gated layer between its input and output projections (page "28.
    Linear attention and Gated DeltaNet", section "The full layer"): prologue,
    the rule (the recurrent step for T == 1 with a carried state, the chunked
    form otherwise), epilogue. The projections themselves are plain GEMMs and
    stay with the caller: qkv, z, b, a are their outputs.

    S [B,Hv,d,d] fp32 (or None: zeros) is the carried recurrent state; it is
    updated in place when given. One token with a carried state runs as the
    single-kernel layer step (layer_decode_step); a bf16 prefill at d = 128 as
    layer_prefill (the prologue inside the prefill's prep). Returns (out [B,T,Hv*d], new conv state,
    new recurrent state).
    """
    if qkv.dim() == 3 and qkv.shape[1] == 1 and S is not None:
        # one token with a carried state: the single-kernel layer step
        out, cst = layer_decode_step(qkv, z, b, a, conv_w, A_log, dt_bias, norm_w, Hk, Hv, S,
                                     conv_state=conv_state, eps=eps,
                                     allow_neg_eigval=allow_neg_eigval, stream=stream)
        return out, cst, S
    B, T, C = qkv.shape
    d = C // (2 * Hk + Hv) if Hk >= 1 and Hv >= 1 else 0
    if qkv.dtype == torch.bfloat16 and d == 128 and T >= 1:
        # the prologue inside the prefill's prep (bitwise the three calls below)
        need = lib().dn_layer_prefill_workspace(B, T, Hk, Hv, d, _DT[qkv.dtype])
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = None
        return layer_prefill(qkv, z, b, a, conv_w, A_log, dt_bias, norm_w, Hk, Hv,
                             conv_state=conv_state, S0=S, S_final=S, eps=eps,
                             allow_neg_eigval=allow_neg_eigval, workspace=workspace, stream=stream)
    q, k, v, beta, g, cst = layer_prologue(qkv, conv_w, b, a, A_log, dt_bias, Hk, Hv,
                                           conv_state=conv_state,
                                           allow_neg_eigval=allow_neg_eigval, stream=stream)
    o, S_new = chunk_fwd_gqa(q, k, v, beta, g, S, S_final=S, workspace=workspace, stream=stream)
    return layer_epilogue(o, z, norm_w, eps, stream=stream), cst, S_new


def _ssm_args(q, k, v, g, S0):
    if q.dim() != 4:
        raise ValueError("q must be [B,H,T,dk]")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    if dt not in _DT:
        raise TypeError("q must be bfloat16 or float32")
    _check_tensor("q", q, (B, H, T, dk), dt, dev)
    _check_tensor("k", k, (B, H, T, dk), dt, dev)
    _check_tensor("v", v, (B, H, T, dv), dt, dev)
    _check_tensor("g", g, (B, H, T), dt, dev)
    if S0 is not None:
        _check_tensor("S0", S0, (B, H, dk, dv), torch.float32, dev)
    return B, H, T, dk, dv, dev, dt


def ssm_chunk_fwd(q, k, v, g, S0=None, *, output_final_state=True, o=None, S_final=None,
                  workspace=None, stream=None):
    """Chunked selective state-space recurrence S = exp(g) S + k v^T,
    o = S^T q (Gated DeltaNet without the correction term; no beta).
    q, k [B,H,T,dk]; v [B,H,T,dv]; g [B,H,T] (zeros: plain causal linear
    attention). Returns (o, S_final)."""
    B, H, T, dk, dv, dev, dt = _ssm_args(q, k, v, g, S0)
    if o is None:
        o = torch.empty(B, H, T, dv, dtype=dt, device=dev)
    else:
        _check_tensor("o", o, (B, H, T, dv), dt, dev)
    if S_final is None and output_final_state:
        S_final = torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev)
    elif S_final is not None:
        _check_tensor("S_final", S_final, (B, H, dk, dv), torch.float32, dev)
    if workspace is None:
        workspace = _alloc_workspace(workspace_bytes(B, H, T, dk, dv, dt), dev)
    st = lib().dn_ssm_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(S0), _ptr(o),
                                _ptr(S_final), B, H, T, dk, dv, _DT[dt], _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream))
    _lib.check("dn_ssm_chunk_fwd", st)
    return o, S_final


def ssm_recurrent_fwd(q, k, v, g, S0=None, *, output_final_state=True, stream=None):
    """Token-by-token form of ssm_chunk_fwd. Returns (o, S_final)."""
    B, H, T, dk, dv, dev, dt = _ssm_args(q, k, v, g, S0)
    o = torch.empty(B, H, T, dv, dtype=dt, device=dev)
    S_final = torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev) if output_final_state else None
    st = lib().dn_ssm_recurrent_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(S0), _ptr(o),
                                    _ptr(S_final), B, H, T, dk, dv, _DT[dt], _stream(stream))
    _lib.check("dn_ssm_recurrent_fwd", st)
    return o, S_final


def ssm_decode_step(q, k, v, g, S, *, o=None, stream=None):
    """One token of the selective state-space recurrence: q, k [B,H,dk];
    v [B,H,dv]; g [B,H]; S [B,H,dk,dv] fp32 updated in place. Returns o [B,H,dv]."""
    if q.dim() != 3:
        raise ValueError("q must be [B,H,dk]")
    B, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    if dt not in _DT:
        raise TypeError("q must be bfloat16 or float32")
    _check_tensor("k", k, (B, H, dk), dt, dev)
    _check_tensor("v", v, (B, H, dv), dt, dev)
    _check_tensor("g", g, (B, H), dt, dev)
    _check_tensor("S", S, (B, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty(B, H, dv, dtype=dt, device=dev)
    else:
        _check_tensor("o", o, (B, H, dv), dt, dev)
    st = lib().dn_ssm_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(S), _ptr(o), B, H, dk,
                                  dv, _DT[dt], _stream(stream))
    _lib.check("dn_ssm_decode_step", st)
    return o


def gdr_recurrent_fwd(q, kw, v, kr, a, g, S0=None, *, output_final_state=True, o=None,
                      S_final=None, stream=None):
    """Generalized delta rule, token by token:
    S = (diag(exp g) - (a * kr) kr^T) S + kw v^T, o = S^T q.
    q, kw (write key), kr (removal key), a (removal rate), g (log-decay)
    [B,H,T,dk]; v [B,H,T,dv]; S0 [B,H,dk,dv] fp32 or None. Returns (o, S_final)."""
    if q.dim() != 4:
        raise ValueError("q must be [B,H,T,dk]")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    if dt not in _DT:
        raise TypeError("q must be bfloat16 or float32")
    for name, t in (("kw", kw), ("kr", kr), ("a", a), ("g", g)):
        _check_tensor(name, t, (B, H, T, dk), dt, dev)
    _check_tensor("v", v, (B, H, T, dv), dt, dev)
    if S0 is not None:
        _check_tensor("S0", S0, (B, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty(B, H, T, dv, dtype=dt, device=dev)
    else:
        _check_tensor("o", o, (B, H, T, dv), dt, dev)
    if S_final is None and output_final_state:
        S_final = torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev)
    elif S_final is not None:
        _check_tensor("S_final", S_final, (B, H, dk, dv), torch.float32, dev)
    st = lib().dn_gdr_recurrent_fwd(_ptr(q), _ptr(kw), _ptr(v), _ptr(kr), _ptr(a), _ptr(g),
                                    _ptr(S0), _ptr(o), _ptr(S_final), B, H, T, dk, dv, _DT[dt],
                                    _stream(stream))
    _lib.check("dn_gdr_recurrent_fwd", st)
    return o, S_final


def gdr_chunk_fwd(q, kw, v, kr, a, g, S0=None, *, chunk=64, output_final_state=True, o=None,
                  S_final=None, workspace=None, stream=None):
    """Chunked form of gdr_recurrent_fwd (chunks of ``chunk`` = 16, 32 or 64
    tokens reduced to affine maps of the state, fp32 arithmetic). Same
    arguments; ``workspace`` (uint8, at least dn_gdr_chunk_workspace bytes) is
    allocated when not given. Returns (o, S_final)."""
    if q.dim() != 4:
        raise ValueError("q must be [B,H,T,dk]")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    if dt not in _DT:
        raise TypeError("q must be bfloat16 or float32")
    for name, t in (("kw", kw), ("kr", kr), ("a", a), ("g", g)):
        _check_tensor(name, t, (B, H, T, dk), dt, dev)
    _check_tensor("v", v, (B, H, T, dv), dt, dev)
    if S0 is not None:
        _check_tensor("S0", S0, (B, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty(B, H, T, dv, dtype=dt, device=dev)
    else:
        _check_tensor("o", o, (B, H, T, dv), dt, dev)
    if S_final is None and output_final_state:
        S_final = torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev)
    elif S_final is not None:
        _check_tensor("S_final", S_final, (B, H, dk, dv), torch.float32, dev)
    if workspace is None:
        workspace = _alloc_workspace(
            int(lib().dn_gdr_chunk_workspace(B, H, T, dk, dv, _DT[dt], int(chunk))), dev)
    st = lib().dn_gdr_chunk_fwd(_ptr(q), _ptr(kw), _ptr(v), _ptr(kr), _ptr(a), _ptr(g), _ptr(S0),
                                _ptr(o), _ptr(S_final), B, H, T, dk, dv, _DT[dt], int(chunk),
                                _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream))
    _lib.check("dn_gdr_chunk_fwd", st)
    return o, S_final


def gdr_decode_step(q, kw, v, kr, a, g, S, *, o=None, stream=None):
    """One token of the generalized delta rule: q, kw, kr, a, g [B,H,dk];
    v [B,H,dv]; S [B,H,dk,dv] fp32 updated in place. Returns o [B,H,dv]."""
    if q.dim() != 3:
        raise ValueError("q must be [B,H,dk]")
    B, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    if dt not in _DT:
        raise TypeError("q must be bfloat16 or float32")
    for name, t in (("kw", kw), ("kr", kr), ("a", a), ("g", g)):
        _check_tensor(name, t, (B, H, dk), dt, dev)
    _check_tensor("v", v, (B, H, dv), dt, dev)
    _check_tensor("S", S, (B, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty(B, H, dv, dtype=dt, device=dev)
    else:
        _check_tensor("o", o, (B, H, dv), dt, dev)
    st = lib().dn_gdr_decode_step(_ptr(q), _ptr(kw), _ptr(v), _ptr(kr), _ptr(a), _ptr(g), _ptr(S),
                                  _ptr(o), B, H, dk, dv, _DT[dt], _stream(stream))
    _lib.check("dn_gdr_decode_step", st)
    return o


def chunk_prep(q, k, v, beta, g, workspace, *, kda=False, stream=None):
    """Phase 1 of the chunkwise prefill (all chunks in parallel) into ``workspace``."""
    B, H, T, dk, dv, dev, dt = _prefill_args(q, k, v, beta, g, None, kda)
    st = lib().dn_chunk_prep(int(kda), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), B, H, T, dk,
                             dv, _DT[dt], _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(stream))
    _lib.check("dn_chunk_prep", st)


def chunk_scan(q, o, workspace, S0=None, S_final=None, *, kda=False, stream=None):
    """Phase 2 of the chunkwise prefill: the sequential scan over ``workspace``.

    q is the query tensor given to chunk_prep (read again by this phase);
    o [B,H,T,dv] (input dtype) receives the outputs; S_final (fp32) the end state.
    """
    B, H, T, dv = o.shape
    dk = dv
    dev, dt = o.device, o.dtype
    _check_tensor("q", q, (B, H, T, dk), dt, dev)
    _check_tensor("o", o, (B, H, T, dv), dt, dev)
    if S0 is not None:
        _check_tensor("S0", S0, (B, H, dk, dv), torch.float32, dev)
    if S_final is not None:
        _check_tensor("S_final", S_final, (B, H, dk, dv), torch.float32, dev)
    st = lib().dn_chunk_scan(int(kda), _ptr(q), _ptr(S0), _ptr(o), _ptr(S_final), B, H, T, dk, dv,
                             _DT[dt], _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(stream))
    _lib.check("dn_chunk_scan", st)


def _recurrent(fn_name, q, k, v, beta, g, S0, output_final_state, stream, kda):
    B, H, T, dk, dv, dev, dt = _prefill_args(q, k, v, beta, g, S0, kda)
    o = torch.empty(B, H, T, dv, dtype=dt, device=dev)
    S_final = torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev) if output_final_state else None
    st = getattr(lib(), fn_name)(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(S0), _ptr(o),
                                 _ptr(S_final), B, H, T, dk, dv, _DT[dt], _stream(stream))
    _lib.check(fn_name, st)
    return o, S_final


def recurrent_fwd(q, k, v, beta, g=None, S0=None, *, output_final_state=True, stream=None):
    """Token-by-token recurrent form (same contract and result as chunk_fwd)."""
    return _recurrent("dn_recurrent_fwd", q, k, v, beta, g, S0, output_final_state, stream, False)


def kda_recurrent_fwd(q, k, v, beta, g, S0=None, *, output_final_state=True, stream=None):
    """Token-by-token KDA recurrence; g [B,H,T,dk]."""
    return _recurrent("dn_kda_recurrent_fwd", q, k, v, beta, g, S0, output_final_state, stream,
                      True)


def _decode(fn_name, q, k, v, beta, g, S, o, stream, kda):
    if q.dim() != 3:
        raise ValueError("q must be [B,H,dk]")
    B, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    if dt not in _DT:
        raise TypeError("inputs must be float32 or bfloat16")
    _check_tensor("k", k, (B, H, dk), dt, dev)
    _check_tensor("v", v, (B, H, dv), dt, dev)
    _check_tensor("beta", beta, (B, H), dt, dev)
    if kda:
        if g is None:
            raise ValueError("KDA needs g [B,H,dk]")
        _check_tensor("g", g, (B, H, dk), dt, dev)
    elif g is not None:
        _check_tensor("g", g, (B, H), dt, dev)
    _check_tensor("S", S, (B, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty(B, H, dv, dtype=dt, device=dev)
    else:
        _check_tensor("o", o, (B, H, dv), dt, dev)
    st = getattr(lib(), fn_name)(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(S), _ptr(o),
                                 B, H, dk, dv, _DT[dt], _stream(stream))
    _lib.check(fn_name, st)
    return o


def decode_step(q, k, v, beta, g, S, *, o=None, stream=None):
    """One decode step: S [B,H,dk,dv] fp32 is updated in place; returns o [B,H,dv]."""
    return _decode("dn_decode_step", q, k, v, beta, g, S, o, stream, False)


def kda_decode_step(q, k, v, beta, g, S, *, o=None, stream=None):
    """One KDA decode step; g [B,H,dk]."""
    return _decode("dn_kda_decode_step", q, k, v, beta, g, S, o, stream, True)

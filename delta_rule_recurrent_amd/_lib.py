"""ctypes loader for libdeltanet.so (the HIP library behind include/deltanet.h).

The library is built in-tree (``delta_rule_recurrent_amd/libdeltanet.so``). If
it is missing it is built once with hipcc; if that is impossible the import
fails loudly: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading

from . import build as _build

LIB_PATH = _build.LIB

DN_OK, DN_EINVAL, DN_ENOTSUP, DN_EWORKSPACE, DN_EHIP, DN_EHANDOFF, DN_ESCRATCH = 0, -1, -2, -3, -4, -5, -6
DN_F32, DN_BF16 = 0, 1

# Every symbol include/deltanet.h declares, with its ctypes signature.
_vp, _i, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_PREFILL = [_vp] * 8 + [_i] * 6
SIGNATURES = {
    "dn_strerror": (ctypes.c_char_p, [_i]),
    "dn_version": (_i, []),
    "dn_chunk_fwd_workspace": (_sz, [_i] * 6),
    "dn_chunk_fwd": (_i, _PREFILL + [_vp, _sz, _vp]),
    "dn_chunk_fwd_fused": (_i, _PREFILL + [_vp, _sz, _vp]),
    "dn_chunk_fwd_handoff_status": (_i, [_vp, _sz] + [_i] * 6 + [_vp]),
    "dn_chunk_fwd_noalloc": (_i, _PREFILL + [_vp]),
    "dn_kda_chunk_fwd": (_i, _PREFILL + [_vp, _sz, _vp]),
    "dn_chunk_fwd_len_workspace": (_sz, [_i] * 7),
    "dn_chunk_fwd_len": (_i, _PREFILL + [_i, _vp, _sz, _vp]),
    "dn_chunk_fwd_states": (_i, [_i] + [_vp] * 9 + [_i] * 6 + [_vp, _sz, _vp]),
    "dn_chunk_fwd_gqa": (_i, [_i] + [_vp] * 8 + [_i] * 7 + [_vp, _sz, _vp]),
    "dn_decode_step_gqa": (_i, [_i] + [_vp] * 7 + [_i] * 6 + [_vp]),
    "dn_chunk_fwd_varlen_workspace": (_sz, [_i] * 6),
    "dn_chunk_fwd_varlen": (_i, [_i] + [_vp] * 9 + [_i] * 6 + [_vp, _sz, _vp]),
    "dn_decode_tokens": (_i, [_i] + [_vp] * 8 + [_i] * 6 + [_vp]),
    "dn_layer_prologue": (_i, [_vp] * 13 + [_i] * 8 + [_vp]),
    "dn_ssm_chunk_fwd": (_i, [_vp] * 7 + [_i] * 6 + [_vp, _sz, _vp]),
    "dn_ssm_recurrent_fwd": (_i, [_vp] * 7 + [_i] * 6 + [_vp]),
    "dn_ssm_decode_step": (_i, [_vp] * 6 + [_i] * 5 + [_vp]),
    "dn_layer_epilogue": (_i, [_vp] * 4 + [_i] * 4 + [ctypes.c_float, _i, _vp]),
    "dn_layer_decode_step": (_i, [_vp] * 10 + [ctypes.c_float, _vp, _vp] + [_i] * 6 + [_vp]),
    "dn_layer_prefill_workspace": (_sz, [_i] * 6),
    "dn_layer_prefill": (_i, [_vp] * 10 + [ctypes.c_float, _vp, _vp, _vp] + [_i] * 7 + [_vp, _sz, _vp]),
    "dn_gdr_recurrent_fwd": (_i, [_vp] * 9 + [_i] * 6 + [_vp]),
    "dn_gdr_decode_step": (_i, [_vp] * 8 + [_i] * 5 + [_vp]),
    "dn_gdr_chunk_workspace": (_sz, [_i] * 7),
    "dn_gdr_chunk_fwd": (_i, [_vp] * 9 + [_i] * 7 + [_vp, _sz, _vp]),
    "dn_chunk_prep": (_i, [_i] + [_vp] * 5 + [_i] * 6 + [_vp, _sz, _vp]),
    "dn_chunk_scan": (_i, [_i] + [_vp] * 4 + [_i] * 6 + [_vp, _sz, _vp]),
    "dn_recurrent_fwd": (_i, _PREFILL + [_vp]),
    "dn_kda_recurrent_fwd": (_i, _PREFILL + [_vp]),
    "dn_decode_step": (_i, [_vp] * 7 + [_i] * 5 + [_vp]),
    "dn_kda_decode_step": (_i, [_vp] * 7 + [_i] * 5 + [_vp]),
}

_lock = threading.Lock()
_lib = None


class DeltaNetError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (fn, strerror(status), status))


def lib() -> ctypes.CDLL:
    """The loaded library (built first if the .so does not exist yet)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                _build.build()
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
    return _lib


def strerror(status: int) -> str:
    return lib().dn_strerror(int(status)).decode()


def check(fn: str, status: int) -> None:
    if status != DN_OK:
        raise DeltaNetError(fn, status)

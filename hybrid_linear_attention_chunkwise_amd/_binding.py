"""ctypes binding of liblola.so (the C ABI in include/lola.h).

Argument marshalling only: every step of the method runs in the library's HIP kernels.  torch tensors
are used for device memory and streams; their data pointers cross the ABI as plain integers.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblola.so")

LOLA_OK = 0
LOLA_EINVAL = -1
LOLA_EUNSUPPORTED = -2
LOLA_EDEVICE = -3
LOLA_F32 = 0
LOLA_BF16 = 1
LOLA_PHI_ELU1 = 0
LOLA_PHI_SOFTMAX_PM = 1

EXPORTED = ("lola_workspace_bytes", "lola_state_init", "lola_prefill", "lola_prefill_ex",
            "lola_prefill_profiled", "lola_decode_step", "lola_decode_step_ex", "lola_sre_collisions",
            "lola_status_string", "hola_workspace_bytes", "hola_prefill", "hola_state_init",
            "hola_prefill_state", "hola_decode_step", "lola_peak_mfma_bf16", "lola_peak_copy",
            "lola_prefill_noalloc")
LOLA_NOALLOC_SCRATCH_BYTES = 64 << 20
LOLA_READ_STATE = 1
LOLA_READ_SPARSE = 2
LOLA_READ_WINDOW = 4
LOLA_READ_ALL = 7
SCORE_RULES = {"sre": 0, "kernel_sq": 1, "kernel_abs": 2, "ratio": 3, "attn": 4}


class LolaPhi(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("d_k", ctypes.c_int32), ("D", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("W", ctypes.c_void_p)]


class LolaState(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("d_k", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("D", ctypes.c_int32), ("eta", ctypes.c_int32),
                ("lambda_", ctypes.c_int32), ("dtype", ctypes.c_int32), ("t", ctypes.c_int64),
                ("H", ctypes.c_void_p), ("s", ctypes.c_void_p), ("win_k", ctypes.c_void_p),
                ("win_v", ctypes.c_void_p), ("cache_k", ctypes.c_void_p), ("cache_v", ctypes.c_void_p),
                ("cache_pos", ctypes.c_void_p), ("win_score", ctypes.c_void_p),
                ("cache_score", ctypes.c_void_p), ("dec_fold", ctypes.c_void_p), ("dec_chunk", ctypes.c_int32),
                ("reserved_state", ctypes.c_int32)]


LOLA_OVERLAP_EVENTS = 9


class HolaState(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("d", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("C", ctypes.c_int32), ("w", ctypes.c_int32), ("t", ctypes.c_int64),
                ("S", ctypes.c_void_p), ("cache_pos", ctypes.c_void_p), ("cache_score", ctypes.c_void_p),
                ("cache_k", ctypes.c_void_p), ("cache_v", ctypes.c_void_p), ("open_k", ctypes.c_void_p),
                ("open_v", ctypes.c_void_p), ("open_score", ctypes.c_void_p)]


class LolaOverlap(ctypes.Structure):
    _fields_ = [("stream", ctypes.c_void_p), ("events", ctypes.c_void_p * LOLA_OVERLAP_EVENTS)]


class LolaOptions(ctypes.Structure):
    _fields_ = [("read_mask", ctypes.c_int32), ("score_rule", ctypes.c_int32),
                ("decode_chunk", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("overlap", ctypes.POINTER(LolaOverlap))]


class LolaError(RuntimeError):
    def __init__(self, fn: str, code: int, text: str):
        super().__init__(f"{fn} returned {code}: {text}")
        self.code = code


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads liblola.so; raises if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m hybrid_linear_attention_chunkwise_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sp, pp = ctypes.POINTER(LolaState), ctypes.POINTER(LolaPhi)
    lib.lola_workspace_bytes.argtypes = [sp, i64, i32]
    lib.lola_workspace_bytes.restype = sz
    lib.lola_state_init.argtypes = [sp, vp]
    lib.lola_state_init.restype = i32
    lib.lola_prefill.argtypes = [sp, pp, vp, vp, vp, i64, i32, vp, vp, vp, sz, vp]
    lib.lola_prefill.restype = i32
    lib.lola_prefill_profiled.argtypes = [sp, pp, vp, vp, vp, i64, i32, vp, vp, vp, sz, vp,
                                          ctypes.POINTER(vp)]
    lib.lola_prefill_profiled.restype = i32
    lib.lola_decode_step.argtypes = [sp, pp, vp, vp, vp, vp, vp, vp]
    lib.lola_decode_step.restype = i32
    op = ctypes.POINTER(LolaOptions)
    lib.lola_prefill_ex.argtypes = [sp, pp, vp, vp, vp, i64, i32, op, vp, vp, vp, sz, vp]
    lib.lola_prefill_ex.restype = i32
    lib.lola_prefill_noalloc.argtypes = [sp, pp, vp, vp, vp, i64, i32, op, vp, vp, vp]
    lib.lola_prefill_noalloc.restype = i32
    lib.lola_decode_step_ex.argtypes = [sp, pp, vp, vp, vp, op, vp, vp, vp]
    lib.lola_decode_step_ex.restype = i32
    lib.lola_sre_collisions.argtypes = [sp, vp, vp, i64, i32, vp, sz, i32, vp, vp]
    lib.lola_sre_collisions.restype = i32
    lib.hola_workspace_bytes.argtypes = [i32, i32, i32, i32, i64, i32]
    lib.hola_workspace_bytes.restype = sz
    lib.hola_prefill.argtypes = [i32, i32, i32, i32, i64, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                 vp, vp, vp, vp, sz, vp]
    lib.hola_prefill.restype = i32
    hp = ctypes.POINTER(HolaState)
    lib.hola_state_init.argtypes = [hp, vp]
    lib.hola_state_init.restype = i32
    lib.hola_prefill_state.argtypes = [hp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hola_prefill_state.restype = i32
    lib.hola_decode_step.argtypes = [hp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.hola_decode_step.restype = i32
    lib.lola_peak_mfma_bf16.argtypes = [i32, i32, vp, vp]
    lib.lola_peak_mfma_bf16.restype = i32
    lib.lola_peak_copy.argtypes = [vp, vp, sz, vp]
    lib.lola_peak_copy.restype = i32
    lib.lola_status_string.argtypes = [i32]
    lib.lola_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().lola_status_string(code).decode()


def check(fn: str, code: int) -> None:
    if code != LOLA_OK:
        raise LolaError(fn, code, status_string(code))

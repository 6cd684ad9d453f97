"""LoLA hot path on AMD MI355X: hybrid linear attention + sliding window + SRE-scored sparse cache.

The computation lives in liblola.so (HIP kernels for gfx950 behind the C ABI of include/lola.h).
This module is its thin Python face: it owns device memory through torch tensors and marshals
pointers; the functions carry the ABI's names.  It never computes any part of the method itself.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _binding as _b
from ._binding import (LOLA_BF16, LOLA_EDEVICE, LOLA_EINVAL, LOLA_EUNSUPPORTED, LOLA_F32, LOLA_OK,
                       LOLA_PHI_ELU1, LOLA_PHI_SOFTMAX_PM, LOLA_READ_ALL, LOLA_READ_SPARSE,
                       LOLA_READ_STATE, LOLA_READ_WINDOW, SCORE_RULES, LolaError)

__all__ = ["LolaState", "LolaPhi", "LolaOverlap", "lola_state_init", "lola_workspace_bytes", "lola_prefill",
           "lola_decode_step", "lola_sre_collisions", "LolaError", "LOLA_OK", "LOLA_EINVAL", "LOLA_EUNSUPPORTED",
           "LOLA_EDEVICE", "library_path", "PHI_KINDS", "LOLA_READ_STATE", "LOLA_READ_SPARSE",
           "LOLA_READ_WINDOW", "LOLA_READ_ALL", "SCORE_RULES", "hola_workspace_bytes", "hola_prefill",
           "lola_prefill_noalloc", "HolaState", "hola_state_init", "hola_prefill_state", "hola_decode_step"]

PHI_KINDS = {"elu1": LOLA_PHI_ELU1, "softmax_pm": LOLA_PHI_SOFTMAX_PM}
_DTYPES = {torch.float32: LOLA_F32, torch.bfloat16: LOLA_BF16}


def library_path() -> str:
    return _b.LIB_PATH


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


class LolaPhi:
    """Feature map phi (kind "elu1" or "softmax_pm") with its fp32 weight W [d_k][D or D/2]."""

    def __init__(self, kind: str, W: torch.Tensor, D: int = 128):
        if W.dtype != torch.float32 or not W.is_contiguous():
            raise ValueError("W must be a contiguous float32 tensor")
        self.kind = kind
        self.W = W
        self.c = _b.LolaPhi(PHI_KINDS[kind], W.shape[0], D, 0, W.data_ptr())


class LolaState:
    """Per-layer state of B sequences x n_heads heads, allocated on `device` (see lola_state)."""

    def __init__(self, B: int, n_heads: int, d_k: int, d_v: int, D: int, eta: int, lam: int,
                 dtype: torch.dtype, device="cuda"):
        kw = dict(device=device)
        self.dtype = dtype
        self.H = torch.zeros(B, n_heads, d_v, D, dtype=torch.float32, **kw)
        self.s = torch.zeros(B, n_heads, D, dtype=torch.float32, **kw)
        self.win_k = torch.zeros(B, n_heads, max(eta, 1), d_k, dtype=dtype, **kw)
        self.win_v = torch.zeros(B, n_heads, max(eta, 1), d_v, dtype=dtype, **kw)
        self.cache_k = torch.zeros(B, n_heads, max(lam, 1), d_k, dtype=dtype, **kw)
        self.cache_v = torch.zeros(B, n_heads, max(lam, 1), d_v, dtype=dtype, **kw)
        self.cache_pos = torch.full((B, n_heads, max(lam, 1)), -1, dtype=torch.int32, **kw)
        self.win_score = torch.zeros(B, n_heads, max(eta, 1), dtype=torch.float32, **kw)
        self.cache_score = torch.zeros(B, n_heads, max(lam, 1), dtype=torch.float32, **kw)
        self.dec_fold = torch.zeros(B, n_heads, dtype=torch.int64, **kw)
        self.c = _b.LolaState(B, n_heads, d_k, d_v, D, eta, lam, _DTYPES[dtype], 0,
                              self.H.data_ptr(), self.s.data_ptr(), self.win_k.data_ptr(),
                              self.win_v.data_ptr(), self.cache_k.data_ptr(), self.cache_v.data_ptr(),
                              self.cache_pos.data_ptr(), self.win_score.data_ptr(),
                              self.cache_score.data_ptr(), self.dec_fold.data_ptr(), 0, 0)

    @property
    def t(self) -> int:
        return int(self.c.t)

    @property
    def shape(self) -> Tuple[int, int, int, int, int, int, int]:
        c = self.c
        return c.B, c.n_heads, c.d_k, c.d_v, c.D, c.eta, c.lambda_

    def snapshot(self) -> dict:
        """Device copies of every state array plus t (for restore / checkpoint)."""
        return {k: getattr(self, k).clone() for k in self._ARRAYS} | {"t": self.t, "dec_chunk": int(self.c.dec_chunk)}

    _ARRAYS = ("H", "s", "win_k", "win_v", "cache_k", "cache_v", "cache_pos", "win_score", "cache_score",
               "dec_fold")

    def restore(self, snap: dict) -> None:
        for k in self._ARRAYS:
            getattr(self, k).copy_(snap[k])
        self.c.t = snap["t"]
        self.c.dec_chunk = snap.get("dec_chunk", 0)


class LolaOverlap:
    """A second stream and its events (lola_overlap) for the overlapped prefill schedule, owned here by
    torch.  One object serves any number of calls issued one after another from one thread."""

    def __init__(self, device="cuda"):
        self.stream = torch.cuda.Stream(device=device)      # default priority
        self.events = [torch.cuda.Event() for _ in range(_b.LOLA_OVERLAP_EVENTS)]
        with torch.cuda.stream(self.stream):
            for e in self.events:
                e.record()                                    # creates the HIP event behind it
        self.c = _b.LolaOverlap(self.stream.cuda_stream,
                                (ctypes.c_void_p * _b.LOLA_OVERLAP_EVENTS)(*[e.cuda_event for e in self.events]))


def lola_workspace_bytes(state: LolaState, n_max: int, C: int) -> int:
    return int(_b.load().lola_workspace_bytes(ctypes.byref(state.c), n_max, C))


def lola_state_init(state: LolaState, stream=None) -> None:
    _b.check("lola_state_init", _b.load().lola_state_init(ctypes.byref(state.c), _stream(stream)))


def _options(read_mask: int, score_rule: str, overlap: Optional[LolaOverlap] = None, decode_chunk: int = 0):
    """ctypes options, or None for the defaults."""
    if read_mask == LOLA_READ_ALL and score_rule == "sre" and overlap is None and decode_chunk <= 1:
        return None
    ov = ctypes.pointer(overlap.c) if overlap is not None else None
    return _b.LolaOptions(read_mask, SCORE_RULES[score_rule], decode_chunk, 0, ov)


def lola_prefill(state: LolaState, phi: LolaPhi, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                 C: int, y: Optional[torch.Tensor] = None, fold_at: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, stream=None, events=None,
                 read_mask: int = LOLA_READ_ALL, score_rule: str = "sre",
                 overlap: Optional[LolaOverlap] = None):
    """Chunked prefill of q, k, v [B][h][n][d]; returns (y, fold_at).  Asynchronous on `stream`.

    ``events``: optional 5 torch.cuda.Event (created with enable_timing=True) recorded at the kernel
    boundaries: before the feature kernel, then after the feature, chain, read-out and commit kernels.
    ``read_mask`` / ``score_rule``: see lola_options (lola_prefill_ex); not combinable with events.
    ``overlap``: a LolaOverlap whose stream runs the read-out beside the allocation chain (the
    results are the same bits as without it)."""
    n = q.shape[2]
    if y is None:
        y = torch.empty(q.shape[0], q.shape[1], n, v.shape[3], dtype=v.dtype, device=v.device)
    need = lola_workspace_bytes(state, n, C)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    lib = _b.load()
    args = (ctypes.byref(state.c), ctypes.byref(phi.c), _ptr(q), _ptr(k), _ptr(v), n, C, _ptr(y),
            _ptr(fold_at), _ptr(workspace), workspace.numel(), _stream(stream))
    opts = _options(read_mask, score_rule, overlap)
    if opts is not None:
        if events is not None:
            raise ValueError("events are recorded by the default-options entry point only")
        code = lib.lola_prefill_ex(*args[:7], ctypes.byref(opts), *args[7:])
    elif events is None:
        code = lib.lola_prefill(*args)
    else:
        handles = (ctypes.c_void_p * 5)(*[None if e is None else e.cuda_event for e in events])
        code = lib.lola_prefill_profiled(*args, handles)
    _b.check("lola_prefill", code)
    return y, fold_at


def lola_prefill_noalloc(state: LolaState, phi: LolaPhi, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         C: int, y: torch.Tensor, fold_at: Optional[torch.Tensor] = None, stream=None,
                         read_mask: int = LOLA_READ_ALL, score_rule: str = "sre",
                         overlap: Optional[LolaOverlap] = None):
    """lola_prefill with the library's own per-device scratch (no workspace; nothing is allocated here
    either: y is the caller's).  Asynchronous on `stream`; returns (y, fold_at)."""
    opts = _options(read_mask, score_rule, overlap)
    code = _b.load().lola_prefill_noalloc(ctypes.byref(state.c), ctypes.byref(phi.c), _ptr(q), _ptr(k), _ptr(v),
                                          q.shape[2], C, None if opts is None else ctypes.byref(opts), _ptr(y),
                                          _ptr(fold_at), _stream(stream))
    _b.check("lola_prefill_noalloc", code)
    return y, fold_at


def lola_decode_step(state: LolaState, phi: LolaPhi, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                     y: Optional[torch.Tensor] = None, folded_pos: Optional[torch.Tensor] = None,
                     stream=None, read_mask: int = LOLA_READ_ALL, score_rule: str = "sre",
                     decode_chunk: int = 0):
    """One decode token, q, k, v [B][h][d]; returns (y, folded_pos).  Asynchronous on `stream`.
    decode_chunk > 1: chunked decode (allocation once per group of that many steps; folded_pos must
    be None)."""
    if y is None:
        y = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    lib = _b.load()
    opts = _options(read_mask, score_rule, None, decode_chunk)
    if opts is None:
        code = lib.lola_decode_step(ctypes.byref(state.c), ctypes.byref(phi.c), _ptr(q), _ptr(k),
                                    _ptr(v), _ptr(y), _ptr(folded_pos), _stream(stream))
    else:
        code = lib.lola_decode_step_ex(ctypes.byref(state.c), ctypes.byref(phi.c), _ptr(q), _ptr(k),
                                       _ptr(v), ctypes.byref(opts), _ptr(y), _ptr(folded_pos),
                                       _stream(stream))
    _b.check("lola_decode_step", code)
    return y, folded_pos


def lola_sre_collisions(state: LolaState, v: torch.Tensor, fold_at: torch.Tensor, C: int,
                        workspace: torch.Tensor, relative: bool = False,
                        out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """SRE collision map [B][h][ceil(n / C)][n] fp32 of the lola_prefill call that just ran with these
    v, fold_at, C and workspace (see include/lola.h).  Asynchronous on `stream`."""
    n = v.shape[2]
    R = (n + C - 1) // C
    if out is None:
        out = torch.empty(v.shape[0], v.shape[1], R, n, dtype=torch.float32, device=v.device)
    code = _b.load().lola_sre_collisions(ctypes.byref(state.c), _ptr(v), _ptr(fold_at), n, C,
                                         _ptr(workspace), workspace.numel(), int(bool(relative)),
                                         _ptr(out), _stream(stream))
    _b.check("lola_sre_collisions", code)
    return out


def hola_workspace_bytes(B: int, n_heads: int, d: int, dtype: torch.dtype, n: int, C: int) -> int:
    return int(_b.load().hola_workspace_bytes(B, n_heads, d, _DTYPES[dtype], n, C))


def hola_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor, beta: torch.Tensor,
                 gamma_q: torch.Tensor, gamma_k: torch.Tensor, sink: torch.Tensor, gate: torch.Tensor,
                 C: int, w: int, y: Optional[torch.Tensor] = None, S_out: Optional[torch.Tensor] = None,
                 cache_pos: Optional[torch.Tensor] = None, cache_score: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """HOLA layer call (include/lola.h) on q, k, v [B][h][n][d]; returns y.  Asynchronous on `stream`."""
    B, h, n, d = q.shape
    if y is None:
        y = torch.empty_like(v)
    need = hola_workspace_bytes(B, h, d, q.dtype, n, C)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    code = _b.load().hola_prefill(B, h, d, _DTYPES[q.dtype], n, C, w, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                  _ptr(beta), _ptr(gamma_q), _ptr(gamma_k), _ptr(sink), _ptr(gate), _ptr(y),
                                  _ptr(S_out), _ptr(cache_pos), _ptr(cache_score), _ptr(workspace),
                                  workspace.numel(), _stream(stream))
    _b.check("hola_prefill", code)
    return y


class HolaState:
    """HOLA decode memory of B sequences x n_heads heads on `device` (see hola_state): the state S, the
    persistent cache at the start of the open chunk and the open chunk's tokens."""

    def __init__(self, B: int, n_heads: int, d: int, C: int, w: int, dtype: torch.dtype, device="cuda"):
        kw = dict(device=device)
        self.dtype = dtype
        self.S = torch.zeros(B, n_heads, d, d, dtype=torch.float32, **kw)
        self.cache_pos = torch.full((B, n_heads, max(w, 1)), -1, dtype=torch.int32, **kw)
        self.cache_score = torch.zeros(B, n_heads, max(w, 1), dtype=torch.float32, **kw)
        self.cache_k = torch.zeros(B, n_heads, max(w, 1), d, dtype=dtype, **kw)
        self.cache_v = torch.zeros(B, n_heads, max(w, 1), d, dtype=dtype, **kw)
        self.open_k = torch.zeros(B, n_heads, C, d, dtype=dtype, **kw)
        self.open_v = torch.zeros(B, n_heads, C, d, dtype=dtype, **kw)
        self.open_score = torch.zeros(B, n_heads, C, dtype=torch.float32, **kw)
        self.c = _b.HolaState(B, n_heads, d, _DTYPES[dtype], C, w, 0, self.S.data_ptr(), self.cache_pos.data_ptr(),
                              self.cache_score.data_ptr(), self.cache_k.data_ptr(), self.cache_v.data_ptr(),
                              self.open_k.data_ptr(), self.open_v.data_ptr(), self.open_score.data_ptr())

    @property
    def t(self) -> int:
        return int(self.c.t)


def hola_state_init(state: HolaState, stream=None) -> None:
    _b.check("hola_state_init", _b.load().hola_state_init(ctypes.byref(state.c), _stream(stream)))


def hola_prefill_state(state: HolaState, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor,
                       beta: torch.Tensor, gamma_q: torch.Tensor, gamma_k: torch.Tensor, sink: torch.Tensor,
                       gate: torch.Tensor, y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    """hola_prefill from the empty memory `state`, leaving the decode memory in it; returns y."""
    B, h, n, d = q.shape
    if y is None:
        y = torch.empty_like(v)
    need = hola_workspace_bytes(B, h, d, q.dtype, n, state.c.C)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    code = _b.load().hola_prefill_state(ctypes.byref(state.c), n, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                        _ptr(gamma_q), _ptr(gamma_k), _ptr(sink), _ptr(gate), _ptr(y),
                                        _ptr(workspace), workspace.numel(), _stream(stream))
    _b.check("hola_prefill_state", code)
    return y


def hola_decode_step(state: HolaState, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor,
                     beta: torch.Tensor, gamma_q: torch.Tensor, gamma_k: torch.Tensor, sink: torch.Tensor,
                     gate: torch.Tensor, y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One token through the HOLA memory: q, k, v [B][h][d], alpha, beta [B][h]; returns y [B][h][d]."""
    if y is None:
        y = torch.empty_like(v)
    code = _b.load().hola_decode_step(ctypes.byref(state.c), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                      _ptr(gamma_q), _ptr(gamma_k), _ptr(sink), _ptr(gate), _ptr(y), _stream(stream))
    _b.check("hola_decode_step", code)
    return y

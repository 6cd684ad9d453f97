"""Seeded synthetic workloads for the LoLA hot path (hybrid linear attention + SRE-scored cache).

This module only draws random inputs and describes shapes. It holds none of the method's arithmetic,
so both the fp64 oracle and the GPU library can consume its arrays without sharing any compute code.

Every array is generated with ``numpy.random.default_rng(SeedSequence([cfg_id, stream]))``; streams:
0 = W (feature-map weights), 1 = q, 2 = k, 3 = v, 4 = outlier positions, 5 = planted pairs,
6 = decode tokens.  Inputs of bf16 workloads are rounded to bf16 (round-to-nearest-even) before anyone
sees them, so the oracle and the GPU consume identical values.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "round_to_bf16", "make_weights", "make_qkv", "make_inputs",
           "make_decode_tokens", "small_workload", "make_qkv_device", "make_decode_tokens_device"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    h: int
    n: int
    d_k: int
    d_v: int
    phi: str          # "elu1": elu(xW)+1, W [d_k][D];  "softmax_pm": [softmax(xW); softmax(-xW)], W [d_k][D/2]
    D: int
    C: int
    eta: int
    lam: int
    dtype: str        # "f32" or "bf16": the storage type of q/k/v/y (H, s are always fp32)
    structure: str = "iid"    # "iid", "outlier_keys", "planted_pairs"
    decode_steps: int = 0     # >0: a decode workload (n = prior context length)
    seed: int = 0

    @property
    def w_cols(self) -> int:
        return self.D if self.phi == "elu1" else self.D // 2

    @property
    def w_std(self) -> float:
        # "N(0, 1/d)" is read as variance 1/d, i.e. std 1/sqrt(d).
        return 1.0 / np.sqrt(self.d_k)


# The five workloads of the hot path (one attention layer, all heads).
WORKLOADS: Dict[int, Workload] = {
    1: Workload("n512_h1_d64_elu1_f32", B=1, h=1, n=512, d_k=64, d_v=64, phi="elu1", D=128, C=64,
                eta=64, lam=64, dtype="f32", seed=1),
    2: Workload("n4096_h32_d128_pm_outliers_bf16", B=1, h=32, n=4096, d_k=128, d_v=128,
                phi="softmax_pm", D=128, C=64, eta=256, lam=256, dtype="bf16",
                structure="outlier_keys", seed=2),
    3: Workload("b4_n16384_h32_d128_pm_bf16", B=4, h=32, n=16384, d_k=128, d_v=128,
                phi="softmax_pm", D=128, C=64, eta=256, lam=256, dtype="bf16", seed=3),
    4: Workload("decode_b64_h32_ctx8192_d128_pm_bf16", B=64, h=32, n=8192, d_k=128, d_v=128,
                phi="softmax_pm", D=128, C=64, eta=256, lam=256, dtype="bf16", decode_steps=256,
                seed=4),
    5: Workload("n131072_h8_d128_pm_planted_bf16", B=1, h=8, n=131072, d_k=128, d_v=128,
                phi="softmax_pm", D=128, C=128, eta=512, lam=512, dtype="bf16",
                structure="planted_pairs", seed=5),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32 holding bf16 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    r = ((u + bias) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def _rng(cfg_seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg_seed, stream]))


def make_weights(wl: Workload) -> np.ndarray:
    """Feature-map weights W [d_k][w_cols], fp32, shared by every batch and head."""
    W = _rng(wl.seed, 0).standard_normal((wl.d_k, wl.w_cols), dtype=np.float32) * np.float32(wl.w_std)
    return W.astype(np.float32)


def _plant_pairs(k: np.ndarray, v: np.ndarray, rng: np.random.Generator, n_pairs: int,
                 max_lag: int) -> None:
    """Copy (k, v) of a source position to source+lag, bit for bit, lag ~ U{1..max_lag}.

    Sources and targets never collide with an earlier pair (a clash is redrawn)."""
    n = k.shape[-2]
    for idx in np.ndindex(*k.shape[:-2]):
        used = set()
        placed = 0
        while placed < n_pairs:
            lag = int(rng.integers(1, max_lag + 1))
            p = int(rng.integers(0, n - lag))
            tgt = p + lag
            if p in used or tgt in used:
                continue
            used.add(p)
            used.add(tgt)
            k[idx + (tgt,)] = k[idx + (p,)]
            v[idx + (tgt,)] = v[idx + (p,)]
            placed += 1


def make_qkv(wl: Workload, n: Optional[int] = None, B: Optional[int] = None,
             h: Optional[int] = None):
    """q, k, v as float32 arrays [B][h][n][d] (bf16-representable for bf16 workloads)."""
    n = wl.n if n is None else n
    B = wl.B if B is None else B
    h = wl.h if h is None else h
    q = _rng(wl.seed, 1).standard_normal((B, h, n, wl.d_k), dtype=np.float32)
    k = _rng(wl.seed, 2).standard_normal((B, h, n, wl.d_k), dtype=np.float32)
    v = _rng(wl.seed, 3).standard_normal((B, h, n, wl.d_v), dtype=np.float32)
    if wl.structure == "outlier_keys":
        rng = _rng(wl.seed, 4)
        n_out = int(round(0.02 * n))
        for b in range(B):
            for hh in range(h):
                pos = rng.choice(n, size=n_out, replace=False)
                k[b, hh, pos, :] *= np.float32(4.0)
    if wl.dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    if wl.structure == "planted_pairs":
        _plant_pairs(k, v, _rng(wl.seed, 5), n_pairs=min(1024, n // 4), max_lag=min(65536, n // 2))
    return q, k, v


def make_decode_tokens(wl: Workload, B: Optional[int] = None, h: Optional[int] = None,
                       steps: Optional[int] = None):
    """Decode-step tokens q, k, v [steps][B][h][d] (one token per sequence and head per step)."""
    B = wl.B if B is None else B
    h = wl.h if h is None else h
    steps = wl.decode_steps if steps is None else steps
    rng = _rng(wl.seed, 6)
    q = rng.standard_normal((steps, B, h, wl.d_k), dtype=np.float32)
    k = rng.standard_normal((steps, B, h, wl.d_k), dtype=np.float32)
    v = rng.standard_normal((steps, B, h, wl.d_v), dtype=np.float32)
    if wl.dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return q, k, v


def make_inputs(cfg_id: int, **overrides):
    """(workload, W, q, k, v) for one of the five configurations; keyword overrides shrink B/h/n."""
    wl = WORKLOADS[cfg_id]
    q, k, v = make_qkv(wl, n=overrides.get("n"), B=overrides.get("B"), h=overrides.get("h"))
    return wl, make_weights(wl), q, k, v


def small_workload(seed: int, *, B=1, h=2, n=200, d_k=64, d_v=64, phi="softmax_pm", D=128, C=16,
                   eta=24, lam=20, dtype="f32", structure="iid") -> Workload:
    """A small workload for parity tests (several tiles and a ragged tail)."""
    return Workload(f"small_s{seed}", B=B, h=h, n=n, d_k=d_k, d_v=d_v, phi=phi, D=D, C=C, eta=eta,
                    lam=lam, dtype=dtype, structure=structure, seed=1000 + seed)


def _torch_gen(wl: Workload, stream: int, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence([wl.seed, stream, 7]).generate_state(1)[0]))
    return g


def make_qkv_device(wl: Workload, device, dtype, n: Optional[int] = None, B: Optional[int] = None,
                    h: Optional[int] = None):
    """Device-side seeded N(0, 1) q, k, v [B][h][n][d] in `dtype` (for workloads too large to draw on
    the host, such as the 8192-token prior context of the decode workload).  Consumers that need
    host copies (the oracle) copy these tensors back."""
    import torch
    n = wl.n if n is None else n
    B = wl.B if B is None else B
    h = wl.h if h is None else h
    out = []
    for stream, d in ((11, wl.d_k), (12, wl.d_k), (13, wl.d_v)):
        g = _torch_gen(wl, stream, device)
        out.append(torch.randn((B, h, n, d), generator=g, device=device, dtype=torch.float32).to(dtype))
    return tuple(out)


def make_decode_tokens_device(wl: Workload, device, dtype, steps: Optional[int] = None):
    """Device-side seeded decode tokens q, k, v [steps][B][h][d] in `dtype`."""
    import torch
    steps = wl.decode_steps if steps is None else steps
    out = []
    for stream, d in ((16, wl.d_k), (17, wl.d_k), (18, wl.d_v)):
        g = _torch_gen(wl, stream, device)
        out.append(torch.randn((steps, wl.B, wl.h, d), generator=g, device=device,
                               dtype=torch.float32).to(dtype))
    return tuple(out)

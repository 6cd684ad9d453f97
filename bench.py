#!/usr/bin/env python3
"""Throughput of the LoLA hot path on one MI355X; prints one JSON line.

Headline step: one chunked prefill of the largest single-GPU prefill workload, 4 sequences x 32 heads
x 16384 tokens, d = 128, bf16 (softmax-pair feature map, C = 64, eta = lambda = 256), from a freshly
initialised state, with the read-out overlapped on a second stream.  Also measured: the 32-head
n = 4096 workload with 2% outlier keys, the 8-head n = 131072 workload with planted pairs (C = 128,
eta = lambda = 512), 256 decode steps of 64 sequences x 32 heads after an 8192-token prior context, the
device's attainable bf16 matrix rate and copy bandwidth, and the fp64 CPU oracle on a bounded sample
of the headline workload.

Inputs are seeded synthetic data resident in device memory before timing starts.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill tokens/s and decode tokens/s per GPU; % of MFMA / HBM roofline"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_MFMA_TFLOPS = 157.3  # MI355X dense fp32 matrix (and fp32 vector)
PEAK_HBM_GBS = 8000.0
MULTI_TOKEN_C = 16          # tokens per call in the multi-token decode measurement
# The sources each measured kernel is built from (shared headers included): a counter figure stays
# valid until one of them changes.
_SHARED_SOURCES = ("lola_common.hpp", "lola_internal.hpp")
KERNEL_SOURCES = {
    "phi": ("lola_phi.hip",),
    "chain": ("lola_chain_fast.hip", "lola_chain.hip"),
    "readout": ("lola_readout.hip", "lola_readout_fast.hip", "lola_readout_common.hpp"),
    "commit": ("lola_readout.hip",),
    "decode": ("lola_decode_fast.hip", "lola_decode.hip"),
    "decode_group": ("lola_decode_group.hip",),
    "collide": ("lola_collide.hip",),
    "qscore": ("lola_qscore.hip",),
    "hola": ("lola_hola.hip",),
}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash(kernel: str = None) -> str:
    """Hash of the sources one kernel is built from (all kernel sources if none is named)."""
    if kernel is None:
        files = sorted({f for fs in KERNEL_SOURCES.values() for f in fs})
    else:
        files = list(KERNEL_SOURCES[kernel])
    h = hashlib.sha256()
    for f in _SHARED_SOURCES + tuple(files):
        with open(os.path.join(ROOT, "hybrid_linear_attention_chunkwise_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def prefill_flops(wl) -> dict:
    """Algorithmic FLOPs per launch of each prefill kernel (per token and head, times B*h*n).

    Per token and head: features of the key (feature kernel) and of the query (read-out), 2 d_k D_W
    each; the exact branch 2 (d_k + d_v)(eta + lambda) (an upper bound: a query reads at most eta + lambda
    exact keys); the linear read 2 D (d_v + 1); the intra-chunk fold term (D + d_v + 1)(C + 1); SRE
    scoring of the C + lambda candidates of a chunk, 2 D (d_v + 1)(C + lambda) / C; the fold 2 D (d_v + 1).
    The chain kernel does the scoring and the fold, the read-out the rest but the key features."""
    dw = wl.D if wl.phi == "elu1" else wl.D // 2
    phi = 2 * wl.d_k * dw
    chain = 2 * wl.D * (wl.d_v + 1) * (wl.C + wl.lam) / wl.C + 2 * wl.D * (wl.d_v + 1)
    readout = (phi + 2 * (wl.d_k + wl.d_v) * (wl.eta + wl.lam) + 2 * wl.D * (wl.d_v + 1)
               + (wl.D + wl.d_v + 1) * (wl.C + 1))
    units = wl.B * wl.h * wl.n
    return {"phi": phi * units, "chain": chain * units, "readout": readout * units,
            "per_token_head": phi + chain + readout, "total": (phi + chain + readout) * units}


def decode_bytes_per_seq_head(wl) -> int:
    """Minimum HBM bytes one decode step moves per (sequence, head) under the natural layout."""
    esz = 2 if wl.dtype == "bf16" else 4
    H = 2 * wl.D * wl.d_v * 4
    s = 2 * wl.D * 4
    window = wl.eta * (wl.d_k + wl.d_v) * esz
    cache = wl.lam * (wl.d_k + wl.d_v) * esz
    writes = (wl.d_k + wl.d_v) * esz * 2
    io = (2 * wl.d_k + wl.d_v) * esz + wl.d_v * esz
    return H + s + window + cache + writes + io


def load_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it matches the source.

    The summary's table has one row per kernel: name, workload, grid, launches, FETCH_SIZE KiB,
    WRITE_SIZE KiB, calibrated bytes per launch, and the hash of that kernel's sources.  A row taken
    from other sources than the current ones is stale and ignored.
    """
    src_hash = kernel_source_hash(kernel)
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            cols = [c.strip() for c in line.strip().strip("|").split("|")]
            if len(cols) == 8 and cols[0] == kernel and cols[7] == src_hash:
                return int(cols[6])
    return None


def bench_prefill(args, lola, torch, wl, steps=None, warmup=None, kernel_steps=20):
    """Whole-prefill timing of one workload, then per-kernel timing.

    Timed region: `steps` back-to-back steps, each a state reset (lola_state_init) and one overlapped
    prefill call, bracketed by synchronisations (wall clock).  HIP events on the caller's stream around
    each prefill call alone (the reset excluded) give the per-call median and minimum.  A second pass
    runs the sequential schedule with events between its kernels (lola_prefill_profiled) for the
    per-kernel durations; every kernel there is launched on the caller's stream."""
    import statistics
    from workloads import make_qkv, make_weights
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    W = make_weights(wl)
    q, k, v = make_qkv(wl)
    qt = torch.from_numpy(q).to(dev).to(tdt)
    kt = torch.from_numpy(k).to(dev).to(tdt)
    vt = torch.from_numpy(v).to(dev).to(tdt)
    del q, k, v
    st = lola.LolaState(wl.B, wl.h, wl.d_k, wl.d_v, wl.D, wl.eta, wl.lam, tdt, device=dev)
    phi = lola.LolaPhi(wl.phi, torch.from_numpy(W).to(dev), wl.D)
    y = torch.empty_like(vt)
    ws = torch.empty(lola.lola_workspace_bytes(st, wl.n, wl.C), dtype=torch.uint8, device=dev)
    ov = lola.LolaOverlap(dev)
    log(f"prefill {wl.name}: inputs resident, {warmup} warm-up + {steps} timed steps")

    def step(e0=None, e1=None):
        lola.lola_state_init(st)
        if e0 is not None:
            e0.record()
        lola.lola_prefill(st, phi, qt, kt, vt, wl.C, y=y, workspace=ws, overlap=ov)
        if e1 is not None:
            e1.record()

    for _ in range(warmup):
        step()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(*evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    call_ms = [a.elapsed_time(b) for a, b in evs]
    # per-kernel durations: sequential schedule with events between the kernels (same stream)
    kev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    for e in kev:
        e.record()                      # creates the HIP events the library records into
    kern = {"phi": 0.0, "chain": 0.0, "readout": 0.0, "commit": 0.0}
    for _ in range(kernel_steps):
        lola.lola_state_init(st)
        lola.lola_prefill(st, phi, qt, kt, vt, wl.C, y=y, workspace=ws, events=kev)
        kev[4].synchronize()
        for i, name in enumerate(("phi", "chain", "readout", "commit")):
            kern[name] += kev[i].elapsed_time(kev[i + 1])
    kern = {k_: v_ / kernel_steps for k_, v_ in kern.items()}   # ms per launch
    med, mn = statistics.median(call_ms), min(call_ms)
    log(f"prefill {wl.name}: {elapsed / steps * 1e3:.3f} ms/step wall, prefill call median {med:.3f} ms, "
        f"min {mn:.3f} ms; kernels ms (sequential): {kern}")
    del qt, kt, vt, y, ws
    return {"elapsed": elapsed, "steps": steps, "call_ms_median": med, "call_ms_min": mn, "kernels_ms": kern}


def prefill_report(wl, r) -> dict:
    """Throughput and roofline figures of one prefill workload from bench_prefill's timings."""
    fl = prefill_flops(wl)
    kern = r["kernels_ms"]
    tokens = wl.B * wl.n
    out = {"workload": wl.name, "tokens_per_s": round(tokens * r["steps"] / r["elapsed"], 1),
           "ms_per_step": round(r["elapsed"] / r["steps"] * 1e3, 4),
           "prefill_call_ms": {"median": round(r["call_ms_median"], 4), "min": round(r["call_ms_min"], 4),
                               "runs": r["steps"]},
           "kernels_ms_sequential": {k_: round(v_, 4) for k_, v_ in kern.items()}}
    fr = {}
    for name in ("chain", "readout"):
        ach = fl[name] / (kern[name] * 1e-3) / 1e12
        fr[name] = {"achieved_tflops": round(ach, 3), "frac": round(ach / PEAK_BF16_TFLOPS, 5),
                    "algorithmic_flop_per_launch": fl[name], "kernel_ms": round(kern[name], 4)}
    out["kernel_fractions"] = fr
    out["mfma_frac_whole_step"] = round(fl["total"] / (r["call_ms_median"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 5)
    out["algorithmic_flop_per_step"] = fl["total"]
    return out


def bench_collisions(args, lola, torch, wl):
    """SRE collision map of one prefill call of the workload (every token against every chunk-end
    state): one prefill, then the map timed on its own.  Algorithmic flops: 2 D d_v per map entry whose
    token is in the state (the recall H^T phi(k)); the normaliser and the norm are not counted."""
    import numpy as np
    from workloads import make_qkv, make_weights
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    W = make_weights(wl)
    q, k, v = make_qkv(wl)
    qt, kt, vt = (torch.from_numpy(x).to(dev).to(tdt) for x in (q, k, v))
    st = lola.LolaState(wl.B, wl.h, wl.d_k, wl.d_v, wl.D, wl.eta, wl.lam, tdt, device=dev)
    phi = lola.LolaPhi(wl.phi, torch.from_numpy(W).to(dev), wl.D)
    ws = torch.empty(lola.lola_workspace_bytes(st, wl.n, wl.C), dtype=torch.uint8, device=dev)
    fold = torch.empty(wl.B, wl.h, wl.n, dtype=torch.int32, device=dev)
    lola.lola_state_init(st)
    lola.lola_prefill(st, phi, qt, kt, vt, wl.C, fold_at=fold, workspace=ws)
    R = (wl.n + wl.C - 1) // wl.C
    out = torch.empty(wl.B, wl.h, R, wl.n, dtype=torch.float32, device=dev)
    fa = fold.cpu().numpy().astype(np.int64)
    entries = int(np.where(fa >= 0, R - fa, 0).sum())
    for _ in range(args.warmup):
        lola.lola_sre_collisions(st, vt, fold, wl.C, ws, out=out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        lola.lola_sre_collisions(st, vt, fold, wl.C, ws, out=out)
    e1.record()
    e1.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    flop = 2.0 * wl.D * wl.d_v * entries
    ach = flop / (ms * 1e-3) / 1e12
    log(f"collision map: {ms:.4f} ms, {entries} entries in the state of {wl.B * wl.h * R * wl.n}, "
        f"{ach:.1f} TFLOP/s")
    return {"kernel": "lola_collide", "workload": wl.name, "rows": R, "kernel_ms": round(ms, 4),
            "entries_in_state": entries, "entries_total": wl.B * wl.h * R * wl.n,
            "roofline": {"bound": "mfma", "achieved": round(ach, 3), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 5),
                         "traffic": load_traffic("collide"),
                         "algorithmic_flop_per_launch": flop}}


def bench_options(args, lola, torch, wl):
    """Whole-step prefill time of the workload under other lola_options: each query-accumulated
    scoring rule (score kernel + chain ranking by the sums) and the read masks (window only; window
    and cache).  Same step as the headline: state init + one prefill call, K back-to-back steps."""
    from workloads import make_qkv, make_weights
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    W = make_weights(wl)
    q, k, v = make_qkv(wl)
    qt, kt, vt = (torch.from_numpy(x).to(dev).to(tdt) for x in (q, k, v))
    st = lola.LolaState(wl.B, wl.h, wl.d_k, wl.d_v, wl.D, wl.eta, wl.lam, tdt, device=dev)
    phi = lola.LolaPhi(wl.phi, torch.from_numpy(W).to(dev), wl.D)
    y = torch.empty_like(vt)
    ws = torch.empty(lola.lola_workspace_bytes(st, wl.n, wl.C), dtype=torch.uint8, device=dev)
    ov = lola.LolaOverlap(dev)
    out = {}
    cases = [(r, lola.LOLA_READ_ALL) for r in ("kernel_sq", "kernel_abs", "ratio", "attn")]
    cases += [("sre", lola.LOLA_READ_WINDOW), ("sre", lola.LOLA_READ_WINDOW | lola.LOLA_READ_SPARSE)]
    for rule, mask in cases:
        def step():
            lola.lola_state_init(st)
            lola.lola_prefill(st, phi, qt, kt, vt, wl.C, y=y, workspace=ws, read_mask=mask, score_rule=rule,
                              overlap=ov)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / args.steps * 1e3
        name = rule if mask == lola.LOLA_READ_ALL else ("read_window" if mask == lola.LOLA_READ_WINDOW
                                                         else "read_window_cache")
        out[name] = {"ms_per_step": round(ms, 4), "tokens_per_s": round(wl.B * wl.n / (ms * 1e-3), 1)}
    log(f"options: {out}")
    return out


HOLA_W, HOLA_C = 64, 256     # the HOLA page's persistent cache and chunk


def bench_hola(args, lola, torch, B, h, n, d):
    """The HOLA variant (hola_prefill) with the page's w = 64 and C = 256 on B x h heads of n tokens and
    head dimension d, bf16: K back-to-back layer calls on resident seeded inputs.  The delta rule's
    algorithmic work is three d x d matrix-vector products per token and head (prediction S^T k, the
    write k e^T, the read-out S^T q): 6 d^2 fp32 FLOP.  It runs on fp32 MFMA in blocks of 16 tokens, so
    it is priced against the fp32 matrix peak."""
    import numpy as np
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(20)
    q, k, v = (torch.from_numpy(rng.standard_normal((B, h, n, d)).astype(np.float32)).to(dev).to(torch.bfloat16)
               for _ in range(3))
    alpha = torch.from_numpy(rng.uniform(0.9, 1.0, (B, h, n)).astype(np.float32)).to(dev)
    beta = torch.from_numpy(rng.uniform(0.0, 1.0, (B, h, n)).astype(np.float32)).to(dev)
    gq = torch.from_numpy(rng.uniform(0.5, 1.5, (h, d)).astype(np.float32)).to(dev)
    gk = torch.from_numpy(rng.uniform(0.5, 1.5, (h, d)).astype(np.float32)).to(dev)
    sink = torch.zeros(h, device=dev)
    gate = torch.full((h,), -4.0, device=dev)                 # the page's gate initialisation
    y = torch.empty_like(v)
    ws = torch.empty(lola.hola_workspace_bytes(B, h, d, torch.bfloat16, n, HOLA_C), dtype=torch.uint8, device=dev)

    def call():
        lola.hola_prefill(q, k, v, alpha, beta, gq, gk, sink, gate, HOLA_C, HOLA_W, y=y, workspace=ws)
    for _ in range(max(1, args.warmup)):
        call()
    torch.cuda.synchronize()
    steps = max(1, args.steps // 4)
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    flop = 6.0 * d * d * B * h * n
    ach = flop / (ms * 1e-3) / 1e12
    log(f"hola: {ms:.3f} ms/call")
    return {"workload": f"hola_n{n}_h{h}_d{d}_w{HOLA_W}_C{HOLA_C}_bf16", "ms_per_call": round(ms, 4),
            "tokens_per_s": round(B * n / (ms * 1e-3), 1),
            "roofline": {"bound": "mfma", "kernel": "hola (whole call)", "achieved": round(ach, 3),
                         "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(ach / PEAK_FP32_MFMA_TFLOPS, 5), "algorithmic_flop_per_call": flop}}


def bench_hola_decode(args, lola, torch, B, h, n0, d, steps=64, runs=3):
    """HOLA decode (hola_decode_step) after an untimed hola_prefill_state of n0 tokens, with the page's
    w = 64 and C = 256, bf16: each run restores the post-prefill memory (untimed) and times `steps`
    single-token steps with HIP events on the calling stream.  HBM-bound: per (sequence, head, step) the
    step reads and writes the fp32 state (8 d^2 bytes), reads the cached rows and the open chunk's rows
    (keys and values) and the token, writes y and the token's open row."""
    import numpy as np
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(21)
    bf = torch.bfloat16
    mk = lambda *shape: torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(dev).to(bf)
    q, k, v = mk(B, h, n0, d), mk(B, h, n0, d), mk(B, h, n0, d)
    alpha = torch.from_numpy(rng.uniform(0.9, 1.0, (B, h, n0)).astype(np.float32)).to(dev)
    beta = torch.from_numpy(rng.uniform(0.0, 1.0, (B, h, n0)).astype(np.float32)).to(dev)
    gq = torch.from_numpy(rng.uniform(0.5, 1.5, (h, d)).astype(np.float32)).to(dev)
    gk = torch.from_numpy(rng.uniform(0.5, 1.5, (h, d)).astype(np.float32)).to(dev)
    sink = torch.zeros(h, device=dev)
    gate = torch.full((h,), -4.0, device=dev)
    tq, tk, tv = mk(steps, B, h, d), mk(steps, B, h, d), mk(steps, B, h, d)
    ta = torch.from_numpy(rng.uniform(0.9, 1.0, (steps, B, h)).astype(np.float32)).to(dev)
    tb = torch.from_numpy(rng.uniform(0.0, 1.0, (steps, B, h)).astype(np.float32)).to(dev)
    st = lola.HolaState(B, h, d, HOLA_C, HOLA_W, bf, device=dev)
    lola.hola_state_init(st)
    lola.hola_prefill_state(st, q, k, v, alpha, beta, gq, gk, sink, gate)
    torch.cuda.synchronize()
    del q, k, v, alpha, beta
    names = ("S", "cache_pos", "cache_score", "cache_k", "cache_v", "open_k", "open_v", "open_score")
    snap = {nm: getattr(st, nm).clone() for nm in names}
    y = torch.empty(B, h, d, dtype=bf, device=dev)
    times = []
    for r in range(runs + 1):
        for nm in names:
            getattr(st, nm).copy_(snap[nm])
        st.c.t = n0
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            lola.hola_decode_step(st, tq[i], tk[i], tv[i], ta[i], tb[i], gq, gk, sink, gate, y=y)
        e1.record()
        torch.cuda.synchronize()
        if r > 0:                                             # the first run warms up
            times.append(e0.elapsed_time(e1) / steps)
    ms = float(np.median(times))
    nopen_avg = n0 % HOLA_C + (steps - 1) / 2.0
    nv = min(HOLA_W, n0 - n0 % HOLA_C)
    per = 8 * d * d + (nv + nopen_avg) * 2 * d * 2 + 6 * d * 2 + 8 * d + 32
    byts = per * B * h
    ach = byts / (ms * 1e-3) / 1e9
    log(f"hola decode: {ms:.4f} ms/step")
    return {"workload": f"hola_decode_b{B}_h{h}_ctx{n0}_d{d}_w{HOLA_W}_C{HOLA_C}_bf16", "ms_per_step": round(ms, 4),
            "tokens_per_s": round(B / (ms * 1e-3), 1), "steps": steps,
            "roofline": {"bound": "hbm", "kernel": "hola_decode", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                         "algorithmic_bytes_per_step": round(byts)}}


def bench_decode(args, lola, torch, wl):
    """256 single-token decode steps of every (sequence, head) after the untimed prior context; each run
    restores the same post-prefill snapshot (untimed) and times the steps with HIP events on the caller's
    stream, one event per step boundary (per-step kernel time) and the wall clock around the run.  Then
    the same tokens in prefill calls of MULTI_TOKEN_C tokens (allocation once per call)."""
    import statistics
    from workloads import make_decode_tokens_device, make_qkv_device, make_weights
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    W = make_weights(wl)
    st = lola.LolaState(wl.B, wl.h, wl.d_k, wl.d_v, wl.D, wl.eta, wl.lam, tdt, device=dev)
    phi = lola.LolaPhi(wl.phi, torch.from_numpy(W).to(dev), wl.D)
    lola.lola_state_init(st)
    # prior context, untimed, in two prefill calls
    part = wl.n // 2
    ws = torch.empty(lola.lola_workspace_bytes(st, part, wl.C), dtype=torch.uint8, device=dev)
    qp, kp, vp = make_qkv_device(wl, dev, tdt)
    for s0 in (0, part):
        lola.lola_prefill(st, phi, qp[:, :, s0:s0 + part].contiguous(), kp[:, :, s0:s0 + part].contiguous(),
                          vp[:, :, s0:s0 + part].contiguous(), wl.C, workspace=ws)
    del qp, kp, vp, ws
    torch.cuda.synchronize()
    snap = st.snapshot()
    dq, dk, dv = make_decode_tokens_device(wl, dev, tdt)
    y = torch.empty(wl.B, wl.h, wl.d_v, dtype=tdt, device=dev)
    steps = wl.decode_steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    walls, kerns = [], []
    for run in range(args.decode_runs + 1):      # first run is warm-up
        st.restore(snap)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(steps):
            evs[s].record()
            lola.lola_decode_step(st, phi, dq[s], dk[s], dv[s], y=y)
        evs[steps].record()
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        if run > 0:
            walls.append(el)
            kerns.append(sum(evs[s].elapsed_time(evs[s + 1]) for s in range(steps)) / steps)
    wall = statistics.median(walls)
    kern_ms = statistics.median(kerns)
    log(f"decode: {wall / steps * 1e3:.3f} ms/step wall (median of {len(walls)} runs), kernel {kern_ms:.4f} ms/step "
        f"(min {min(kerns):.4f})")
    # multi-token decode: the same tokens in calls of C_DEC tokens (allocation once per call)
    c_dec = MULTI_TOKEN_C
    calls = steps // c_dec
    parts = [tuple(torch.stack([x[s] for s in range(c * c_dec, (c + 1) * c_dec)], dim=2).contiguous()
                   for x in (dq, dk, dv)) for c in range(calls)]
    ws_m = torch.empty(lola.lola_workspace_bytes(st, c_dec, c_dec), dtype=torch.uint8, device=dev)
    ym = torch.empty(wl.B, wl.h, c_dec, wl.d_v, dtype=tdt, device=dev)
    walls_m = []
    for run in range(args.decode_runs + 1):
        st.restore(snap)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for mq, mk, mv in parts:
            lola.lola_prefill(st, phi, mq, mk, mv, c_dec, y=ym, workspace=ws_m)
        torch.cuda.synchronize()
        if run > 0:
            walls_m.append(time.perf_counter() - t0)
    best_m = statistics.median(walls_m)
    log(f"multi-token decode ({c_dec} tokens per call): {best_m / calls * 1e3:.3f} ms/call")
    multi = {"value": round(wl.B * calls * c_dec / best_m, 1), "unit": "decode tokens/s", "tokens_per_call": c_dec,
             "ms_per_call": round(best_m / calls * 1e3, 4)}
    # chunked decode: the same single-token steps with the allocation once per group of C_DEC steps
    walls_c, kerns_c = [], []
    for run in range(args.decode_runs + 1):
        st.restore(snap)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(steps):
            evs[s].record()
            lola.lola_decode_step(st, phi, dq[s], dk[s], dv[s], y=y, decode_chunk=c_dec)
        evs[steps].record()
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        if run > 0:
            walls_c.append(el)
            kerns_c.append(sum(evs[s].elapsed_time(evs[s + 1]) for s in range(steps)) / steps)
    wall_c, kern_c = statistics.median(walls_c), statistics.median(kerns_c)
    log(f"chunked decode (groups of {c_dec} steps): {wall_c / steps * 1e3:.3f} ms/step wall, kernel "
        f"{kern_c:.4f} ms/step")
    chunked = {"value": round(wl.B * steps / wall_c, 1), "unit": "decode tokens/s", "decode_chunk": c_dec,
               "kernel_ms_per_step": round(kern_c, 5), "kernel_ms_per_step_min": round(min(kerns_c), 5),
               "ms_per_step_wall": round(wall_c / steps * 1e3, 4)}
    return {"wall": wall, "kern_ms": kern_ms, "kern_ms_min": min(kerns), "runs": len(walls), "multi": multi,
            "chunked": chunked}


def bench_peaks(lola, torch):
    """The device's attainable dense bf16 matrix rate (an MFMA loop from registers) and streaming copy
    bandwidth (a 4 GiB device-to-device copy), each the best of several event-timed launches."""
    import ctypes
    lib = lola._b.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    wgs, iters = 8 * torch.cuda.get_device_properties(dev).multi_processor_count, 2048
    out = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
    flop = wgs * 4 * 4 * iters * 32768.0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = None
    for i in range(6):
        e0.record()
        lola._b.check("lola_peak_mfma_bf16", lib.lola_peak_mfma_bf16(wgs, iters, ctypes.c_void_p(out.data_ptr()), stream))
        e1.record()
        e1.synchronize()
        if i > 0:
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
    mfma = flop / (best * 1e-3) / 1e12
    nbytes = 4 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    bestc = None
    for i in range(6):
        e0.record()
        lola._b.check("lola_peak_copy", lib.lola_peak_copy(src.data_ptr(), dst.data_ptr(), nbytes, stream))
        e1.record()
        e1.synchronize()
        if i > 0:
            ms = e0.elapsed_time(e1)
            bestc = ms if bestc is None else min(bestc, ms)
    copy = 2.0 * nbytes / (bestc * 1e-3) / 1e9
    del src, dst
    log(f"peaks: bf16 MFMA loop {mfma:.1f} TFLOP/s ({best:.3f} ms), copy {copy:.1f} GB/s ({bestc:.3f} ms)")
    return {"mfma_bf16_tflops": round(mfma, 1), "copy_gbs": round(copy, 1),
            "mfma_loop": f"{wgs} workgroups x 4 waves x {4 * iters} v_mfma_f32_32x32x16_bf16 per wave, best of 5",
            "copy": f"{nbytes} bytes read + written, 16-byte pieces, best of 5",
            "vendor": {"mfma_bf16_tflops": PEAK_BF16_TFLOPS, "hbm_gbs": PEAK_HBM_GBS}}


def _oracle_head(job):
    import numpy as np
    from oracle import lola_oracle as O
    phi = O.make_phi(job["phi"], job["W"])
    st = O.new_state(job["q"].shape[1], job["v"].shape[1], job["D"], job["eta"], job["lam"])
    O.prefill(st, phi, job["q"].astype(np.float64), job["k"].astype(np.float64),
              job["v"].astype(np.float64), job["C"])
    return True


def cpu_baseline(wl, heads: int):
    """The fp64 oracle, as it stands, on `heads` full (sequence, head) pairs of the headline workload,
    one pair per worker process with BLAS pinned to one thread in each."""
    import concurrent.futures
    import multiprocessing
    from workloads import make_qkv, make_weights
    heads = min(heads, wl.B * wl.h)
    W = make_weights(wl)
    bsel = max(1, min(wl.B, (heads + wl.h - 1) // wl.h))
    q, k, v = make_qkv(wl, B=bsel)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    workers = max(1, min(16, cores, heads))
    pairs = [(b, h) for b in range(bsel) for h in range(wl.h)][:heads]
    jobs = [dict(phi=wl.phi, W=W, q=q[b, h], k=k[b, h], v=v[b, h], C=wl.C, eta=wl.eta, lam=wl.lam, D=wl.D)
            for (b, h) in pairs]
    # spawned workers inherit these before they import numpy: one BLAS thread per worker
    pinned = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS")
    saved = {key: os.environ.get(key) for key in pinned}
    for key in pinned:
        os.environ[key] = "1"
    try:
        ctx = multiprocessing.get_context("spawn")
        with concurrent.futures.ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as ex:
            list(ex.map(_oracle_head, [dict(jobs[0], q=jobs[0]["q"][:8], k=jobs[0]["k"][:8], v=jobs[0]["v"][:8])] * workers))
            t0 = time.perf_counter()
            list(ex.map(_oracle_head, jobs))
            wall = time.perf_counter() - t0
    finally:
        for key, val in saved.items():
            if val is None:
                os.environ.pop(key, None)
            else:
                os.environ[key] = val
    layer_tokens = wl.B * wl.n * heads / (wl.B * wl.h)        # tokens of the whole layer this sample equals
    return {"value": round(layer_tokens / wall, 2), "unit": "prefill tokens/s", "cores": workers, "kind": "oracle",
            "host_cores": cores, "workers": workers, "blas_threads_per_worker": 1,
            "wall_s": round(wall, 2), "core_seconds": round(wall * workers, 1),
            "sample": f"{heads} of {wl.B * wl.h} (sequence, head) pairs of {wl.name}, full n = {wl.n} each, "
                      f"fp64 numpy, {workers} worker processes with one BLAS thread each on {cores} host cores; "
                      f"value = {wl.B * wl.n} * {heads}/{wl.B * wl.h} layer tokens / {wall:.2f} s wall"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100, help="timed steps of the headline prefill")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--leg-steps", type=int, default=20, help="timed steps of the other prefill legs")
    ap.add_argument("--decode-runs", type=int, default=10)
    ap.add_argument("--headline", type=int, default=3, choices=(2, 3, 5), help="workload of the headline line")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-legs", action="store_true", help="skip the other prefill workloads")
    ap.add_argument("--no-collisions", action="store_true")
    ap.add_argument("--no-options", action="store_true")
    ap.add_argument("--no-hola", action="store_true")
    ap.add_argument("--no-peaks", action="store_true")
    ap.add_argument("--only-hola", action="store_true", help="only the HOLA legs (prefill, d = 256, decode)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: every (sequence, head) is independent, so a multi-GPU "
              "run is N copies of this one; run it with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import hybrid_linear_attention_chunkwise_amd as lola
    from workloads import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    lola._b.load()
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        lola._b.check("lola_peak_copy", lola._b.load().lola_peak_copy(src.data_ptr(), dst.data_ptr(), n * 4,
                                                                     torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4}))
        return 0
    src_hash = kernel_source_hash()
    if args.only_hola:
        hw = WORKLOADS[2]
        r = bench_hola(args, lola, torch, hw.B, hw.h, hw.n, hw.d_k)
        r["d256"] = bench_hola(args, lola, torch, 1, 4, hw.n, 256)
        r["decode"] = bench_hola_decode(args, lola, torch, 32, hw.h, 4196, hw.d_k)
        print(json.dumps({"hola": r}))
        return 0
    if args.no_prefill:        # profiling mode: the decode workload only
        dwl = WORKLOADS[4]
        r = bench_decode(args, lola, torch, dwl)
        print(json.dumps({"decode_ms_per_step": r["wall"] / dwl.decode_steps * 1e3, "decode_kernel_ms": r["kern_ms"]}))
        return 0
    wl = WORKLOADS[args.headline]
    head = prefill_report(wl, bench_prefill(args, lola, torch, wl))
    kern = head["kernels_ms_sequential"]
    dominant = max(("chain", "readout"), key=lambda k_: kern[k_])
    fr = head["kernel_fractions"][dominant]
    roofline = {"bound": "mfma", "kernel": f"lola_{dominant}", "achieved": fr["achieved_tflops"],
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": fr["frac"],
                "traffic": load_traffic(dominant), "kernel_ms": fr["kernel_ms"],
                "algorithmic_flop_per_launch": fr["algorithmic_flop_per_launch"]}
    out = {"metric": METRIC, "value": head["tokens_per_s"], "unit": "prefill tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic: seeded N(0,1) q/k/v rounded to bf16, seeded N(0, 1/d_k) feature weights",
           "config": {"workload": wl.name, "B": wl.B, "heads": wl.h, "n": wl.n, "d_k": wl.d_k,
                      "d_v": wl.d_v, "D": wl.D, "phi": wl.phi, "C": wl.C, "eta": wl.eta, "lambda": wl.lam},
           "roofline": roofline,
           "prefill_call_ms": head["prefill_call_ms"],
           "kernels_ms": kern,
           "kernel_fractions": head["kernel_fractions"],
           "prefill_mfma_frac_whole_step": head["mfma_frac_whole_step"],
           "algorithmic_flop_per_step": head["algorithmic_flop_per_step"],
           "kernel_source_hash": src_hash}
    if not args.no_peaks:
        pk = bench_peaks(lola, torch)
        pk["roofline_frac_vs_measured"] = round(roofline["achieved"] / pk["mfma_bf16_tflops"], 5)
        out["peaks_measured"] = pk
    if not args.no_legs:
        legs = {}
        for cid in (2, 3, 5):
            if cid == args.headline:
                continue
            lw = WORKLOADS[cid]
            legs[lw.name] = prefill_report(lw, bench_prefill(args, lola, torch, lw, steps=args.leg_steps,
                                                             warmup=max(2, args.warmup // 2), kernel_steps=5))
        out["prefill_legs"] = legs
    if not args.no_decode:
        dwl = WORKLOADS[4]
        r = bench_decode(args, lola, torch, dwl)
        per_step = r["wall"] / dwl.decode_steps
        byts = decode_bytes_per_seq_head(dwl) * dwl.B * dwl.h
        ach_d = byts / (r["kern_ms"] * 1e-3) / 1e9
        out["decode"] = {"value": round(dwl.B * dwl.decode_steps / r["wall"], 1), "unit": "decode tokens/s",
                         "workload": dwl.name, "ms_per_step": round(per_step * 1e3, 4), "runs": r["runs"],
                         "roofline": {"bound": "hbm", "kernel": "lola_decode", "achieved": round(ach_d, 1),
                                      "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach_d / PEAK_HBM_GBS, 4),
                                      "traffic": load_traffic("decode"), "kernel_ms": round(r["kern_ms"], 4),
                                      "kernel_ms_min": round(r["kern_ms_min"], 4),
                                      "algorithmic_bytes_per_launch": byts},
                         "multi_token": r["multi"], "chunked": r["chunked"]}
        if "peaks_measured" in out:
            out["decode"]["roofline"]["frac_vs_measured_copy"] = round(ach_d / out["peaks_measured"]["copy_gbs"], 4)
    import argparse as _ap
    leg_args = _ap.Namespace(**{**vars(args), "steps": args.leg_steps, "warmup": max(2, args.warmup // 2)})
    if not args.no_collisions:
        out["collision_map"] = bench_collisions(leg_args, lola, torch, WORKLOADS[2])
    if not args.no_options:
        out["options"] = bench_options(leg_args, lola, torch, WORKLOADS[2])
    if not args.no_hola:
        hw = WORKLOADS[2]
        out["hola"] = bench_hola(leg_args, lola, torch, hw.B, hw.h, hw.n, hw.d_k)
        # the HOLA page's own setup: 4 heads of dimension 256
        out["hola"]["d256"] = bench_hola(leg_args, lola, torch, 1, 4, hw.n, 256)
        # decode after a 4196-token prefill (an open chunk of 100 tokens), 32 sequences x 32 heads
        out["hola"]["decode"] = bench_hola_decode(leg_args, lola, torch, 32, hw.h, 4196, hw.d_k)
    if not args.no_cpu_baseline:
        log("cpu baseline: running the oracle ...")
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_heads)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

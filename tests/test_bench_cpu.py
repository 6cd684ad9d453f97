"""Host-side pieces of bench.py, without a GPU: the helpers the timed legs call, the counter-summary
lookup keyed to each kernel's sources, and the refusal of a multi-GPU run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_helpers_exist_and_hashes_are_per_kernel():
    import bench
    for name in ("log", "kernel_source_hash", "load_traffic", "prefill_flops", "decode_bytes_per_seq_head",
                 "bench_prefill", "bench_decode", "bench_hola", "main"):
        assert callable(getattr(bench, name)), name
    bench.log("bench helpers: log works")
    hs = {k: bench.kernel_source_hash(k) for k in bench.KERNEL_SOURCES}
    assert all(len(h) == 16 for h in hs.values())
    assert hs["readout"] != hs["commit"]                      # the read-out also covers its bf16 kernel
    assert len({hs[k] for k in ("phi", "chain", "readout", "decode", "decode_group", "hola")}) == 6
    assert len(bench.kernel_source_hash()) == 16


def test_traffic_rows_match_current_sources_or_are_ignored():
    """A row of the committed counter summary is used only while its hash names the current sources."""
    import bench
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    rows = {}
    with open(path) as f:
        for line in f:
            cols = [c.strip() for c in line.strip().strip("|").split("|")]
            if len(cols) == 8 and cols[0] in bench.KERNEL_SOURCES:
                rows[cols[0]] = cols
    assert {"chain", "readout", "decode"} <= set(rows)
    for k, cols in rows.items():
        got = bench.load_traffic(k)
        if cols[7] == bench.kernel_source_hash(k):
            assert got == int(cols[6])
        else:
            assert got is None


def test_multi_gpu_request_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "gpus 1" in r.stderr


def test_flop_model_matches_the_scope_table():
    """The algorithmic work per token and head at the 128-dimensional workloads (C = 64,
    eta = lambda = 256): features 2 x 2 d D/2, exact branch 2 (d_k + d_v)(eta + lambda), linear read
    2 D (d_v + 1), intra-chunk term (D + d_v + 1)(C + 1), scoring 2 D (d_v + 1)(C + lambda) / C and fold
    2 D (d_v + 1) add up to 542,785 FLOP; the chain kernel's share is the scoring and the fold."""
    import bench
    from workloads import WORKLOADS
    for cid in (2, 3):
        fl = bench.prefill_flops(WORKLOADS[cid])
        assert fl["per_token_head"] == 542785
        units = WORKLOADS[cid].B * WORKLOADS[cid].h * WORKLOADS[cid].n
        assert fl["chain"] == (165120 + 33024) * units
        assert abs(fl["phi"] + fl["chain"] + fl["readout"] - fl["total"]) < 1

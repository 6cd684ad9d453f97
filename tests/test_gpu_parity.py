"""GPU parity: liblola.so (through its C ABI) against the fp64 oracle on the same seeded inputs.

Small cases span several tiles and a ragged tail; edge cases cover empty input, lambda = 0, eta = 0,
eta >= n, n < C, C = 1 and continuation calls.  Tolerances are in tests/lola_testlib.py.
"""
import numpy as np
import pytest

import lola_testlib as TL
from workloads import make_decode_tokens, make_qkv, make_weights, small_workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import hybrid_linear_attention_chunkwise_amd as lola
    lola._b.load()   # fails loudly if the library is missing


def _jobs(wl, W, q, k, v, fold, heads, tol):
    jobs = []
    for (b, h) in heads:
        jobs.append(dict(phi=wl.phi, W=W, q=q[b, h].astype(np.float64), k=k[b, h].astype(np.float64),
                         v=v[b, h].astype(np.float64), C=wl.C, eta=wl.eta, lam=wl.lam, D=wl.D,
                         fold_at_gpu=fold[b, h].astype(np.int64), tol=tol))
    return jobs


def _check_workload(wl, heads=None, chunks=None):
    W = make_weights(wl)
    q, k, v = make_qkv(wl)
    print(f"[parity] {wl.name} B={wl.B} h={wl.h} n={wl.n} d={wl.d_k} C={wl.C} eta={wl.eta} "
          f"lam={wl.lam} {wl.dtype}", flush=True)
    y, fold, state, _ = TL.gpu_run_prefill(q, k, v, W, wl.phi, wl.eta, wl.lam, wl.C, wl.dtype,
                                           D=wl.D, chunks=chunks)
    host = TL.state_to_host(state)
    assert np.isfinite(y).all()
    if heads is None:
        heads = [(b, h) for b in range(wl.B) for h in range(wl.h)]
    tol = TL.TIE_BAND if wl.dtype == "f32" else TL.BF16_TOL
    if chunks is not None:
        # fold_at of a call only covers that call's own tokens (call-local chunk ids): translate the
        # oracle's one-call schedule into what each call must report, then grade against the oracle.
        results = TL.run_oracle_heads(_jobs(wl, W, q, k, v, fold, heads, tol))
        for (b, h), res in zip(heads, results):
            exp = np.full(wl.n, -1, dtype=np.int64)
            start = 0
            for ln in chunks:
                c_lo, c_hi = start // wl.C, (start + ln + wl.C - 1) // wl.C
                for i in range(start, start + ln):
                    c = res["fold_at_oracle"][i]
                    if c_lo <= c < c_hi:
                        exp[i] = c - c_lo
                start += ln
            assert np.array_equal(exp, fold[b, h]), "per-call fold schedule differs"
            assert TL.row_rel_err(y[b, h], res["y_oracle"]) <= TL.FP32_TOL
            assert TL.cache_members(host["cache_pos"][b, h]) == res["cache_oracle"]
        return None, y, fold, host
    results = TL.run_oracle_heads(_jobs(wl, W, q, k, v, fold, heads, tol))
    reps = []
    for (b, h), res in zip(heads, results):
        rep = TL.grade_prefill(res, y[b, h], fold[b, h], wl.dtype,
                               cache_gpu=TL.cache_members(host["cache_pos"][b, h]) if wl.lam > 0 else None)
        same = rep["schedule_identical"]
        Href = res["H_oracle"] if same else res["H_replay"]
        sref = res["s_oracle"] if same else res["s_replay"]
        hs_tol = 1e-4 if wl.dtype == "f32" else 2e-2
        scale = max(1.0, float(np.abs(Href).max()))
        assert np.abs(host["H"][b, h].T - Href).max() <= hs_tol * scale
        assert np.abs(host["s"][b, h] - sref).max() <= hs_tol * max(1.0, float(np.abs(sref).max()))
        reps.append(rep)
    print(f"[parity] {wl.name}: max err {max(r['max_row_rel_err'] for r in reps):.3e}, "
          f"identical schedules {sum(r['schedule_identical'] for r in reps)}/{len(reps)}", flush=True)
    return reps, y, fold, host


SMALL_CASES = [
    # (seed, kwargs)
    (1, dict(n=200, C=16, eta=24, lam=20)),                         # several chunks, ragged tail
    (2, dict(n=333, C=64, eta=64, lam=64, d_k=64, d_v=64)),        # cfg1-like tile shape, ragged
    (3, dict(n=150, C=32, eta=40, lam=0)),                          # lambda = 0 (window + linear)
    (4, dict(n=90, C=8, eta=0, lam=0)),                             # pure linear attention
    (5, dict(n=70, C=1, eta=0, lam=5)),                             # eta = 0 needs C = 1
    (6, dict(n=120, C=16, eta=200, lam=10)),                        # eta >= n: exact softmax
    (7, dict(n=40, C=64, eta=64, lam=16)),                          # n < C
    (8, dict(n=260, C=32, eta=31, lam=48, phi="elu1")),             # eta = C - 1, elu feature map
    (9, dict(n=300, C=64, eta=100, lam=37, d_k=128, d_v=128)),      # d = 128, odd lambda
    (10, dict(n=97, C=5, eta=7, lam=9)),                            # tiny chunks
]


@pytest.mark.parametrize("seed,kw", SMALL_CASES, ids=[f"s{s}" for s, _ in SMALL_CASES])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_small_prefill(seed, kw, dtype):
    kw = dict(kw)
    kw.setdefault("d_k", 64)
    kw.setdefault("d_v", kw["d_k"])
    wl = small_workload(seed, B=2, h=2, dtype=dtype, **kw)
    _check_workload(wl)


def test_outlier_keys_and_planted_pairs_small():
    wl = small_workload(20, B=1, h=2, n=400, C=32, eta=48, lam=40, d_k=128, d_v=128, dtype="f32",
                        structure="outlier_keys")
    _check_workload(wl)
    wl = small_workload(21, B=1, h=2, n=400, C=32, eta=48, lam=40, d_k=128, d_v=128, dtype="f32",
                        structure="planted_pairs")
    _check_workload(wl)


LARGEST_CASES = [
    # the largest cache (lambda = 1024) and chunk (C = 128) the library accepts; the cache fills after
    # eta + lambda tokens, so the last chunks each select among lambda + C candidates
    (90, dict(n=1700, C=128, eta=128, lam=1024, d_k=128, d_v=128)),   # d = 128, ragged last chunk
    (91, dict(n=1500, C=128, eta=127, lam=1024, d_k=64, d_v=64)),     # d = 64, eta = C - 1
]


@pytest.mark.parametrize("seed,kw", LARGEST_CASES, ids=[f"s{s}" for s, _ in LARGEST_CASES])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_at_the_largest_cache_and_chunk(seed, kw, dtype):
    wl = small_workload(seed, B=1, h=2, dtype=dtype, **kw)
    _check_workload(wl)


@pytest.mark.parametrize("split", [[64, 136], [32, 32, 96, 40], [192, 8]])
def test_continuation_calls_equal_one_call(split):
    wl = small_workload(30, B=1, h=2, n=200, C=16, eta=24, lam=20, dtype="f32")
    _check_workload(wl, chunks=split)


def test_empty_call_is_noop():
    import hybrid_linear_attention_chunkwise_amd as lola
    st = lola.LolaState(1, 1, 64, 64, 128, 8, 4, torch.float32)
    lola.lola_state_init(st)
    W = torch.zeros(64, 64, device="cuda")
    phi = lola.LolaPhi("softmax_pm", W)
    e = torch.zeros(1, 1, 0, 64, device="cuda")
    y, _ = lola.lola_prefill(st, phi, e, e, e, 4)
    assert st.t == 0 and y.numel() == 0


def test_invalid_arguments_leave_state_untouched():
    import hybrid_linear_attention_chunkwise_amd as lola
    wl = small_workload(40, B=1, h=2, n=64, C=16, eta=20, lam=10, dtype="f32")
    W = make_weights(wl)
    q, k, v = make_qkv(wl)
    _, _, st, phi = TL.gpu_run_prefill(q, k, v, W, wl.phi, wl.eta, wl.lam, wl.C, "f32")
    before = TL.state_to_host(st)
    qt = torch.from_numpy(q).cuda()
    with pytest.raises(lola.LolaError) as ei:           # chunk too long for the window (lam > 0)
        lola.lola_prefill(st, phi, qt, qt, qt, 64)
    assert ei.value.code == lola.LOLA_EINVAL
    with pytest.raises(lola.LolaError) as ei:           # workspace too small
        lola.lola_prefill(st, phi, qt, qt, qt, 16, workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))
    assert ei.value.code == lola.LOLA_EINVAL
    bad = lola.LolaPhi("softmax_pm", torch.zeros(32, 64, device="cuda"))
    with pytest.raises(lola.LolaError):
        lola.lola_prefill(st, bad, qt, qt, qt, 16)
    after = TL.state_to_host(st)
    for key in before:
        assert np.array_equal(np.asarray(before[key]), np.asarray(after[key])), key


def test_prefill_is_deterministic():
    wl = small_workload(41, B=2, h=2, n=180, C=16, eta=24, lam=20, dtype="bf16")
    W = make_weights(wl)
    q, k, v = make_qkv(wl)
    y1, f1, _, _ = TL.gpu_run_prefill(q, k, v, W, wl.phi, wl.eta, wl.lam, wl.C, "bf16")
    y2, f2, _, _ = TL.gpu_run_prefill(q, k, v, W, wl.phi, wl.eta, wl.lam, wl.C, "bf16")
    assert np.array_equal(y1, y2) and np.array_equal(f1, f2)


def _decode_check(wl, n0, steps, heads, C0, read_mask=7):
    """Prefill n0 tokens, then `steps` decode tokens; oracle continues from the GPU's post-prefill
    state and must reproduce every decode output and fold.  read_mask applies to the decode steps."""
    import hybrid_linear_attention_chunkwise_amd as lola
    from oracle import lola_oracle as O
    W = make_weights(wl)
    q, k, v = make_qkv(wl, n=n0)
    tdt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    _, _, st, phi = TL.gpu_run_prefill(q, k, v, W, wl.phi, wl.eta, wl.lam, C0, wl.dtype, D=wl.D)
    snap = TL.state_to_host(st)
    dq, dk, dv = make_decode_tokens(wl, steps=steps)
    ys, folds = [], []
    for s in range(steps):
        fp = torch.full((wl.B, wl.h), -7, dtype=torch.int32, device="cuda")
        y, _ = lola.lola_decode_step(st, phi, torch.from_numpy(dq[s]).cuda().to(tdt),
                                     torch.from_numpy(dk[s]).cuda().to(tdt),
                                     torch.from_numpy(dv[s]).cuda().to(tdt), folded_pos=fp,
                                     read_mask=read_mask)
        ys.append(y.float())
        folds.append(fp)
    torch.cuda.synchronize()
    ys = torch.stack(ys).cpu().numpy()
    folds = torch.stack(folds).cpu().numpy()
    phi_o = O.make_phi(wl.phi, W)
    worst, mism = 0.0, 0
    for (b, h) in heads:
        so = O.state_from_arrays(snap["t"], wl.eta, wl.lam, snap["H"][b, h].T, snap["s"][b, h],
                                 snap["win_k"][b, h], snap["win_v"][b, h], snap["cache_k"][b, h],
                                 snap["cache_v"][b, h], snap["cache_pos"][b, h])
        rep = TL.grade_decode_steps(so, phi_o, dq[:, b, h], dk[:, b, h], dv[:, b, h], ys[:, b, h],
                                    folds[:, b, h], wl.dtype, read_mask=read_mask)
        worst = max(worst, rep["max_row_rel_err"])
        mism += rep["fold_mismatches"]
    print(f"[decode] {wl.name}: max err {worst:.3e}, fold mismatches {mism} (all {steps} steps graded "
          f"per head)", flush=True)
    return worst


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_steps_small(dtype):
    wl = small_workload(50, B=2, h=2, n=0, C=1, eta=16, lam=12, d_k=64, d_v=64, dtype=dtype)
    _decode_check(wl, n0=48, steps=40, heads=[(0, 0), (1, 1)], C0=16)


def test_decode_from_empty_state_eta0():
    wl = small_workload(51, B=1, h=2, n=0, C=1, eta=0, lam=6, d_k=64, d_v=64, dtype="f32")
    _decode_check(wl, n0=1, steps=30, heads=[(0, 0), (0, 1)], C0=1)


def test_decode_equals_prefill_c1():
    """n decode steps from an empty state = prefill with C = 1 (same kernels' semantics)."""
    import hybrid_linear_attention_chunkwise_amd as lola
    wl = small_workload(52, B=1, h=2, n=60, C=1, eta=8, lam=6, d_k=64, d_v=64, dtype="f32")
    W = make_weights(wl)
    q, k, v = make_qkv(wl)
    y_p, f_p, _, _ = TL.gpu_run_prefill(q, k, v, W, wl.phi, wl.eta, wl.lam, 1, "f32")
    st = lola.LolaState(1, 2, 64, 64, 128, wl.eta, wl.lam, torch.float32)
    lola.lola_state_init(st)
    phi = lola.LolaPhi(wl.phi, torch.from_numpy(W).cuda())
    ys = []
    for t in range(wl.n):
        y, _ = lola.lola_decode_step(st, phi, torch.from_numpy(q[:, :, t]).cuda().contiguous(),
                                     torch.from_numpy(k[:, :, t]).cuda().contiguous(),
                                     torch.from_numpy(v[:, :, t]).cuda().contiguous())
        ys.append(y)
    y_d = torch.stack(ys, dim=2).cpu().numpy()
    assert TL.row_rel_err(y_d, y_p) <= 1e-5


@pytest.mark.parametrize("path", ["register", "general"])
def test_decode_bf16_d128_both_kernels(path, monkeypatch):
    """bf16 decode at d = 128 through the register-resident kernel and through the general one
    (forced by LOLA_DECODE_GENERAL), each against the oracle."""
    if path == "general":
        monkeypatch.setenv("LOLA_DECODE_GENERAL", "1")
    else:
        monkeypatch.delenv("LOLA_DECODE_GENERAL", raising=False)
    wl = small_workload(53, B=2, h=2, n=0, C=1, eta=24, lam=20, d_k=128, d_v=128, dtype="bf16")
    _decode_check(wl, n0=72, steps=40, heads=[(0, 1), (1, 0)], C0=16)


def test_decode_bf16_cache_beyond_register_path():
    """A cache too large for the register-resident decode kernel (lambda + 1 > 384) takes the
    general kernel automatically."""
    wl = small_workload(54, B=1, h=2, n=0, C=1, eta=32, lam=400, d_k=128, d_v=128, dtype="bf16")
    _decode_check(wl, n0=480, steps=24, heads=[(0, 0), (0, 1)], C0=32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_at_the_largest_cache(dtype):
    """Decode with the largest cache the library accepts (lambda = 1024, d = 128): every step scores
    lambda + 1 candidates through the general decode kernel."""
    wl = small_workload(92, B=1, h=2, n=0, C=1, eta=128, lam=1024, d_k=128, d_v=128, dtype=dtype)
    _decode_check(wl, n0=1300, steps=16, heads=[(0, 0), (0, 1)], C0=128)


def test_overlapped_prefill_equals_sequential():
    """The overlapped schedule (read-out of finished chunk ranges on the caller's second stream) gives
    the same bits as the sequential one, with and without kernel-boundary events."""
    import hybrid_linear_attention_chunkwise_amd as lola
    wl = small_workload(55, B=2, h=3, n=700, C=16, eta=24, lam=20, dtype="bf16")
    W = make_weights(wl)
    q, k, v = make_qkv(wl)
    dev = torch.device("cuda:0")
    phi = lola.LolaPhi(wl.phi, torch.from_numpy(W).to(dev))
    qt, kt, vt = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (q, k, v))
    ov = lola.LolaOverlap(dev)
    outs = []
    for mode in ("overlap", "profiled", "plain"):
        st = lola.LolaState(wl.B, wl.h, wl.d_k, wl.d_v, wl.D, wl.eta, wl.lam, torch.bfloat16, device=dev)
        lola.lola_state_init(st)
        fold = torch.full((wl.B, wl.h, wl.n), -7, dtype=torch.int32, device=dev)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)] if mode == "profiled" else None
        y, _ = lola.lola_prefill(st, phi, qt, kt, vt, wl.C, fold_at=fold, events=ev,
                                 overlap=ov if mode == "overlap" else None)
        torch.cuda.synchronize()
        outs.append((y.float().cpu().numpy(), fold.cpu().numpy(), TL.state_to_host(st)))
    for y1, f1, s1 in outs[1:]:
        y0, f0, s0 = outs[0]
        assert np.array_equal(y0, y1) and np.array_equal(f0, f1)
        for key in s0:
            assert np.array_equal(np.asarray(s0[key]), np.asarray(s1[key])), key


def test_two_states_two_threads_two_streams():
    """Two states, each driven from its own host thread on its own stream with its own overlap block,
    two calls each (a fresh state, then a continuation), reproduce the bits of the same calls made one
    after another on one stream.  Nothing is shared between the two callers but the library."""
    import threading
    import hybrid_linear_attention_chunkwise_amd as lola
    dev = torch.device("cuda:0")
    wls = [small_workload(57, B=1, h=2, n=640, C=16, eta=24, lam=20, dtype="bf16"),
           small_workload(58, B=2, h=1, n=640, C=16, eta=24, lam=20, dtype="bf16")]
    inputs = []
    for wl in wls:
        W = make_weights(wl)
        q, k, v = make_qkv(wl)
        inputs.append((lola.LolaPhi(wl.phi, torch.from_numpy(W).to(dev)),
                       *(torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (q, k, v))))

    def run(i, stream, overlap):
        wl = wls[i]
        phi, qt, kt, vt = inputs[i]
        with torch.cuda.stream(stream):
            st = lola.LolaState(wl.B, wl.h, wl.d_k, wl.d_v, wl.D, wl.eta, wl.lam, torch.bfloat16, device=dev)
            lola.lola_state_init(st, stream=stream)
            ys = []
            for lo, hi in ((0, 320), (320, 640)):
                y, _ = lola.lola_prefill(st, phi, qt[:, :, lo:hi].contiguous(), kt[:, :, lo:hi].contiguous(),
                                         vt[:, :, lo:hi].contiguous(), wl.C, stream=stream, overlap=overlap)
                ys.append(y)
            stream.synchronize()
            return torch.cat(ys, dim=2).float().cpu().numpy(), TL.state_to_host(st)

    ref = [run(i, torch.cuda.current_stream(), None) for i in range(2)]
    got = [None, None]
    streams = [torch.cuda.Stream(device=dev) for _ in range(2)]
    ovs = [lola.LolaOverlap(dev) for _ in range(2)]

    def worker(i):
        got[i] = run(i, streams[i], ovs[i])
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    for i in range(2):
        assert got[i] is not None
        assert np.array_equal(ref[i][0], got[i][0])
        for key in ref[i][1]:
            assert np.array_equal(np.asarray(ref[i][1][key]), np.asarray(got[i][1][key])), key


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("c_dec", [4, 8])
def test_multi_token_decode_calls(dtype, c_dec):
    """Multi-token decode: a live state (full window and cache) takes short prefill calls of c_dec
    tokens with C = c_dec, so the allocation runs once per c_dec tokens.  Each call is checked
    against the oracle continuing from the GPU's state before that call (so a bf16 near-tie in one
    call cannot shift the next), output by output, and in fp32 also the resulting cache."""
    import hybrid_linear_attention_chunkwise_amd as lola
    from oracle import lola_oracle as O
    wl = small_workload(56, B=1, h=2, n=0, C=c_dec, eta=24, lam=20, d_k=64, d_v=64, dtype=dtype)
    W = make_weights(wl)
    n0, calls = 64, 6
    q, k, v = make_qkv(wl, n=n0 + calls * c_dec)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    _, _, st, phi = TL.gpu_run_prefill(q[:, :, :n0], k[:, :, :n0], v[:, :, :n0], W, wl.phi, wl.eta,
                                       wl.lam, 16, dtype, D=wl.D)
    phi_o = O.make_phi(wl.phi, W)
    tol = TL.FP32_TOL if dtype == "f32" else TL.BF16_TOL
    worst = 0.0
    for call in range(calls):
        lo, hi = n0 + call * c_dec, n0 + (call + 1) * c_dec
        snap = TL.state_to_host(st)
        qc, kc, vc = (np.ascontiguousarray(x[:, :, lo:hi]) for x in (q, k, v))
        y, _ = lola.lola_prefill(st, phi, *(torch.from_numpy(x).cuda().to(tdt) for x in (qc, kc, vc)), c_dec)
        y = y.float().cpu().numpy()
        after = TL.state_to_host(st)
        for h in range(wl.h):
            so = O.state_from_arrays(snap["t"], wl.eta, wl.lam, snap["H"][0, h].T, snap["s"][0, h],
                                     snap["win_k"][0, h], snap["win_v"][0, h], snap["cache_k"][0, h],
                                     snap["cache_v"][0, h], snap["cache_pos"][0, h])
            y_o, _ = O.prefill(so, phi_o, qc[0, h], kc[0, h], vc[0, h], C=c_dec)
            worst = max(worst, TL.row_rel_err(y[0, h], y_o))
            if dtype == "f32":
                assert TL.cache_members(after["cache_pos"][0, h]) == sorted(so.cache)
    print(f"[multi-token decode] {dtype} c_dec={c_dec}: max err {worst:.3e}", flush=True)
    assert worst <= tol


# ------------------------------------------------------------------------------------------------
# SRE collision map (lola_sre_collisions) against the oracle's map under the GPU's schedule.
# ------------------------------------------------------------------------------------------------

def collision_check(wl, heads, relative_modes=(False, True)):
    """Runs lola_prefill with a kept workspace, then the collision map in each mode, and compares
    every entry with the oracle's map (sre_collisions replaying the GPU's fold schedule).

    Zero entries (tokens not yet in a state) must match exactly.  Other entries: |gpu - oracle| <=
    tol * (||v_i|| + max_r SRE_r(i)), tol the output tolerance of the storage type (1e-4 fp32, 2e-2
    bf16); an SRE is a distance to v_i, so an error in the recall moves it by at most that much."""
    import hybrid_linear_attention_chunkwise_amd as lola
    from oracle import lola_oracle as O
    W = make_weights(wl)
    q, k, v = make_qkv(wl)
    dev = torch.device("cuda:0")
    tdt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    print(f"[collisions] {wl.name} B={wl.B} h={wl.h} n={wl.n} d={wl.d_k} C={wl.C} eta={wl.eta} "
          f"lam={wl.lam} {wl.dtype}", flush=True)
    st = lola.LolaState(wl.B, wl.h, wl.d_k, wl.d_v, wl.D, wl.eta, wl.lam, tdt, device=dev)
    lola.lola_state_init(st)
    phi = lola.LolaPhi(wl.phi, torch.from_numpy(W).to(dev), wl.D)
    qt, kt, vt = (torch.from_numpy(x).to(dev).to(tdt) for x in (q, k, v))
    ws = torch.empty(max(lola.lola_workspace_bytes(st, wl.n, wl.C), 256), dtype=torch.uint8, device=dev)
    fold = torch.full((wl.B, wl.h, wl.n), -7, dtype=torch.int32, device=dev)
    lola.lola_prefill(st, phi, qt, kt, vt, wl.C, fold_at=fold, workspace=ws)
    maps = {}
    for rel in relative_modes:
        maps[rel] = lola.lola_sre_collisions(st, vt, fold, wl.C, ws, relative=rel).cpu().numpy()
    fold_h = fold.cpu().numpy()
    R = (wl.n + wl.C - 1) // wl.C
    tol = TL.FP32_TOL if wl.dtype == "f32" else TL.BF16_TOL
    phi_o = O.make_phi(wl.phi, W)
    worst = 0.0
    for (b, h) in heads:
        args = (phi_o, q[b, h].astype(np.float64), k[b, h].astype(np.float64), v[b, h].astype(np.float64), wl.C)
        ref = {}
        for rel in sorted(set(relative_modes) | {False}):
            st_o = O.new_state(wl.d_k, wl.d_v, wl.D, wl.eta, wl.lam)
            ref[rel], _, sched = O.sre_collisions(st_o, *args, fold_at_in=fold_h[b, h].astype(np.int64),
                                                  tol=1.0, relative=rel)
        scale = np.linalg.norm(v[b, h].astype(np.float64), axis=1) + ref[False].max(axis=0)
        for rel in relative_modes:
            got = maps[rel][b, h]
            assert got.shape == (R, wl.n)
            assert np.isfinite(got).all()
            fa = fold_h[b, h][None, :]
            zero = ~((fa >= 0) & (fa <= np.arange(R)[:, None]))
            assert np.array_equal(got[zero], np.zeros(zero.sum())), "entries outside the state must be 0"
            err = float((np.abs(got - ref[rel]) / scale[None, :]).max()) if got.size else 0.0
            worst = max(worst, err)
            assert err <= tol, f"head ({b},{h}) relative={rel}: error {err:.3e} > {tol}"
    print(f"[collisions] {wl.name}: max scaled error {worst:.3e}", flush=True)
    return worst


COLLIDE_CASES = [
    (60, dict(n=300, C=16, eta=24, lam=20)),                        # window + cache, ragged last chunk
    (61, dict(n=1100, C=64, eta=64, lam=64)),                       # several token blocks, ragged block
    (62, dict(n=90, C=8, eta=0, lam=0)),                            # pure linear: in from its own chunk
    (63, dict(n=120, C=16, eta=200, lam=10)),                       # eta >= n: nothing folded, all 0
    (64, dict(n=530, C=32, eta=40, lam=0, d_k=128, d_v=128)),       # d = 128, window only
    (65, dict(n=70, C=1, eta=0, lam=5)),                            # C = 1: one row per token
]


@pytest.mark.parametrize("seed,kw", COLLIDE_CASES, ids=[f"s{s}" for s, _ in COLLIDE_CASES])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sre_collisions_small(seed, kw, dtype):
    wl = small_workload(seed, B=1, h=2, dtype=dtype, **kw)
    collision_check(wl, [(0, 0), (0, 1)])


def test_sre_collisions_rejects_bad_arguments():
    import hybrid_linear_attention_chunkwise_amd as lola
    wl = small_workload(66, B=1, h=1, n=64, C=16, eta=24, lam=20, dtype="f32")
    dev = torch.device("cuda:0")
    st = lola.LolaState(wl.B, wl.h, wl.d_k, wl.d_v, wl.D, wl.eta, wl.lam, torch.float32, device=dev)
    lola.lola_state_init(st)
    vt = torch.zeros(1, 1, 64, 64, device=dev)
    fold = torch.full((1, 1, 64), -1, dtype=torch.int32, device=dev)
    need = lola.lola_workspace_bytes(st, 64, 16)
    small_ws = torch.empty(need - 256, dtype=torch.uint8, device=dev)
    with pytest.raises(lola.LolaError) as e:
        lola.lola_sre_collisions(st, vt, fold, 16, small_ws)
    assert e.value.code == lola.LOLA_EINVAL
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    out = lola.lola_sre_collisions(st, vt, fold, 16, ws)   # nothing folded: all zeros
    assert torch.count_nonzero(out).item() == 0


# ------------------------------------------------------------------------------------------------
# Read-branch masks (lola_prefill_ex / lola_decode_step_ex): the query reads only some memories.
# ------------------------------------------------------------------------------------------------

READ_MASKS = [("window", 4), ("state_window", 5), ("sparse_window", 6)]


@pytest.mark.parametrize("mname,mask", READ_MASKS, ids=[m for m, _ in READ_MASKS])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_read_masks_prefill(mname, mask, dtype):
    """Masked prefill: the allocation is the unmasked one (same fold schedule, bit for bit) and the
    outputs match the oracle's masked read-out under that schedule."""
    import hybrid_linear_attention_chunkwise_amd as lola
    from oracle import lola_oracle as O
    wl = small_workload(70, B=1, h=2, n=260, C=16, eta=24, lam=20, dtype=dtype)
    W = make_weights(wl)
    q, k, v = make_qkv(wl)
    dev = torch.device("cuda:0")
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    phi = lola.LolaPhi(wl.phi, torch.from_numpy(W).to(dev))
    qt, kt, vt = (torch.from_numpy(x).to(dev).to(tdt) for x in (q, k, v))
    res = {}
    for m in (7, mask):
        st = lola.LolaState(wl.B, wl.h, wl.d_k, wl.d_v, wl.D, wl.eta, wl.lam, tdt, device=dev)
        lola.lola_state_init(st)
        fold = torch.full((wl.B, wl.h, wl.n), -7, dtype=torch.int32, device=dev)
        y, _ = lola.lola_prefill(st, phi, qt, kt, vt, wl.C, fold_at=fold, read_mask=m)
        torch.cuda.synchronize()
        res[m] = (y.float().cpu().numpy(), fold.cpu().numpy(), TL.state_to_host(st))
    y, fold, host = res[mask]
    assert np.array_equal(fold, res[7][1]) and np.array_equal(host["cache_pos"], res[7][2]["cache_pos"])
    phi_o = O.make_phi(wl.phi, W)
    worst = 0.0
    for h in range(wl.h):
        so = O.new_state(wl.d_k, wl.d_v, wl.D, wl.eta, wl.lam)
        y_o, _ = O.prefill(so, phi_o, q[0, h].astype(np.float64), k[0, h].astype(np.float64),
                           v[0, h].astype(np.float64), wl.C, fold_at_in=fold[0, h].astype(np.int64), tol=1.0,
                           read_mask=mask)
        worst = max(worst, TL.row_rel_err(y[0, h], y_o))
    print(f"[read mask] prefill {mname} {dtype}: max err {worst:.3e}", flush=True)
    assert worst <= (TL.FP32_TOL if dtype == "f32" else TL.BF16_TOL)


@pytest.mark.parametrize("mname,mask", READ_MASKS, ids=[m for m, _ in READ_MASKS])
@pytest.mark.parametrize("path", ["register", "general"])
def test_read_masks_decode(mname, mask, path, monkeypatch):
    """Masked decode through both bf16 decode kernels, against the oracle from the GPU's state."""
    if path == "general":
        monkeypatch.setenv("LOLA_DECODE_GENERAL", "1")
    else:
        monkeypatch.delenv("LOLA_DECODE_GENERAL", raising=False)
    wl = small_workload(71, B=1, h=2, n=0, C=1, eta=24, lam=20, d_k=128, d_v=128, dtype="bf16")
    _decode_check(wl, n0=72, steps=24, heads=[(0, 0), (0, 1)], C0=16, read_mask=mask)


def test_read_mask_decode_f32():
    wl = small_workload(72, B=1, h=2, n=0, C=1, eta=16, lam=12, d_k=64, d_v=64, dtype="f32")
    _decode_check(wl, n0=48, steps=30, heads=[(0, 0), (0, 1)], C0=16, read_mask=6)


# ------------------------------------------------------------------------------------------------
# Query-accumulated cache-scoring rules (lola_prefill_ex with lola_options.score_rule).
# ------------------------------------------------------------------------------------------------

SCORE_RULES = ["kernel_sq", "kernel_abs", "ratio", "attn"]
# fp32 validity tolerance of a schedule under these rules: a score is a sum of up to eta terms, each
# with an exponential good to a few ulp, summed in fp32 in another order than the oracle's fp64.
QSCORE_FP32_TOL = 1e-4


def _score_rule_check(wl, rule, heads, calls=None):
    """GPU prefill (one call, or consecutive calls of the given lengths) under a scoring rule against
    the oracle's single call: identical schedule, or (near-ties) a schedule the oracle validates with
    the tolerance of the dtype, then outputs and the carried scores."""
    import hybrid_linear_attention_chunkwise_amd as lola
    from oracle import lola_oracle as O
    W = make_weights(wl)
    q, k, v = make_qkv(wl)
    dev = torch.device("cuda:0")
    tdt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    phi = lola.LolaPhi(wl.phi, torch.from_numpy(W).to(dev))
    st = lola.LolaState(wl.B, wl.h, wl.d_k, wl.d_v, wl.D, wl.eta, wl.lam, tdt, device=dev)
    lola.lola_state_init(st)
    ys, folds, call_chunks = [], [], np.full(wl.n, -1, dtype=np.int64)
    start = 0
    for ln in (calls or [wl.n]):
        call_chunks[start:start + ln] = start // wl.C   # first chunk id of the call holding the token
        sl = slice(start, start + ln)
        qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x[:, :, sl])).to(dev).to(tdt) for x in (q, k, v))
        fold = torch.full((wl.B, wl.h, ln), -7, dtype=torch.int32, device=dev)
        y, _ = lola.lola_prefill(st, phi, qt, kt, vt, wl.C, fold_at=fold, score_rule=rule)
        ys.append(y.float())
        f = fold.clone()
        c_lo = start // wl.C
        f[f >= 0] += c_lo                                  # call-local chunk ids -> whole-sequence ids
        folds.append(f)
        start += ln
    torch.cuda.synchronize()
    y = torch.cat(ys, dim=2).cpu().numpy()
    fold = torch.cat(folds, dim=2).cpu().numpy()
    host = TL.state_to_host(st)
    win_score = st.win_score.cpu().numpy()
    cache_score = st.cache_score.cpu().numpy()
    phi_o = O.make_phi(wl.phi, W)
    out_tol = TL.FP32_TOL if wl.dtype == "f32" else TL.BF16_TOL
    sched_tol = QSCORE_FP32_TOL if wl.dtype == "f32" else TL.BF16_TOL
    worst, differing = 0.0, 0
    for (b, h) in heads:
        args = (phi_o, q[b, h].astype(np.float64), k[b, h].astype(np.float64), v[b, h].astype(np.float64), wl.C)
        so = O.new_state(wl.d_k, wl.d_v, wl.D, wl.eta, wl.lam)
        y_o, sched = O.prefill(so, *args, score_rule=rule)
        if calls is not None:
            # a call reports only its own tokens' folds, and only those it made itself
            ends = np.cumsum(calls)
            call_end_chunk = np.array([(ends[np.searchsorted(ends, i, side="right")] + wl.C - 1) // wl.C
                                       for i in range(wl.n)])
            own = (sched.fold_at >= call_chunks) & (sched.fold_at < call_end_chunk)
            exp = np.where(own, sched.fold_at, -1)
            assert np.array_equal(fold[b, h], exp), f"head ({b},{h}): per-call fold schedule differs"
        elif not np.array_equal(fold[b, h], sched.fold_at):
            differing += 1
            so = O.new_state(wl.d_k, wl.d_v, wl.D, wl.eta, wl.lam)
            y_o, sched = O.prefill(so, *args, fold_at_in=fold[b, h].astype(np.int64), tol=sched_tol,
                                   score_rule=rule)
            assert not sched.problems, f"head ({b},{h}): invalid GPU schedule {sched.problems[:3]}"
        worst = max(worst, TL.row_rel_err(y[b, h], y_o))
        assert TL.cache_members(host["cache_pos"][b, h]) == sorted(so.cache)
        # carried scores: cache slots and window ring, relative to the largest score held
        ref_c = np.array([so.score[p] if p >= 0 else 0.0 for p in host["cache_pos"][b, h][:wl.lam]])
        t_end = wl.n
        ring = [p for p in range(max(0, t_end - wl.eta), t_end)]
        ref_w = np.zeros(max(wl.eta, 1))
        for p in ring:
            ref_w[p % wl.eta] = so.score[p]
        scale = max(1e-30, float(np.abs(ref_c).max(initial=0.0)), float(np.abs(ref_w).max(initial=0.0)))
        if wl.lam > 0:
            assert np.abs(cache_score[b, h][:wl.lam] - ref_c).max() <= sched_tol * scale
        if wl.eta > 0:
            got_w = np.array([win_score[b, h][p % wl.eta] for p in ring])
            assert np.abs(got_w - np.array([so.score[p] for p in ring])).max() <= sched_tol * scale
    print(f"[score rule] {rule} {wl.dtype} calls={calls}: max err {worst:.3e}, heads with a different "
          f"schedule {differing}/{len(heads)}", flush=True)
    assert worst <= out_tol


@pytest.mark.parametrize("rule", SCORE_RULES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_score_rules_prefill(rule, dtype):
    wl = small_workload(80, B=1, h=2, n=260, C=16, eta=24, lam=20, dtype=dtype)
    _score_rule_check(wl, rule, [(0, 0), (0, 1)])


@pytest.mark.parametrize("rule", ["kernel_abs", "attn"])
def test_score_rules_d128_and_continuation(rule):
    """d = 128, and the scores carried across call boundaries (window partial sums, cache finals)."""
    wl = small_workload(81, B=1, h=2, n=300, C=32, eta=40, lam=24, d_k=128, d_v=128, dtype="f32")
    _score_rule_check(wl, rule, [(0, 0), (0, 1)])
    _score_rule_check(wl, rule, [(0, 0), (0, 1)], calls=[64, 96, 140])


def test_score_rule_multi_token_decode():
    """Decode under a query-accumulated rule goes through lola_prefill_ex (calls of 1, then of 4
    tokens, C = 1) and equals the oracle's single call; lola_decode_step_ex rejects the rule."""
    import hybrid_linear_attention_chunkwise_amd as lola
    wl = small_workload(82, B=1, h=2, n=96, C=1, eta=12, lam=8, dtype="f32")
    _score_rule_check(wl, "kernel_sq", [(0, 0), (0, 1)], calls=[1] * 32 + [4] * 16)
    st = lola.LolaState(1, 1, 64, 64, 128, 12, 8, torch.float32)
    lola.lola_state_init(st)
    phi = lola.LolaPhi("softmax_pm", torch.zeros(64, 64).cuda())
    x = torch.zeros(1, 1, 64, device="cuda")
    with pytest.raises(lola.LolaError) as e:
        lola.lola_decode_step(st, phi, x, x, x, score_rule="attn")
    assert e.value.code == lola.LOLA_EUNSUPPORTED


# ------------------------------------------------------------------------------------------------
# HOLA variant (hola_prefill): gated delta rule + write-magnitude cache against oracle/hola_oracle.py.
# ------------------------------------------------------------------------------------------------

def _hola_inputs(seed, B, h, n, d, dtype, alpha_range=(0.9, 1.0)):
    """Seeded synthetic inputs; in bf16 mode the oracle gets the same bf16-rounded q, k, v."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, h, n, d)).astype(np.float32)
    k = rng.standard_normal((B, h, n, d)).astype(np.float32)
    v = rng.standard_normal((B, h, n, d)).astype(np.float32)
    if dtype == "bf16":
        q, k, v = (torch.from_numpy(x).to(torch.bfloat16).float().numpy() for x in (q, k, v))
    alpha = rng.uniform(*alpha_range, (B, h, n)).astype(np.float32)
    beta = rng.uniform(0.0, 1.0, (B, h, n)).astype(np.float32)
    gq = rng.uniform(0.5, 1.5, (h, d)).astype(np.float32)
    gk = rng.uniform(0.5, 1.5, (h, d)).astype(np.float32)
    sink = rng.standard_normal(h).astype(np.float32)
    gate = rng.standard_normal(h).astype(np.float32)
    return q, k, v, alpha, beta, gq, gk, sink, gate


HOLA_CASES = [
    (90, dict(n=300, C=64, w=16, d=64)),        # several chunks, ragged tail
    (91, dict(n=530, C=256, w=64, d=128)),      # the page's w and C, d = 128
    (92, dict(n=100, C=1, w=8, d=64)),          # one-token chunks
    (93, dict(n=70, C=256, w=64, d=128)),       # n < C: no persistent cache is ever read
    (94, dict(n=200, C=32, w=0, d=64)),         # w = 0: chunk tokens and the sink only
    (95, dict(n=530, C=256, w=64, d=256)),      # the page's head dimension, w and C
    (96, dict(n=300, C=64, w=16, d=256)),       # d = 256, several chunks, ragged tail
    # the largest chunk and cache: two full chunks and a ragged one.  The bound is relative to each
    # output row's norm; the seed is one whose rows are all at least a quarter of the median row norm
    # (with seed 97 the state and cache terms of row 0 cancel to 3% of it, and that row's bf16
    # rounding, no larger than any other row's, exceeds the relative bound)
    (98, dict(n=2500, C=1024, w=64, d=128)),
]


@pytest.mark.parametrize("seed,kw", HOLA_CASES, ids=[f"s{s}" for s, _ in HOLA_CASES])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_hola_prefill(seed, kw, dtype):
    """Outputs, final state, final cache and its magnitudes against the oracle; in bf16 the oracle
    takes the same bf16 inputs (the GPU also rounds the normalised cache-path q, k to bf16)."""
    import hybrid_linear_attention_chunkwise_amd as lola
    from oracle import hola_oracle as HO
    B, h = 1, 2
    n, C, w, d = kw["n"], kw["C"], kw["w"], kw["d"]
    q, k, v, alpha, beta, gq, gk, sink, gate = _hola_inputs(seed, B, h, n, d, dtype)
    dev = torch.device("cuda:0")
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    T = lambda x, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(dt)
    S_out = torch.empty(B, h, d, d, device=dev)
    cpos = torch.full((B, h, max(w, 1)), -7, dtype=torch.int32, device=dev)
    cscore = torch.empty(B, h, max(w, 1), device=dev)
    print(f"[hola] n={n} C={C} w={w} d={d} {dtype}", flush=True)
    y = lola.hola_prefill(T(q, tdt), T(k, tdt), T(v, tdt), T(alpha), T(beta), T(gq), T(gk), T(sink), T(gate),
                          C, w, S_out=S_out, cache_pos=cpos, cache_score=cscore)
    torch.cuda.synchronize()
    y, S_out, cpos, cscore = (x.float().cpu().numpy() if x.dtype != torch.int32 else x.cpu().numpy()
                              for x in (y, S_out, cpos, cscore))
    tol = TL.FP32_TOL if dtype == "f32" else TL.BF16_TOL
    worst = 0.0
    for hh in range(h):
        y_o, S_o, cache_o, m_o, _ = HO.hola_prefill(q[0, hh], k[0, hh], v[0, hh], alpha[0, hh], beta[0, hh],
                                                     gq[hh], gk[hh], float(sink[hh]), float(gate[hh]), C, w)
        got_cache = [int(p) for p in cpos[0, hh][:w] if p >= 0]
        assert got_cache == cache_o, f"head {hh}: final cache differs"
        if w > 0:
            np.testing.assert_allclose(cscore[0, hh][:len(cache_o)], m_o[cache_o], rtol=1e-4 if dtype == "f32" else 2e-2)
        worst = max(worst, TL.row_rel_err(y[0, hh], y_o))
        scale = max(1.0, float(np.abs(S_o).max()))
        assert np.abs(S_out[0, hh] - S_o).max() <= 1e-4 * scale
    print(f"[hola] max output err {worst:.3e}", flush=True)
    assert worst <= tol


# HOLA decode (hola_prefill_state then hola_decode_step): every output of the prefill part and of each
# decode step against the oracle's prefill over the whole sequence, then the memory after the last step.
HOLA_DECODE_CASES = [
    (110, dict(n0=300, steps=40, C=64, w=16, d=64)),    # a chunk closes during the decode
    (111, dict(n0=256, steps=20, C=256, w=64, d=128)),  # the prefill ends on a chunk boundary
    (112, dict(n0=50, steps=34, C=16, w=8, d=128)),     # several closes
    (113, dict(n0=0, steps=40, C=8, w=4, d=64)),        # decode from the empty memory
    (114, dict(n0=100, steps=12, C=1, w=8, d=64)),      # every token closes its chunk
    (115, dict(n0=60, steps=10, C=32, w=0, d=64)),      # no persistent cache
    (116, dict(n0=300, steps=20, C=64, w=16, d=256)),   # the page's head dimension
    (118, dict(n0=1000, steps=40, C=1024, w=64, d=128)),  # the largest chunk closes during the decode
]


@pytest.mark.parametrize("seed,kw", HOLA_DECODE_CASES, ids=[f"s{s}" for s, _ in HOLA_DECODE_CASES])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_hola_prefill_then_decode(seed, kw, dtype):
    import hybrid_linear_attention_chunkwise_amd as lola
    from oracle import hola_oracle as HO
    B, h = 1, 2
    n0, steps, C, w, d = kw["n0"], kw["steps"], kw["C"], kw["w"], kw["d"]
    n = n0 + steps
    q, k, v, alpha, beta, gq, gk, sink, gate = _hola_inputs(seed, B, h, n, d, dtype)
    dev = torch.device("cuda:0")
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    T = lambda x, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(dt)
    st = lola.HolaState(B, h, d, C, w, tdt, device=dev)
    lola.hola_state_init(st)
    print(f"[hola decode] n0={n0} steps={steps} C={C} w={w} d={d} {dtype}", flush=True)
    ys = []
    if n0 > 0:
        ys.append(lola.hola_prefill_state(st, T(q[:, :, :n0], tdt), T(k[:, :, :n0], tdt), T(v[:, :, :n0], tdt),
                                          T(alpha[:, :, :n0]), T(beta[:, :, :n0]), T(gq), T(gk), T(sink), T(gate)))
    assert st.t == n0
    G = (T(gq), T(gk), T(sink), T(gate))
    for t in range(n0, n):
        yt = lola.hola_decode_step(st, T(q[:, :, t], tdt), T(k[:, :, t], tdt), T(v[:, :, t], tdt), T(alpha[:, :, t]),
                                   T(beta[:, :, t]), *G)
        ys.append(yt.unsqueeze(2))
    torch.cuda.synchronize()
    assert st.t == n
    y = torch.cat(ys, dim=2).float().cpu().numpy()
    S = st.S.cpu().numpy()
    cpos = st.cache_pos.cpu().numpy()
    ocnt = n % C
    tol = TL.FP32_TOL if dtype == "f32" else TL.BF16_TOL
    worst = 0.0
    for hh in range(h):
        y_o, S_o, cache_o, m_o, _ = HO.hola_prefill(q[0, hh], k[0, hh], v[0, hh], alpha[0, hh], beta[0, hh],
                                                     gq[hh], gk[hh], float(sink[hh]), float(gate[hh]), C, w)
        worst = max(worst, TL.row_rel_err(y[0, hh], y_o))
        scale = max(1.0, float(np.abs(S_o).max()))
        assert np.abs(S[0, hh] - S_o).max() <= 1e-4 * scale, f"head {hh}: state differs"
        want = HO.persistent_cache(m_o, n - ocnt, w)
        got = [int(p) for p in cpos[0, hh][:w] if p >= 0]
        assert got == want, f"head {hh}: cache at the open chunk's start differs"
        if w > 0:
            assert all(p < 0 for p in cpos[0, hh][len(want):w])
            np.testing.assert_allclose(st.cache_score[0, hh][:len(want)].cpu().numpy(), m_o[want],
                                       rtol=1e-4 if dtype == "f32" else 2e-2)
            kc = st.cache_k[0, hh][:len(want)].float().cpu().numpy()
            np.testing.assert_array_equal(kc, k[0, hh][want])
        if ocnt:
            np.testing.assert_array_equal(st.open_v[0, hh][:ocnt].float().cpu().numpy(), v[0, hh][n - ocnt:n])
            np.testing.assert_allclose(st.open_score[0, hh][:ocnt].cpu().numpy(), m_o[n - ocnt:n],
                                       rtol=1e-4 if dtype == "f32" else 2e-2, atol=1e-6)
    print(f"[hola decode] max output err {worst:.3e}", flush=True)
    assert worst <= tol


# The delta rule runs in blocks of 16 tokens: per-block matrices from all blocks in parallel, then one
# workgroup per (sequence, head, 16 value columns) walks the blocks.  These cases cover many heads at
# both d, ragged last blocks, and (alpha in [0.05, 0.3]) decay products that underflow within a block.
HOLA_LANE_CASES = [
    (96, dict(d=128, B=2, h=32, n=97, C=32, w=8)),
    (97, dict(d=128, B=1, h=32, n=96, C=32, w=8)),    # whole blocks only
    (98, dict(d=128, B=1, h=3, n=97, C=32, w=8)),
    (99, dict(d=64, B=4, h=32, n=65, C=16, w=4)),
    (100, dict(d=64, B=2, h=32, n=7, C=16, w=4)),     # one partial block
]


@pytest.mark.parametrize("decay", ["mild", "strong"])
@pytest.mark.parametrize("seed,kw", HOLA_LANE_CASES, ids=[f"s{s}" for s, _ in HOLA_LANE_CASES])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_hola_blocked_delta_rule(seed, kw, dtype, decay):
    """Final state of every head against the oracle's delta rule; outputs and caches of sampled heads
    against the whole oracle."""
    import hybrid_linear_attention_chunkwise_amd as lola
    from oracle import hola_oracle as HO
    B, h, n, C, w, d = kw["B"], kw["h"], kw["n"], kw["C"], kw["w"], kw["d"]
    arange = (0.9, 1.0) if decay == "mild" else (0.05, 0.3)
    q, k, v, alpha, beta, gq, gk, sink, gate = _hola_inputs(seed, B, h, n, d, dtype, arange)
    dev = torch.device("cuda:0")
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    T = lambda x, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(dt)
    S_out = torch.empty(B, h, d, d, device=dev)
    cpos = torch.full((B, h, w), -7, dtype=torch.int32, device=dev)
    print(f"[hola lanes] B={B} h={h} n={n} d={d} {dtype} {decay}", flush=True)
    y = lola.hola_prefill(T(q, tdt), T(k, tdt), T(v, tdt), T(alpha), T(beta), T(gq), T(gk), T(sink), T(gate),
                          C, w, S_out=S_out, cache_pos=cpos)
    torch.cuda.synchronize()
    y, S_out, cpos = y.float().cpu().numpy(), S_out.cpu().numpy(), cpos.cpu().numpy()
    for b in range(B):
        for hh in range(h):
            _, _, S_o = HO.delta_rule(q[b, hh], k[b, hh], v[b, hh], alpha[b, hh], beta[b, hh])
            scale = max(1.0, float(np.abs(S_o).max()))
            assert np.abs(S_out[b, hh] - S_o).max() <= 1e-4 * scale, f"state of ({b}, {hh})"
    tol = TL.FP32_TOL if dtype == "f32" else TL.BF16_TOL
    for b, hh in {(0, 0), (B - 1, h - 1), (B // 2, h // 2)}:
        y_o, _, cache_o, _, _ = HO.hola_prefill(q[b, hh], k[b, hh], v[b, hh], alpha[b, hh], beta[b, hh], gq[hh],
                                                gk[hh], float(sink[hh]), float(gate[hh]), C, w)
        assert [int(p) for p in cpos[b, hh] if p >= 0] == cache_o, f"cache of ({b}, {hh})"
        assert TL.row_rel_err(y[b, hh], y_o) <= tol, f"outputs of ({b}, {hh})"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_hola_degenerate_gates(dtype):
    """Gates and rows at the edges of their ranges: decays of 1e-30 (the state all but resets inside a
    block) mixed with 1.0, write strengths of exactly 0 (magnitude 0: many tied scores, ranked by the
    older position), and all-zero query and key rows (their unit vectors are zero)."""
    import hybrid_linear_attention_chunkwise_amd as lola
    from oracle import hola_oracle as HO
    B, h, n, d, C, w = 1, 4, 150, 64, 32, 16
    q, k, v, alpha, beta, gq, gk, sink, gate = _hola_inputs(101, B, h, n, d, dtype)
    rng = np.random.default_rng(102)
    alpha = np.where(rng.random(alpha.shape) < 0.2, np.float32(1e-30), alpha).astype(np.float32)
    alpha = np.where(rng.random(alpha.shape) < 0.2, np.float32(1.0), alpha).astype(np.float32)
    beta = np.where(rng.random(beta.shape) < 0.5, np.float32(0.0), beta).astype(np.float32)
    zero_q = rng.random((B, h, n)) < 0.1
    zero_k = rng.random((B, h, n)) < 0.1
    q = np.where(zero_q[..., None], 0.0, q).astype(np.float32)
    k = np.where(zero_k[..., None], 0.0, k).astype(np.float32)
    dev = torch.device("cuda:0")
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    T = lambda x, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(dt)
    S_out = torch.empty(B, h, d, d, device=dev)
    cpos = torch.full((B, h, w), -7, dtype=torch.int32, device=dev)
    cscore = torch.empty(B, h, w, device=dev)
    print(f"[hola degenerate] {dtype}", flush=True)
    y = lola.hola_prefill(T(q, tdt), T(k, tdt), T(v, tdt), T(alpha), T(beta), T(gq), T(gk), T(sink), T(gate),
                          C, w, S_out=S_out, cache_pos=cpos, cache_score=cscore)
    torch.cuda.synchronize()
    y, S_out, cpos, cscore = y.float().cpu().numpy(), S_out.cpu().numpy(), cpos.cpu().numpy(), cscore.cpu().numpy()
    tol = TL.FP32_TOL if dtype == "f32" else TL.BF16_TOL
    for hh in range(h):
        y_o, S_o, cache_o, m_o, _ = HO.hola_prefill(q[0, hh], k[0, hh], v[0, hh], alpha[0, hh], beta[0, hh], gq[hh],
                                                     gk[hh], float(sink[hh]), float(gate[hh]), C, w)
        assert (m_o == 0).sum() > w, "the case must hold more zero magnitudes than cache slots"
        assert [int(p) for p in cpos[0, hh]] == cache_o, f"head {hh}: final cache differs"
        np.testing.assert_allclose(cscore[0, hh], m_o[cache_o], rtol=1e-4 if dtype == "f32" else 2e-2, atol=1e-6)
        scale = max(1.0, float(np.abs(S_o).max()))
        assert np.abs(S_out[0, hh] - S_o).max() <= 1e-4 * scale
        assert TL.row_rel_err(y[0, hh], y_o) <= tol


# ------------------------------------------------------------------------------------------------
# Chunked single-token decode (allocation once per group of decode_chunk steps).
# ------------------------------------------------------------------------------------------------

def chunked_decode_check(wl, n0, steps, cd, heads):
    """Prefill n0 tokens, then `steps` single-token decode steps with decode_chunk = cd.  Each group
    of steps is graded against the oracle's prefill of the same tokens as one chunk, continuing from
    the GPU's post-prefill state (grade_chunked_decode)."""
    import hybrid_linear_attention_chunkwise_amd as lola
    from oracle import lola_oracle as O
    W = make_weights(wl)
    q, k, v = make_qkv(wl, n=n0)
    tdt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    C0 = 16 if wl.lam == 0 else min(16, wl.eta + 1)
    _, _, st, phi = TL.gpu_run_prefill(q, k, v, W, wl.phi, wl.eta, wl.lam, C0, wl.dtype, D=wl.D)
    snap = TL.state_to_host(st)
    dq, dk, dv = make_decode_tokens(wl, steps=steps)
    ys, caches = [], [st.cache_pos.cpu().numpy().copy()]
    for s in range(steps):
        y, _ = lola.lola_decode_step(st, phi, torch.from_numpy(dq[s]).cuda().to(tdt),
                                     torch.from_numpy(dk[s]).cuda().to(tdt),
                                     torch.from_numpy(dv[s]).cuda().to(tdt), decode_chunk=cd)
        ys.append(y.float())
        caches.append(st.cache_pos.cpu().numpy().copy())
    torch.cuda.synchronize()
    assert st.c.dec_chunk == (0 if (n0 + steps) % cd == 0 else cd)
    ys = torch.stack(ys).cpu().numpy()
    phi_o = O.make_phi(wl.phi, W)
    worst, mism = 0.0, 0
    for (b, h) in heads:
        so = O.state_from_arrays(snap["t"], wl.eta, wl.lam, snap["H"][b, h].T, snap["s"][b, h],
                                 snap["win_k"][b, h], snap["win_v"][b, h], snap["cache_k"][b, h],
                                 snap["cache_v"][b, h], snap["cache_pos"][b, h])
        cl = [TL.cache_members(c_[b, h]) for c_ in caches]
        rep = TL.grade_chunked_decode(so, phi_o, dq[:, b, h].astype(np.float64), dk[:, b, h].astype(np.float64),
                                      dv[:, b, h].astype(np.float64), ys[:, b, h], cl, n0, cd, wl.dtype)
        worst = max(worst, rep["max_row_rel_err"])
        mism += rep["group_mismatches"]
    print(f"[chunked decode] {wl.name} cd={cd}: max err {worst:.3e}, group mismatches {mism}", flush=True)
    return worst


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("cd", [4, 16])
def test_chunked_decode_small(dtype, cd):
    wl = small_workload(140 + cd, B=2, h=2, n=0, C=1, eta=20, lam=16, d_k=64, d_v=64, dtype=dtype)
    chunked_decode_check(wl, n0=64, steps=48, cd=cd, heads=[(0, 0), (1, 1)])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunked_decode_largest_group(dtype):
    """decode_chunk = 64, the largest group: the fold mask uses all 64 bits of its word."""
    wl = small_workload(153, B=1, h=2, n=0, C=1, eta=64, lam=48, d_k=64, d_v=64, dtype=dtype)
    chunked_decode_check(wl, n0=200, steps=184, cd=64, heads=[(0, 0), (0, 1)])


def test_chunked_decode_d128_unaligned_start():
    """d = 128; the decode starts at t = 70 (not a multiple of 16), so the first group is 10 steps."""
    wl = small_workload(150, B=1, h=2, n=0, C=1, eta=40, lam=36, d_k=128, d_v=128, dtype="bf16")
    chunked_decode_check(wl, n0=70, steps=58, cd=16, heads=[(0, 0), (0, 1)])


def test_chunked_decode_edge_cases():
    """lambda = 0 (every leaving token folds at its exit), a cache that is not yet full (no scoring),
    and eta = Cd - 1 (the group's last leaving token is the current token)."""
    for kw in (dict(eta=12, lam=0, n0=40), dict(eta=24, lam=300, n0=40), dict(eta=7, lam=10, n0=64)):
        n0 = kw.pop("n0")
        wl = small_workload(151, B=1, h=2, n=0, C=1, d_k=64, d_v=64, dtype="f32", **kw)
        chunked_decode_check(wl, n0=n0, steps=32, cd=8, heads=[(0, 0), (0, 1)])


def test_chunked_decode_open_group_is_exclusive():
    """While a group is open, prefill, per-token decode and another decode_chunk are refused (state
    untouched); the group's own steps continue."""
    import hybrid_linear_attention_chunkwise_amd as lola
    wl = small_workload(152, B=1, h=2, n=0, C=1, eta=20, lam=16, d_k=64, d_v=64, dtype="f32")
    W = make_weights(wl)
    q, k, v = make_qkv(wl, n=32)
    _, _, st, phi = TL.gpu_run_prefill(q, k, v, W, wl.phi, wl.eta, wl.lam, 16, "f32", D=wl.D)
    dq = torch.randn(wl.B, wl.h, wl.d_k, device="cuda")
    lola.lola_decode_step(st, phi, dq, dq, dq, decode_chunk=8)
    assert st.c.dec_chunk == 8 and st.t == 33
    for call in (lambda: lola.lola_decode_step(st, phi, dq, dq, dq),
                 lambda: lola.lola_decode_step(st, phi, dq, dq, dq, decode_chunk=4),
                 lambda: lola.lola_prefill(st, phi, dq[:, :, None].contiguous(), dq[:, :, None].contiguous(),
                                           dq[:, :, None].contiguous(), 1)):
        with pytest.raises(lola.LolaError):
            call()
        assert st.t == 33
    for _ in range(7):
        lola.lola_decode_step(st, phi, dq, dq, dq, decode_chunk=8)
    assert st.c.dec_chunk == 0 and st.t == 40
    lola.lola_decode_step(st, phi, dq, dq, dq)
    torch.cuda.synchronize()

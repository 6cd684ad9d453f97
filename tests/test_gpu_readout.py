"""GPU parity of the bf16 read-out for chunks of 64 and 128 tokens (128 queries per workgroup, window
band and cache keys in one block stream, the linear part seeding the running softmax), against the
fp64 oracle replaying the GPU's schedule (LoLA notes 2.5, Eq. (14), and 2.6).

Small cases span several 128-query tiles with ragged ends, n < C, lambda = 0, caches of several
key blocks, eta = C - 1, eta >= n, the elu feature map and outlier keys; continuation calls start
from a live state (window keys from the state's ring, cache members from its slots); the read masks
and the overlapped schedule go through the same kernel.
"""
import numpy as np
import pytest

import lola_testlib as TL
from workloads import make_qkv, make_weights, small_workload

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import hybrid_linear_attention_chunkwise_amd as lola
    lola._b.load()


FAST_CASES = [
    # (seed, kwargs)
    (101, dict(n=700, C=64, eta=64, lam=64, d_k=128)),                 # several tiles, ragged second chunk
    (102, dict(n=450, C=128, eta=128, lam=96, d_k=64)),                # C = 128, ragged
    (103, dict(n=40, C=64, eta=256, lam=256, d_k=128)),                # n < C, eta >= n
    (104, dict(n=330, C=64, eta=70, lam=0, d_k=64)),                   # lambda = 0: window + linear
    (105, dict(n=650, C=64, eta=100, lam=300, d_k=128)),               # five cache blocks, ragged one
    (106, dict(n=200, C=64, eta=63, lam=40, d_k=64, phi="elu1")),      # eta = C - 1, elu feature map
    (107, dict(n=520, C=128, eta=512, lam=8, d_k=128)),                # the window spans every tile
    (108, dict(n=300, C=64, eta=130, lam=128, d_k=128, structure="outlier_keys")),
]


@pytest.mark.parametrize("seed,kw", FAST_CASES, ids=[f"s{s}" for s, _ in FAST_CASES])
def test_fast_readout_small(seed, kw):
    from test_gpu_parity import _check_workload
    kw = dict(kw)
    kw.setdefault("d_v", kw["d_k"])
    wl = small_workload(seed, B=2, h=2, dtype="bf16", **kw)
    _check_workload(wl)


@pytest.mark.parametrize("C,split", [(64, [128, 300]), (64, [64, 401]), (128, [100, 350]), (64, [300, 150])])
def test_fast_readout_continuation(C, split):
    """A second call on a live state: its window band starts in the state's ring and its first
    chunk's cache holds members from the state's slots.  Each call is graded against the oracle
    continuing from the GPU's state before it.  A call's fold_at names only its own tokens, so a bf16
    schedule that folded an older cache member cannot be replayed: the oracle's own schedule must
    match the GPU's (fold chunks and final cache); where it does not, the first difference must be a
    bf16 near-tie (oracle gap within the bf16 tolerance), that head's outputs are not graded for the
    call, and most (head, call) pairs must be graded."""
    import hybrid_linear_attention_chunkwise_amd as lola
    from oracle import lola_oracle as O
    wl = small_workload(110 + C + split[0], B=1, h=2, n=sum(split), C=C, eta=96 if C == 64 else 160, lam=80,
                        d_k=128, d_v=128, dtype="bf16")
    W = make_weights(wl)
    q, k, v = make_qkv(wl)
    dev = torch.device("cuda:0")
    phi = lola.LolaPhi(wl.phi, torch.from_numpy(W).to(dev))
    st = lola.LolaState(wl.B, wl.h, wl.d_k, wl.d_v, wl.D, wl.eta, wl.lam, torch.bfloat16, device=dev)
    lola.lola_state_init(st)
    phi_o = O.make_phi(wl.phi, W)
    start, worst, graded, pairs = 0, 0.0, 0, 0
    for ln in split:
        snap = TL.state_to_host(st)
        sl = slice(start, start + ln)
        qc, kc, vc = (np.ascontiguousarray(x[:, :, sl]) for x in (q, k, v))
        fold = torch.full((wl.B, wl.h, ln), -7, dtype=torch.int32, device=dev)
        y, _ = lola.lola_prefill(st, phi, *(torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (qc, kc, vc)),
                                 C, fold_at=fold)
        y = y.float().cpu().numpy()
        fold = fold.cpu().numpy().astype(np.int64)
        after = TL.state_to_host(st)
        for h in range(wl.h):
            pairs += 1
            so = O.state_from_arrays(snap["t"], wl.eta, wl.lam, snap["H"][0, h].T, snap["s"][0, h],
                                     snap["win_k"][0, h], snap["win_v"][0, h], snap["cache_k"][0, h],
                                     snap["cache_v"][0, h], snap["cache_pos"][0, h])
            y_o, sch = O.prefill(so, phi_o, qc[0, h].astype(np.float64), kc[0, h].astype(np.float64),
                                 vc[0, h].astype(np.float64), C)
            same = np.array_equal(sch.fold_at, fold[0, h]) and \
                TL.cache_members(after["cache_pos"][0, h]) == sorted(so.cache)
            if not same:
                diff = np.nonzero(sch.fold_at != fold[0, h])[0]
                chunks = [int(f) for i in diff for f in (sch.fold_at[i], fold[0, h][i]) if f >= 0]
                c0 = min(chunks) if chunks else None
                gap = sch.gap[c0] if c0 is not None else None
                print(f"[fast read-out continuation] head {h}, call at {start}: schedule differs at chunk {c0}, "
                      f"oracle gap {gap}", flush=True)
                assert gap is not None and gap <= TL.BF16_TOL
                continue
            graded += 1
            worst = max(worst, TL.row_rel_err(y[0, h], y_o))
        start += ln
    print(f"[fast read-out continuation] C={C} split={split}: max err {worst:.3e}, graded {graded}/{pairs}",
          flush=True)
    assert graded * 2 > pairs
    assert worst <= TL.BF16_TOL


@pytest.mark.parametrize("mask", [4, 5, 6], ids=["window", "state_window", "sparse_window"])
def test_fast_readout_read_masks(mask):
    """Read masks through the bf16 read-out: the schedule is the unmasked one, bit for bit, and the
    outputs match the oracle's masked read-out under it (LoLA notes 4.8, Table 12)."""
    import hybrid_linear_attention_chunkwise_amd as lola
    from oracle import lola_oracle as O
    wl = small_workload(120, B=1, h=2, n=460, C=64, eta=70, lam=90, d_k=128, d_v=128, dtype="bf16")
    W = make_weights(wl)
    q, k, v = make_qkv(wl)
    dev = torch.device("cuda:0")
    phi = lola.LolaPhi(wl.phi, torch.from_numpy(W).to(dev))
    qt, kt, vt = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (q, k, v))
    res = {}
    for m in (7, mask):
        st = lola.LolaState(wl.B, wl.h, wl.d_k, wl.d_v, wl.D, wl.eta, wl.lam, torch.bfloat16, device=dev)
        lola.lola_state_init(st)
        fold = torch.full((wl.B, wl.h, wl.n), -7, dtype=torch.int32, device=dev)
        y, _ = lola.lola_prefill(st, phi, qt, kt, vt, wl.C, fold_at=fold, read_mask=m)
        torch.cuda.synchronize()
        res[m] = (y.float().cpu().numpy(), fold.cpu().numpy())
    y, fold = res[mask]
    assert np.array_equal(fold, res[7][1])
    phi_o = O.make_phi(wl.phi, W)
    worst = 0.0
    for h in range(wl.h):
        so = O.new_state(wl.d_k, wl.d_v, wl.D, wl.eta, wl.lam)
        y_o, _ = O.prefill(so, phi_o, q[0, h].astype(np.float64), k[0, h].astype(np.float64),
                           v[0, h].astype(np.float64), wl.C, fold_at_in=fold[0, h].astype(np.int64), tol=1.0,
                           read_mask=mask)
        worst = max(worst, TL.row_rel_err(y[0, h], y_o))
    print(f"[fast read-out] mask {mask}: max err {worst:.3e}", flush=True)
    assert worst <= TL.BF16_TOL


@pytest.mark.parametrize("C,h", [(64, 2), (128, 2), (64, 48)])
def test_fast_readout_overlapped_equals_sequential(C, h):
    """Chunk ranges of the overlapped schedule are cut between 128-query tiles: the same bits as the
    sequential schedule.  With 96 (sequence, head) pairs the chain holds over a quarter of the compute
    units, so the read-outs beside it run in launches of a few 128-query units each."""
    import hybrid_linear_attention_chunkwise_amd as lola
    wl = small_workload(130 + C + h, B=2, h=h, n=1500, C=C, eta=96 if C == 64 else 160, lam=80, d_k=128, d_v=128,
                        dtype="bf16")
    W = make_weights(wl)
    q, k, v = make_qkv(wl)
    dev = torch.device("cuda:0")
    phi = lola.LolaPhi(wl.phi, torch.from_numpy(W).to(dev))
    qt, kt, vt = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (q, k, v))
    ov = lola.LolaOverlap(dev)
    outs = []
    for use in (ov, None):
        st = lola.LolaState(wl.B, wl.h, wl.d_k, wl.d_v, wl.D, wl.eta, wl.lam, torch.bfloat16, device=dev)
        lola.lola_state_init(st)
        y, _ = lola.lola_prefill(st, phi, qt, kt, vt, wl.C, overlap=use)
        torch.cuda.synchronize()
        outs.append(y.float().cpu().numpy())
    assert np.array_equal(outs[0], outs[1])

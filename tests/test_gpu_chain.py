"""The register-resident allocation chain (bf16, d = 128, lambda <= 256, C <= 64, SRE scoring) against
the general chain kernel: both take the same decisions with the same arithmetic, so every output of a
prefill call (y, fold_at, the state after it) must agree bit for bit (LoLA notes 2.6 Eq. (15),
2.4 Eqs. (11)-(13)).  The general kernel is selected with LOLA_CHAIN_GENERAL, read at each launch.
Oracle parity of the same path is covered by the bf16 d = 128 cases of the other GPU tests, which
now run through this kernel.

Cases: several chunks with a ragged end, lambda that is not a multiple of 16, lambda = 0, a cache
that never fills, C = 16 and 32, eta = C - 1, n < C, outlier keys, planted duplicate pairs (exact SRE
ties), inputs of a few repeated tokens (ties in groups of tens to hundreds, so the selection's boundary
bin overflows its bucket), continuation calls from a live state, and the overlapped schedule (several
chain launches per call, the slot table carried through the workspace).
"""
import os

import numpy as np
import pytest

from workloads import make_qkv, make_weights, small_workload

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import hybrid_linear_attention_chunkwise_amd as lola
    lola._b.load()


def _run(wl, split, general: bool, overlap: bool = False, repeat: int = 0):
    import hybrid_linear_attention_chunkwise_amd as lola
    dev = torch.device("cuda:0")
    W = make_weights(wl)
    q, k, v = make_qkv(wl)
    if repeat:   # only `repeat` distinct tokens: SREs collide in large groups of exact ties
        idx = np.arange(wl.n) % repeat
        q, k, v = q[:, :, idx].copy(), k[:, :, idx].copy(), v[:, :, idx].copy()
    phi = lola.LolaPhi(wl.phi, torch.from_numpy(W).to(dev), wl.D)
    st = lola.LolaState(wl.B, wl.h, wl.d_k, wl.d_v, wl.D, wl.eta, wl.lam, torch.bfloat16, device=dev)
    lola.lola_state_init(st)
    ov = lola.LolaOverlap(dev) if overlap else None
    qt, kt, vt = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (q, k, v))
    old = os.environ.pop("LOLA_CHAIN_GENERAL", None)
    if general:
        os.environ["LOLA_CHAIN_GENERAL"] = "1"
    try:
        ys, folds, start = [], [], 0
        for ln in split:
            sl = slice(start, start + ln)
            fold = torch.full((wl.B, wl.h, ln), -7, dtype=torch.int32, device=dev)
            y, _ = lola.lola_prefill(st, phi, qt[:, :, sl].contiguous(), kt[:, :, sl].contiguous(),
                                     vt[:, :, sl].contiguous(), wl.C, fold_at=fold, overlap=ov)
            ys.append(y)
            folds.append(fold)
            start += ln
        torch.cuda.synchronize()
    finally:
        os.environ.pop("LOLA_CHAIN_GENERAL", None)
        if old is not None:
            os.environ["LOLA_CHAIN_GENERAL"] = old
    out = {"y": torch.cat(ys, dim=2).view(torch.int16).cpu().numpy(),
           "fold": torch.cat(folds, dim=2).cpu().numpy()}
    for name in ("H", "s", "cache_pos", "cache_k", "cache_v", "win_k", "win_v"):
        t = getattr(st, name)
        out[name] = (t.view(torch.int16) if t.dtype == torch.bfloat16 else t).cpu().numpy()
    return out


CASES = [
    # (seed, workload kwargs, call lengths, overlapped)
    (201, dict(n=700, C=64, eta=64, lam=64), [700], False),
    (202, dict(n=1000, C=32, eta=100, lam=200), [1000], False),          # lambda not a multiple of 16
    (203, dict(n=300, C=64, eta=70, lam=0), [300], False),               # no cache
    (204, dict(n=500, C=16, eta=40, lam=256), [500], False),             # C = 16, full-size cache
    (205, dict(n=400, C=64, eta=200, lam=256), [400], False),            # the cache never fills
    (206, dict(n=450, C=64, eta=63, lam=40), [450], False),              # eta = C - 1
    (207, dict(n=40, C=64, eta=256, lam=256), [40], False),              # n < C
    (208, dict(n=1500, C=64, eta=256, lam=256, structure="outlier_keys"), [1500], False),
    (209, dict(n=900, C=64, eta=96, lam=100, structure="planted_pairs"), [900], False),   # exact ties
    (210, dict(n=757, C=64, eta=96, lam=80), [300, 1, 456], False),      # continuation calls
    (211, dict(n=2100, C=64, eta=256, lam=256), [2100], True),           # several chain launches
    (212, dict(n=1300, C=32, eta=64, lam=144), [700, 600], True),
    (213, dict(n=900, C=64, eta=64, lam=256, repeat=3), [900], False),    # boundary bins of ~100 tied keys
    (214, dict(n=700, C=64, eta=80, lam=100, repeat=40), [700], False),
]


@pytest.mark.parametrize("seed,kw,split,overlap", CASES, ids=[f"s{c[0]}" for c in CASES])
def test_register_chain_equals_general_chain(seed, kw, split, overlap):
    kw = dict(kw)
    repeat = kw.pop("repeat", 0)
    wl = small_workload(seed, B=2, h=2, d_k=128, d_v=128, dtype="bf16", **kw)
    fast = _run(wl, split, general=False, overlap=overlap, repeat=repeat)
    gen = _run(wl, split, general=True, overlap=overlap, repeat=repeat)
    nfold = int((gen["fold"] >= 0).sum())
    print(f"[chain] {wl.name} split={split} overlap={overlap}: {nfold} tokens folded", flush=True)
    for name in gen:
        assert np.array_equal(fast[name], gen[name]), f"{name} differs between the two chain kernels"

"""The allocation-free prefill entry point (lola_prefill_noalloc: the library's own per-device scratch)
against lola_prefill_ex with a caller workspace.  The kernels are the same, so the outputs, fold
chunks and final states must be the same bits.  Two calls in a row on one GPU, the second smaller and
of another shape, so it runs on a scratch array still holding the first call's data."""
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


def _run(wl, noalloc):
    import hybrid_linear_attention_chunkwise_amd as lola
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    W = make_weights(wl)
    q, k, v = make_qkv(wl)
    phi = lola.LolaPhi(wl.phi, torch.from_numpy(W).to(dev))
    qt, kt, vt = (torch.from_numpy(x).to(dev).to(tdt) for x in (q, k, v))
    st = lola.LolaState(wl.B, wl.h, wl.d_k, wl.d_v, wl.D, wl.eta, wl.lam, tdt, device=dev)
    lola.lola_state_init(st)
    y = torch.empty_like(vt)
    fold = torch.full((wl.B, wl.h, wl.n), -7, dtype=torch.int32, device=dev)
    if noalloc:
        lola.lola_prefill_noalloc(st, phi, qt, kt, vt, wl.C, y, fold_at=fold)
    else:
        ws = torch.randint(0, 255, (lola.lola_workspace_bytes(st, wl.n, wl.C),), dtype=torch.uint8, device=dev)
        lola.lola_prefill(st, phi, qt, kt, vt, wl.C, y=y, fold_at=fold, workspace=ws)
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), fold.cpu().numpy(), TL.state_to_host(st)


def test_noalloc_equals_workspace_entry_point():
    import hybrid_linear_attention_chunkwise_amd as lola
    cases = [small_workload(201, B=2, h=3, n=700, C=64, eta=80, lam=72, d_k=128, d_v=128, dtype="bf16"),
             small_workload(202, B=1, h=2, n=150, C=16, eta=24, lam=20, d_k=64, d_v=64, dtype="f32")]
    for wl in cases:
        print(f"[noalloc] {wl.name} B={wl.B} h={wl.h} n={wl.n} C={wl.C} {wl.dtype}", flush=True)
        st = lola.LolaState(wl.B, wl.h, wl.d_k, wl.d_v, wl.D, wl.eta, wl.lam, torch.float32, device="cuda")
        assert lola.lola_workspace_bytes(st, wl.n, wl.C) <= lola._b.LOLA_NOALLOC_SCRATCH_BYTES
        ref = _run(wl, noalloc=False)
        got = _run(wl, noalloc=True)
        assert np.array_equal(ref[0], got[0]), "outputs differ"
        assert np.array_equal(ref[1], got[1]), "fold chunks differ"
        for key in ref[2]:
            assert np.array_equal(np.asarray(ref[2][key]), np.asarray(got[2][key])), key

"""Helpers shared by the GPU parity tests: run the library through its C ABI, run the fp64 oracle on
sampled (sequence, head) pairs in a process pool, and compare.

Tolerances (written here, used by every parity test):
  * fp32 storage: outputs within 1e-4 max row-relative error; fold schedule bit-exact except at
    near-ties, i.e. chunks where the oracle's boundary gap (SRE_(lam) - SRE_(lam+1)) / SRE_(lam) is
    at most 1e-6; from such a chunk on the oracle follows the GPU schedule (replay) and the
    remaining outputs are graded against that replay.
  * bf16 storage: outputs within 2e-2 max row-relative error against the oracle replaying the GPU
    schedule, whose validity is checked in fp64 with relative tolerance 2e-2.
Row-relative error of a row t is ||y_t - yhat_t||_2 / ||yhat_t||_2; the maximum over rows is reported.
"""
from __future__ import annotations

import concurrent.futures
import multiprocessing
import os
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

FP32_TOL = 1e-4
BF16_TOL = 2e-2
TIE_BAND = 1e-6


def n_workers() -> int:
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    return max(1, min(16, cores))


def row_rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    y = np.asarray(y, dtype=np.float64).reshape(-1, ref.shape[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    num = np.linalg.norm(y - ref, axis=1)
    den = np.maximum(np.linalg.norm(ref, axis=1), 1e-300)
    return float((num / den).max()) if len(num) else 0.0


# --------------------------------------------------------------------------------------------------
# oracle jobs (run in worker processes; they import only numpy and the oracle)
# --------------------------------------------------------------------------------------------------

def _progress(tag: str, every: int):
    """on_chunk_end hook printing a line every `every` chunks (long oracle runs stay visibly alive)."""
    def hook(c, _st):
        if every and (c + 1) % every == 0:
            print(f"[oracle {tag}] chunk {c + 1}", flush=True)
    return hook


def _oracle_job(job: dict) -> dict:
    """The oracle on one (sequence, head): its own schedule, and where the GPU's differs, a replay of the
    GPU's (validated in fp64).  replay_only (bf16 jobs of long sequences, whose membership is not graded
    bit-exactly): only the replay of the GPU schedule."""
    import numpy as _np
    from oracle import lola_oracle as O
    phi = O.make_phi(job["phi"], job["W"])
    d_k, d_v = job["q"].shape[1], job["v"].shape[1]
    every = job.get("progress_every", 0)
    tag = job.get("tag", "")
    out = {}
    gpu_fold = job.get("fold_at_gpu")
    if not job.get("replay_only"):
        st = O.new_state(d_k, d_v, job["D"], job["eta"], job["lam"])
        y_o, sched_o = O.prefill(st, phi, job["q"], job["k"], job["v"], job["C"],
                                 on_chunk_end=_progress(tag + " own", every))
        out["y_oracle"] = y_o
        out["fold_at_oracle"] = sched_o.fold_at
        out["gap"] = sched_o.gap
        out["cache_oracle"] = sorted(st.cache)
        out["H_oracle"] = st.H
        out["s_oracle"] = st.s
    if gpu_fold is not None and (job.get("replay_only") or not _np.array_equal(gpu_fold, out["fold_at_oracle"])):
        st2 = O.new_state(d_k, d_v, job["D"], job["eta"], job["lam"])
        y_r, sched_r = O.prefill(st2, phi, job["q"], job["k"], job["v"], job["C"], fold_at_in=gpu_fold,
                                 tol=job["tol"], on_chunk_end=_progress(tag + " replay", every))
        out["y_replay"] = y_r
        out["replay_problems"] = sched_r.problems
        out["replay_worst"] = sched_r.worst_inversion
        out["cache_replay"] = sorted(st2.cache)
        out["H_replay"] = st2.H
        out["s_replay"] = st2.s
        if not job.get("replay_only"):
            # first chunk where the two schedules differ, and the oracle's gap there
            diff = _np.nonzero(gpu_fold != out["fold_at_oracle"])[0]
            chunks = set()
            for i in diff:
                for f in (gpu_fold[i], out["fold_at_oracle"][i]):
                    if f >= 0:
                        chunks.add(int(f))
            out["first_diff_chunk"] = min(chunks) if chunks else None
    return out


def _ctx():
    return multiprocessing.get_context("spawn")


def run_oracle_heads(jobs: Sequence[dict]) -> List[dict]:
    if len(jobs) == 1:
        return [_oracle_job(jobs[0])]
    with concurrent.futures.ProcessPoolExecutor(max_workers=min(n_workers(), len(jobs)),
                                                mp_context=_ctx()) as ex:
        return list(ex.map(_oracle_job, jobs))


def grade_prefill(res: dict, y_gpu: np.ndarray, fold_gpu: np.ndarray, dtype: str,
                  cache_gpu: Optional[List[int]] = None) -> dict:
    """Checks one (sequence, head) against the oracle result; returns a report, raises on failure."""
    rep: Dict[str, object] = {}
    if "fold_at_oracle" not in res:                    # replay only (bf16): the GPU schedule, validated
        assert dtype != "f32", "fp32 schedules are graded against the oracle's own"
        assert not res["replay_problems"], f"invalid GPU schedule: {res['replay_problems'][:3]}"
        rep["schedule_identical"] = None
        rep["replay_worst_inversion"] = res["replay_worst"]
        ref, cache_ref = res["y_replay"], res["cache_replay"]
    else:
        same = np.array_equal(fold_gpu, res["fold_at_oracle"])
        rep["schedule_identical"] = bool(same)
        if same:
            ref, cache_ref = res["y_oracle"], res["cache_oracle"]
        else:
            ref, cache_ref = res["y_replay"], res["cache_replay"]
            assert not res["replay_problems"], f"invalid GPU schedule: {res['replay_problems'][:3]}"
            if dtype == "f32":
                c = res["first_diff_chunk"]
                gap = res["gap"][c] if c is not None else None
                assert gap is not None and gap <= TIE_BAND, (
                    f"fp32 schedule differs at chunk {c} with oracle gap {gap} > {TIE_BAND}")
                rep["near_tie_chunk"] = c
                rep["near_tie_gap"] = gap
            rep["membership_agreement"] = float(np.mean(fold_gpu == res["fold_at_oracle"]))
    err = row_rel_err(y_gpu, ref)
    rep["max_row_rel_err"] = err
    tol = FP32_TOL if dtype == "f32" else BF16_TOL
    assert err <= tol, f"output error {err:.3e} > {tol}"
    if cache_gpu is not None:
        assert sorted(cache_gpu) == list(cache_ref), "final cache membership differs"
    return rep


def grade_decode_steps(so, phi_o, dq, dk, dv, ys, folds, dtype: str, read_mask: int = 7) -> dict:
    """Grades single-token decode steps of one (sequence, head) against the oracle state ``so``
    (mutated: it follows the GPU).

    dq, dk, dv [steps][d]; ys [steps][d_v] GPU outputs; folds [steps] GPU folded positions (-1: none).
    Each step is decided by the oracle on a copy of the state.  Where the GPU folded another candidate:
    in fp32 the oracle's boundary gap must lie within the tie band; in both modes the GPU's choice is
    replayed (validated in fp64: the folded SRE may exceed the smallest kept SRE by at most the
    dtype's tolerance) and the oracle continues from there, so every step is graded."""
    from oracle import lola_oracle as O
    tol = TIE_BAND if dtype == "f32" else BF16_TOL
    out_tol = FP32_TOL if dtype == "f32" else BF16_TOL
    worst, mism = 0.0, 0
    for s in range(len(ys)):
        trial = so.copy()
        y_o, f_o, sch = O.decode_step(trial, phi_o, dq[s], dk[s], dv[s], read_mask=read_mask, want_schedule=True)
        f_g = int(folds[s])
        if f_o == f_g:
            so.__dict__.update(trial.__dict__)
        else:
            mism += 1
            if dtype == "f32":
                gap = sch.gap[0]
                assert gap is not None and gap <= TIE_BAND, (
                    f"fp32 decode fold differs at step {s}: oracle {f_o}, GPU {f_g}, gap {gap}")
            y_o, f_r, sch_r = O.decode_step(so, phi_o, dq[s], dk[s], dv[s], read_mask=read_mask,
                                            fold=f_g, tol=tol, want_schedule=True)
            assert not sch_r.problems, f"invalid GPU fold at step {s}: {sch_r.problems}"
            assert f_r == f_g
        err = row_rel_err(np.asarray(ys[s])[None], y_o[None])
        assert err <= out_tol, f"decode output error {err:.3e} > {out_tol} at step {s}"
        worst = max(worst, err)
    return {"max_row_rel_err": worst, "fold_mismatches": mism, "steps": len(ys)}


def grade_chunked_decode(so, phi_o, q, k, v, ys, caches, t0: int, cd: int, dtype: str) -> dict:
    """Grades chunked decode steps of one (sequence, head) against the oracle state ``so`` (mutated:
    it follows the GPU).  Each group of steps [a, b) (b the next multiple of cd after a) is one chunk
    of the oracle's prefill (LoLA notes 2.6).

    q, k, v [steps][d]; ys [steps][d_v] GPU outputs; caches [steps + 1] GPU cache positions (sorted
    lists) before the first step and after every step.  The GPU's folds of a group are the group's
    candidates (the cache at its start and the tokens leaving during it) minus its cache at the end.
    Where they differ from the oracle's own: fp32 needs the oracle's boundary gap within the tie band;
    both modes replay the GPU's choice (validated in fp64) and continue from it."""
    from oracle import lola_oracle as O
    tol = TIE_BAND if dtype == "f32" else BF16_TOL
    out_tol = FP32_TOL if dtype == "f32" else BF16_TOL
    worst, mism, s, steps = 0.0, 0, 0, len(ys)
    # A group's allocation covers every token that leaves during the whole group, so a group the
    # steps stop inside cannot be compared with a prefill chunk of the steps taken: whole groups only.
    assert (t0 + steps) % cd == 0, "chunked decode grading needs the steps to end on a group boundary"
    while s < steps:
        a = t0 + s
        b = (a // cd + 1) * cd
        n = b - a
        X = [p for p in range(a - so.eta, b - so.eta) if p >= 0]
        cand = set(caches[s]) | set(X)
        s_gpu = sorted(cand - set(caches[s + n - 1 + 1]))
        trial = so.copy()
        y_o, sch = O.prefill(trial, phi_o, q[s:s + n], k[s:s + n], v[s:s + n], C=n)
        if sorted(sch.folded[0]) == s_gpu:
            so.__dict__.update(trial.__dict__)
        else:
            mism += 1
            if dtype == "f32":
                gap = sch.gap[0]
                assert gap is not None and gap <= TIE_BAND, (
                    f"fp32 group at {a}: oracle folds {sch.folded[0]}, GPU {s_gpu}, gap {gap}")
            y_o, sch_r = O.prefill(so, phi_o, q[s:s + n], k[s:s + n], v[s:s + n], C=n, fold_sets_in=[s_gpu],
                                   tol=tol)
            assert not sch_r.problems, f"invalid GPU group fold at {a}: {sch_r.problems}"
        assert sorted(so.cache) == sorted(caches[s + n]), f"cache after the group at {a} differs"
        err = row_rel_err(np.asarray(ys[s:s + n]), y_o)
        assert err <= out_tol, f"chunked decode output error {err:.3e} > {out_tol} in the group at {a}"
        worst = max(worst, err)
        s += n
    return {"max_row_rel_err": worst, "group_mismatches": mism, "steps": steps}


def gpu_run_prefill(q, k, v, W, phi_kind: str, eta: int, lam: int, C: int, dtype: str, D: int = 128,
                    chunks: Optional[Sequence[int]] = None, state=None):
    """Runs lola_prefill on cuda:0 for numpy q, k, v [B][h][n][d]; returns host arrays.

    ``chunks`` splits the call into several consecutive prefill calls of the given lengths."""
    import torch
    import hybrid_linear_attention_chunkwise_amd as lola
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    dev = torch.device("cuda:0")
    B, h, n, d_k = q.shape
    d_v = v.shape[-1]
    if state is None:
        state = lola.LolaState(B, h, d_k, d_v, D, eta, lam, tdt, device=dev)
        lola.lola_state_init(state)
    phi = lola.LolaPhi(phi_kind, torch.from_numpy(np.ascontiguousarray(W, dtype=np.float32)).to(dev), D)
    qt = torch.from_numpy(q).to(dev).to(tdt)
    kt = torch.from_numpy(k).to(dev).to(tdt)
    vt = torch.from_numpy(v).to(dev).to(tdt)
    ys, folds = [], []
    bounds = [n] if chunks is None else list(chunks)
    start = 0
    for ln in bounds:
        sl = slice(start, start + ln)
        fold = torch.full((B, h, ln), -7, dtype=torch.int32, device=dev)
        y, _ = lola.lola_prefill(state, phi, qt[:, :, sl].contiguous(), kt[:, :, sl].contiguous(),
                                 vt[:, :, sl].contiguous(), C, fold_at=fold)
        ys.append(y)
        folds.append(fold)
        start += ln
    torch.cuda.synchronize()
    y = torch.cat(ys, dim=2).float().cpu().numpy()
    fold = torch.cat(folds, dim=2).cpu().numpy()
    return y, fold, state, phi


def state_to_host(state) -> dict:
    import torch
    torch.cuda.synchronize()
    return {"H": state.H.cpu().numpy(), "s": state.s.cpu().numpy(),
            "win_k": state.win_k.float().cpu().numpy(), "win_v": state.win_v.float().cpu().numpy(),
            "cache_k": state.cache_k.float().cpu().numpy(), "cache_v": state.cache_v.float().cpu().numpy(),
            "cache_pos": state.cache_pos.cpu().numpy(), "t": state.t}


def cache_members(cache_pos_row: np.ndarray) -> List[int]:
    return sorted(int(p) for p in cache_pos_row if p >= 0)

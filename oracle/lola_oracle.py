"""Plain fp64 CPU oracle for LoLA: linear attention + sliding window + SRE-scored sparse cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this module: only the tests, the
smoke check and the CPU-baseline leg of the benchmark use it.  It shares no code with the HIP library.

Source: "LoLA: Low-Rank Linear Attention With Sparse Caching" reading notes (cc.laoqi.cc, paper
2505.23666 v3), part 2 ("Method"):
  * 2.2, Eqs. (3)-(5): H_t = H_{t-1} + phi(k_t) v_t^T, s_t = s_{t-1} + phi(k_t); the linear read-out
    is H^T phi(q) / (phi(q)^T s); H and s receive only the KV allocated to them.
  * 2.3, Eq. (10): SRE(k, v | H, s) = || H^T phi(k) / (phi(k)^T s) - v ||_2 (an L2 norm, not squared).
  * 2.4, Eqs. (11)-(13): candidates E = G_{t-1} U {token leaving the window}; keep the lambda with the
    largest SRE scored against the state *before* the update; fold the rest into H, s; keep all when
    there are at most lambda candidates.  Allocation is greedy and irreversible.
  * 2.5, Eq. (14): one shared denominator over the linear state, the sparse cache and the window,
    with a_ti = exp(q_t^T k_i / sqrt(d_k)).
  * 2.6, Eq. (15) and Fig. 2: chunked prefill of length C; after a chunk the oldest window chunk and
    the cache are scored together (about C + lambda candidates) and the rest folded in one batch.
  * 2.7: per-head persistent element count.
  * 4.5, Table 4 (App. F): alternative cache-scoring rules, each accumulated over the queries that
    see the key in their window: squared and absolute difference of the exp kernel and the feature
    kernel, their ratio (feature over exp), and the exp kernel alone.
  * 4.8, Table 12 (App. I): read-branch masks; storage and allocation are unchanged, the query reads
    only some of {linear state, sparse cache, window}.
  * 4.4, Fig. 3 and Fig. 10 with Eq. (26): the collision map, the SRE of each KV held by the linear
    state against each later state, zero while the KV is not in the state; its relative form subtracts
    the SRE the KV had right after it was written (a difference, not a ratio).

Readings where the notes leave a step open (each is listed in the design notes of the repository):
  R1 window: the window seen by query t is positions max(0, t-eta+1) .. t (it includes the current
     token and holds eta tokens when full); token i leaves the window at time i + eta.
  R2 order inside a step: score against the state before the update, fold, then read out; the fold of
     a step is visible to the same step's query.
  R3 chunk semantics: allocation is chunk-granular (candidates = cache + the tokens that leave the
     window during the chunk, all scored against the chunk-start state); the read-out keeps an exact
     per-token window, and a folded token becomes visible in the linear state at its own exit time
     (old cache members that are folded become linear at the chunk start).
  R4 causality: a chunk may only promote tokens every query of the chunk has already seen, so
     lambda == 0 or eta >= C - 1.
  R5 empty state: if phi(k)^T s == 0 the recall is the zero vector, so SRE = ||v||_2.
  R6 ties: exactly lambda are kept; equal SRE is broken toward the older (smaller) position.
  R7 a single feature map phi (and weight W) is shared by queries and keys, heads and batches.
  R18 read masks: a hidden branch leaves both the numerator and the denominator of Eq. (14); every
     mask includes the window, the one memory that always holds the current token.
  R19 query-accumulated scores: key i gathers f(q_t, k_i) from every query t whose window holds it
     (i <= t <= i + eta - 1, reading R1); an allocation at chunk start a uses what queries t < a have
     added, so a leaving token's score may still be partial while a cache member's is complete.  The
     kept keys are the lambda largest scores (ties: older position), like SRE.  The score is fixed
     once the key leaves the window; the state carries it with the key.
  R17 collision map: the states are the chunk-end states of a chunked prefill (the figure's per-token
     states are read at chunk granularity, where the chunked path has complete states), one row per
     chunk; a KV enters the map at the end of the chunk that folds it, and "right after it was
     written" is that same row.

Parity status: every function here is pinned by the tests in tests/test_oracle_*.py (closed forms,
textbook special cases, hand-derived schedules, invariants and an independent per-pair evaluation).
"""
from __future__ import annotations

import dataclasses
from typing import Callable, List, Optional, Sequence

import numpy as np

__all__ = ["phi_elu1", "phi_softmax_pm", "make_phi", "sre", "SeqState", "new_state", "prefill",
           "decode_step", "replay", "exact_attention_read", "state_elements", "Schedule",
           "state_from_arrays", "sre_collisions", "READ_STATE", "READ_SPARSE", "READ_WINDOW",
           "READ_ALL", "SCORE_RULES", "query_score"]

# Read-branch masks (4.8, Table 12).
READ_STATE, READ_SPARSE, READ_WINDOW = 1, 2, 4
READ_ALL = READ_STATE | READ_SPARSE | READ_WINDOW
# Cache-scoring rules (4.5, Table 4): SRE against the state, or a score accumulated over queries.
SCORE_RULES = ("sre", "kernel_sq", "kernel_abs", "ratio", "attn")


# --------------------------------------------------------------------------------------------------
# Feature maps.  Section 2.2: exp(q^T k / sqrt(d_k)) is approximated by phi(q)^T phi(k).  The two
# concrete maps are elu(xW)+1 and [softmax(xW); softmax(-xW)] (the LoLCATs form, section 3.1).
# --------------------------------------------------------------------------------------------------

def phi_elu1(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    """elu(xW) + 1, where elu(z) = z for z > 0 and exp(z) - 1 otherwise."""
    z = np.asarray(x, dtype=np.float64) @ np.asarray(W, dtype=np.float64)
    return np.where(z > 0.0, z + 1.0, np.exp(np.minimum(z, 0.0)))


def _softmax_last(z: np.ndarray) -> np.ndarray:
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def phi_softmax_pm(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    """[softmax(xW); softmax(-xW)], each softmax over the columns of W."""
    z = np.asarray(x, dtype=np.float64) @ np.asarray(W, dtype=np.float64)
    return np.concatenate([_softmax_last(z), _softmax_last(-z)], axis=-1)


def make_phi(kind: str, W: np.ndarray):
    W = np.asarray(W, dtype=np.float64)
    if kind == "elu1":
        return lambda x: phi_elu1(x, W)
    if kind == "softmax_pm":
        return lambda x: phi_softmax_pm(x, W)
    raise ValueError(f"unknown feature map {kind!r}")


# --------------------------------------------------------------------------------------------------
# Self-recall error (section 2.3, Eq. (10)), with reading R5 for the empty state.
# --------------------------------------------------------------------------------------------------

def sre(phi_k: np.ndarray, v: np.ndarray, H: np.ndarray, s: np.ndarray) -> np.ndarray:
    """SRE of each row (phi(k_i), v_i) against the state (H [D][d_v], s [D]).

    phi_k: [m][D], v: [m][d_v] -> [m] float64."""
    phi_k = np.atleast_2d(np.asarray(phi_k, dtype=np.float64))
    v = np.atleast_2d(np.asarray(v, dtype=np.float64))
    num = phi_k @ H                     # row i = (H^T phi(k_i))^T
    den = phi_k @ s                     # phi(k_i)^T s
    recall = np.zeros_like(num)
    ok = den != 0.0
    recall[ok] = num[ok] / den[ok, None]
    return np.sqrt(((recall - v) ** 2).sum(axis=-1))


def query_score(rule: str, q_t, phi_q, k, phi_k, d_k: int) -> np.ndarray:
    """One query's contribution to the query-accumulated scores of keys k [m][d_k] (reading R19).

    e = exp(q^T k / sqrt(d_k)) is the exp kernel, p = phi(q)^T phi(k) the feature kernel:
    kernel_sq (e - p)^2, kernel_abs |e - p|, ratio p / e, attn e."""
    e = np.exp(np.atleast_2d(k) @ q_t / np.sqrt(d_k))
    p = np.atleast_2d(phi_k) @ phi_q
    if rule == "kernel_sq":
        return (e - p) ** 2
    if rule == "kernel_abs":
        return np.abs(e - p)
    if rule == "ratio":
        return p / e
    if rule == "attn":
        return e
    raise ValueError(f"unknown query-accumulated rule {rule!r}")


# --------------------------------------------------------------------------------------------------
# Per-sequence state: the three memories of section 2.4 (window, sparse cache, linear state).
# --------------------------------------------------------------------------------------------------

@dataclasses.dataclass
class SeqState:
    eta: int
    lam: int
    H: np.ndarray                  # [D][d_v]: sum of phi(k) v^T over folded tokens
    s: np.ndarray                  # [D]: sum of phi(k) over folded tokens
    t: int                         # tokens consumed so far
    K: np.ndarray                  # [capacity][d_k]: exact keys by absolute position (NaN = not held)
    V: np.ndarray                  # [capacity][d_v]
    cache: List[int]               # positions in the sparse cache G
    folded: List[int]              # positions folded into (H, s), in fold order
    score: np.ndarray = None       # [capacity]: query-accumulated score by position (reading R19)

    def window(self, t: int) -> range:
        """Positions in the window of query t (reading R1)."""
        return range(max(0, t - self.eta + 1), t + 1)

    def ensure(self, cap: int) -> None:
        if self.score is None:
            self.score = np.zeros(self.K.shape[0])
        if self.K.shape[0] < cap:
            grow = cap - self.K.shape[0]
            self.K = np.concatenate([self.K, np.full((grow, self.K.shape[1]), np.nan)])
            self.V = np.concatenate([self.V, np.full((grow, self.V.shape[1]), np.nan)])
            self.score = np.concatenate([self.score, np.zeros(grow)])

    def forget(self, i: int) -> None:
        self.K[i] = np.nan
        self.V[i] = np.nan

    def copy(self) -> "SeqState":
        return SeqState(self.eta, self.lam, self.H.copy(), self.s.copy(), self.t, self.K.copy(),
                        self.V.copy(), list(self.cache), list(self.folded),
                        None if self.score is None else self.score.copy())


def new_state(d_k: int, d_v: int, D: int, eta: int, lam: int) -> SeqState:
    return SeqState(eta=eta, lam=lam, H=np.zeros((D, d_v)), s=np.zeros(D), t=0,
                    K=np.zeros((0, d_k)), V=np.zeros((0, d_v)), cache=[], folded=[])


def state_from_arrays(t, eta, lam, H, s, win_k, win_v, cache_k, cache_v, cache_pos, win_score=None,
                      cache_score=None) -> SeqState:
    """Build a state from a ring window (slot = pos mod eta) and a slotted cache (pos -1 = empty).

    Used to continue from a state produced elsewhere (for example a post-prefill snapshot).
    win_score / cache_score (optional, same slots) restore the query-accumulated scores."""
    d_k = win_k.shape[-1] if eta > 0 else cache_k.shape[-1]
    d_v = win_v.shape[-1] if eta > 0 else cache_v.shape[-1]
    st = SeqState(eta=eta, lam=lam, H=np.array(H, dtype=np.float64),
                  s=np.array(s, dtype=np.float64), t=int(t), K=np.zeros((0, d_k)),
                  V=np.zeros((0, d_v)), cache=[], folded=[])
    st.ensure(int(t))
    for pos in range(max(0, t - eta), t):
        st.K[pos] = win_k[pos % eta]
        st.V[pos] = win_v[pos % eta]
        if win_score is not None:
            st.score[pos] = win_score[pos % eta]
    for slot, pos in enumerate(np.asarray(cache_pos).tolist()):
        if pos >= 0:
            st.K[pos] = cache_k[slot]
            st.V[pos] = cache_v[slot]
            st.cache.append(int(pos))
            if cache_score is not None:
                st.score[pos] = cache_score[slot]
    st.cache.sort()
    return st


@dataclasses.dataclass
class Schedule:
    """What one call decided: per chunk the folded set S and the kept cache G' (sorted positions)."""
    chunk_start: List[int] = dataclasses.field(default_factory=list)
    folded: List[List[int]] = dataclasses.field(default_factory=list)
    kept: List[List[int]] = dataclasses.field(default_factory=list)
    gap: List[Optional[float]] = dataclasses.field(default_factory=list)   # boundary gap per chunk
    fold_at: Optional[np.ndarray] = None          # [n]: call-local chunk index that folded token i, or -1
    problems: List[tuple] = dataclasses.field(default_factory=list)       # replay validation failures
    worst_inversion: float = 0.0                  # replay: max (max_S SRE - min_G' SRE) / max_S SRE


def exact_attention_read(q_t, phi_q, H, s, keys, vals, d_k, use_state: bool = True):
    """Eq. (14): one shared denominator over the linear state and the exact keys.

    Numerator and denominator are both multiplied by exp(-m), m the largest exact logit, which is an
    exact identity that keeps the exponentials in range.  use_state=False drops the linear terms
    (read mask without the state, reading R18)."""
    lin_num = H.T @ phi_q if use_state else np.zeros(H.shape[1])
    lin_den = float(phi_q @ s) if use_state else 0.0
    if len(keys) == 0:
        return lin_num / lin_den
    logits = (keys @ q_t) / np.sqrt(d_k)
    m = logits.max()
    a = np.exp(logits - m)
    scale = np.exp(-m)
    return (lin_num * scale + a @ vals) / (lin_den * scale + a.sum())


def prefill(st: SeqState, phi, q, k, v, C: int, fold_at_in: Optional[np.ndarray] = None,
            tol: float = 0.0, on_chunk_end: Optional[Callable[[int, SeqState], None]] = None,
            read_mask: int = READ_ALL, score_rule: str = "sre",
            fold_sets_in: Optional[Sequence[Sequence[int]]] = None):
    """Chunked prefill of n tokens for one sequence and head (section 2.6), read out token by token.

    q, k: [n][d_k]; v: [n][d_v].  Mutates ``st``.  Returns (y [n][d_v], Schedule).
    ``fold_at_in`` replays an external schedule (call-local chunk id per input token, -1 = not
    folded): its decisions replace the top-lambda, and each is checked against the fp64 SRE order
    with relative tolerance ``tol`` (problems are recorded in the returned Schedule).
    ``fold_sets_in`` replays an external schedule given as the folded positions of each chunk (any
    position, so it can also name tokens of earlier calls, as a decode step does); it is validated in
    the same way.  At most one of ``fold_at_in`` and ``fold_sets_in`` may be given.
    ``on_chunk_end(c, st)`` is called once per chunk, after the chunk's folds and commit.
    ``read_mask`` (READ_*) selects the memories the queries read (reading R18); ``score_rule`` one of
    SCORE_RULES ranks the candidates (SRE against the state, or reading R19's accumulated scores)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d_k = q.shape
    eta, lam = st.eta, st.lam
    if C < 1:
        raise ValueError("chunk length must be >= 1")
    if lam > 0 and eta < C - 1:
        raise ValueError("reading R4: lambda > 0 needs eta >= C - 1")
    if not read_mask & READ_WINDOW or read_mask & ~READ_ALL:
        raise ValueError("reading R18: a read mask holds the window and nothing but the three memories")
    if score_rule not in SCORE_RULES:
        raise ValueError(f"unknown score rule {score_rule!r}")
    if fold_at_in is not None and fold_sets_in is not None:
        raise ValueError("give fold_at_in or fold_sets_in, not both")
    t0 = st.t
    st.ensure(t0 + n)
    st.K[t0:t0 + n] = k
    st.V[t0:t0 + n] = v
    y = np.zeros((n, v.shape[1]))
    sched = Schedule(fold_at=np.full(n, -1, dtype=np.int64))
    for c, a in enumerate(range(t0, t0 + n, C)):
        b = min(a + C, t0 + n)
        # 1. the tokens that leave the window while the chunk runs: i + eta in [a, b)
        X = [i for i in range(a - eta, b - eta) if i >= 0]
        # 2. candidates = sparse cache U leaving tokens; score only if there are more than lambda
        E = sorted(set(st.cache) | set(X))
        scores = None
        if len(E) > lam and lam > 0:
            if score_rule == "sre":
                scores = dict(zip(E, sre(phi(st.K[E]), st.V[E], st.H, st.s)))
            else:   # reading R19: what queries before the chunk start have added
                scores = {i: float(st.score[i]) for i in E}
        gap = None
        if fold_at_in is None and fold_sets_in is None:
            if len(E) <= lam:
                kept, S = E, []
            elif lam == 0:
                kept, S = [], E
            else:
                order = sorted(E, key=lambda i: (-scores[i], i))   # SRE descending, older first
                kept, S = sorted(order[:lam]), sorted(order[lam:])
                hi = scores[order[lam - 1]]
                gap = (hi - scores[order[lam]]) / hi if hi > 0 else 0.0
        else:
            if fold_at_in is not None:
                S = sorted(i for i in E if i >= t0 and fold_at_in[i - t0] == c)
            else:
                given = sorted(int(i) for i in fold_sets_in[c])
                S = [i for i in given if i in set(E)]
                if len(S) != len(given):
                    sched.problems.append((c, "not a candidate", sorted(set(given) - set(E))))
            kept = sorted(set(E) - set(S))
            if len(kept) != min(lam, len(E)):
                sched.problems.append((c, "size", len(kept), min(lam, len(E))))
            if scores is not None and S and kept:
                lo = min(scores[i] for i in kept)
                hi = max(scores[i] for i in S)
                if hi > 0:
                    sched.worst_inversion = max(sched.worst_inversion, (hi - lo) / hi)
                if lo < hi * (1.0 - tol):
                    sched.problems.append((c, "order", lo, hi))
        sched.chunk_start.append(a)
        sched.folded.append(S)
        sched.kept.append(kept)
        sched.gap.append(gap)
        for i in S:
            if i >= t0:
                sched.fold_at[i - t0] = c
        # 3. a folded token becomes linear at tau = max(exit time, chunk start)  (reading R3)
        tau = {i: max(i + eta, a) for i in S}
        phi_S = {i: phi(st.K[i][None, :])[0] for i in S}
        v_S = {i: st.V[i].copy() for i in S}
        kept_set = set(kept)
        assert all(i <= a for i in kept), "reading R4 violated: a kept token is newer than the chunk"
        # 4. token-by-token read-out (Eq. (14)) over window U kept cache, plus the linear state
        for t in range(a, b):
            for i in S:
                if tau[i] == t:
                    st.H += np.outer(phi_S[i], v_S[i])
                    st.s += phi_S[i]
            win = st.window(t)
            extra = [i for i in kept if i < win.start] if read_mask & READ_SPARSE else []
            idx = np.concatenate([np.arange(win.start, win.stop, dtype=np.int64),
                                  np.asarray(extra, dtype=np.int64)])
            phi_q = phi(q[t - t0][None, :])[0]
            y[t - t0] = exact_attention_read(q[t - t0], phi_q, st.H, st.s, st.K[idx], st.V[idx], d_k,
                                             use_state=bool(read_mask & READ_STATE))
            if score_rule != "sre" and len(win) > 0:   # query t adds to every key in its window
                wi = np.arange(win.start, win.stop, dtype=np.int64)
                st.score[wi] += query_score(score_rule, q[t - t0], phi_q, st.K[wi], phi(st.K[wi]), d_k)
        # 5. commit: G <- G', folded tokens lose their exact KV
        for i in S:
            st.forget(i)
            st.folded.append(i)
        st.cache = kept
        st.t = b
        assert kept_set.isdisjoint(S)
        if on_chunk_end is not None:
            on_chunk_end(c, st)
    return y, sched


def decode_step(st: SeqState, phi, q, k, v, read_mask: int = READ_ALL, score_rule: str = "sre",
                fold: Optional[int] = None, tol: float = 0.0, want_schedule: bool = False):
    """One decode token (section 2.4 single-token update, then Eq. (14)): prefill with C = 1.

    ``fold`` (a position, or -1 for none) replays an external decision in place of the top-lambda and
    validates it with relative tolerance ``tol`` (see ``replay``).  Returns (y [d_v], folded position
    or -1), plus the step's Schedule when ``want_schedule``."""
    sets = None if fold is None else [[] if fold < 0 else [int(fold)]]
    y, sched = prefill(st, phi, np.asarray(q)[None, :], np.asarray(k)[None, :],
                       np.asarray(v)[None, :], C=1, read_mask=read_mask, score_rule=score_rule,
                       tol=tol, fold_sets_in=sets)
    S = sched.folded[0]
    out = (y[0], (S[0] if S else -1))
    return out + (sched,) if want_schedule else out


def replay(st: SeqState, phi, q, k, v, C: int, fold_at: np.ndarray, tol: float):
    """Read-out under an external schedule (e.g. one taken in lower precision), with validation.

    Valid: every chunk keeps min(lambda, |E|) candidates and min_{kept} SRE >= max_{folded} SRE *
    (1 - tol), SRE in fp64 against the chunk-start state.  Mutates ``st``; returns (y, Schedule)."""
    return prefill(st, phi, q, k, v, C, fold_at_in=np.asarray(fold_at), tol=tol)


def sre_collisions(st: SeqState, phi, q, k, v, C: int, fold_at_in: Optional[np.ndarray] = None,
                   tol: float = 0.0, relative: bool = False):
    """Collision map of one prefill call (section 4.4, Fig. 3; relative form Fig. 10, Eq. (26)).

    Runs ``prefill`` (mutating ``st``; ``fold_at_in`` / ``tol`` as there) and returns (M, y, Schedule)
    with M [n_chunks][n]: M[r, i] = SRE(phi(k_i), v_i | H_r, s_r) for the state (H_r, s_r) at the end
    of chunk r, for every input token i folded in chunk r or before; 0 for a token not in that state
    (still in the window or the cache, reading R17).  relative: each entry minus the token's entry in
    the row of its own fold, so that row reads 0 and rows before it stay 0."""
    states = []
    y, sched = prefill(st, phi, q, k, v, C, fold_at_in=fold_at_in, tol=tol,
                       on_chunk_end=lambda c, s_: states.append((s_.H.copy(), s_.s.copy())))
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    phi_k = phi(k)
    fa = sched.fold_at
    M = np.zeros((len(states), k.shape[0]))
    for r, (H, s) in enumerate(states):
        held = (fa >= 0) & (fa <= r)
        if held.any():
            M[r, held] = sre(phi_k[held], v[held], H, s)
    if relative:
        for i in np.nonzero(fa >= 0)[0]:
            first = M[fa[i], i]
            M[fa[i]:, i] -= first
    return M, y, sched


def state_elements(t: int, d_k: int, d_v: int, D: int, eta: int, lam: int) -> int:
    """Per-head persistent element count (section 2.7): min{t(d_k+d_v), (eta+lam)(d_k+d_v)+D d_v+D}."""
    return min(t * (d_k + d_v), (eta + lam) * (d_k + d_v) + D * d_v + D)

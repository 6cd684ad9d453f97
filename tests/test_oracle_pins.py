"""Pins for the fp64 oracle: each check fixes the oracle to something other than itself.

Closed forms, textbook special cases (causal softmax attention from torch's SDPA, brute-force
quadratic kernel attention), hand-derived schedules, invariants of the method and an independent
per-pair evaluation of Eq. (14).  Citations are to the LoLA reading notes (cc.laoqi.cc, paper
2505.23666 v3), part 2 ("Method").
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import lola_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _rand_problem(seed, n, d_k=8, d_v=6, D=8, kind="softmax_pm", scale=1.0):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((d_k, D if kind == "elu1" else D // 2)) / np.sqrt(d_k)
    q = rng.standard_normal((n, d_k)) * scale
    k = rng.standard_normal((n, d_k)) * scale
    v = rng.standard_normal((n, d_v))
    return O.make_phi(kind, W), q, k, v


def _run(phi, q, k, v, eta, lam, C, D=8):
    st = O.new_state(q.shape[1], v.shape[1], D, eta, lam)
    y, sched = O.prefill(st, phi, q, k, v, C)
    return y, sched, st


# ------------------------------------------------------------------------------------------------
# Feature maps: hand-computed values and closed-form properties (2.2, 3.1).
# ------------------------------------------------------------------------------------------------

def test_phi_hand_values():
    g = _gold("phi_hand_values.json")
    for key, fn in (("softmax_pm", O.phi_softmax_pm), ("softmax_pm_zero", O.phi_softmax_pm),
                    ("elu1", O.phi_elu1)):
        case = g[key]
        got = fn(np.array(case["x"]), np.array(case["W"]))
        np.testing.assert_allclose(got, case["phi"], rtol=0, atol=1e-12)


def test_phi_softmax_pm_halves_sum_to_one_and_positive():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 16)) * 3
    W = rng.standard_normal((16, 32))
    f = O.phi_softmax_pm(x, W)
    assert f.shape == (50, 64)
    np.testing.assert_allclose(f[:, :32].sum(1), 1.0, atol=1e-12)
    np.testing.assert_allclose(f[:, 32:].sum(1), 1.0, atol=1e-12)
    assert (f > 0).all()


def test_phi_elu1_positive_and_matches_piecewise():
    x = np.array([[1.0]])
    for z in (-3.0, -0.5, 0.0, 0.25, 4.0):
        got = O.phi_elu1(x, np.array([[z]]))[0, 0]
        want = np.exp(z) if z <= 0 else z + 1.0
        assert got == pytest.approx(want, abs=1e-15)
        assert got > 0


# ------------------------------------------------------------------------------------------------
# SRE (2.3, Eq. (10)).
# ------------------------------------------------------------------------------------------------

def test_sre_single_kv_recalls_itself():
    """Invariant (c): a state that holds one KV recalls it exactly, whatever the key."""
    rng = np.random.default_rng(1)
    f0 = rng.random(8) + 0.1
    v0 = rng.standard_normal(5)
    H = np.outer(f0, v0)
    s = f0.copy()
    assert O.sre(f0, v0, H, s)[0] == pytest.approx(0.0, abs=1e-12)
    others = rng.random((4, 8)) + 0.1
    vs = rng.standard_normal((4, 5))
    np.testing.assert_allclose(O.sre(others, vs, H, s), np.linalg.norm(vs - v0, axis=1), atol=1e-12)


def test_sre_teaching_example_opposite_values():
    """2.4 teaching example: equal features with values +1 / -1 in one state recall 0; error = |v|."""
    f = np.array([0.2, 0.3, 0.5, 0.1])
    v1 = np.array([1.0])
    H = np.outer(f, v1) + np.outer(f, -v1)
    s = 2 * f
    np.testing.assert_allclose(O.sre(np.stack([f, f]), np.array([[1.0], [-1.0]]), H, s), [1.0, 1.0])


def test_sre_hand_values_two_token_state():
    # phi_a = (1, 0) with v_a = 2, phi_b = (0, 1) with v_b = 4: H = [[2], [4]], s = (1, 1)
    H = np.array([[2.0], [4.0]])
    s = np.array([1.0, 1.0])
    # phi(k) = (1, 1): recall (2 + 4) / 2 = 3, v = 5 -> 2.   phi(k) = (3, 1): recall 10/4, v = 0 -> 2.5
    got = O.sre(np.array([[1.0, 1.0], [3.0, 1.0]]), np.array([[5.0], [0.0]]), H, s)
    np.testing.assert_allclose(got, [2.0, 2.5], atol=1e-15)


def test_sre_empty_state_is_value_norm():
    """Reading R5: with phi(k)^T s = 0 the recall is zero."""
    v = np.array([[3.0, 4.0], [0.0, 1.0]])
    got = O.sre(np.ones((2, 3)), v, np.zeros((3, 2)), np.zeros(3))
    np.testing.assert_allclose(got, [5.0, 1.0])


# ------------------------------------------------------------------------------------------------
# Hand-derived schedule (2.4 single-token update, Eqs. (11)-(13)).
# ------------------------------------------------------------------------------------------------

def test_hand_schedule():
    g = _gold("hand_schedule.json")
    v = np.array(g["v"])
    n = len(v)
    rng = np.random.default_rng(7)
    k = rng.standard_normal((n, 2))
    for a, b in g["k_equal_pairs"]:
        k[b] = k[a]
    q = rng.standard_normal((n, 2))
    phi = O.make_phi("softmax_pm", rng.standard_normal((2, 3)))
    st = O.new_state(2, 2, 6, g["eta"], g["lam"])
    _, sched = O.prefill(st, phi, q, k, v, g["C"])
    fold_time = {str(i): int(sched.fold_at[i]) for i in range(n) if sched.fold_at[i] >= 0}
    assert fold_time == g["fold_time_of_token"]
    assert st.cache == g["cache_after_t5"]


def test_exact_tie_keeps_older_position():
    """Reading R6 (2.4, exactly lambda kept): an exact duplicate competes with its original for the
    one slot, so both have the same SRE against the same state; the older copy stays, the newer is
    folded.  Worked by hand with eta = lambda = C = 1 over four tokens:
      t = 1: token 0 leaves the window, the cache is empty, so it is kept (no scoring);
      t = 2: token 1 leaves; candidates {0, 1} score against the empty state, SRE = ||v|| (reading R5):
             1 for token 0, 3 for token 1, so token 0 is folded and token 1 kept;
      t = 3: token 2 (a copy of token 1) leaves; candidates {1, 2} tie exactly; token 1 is kept."""
    k = np.array([[0.3, -0.2], [1.1, 0.4], [1.1, 0.4], [-0.5, 0.9]])
    v = np.array([[1.0, 0.0], [0.0, 3.0], [0.0, 3.0], [5.0, 5.0]])
    q = np.array([[0.1, 0.2], [0.3, -0.1], [-0.4, 0.5], [0.2, 0.2]])
    phi = O.make_phi("softmax_pm", np.array([[0.5, -0.3], [0.2, 0.8]]))
    st = O.new_state(2, 2, 4, 1, 1)
    _, sched = O.prefill(st, phi, q, k, v, C=1)
    assert sched.fold_at.tolist() == [2, -1, 3, -1]
    assert st.cache == [1]
    assert sched.gap[3] == 0.0        # the last allocation was decided by the tie rule alone
    assert sched.folded[3] == [2] and sched.kept[3] == [1]


def _chunked_tie_case():
    """A duplicate pair inside one leaving block (C = 4): tokens 4 and 5 carry the same key and the
    same large value, so in chunk 2 (positions 8..11, leaving block 4..7) they have the two largest
    SREs and tie for the single cache slot."""
    phi, q, k, v = _rand_problem(31, 16, d_k=6, d_v=6)
    k[5] = k[4]
    v[4] = 100.0 * v[4]
    v[5] = v[4]
    st = O.new_state(6, 6, 8, 4, 1)
    _, sched = O.prefill(st, phi, q, k, v, C=4)
    return sched


def test_exact_tie_in_a_chunk_keeps_older_position():
    """Reading R6 in a chunked allocation (2.6): |E| = 5 > lambda = 1 and the boundary falls inside
    an exact tie; the older token 4 is kept, token 5 is folded in chunk 2."""
    sched = _chunked_tie_case()
    assert sched.chunk_start[2] == 8 and 4 in sched.kept[2] + sched.folded[2]
    assert len(sched.kept[2]) + len(sched.folded[2]) == 5
    assert sched.gap[2] == 0.0
    assert sched.kept[2] == [4]
    assert sched.fold_at[5] == 2


def test_tie_pins_catch_a_reversed_tie_rule(monkeypatch):
    """Negative control: plant 'equal SRE keeps the newer position' in the oracle's ranking; both tie
    pins must fail."""
    import builtins

    def newer_first(it, key=None, reverse=False):
        if key is None:
            return builtins.sorted(it, reverse=reverse)
        return builtins.sorted(it, key=lambda i: (key(i)[0], -key(i)[1]), reverse=reverse)
    monkeypatch.setattr(O, "sorted", newer_first, raising=False)
    with pytest.raises(AssertionError):
        test_exact_tie_keeps_older_position()
    with pytest.raises(AssertionError):
        test_exact_tie_in_a_chunk_keeps_older_position()


def test_decode_replay_validates_the_fold():
    """A decode step replayed under an external fold (2.4, one fold per overflowing step): the
    oracle's own choice replays to the same output with no problem; folding the candidate with the
    largest SRE instead is reported as an order problem, and a position that is no candidate as such."""
    phi, q, k, v = _rand_problem(32, 40)
    st = O.new_state(8, 6, 8, 5, 4)
    O.prefill(st, phi, q[:30], k[:30], v[:30], C=5)
    base = st.copy()
    y_o, f_o, sch = O.decode_step(base.copy(), phi, q[30], k[30], v[30], want_schedule=True)
    assert f_o >= 0 and not sch.problems
    y_r, f_r, sch_r = O.decode_step(base.copy(), phi, q[30], k[30], v[30], fold=f_o, want_schedule=True)
    assert f_r == f_o and not sch_r.problems
    np.testing.assert_array_equal(y_r, y_o)
    E = sorted(set(base.cache) | {30 - 5})
    scores = O.sre(phi(base.K[E]), base.V[E], base.H, base.s)
    worst = E[int(np.argmax(scores))]
    _, _, sch_w = O.decode_step(base.copy(), phi, q[30], k[30], v[30], fold=worst, tol=2e-2, want_schedule=True)
    assert [p[1] for p in sch_w.problems] == ["order"]
    _, _, sch_n = O.decode_step(base.copy(), phi, q[30], k[30], v[30], fold=29, want_schedule=True)
    assert "not a candidate" in [p[1] for p in sch_n.problems]


# ------------------------------------------------------------------------------------------------
# Textbook special cases.
# ------------------------------------------------------------------------------------------------

def _causal_softmax_torch(q, k, v):
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None], torch.from_numpy(v)[None, None],
        is_causal=True)
    return out[0, 0].numpy()


@pytest.mark.parametrize("C,lam", [(1, 0), (4, 3), (16, 8), (7, 100)])
def test_invariant_b_window_covers_everything_is_causal_softmax(C, lam):
    """Invariant (b): eta >= n means nothing ever leaves the window: exact causal softmax."""
    phi, q, k, v = _rand_problem(11, 40)
    y, sched, _ = _run(phi, q, k, v, eta=40, lam=lam, C=C)
    np.testing.assert_allclose(y, _causal_softmax_torch(q, k, v), rtol=1e-12, atol=1e-12)
    assert all(len(S) == 0 for S in sched.folded)


@pytest.mark.parametrize("C", [1, 2, 5])
def test_cache_large_enough_is_causal_softmax(C):
    """lambda >= n - eta: every leaving token fits in the cache, nothing is folded (2.4: keep all)."""
    n, eta = 37, 6
    phi, q, k, v = _rand_problem(12, n)
    y, sched, st = _run(phi, q, k, v, eta=eta, lam=n - eta, C=C)
    np.testing.assert_allclose(y, _causal_softmax_torch(q, k, v), rtol=1e-12, atol=1e-12)
    assert st.folded == []


def _brute_force_phi_attention(phi, q, k, v):
    fq, fk = phi(q), phi(k)
    A = np.tril(fq @ fk.T)
    return (A @ v) / A.sum(1, keepdims=True)


@pytest.mark.parametrize("kind", ["softmax_pm", "elu1"])
@pytest.mark.parametrize("C", [1, 3, 8, 64])
def test_invariant_a_no_window_no_cache_is_linear_attention(kind, C):
    """Invariant (a): eta = lambda = 0 is brute-force quadratic phi-kernel attention, any C."""
    phi, q, k, v = _rand_problem(13, 45, kind=kind)
    y, _, st = _run(phi, q, k, v, eta=0, lam=0, C=C)
    np.testing.assert_allclose(y, _brute_force_phi_attention(phi, q, k, v), rtol=1e-11, atol=1e-12)
    assert sorted(st.folded) == list(range(45))


def _lolcats_closed_form(phi, q, k, v, eta):
    """lambda = 0: key i is read through phi for t - i >= eta and through exp otherwise."""
    n, d_k = q.shape
    fq, fk = phi(q), phi(k)
    y = np.zeros_like(v)
    for t in range(n):
        w = np.zeros(n)
        for i in range(t + 1):
            w[i] = fq[t] @ fk[i] if t - i >= eta else np.exp(q[t] @ k[i] / np.sqrt(d_k))
        y[t] = w @ v / w.sum()
    return y


@pytest.mark.parametrize("C", [1, 4, 7])
def test_lambda_zero_is_sliding_window_plus_linear(C):
    """lambda = 0: window of eta exact tokens plus linear attention over the rest, independent of C."""
    eta = 7
    phi, q, k, v = _rand_problem(14, 40)
    y, _, _ = _run(phi, q, k, v, eta=eta, lam=0, C=C)
    np.testing.assert_allclose(y, _lolcats_closed_form(phi, q, k, v, eta), rtol=1e-11, atol=1e-12)


# ------------------------------------------------------------------------------------------------
# Invariants of the allocation (2.2 no double counting, 2.4 greedy irreversible top-lambda).
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("eta,lam,C", [(4, 3, 1), (6, 5, 4), (8, 8, 9), (3, 0, 2), (0, 2, 1)])
def test_invariant_d_partition_every_chunk(eta, lam, C):
    n = 50
    phi, q, k, v = _rand_problem(15, n)
    st = O.new_state(8, 6, 8, eta, lam)
    folded_before = []
    H = np.zeros((8, 6))
    for a in range(0, n, C):
        b = min(a + C, n)
        O.prefill(st, phi, q[a:b], k[a:b], v[a:b], C)
        window = set(range(max(0, b - eta), b))
        cache, folded = set(st.cache), set(st.folded)
        assert len(st.cache) <= lam
        assert window.isdisjoint(cache) and window.isdisjoint(folded) and cache.isdisjoint(folded)
        assert window | cache | folded == set(range(b))
        assert st.folded[:len(folded_before)] == folded_before      # folds are never undone
        folded_before = list(st.folded)
        # (H, s) hold exactly the folded tokens (2.2: only the KV allocated to the state)
        fk = phi(k[st.folded]) if st.folded else np.zeros((0, 8))
        H = fk.T @ v[st.folded] if st.folded else np.zeros((8, 6))
        np.testing.assert_allclose(st.H, H, atol=1e-12)
        np.testing.assert_allclose(st.s, fk.sum(0), atol=1e-12)


def test_kept_set_is_top_lambda_by_brute_force():
    """Each allocation keeps a size-lambda subset whose smallest SRE beats every folded SRE."""
    n, eta, lam, C = 60, 5, 6, 4
    phi, q, k, v = _rand_problem(16, n)
    st = O.new_state(8, 6, 8, eta, lam)
    for a in range(0, n, C):
        before = st.copy()
        _, sched = O.prefill(st, phi, q[a:a + C], k[a:a + C], v[a:a + C], C)
        S, kept = sched.folded[0], sched.kept[0]
        if not S:
            continue
        cand = sorted(set(S) | set(kept))
        scores = {}
        for i in cand:   # score each candidate separately, by the definition
            fk = phi(k[i][None])[0]
            den = fk @ before.s
            recall = before.H.T @ fk / den if den != 0 else np.zeros(6)
            scores[i] = np.linalg.norm(recall - v[i])
        assert len(kept) == lam
        assert min(scores[i] for i in kept) >= max(scores[i] for i in S)


def test_equivariance_under_affine_values_detects_norm_ranking():
    """v -> alpha Q v + c (Q orthogonal) scales every SRE by |alpha| once the state is non-empty, so
    the schedule is unchanged and y -> alpha Q y + c.  A 'rank by ||v||' rule would fail this."""
    n, eta, lam, C, d_v = 70, 5, 4, 3, 6
    phi, q, k, v = _rand_problem(17, n + 10, d_v=d_v)
    rng = np.random.default_rng(99)
    Qm, _ = np.linalg.qr(rng.standard_normal((d_v, d_v)))
    alpha, cvec = -1.7, rng.standard_normal(d_v) * 25.0

    def run(vals):
        st = O.new_state(8, d_v, 8, eta, 0)
        O.prefill(st, phi, q[:10], k[:10], vals[:10], C)     # warm-up with lambda = 0: s != 0
        st.lam = lam
        y, sched = O.prefill(st, phi, q[10:], k[10:], vals[10:], C)
        return y, sched

    y1, s1 = run(v)
    v2 = v @ (alpha * Qm).T + cvec
    y2, s2 = run(v2)
    assert s1.folded == s2.folded and sum(len(S) for S in s1.folded) > 10
    np.testing.assert_allclose(y2, y1 @ (alpha * Qm).T + cvec, rtol=1e-9, atol=1e-9)


def test_equivariance_catches_a_planted_norm_ranking(monkeypatch):
    """Negative control: plant 'SRE = ||v||' in the oracle and the equivariance check must break."""
    monkeypatch.setattr(O, "sre", lambda phi_k, v, H, s: np.linalg.norm(np.atleast_2d(v), axis=1))
    with pytest.raises(AssertionError):
        test_equivariance_under_affine_values_detects_norm_ranking()


# ------------------------------------------------------------------------------------------------
# Schedule plumbing: C = 1 equals decode steps; chunk-aligned splits are invisible.
# ------------------------------------------------------------------------------------------------

def test_prefill_c1_equals_decode_steps():
    n, eta, lam = 30, 4, 3
    phi, q, k, v = _rand_problem(18, n)
    y1, s1, st1 = _run(phi, q, k, v, eta, lam, 1)
    st2 = O.new_state(8, 6, 8, eta, lam)
    ys, folds = [], []
    for t in range(n):
        y, f = O.decode_step(st2, phi, q[t], k[t], v[t])
        ys.append(y)
        folds.append(f)
    np.testing.assert_array_equal(np.array(ys), y1)
    assert [f for f in folds if f >= 0] == [S[0] for S in s1.folded if S]


@pytest.mark.parametrize("split", [8, 16, 24])
def test_chunk_aligned_split_invariance(split):
    n, eta, lam, C = 50, 9, 6, 8
    phi, q, k, v = _rand_problem(19, n)
    y_all, _, st_all = _run(phi, q, k, v, eta, lam, C)
    st = O.new_state(8, 6, 8, eta, lam)
    ya, _ = O.prefill(st, phi, q[:split], k[:split], v[:split], C)
    yb, _ = O.prefill(st, phi, q[split:], k[split:], v[split:], C)
    np.testing.assert_allclose(np.concatenate([ya, yb]), y_all, rtol=1e-13, atol=1e-13)
    assert st.cache == st_all.cache and st.folded == st_all.folded


def test_state_from_arrays_round_trip():
    n, eta, lam, C = 40, 6, 5, 4
    phi, q, k, v = _rand_problem(20, n + 8)
    y_ref, _, _ = _run(phi, q, k, v, eta, lam, C)
    st = O.new_state(8, 6, 8, eta, lam)
    O.prefill(st, phi, q[:n], k[:n], v[:n], C)
    ring_k = np.zeros((eta, 8))
    ring_v = np.zeros((eta, 6))
    for p in range(n - eta, n):
        ring_k[p % eta], ring_v[p % eta] = k[p], v[p]
    cache_pos = np.full(lam + 2, -1)
    ck, cv = np.zeros((lam + 2, 8)), np.zeros((lam + 2, 6))
    for j, p in enumerate(reversed(st.cache)):
        cache_pos[j + 2], ck[j + 2], cv[j + 2] = p, k[p], v[p]
    st2 = O.state_from_arrays(n, eta, lam, st.H, st.s, ring_k, ring_v, ck, cv, cache_pos)
    y2, _ = O.prefill(st2, phi, q[n:], k[n:], v[n:], C)
    np.testing.assert_allclose(y2, y_ref[n:], rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------------------------------------
# Eq. (14) evaluated directly, pair by pair, from the schedule: an independent read-out.
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("eta,lam,C", [(6, 5, 4), (5, 8, 6), (0, 3, 1), (10, 4, 1), (12, 12, 13)])
def test_recurrent_path_equals_direct_per_pair_evaluation(eta, lam, C):
    n = 64
    phi, q, k, v = _rand_problem(21, n, scale=1.3)
    y, sched, _ = _run(phi, q, k, v, eta, lam, C)
    fq, fk = phi(q), phi(k)
    d_k = q.shape[1]
    fold_chunk = {}
    for c, S in enumerate(sched.folded):
        for i in S:
            fold_chunk[i] = c
    for t in range(n):
        c = t // C
        kept = set(sched.kept[c])
        num = np.zeros(v.shape[1])
        den = 0.0
        for i in range(t + 1):
            fc = fold_chunk.get(i, n)
            linear = fc <= c and max(i + eta, fc * C) <= t      # folded, and visible by time t
            exact = (t - eta + 1 <= i) or (i in kept)
            assert linear != exact, (t, i)           # every past token is read exactly one way
            w = fq[t] @ fk[i] if linear else np.exp(q[t] @ k[i] / np.sqrt(d_k))
            num += w * v[i]
            den += w
        np.testing.assert_allclose(y[t], num / den, rtol=1e-11, atol=1e-12)


# ------------------------------------------------------------------------------------------------
# State size accounting (2.7) and the page's own arithmetic.
# ------------------------------------------------------------------------------------------------

def test_state_size_ratio_matches_page():
    g = _gold("state_size_ratio.json")
    full = g["t"] * (g["d_k"] + g["d_v"])
    lola = O.state_elements(g["t"], g["d_k"], g["d_v"], g["D"], g["eta"], g["lam"])
    assert round(full / lola, g["printed_digits"]) == g["ratio_printed"]
    assert O.state_elements(5, 4, 4, 8, 2, 2) == 40                  # 5 * (4 + 4): below the budget
    assert O.state_elements(10, 4, 4, 8, 2, 2) == 72                 # 4 * 8 + 8 * 4 + 8: saturated
    assert O.state_elements(10**9, 128, 128, 128, 256, 256) == 147584


def test_replay_of_own_schedule_reproduces_output():
    n, eta, lam, C = 60, 7, 6, 5
    phi, q, k, v = _rand_problem(22, n)
    y, sched, _ = _run(phi, q, k, v, eta, lam, C)
    st = O.new_state(8, 6, 8, eta, lam)
    y2, s2 = O.replay(st, phi, q, k, v, C, sched.fold_at, tol=0.0)
    assert s2.problems == []
    np.testing.assert_array_equal(y2, y)


def test_replay_flags_a_wrong_schedule():
    n, eta, lam, C = 60, 7, 6, 5
    phi, q, k, v = _rand_problem(23, n)
    y, sched, _ = _run(phi, q, k, v, eta, lam, C)
    bad = sched.fold_at.copy()
    c = next(c for c, S in enumerate(sched.folded) if S and sched.kept[c])
    i_out, i_in = sched.folded[c][0], max(sched.kept[c])   # swap a folded and a kept candidate
    bad[i_out], bad[i_in] = -1, c
    st = O.new_state(8, 6, 8, eta, lam)
    _, s2 = O.replay(st, phi, q, k, v, C, bad, tol=0.0)
    assert s2.problems


# ------------------------------------------------------------------------------------------------
# Collision map (4.4, Fig. 3; relative form Fig. 10, Eq. (26)).
# ------------------------------------------------------------------------------------------------

def _pairwise_sre(phi_k, v, members, i):
    """SRE of token i against the state holding exactly ``members``, in kernel form: the recall is the
    kappa-weighted mean of the members' values with kappa(i, j) = phi(k_i)^T phi(k_j), written with
    scalar loops (no H, no s)."""
    num = np.zeros(v.shape[1])
    den = 0.0
    for j in members:
        kap = sum(float(phi_k[i, e]) * float(phi_k[j, e]) for e in range(phi_k.shape[1]))
        num += kap * v[j]
        den += kap
    rec = num / den if den != 0.0 else np.zeros_like(num)
    return float(np.sqrt(((rec - v[i]) ** 2).sum()))


def test_collision_single_kv_recalls_itself():
    # (c) of the method's checks: a state holding one KV recalls v exactly, so its map entry is 0.
    phi, q, k, v = _rand_problem(30, 1)
    st = O.new_state(8, 6, 8, 0, 0)
    M, _, sched = O.sre_collisions(st, phi, q, k, v, C=1)
    assert M.shape == (1, 1) and sched.fold_at.tolist() == [0]
    assert abs(M[0, 0]) < 1e-12 * np.linalg.norm(v[0])


@pytest.mark.parametrize("relative", [False, True])
def test_collision_pure_linear_is_pairwise_kernel_form(relative):
    # eta = lambda = 0, C = 1: token i is written at step i, so row r holds tokens 0..r.
    phi, q, k, v = _rand_problem(31, 10)
    st = O.new_state(8, 6, 8, 0, 0)
    M, _, sched = O.sre_collisions(st, phi, q, k, v, C=1, relative=relative)
    assert sched.fold_at.tolist() == list(range(10))
    pk = phi(k)
    for r in range(10):
        for i in range(10):
            want = _pairwise_sre(pk, v, range(r + 1), i) if i <= r else 0.0
            if relative and i <= r:
                want -= _pairwise_sre(pk, v, range(i + 1), i)
            assert abs(M[r, i] - want) < 1e-10, (r, i, M[r, i], want)


def test_collision_one_hot_features_is_bucket_mean():
    # With one-hot features (bucket = argmax of the first D entries of k) two keys collide exactly
    # when they share a bucket, and the recall is the mean value of the bucket's stored KV.  A window
    # of eta and no cache: token i leaves the window at time i + eta, so chunk (i + eta) // C folds it.
    D, eta, C, n = 4, 4, 3, 23
    rng = np.random.default_rng(32)
    k = rng.standard_normal((n, 8))
    q = rng.standard_normal((n, 8))
    v = rng.standard_normal((n, 6))
    bucket = np.argmax(k[:, :D], axis=1)

    def onehot(x):
        x = np.atleast_2d(x)
        return np.eye(D)[np.argmax(x[:, :D], axis=1)]

    st = O.new_state(8, 6, D, eta, 0)
    M, _, sched = O.sre_collisions(st, onehot, q, k, v, C=C)
    fa_want = [(i + eta) // C if i + eta < n else -1 for i in range(n)]
    assert sched.fold_at.tolist() == fa_want
    for r in range(M.shape[0]):
        for i in range(n):
            if fa_want[i] < 0 or fa_want[i] > r:
                assert M[r, i] == 0.0
                continue
            same = [j for j in range(n) if bucket[j] == bucket[i] and 0 <= fa_want[j] <= r]
            want = np.linalg.norm(v[same].mean(axis=0) - v[i])
            assert abs(M[r, i] - want) < 1e-12, (r, i)


@pytest.mark.parametrize("relative", [False, True])
def test_collision_with_cache_matches_rebuilt_states(relative):
    # Window, cache and chunks together: row r must equal the SRE against the state rebuilt from the
    # schedule alone (every token folded in chunk r or before), and a token the cache holds past its
    # window exit keeps a zero column until its own fold.
    eta, lam, C, n = 6, 4, 4, 40
    phi, q, k, v = _rand_problem(33, n, scale=1.5)
    st = O.new_state(8, 6, 8, eta, lam)
    M, _, sched = O.sre_collisions(st, phi, q, k, v, C=C, relative=relative)
    fa = sched.fold_at
    pk = phi(k)
    held_late = [i for i in range(n) if fa[i] > (i + eta) // C or (fa[i] < 0 and i + eta < n)]
    assert held_late, "the cache never held a token past its window exit"
    for r in range(M.shape[0]):
        members = [j for j in range(n) if 0 <= fa[j] <= r]
        for i in range(n):
            if fa[i] < 0 or fa[i] > r:
                assert M[r, i] == 0.0
                continue
            want = _pairwise_sre(pk, v, members, i)
            if relative:
                first = [j for j in range(n) if 0 <= fa[j] <= fa[i]]
                want -= _pairwise_sre(pk, v, first, i)
            assert abs(M[r, i] - want) < 1e-10, (r, i)
    if relative:
        for i in np.nonzero(fa >= 0)[0]:
            assert M[fa[i], i] == 0.0


# ------------------------------------------------------------------------------------------------
# Read-branch masks (4.8, Table 12) and query-accumulated scoring rules (4.5, Table 4).
# ------------------------------------------------------------------------------------------------

def _sliding_window_softmax(q, k, v, eta):
    n, d_k = q.shape
    y = np.zeros_like(v)
    for t in range(n):
        lo = max(0, t - eta + 1)
        w = np.array([np.exp(float(np.dot(q[t], k[i])) / np.sqrt(d_k)) for i in range(lo, t + 1)])
        y[t] = w @ v[lo:t + 1] / w.sum()
    return y


@pytest.mark.parametrize("lam,C", [(0, 1), (5, 4), (9, 7)])
def test_read_window_only_is_sliding_window_softmax(lam, C):
    """Only the window read: softmax over the last eta tokens, whatever the cache and state hold."""
    eta, n = 6, 40
    phi, q, k, v = _rand_problem(40, n)
    st = O.new_state(8, 6, 8, eta, lam)
    y, _ = O.prefill(st, phi, q, k, v, C, read_mask=O.READ_WINDOW)
    np.testing.assert_allclose(y, _sliding_window_softmax(q, k, v, eta), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("mask", [O.READ_WINDOW, O.READ_WINDOW | O.READ_STATE, O.READ_WINDOW | O.READ_SPARSE,
                                  O.READ_ALL])
@pytest.mark.parametrize("eta,lam,C", [(6, 5, 4), (10, 4, 1), (5, 8, 6)])
def test_read_masks_per_pair_and_schedule_unchanged(mask, eta, lam, C):
    """Eq. (14) pair by pair with the hidden branches' terms removed from numerator and denominator;
    the allocation (fold sets, kept sets) is the unmasked one."""
    n = 48
    phi, q, k, v = _rand_problem(41, n, scale=1.3)
    _, sched_full, _ = _run(phi, q, k, v, eta, lam, C)
    st = O.new_state(8, 6, 8, eta, lam)
    y, sched = O.prefill(st, phi, q, k, v, C, read_mask=mask)
    assert sched.folded == sched_full.folded and sched.kept == sched_full.kept
    fq, fk = phi(q), phi(k)
    fold_chunk = {i: c for c, S in enumerate(sched.folded) for i in S}
    for t in range(n):
        c = t // C
        kept = set(sched.kept[c])
        num, den = np.zeros(v.shape[1]), 0.0
        for i in range(t + 1):
            fc = fold_chunk.get(i, n)
            if fc <= c and max(i + eta, fc * C) <= t:
                if not mask & O.READ_STATE:
                    continue
                w = fq[t] @ fk[i]
            elif t - eta + 1 <= i:
                w = np.exp(q[t] @ k[i] / np.sqrt(8))
            else:
                assert i in kept
                if not mask & O.READ_SPARSE:
                    continue
                w = np.exp(q[t] @ k[i] / np.sqrt(8))
            num += w * v[i]
            den += w
        np.testing.assert_allclose(y[t], num / den, rtol=1e-11, atol=1e-12)


def test_read_mask_without_window_is_rejected():
    phi, q, k, v = _rand_problem(42, 5)
    with pytest.raises(ValueError):
        O.prefill(O.new_state(8, 6, 8, 2, 2), phi, q, k, v, 1, read_mask=O.READ_STATE | O.READ_SPARSE)


def _rule_value(rule, qt, kt, fqt, fkt):
    """One query's contribution, written with scalar loops."""
    dot = sum(float(a) * float(b) for a, b in zip(qt, kt))
    e = float(np.exp(dot / np.sqrt(len(qt))))
    p = sum(float(a) * float(b) for a, b in zip(fqt, fkt))
    return {"kernel_sq": (e - p) ** 2, "kernel_abs": abs(e - p), "ratio": p / e, "attn": e}[rule]


@pytest.mark.parametrize("rule", ["kernel_sq", "kernel_abs", "ratio", "attn"])
@pytest.mark.parametrize("eta,lam,C", [(4, 3, 1), (6, 5, 4), (8, 4, 3)])
def test_query_scores_kept_sets_are_top_lambda_by_brute_force(rule, eta, lam, C):
    """At each chunk start a, a candidate's score is the sum of its contributions from the queries
    t < a whose window held it (i <= t <= i + eta - 1), and the kept set is the lambda largest
    (ties: older)."""
    n = 36
    phi, q, k, v = _rand_problem(43, n, scale=1.4)
    fq, fk = phi(q), phi(k)
    st = O.new_state(8, 6, 8, eta, lam)
    _, sched = O.prefill(st, phi, q, k, v, C, score_rule=rule)
    cache = []
    for c, a in enumerate(sched.chunk_start):
        b = min(a + C, n)
        E = sorted(set(cache) | {i for i in range(a - eta, b - eta) if i >= 0})
        if len(E) <= lam:
            want = E
        else:
            sc = {i: sum(_rule_value(rule, q[t], k[i], fq[t], fk[i]) for t in range(i, min(i + eta, a)))
                  for i in E}
            want = sorted(sorted(E, key=lambda i: (-sc[i], i))[:lam])
        assert sched.kept[c] == want, (c, sched.kept[c], want)
        cache = want


@pytest.mark.parametrize("rule", ["kernel_sq", "attn", "ratio"])
def test_query_scores_c1_final_cache_is_global_top_lambda(rule):
    """C = 1: a leaving token's score is complete and fixed, so greedy keep-the-largest leaves the
    lambda best of all tokens that have left the window."""
    n, eta, lam = 40, 5, 6
    phi, q, k, v = _rand_problem(44, n, scale=1.2)
    fq, fk = phi(q), phi(k)
    st = O.new_state(8, 6, 8, eta, lam)
    O.prefill(st, phi, q, k, v, 1, score_rule=rule)
    left = list(range(n - eta))
    sc = {i: sum(_rule_value(rule, q[t], k[i], fq[t], fk[i]) for t in range(i, i + eta)) for i in left}
    assert sorted(st.cache) == sorted(sorted(left, key=lambda i: (-sc[i], i))[:lam])


def test_query_scores_survive_a_call_boundary():
    """Scores carried by the state: two calls equal one call, with any rule."""
    phi, q, k, v = _rand_problem(45, 48, scale=1.2)
    for rule in ("kernel_abs", "attn"):
        st1 = O.new_state(8, 6, 8, 6, 5)
        y1, s1 = O.prefill(st1, phi, q, k, v, 4, score_rule=rule)
        st2 = O.new_state(8, 6, 8, 6, 5)
        ya, _ = O.prefill(st2, phi, q[:20], k[:20], v[:20], 4, score_rule=rule)
        yb, _ = O.prefill(st2, phi, q[20:], k[20:], v[20:], 4, score_rule=rule)
        np.testing.assert_allclose(np.concatenate([ya, yb]), y1, rtol=1e-12, atol=1e-13)
        assert sorted(st1.cache) == sorted(st2.cache)

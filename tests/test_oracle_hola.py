"""Pins for the HOLA oracle (oracle/hola_oracle.py): each check fixes it to something other than
itself.  Citations are to the HOLA reading notes (cc.laoqi.cc, paper 2607.02303 v1), part 2
("Method"): 3.1 Eq. (1) and 3.5 (gated delta rule), 3.3 Eqs. (5)-(6) (write magnitude, persistent
top-w cache, visible set), 3.4 Eq. (7) (cache-path normalisation)."""
import numpy as np
import pytest
import torch

from oracle import hola_oracle as H


def _problem(seed, n, d=8, dv=6):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, dv))
    alpha = rng.uniform(0.7, 1.0, n)
    beta = rng.uniform(0.0, 1.0, n)
    return q, k, v, alpha, beta


def test_single_write_closed_form():
    q, k, v, alpha, beta = _problem(1, 1)
    o, e, S = H.delta_rule(q, k, v, alpha, beta)
    kh = k[0] / np.linalg.norm(k[0])
    qh = q[0] / np.linalg.norm(q[0])
    np.testing.assert_allclose(e[0], v[0], atol=1e-14)                       # empty state predicts 0
    np.testing.assert_allclose(S, beta[0] * np.outer(kh, v[0]), atol=1e-14)
    np.testing.assert_allclose(o[0], beta[0] * float(kh @ qh) * v[0], atol=1e-14)
    assert abs(H.write_magnitude(e, beta)[0] - beta[0] * np.linalg.norm(v[0])) < 1e-14


def test_orthonormal_keys_store_exactly():
    """alpha = beta = 1 with orthonormal keys: nothing interferes, so S^T k_i = v_i for every stored
    pair, each residual is the value itself, and reading with q = k_i returns v_i."""
    d, n = 8, 6
    rng = np.random.default_rng(2)
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    k = Q[:n] * rng.uniform(0.5, 3.0, (n, 1))                               # any norms: unit() rescales
    v = rng.standard_normal((n, 5))
    o, e, S = H.delta_rule(k, k, v, np.ones(n), np.ones(n))
    np.testing.assert_allclose(e, v, atol=1e-12)
    np.testing.assert_allclose(o, v, atol=1e-12)
    np.testing.assert_allclose(Q[:n] @ S, v, atol=1e-12)


def test_repeated_association_writes_nothing():
    """The delta rule only writes what the state fails to predict: the same (k, v) again with
    alpha = beta = 1 has residual 0, so its write magnitude is 0."""
    q, k, v, _, _ = _problem(3, 1)
    k2, v2 = np.repeat(k, 2, axis=0), np.repeat(v, 2, axis=0)
    _, e, _ = H.delta_rule(np.repeat(q, 2, axis=0), k2, v2, np.ones(2), np.ones(2))
    assert np.linalg.norm(e[1]) < 1e-13
    assert H.write_magnitude(e, np.ones(2))[1] < 1e-13


def test_matches_the_householder_form():
    """GDN written as S_t = alpha_t (I - beta_t k k^T) S_{t-1} + beta_t k v^T (unit k): the same state."""
    q, k, v, alpha, beta = _problem(4, 30)
    _, _, S = H.delta_rule(q, k, v, alpha, beta)
    Sr = np.zeros((k.shape[1], v.shape[1]))
    for t in range(len(v)):
        kt = k[t] / np.linalg.norm(k[t])
        Sr = alpha[t] * (np.eye(len(kt)) - beta[t] * np.outer(kt, kt)) @ Sr + beta[t] * np.outer(kt, v[t])
    np.testing.assert_allclose(S, Sr, atol=1e-12)


def test_pure_decay_after_one_write():
    q, k, v, alpha, beta = _problem(5, 12)
    beta[1:] = 0.0
    o, _, _ = H.delta_rule(q, k, v, alpha, beta)
    S1 = beta[0] * np.outer(k[0] / np.linalg.norm(k[0]), v[0])
    for t in range(12):
        St = np.prod(alpha[1:t + 1]) * S1
        np.testing.assert_allclose(o[t], St.T @ (q[t] / np.linalg.norm(q[t])), atol=1e-13)


def test_persistent_cache_is_brute_force_top_w_with_older_ties():
    rng = np.random.default_rng(6)
    m = rng.integers(0, 5, 40).astype(float)                                   # many exact ties
    for upto in (0, 7, 23, 40):
        for w in (0, 3, 10, 64):
            got = H.persistent_cache(m, upto, w)
            order = sorted(range(upto), key=lambda i: (-m[i], i))
            assert got == sorted(order[:w])
            if w < upto and w > 0:     # every kept score >= every dropped one, ties kept older
                kept, drop = set(got), [i for i in range(upto) if i not in got]
                lo = min(m[i] for i in kept)
                assert all(m[i] < lo or (m[i] == lo and i > max(j for j in kept if m[j] == lo)) for i in drop)


@pytest.mark.parametrize("C", [1, 4, 16])
def test_large_cache_no_sink_is_causal_softmax_of_normalised_qk(C):
    """w >= n and a sink that never wins: every earlier token is visible (persistent cache plus the
    current chunk), so the cache path is causal softmax attention on the RMS-normalised q, k, which
    torch's attention computes on its own; the gate then scales it."""
    n, d = 20, 8
    q, k, v, alpha, beta = _problem(7, n, d=d, dv=5)
    rng = np.random.default_rng(8)
    gq, gk = rng.uniform(0.5, 1.5, d), rng.uniform(0.5, 1.5, d)
    gate = 0.3
    y, _, _, _, _ = H.hola_prefill(q, k, v, alpha, beta, gq, gk, sink=-1e30, gate=gate, C=C, w=n)
    o, _, _ = H.delta_rule(q, k, v, alpha, beta)
    qt = torch.from_numpy(H.rms_norm(q, gq))[None, None]
    kt = torch.from_numpy(H.rms_norm(k, gk))[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, torch.from_numpy(v)[None, None],
                                                           is_causal=True)[0, 0].numpy()
    g = 1.0 / (1.0 + np.exp(-gate))
    np.testing.assert_allclose(y, o + g * ref, rtol=1e-12, atol=1e-12)


def test_no_cache_c1_sees_itself_and_the_sink():
    """w = 0, C = 1: the visible set is the token itself plus the sink."""
    n, d = 10, 8
    q, k, v, alpha, beta = _problem(9, n, d=d)
    gq, gk = np.ones(d), np.ones(d)
    sink, gate = 0.4, -0.2
    y, _, cache, _, _ = H.hola_prefill(q, k, v, alpha, beta, gq, gk, sink=sink, gate=gate, C=1, w=0)
    o, _, _ = H.delta_rule(q, k, v, alpha, beta)
    assert cache == []
    g = 1.0 / (1.0 + np.exp(-gate))
    for t in range(n):
        qn = q[t] / np.sqrt((q[t] ** 2).mean() + 1e-6)
        kn = k[t] / np.sqrt((k[t] ** 2).mean() + 1e-6)
        p = np.exp(float(qn @ kn) / np.sqrt(d))
        np.testing.assert_allclose(y[t], o[t] + g * p * v[t] / (p + np.exp(sink)), rtol=1e-12)


def test_visible_set_bound_and_partition():
    """3.3: at most w + C + 1 entries (with the sink); the chunk part and the persistent part never
    share a position; the persistent cache only holds earlier chunks."""
    n, C, w = 50, 8, 5
    q, k, v, alpha, beta = _problem(10, n)
    _, _, _, m, caches = H.hola_prefill(q, k, v, alpha, beta, np.ones(8), np.ones(8), 0.0, 0.0, C, w)
    for c, A in enumerate(caches):
        a = c * C
        assert len(A) <= w and all(i < a for i in A)
        assert len(A) + C + 1 <= w + C + 1
        assert A == H.persistent_cache(m, a, w)


def test_gate_closed_is_the_state_alone():
    q, k, v, alpha, beta = _problem(11, 15)
    y, _, _, _, _ = H.hola_prefill(q, k, v, alpha, beta, np.ones(8), np.ones(8), 0.0, -80.0, 4, 3)
    o, _, _ = H.delta_rule(q, k, v, alpha, beta)
    np.testing.assert_allclose(y, o, atol=1e-30)


# ---- decode (reading H6): the step is pinned to the prefill, itself pinned above ----

def _gates(seed, d):
    rng = np.random.default_rng(seed + 1000)
    return rng.uniform(0.5, 1.5, d), rng.uniform(0.5, 1.5, d), float(rng.normal()), float(rng.normal())


@pytest.mark.parametrize("n0,steps,C,w", [(8, 9, 4, 3), (10, 7, 4, 3), (0, 13, 5, 2), (12, 12, 3, 6),
                                          (7, 10, 16, 4), (9, 6, 1, 2), (6, 8, 4, 0)])
def test_decode_steps_continue_the_prefill(n0, steps, C, w):
    """Prefill of n0 tokens then decode steps over the next ones gives the prefill of n0 + steps tokens:
    the outputs, the final state and the persistent cache (chunk closes inside the decode included)."""
    n = n0 + steps
    q, k, v, alpha, beta = _problem(30 + n0 + 7 * C, n, d=8, dv=8)
    gq, gk, sink, gate = _gates(n0 + C, 8)
    y_ref, S_ref, cache_ref, m_ref, _ = H.hola_prefill(q, k, v, alpha, beta, gq, gk, sink, gate, C, w)
    st = H.hola_state_after_prefill(q[:n0], k[:n0], v[:n0], alpha[:n0], beta[:n0], C, w)
    assert st.t == n0
    for t in range(n0, n):
        y_t = H.hola_decode_step(st, q[t], k[t], v[t], alpha[t], beta[t], gq, gk, sink, gate, C, w)
        np.testing.assert_allclose(y_t, y_ref[t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st.S, S_ref, rtol=1e-12, atol=1e-12)
    # the memory after n tokens: cache at the start of the open chunk, then the open tokens
    a = (n // C) * C
    assert [e[0] for e in st.cache] == H.persistent_cache(m_ref, a, w)
    assert [e[0] for e in st.open_] == list(range(a, n))
    if n % C == 0:
        assert [e[0] for e in st.cache] == list(cache_ref)
    for e in st.cache + st.open_:
        np.testing.assert_array_equal(e[1], k[e[0]])
        np.testing.assert_allclose(e[3], m_ref[e[0]], rtol=1e-12)


def test_decode_memory_is_bounded_and_sees_the_token():
    """3.5: at most w + C exact rows at any time; with C = 1 and w = 0 and no sink weight the cache path
    of a step reads only the token itself (its own value, whatever the logit)."""
    q, k, v, alpha, beta = _problem(5, 30, d=8, dv=8)
    gq, gk, _, _ = _gates(5, 8)
    st = H.hola_state_after_prefill(q[:1], k[:1], v[:1], alpha[:1], beta[:1], 4, 3)
    for t in range(1, 30):
        H.hola_decode_step(st, q[t], k[t], v[t], alpha[t], beta[t], gq, gk, 0.0, 0.0, 4, 3)
        assert len(st.cache) <= 3 and len(st.open_) < 4 and len(st.open_) == st.t % 4
    st = H.hola_state_after_prefill(q[:3], k[:3], v[:3], alpha[:3], beta[:3], 1, 0)
    o_prev = st.S.copy()
    y = H.hola_decode_step(st, q[3], k[3], v[3], alpha[3], beta[3], gq, gk, -80.0, 80.0, 1, 0)
    kh = k[3] / np.linalg.norm(k[3])
    e = v[3] - alpha[3] * (o_prev.T @ kh)
    S = alpha[3] * o_prev + beta[3] * np.outer(kh, e)
    np.testing.assert_allclose(y, S.T @ (q[3] / np.linalg.norm(q[3])) + v[3], rtol=1e-12, atol=1e-12)


def test_decode_negative_control_wrong_merge(monkeypatch):
    """Control: a chunk close that kept the smallest magnitudes instead of the largest makes the decode
    differ from the prefill, so the continuation pin above does see the merge rule."""
    q, k, v, alpha, beta = _problem(77, 20, d=8, dv=8)
    gq, gk, sink, gate = _gates(77, 8)
    C, w = 3, 2
    y_ref, *_ = H.hola_prefill(q, k, v, alpha, beta, gq, gk, sink, gate, C, w)
    monkeypatch.setattr(H, "_top_w", lambda entries, w_: sorted(sorted(entries, key=lambda e: (e[3], e[0]))[:w_],
                                                                   key=lambda e: e[0]))
    st = H.hola_state_after_prefill(q[:4], k[:4], v[:4], alpha[:4], beta[:4], C, w)
    worst = 0.0
    for t in range(4, 20):
        y_t = H.hola_decode_step(st, q[t], k[t], v[t], alpha[t], beta[t], gq, gk, sink, gate, C, w)
        worst = max(worst, float(np.abs(y_t - y_ref[t]).max()))
    assert worst > 1e-6

"""Plain fp64 CPU oracle for the HOLA variant: Gated DeltaNet state + exact KV cache chosen by write
magnitude.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this module: only the tests, the
smoke check and the CPU-baseline leg of the benchmark use it.  It shares no code with the HIP library.

Source: "A Hippocampus for Linear Attention: An Exact Memory for What the Recurrent State Forgets"
reading notes (cc.laoqi.cc, paper 2607.02303 v1), part 2 ("Method"):
  * 3.1 Eq. (1) and 3.5: the gated delta rule.  The state S (d_k x d_v) first predicts the value of the
    current key with the decayed state, e_t = v_t - alpha_t S_{t-1}^T k_t, then writes only that
    residual: S_t = alpha_t S_{t-1} + beta_t k_t e_t^T, alpha_t in (0, 1], beta_t in [0, 1].  Keys and
    queries of the state path have unit L2 norm.
  * 3.3 Eqs. (5)-(6): the write magnitude m_t = beta_t ||e_t||_2 (the Frobenius norm of the rank-one
    write for a unit key), fixed at write time; the persistent cache keeps the w entries with the
    largest m, never rescored.
  * 3.3: the cache read sees the persistent cache, the current chunk's tokens up to the query, and a
    null sink; at most w + C + 1 entries.
  * 3.4 Eq. (7): the cache path reads with its own RMS-normalised query and key, each with a learned
    per-dimension scale gamma, temperature tau = 1.
  * 3.2 Eq. (3) and 3.5: the output adds the state read-out and the gated cache read-out.

Readings where the notes leave a step open (listed in the design notes of the repository):
  H1 state read-out after the write: o_t = S_t^T q_t (the delta rule's usual order).
  H2 the persistent cache at the start of chunk c holds the w largest write magnitudes among the
     positions of earlier chunks (ties: older position); with fixed scores, merging chunk by chunk and
     keeping the top w is exactly this.  A token of the current chunk is visible to the queries at or
     after it through the chunk part, never twice.
  H3 cache logits: (gamma_q * q / rms(q))^T (gamma_k * k / rms(k)) / sqrt(d) with rms(x) =
     sqrt(mean(x^2) + 1e-6); the null sink is one more logit (a per-head value) with a zero value.
  H4 output y_t = o_t + sigmoid(g) * (cache read-out), g a per-head gate value.
  H5 unit-norm state keys and queries: x / ||x||_2 (a zero vector stays zero).
  H6 decode, one token at a time after a prefill, keeps the prefill's chunk grid (chunks of C
     positions from position 0).  The memory between tokens is what 3.5 sizes for one head: the state
     S plus at most w + C exact key-value rows, here the persistent cache at the start of the open
     chunk (positions, raw keys and values, magnitudes) and the open chunk's tokens so far.  When a
     token closes its chunk, the cache becomes the top w of the cache and the chunk's tokens (ties:
     older), as in H2.

Parity status: every function here is pinned by tests/test_oracle_hola.py (closed forms of the delta
rule, brute-force top-w, causal softmax through torch's attention, invariants; the decode step by
equality with a prefill over the longer sequence).
"""
from __future__ import annotations

import numpy as np

__all__ = ["unit", "rms_norm", "delta_rule", "write_magnitude", "persistent_cache", "cache_read",
           "hola_prefill", "HolaState", "hola_state_after_prefill", "hola_decode_step", "RMS_EPS"]

RMS_EPS = 1e-6


def unit(x: np.ndarray) -> np.ndarray:
    """Reading H5: rows scaled to unit L2 norm (zero rows stay zero)."""
    x = np.asarray(x, dtype=np.float64)
    nrm = np.sqrt((x * x).sum(axis=-1, keepdims=True))
    return np.where(nrm > 0, x / np.where(nrm > 0, nrm, 1.0), 0.0)


def rms_norm(x: np.ndarray, gamma: np.ndarray) -> np.ndarray:
    """Eq. (7) normalisation of the cache path (reading H3): gamma * x / sqrt(mean(x^2) + eps)."""
    x = np.asarray(x, dtype=np.float64)
    return np.asarray(gamma, dtype=np.float64) * x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + RMS_EPS)


def delta_rule(q, k, v, alpha, beta):
    """Gated delta rule over a sequence from S_0 = 0 (3.1 Eq. (1), 3.5).

    q, k [n][d_k], v [n][d_v], alpha, beta [n].  Returns (o [n][d_v] with o_t = S_t^T q_t (reading H1),
    e [n][d_v] residuals, S_n [d_k][d_v])."""
    qh, kh = unit(q), unit(k)
    v = np.asarray(v, dtype=np.float64)
    n, d_k = kh.shape
    S = np.zeros((d_k, v.shape[1]))
    o = np.zeros_like(v)
    e = np.zeros_like(v)
    for t in range(n):
        e[t] = v[t] - alpha[t] * (S.T @ kh[t])            # predict with the decayed state
        S = alpha[t] * S + beta[t] * np.outer(kh[t], e[t])   # write the residual only
        o[t] = S.T @ qh[t]
    return o, e, S


def write_magnitude(e, beta):
    """Eqs. (5)-(6): m_t = beta_t ||e_t||_2."""
    e = np.asarray(e, dtype=np.float64)
    return np.asarray(beta, dtype=np.float64) * np.sqrt((e * e).sum(axis=-1))


def persistent_cache(m, upto: int, w: int):
    """Reading H2: positions of the w largest scores among 0 .. upto-1 (ties: older), sorted."""
    cand = list(range(upto))
    cand.sort(key=lambda i: (-m[i], i))
    return sorted(cand[:w])


def cache_read(q_t, keys, vals, sink: float, gamma_q, gamma_k):
    """Softmax read over the visible keys plus the null sink (3.3, 3.4 Eq. (7), reading H3).

    keys [m][d], vals [m][d_v]: the visible entries (raw q/k; normalised here)."""
    d = len(q_t)
    qt = rms_norm(np.asarray(q_t)[None, :], gamma_q)[0]
    kt = rms_norm(keys, gamma_k)
    logits = kt @ qt / np.sqrt(d)
    mx = max(logits.max(initial=-np.inf), sink)
    p = np.exp(logits - mx)
    den = p.sum() + np.exp(sink - mx)
    return (p @ np.asarray(vals, dtype=np.float64)) / den


def hola_prefill(q, k, v, alpha, beta, gamma_q, gamma_k, sink: float, gate: float, C: int, w: int):
    """One sequence, one head, from an empty memory.

    Returns (y [n][d_v], S_n, cache positions after the last chunk, m [n], per-chunk cache lists)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    o, e, S = delta_rule(q, k, v, alpha, beta)
    m = write_magnitude(e, beta)
    g = 1.0 / (1.0 + np.exp(-gate))
    y = np.zeros_like(v)
    caches = []
    for c, a in enumerate(range(0, n, C)):
        A = persistent_cache(m, a, w)
        caches.append(A)
        for t in range(a, min(a + C, n)):
            vis = A + list(range(a, t + 1))
            y[t] = o[t] + g * cache_read(q[t], k[vis], v[vis], sink, gamma_q, gamma_k)
    return y, S, persistent_cache(m, n, w), m, caches


class HolaState:
    """Reading H6: the memory of one sequence and head between decode steps.

    t tokens seen; S [d_k][d_v]; cache: the persistent cache at the start of the open chunk, a list of
    (position, raw key, raw value, magnitude) sorted by position; open_: the open chunk's tokens so far,
    the same tuples in position order."""

    def __init__(self, t, S, cache, open_):
        self.t = int(t)
        self.S = np.array(S, dtype=np.float64)
        self.cache = list(cache)
        self.open_ = list(open_)


def _top_w(entries, w):
    """Reading H2 on explicit entries: the w largest magnitudes (ties: older), sorted by position."""
    kept = sorted(entries, key=lambda e: (-e[3], e[0]))[:w]
    return sorted(kept, key=lambda e: e[0])


def hola_state_after_prefill(q, k, v, alpha, beta, C: int, w: int) -> HolaState:
    """The memory hola_prefill leaves after n tokens from an empty memory (reading H6)."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = k.shape[0]
    _, e, S = delta_rule(q, k, v, alpha, beta)
    m = write_magnitude(e, beta)
    a = (n // C) * C                                          # start of the open chunk
    cache = [(i, k[i].copy(), v[i].copy(), float(m[i])) for i in persistent_cache(m, a, w)]
    open_ = [(i, k[i].copy(), v[i].copy(), float(m[i])) for i in range(a, n)]
    return HolaState(n, S, cache, open_)


def hola_decode_step(st: HolaState, q_t, k_t, v_t, alpha_t: float, beta_t: float, gamma_q, gamma_k,
                     sink: float, gate: float, C: int, w: int) -> np.ndarray:
    """One token through the memory (readings H1-H6); mutates ``st`` and returns y_t.

    The delta rule writes the token, the cache path reads the cache, the open chunk's earlier tokens and
    the token itself, plus the sink; then the token joins the open chunk, and a full chunk is merged
    into the cache."""
    q_t = np.asarray(q_t, dtype=np.float64)
    k_t = np.asarray(k_t, dtype=np.float64)
    v_t = np.asarray(v_t, dtype=np.float64)
    qh, kh = unit(q_t[None, :])[0], unit(k_t[None, :])[0]
    e = v_t - alpha_t * (st.S.T @ kh)
    st.S = alpha_t * st.S + beta_t * np.outer(kh, e)
    o = st.S.T @ qh
    m = float(beta_t * np.sqrt((e * e).sum()))
    vis = st.cache + st.open_ + [(st.t, k_t, v_t, m)]
    keys = np.array([x[1] for x in vis])
    vals = np.array([x[2] for x in vis])
    g = 1.0 / (1.0 + np.exp(-gate))
    y = o + g * cache_read(q_t, keys, vals, sink, gamma_q, gamma_k)
    st.open_.append((st.t, k_t.copy(), v_t.copy(), m))
    st.t += 1
    if st.t % C == 0:
        st.cache = _top_w(st.cache + st.open_, w)
        st.open_ = []
    return y

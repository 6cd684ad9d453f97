"""CPU checks of the parity harness itself: the decode grader accepts the oracle's own decisions and
rejects a fold the oracle's fp64 SRE order does not allow (2.4, Eqs. (11)-(13): the candidate with the
smallest SRE is the one folded)."""
import numpy as np
import pytest

import lola_testlib as TL
from oracle import lola_oracle as O


def _fixture(seed=5, n0=40, steps=12, eta=6, lam=5, d=8, D=8):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((d, D // 2)) / np.sqrt(d)
    phi = O.make_phi("softmax_pm", W)
    q, k, v = (rng.standard_normal((n0 + steps, d)) for _ in range(3))
    st = O.new_state(d, d, D, eta, lam)
    O.prefill(st, phi, q[:n0], k[:n0], v[:n0], C=4)
    ref = st.copy()
    ys, folds = [], []
    for s in range(steps):
        y, f = O.decode_step(ref, phi, q[n0 + s], k[n0 + s], v[n0 + s])
        ys.append(y)
        folds.append(f)
    return phi, st, q[n0:], k[n0:], v[n0:], np.array(ys), np.array(folds)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_grader_accepts_the_oracles_own_steps(dtype):
    phi, st, q, k, v, ys, folds = _fixture()
    assert (folds >= 0).sum() >= 6
    rep = TL.grade_decode_steps(st, phi, q, k, v, ys, folds, dtype)
    assert rep["fold_mismatches"] == 0 and rep["max_row_rel_err"] < 1e-12


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_grader_rejects_a_wrong_fold(dtype):
    """Negative control: at the first folding step, report the candidate with the largest SRE as the
    GPU's fold; the grader must fail in both modes."""
    phi, st, q, k, v, ys, folds = _fixture()
    s = int(np.nonzero(folds >= 0)[0][0])
    probe = st.copy()
    for i in range(s):
        O.decode_step(probe, phi, q[i], k[i], v[i])
    t = probe.t
    E = sorted(set(probe.cache) | ({t - probe.eta} if t - probe.eta >= 0 else set()))
    sc = O.sre(phi(probe.K[E]), probe.V[E], probe.H, probe.s)
    bad = folds.copy()
    bad[s] = E[int(np.argmax(sc))]
    assert bad[s] != folds[s]
    with pytest.raises(AssertionError):
        TL.grade_decode_steps(st, phi, q, k, v, ys, bad, dtype)


def test_chunked_decode_grader_needs_whole_groups():
    """A run that stops inside a group is refused before any grading: the group's allocation covers
    tokens whose steps were never taken."""
    with pytest.raises(AssertionError, match="group boundary"):
        TL.grade_chunked_decode(None, None, None, None, None, [None] * 5, None, t0=2, cd=4, dtype="f32")

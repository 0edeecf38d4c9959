"""The rule that explains a GPU row differing from the oracle (parity_util.explain_divergence),
checked on the CPU with trajectories made by the oracle and mistakes planted in them:
it must accept only a first divergence that is an excused near-tie or an M-step rounding
within the centroid tolerance, and reject everything else."""
import numpy as np
import pytest

import oracle
from parity_util import explain_divergence
from workloads import BF16, make_matrix


def _row(k=16, iters=8):
    m = make_matrix("explain", 1, 1024, BF16, 401)
    ref = oracle.quantize(m.w, BF16, m.act, 128, k, iters, trace=True)
    ws, a, _, _, bad = oracle.prepare_row(m.w[0], BF16, m.act, 128, k)
    assert not bad
    q_final = oracle.estep_row(ws, ref["c_trace"][0, iters])
    return ws, a, ref["c_trace"][0], q_final


def _assign(ws):
    return lambda c: oracle.estep_row(ws, c)


def test_identical_trajectory_is_not_an_explanation():
    ws, a, ct, q = _row()
    with pytest.raises(AssertionError):
        explain_divergence(ws, a, ct, lambda t: ct[t], _assign(ws), q)


def test_one_ulp_mstep_rounding_is_explained():
    ws, a, ct, q = _row()

    def c_at(t):
        c = ct[t].copy()
        if t >= 3:
            c[0] = np.nextafter(c[0], np.float32(np.inf))
        return c
    why = explain_divergence(ws, a, ct, c_at, _assign(ws), q)
    assert "round 3" in why and "M-step rounding" in why


def test_centroid_beyond_tolerance_is_rejected():
    ws, a, ct, q = _row()

    def c_at(t):
        c = ct[t].copy()
        if t >= 2:
            c[1] += np.float32(1e-3)
        return c
    with pytest.raises(AssertionError):
        explain_divergence(ws, a, ct, c_at, _assign(ws), q)


def test_assignment_flip_that_is_not_a_tie_is_rejected():
    ws, a, ct, q = _row()
    t_div = 4

    def assign_at(c):
        qq = oracle.estep_row(ws, c).copy()
        j = int(np.argmax(ws))                   # the row's maximum: never near a tie here
        qq[j] = (qq[j] + 1) % ct.shape[1]
        return qq

    def c_at(t):
        if t < t_div:
            return ct[t]
        return oracle.mstep_row(ws, a, assign_at(ct[t_div - 1]), ct[t_div - 1])
    with pytest.raises(AssertionError, match="beyond a near-tie"):
        explain_divergence(ws, a, ct, c_at, assign_at, q)


def test_exact_tie_flip_is_excused_in_a_round_and_in_the_final_step():
    # centroids 1 and 2: the element at 1.5 is an exact tie (lowest index wins in the
    # oracle); a GPU that gave it to centroid 1 differs only at an excused near-tie
    ws = np.array([0.0, 0.5, 1.5, 2.5, 3.0, 1.0, 2.0], np.float32)
    a = np.array([1, 2, 1, 1, 2, 1, 1], np.float32)
    c0 = np.array([1.0, 2.0], np.float32)
    q_ref = oracle.estep_row(ws, c0)
    assert q_ref[2] == 0
    q_tie = q_ref.copy()
    q_tie[2] = 1
    c1_ref = oracle.mstep_row(ws, a, q_ref, c0)
    ct = np.stack([c0, c1_ref])
    c1_gpu = oracle.mstep_row(ws, a, q_tie, c0)
    why = explain_divergence(ws, a, ct, lambda t: c0 if t == 0 else c1_gpu,
                             lambda c: q_tie if np.array_equal(c, c0) else oracle.estep_row(ws, c))
    assert "1 excused near-ties" in why
    # no round diverges (zero rounds); the final assignment differs at the tie only
    why = explain_divergence(ws, a, ct[:1], lambda t: c0, lambda c: q_tie, q_tie)
    assert why.startswith("final E-step")
    # a final assignment differing away from a tie is rejected
    q_bad = q_ref.copy()
    q_bad[0] = 1
    with pytest.raises(AssertionError):
        explain_divergence(ws, a, ct[:1], lambda t: c0, lambda c: q_bad, q_bad)

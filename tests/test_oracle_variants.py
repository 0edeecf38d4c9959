"""Pins for the oracle's method variants (the ablations of "any4: Learned 4-bit
Numeric Representation for LLMs").

  * symmetric scaling (Section 2.5.1, Eq. 3): a worked example with exact arithmetic;
    negating W negates the LUT and keeps codes and picks (the rule is symmetric);
    exact reconstruction of rows holding at most k symmetric integer levels.
  * sample weights (Appendix C.1): with every group's alpha the same power of two,
    alpha * E|x| and E|x| give bit-identical results (a common power-of-two factor is
    exact through the integer sampling and Eq. 23); without weights the result does
    not depend on E|x|, and equals E|x| weighting with a constant power-of-two E|x|.
  * initialization (Appendix C.2): uniform levels with no Lloyd round give the nearest
    integer level (the lower one on exact halves); random init draws each element with
    probability proportional to a_j, never twice (chi-square over many Philox keys);
    greedy k-means++ (scikit-learn's default seeding) keeps the best of 2 + floor(ln k)
    D^2 candidates: on a three-point row the worse second centre survives only when every
    candidate is the worse one (probability 0.1^L instead of 0.1), its first centre and
    first candidate are the plain draw, so its potential after two centres is never above
    plain k-means++'s, and over real-like rows its final seeding potential is lower.
  * restarts: the kept objective is the minimum over the single restarts, whose
    centroids it reproduces, and one restart is the default path bit for bit.
"""
import numpy as np
import pytest

import oracle
from oracle import (INIT_GREEDY, INIT_RANDOM, INIT_UNIFORM, SYMMETRIC, WEIGHT_ACT, WEIGHT_NONE,
                    restarts)
from workloads import BF16, F32, make_matrix


# --- symmetric scaling ---------------------------------------------------------------------

def test_symmetric_worked_example():
    """Eq. 3 by hand: group [-0.5, 0.25, 1.0, -2.0] has max|w| = 2; with 16 levels
    Qmax = 8, alpha = 2/8 = 0.25, beta = 0, w_S = w / alpha = [-2, 1, 4, -8] (exact)."""
    w = np.array([-0.5, 0.25, 1.0, -2.0, 3.0, -1.5, 0.75, 0.0], np.float32)
    ws, al, be, bad = oracle.scale_row(w, 4, 16, symmetric=True)
    assert not bad
    assert np.array_equal(al, np.array([0.25, 0.375], np.float32))
    assert np.array_equal(be, np.zeros(2, np.float32))
    assert np.array_equal(ws[:4], np.array([-2, 1, 4, -8], np.float32))
    assert np.array_equal(ws[4:], np.array([8, -4, 2, 0], np.float32))
    # any2: Qmax = 2
    ws2, al2, _, _ = oracle.scale_row(w[:4], 4, 4, symmetric=True)
    assert al2[0] == 1.0 and np.array_equal(ws2, w[:4])


@pytest.mark.parametrize("k", [4, 16])
def test_symmetric_negation_mirrors_lut(k):
    m = make_matrix("sym", 6, 512, F32, 61)
    v = SYMMETRIC
    a = oracle.quantize(m.w, F32, m.act, 128, k, 12, variant=v)
    b = oracle.quantize(-m.w, F32, m.act, 128, k, 12, variant=v)
    assert a["status"] == 0 and b["status"] == 0
    assert np.array_equal(a["codes"], b["codes"])
    assert np.array_equal(a["picks"], b["picks"])
    assert np.array_equal(a["c_final"], -b["c_final"])
    assert np.array_equal(a["lut"] ^ np.uint16(0x8000), b["lut"])
    assert np.array_equal(a["scale"], b["scale"]) and not a["offset"].any()


def test_symmetric_exact_levels_reconstruct():
    """Rows whose groups hold at most 16 integer multiples of a power-of-two alpha in
    [-8, 8], each group reaching |w| = 8 alpha: w_S are those integers and the objective is 0."""
    rng = np.random.default_rng(62)
    K, g = 512, 64
    rows = []
    for _ in range(5):
        levels = rng.choice(np.arange(-8, 9), 16, replace=False)
        levels[0] = 8 if rng.random() < 0.5 else -8
        L = rng.choice(levels, K)
        for t in range(K // g):
            L[t * g] = levels[0]
        rows.append((L * 2.0 ** rng.integers(-9, -4)).astype(np.float32))
    w = np.stack(rows)
    out = oracle.quantize(w, F32, np.ones(K, np.float32), g, 16, 10, variant=SYMMETRIC)
    assert np.all(out["objective"] == 0.0)
    rec = oracle.dequantize(out["codes"], out["lut"], out["scale"], out["offset"], g, 16)
    assert np.array_equal(rec, w)


# --- sample weights -----------------------------------------------------------------------

def _equal_alpha_rows(n, K, g, seed):
    """Random rows in which every group has min 0 and max 15 * 2^-7, so that every
    group's alpha is 2^-7."""
    rng = np.random.default_rng(seed)
    w = (rng.random((n, K)) * 15 * 2.0 ** -7).astype(np.float32)
    for t in range(K // g):
        w[:, t * g] = 0.0
        w[:, t * g + 1] = 15 * 2.0 ** -7
    return w


def test_weighting_alpha_act_equals_act_for_a_common_power_of_two_alpha():
    w = _equal_alpha_rows(6, 512, 64, 63)
    act = np.random.default_rng(64).lognormal(0, 0.5, 512).astype(np.float32)
    a = oracle.quantize(w, F32, act, 64, 16, 10)
    b = oracle.quantize(w, F32, act, 64, 16, 10, variant=WEIGHT_ACT)
    for key in ("codes", "lut", "picks"):
        assert np.array_equal(a[key], b[key]), key
    assert np.array_equal(a["c_final"], b["c_final"])


def test_unweighted_ignores_act_and_equals_constant_act():
    m = make_matrix("nw", 5, 512, BF16, 65)
    a = oracle.quantize(m.w, BF16, m.act, 128, 16, 8, variant=WEIGHT_NONE)
    b = oracle.quantize(m.w, BF16, m.act[::-1].copy(), 128, 16, 8, variant=WEIGHT_NONE)
    c = oracle.quantize(m.w, BF16, np.full(512, 4.0, np.float32), 128, 16, 8, variant=WEIGHT_ACT)
    for key in ("codes", "lut", "picks"):
        assert np.array_equal(a[key], b[key]) and np.array_equal(a[key], c[key]), key
    d = oracle.quantize(m.w, BF16, m.act, 128, 16, 8)
    assert not np.array_equal(a["codes"], d["codes"])     # the weights do matter by default


# --- initialization ------------------------------------------------------------------------

def test_uniform_init_without_rounds_is_nearest_level():
    m = make_matrix("uni", 8, 512, F32, 66)
    for k in (16, 8):
        out = oracle.quantize(m.w, F32, m.act, 128, k, 0, variant=INIT_UNIFORM)
        assert np.all(out["picks"] == -1)
        assert np.array_equal(out["lut"].view(np.float16).astype(np.float32),
                              np.tile(np.arange(k, dtype=np.float32), (8, 1)))
        q = np.stack([out["codes"] & 0xF, out["codes"] >> 4], -1).reshape(8, 512)
        for i in range(8):
            ws, _, _, _ = oracle.scale_row(m.w[i], 128, k)
            want = np.clip(np.ceil(ws.astype(np.float64) - 0.5), 0, k - 1)
            assert np.array_equal(q[i], want), (k, i)
    # symmetric scaling: levels 1 - k/2 .. k/2 (int4's -7..8 for k = 16)
    out = oracle.quantize(m.w, F32, m.act, 128, 16, 0, variant=INIT_UNIFORM | SYMMETRIC)
    assert np.array_equal(out["lut"][0].view(np.float16).astype(np.float32),
                          np.arange(-7, 9, dtype=np.float32))


def test_random_init_draws_proportional_to_weight_without_replacement():
    x = np.arange(8, dtype=np.float32)
    a = np.array([1, 2, 3, 4, 0, 6, 7, 8], np.float32)
    n = 40000
    picks = np.array([oracle.seed_row(x, a, 3, seed=s, init=1)[1] for s in range(n)])
    assert np.all(picks[:, 0] != picks[:, 1]) and np.all(picks[:, 1] != picks[:, 2])
    assert not np.any(picks == 4)
    counts = np.bincount(picks[:, 0], minlength=8)
    p = a / a.sum()
    nz = p > 0
    assert ((counts[nz] - n * p[nz]) ** 2 / (n * p[nz])).sum() < 24.3  # 6 dof
    for first in (3, 7):
        sel = picks[picks[:, 0] == first, 1]
        q = a.copy()
        q[first] = 0
        q /= q.sum()
        c = np.bincount(sel, minlength=8)
        nz = q > 0
        assert ((c[nz] - sel.size * q[nz]) ** 2 / (sel.size * q[nz])).sum() < 22.5  # 5 dof


def test_random_init_all_weights_used_then_copies():
    x = np.array([5, 6, 7], np.float32)
    a = np.array([1, 0, 1], np.float32)
    c0, picks = oracle.seed_row(x, a, 4, seed=3, init=1)
    assert sorted(picks[:2].tolist()) == [0, 2] and np.all(picks[2:] == -1)
    assert np.all(c0[2:] == c0[0])


def _binom_ok(hits, n, p, z=4.0):
    mu = n * p
    return abs(hits - mu) <= z * np.sqrt(n * p * (1 - p)) + 1


@pytest.mark.parametrize("k", [2, 4])
def test_greedy_keeps_the_best_candidate(k):
    """Row [0, 1, 3], unit weights.  After a first centre at 0, D = [0, 1, 9]: a D^2 draw
    gives 1 with probability 0.1 and 3 with 0.9; centre 1 leaves potential 4, centre 3
    leaves 1.  Greedy seeding keeps 1 only if all its L candidates are 1 (0.1^L, L = 2
    for k = 2 and 3 for k = 4); plain seeding keeps it with probability 0.1."""
    x = np.array([0, 1, 3], np.float32)
    a = np.ones(3, np.float32)
    L = oracle.greedy_trials(k)
    assert L == {2: 2, 4: 3}[k]
    n_first0 = {0: 0, 3: 0}
    worse = {0: 0, 3: 0}
    for s in range(9000):
        plain = oracle.seed_row(x, a, k, seed=s, init=0)[1]
        greedy = oracle.seed_row(x, a, k, seed=s, init=3)[1]
        assert plain[0] == greedy[0]                   # the first centre is the plain draw
        for init, p in ((0, plain), (3, greedy)):
            if p[0] == 0:
                n_first0[init] += 1
                worse[init] += int(p[1] == 1)
    assert _binom_ok(worse[0], n_first0[0], 0.1)
    assert _binom_ok(worse[3], n_first0[3], 0.1 ** L)
    assert worse[3] < worse[0] / 4


def _potential(ws, a, centres):
    d = (ws.astype(np.float64)[:, None] - centres.astype(np.float64)[None, :]) ** 2
    return float((a.astype(np.float64) * d.min(axis=1)).sum())


def test_greedy_never_worse_after_two_centres():
    """With k = 2 the greedy draw at t = 1 includes the plain draw as its first
    candidate and keeps the candidate of smallest potential, so its potential is never
    above plain k-means++'s (fp64 potentials; the exact integer ones order the same up
    to the 2^-40 quantization)."""
    m = make_matrix("greedy2", 40, 512, F32, 68)
    for i in range(40):
        ws, al, _, _ = oracle.scale_row(m.w[i], 128, 2)
        a, _ = oracle.weights_row(al, m.act, 128)
        for s in range(5):
            cp, pp = oracle.seed_row(ws, a, 2, seed=s, row_id=i, init=0)
            cg, pg = oracle.seed_row(ws, a, 2, seed=s, row_id=i, init=3)
            assert pp[0] == pg[0]
            assert _potential(ws, a, cg) <= _potential(ws, a, cp) * (1 + 1e-9)


def test_greedy_lowers_the_seeding_potential():
    m = make_matrix("greedy16", 24, 1024, BF16, 69)
    pot = {0: [], 3: []}
    for i in range(24):
        w32 = (m.w[i].astype(np.uint32) << 16).view(np.float32)
        ws, al, _, _ = oracle.scale_row(w32, 128, 16)
        a, _ = oracle.weights_row(al, m.act, 128)
        for init in (0, 3):
            c0, _ = oracle.seed_row(ws, a, 16, seed=7, row_id=i, init=init)
            pot[init].append(_potential(ws, a, c0))
    pg, pp = np.array(pot[3]), np.array(pot[0])
    assert pg.mean() < 0.9 * pp.mean()
    assert np.mean(pg < pp) > 0.7


def test_greedy_variant_end_to_end_status():
    m = make_matrix("greedyq", 4, 512, BF16, 70)
    out = oracle.quantize(m.w, BF16, m.act, 128, 16, 6, variant=INIT_GREEDY)
    assert out["status"] == 0
    plain = oracle.quantize(m.w, BF16, m.act, 128, 16, 6)
    assert np.array_equal(out["picks"][:, 0], plain["picks"][:, 0])


# --- restarts ------------------------------------------------------------------------------

@pytest.mark.parametrize("init", [0, INIT_RANDOM])
def test_restarts_keep_the_lowest_objective(init):
    m = make_matrix("rs", 6, 512, BF16, 67)
    n = 4
    out = oracle.quantize(m.w, BF16, m.act, 128, 16, 6, variant=init | restarts(n))
    plain = (init >> 2)
    for i in range(6):
        w32 = (m.w[i].astype(np.uint32) << 16).view(np.float32)
        ws, al, _, _ = oracle.scale_row(w32, 128, 16)
        a, _ = oracle.weights_row(al, m.act, 128)
        best = None
        for r in range(n):
            c0, _ = oracle.seed_row(ws, a, 16, seed=0, row_id=i, init=plain, restart=r)
            c, q, Js = oracle.lloyd_row(ws, a, c0, 6)
            if best is None or Js[-1] < best[0]:
                best = (Js[-1], c)
        assert out["objective"][i] == best[0]
        assert np.array_equal(out["c_final"][i], best[1])
    single = oracle.quantize(m.w, BF16, m.act, 128, 16, 6, variant=init)
    assert np.all(out["objective"] <= single["objective"])
    if init == 0:
        default = oracle.quantize(m.w, BF16, m.act, 128, 16, 6)
        for key in ("codes", "lut", "picks", "c_final", "objective"):
            assert np.array_equal(single[key], default[key]), key


def test_variant_validation():
    w = np.zeros((1, 8), np.float32)
    act = np.ones(8, np.float32)
    for v in (3, 1 << 5, 1 << 16):
        assert oracle.quantize(w, F32, act, 4, 4, 1, variant=v)["status"] == 1

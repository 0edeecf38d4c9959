"""Pins for the oracle's scaling, E-step, M-step, seeding and whole-row path.

What pins what:
  * Eq. 1-2 scaling (any4 paper, Section 2.5.1): a worked example with exact
    arithmetic, group independence, dequantization bound, power-of-two invariance.
  * E-step (Section 4.1, Eq. 18): numpy argmin on the same fp32 distances (first
    minimum = lowest index), and exact nearest-centroid in fp64 away from ties.
  * M-step (Eq. 23) and the Lloyd loop: scikit-learn's weighted Lloyd from the same
    initial centres; the 1-D optimum by dynamic programming over sorted points (the
    Lloyd-Max scalar quantizer the paper cites) checked itself by brute force;
    replication of integer-weighted points; monotone objective.
  * k-means++ seeding (Appendix C.2): empirical pick frequencies against a_j and
    a_j * D_j over many Philox keys; zero-weight points are never drawn.
  * whole path: exact reconstruction of rows with at most k scaled levels;
    bit-identical outputs under power-of-two scaling of W and of E|x|.
"""
import itertools

import numpy as np
import pytest

import oracle
from workloads import BF16, F32, make_matrix


# --- scaling ---------------------------------------------------------------------------

def test_scaling_worked_example():
    """Eq. 1-2 by hand, with numbers chosen so every operation is exact:
    group [-0.5, -0.0625, 0.4375, 0.0] has min -0.5, max 0.4375, range 0.9375;
    alpha = 0.9375 / 15 = 0.0625, beta = -0.5, w_S = (w + 0.5) / 0.0625 = [0, 7, 15, 8]."""
    w = np.array([-0.5, -0.0625, 0.4375, 0.0, 1.0, 1.0, 1.0, 1.0], np.float32)
    ws, al, be, bad = oracle.scale_row(w, 4, 16)
    assert not bad
    assert al.tolist() == [0.0625, 0.0]          # second group is constant: alpha = 0
    assert be.tolist() == [-0.5, 1.0]
    assert ws.tolist() == [0.0, 7.0, 15.0, 8.0, 0.0, 0.0, 0.0, 0.0]
    # any3 / any2 use 2^n - 1 levels
    ws3, al3, _, _ = oracle.scale_row(w, 4, 8)
    assert al3[0] == np.float32(0.9375) / np.float32(7)


def test_scaling_groups_are_independent():
    rng = np.random.default_rng(3)
    w = rng.standard_normal(512).astype(np.float32)
    ws, al, be, _ = oracle.scale_row(w, 128, 16)
    w2 = w.copy()
    w2[128:256] *= 7.0  # change only group 1
    ws2, al2, be2, _ = oracle.scale_row(w2, 128, 16)
    keep = np.r_[0:128, 256:512]
    assert np.array_equal(ws[keep], ws2[keep])
    assert np.array_equal(al[[0, 2, 3]], al2[[0, 2, 3]]) and al[1] != al2[1]
    # each group hits 0 at its argmin and ~15 at its argmax
    for t in range(4):
        g = slice(128 * t, 128 * (t + 1))
        assert ws[g][np.argmin(w[g])] == 0.0
        assert abs(ws[g][np.argmax(w[g])] - 15.0) <= 15.0 * 2**-22
        assert ws[g].min() >= 0.0


def test_scaling_dequant_bound():
    """dequant(w_S) = alpha * w_S + beta reproduces w up to fp32 rounding (Eq. 4 with the
    identity in place of rounding)."""
    rng = np.random.default_rng(4)
    w = (rng.standard_t(5, 4096) * 0.02).astype(np.float32)
    ws, al, be, _ = oracle.scale_row(w, 64, 16)
    rec = np.repeat(al.astype(np.float64), 64) * ws + np.repeat(be.astype(np.float64), 64)
    rng_w = np.repeat(al.astype(np.float64) * 15, 64)
    assert np.all(np.abs(rec - w) <= 4 * 2**-24 * (np.abs(w) + rng_w))


# --- E-step ----------------------------------------------------------------------------

def test_estep_is_first_argmin_of_fp32_distances():
    rng = np.random.default_rng(5)
    ws = rng.uniform(0, 15, 5000).astype(np.float32)
    c = rng.uniform(0, 15, 16).astype(np.float32)
    c[5] = c[2]          # duplicate: the lower index must win
    ws[:16] = c          # exact hits
    ws[16] = (c[0] + c[1]) / 2
    q = oracle.estep_row(ws, c)
    d = (ws[:, None] - c[None, :]) ** 2       # numpy fp32 arithmetic
    assert d.dtype == np.float32
    assert np.array_equal(q, np.argmin(d, axis=1))
    assert not np.any(q == 5)


def test_estep_nearest_in_exact_arithmetic():
    rng = np.random.default_rng(6)
    ws = rng.uniform(0, 15, 20000).astype(np.float32)
    c = np.sort(rng.uniform(0, 15, 16)).astype(np.float32)
    q = oracle.estep_row(ws, c)
    d = np.abs(ws[:, None].astype(np.float64) - c[None, :].astype(np.float64))
    best = d.min(axis=1)
    chosen = d[np.arange(ws.size), q]
    assert np.all(chosen <= best * (1 + 1e-6) + 1e-30)


# --- M-step / Lloyd ----------------------------------------------------------------------

def dp_optimum(x, a, k):
    """Optimal weighted 1-D k-clustering: clusters are contiguous in sorted order
    (Lloyd-Max).  O(k n^2) dynamic programming in fp64 with prefix sums."""
    order = np.argsort(x, kind="stable")
    xs, as_ = x[order].astype(np.float64), a[order].astype(np.float64)
    n = xs.size
    P0 = np.concatenate([[0.0], np.cumsum(as_)])
    P1 = np.concatenate([[0.0], np.cumsum(as_ * xs)])
    P2 = np.concatenate([[0.0], np.cumsum(as_ * xs * xs)])

    def cost(i, j):  # points i..j-1
        s0 = P0[j] - P0[i]
        if s0 <= 0:
            return 0.0
        s1 = P1[j] - P1[i]
        return max(P2[j] - P2[i] - s1 * s1 / s0, 0.0)

    INF = float("inf")
    best = np.full((k + 1, n + 1), INF)
    arg = np.zeros((k + 1, n + 1), int)
    best[0, 0] = 0.0
    for m in range(1, k + 1):
        for j in range(n + 1):
            for i in range(j + 1):
                v = best[m - 1, i] + cost(i, j)
                if v < best[m, j]:
                    best[m, j], arg[m, j] = v, i
    # centres of the optimal partition
    cuts, j = [], n
    for m in range(k, 0, -1):
        i = arg[m, j]
        cuts.append((i, j))
        j = i
    cents = []
    for i, j in reversed(cuts):
        s0 = P0[j] - P0[i]
        if s0 > 0:
            cents.append((P1[j] - P1[i]) / s0)
    return best[k, n], np.array(cents)


def brute_force_optimum(x, a, k):
    best = float("inf")
    for lab in itertools.product(range(k), repeat=x.size):
        lab = np.array(lab)
        J = 0.0
        for t in range(k):
            m = lab == t
            if a[m].sum() > 0:
                mu = (a[m] * x[m]).sum() / a[m].sum()
                J += (a[m] * (x[m] - mu) ** 2).sum()
        best = min(best, J)
    return best


def test_dp_matches_brute_force():
    rng = np.random.default_rng(7)
    for trial in range(6):
        n = 7
        k = 2 + trial % 2
        x = rng.uniform(0, 15, n)
        a = rng.uniform(0.1, 2.0, n)
        assert abs(dp_optimum(x, a, k)[0] - brute_force_optimum(x, a, k)) <= 1e-9


def test_lloyd_not_below_optimum_and_optimum_is_fixed_point():
    rng = np.random.default_rng(8)
    for k, n in [(2, 120), (4, 160), (8, 200)]:
        x = np.concatenate([rng.normal(7, 2, n // 2), rng.normal(3, 0.5, n - n // 2)])
        x = np.clip(x, 0, 15).astype(np.float32)
        a = rng.lognormal(0, 0.5, n).astype(np.float32)
        J_opt, c_opt = dp_optimum(x, a, k)
        # Lloyd from k-means++ seeds never beats the optimum
        for s in range(5):
            c0, _ = oracle.seed_row(x, a, k, seed=s)
            _, _, Js = oracle.lloyd_row(x, a, c0, 30)
            assert Js[-1] >= J_opt * (1 - 1e-12)
        # Lloyd started at the optimum stays there
        c_start = c_opt.astype(np.float32)
        c_end, q_end, Js = oracle.lloyd_row(x, a, c_start, 5)
        assert np.all(np.abs(Js - J_opt) <= 1e-6 * J_opt)
        assert np.allclose(c_end, c_start, rtol=1e-6, atol=1e-6)


def test_lloyd_matches_sklearn():
    """scikit-learn's weighted Lloyd (algorithm='lloyd') from the same initial centres.
    sklearn works in fp64; the oracle keeps fp32 centres, so centres agree to fp32
    rounding while assignments agree exactly away from near-ties."""
    from sklearn.cluster import KMeans
    rng = np.random.default_rng(9)
    checked = 0
    for trial in range(12):
        n, k, iters = 600, 4 + 4 * (trial % 2), 8
        x = np.clip(rng.standard_t(5, n) * 2 + 7.5, 0, 15).astype(np.float32)
        a = (rng.lognormal(0, 0.5, n) * rng.uniform(0.2, 1, n)).astype(np.float32)
        c0, _ = oracle.seed_row(x, a, k, seed=trial)
        if np.unique(c0).size < k:
            continue
        c_or, q_or, _ = oracle.lloyd_row(x, a, c0, iters)
        # skip runs where a cluster went empty (sklearn relocates, the oracle keeps)
        c = c0.copy()
        empty = False
        for _ in range(iters):
            q = oracle.estep_row(x, c)
            if np.bincount(q, minlength=k).min() == 0:
                empty = True
            c = oracle.mstep_row(x, a, q, c)
        if empty:
            continue
        km = KMeans(n_clusters=k, init=c0.astype(np.float64).reshape(-1, 1), n_init=1, tol=0.0,
                    max_iter=iters, algorithm="lloyd")
        km.fit(x.astype(np.float64).reshape(-1, 1), sample_weight=a.astype(np.float64))
        c_sk = km.cluster_centers_.ravel()
        assert np.all(np.abs(c_or - c_sk) <= 1e-5 * np.maximum(np.abs(c_sk), 1.0))
        # labels: equal except near-ties between the two nearest centres
        d = np.abs(x[:, None].astype(np.float64) - c_sk[None, :])
        ds = np.sort(d, axis=1)
        tie = (ds[:, 1] - ds[:, 0]) <= 1e-4 * np.maximum(ds[:, 1], 1e-12)
        assert np.array_equal(q_or[~tie], km.labels_[~tie])
        checked += 1
    assert checked >= 6


def test_mstep_weights_are_multiplicities():
    """An integer weight equals that many copies of the point (Eq. 23 is a weighted mean)."""
    rng = np.random.default_rng(10)
    x = rng.uniform(0, 15, 300).astype(np.float32)
    a = rng.integers(1, 4, 300).astype(np.float32)
    c = np.sort(rng.uniform(0, 15, 8)).astype(np.float32)
    q = oracle.estep_row(x, c)
    c1 = oracle.mstep_row(x, a, q, c)
    xr = np.repeat(x, a.astype(int))
    qr = np.repeat(q, a.astype(int))
    c2 = oracle.mstep_row(xr, np.ones(xr.size, np.float32), qr, c)
    assert np.all(np.abs(c1.view(np.int32) - c2.view(np.int32)) <= 1)
    J1 = oracle.objective_row(x, a, q, c1)
    J2 = oracle.objective_row(xr, np.ones(xr.size, np.float32), qr, c1)
    assert abs(J1 - J2) <= 1e-12 * J1


def test_empty_cluster_keeps_value():
    x = np.array([1.0, 1.1, 5.0, 5.2], np.float32)
    a = np.ones(4, np.float32)
    c = np.array([1.0, 5.0, 14.0, 0.0], np.float32)   # 14 gets nothing; 0 loses ties to 1.0? no: farther
    q = oracle.estep_row(x, c)
    cn = oracle.mstep_row(x, a, q, c)
    assert cn[2] == np.float32(14.0) and cn[3] == np.float32(0.0)
    assert cn[0] == np.float32((1.0 + np.float64(np.float32(1.1))) / 2)


def test_objective_monotone_on_workload_rows():
    m = make_matrix("t", 16, 512, F32, 11)
    out = oracle.quantize(m.w, 0, m.act, 128, 16, iters=20, trace=True)
    Jt = out["j_trace"]
    assert np.all(Jt[:, 1:] <= Jt[:, :-1] * (1 + 1e-6))
    assert np.allclose(Jt[:, -1], out["objective"], rtol=0, atol=0)


# --- seeding -----------------------------------------------------------------------------

def test_seed_first_pick_proportional_to_weight():
    x = np.arange(8, dtype=np.float32)
    a = np.array([1, 2, 3, 4, 0, 6, 7, 8], np.float32)
    n = 40000
    first = np.array([oracle.seed_row(x, a, 2, seed=s)[1][0] for s in range(n)])
    counts = np.bincount(first, minlength=8)
    assert counts[4] == 0
    p = a / a.sum()
    nz = p > 0
    chi2 = ((counts[nz] - n * p[nz]) ** 2 / (n * p[nz])).sum()
    assert chi2 < 24.3  # 6 dof, p ~ 5e-4


def test_seed_second_pick_proportional_to_weight_times_d2():
    x = np.array([0, 1, 2, 4, 7, 11, 13, 15], np.float32)
    a = np.array([1, 1, 2, 1, 3, 1, 2, 1], np.float32)
    n = 60000
    pairs = np.array([oracle.seed_row(x, a, 2, seed=s, row_id=3)[1] for s in range(n)])
    for first in [2, 4]:
        sel = pairs[pairs[:, 0] == first, 1]
        D = (x - x[first]) ** 2
        p = a * D / (a * D).sum()
        counts = np.bincount(sel, minlength=8)
        assert counts[first] == 0
        nz = p > 0
        m = sel.size
        chi2 = ((counts[nz] - m * p[nz]) ** 2 / (m * p[nz])).sum()
        assert chi2 < 26.1  # 7 dof, p ~ 5e-4


def test_seed_picks_distinct_values_then_copies():
    """With fewer distinct values than k, D^2 sampling takes every value once and
    then copies centre 0 (its pick is recorded as -1)."""
    x = np.array([3, 3, 9, 9, 9, 12], np.float32)
    a = np.ones(6, np.float32)
    c0, picks = oracle.seed_row(x, a, 8, seed=1)
    assert sorted(set(c0[:3].tolist())) == [3.0, 9.0, 12.0]
    assert np.all(picks[3:] == -1) and np.all(c0[3:] == c0[0])
    # all weights zero: everything copies w_S[0]
    c0, picks = oracle.seed_row(x, np.zeros(6, np.float32), 4, seed=1)
    assert np.all(c0 == x[0]) and np.all(picks == -1)


def test_seed_scale_is_fixed_after_the_first_pick():
    """After the first pick every draw uses one fixed-point scale 2^(40 - e), e from the
    bound B = max a * m^2 (m the larger distance from the first centre to the row's
    extremes).  Weights below 2^(e - 40) become 0: on a row whose other elements weigh
    2^-60 against B = 225, the first centre is element 0 (the others' q_j are 0 even at
    the first draw's scale 2^40), and every later draw has Q = 0, so it copies centre 0
    (pick -1) although its weights are not all 0.  With weights 2^-20 instead (q_j =
    floor(225 * 2^-20 * 2^33) > 0) the later draws do pick them."""
    x = np.array([0.0, 15.0, 15.0, 15.0], np.float32)
    for seed in range(20):
        c0, picks = oracle.seed_row(x, np.array([1, 2 ** -60, 2 ** -60, 2 ** -60], np.float32), 4, seed=seed)
        assert picks[0] == 0 and np.all(picks[1:] == -1) and np.all(c0 == 0.0), (seed, picks)
        c0, picks = oracle.seed_row(x, np.array([1, 2 ** -20, 2 ** -20, 2 ** -20], np.float32), 4, seed=seed)
        assert picks[0] == 0 and picks[1] in (1, 2, 3), (seed, picks)
        assert np.all(picks[2:] == -1)        # after 15 is drawn every D is 0: copies


def test_seed_picks_invariant_under_power_of_two_weights():
    """D^2 sampling is scale-free in the weights, and the integer CDF keeps it so down to
    the bottom of fp32: from the second draw on, a_j is scaled by 2^(40-e) before its
    product with D_j.  A row whose weights are another's times 2^-123 (still normal
    numbers) draws the same picks, although the products a_j * D_j of its tight cluster
    lie near 2^-146, where fp32 keeps 2-3 bits: rounding those products first would move
    their terms q_j (around 2^10) by up to a fifth and change the picks."""
    rng = np.random.default_rng(31)
    x = np.concatenate([[0.0, 15.0], 7.0 + rng.uniform(0, 7e-4, 46)]).astype(np.float32)
    a = rng.uniform(0.5, 1.0, x.size).astype(np.float32)       # full 24-bit mantissas
    a_tiny = (a * np.float32(2.0 ** -123)).astype(np.float32)  # exact: still normal numbers
    assert np.array_equal((a_tiny.astype(np.float64) * 2.0 ** 123).astype(np.float32), a)
    inside = 0
    for seed in range(300):
        p1 = oracle.seed_row(x, a, 8, seed=seed)[1]
        p2 = oracle.seed_row(x, a_tiny, 8, seed=seed)[1]
        assert np.array_equal(p1, p2), (seed, p1, p2)
        inside += int(np.sum(p1[1:] >= 2))  # later picks inside the tight cluster
    assert inside > 900  # the draws do reach the elements whose products are subnormal


def test_seed_depends_on_row_matrix_and_key():
    rng = np.random.default_rng(12)
    x = rng.uniform(0, 15, 256).astype(np.float32)
    a = np.ones(256, np.float32)
    base = oracle.seed_row(x, a, 16, seed=0, row_id=0, matrix_index=0)[1]
    for kw in [dict(seed=1), dict(row_id=1), dict(matrix_index=1), dict(row_id=2**32)]:
        args = dict(seed=0, row_id=0, matrix_index=0)
        args.update(kw)
        assert not np.array_equal(oracle.seed_row(x, a, 16, **args)[1], base)


# --- whole path ------------------------------------------------------------------------------

def exact_level_rows(n, K, group, k, seed):
    """Rows whose scaled values are at most k integer levels, every group holding
    both 0 and Qr, alpha a power of two, beta exactly representable."""
    rng = np.random.default_rng(seed)
    qr = k - 1
    rows = []
    for _ in range(n):
        levels = np.sort(rng.choice(np.arange(1, qr), size=min(k - 2, qr - 1), replace=False))
        levels = np.concatenate([[0], levels, [qr]])
        L = rng.choice(levels, size=K)
        for t in range(K // group):
            L[t * group] = 0
            L[t * group + 1] = qr
        alpha = 2.0 ** rng.integers(-9, -4)
        beta = -rng.integers(0, 64) * 2.0 ** -8
        rows.append((beta + alpha * L).astype(np.float32))
    return np.stack(rows)


@pytest.mark.parametrize("k", [4, 16])
def test_exact_reconstruction_rows(k):
    K, g = 512, 64
    w = exact_level_rows(6, K, g, k, 13)
    act = np.random.default_rng(14).lognormal(0, 0.5, K).astype(np.float32)
    out = oracle.quantize(w, 0, act, g, k, iters=10)
    assert out["status"] == 0
    assert np.all(out["objective"] == 0.0)
    lut = out["lut"].view(np.float16).astype(np.float64)
    q = np.stack([out["codes"] & 0xF, out["codes"] >> 4], axis=-1).reshape(w.shape[0], K)
    al = np.repeat(out["scale"].view(np.float16).astype(np.float64), g, axis=1)
    be = np.repeat(out["offset"].view(np.float16).astype(np.float64), g, axis=1)
    rec = al * np.take_along_axis(lut, q.astype(int), axis=1) + be
    assert np.array_equal(rec, w.astype(np.float64))


def test_fewer_levels_than_clusters():
    K, g = 256, 64
    w = exact_level_rows(3, K, g, 4, 15)       # 4 levels, 16 clusters
    act = np.ones(K, np.float32)
    out = oracle.quantize(w, 0, act, g, 16, iters=5)
    assert np.all(out["objective"] == 0.0)
    assert np.all((out["picks"] >= 0).sum(axis=1) == 4)


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_power_of_two_invariance(dtype):
    m = make_matrix("t", 12, 512, dtype, 16)
    base = oracle.quantize(m.w, dtype, m.act, 128, 16, iters=8)
    # E|x| * 2^5
    o2 = oracle.quantize(m.w, dtype, m.act * np.float32(32.0), 128, 16, iters=8)
    for key in ["codes", "lut", "scale", "offset", "picks"]:
        assert np.array_equal(base[key], o2[key]), key
    assert np.allclose(o2["objective"], base["objective"] * 32.0, rtol=1e-12)
    # W * 2^-3
    if dtype == F32:
        w3 = m.w * np.float32(0.125)
    else:
        w3 = ((m.w.astype(np.uint32) << 16).view(np.float32) * np.float32(0.125))
        w3 = (w3.view(np.uint32) >> 16).astype(np.uint16)
    o3 = oracle.quantize(w3, dtype, m.act, 128, 16, iters=8)
    for key in ["codes", "lut", "picks"]:
        assert np.array_equal(base[key], o3[key]), key
    sc = base["scale"].view(np.float16).astype(np.float64) * 0.125
    assert np.array_equal(o3["scale"].view(np.float16).astype(np.float64), sc)


def test_iters_zero_codes_are_nearest_seeds():
    m = make_matrix("t", 4, 512, F32, 17)
    out = oracle.quantize(m.w, 0, m.act, 128, 16, iters=0)
    for i in range(4):
        ws, a, _, _, _ = oracle.prepare_row(m.w[i], 0, m.act, 128, 16)
        c0, picks = oracle.seed_row(ws, a, 16, 0, i, 0)
        assert np.array_equal(c0, out["c_final"][i])
        assert np.array_equal(oracle.pack_row(oracle.estep_row(ws, c0)), out["codes"][i])


def test_constant_row_and_zero_activations():
    K = 256
    w = np.full((2, K), 0.25, np.float32)
    act = np.ones(K, np.float32)
    out = oracle.quantize(w, 0, act, 64, 16, iters=3)
    assert np.all(out["objective"] == 0.0)
    assert np.all(out["lut"] == 0) and np.all(out["codes"] == 0)
    assert np.all(out["offset"].view(np.float16) == np.float16(0.25))
    w2 = np.random.default_rng(18).standard_normal((2, K)).astype(np.float32)
    out2 = oracle.quantize(w2, 0, np.zeros(K, np.float32), 64, 16, iters=3)
    assert np.all(out2["objective"] == 0.0) and np.all(out2["picks"] == -1)


def test_invalid_rows_flagged():
    K = 256
    w = np.random.default_rng(19).standard_normal((3, K)).astype(np.float32)
    w[1, 7] = np.nan
    act = np.ones(K, np.float32)
    out = oracle.quantize(w, 0, act, 64, 16, iters=2)
    assert out["status"] == 5
    assert np.isnan(out["objective"][1]) and np.all(out["codes"][1] == 0)
    assert np.isfinite(out["objective"][[0, 2]]).all()
    act2 = act.copy()
    act2[3] = -1.0
    assert oracle.quantize(w[[0]], 0, act2, 64, 16, iters=2)["status"] == 5


def test_argument_validation():
    w = np.zeros((2, 96), np.float32)
    act = np.ones(96, np.float32)
    for args in [dict(group=64), dict(n_clusters=3), dict(iters=-1)]:
        kw = dict(group=32, n_clusters=16, iters=1)
        kw.update(args)
        assert oracle.quantize(w, 0, act, **kw)["status"] == 1

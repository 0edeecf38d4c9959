"""Sorted-row Lloyd (`any4_stage_lloyd_sorted`): Lloyd rounds taken on the sorted row
with fp64 prefix sums, checked against the oracle's Lloyd rounds (Section 4.1: Eq. 18
assignment, Eq. 23 update) from the same scaled rows, sample weights and starting
centroids, all computed by the oracle.  The assignment rule equals the register path's,
so only the fp64 summation order differs: every row's final objective agrees within the
objective tolerance, at least 90% of rows have every centroid within the per-round
centroid tolerance, and most rows end bit-identical.
"""
import numpy as np
import pytest

import oracle
from parity_util import OBJECTIVE_REL, centroid_close, say, widen
from workloads import BF16, F32, make_matrix

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SYM = 1 << 4
W_NONE = 2

# (name, N, K, dtype, group, n_clusters, iters, variant, seed)
SHAPES = [
    ("k4096_g128", 16, 4096, BF16, 128, 16, 20, 0, 301),
    ("ragged_k1000_g8", 9, 1000, BF16, 8, 16, 20, 0, 302),
    ("k96_any2_f32", 7, 96, F32, 32, 4, 5, 0, 303),
    ("k2_min", 5, 2, F32, 2, 2, 3, 0, 304),
    ("symmetric_k2048_any3", 8, 2048, BF16, 64, 8, 20, SYM, 305),
    ("unweighted_k3000_any1", 6, 3000, BF16, 8, 2, 20, W_NONE, 306),
    ("many_rounds_k512", 6, 512, BF16, 128, 16, 200, 0, 307),
]


def any4():
    import weight_only_bit_row_amd as mod
    return mod


def oracle_inputs(m, g, k, variant, seed):
    """Scaled rows, sample weights and k-means++ centres of every row, from the oracle."""
    ws_rows, a_rows, c0_rows = [], [], []
    for i in range(m.w.shape[0]):
        ws, al, _, bad = oracle.scale_row(widen(m.w[i], m.dtype), g, k, symmetric=bool(variant & SYM))
        a, bad2 = oracle.weights_row(al, m.act, g, variant & 3)
        assert not bad and not bad2
        c0, _ = oracle.seed_row(ws, a, k, seed=seed, row_id=i)
        ws_rows.append(ws)
        a_rows.append(a)
        c0_rows.append(c0)
    return np.stack(ws_rows), np.stack(a_rows), np.stack(c0_rows)


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_sorted_lloyd_matches_oracle(shape):
    name, N, K, dtype, g, k, iters, variant, seed = shape
    say("sorted lloyd", name, N, K, g, k, iters, variant)
    m = make_matrix(name, N, K, dtype, seed)
    ws, a, c0 = oracle_inputs(m, g, k, variant, seed)
    dev = torch.device("cuda")
    c_gpu = any4().stage_lloyd_sorted(torch.from_numpy(ws).to(dev), torch.from_numpy(a).to(dev),
                                      torch.from_numpy(c0).to(dev), n_clusters=k, iters=iters,
                                      variant=variant, group=g).cpu().numpy()
    close = np.zeros(N, bool)
    same = np.zeros(N, bool)
    for i in range(N):
        c_ref, _, Js = oracle.lloyd_row(ws[i], a[i], c0[i], iters)
        # the objective at each side's final centroids, both evaluated by the oracle
        J_ref = Js[-1]
        J_gpu = oracle.objective_row(ws[i], a[i], oracle.estep_row(ws[i], c_gpu[i]), c_gpu[i])
        assert abs(J_gpu - J_ref) <= OBJECTIVE_REL * max(J_ref, 1e-30), (name, i, J_gpu, J_ref)
        close[i] = centroid_close(c_gpu[i], c_ref).all()
        same[i] = np.array_equal(c_gpu[i].view(np.uint32), c_ref.view(np.uint32))
    say(f"  rows within tolerance {close.mean():.3f}, bit-identical {same.mean():.3f}")
    assert close.mean() >= 0.9
    assert same.mean() >= 0.75


def test_sorted_lloyd_rows_of_few_distinct_values():
    """Rows holding only 3 to 6 distinct values: runs of equal keys in the sorted row,
    empty clusters and centroids that merge (fewer distinct centroids than k)."""
    rng = np.random.default_rng(320)
    N, K, g, k = 6, 1024, 128, 16
    w = np.stack([rng.choice(rng.normal(0, 0.02, size=3 + i % 4).astype(np.float32), size=K)
                  for i in range(N)]).astype(np.float32)
    act = rng.lognormal(0, 0.5, size=K).astype(np.float32)

    class M:
        pass
    m = M()
    m.w, m.dtype, m.act = w, F32, act
    ws, a, c0 = oracle_inputs(m, g, k, 0, 5)
    dev = torch.device("cuda")
    c_gpu = any4().stage_lloyd_sorted(torch.from_numpy(ws).to(dev), torch.from_numpy(a).to(dev),
                                      torch.from_numpy(c0).to(dev), n_clusters=k, iters=20).cpu().numpy()
    for i in range(N):
        c_ref, _, _ = oracle.lloyd_row(ws[i], a[i], c0[i], 20)
        assert np.array_equal(c_gpu[i].view(np.uint32), c_ref.view(np.uint32)), i


def test_sorted_lloyd_zero_rounds_returns_the_start():
    m = make_matrix("zero", 4, 256, BF16, 310)
    ws, a, c0 = oracle_inputs(m, 128, 16, 0, 0)
    dev = torch.device("cuda")
    c = any4().stage_lloyd_sorted(torch.from_numpy(ws).to(dev), torch.from_numpy(a).to(dev),
                                  torch.from_numpy(c0).to(dev), n_clusters=16, iters=0)
    assert np.array_equal(c.cpu().numpy().view(np.uint32), c0.view(np.uint32))


def test_sorted_lloyd_is_deterministic_and_agrees_with_the_register_path():
    """Same bits on a repeated call; against the full register path (same seeds, 20
    rounds) most rows are bit-identical and at least 90% within the centroid tolerance."""
    m = make_matrix("reg", 32, 4096, BF16, 311)
    ws, a, c0 = oracle_inputs(m, 128, 16, 0, 0)
    dev = torch.device("cuda")
    args = (torch.from_numpy(ws).to(dev), torch.from_numpy(a).to(dev), torch.from_numpy(c0).to(dev))
    c1 = any4().stage_lloyd_sorted(*args, n_clusters=16, iters=20).cpu().numpy()
    c2 = any4().stage_lloyd_sorted(*args, n_clusters=16, iters=20).cpu().numpy()
    assert np.array_equal(c1.view(np.uint32), c2.view(np.uint32))
    w = torch.from_numpy(np.ascontiguousarray(m.w).view(np.int16)).to(dev).view(torch.bfloat16)
    act = torch.from_numpy(m.act).to(dev)
    _, c_reg, _, _ = any4().stage_full(w, act, 128, 16, 20, seed=0)
    c_reg = c_reg.cpu().numpy()
    same = np.array([np.array_equal(c1[i].view(np.uint32), c_reg[i].view(np.uint32)) for i in range(32)])
    close = np.array([centroid_close(c1[i], c_reg[i]).all() for i in range(32)])
    assert close.mean() >= 0.9
    assert same.mean() >= 0.75


def test_sorted_lloyd_rejects_long_rows_and_bad_shapes():
    dev = torch.device("cuda")
    ws = torch.zeros((2, 4098), device=dev)
    c0 = torch.zeros((2, 16), device=dev)
    with pytest.raises(any4().Any4Error):
        any4().stage_lloyd_sorted(ws, ws, c0)
    with pytest.raises(ValueError):
        any4().stage_lloyd_sorted(ws[:, :64], ws[:, :32], c0)
    empty = torch.zeros((0, 64), device=dev)
    assert any4().stage_lloyd_sorted(empty, empty, torch.zeros((0, 16), device=dev)).shape == (0, 16)

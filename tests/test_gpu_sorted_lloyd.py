"""Sorted-row Lloyd (`any4_stage_lloyd_sorted`): Lloyd rounds taken on the sorted row
with fp64 prefix sums, checked against the oracle's Lloyd rounds (Section 4.1: Eq. 18
assignment, Eq. 23 update) from the same scaled rows, sample weights and starting
centroids, all computed by the oracle.  The assignment rule equals the register path's,
so only the fp64 summation order differs: every row's final objective agrees within the
objective tolerance, and every row ends with centroids bit-identical to the oracle's or
has a first divergent round (found by replaying the oracle's trajectory) whose only
differences are excused near-ties or an M-step rounding within the centroid tolerance.
"""
import numpy as np
import pytest

import oracle
from parity_util import OBJECTIVE_REL, explain_divergence, identical_centroids, say, widen
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
    # rows past 4096 columns (the instance with 32 compare pairs per thread): the layer's
    # down_proj length, the longest supported row, and a ragged one
    ("down_proj_k14336", 4, 14336, BF16, 128, 16, 20, 0, 308),
    ("max_k16384_any3_sym", 3, 16384, BF16, 64, 8, 20, SYM, 309),
    ("ragged_k10002_g2", 3, 10002, F32, 2, 16, 12, W_NONE, 310),
    # rows past 16384 columns, sorted as two halves with the sorted weights in the
    # workspace: the 70B down_proj length, the longest supported row, the shortest one
    ("down_70b_k28672", 2, 28672, BF16, 128, 16, 20, 0, 312),
    ("max_k32768_any3_sym", 2, 32768, BF16, 64, 8, 20, SYM, 313),
    ("ragged_k16386_g2", 2, 16386, F32, 2, 16, 12, W_NONE, 314),
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


def oracle_trace(ws, a, c0, iters):
    """The oracle's centroids c^0 .. c^iters of one row (Eq. 18 then Eq. 23 per round)."""
    c = [np.asarray(c0, np.float32)]
    for _ in range(iters):
        c.append(oracle.mstep_row(ws, a, oracle.estep_row(ws, c[-1]), c[-1]))
    return np.stack(c)


class Replay:
    """GPU trajectories for explain_divergence: the sorted stage after t rounds (one launch
    over the whole matrix per t, cached), and the register path's E-step assignment at
    given centroids (the sorted stage has the same assignment rule but does not expose it)."""

    def __init__(self, m, ws, a, c0, g, k, variant):
        dev = torch.device("cuda")
        self.args = (torch.from_numpy(ws).to(dev), torch.from_numpy(a).to(dev), torch.from_numpy(c0).to(dev))
        self.k, self.g, self.variant, self.cache = k, g, variant, {}
        self.w = torch.from_numpy(np.ascontiguousarray(m.w).view(np.int16 if m.dtype == BF16 else np.float32)).to(dev)
        if m.dtype == BF16:
            self.w = self.w.view(torch.bfloat16)
        self.act = torch.from_numpy(m.act).to(dev)

    def sorted_at(self, t):
        if t not in self.cache:
            self.cache[t] = any4().stage_lloyd_sorted(*self.args, n_clusters=self.k, iters=t,
                                                      variant=self.variant, group=self.g).cpu().numpy()
        return self.cache[t]

    def assign_at(self, i, c):
        c_in = np.repeat(np.asarray(c, np.float32)[None], self.w.shape[0], axis=0)
        q, _, _ = any4().stage_lloyd_step(self.w, self.act, torch.from_numpy(c_in).to(self.w.device),
                                          self.g, self.k, variant=self.variant)
        return q.cpu().numpy()[i]


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_sorted_lloyd_matches_oracle(shape):
    name, N, K, dtype, g, k, iters, variant, seed = shape
    say("sorted lloyd", name, N, K, g, k, iters, variant)
    m = make_matrix(name, N, K, dtype, seed)
    ws, a, c0 = oracle_inputs(m, g, k, variant, seed)
    replay = Replay(m, ws, a, c0, g, k, variant)
    c_gpu = replay.sorted_at(iters)
    same = np.zeros(N, bool)
    for i in range(N):
        ct = oracle_trace(ws[i], a[i], c0[i], iters)
        # the objective at each side's final centroids, both evaluated by the oracle
        J_ref = oracle.objective_row(ws[i], a[i], oracle.estep_row(ws[i], ct[-1]), ct[-1])
        J_gpu = oracle.objective_row(ws[i], a[i], oracle.estep_row(ws[i], c_gpu[i]), c_gpu[i])
        assert abs(J_gpu - J_ref) <= OBJECTIVE_REL * max(J_ref, 1e-30), (name, i, J_gpu, J_ref)
        same[i] = identical_centroids(c_gpu[i], ct[-1])
        if not same[i]:
            why = explain_divergence(ws[i], a[i], ct, lambda t: replay.sorted_at(t)[i],
                                     lambda c: replay.assign_at(i, c))
            say(f"  row {i}: {why}")
    say(f"  rows bit-identical {same.mean():.3f}")


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
    """Same bits on a repeated call.  Against the full register path (same seeds, 20
    rounds): a row where the two differ must be explained, on each side that differs
    from the oracle, by that side's first divergent round."""
    m = make_matrix("reg", 32, 4096, BF16, 311)
    g, k, iters = 128, 16, 20
    ws, a, c0 = oracle_inputs(m, g, k, 0, 0)
    replay = Replay(m, ws, a, c0, g, k, 0)
    c1 = replay.sorted_at(iters)
    c2 = any4().stage_lloyd_sorted(*replay.args, n_clusters=k, iters=iters).cpu().numpy()
    assert np.array_equal(c1.view(np.uint32), c2.view(np.uint32))
    reg_cache = {}

    def reg_at(t):
        if t not in reg_cache:
            reg_cache[t] = any4().stage_full(replay.w, replay.act, g, k, t, seed=0)[1].cpu().numpy()
        return reg_cache[t]

    c_reg = reg_at(iters)
    n_same = 0
    for i in range(32):
        if identical_centroids(c1[i], c_reg[i]):
            n_same += 1
            continue
        ct = oracle_trace(ws[i], a[i], c0[i], iters)
        if not identical_centroids(c1[i], ct[-1]):
            say(f"  row {i} sorted: " + explain_divergence(ws[i], a[i], ct, lambda t: replay.sorted_at(t)[i],
                                                           lambda c: replay.assign_at(i, c)))
        if not identical_centroids(c_reg[i], ct[-1]):
            say(f"  row {i} register: " + explain_divergence(ws[i], a[i], ct, lambda t: reg_at(t)[i],
                                                             lambda c: replay.assign_at(i, c)))
    say(f"  rows identical to the register path: {n_same}/32")


def test_sorted_lloyd_split_rows_ignore_the_workspace_contents():
    """Rows over 16384 columns keep their sorted weights in the workspace: a caller's
    workspace full of NaN bytes, and a second call reusing it, give the same bits as a
    fresh one."""
    m = make_matrix("split_ws", 3, 20480, BF16, 315)
    ws, a, c0 = oracle_inputs(m, 128, 16, 0, 0)
    dev = torch.device("cuda")
    args = (torch.from_numpy(ws).to(dev), torch.from_numpy(a).to(dev), torch.from_numpy(c0).to(dev))
    ref = any4().stage_lloyd_sorted(*args, n_clusters=16, iters=20).cpu().numpy()
    work = torch.full((3 * 3 * 16384,), float("nan"), dtype=torch.float32, device=dev)
    for _ in range(2):
        c = any4().stage_lloyd_sorted(*args, n_clusters=16, iters=20, ws=work).cpu().numpy()
        assert np.array_equal(c.view(np.uint32), ref.view(np.uint32))
    with pytest.raises(ValueError):
        any4().stage_lloyd_sorted(*args, n_clusters=16, iters=20, ws=work[:-1])


def test_sorted_lloyd_rejects_long_rows_and_bad_shapes():
    dev = torch.device("cuda")
    ws = torch.zeros((2, 32770), device=dev)
    c0 = torch.zeros((2, 16), device=dev)
    with pytest.raises(any4().Any4Error):
        any4().stage_lloyd_sorted(ws, ws, c0)
    with pytest.raises(ValueError):
        any4().stage_lloyd_sorted(ws[:, :64], ws[:, :32], c0)
    empty = torch.zeros((0, 64), device=dev)
    assert any4().stage_lloyd_sorted(empty, empty, torch.zeros((0, 16), device=dev)).shape == (0, 16)

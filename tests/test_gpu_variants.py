"""GPU parity of the method variants (the paper's ablations) against the CPU oracle.

Each variant goes through the same protocol as the default path: scaling and sample
weights bit-exact (T1), initial centres and picks bit-exact (T2), one Lloyd round from
the oracle's centroids with assignments bit-exact except near-ties and the M-step within
tolerance (T3, for every variant: initialization-only ones run the variant kernel with the
default scaled weights and Eq. 23 sample weights), and the whole path (T4: picks exact, objective within 1e-4, every row's codes
identical or its first divergence an excused near-tie or in-tolerance M-step rounding,
scale/offset bit-exact).  Restarts are checked end to end the same way (every row
identical), plus: never worse than one restart.
"""
import numpy as np
import pytest

import oracle
from parity_util import (OBJECTIVE_REL, centroid_close, check_rows, excused_mismatch, say, to_device,
                         widen)
from workloads import BF16, F32, make_matrix

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def any4():
    import weight_only_bit_row_amd as mod
    return mod


W_ACT, W_NONE = 1, 2
I_RANDOM, I_UNIFORM, I_GREEDY = 1 << 2, 2 << 2, 3 << 2
SYM = 1 << 4

VARIANTS = [
    ("weight_act", W_ACT),
    ("weight_none", W_NONE),
    ("init_random", I_RANDOM),
    ("init_uniform", I_UNIFORM),
    ("symmetric", SYM),
    ("symmetric_uniform", SYM | I_UNIFORM),
    ("symmetric_random_act", SYM | I_RANDOM | W_ACT),
    ("init_greedy", I_GREEDY),
    ("symmetric_greedy_none", SYM | I_GREEDY | W_NONE),
]

# (name, N, K, dtype, group, n_clusters, seed): wide and narrow groups, any1..any3, seven
# waves, and twelve waves with narrow groups (the 1024-lane instance)
SHAPES = [
    ("g128_k4096", 24, 4096, BF16, 128, 16, 201),
    ("narrow_g8_k1000", 9, 1000, BF16, 8, 16, 202),
    ("any2_g64_k512_f32", 12, 512, F32, 64, 4, 203),
    ("any3_k14336", 4, 14336, BF16, 128, 8, 204),
    ("any1_g32_k768", 10, 768, BF16, 32, 2, 206),
    ("narrow_g16_k24576", 2, 24576, BF16, 16, 16, 207),
]


@pytest.fixture(scope="module", params=[(v, s) for v in VARIANTS for s in SHAPES],
                ids=[f"{v[0]}-{s[0]}" for v in VARIANTS for s in SHAPES])
def case(request):
    (vname, variant), (name, N, K, dtype, g, k, seed) = request.param
    m = make_matrix(name, N, K, dtype, seed)
    return f"{vname}/{name}", m, g, k, variant


def oracle_rows(m, g, k, variant):
    rows = []
    for i in range(m.w.shape[0]):
        w32 = widen(m.w[i], m.dtype)
        ws, al, be, bad = oracle.scale_row(w32, g, k, symmetric=bool(variant & SYM))
        a, bad2 = oracle.weights_row(al, m.act, g, variant & 3)
        assert not bad and not bad2
        rows.append((ws, a, al, be))
    return rows


def test_variant_scale_bit_exact(case):
    name, m, g, k, variant = case
    say(f"variant T1 {name}")
    w, act = to_device(m)
    ws, al, be, a = (t.cpu().numpy() for t in any4().stage_scale(w, act, g, k, variant=variant))
    for i, (rws, ra, ral, rbe) in enumerate(oracle_rows(m, g, k, variant)):
        assert np.array_equal(ws[i].view(np.uint32), rws.view(np.uint32)), (name, i)
        assert np.array_equal(al[i].view(np.uint32), ral.view(np.uint32)), (name, i)
        assert np.array_equal(be[i].view(np.uint32), rbe.view(np.uint32)), (name, i)
        assert np.array_equal(a[i].view(np.uint32), ra.view(np.uint32)), (name, i)


def test_variant_seed_bit_exact(case):
    name, m, g, k, variant = case
    say(f"variant T2 {name}")
    w, act = to_device(m)
    c0, picks = any4().stage_seed(w, act, g, k, seed=99, row_offset=5, variant=variant)
    c0, picks = c0.cpu().numpy(), picks.cpu().numpy()
    init = (variant >> 2) & 3
    level0 = (1 - k // 2) if variant & SYM else 0
    for i, (ws, a, _, _) in enumerate(oracle_rows(m, g, k, variant)):
        rc, rp = oracle.seed_row(ws, a, k, 99, 5 + i, 0, init=init, level0=level0)
        assert np.array_equal(picks[i], rp), (name, i, picks[i], rp)
        assert np.array_equal(c0[i].view(np.uint32), rc.view(np.uint32)), (name, i)


def test_variant_lloyd_round(case):
    # initialization-only variants run the variant kernel instance with the default
    # scaling and sample weights: its round must match the oracle's too
    name, m, g, k, variant = case
    say(f"variant T3 {name}")
    ref = oracle.quantize(m.w, m.dtype, m.act, g, k, 6, trace=True, variant=variant)
    rows = oracle_rows(m, g, k, variant)
    w, act = to_device(m)
    for t in (0, 3):
        c_in = torch.from_numpy(ref["c_trace"][:, t, :].copy()).cuda()
        assign, c_out, obj = any4().stage_lloyd_step(w, act, c_in, g, k, variant=variant)
        assign, c_out = assign.cpu().numpy(), c_out.cpu().numpy()
        for i, (ws, a, _, _) in enumerate(rows):
            c_t = ref["c_trace"][i, t]
            q_ref = oracle.estep_row(ws, c_t)
            diff, ok = excused_mismatch(ws, c_t, q_ref, assign[i])
            assert ok.all(), (name, i, t, diff[~ok][:5])
            assert centroid_close(c_out[i], oracle.mstep_row(ws, a, assign[i], c_t)).all()


def _end_to_end(name, m, g, k, variant, iters=20):
    w, act = to_device(m)
    out, c_final, picks, ws = any4().stage_full(w, act, g, k, iters, seed=0, variant=variant)
    assert any4().read_status(ws) == 0
    ref = oracle.quantize(m.w, m.dtype, m.act, g, k, iters, seed=0, variant=variant)
    assert ref["status"] == 0
    obj = out.objective.cpu().numpy()
    J, Jr = obj.sum(), ref["objective"].sum()
    assert abs(J - Jr) <= OBJECTIVE_REL * max(Jr, 1e-30), (J, Jr)
    codes = out.codes.cpu().numpy()
    assert np.array_equal(picks.cpu().numpy(), ref["picks"])
    same = check_rows(any4(), m, g, k, iters, 0, codes, c_final.cpu().numpy(),
                      out.lut.cpu().numpy().view(np.uint16), ref, np.arange(m.w.shape[0]),
                      variant=variant)
    assert np.array_equal(out.scale.cpu().numpy().view(np.uint16), ref["scale"])
    assert np.array_equal(out.offset.cpu().numpy().view(np.uint16), ref["offset"])
    say(f"  {name}: rows with identical codes {same.mean():.4f}, dJ/J {(J - Jr) / max(Jr, 1e-300):.2e}")
    return obj


def test_variant_end_to_end(case):
    name, m, g, k, variant = case
    say(f"variant T4 {name}")
    _end_to_end(name, m, g, k, variant)


@pytest.mark.parametrize("init", [0, I_RANDOM, I_GREEDY])
def test_restarts_end_to_end(init):
    m = make_matrix("restarts", 16, 4096, BF16, 205)
    say(f"restarts init={init}")
    three = _end_to_end(f"restarts3/{init}", m, 128, 16, init | (2 << 8), iters=8)
    one = _end_to_end(f"restarts1/{init}", m, 128, 16, init, iters=8)
    assert np.all(three <= one)
    assert np.sum(three < one) > 0      # a later restart wins somewhere

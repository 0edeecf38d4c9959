"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Stage protocol (tolerances in parity_util):
  T1 scaling and sample weights bit-exact;  T2 k-means++ picks and seeds bit-exact;
  T3 one Lloyd round from the oracle's centroids: assignments bit-exact except
     near-ties, M-step within 1e-5 (oracle M-step re-evaluated on the GPU's
     assignment);  T4 end-to-end objective within 1e-4;  T5 emission byte-exact given
     the same inputs;  T6 repeat runs and row-sharded runs bit-identical.
"""
import numpy as np
import pytest

import oracle
from parity_util import (OBJECTIVE_REL, centroid_close, check_rows, excused_mismatch, oracle_row_inputs,
                         say, to_device, unpack_codes, widen)
from workloads import BF16, F32, make, make_matrix

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def any4():
    import weight_only_bit_row_amd as mod
    return mod


# (name, N, K, dtype, group, n_clusters, seed): small cases spanning several lanes and
# waves, ragged rows (a lane only partly filled), and every kernel geometry.
SHAPES = [
    ("tiny_fp32", 128, 512, F32, 128, 16, 101),
    ("g64_bf16", 40, 2048, BF16, 64, 16, 102),
    ("k4096_narrow_g32", 12, 4096, BF16, 32, 16, 31),
    ("k4096_narrow_g2", 6, 4096, BF16, 2, 8, 32),
    ("k4096_g8", 6, 4096, F32, 8, 16, 33),
    ("k4096_wide_g1024", 10, 4096, BF16, 1024, 16, 34),
    ("k4096_row_group", 6, 4096, BF16, 4096, 4, 35),
    ("ragged_k1000", 9, 1000, BF16, 8, 16, 36),
    ("ragged_k96", 7, 96, F32, 32, 4, 37),
    ("k2_min", 5, 2, F32, 2, 2, 38),
    ("e16_g16", 8, 1024, BF16, 16, 16, 39),
    ("two_waves_k8192", 6, 8192, BF16, 128, 16, 40),
    ("two_waves_group_spans_waves", 4, 8192, BF16, 8192, 16, 41),
    ("seven_waves_k14336", 5, 14336, BF16, 128, 16, 42),
    ("fourteen_waves_k28672", 3, 28672, BF16, 128, 16, 43),
    ("sixteen_waves_ragged_g2", 2, 32766, BF16, 2, 16, 46),
    ("eight_waves_group_16384", 3, 16384, BF16, 16384, 8, 44),
    ("any2_k4096", 8, 4096, BF16, 128, 4, 45),
]


def shape_ids():
    return [s[0] for s in SHAPES]


@pytest.fixture(scope="module", params=SHAPES, ids=shape_ids())
def case(request):
    name, N, K, dtype, g, k, seed = request.param
    m = make_matrix(name, N, K, dtype, seed)
    return name, m, g, k


def oracle_rows(m, g, k):
    rows = []
    for i in range(m.w.shape[0]):
        ws, a, al, be, bad = oracle.prepare_row(m.w[i], m.dtype, m.act, g, k)
        assert not bad
        rows.append((ws, a, al, be))
    return rows


# ---- T1 -----------------------------------------------------------------------------

def test_t1_scale_bit_exact(case):
    name, m, g, k = case
    say(f"T1 scale {name} {m.w.shape} g={g} k={k}")
    w, act = to_device(m)
    ws, al, be, a = any4().stage_scale(w, act, group=g, n_clusters=k)
    torch.cuda.synchronize()
    ws, al, be, a = (t.cpu().numpy() for t in (ws, al, be, a))
    for i, (rws, ra, ral, rbe) in enumerate(oracle_rows(m, g, k)):
        assert np.array_equal(ws[i].view(np.uint32), rws.view(np.uint32)), (name, i)
        assert np.array_equal(al[i].view(np.uint32), ral.view(np.uint32)), (name, i)
        assert np.array_equal(be[i].view(np.uint32), rbe.view(np.uint32)), (name, i)
        assert np.array_equal(a[i].view(np.uint32), ra.view(np.uint32)), (name, i)


# ---- T2 -----------------------------------------------------------------------------

@pytest.mark.parametrize("seed,row_offset,matrix_index", [(0, 0, 0), (12345678901234, 77, 3)])
def test_t2_seed_bit_exact(case, seed, row_offset, matrix_index):
    name, m, g, k = case
    say(f"T2 seed {name} seed={seed} row_offset={row_offset}")
    w, act = to_device(m)
    c0, picks = any4().stage_seed(w, act, group=g, n_clusters=k, seed=seed, row_offset=row_offset,
                                  matrix_index=matrix_index)
    torch.cuda.synchronize()
    c0, picks = c0.cpu().numpy(), picks.cpu().numpy()
    for i, (ws, a, _, _) in enumerate(oracle_rows(m, g, k)):
        rc, rp = oracle.seed_row(ws, a, k, seed, row_offset + i, matrix_index)
        assert np.array_equal(picks[i], rp), (name, i, picks[i], rp)
        assert np.array_equal(c0[i].view(np.uint32), rc.view(np.uint32)), (name, i)


# ---- T3 -----------------------------------------------------------------------------

def test_t3_lloyd_rounds(case):
    name, m, g, k = case
    iters = 12
    ref = oracle.quantize(m.w, m.dtype, m.act, g, k, iters, trace=True)
    rows = oracle_rows(m, g, k)
    w, act = to_device(m)
    n_excused = n_checked = 0
    for t in [0, 1, 4, iters - 1]:
        say(f"T3 lloyd {name} from oracle c^{t}")
        c_in = torch.from_numpy(ref["c_trace"][:, t, :].copy()).cuda()
        assign, c_out, obj = any4().stage_lloyd_step(w, act, c_in, group=g, n_clusters=k)
        torch.cuda.synchronize()
        assign, c_out, obj = assign.cpu().numpy(), c_out.cpu().numpy(), obj.cpu().numpy()
        for i, (ws, a, _, _) in enumerate(rows):
            c_t = ref["c_trace"][i, t]
            q_ref = oracle.estep_row(ws, c_t)
            diff, ok = excused_mismatch(ws, c_t, q_ref, assign[i])
            assert ok.all(), (name, i, t, diff[~ok][:5])
            n_excused += diff.size
            n_checked += ws.size
            c_ref = oracle.mstep_row(ws, a, assign[i], c_t)
            assert centroid_close(c_out[i], c_ref).all(), (name, i, t, c_out[i], c_ref)
            J_ref = ref["j_trace"][i, t]
            assert abs(obj[i] - J_ref) <= 1e-6 * max(J_ref, 1e-30), (name, i, t, obj[i], J_ref)
    say(f"  {name}: {n_excused} excused near-ties in {n_checked} assignments")


# ---- T4 / T6 ------------------------------------------------------------------------

def test_t4_end_to_end(case):
    name, m, g, k = case
    iters = 20
    say(f"T4 full {name}")
    w, act = to_device(m)
    out, c_final, picks, ws = any4().stage_full(w, act, group=g, n_clusters=k, iters=iters, seed=0)
    torch.cuda.synchronize()
    assert any4().read_status(ws) == 0
    ref = oracle.quantize(m.w, m.dtype, m.act, g, k, iters, seed=0)
    assert ref["status"] == 0
    assert np.array_equal(picks.cpu().numpy(), ref["picks"])
    obj = out.objective.cpu().numpy()
    J, Jr = obj.sum(), ref["objective"].sum()
    assert abs(J - Jr) <= OBJECTIVE_REL * Jr, (J, Jr)
    codes = out.codes.cpu().numpy()
    cf = c_final.cpu().numpy()
    lut = out.lut.cpu().numpy().view(np.uint16)
    same_rows = check_rows(any4(), m, g, k, iters, 0, codes, cf, lut, ref, np.arange(m.w.shape[0]))
    # scale/offset do not depend on the clustering: bit-exact
    assert np.array_equal(out.scale.cpu().numpy().view(np.uint16), ref["scale"])
    assert np.array_equal(out.offset.cpu().numpy().view(np.uint16), ref["offset"])
    say(f"  {name}: rows with identical codes {same_rows.mean():.4f}, dJ/J {(J - Jr) / max(Jr, 1e-300):.2e}")


# Many rounds: most rows reach an exact fixed point well before the last round and the
# kernel stops there; the oracle runs every round, so the two must still agree row by row.
MANY_ROUNDS = [("g64_bf16_64_rounds", 40, 2048, BF16, 64, 16, 102, 64),
               ("two_waves_k8192_48_rounds", 6, 8192, BF16, 128, 16, 40, 48),
               ("seven_waves_k14336_40_rounds", 5, 14336, BF16, 128, 16, 42, 40),
               ("any2_k4096_30_rounds", 8, 4096, BF16, 128, 4, 45, 30)]


@pytest.mark.parametrize("shape", MANY_ROUNDS, ids=[s[0] for s in MANY_ROUNDS])
def test_t4_many_rounds_fixed_point_stop(shape):
    name, N, K, dtype, g, k, seed, iters = shape
    say(f"T4 many rounds {name}")
    m = make_matrix(name, N, K, dtype, seed)
    w, act = to_device(m)
    out, c_final, picks, ws = any4().stage_full(w, act, group=g, n_clusters=k, iters=iters, seed=0)
    torch.cuda.synchronize()
    assert any4().read_status(ws) == 0
    ref = oracle.quantize(m.w, m.dtype, m.act, g, k, iters, seed=0)
    assert np.array_equal(picks.cpu().numpy(), ref["picks"])
    J, Jr = out.objective.cpu().numpy().sum(), ref["objective"].sum()
    assert abs(J - Jr) <= OBJECTIVE_REL * Jr, (J, Jr)
    same_rows = check_rows(any4(), m, g, k, iters, 0, out.codes.cpu().numpy(), c_final.cpu().numpy(),
                           out.lut.cpu().numpy().view(np.uint16), ref, np.arange(N))
    # one round more changes nothing on a row that reached a fixed point in both runs
    c_more = any4().stage_full(w, act, group=g, n_clusters=k, iters=iters + 1, seed=0)[1].cpu().numpy()
    ref_more = oracle.quantize(m.w, m.dtype, m.act, g, k, iters + 1, seed=0)
    fixed = np.all(ref_more["c_final"].view(np.uint32) == ref["c_final"].view(np.uint32), axis=1)
    for i in np.nonzero(fixed & same_rows)[0]:
        assert np.array_equal(c_more[i].view(np.uint32), c_final.cpu().numpy()[i].view(np.uint32)), (name, i)
    say(f"  {name}: rows identical {same_rows.mean():.3f}, at a fixed point {fixed.mean():.3f}")
    # every round run, no stop at the fixed point: the same bar against the oracle, and
    # the same bits as the stopping run on every row that the tests have seen
    out_a, c_a, picks_a, ws_a = any4().stage_full(w, act, group=g, n_clusters=k, iters=iters, seed=0,
                                                  variant=any4().ALL_ROUNDS)
    torch.cuda.synchronize()
    assert any4().read_status(ws_a) == 0
    assert np.array_equal(picks_a.cpu().numpy(), ref["picks"])
    codes_a, c_a = out_a.codes.cpu().numpy(), c_a.cpu().numpy()
    check_rows(any4(), m, g, k, iters, 0, codes_a, c_a, out_a.lut.cpu().numpy().view(np.uint16), ref,
               np.arange(N), variant=any4().ALL_ROUNDS)
    same_bits = np.all(codes_a == out.codes.cpu().numpy(), axis=1) & \
        np.all(c_a.view(np.uint32) == c_final.cpu().numpy().view(np.uint32), axis=1)
    say(f"  {name}: all rounds vs stopping run, rows with the same bits {same_bits.mean():.3f}")


def test_t6_repeat_and_row_shards(case):
    name, m, g, k = case
    say(f"T6 determinism {name}")
    w, act = to_device(m)
    a1 = any4().quantize(w, act, group=g, n_clusters=k, iters=10, seed=5, matrix_index=2)
    a2 = any4().quantize(w, act, group=g, n_clusters=k, iters=10, seed=5, matrix_index=2)
    N = w.shape[0]
    h = N // 2
    s1 = any4().quantize(w[:h].contiguous(), act, group=g, n_clusters=k, iters=10, seed=5,
                         row_offset=0, matrix_index=2)
    s2 = any4().quantize(w[h:].contiguous(), act, group=g, n_clusters=k, iters=10, seed=5,
                         row_offset=h, matrix_index=2)
    torch.cuda.synchronize()
    for f in ["codes", "lut", "scale", "offset", "objective"]:
        x1, x2 = getattr(a1, f).cpu(), getattr(a2, f).cpu()
        assert torch.equal(x1.view(torch.uint8), x2.view(torch.uint8)), f
        sh = torch.cat([getattr(s1, f).cpu(), getattr(s2, f).cpu()])
        assert torch.equal(x1.view(torch.uint8), sh.view(torch.uint8)), f


# ---- T5 -----------------------------------------------------------------------------

@pytest.mark.parametrize("N,K,g,k", [(7, 512, 128, 16), (3, 4096, 64, 8), (5, 96, 32, 4), (2, 2, 2, 2)])
def test_t5_pack_byte_exact(N, K, g, k):
    say(f"T5 pack {N}x{K} g={g} k={k}")
    rng = np.random.default_rng(N * K + k)
    assign = rng.integers(0, k, (N, K)).astype(np.uint8)
    c = rng.uniform(0, k - 1, (N, k)).astype(np.float32)
    c[0, 0] = 65519.0  # rounds to fp16 max; ties and large values
    al = (rng.standard_normal((N, K // g)) * 0.01).astype(np.float32)
    be = (rng.standard_normal((N, K // g)) * 0.1).astype(np.float32)
    al[0, 0] = 3e-6  # fp16 subnormal
    d = lambda x: torch.from_numpy(x).cuda()
    out = any4().stage_pack(N, K, d(assign), d(c), d(al), d(be), group=g, n_clusters=k)
    torch.cuda.synchronize()
    codes = np.stack([oracle.pack_row(assign[i]) for i in range(N)])
    assert np.array_equal(out.codes.cpu().numpy(), codes)
    assert np.array_equal(out.lut.cpu().numpy().view(np.uint16), oracle.fp16_bits(c).reshape(N, k))
    assert np.array_equal(out.scale.cpu().numpy().view(np.uint16), oracle.fp16_bits(al).reshape(al.shape))
    assert np.array_equal(out.offset.cpu().numpy().view(np.uint16), oracle.fp16_bits(be).reshape(be.shape))


# ---- edge cases -----------------------------------------------------------------------

def test_empty_matrix():
    w = torch.zeros((0, 512), dtype=torch.bfloat16, device="cuda")
    act = torch.ones(512, device="cuda")
    out = any4().quantize(w, act)
    torch.cuda.synchronize()
    assert out.codes.shape == (0, 256)


def test_nonfinite_rows_flagged():
    m = make_matrix("nf", 6, 1024, F32, 50)
    w = m.w.copy()
    w[1, 17] = np.nan
    w[4, 3] = np.inf
    say("edge nonfinite rows")
    wt = torch.from_numpy(w).cuda()
    act = torch.from_numpy(m.act).cuda()
    out, c_final, picks, ws = any4().stage_full(wt, act, group=128, n_clusters=16, iters=5)
    torch.cuda.synchronize()
    assert any4().read_status(ws) == 5
    ref = oracle.quantize(w, 0, m.act, 128, 16, 5)
    assert ref["status"] == 5
    obj = out.objective.cpu().numpy()
    assert np.isnan(obj[[1, 4]]).all() and np.isfinite(obj[[0, 2, 3, 5]]).all()
    for f in ["codes", "lut", "scale", "offset"]:
        g = getattr(out, f).cpu().numpy().view(np.uint8)
        r = ref[f].view(np.uint8)
        assert np.array_equal(g[[1, 4]], r[[1, 4]]), f
        assert not g[[1, 4]].any()
    # negative activation statistic: every row is bad
    act2 = m.act.copy()
    act2[5] = -1.0
    out2, _, _, ws2 = any4().stage_full(torch.from_numpy(m.w).cuda(), torch.from_numpy(act2).cuda(),
                                        group=128, n_clusters=16, iters=2)
    torch.cuda.synchronize()
    assert any4().read_status(ws2) == 5
    assert np.isnan(out2.objective.cpu().numpy()).all()


@pytest.mark.parametrize("k", [2, 4, 8])
def test_fewer_clusters_end_to_end(k):
    m = make_matrix("kk", 16, 2048, BF16, 60 + k)
    say(f"edge k={k}")
    w, act = to_device(m)
    out, c_final, picks, _ = any4().stage_full(w, act, group=128, n_clusters=k, iters=20)
    torch.cuda.synchronize()
    ref = oracle.quantize(m.w, 1, m.act, 128, k, 20)
    assert np.array_equal(picks.cpu().numpy(), ref["picks"])
    J, Jr = out.objective.cpu().numpy().sum(), ref["objective"].sum()
    assert abs(J - Jr) <= OBJECTIVE_REL * Jr
    codes = unpack_codes(out.codes.cpu().numpy())
    assert codes.max() < k


def test_iters_zero_and_degenerate_rows():
    K = 512
    rng = np.random.default_rng(70)
    w = (rng.standard_normal((6, K)) * 0.02).astype(np.float32)
    w[1] = 0.25                      # constant row: alpha = 0 everywhere
    w[2, :128] = -1.0                # one constant group
    act = rng.lognormal(0, 0.5, K).astype(np.float32)
    act[:64] = 0.0                   # zero-weight channels
    say("edge iters=0 / degenerate rows")
    for iters in [0, 3]:
        out, c_final, picks, _ = any4().stage_full(torch.from_numpy(w).cuda(), torch.from_numpy(act).cuda(),
                                                   group=128, n_clusters=16, iters=iters)
        torch.cuda.synchronize()
        ref = oracle.quantize(w, 0, act, 128, 16, iters)
        assert np.array_equal(picks.cpu().numpy(), ref["picks"])
        assert np.array_equal(out.codes.cpu().numpy(), ref["codes"])
        assert np.array_equal(c_final.cpu().numpy().view(np.uint32)[[1]], ref["c_final"].view(np.uint32)[[1]])
        assert out.objective.cpu().numpy()[1] == 0.0


def test_exact_level_rows_reconstruct():
    from test_oracle_kmeans import exact_level_rows
    K, g, k = 1024, 64, 16
    w = exact_level_rows(8, K, g, k, 71)
    act = np.random.default_rng(72).lognormal(0, 0.5, K).astype(np.float32)
    say("edge exact-level rows")
    out = any4().quantize(torch.from_numpy(w).cuda(), torch.from_numpy(act).cuda(), group=g,
                          n_clusters=k, iters=10)
    torch.cuda.synchronize()
    assert (out.objective.cpu().numpy() == 0).all()
    lut = out.lut.cpu().numpy().astype(np.float64)
    q = unpack_codes(out.codes.cpu().numpy()).astype(int)
    al = np.repeat(out.scale.cpu().numpy().astype(np.float64), g, axis=1)
    be = np.repeat(out.offset.cpu().numpy().astype(np.float64), g, axis=1)
    assert np.array_equal(al * np.take_along_axis(lut, q, axis=1) + be, w.astype(np.float64))


def test_batch_equals_single_calls():
    mats = [make_matrix("b0", 33, 4096, BF16, 80), make_matrix("b1", 17, 14336, BF16, 81),
            make_matrix("b2", 9, 1024, F32, 82)]
    say("batch vs single")
    dev = [to_device(m) for m in mats]
    outs = any4().quantize_batch(dev, group=128, n_clusters=16, iters=6, seed=9)
    torch.cuda.synchronize()
    for i, (w, act) in enumerate(dev):
        single = any4().quantize(w, act, group=128, n_clusters=16, iters=6, seed=9, matrix_index=i)
        torch.cuda.synchronize()
        for f in ["codes", "lut", "scale", "offset", "objective"]:
            assert torch.equal(getattr(outs[i], f).cpu().view(torch.uint8),
                               getattr(single, f).cpu().view(torch.uint8)), (i, f)


# ---- the named workloads at full size, on sampled rows ----------------------------------

FULL = [("up_proj", 32), ("down_70b", 32), ("q_proj_g64", 32), ("q_proj_g128", 32)]


def _sample(N, n):
    return np.unique(np.concatenate([[0, N - 1], np.linspace(0, N - 1, n).astype(int)]))


def _check_sampled(m, out, cf, pk, g, k, iters, rows):
    """The oracle on each sampled row alone (row_offset = its index keeps its Philox
    stream): picks and scale/offset bit-exact, codes identical or explained, centroids
    and LUT within tolerance, and the sampled rows' objective sum within 1e-4."""
    codes, obj = out.codes.cpu().numpy(), out.objective.cpu().numpy()
    lut = out.lut.cpu().numpy().view(np.uint16)
    scale = out.scale.cpu().numpy().view(np.uint16)
    offset = out.offset.cpu().numpy().view(np.uint16)
    cf, pk = cf.cpu().numpy(), pk.cpu().numpy()
    J = Jr = 0.0
    same = np.zeros(rows.size, bool)
    for n, i in enumerate(rows):
        r = oracle.quantize(m.w[i:i + 1], m.dtype, m.act, g, k, iters, seed=0, row_offset=int(i),
                            matrix_index=m.matrix_index)
        assert r["status"] == 0
        assert np.array_equal(pk[i], r["picks"][0]), (m.name, i, pk[i], r["picks"][0])
        assert np.array_equal(scale[i], r["scale"][0]) and np.array_equal(offset[i], r["offset"][0]), (m.name, i)
        same[n] = check_rows(any4(), m, g, k, iters, 0, codes, cf, lut, r, [i], [0], m.matrix_index)[0]
        J += obj[i]
        Jr += r["objective"][0]
    assert abs(J - Jr) <= OBJECTIVE_REL * Jr, (m.name, J, Jr)
    return same, (J - Jr) / Jr


@pytest.mark.parametrize("wname,n_sample", FULL, ids=[f[0] for f in FULL])
def test_full_size_sampled_rows(wname, n_sample):
    wl = make(wname)
    m = wl.matrices[0]
    say(f"full-size {wname} {m.w.shape}: one launch over all rows, oracle on {n_sample}+ rows")
    w, act = to_device(m)
    outs, cfs, pks, _ = any4().stage_quantize_batch([(w, act)], group=wl.group, n_clusters=wl.n_clusters,
                                                    iters=wl.iters, seed=0)
    torch.cuda.synchronize()
    rows = _sample(m.w.shape[0], n_sample)
    same, dj = _check_sampled(m, outs[0], cfs[0], pks[0], wl.group, wl.n_clusters, wl.iters, rows)
    say(f"  {wname}: {same.sum()}/{rows.size} sampled rows identical, dJ/J {dj:.2e}")


@pytest.mark.parametrize("bits", [4, 3, 2])
def test_layer_batch_sampled_rows(bits):
    """The 7 matrices of a decoder layer in one call (any4/any3/any2): on 64+ rows of
    every matrix, including its first and last, picks, codes, LUT, scale and offset are
    compared with the oracle row by row, which checks the launch's mapping of blocks to
    matrices, rows, Philox counters and cluster counts."""
    wl = make(f"layer_any{bits}")
    say(f"layer any{bits}: one call over 7 matrices")
    dev = [to_device(m) for m in wl.matrices]
    outs, cfs, pks, ws = any4().stage_quantize_batch(dev, group=wl.group, n_clusters=wl.n_clusters,
                                                     iters=wl.iters, seed=0,
                                                     matrix_indices=[m.matrix_index for m in wl.matrices])
    torch.cuda.synchronize()
    assert any4().read_status(ws) == 0
    for m, o, cf, pk in zip(wl.matrices, outs, cfs, pks):
        rows = _sample(m.w.shape[0], 64)
        same, dj = _check_sampled(m, o, cf, pk, wl.group, wl.n_clusters, wl.iters, rows)
        say(f"  any{bits} {m.name} {m.w.shape}: {same.sum()}/{rows.size} sampled rows identical, "
            f"dJ/J {dj:.2e}")


# Rows of 2-16 waves sum the Eq. 23 terms in 64-bit fixed point scaled to the row's
# largest sample weight.  Weights spread over 2^40 (a tenth of the channels scaled by
# 2^-28, one in a hundred by 2^12) must still give the oracle's rounds and codes, also
# under symmetric scaling, where w_S and so the S1 terms are negative.
WIDE_SPAN = [("two_waves_k4096", 6, 4096, BF16, 128, 16, 54, 0),
             ("three_waves_symmetric_any3_k6144", 4, 6144, BF16, 64, 8, 55, 1 << 4),
             ("five_waves_k10240", 4, 10240, BF16, 128, 16, 51, 0),
             ("fourteen_waves_k28672", 2, 28672, BF16, 128, 16, 52, 0),
             ("seven_waves_symmetric_k14336", 3, 14336, BF16, 128, 16, 53, 1 << 4)]


@pytest.mark.parametrize("shape", WIDE_SPAN, ids=[s[0] for s in WIDE_SPAN])
def test_fixed_point_sums_wide_weight_span(shape):
    name, N, K, dtype, g, k, seed, variant = shape
    say(f"fixed-point M-step, wide weight span {name}")
    m = make_matrix(name, N, K, dtype, seed)
    rng = np.random.default_rng(seed)
    act = m.act.astype(np.float64)
    small = rng.choice(K, K // 10, replace=False)
    act[small] *= 2.0 ** -28
    act[rng.choice(np.setdiff1d(np.arange(K), small), K // 100, replace=False)] *= 2.0 ** 12
    m.act = act.astype(np.float32)
    w, act_d = to_device(m)
    # one round from the oracle's centroids: assignments up to near-ties, M-step within
    # tolerance of the oracle's on the GPU's assignment
    iters = 8
    ref = oracle.quantize(m.w, m.dtype, m.act, g, k, iters, trace=True, variant=variant)
    for t in (0, 3):
        c_in = torch.from_numpy(ref["c_trace"][:, t, :].copy()).cuda()
        assign, c_out, _ = any4().stage_lloyd_step(w, act_d, c_in, group=g, n_clusters=k, variant=variant)
        torch.cuda.synchronize()
        assign, c_out = assign.cpu().numpy(), c_out.cpu().numpy()
        for i in range(N):
            ws, a = oracle_row_inputs(m.w[i], m.dtype, m.act, g, k, variant)
            c_t = ref["c_trace"][i, t]
            diff, ok = excused_mismatch(ws, c_t, oracle.estep_row(ws, c_t), assign[i])
            assert ok.all(), (name, i, t, diff[~ok][:5])
            c_ref = oracle.mstep_row(ws, a, assign[i].astype(np.int32), c_t)
            assert centroid_close(c_out[i], c_ref).all(), (name, i, t, c_out[i], c_ref)
    # the whole path: picks exact, every row identical or explained
    out, c_final, picks, ws_buf = any4().stage_full(w, act_d, group=g, n_clusters=k, iters=iters,
                                                    seed=0, variant=variant)
    torch.cuda.synchronize()
    assert any4().read_status(ws_buf) == 0
    assert np.array_equal(picks.cpu().numpy(), ref["picks"])
    same = check_rows(any4(), m, g, k, iters, 0, out.codes.cpu().numpy(), c_final.cpu().numpy(),
                      out.lut.cpu().numpy().view(np.uint16), ref, np.arange(N), variant=variant)
    say(f"  {name}: rows with identical codes {same.mean():.4f}")

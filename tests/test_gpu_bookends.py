"""GPU parity of the bookends (HIP path through the C ABI) against the CPU oracle.

  * E|x_j| (Section 4.1): within one fp32 ulp of the oracle on every channel (the fp64
    sums are taken over token slices on the GPU and sequentially in the oracle; the
    two can differ only in the last bit of the fp64 sum), bit-identical across runs.
  * dequantization (Section 2.5.2, Eq. 4): bit-exact in fp32 and in bf16 (RNE) on
    quantizer outputs and on random codes/LUTs/scales, vector and scalar paths.
  * LUT matrix-vector products (Eq. 4 applied on the fly): within 1e-5 of
    sum_j |x_j| (|alpha L| + |beta|) of the oracle's fp64 result, one to eight tokens,
    one and several K-slices per row group, NaN where a code lies past the LUT,
    bit-identical across calls.
  * end to end: E|x| from synthetic activations on the GPU -> quantize -> dequantize,
    exact reconstruction of exact-level rows, and any4's output error below uniform
    int4 with the same group scaling.
"""
import numpy as np
import pytest

import oracle
from parity_util import say, to_device
from workloads import BF16, F32, draw_act, draw_activations, make, make_activations, make_matrix
from test_oracle_kmeans import exact_level_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def any4():
    import weight_only_bit_row_amd as mod
    return mod


def _dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def _ulp_diff(a, b):
    ia = a.view(np.int32).astype(np.int64)
    ib = b.view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


# --- E|x_j| ----------------------------------------------------------------------------

# (name, T, K, dtype, seed): vector and scalar paths, one and many token slices,
# ragged channel counts, a single token, a single channel.
ABS_CASES = [
    ("bf16_vec_many_slices", 5000, 256, BF16, 1),
    ("bf16_vec_tail_tokens", 1037, 4096, BF16, 2),
    ("bf16_scalar_k1001", 301, 1001, BF16, 3),
    ("f32_vec", 777, 2048, F32, 4),
    ("f32_scalar_k13", 95, 13, F32, 5),
    ("one_token", 1, 520, F32, 6),
    ("one_channel", 4099, 1, BF16, 7),
    ("k_spans_blocks", 70, 6152, BF16, 8),
]


@pytest.mark.parametrize("case", ABS_CASES, ids=[c[0] for c in ABS_CASES])
def test_absmean_matches_oracle(case):
    name, T, K, dtype, seed = case
    say(f"absmean {name}: T={T} K={K}")
    rng = np.random.default_rng(seed)
    x = draw_activations(rng, T, draw_act(rng, K), dtype)
    got = any4().act_absmean(_dev(x)).cpu().numpy()
    ref = oracle.act_absmean(x, dtype)
    d = _ulp_diff(got, ref)
    assert d.max() <= 1, (name, d.max())
    say(f"  {name}: {np.mean(d == 0):.4f} of channels bit-exact, max {d.max()} ulp")
    again = any4().act_absmean(_dev(x)).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32))


def test_absmean_calibration_batch():
    """The 1000-token calibration case at K = 4096, every channel (the 128 x 2048-token
    batch is checked on sampled channels where bench.py times it)."""
    x = make_activations("calib_small")
    got = any4().act_absmean(_dev(x)).cpu().numpy()
    ref = oracle.act_absmean(x, BF16)
    assert _ulp_diff(got, ref).max() <= 1
    say(f"  calib_small: {np.mean(got == ref):.4f} of channels bit-exact")


def test_absmean_nonfinite_propagates_and_rejects_bad_args():
    x = np.ones((10, 8), np.float32)
    x[3, 2] = np.inf
    x[5, 6] = np.nan
    got = any4().act_absmean(_dev(x)).cpu().numpy()
    assert np.isinf(got[2]) and np.isnan(got[6]) and np.all(got[[0, 1, 3, 4, 5, 7]] == 1.0)
    with pytest.raises(any4().Any4Error):
        any4().act_absmean(torch.empty((0, 8), device="cuda"))


# --- dequantization ---------------------------------------------------------------------

def _check_dequant(q, g, k, codes, lut, scale, offset, name):
    """Bit-exact where the oracle is a number; NaN exactly where it is NaN (NaN payloads
    are not compared)."""
    ref = oracle.dequantize(codes, lut, scale, offset, g, k)
    f32 = any4().dequantize(q, g, k, out_dtype=torch.float32).cpu().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(f32), nan), name
    assert np.array_equal(f32[~nan].view(np.uint32), ref[~nan].view(np.uint32)), name
    b16 = any4().dequantize(q, g, k, out_dtype=torch.bfloat16).cpu().view(torch.int16).numpy()
    b16 = b16.view(np.uint16)
    rb = oracle.bf16_bits(ref)
    b16_nan = ((b16 & 0x7F80) == 0x7F80) & ((b16 & 0x7F) != 0)
    assert np.array_equal(b16_nan, nan), name
    assert np.array_equal(b16[~nan], rb[~nan]), name


# (name, N, K, group, k, seed): vector path (K, group multiples of 16) and scalar path
DQ_RANDOM = [
    ("vec_g128_k16", 33, 4096, 128, 16, 1),
    ("vec_g16_k8_codes_past_lut", 20, 512, 16, 8, 3),
    ("scalar_g8", 17, 1000, 8, 16, 6),
    ("scalar_g2_k34", 9, 34, 2, 4, 4),
    ("vec_long_row", 3, 28672, 128, 16, 5),
]


@pytest.mark.parametrize("case", DQ_RANDOM, ids=[c[0] for c in DQ_RANDOM])
def test_dequant_random_fields_bit_exact(case):
    """Random codes (including codes past the LUT when k < 16), random fp16 LUTs and
    group scales/offsets, including subnormal and negative values."""
    name, N, K, g, k, seed = case
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    if seed % 2 == 0:   # keep every code inside the LUT; odd seeds with k < 16 keep codes past it
        codes &= np.uint8({16: 0xFF, 8: 0x77, 4: 0x33, 2: 0x11}[k])
    lut = (rng.standard_normal((N, k)) * 4).astype(np.float16).view(np.uint16)
    scale = (rng.lognormal(-6, 2, (N, K // g))).astype(np.float16).view(np.uint16)
    offset = (rng.standard_normal((N, K // g)) * 0.05).astype(np.float16).view(np.uint16)
    q = any4().Quantized(codes=_dev(codes), lut=torch.from_numpy(lut.view(np.float16)).cuda(),
                         scale=torch.from_numpy(scale.view(np.float16)).cuda(),
                         offset=torch.from_numpy(offset.view(np.float16)).cuda(), objective=None)
    say(f"dequant {name}: N={N} K={K} g={g} k={k}")
    _check_dequant(q, g, k, codes, lut, scale, offset, name)


@pytest.mark.parametrize("wl", ["q_proj_g128", "q_proj_g64", "layer_any3"])
def test_dequant_of_quantizer_output_bit_exact(wl):
    w = make(wl, rows=64)
    for m in w.matrices[:2]:
        wd, act = to_device(m)
        q = any4().quantize(wd, act, w.group, w.n_clusters, w.iters)
        codes = q.codes.cpu().numpy()
        lut = q.lut.cpu().numpy().view(np.uint16)
        scale = q.scale.cpu().numpy().view(np.uint16)
        offset = q.offset.cpu().numpy().view(np.uint16)
        _check_dequant(q, w.group, w.n_clusters, codes, lut, scale, offset, f"{wl}/{m.name}")


def test_dequant_empty_and_invalid():
    q = any4().Quantized(codes=torch.empty((0, 64), dtype=torch.uint8, device="cuda"),
                         lut=torch.empty((0, 16), dtype=torch.float16, device="cuda"),
                         scale=torch.empty((0, 1), dtype=torch.float16, device="cuda"),
                         offset=torch.empty((0, 1), dtype=torch.float16, device="cuda"),
                         objective=None)
    assert any4().dequantize(q, 128, 16).shape == (0, 128)
    q96 = any4().Quantized(codes=torch.empty((0, 96), dtype=torch.uint8, device="cuda"),
                           lut=torch.empty((0, 16), dtype=torch.float16, device="cuda"),
                           scale=torch.empty((0, 2), dtype=torch.float16, device="cuda"),
                           offset=torch.empty((0, 2), dtype=torch.float16, device="cuda"),
                           objective=None)
    with pytest.raises(any4().Any4Error):
        any4().dequantize(q96, 96, 16)          # group not a power of two (the ABI's check)
    with pytest.raises(ValueError):
        any4().dequantize(q, 64, 16)            # scale/offset extents do not match the group


# --- end to end ---------------------------------------------------------------------------

@pytest.mark.parametrize("k", [4, 16])
def test_exact_level_rows_round_trip(k):
    K, g = 1024, 128
    w = exact_level_rows(8, K, g, k, 70 + k)
    act = torch.from_numpy(np.random.default_rng(71).lognormal(0, 0.5, K).astype(np.float32)).cuda()
    q = any4().quantize(torch.from_numpy(w).cuda(), act, g, k, 10)
    rec = any4().dequantize(q, g, k, out_dtype=torch.float32).cpu().numpy()
    assert np.array_equal(rec, w)


def test_output_error_any4_below_int4_end_to_end():
    """Calibration activations -> E|x| on the GPU -> quantize -> dequantize on the GPU;
    the relative output error ||X W_hat^T - X W^T|| / ||X W^T|| (fp32 GEMMs on the GPU,
    a check, not part of the path) is below that of uniform int4 at the same group
    scaling, whose codes and scales come from the oracle."""
    rng = np.random.default_rng(91)
    K, N, g = 4096, 256, 128
    profile = draw_act(rng, K)
    x = draw_activations(rng, 2048, profile, BF16)
    xd = _dev(x)
    act = any4().act_absmean(xd)
    assert _ulp_diff(act.cpu().numpy(), oracle.act_absmean(x, BF16)).max() <= 1
    m = make_matrix("err", N, K, BF16, 92)
    wd, _ = to_device(m)
    q = any4().quantize(wd, act, g, 16, 20)
    w_any4 = any4().dequantize(q, g, 16, out_dtype=torch.float32)
    w32 = wd.float()
    from test_oracle_bookends import _int4_rtn
    codes, lut, scale, offset = _int4_rtn(w32.cpu().numpy(), g)
    qi = any4().Quantized(codes=_dev(codes), lut=torch.from_numpy(lut.view(np.float16)).cuda(),
                          scale=torch.from_numpy(scale.view(np.float16)).cuda(),
                          offset=torch.from_numpy(offset.view(np.float16)).cuda(), objective=None)
    w_int4 = any4().dequantize(qi, g, 16, out_dtype=torch.float32)
    xf = xd.float()
    y = xf @ w32.t().contiguous()

    def rel(wh):
        return float(torch.linalg.norm(xf @ wh.t().contiguous() - y) / torch.linalg.norm(y))

    e4, ei = rel(w_any4), rel(w_int4)
    say(f"  output error: any4 {e4:.4f}, int4 {ei:.4f}")
    assert e4 < ei


# --- the sizes bench.py times, on sampled outputs -------------------------------------------

def test_absmean_bench_batch_sampled_channels():
    """E|x| of the 65536-token x 4096-channel calibration batch (the launch bench.py
    times), checked on 96 sampled channels."""
    x = make_activations("calib_32x2048")
    say(f"absmean calib_32x2048: T={x.shape[0]} K={x.shape[1]}")
    got = any4().act_absmean(_dev(x)).cpu().numpy()
    cols = np.sort(np.random.default_rng(7).choice(x.shape[1], 96, replace=False))
    ref = oracle.act_absmean(np.ascontiguousarray(x[:, cols]), BF16)
    d = _ulp_diff(got[cols], ref)
    say(f"  {np.mean(d == 0):.4f} of sampled channels bit-exact, max {d.max()} ulp")
    assert d.max() <= 1


def test_dequant_full_up_proj_sampled_rows():
    """Dequantization of the whole quantized 14336 x 4096 up_proj to bf16 (the launch
    bench.py times), checked on 64 sampled rows."""
    w = make("up_proj")
    m = w.matrices[0]
    wd, act = to_device(m)
    q = any4().quantize(wd, act, w.group, w.n_clusters, w.iters)
    out = any4().dequantize(q, w.group, w.n_clusters).cpu().view(torch.int16).numpy().view(np.uint16)
    rows = np.sort(np.random.default_rng(8).choice(m.w.shape[0], 64, replace=False))
    ref = oracle.dequantize(q.codes.cpu().numpy()[rows], q.lut.cpu().numpy()[rows].view(np.uint16),
                            q.scale.cpu().numpy()[rows].view(np.uint16),
                            q.offset.cpu().numpy()[rows].view(np.uint16), w.group, w.n_clusters)
    assert np.array_equal(out[rows], oracle.bf16_bits(ref))


# --- LUT-dequantized matrix-vector products -------------------------------------------------

GEMV_TOL = 1e-5   # relative to sum_j |x_j| (|alpha L| + |beta|), the oracle's magnitude scale


def _check_gemv(q, g, k, codes, lut, scale, offset, x, dtype, name):
    got = any4().lut_gemv(q, _dev(x), g, k).cpu().numpy()
    ref, s = oracle.lut_gemv(codes, lut, scale, offset, g, k, x, dtype)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), name
    err = np.abs(got[~nan].astype(np.float64) - ref[~nan])
    bound = GEMV_TOL * s[~nan] + 1e-30
    assert np.all(err <= bound), (name, float((err / bound).max()))
    return float((err / np.maximum(s[~nan], 1e-300)).max()) if err.size else 0.0


# (name, N, K, group, k, M, x dtype, seed): one to eight tokens, one and several x slices;
# bf16 x of three or more tokens with groups of 32 or more runs on the matrix cores, the
# rest on the VALU kernel
GEMV_RANDOM = [
    ("m1_k4096_bf16", 40, 4096, 128, 16, 1, BF16, 11),
    ("m3_k512_f32", 33, 512, 64, 8, 3, F32, 12),
    ("m5_k2048_bf16_g16", 17, 2048, 16, 16, 5, BF16, 13),
    ("m8_k28672_bf16", 9, 28672, 128, 16, 8, BF16, 14),
    ("m2_k6160_f32_codes_past_lut", 21, 6160, 16, 4, 2, F32, 15),
    ("m6_k4096_bf16_g64_codes_past_lut", 19, 4096, 64, 8, 6, BF16, 16),
    ("m7_k2048_bf16_g32", 50, 2048, 32, 16, 7, BF16, 17),
]


@pytest.mark.parametrize("case", GEMV_RANDOM, ids=[c[0] for c in GEMV_RANDOM])
def test_gemv_random_fields(case):
    name, N, K, g, k, M, dtype, seed = case
    say(f"gemv {name}: N={N} K={K} M={M}")
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    codes &= np.uint8({16: 0xFF, 8: 0x77, 4: 0x33}[k])
    if "past_lut" in name:
        codes[::4, K // 3] |= np.uint8(0xC0)     # one code past the LUT on every 4th row
    lut = (rng.standard_normal((N, k)) * 4).astype(np.float16).view(np.uint16)
    scale = (rng.lognormal(-5, 1, (N, K // g))).astype(np.float16).view(np.uint16)
    offset = (rng.standard_normal((N, K // g)) * 0.05).astype(np.float16).view(np.uint16)
    x = draw_activations(rng, M, draw_act(rng, K), dtype)
    q = any4().Quantized(codes=_dev(codes), lut=torch.from_numpy(lut.view(np.float16)).cuda(),
                         scale=torch.from_numpy(scale.view(np.float16)).cuda(),
                         offset=torch.from_numpy(offset.view(np.float16)).cuda(), objective=None)
    worst = _check_gemv(q, g, k, codes, lut, scale, offset, x, dtype, name)
    say(f"  {name}: worst error {worst:.2e} of the magnitude scale")
    a = any4().lut_gemv(q, _dev(x), g, k).cpu().numpy()
    b = any4().lut_gemv(q, _dev(x), g, k).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))      # fixed summation order


@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("M", list(range(1, 9)))
def test_gemv_every_token_count(M, dtype):
    """Every instance (1, 2, 4, 8 token slots x bf16/fp32 x) on a ragged row count, and
    the smallest K (one 16-column chunk per row)."""
    rng = np.random.default_rng(300 + M + 10 * dtype)
    for N, K, g in ((37, 1536, 32), (5, 16, 16)):
        codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
        lut = (rng.standard_normal((N, 16)) * 3).astype(np.float16).view(np.uint16)
        scale = rng.lognormal(-4, 1, (N, K // g)).astype(np.float16).view(np.uint16)
        offset = (rng.standard_normal((N, K // g)) * 0.1).astype(np.float16).view(np.uint16)
        x = draw_activations(rng, M, draw_act(rng, K), dtype)
        q = any4().Quantized(codes=_dev(codes), lut=torch.from_numpy(lut.view(np.float16)).cuda(),
                             scale=torch.from_numpy(scale.view(np.float16)).cuda(),
                             offset=torch.from_numpy(offset.view(np.float16)).cuda(), objective=None)
        _check_gemv(q, g, 16, codes, lut, scale, offset, x, dtype, f"M{M}/N{N}/K{K}")


@pytest.mark.parametrize("M", [1, 8])
def test_gemv_full_up_proj_sampled_rows(M):
    """The quantized 14336 x 4096 up_proj times M calibration-like tokens (the launch
    bench.py times), checked on 128 sampled rows."""
    w = make("up_proj")
    m = w.matrices[0]
    wd, act = to_device(m)
    q = any4().quantize(wd, act, w.group, w.n_clusters, w.iters)
    x = draw_activations(np.random.default_rng(90 + M), M, m.act, BF16)
    got = any4().lut_gemv(q, _dev(x), w.group, w.n_clusters).cpu().numpy()
    rows = np.sort(np.random.default_rng(91).choice(m.w.shape[0], 128, replace=False))
    ref, s = oracle.lut_gemv(q.codes.cpu().numpy()[rows], q.lut.cpu().numpy()[rows].view(np.uint16),
                             q.scale.cpu().numpy()[rows].view(np.uint16),
                             q.offset.cpu().numpy()[rows].view(np.uint16), w.group, w.n_clusters, x, BF16)
    err = np.abs(got[:, rows].astype(np.float64) - ref)
    assert np.all(err <= GEMV_TOL * s), float((err / s).max())
    say(f"  up_proj M={M}: worst error {float((err / s).max()):.2e} of the magnitude scale")


def test_gemv_unsupported_and_invalid():
    q = any4().Quantized(codes=torch.zeros((4, 256), dtype=torch.uint8, device="cuda"),
                         lut=torch.zeros((4, 16), dtype=torch.float16, device="cuda"),
                         scale=torch.zeros((4, 4), dtype=torch.float16, device="cuda"),
                         offset=torch.zeros((4, 4), dtype=torch.float16, device="cuda"),
                         objective=None)
    assert torch.equal(any4().lut_gemv(q, torch.ones((2, 512), device="cuda")),
                       torch.zeros((2, 4), device="cuda"))
    with pytest.raises(any4().Any4Error):
        any4().lut_gemv(q, torch.ones((9, 512), device="cuda"))        # more than 8 tokens
    q8 = any4().Quantized(codes=q.codes, lut=q.lut,
                          scale=torch.zeros((4, 64), dtype=torch.float16, device="cuda"),
                          offset=torch.zeros((4, 64), dtype=torch.float16, device="cuda"),
                          objective=None)
    with pytest.raises(any4().Any4Error):
        any4().lut_gemv(q8, torch.ones((1, 512), device="cuda"), group=8)  # group below 16
    # extents the C ABI cannot see are checked by the binding
    with pytest.raises(ValueError):
        any4().lut_gemv(q, torch.ones((1, 512), device="cuda"), n_clusters=8)   # lut is [4, 16]
    with pytest.raises(ValueError):
        any4().lut_gemv(q, torch.ones((1, 256), device="cuda"))                 # x too short
    with pytest.raises(ValueError):
        any4().lut_gemv(q, torch.ones((1, 512), device="cuda"), out=torch.empty((1, 3), device="cuda"))

"""Pins for the oracle's bookends: E|x_j| and Eq. 4 dequantization.

What pins what ("any4: Learned 4-bit Numeric Representation for LLMs"):
  * E|x_j| (Section 4.1, the calibration statistic): exact rational means of small
    random batches (Python fractions) after the oracle's fp64 sum and its two
    roundings; one token gives |x| exactly; power-of-two scaling of x scales the
    result exactly; a constant channel gives its magnitude.
  * dequantization (Section 2.5.2, Eq. 4): a worked example by hand; exact
    reconstruction of rows with at most k scaled levels after the oracle quantizer
    (nibble order, group index and LUT row all have to be right for it to hold).
  * fp16 widening: numpy's float16 -> float32 over all 65536 bit patterns.
  * bf16 rounding: torch's float32 -> bfloat16 cast (round to nearest even).
  * the output error on synthetic activations: any4 beats uniform int4 with the same
    group scaling (the paper's comparison of the two formats), in fp64.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import BF16, F32, draw_act, draw_activations, make_matrix
from test_oracle_kmeans import exact_level_rows


def _bf16_to_f32(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)


# --- fp16 / bf16 conversions ---------------------------------------------------------

def test_fp16_widening_matches_numpy_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.fp16_to_f32(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 20000),
        # exact ties between two bf16 values, both parities of the kept bit
        _bf16_to_f32(rng.integers(0, 0x7F00, 2000)).view(np.uint32).__add__(0x8000).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3e38, -3.4e38, 1e-40, -1e-45], np.float32),
    ]).astype(np.float32)
    got = oracle.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    assert oracle.bf16_bits(np.array([np.nan], np.float32))[0] & 0x7FC0 == 0x7FC0


# --- E|x_j| ------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [F32, BF16])
def test_absmean_exact_rational_mean(dtype):
    rng = np.random.default_rng(11 + dtype)
    for T in (1, 2, 3, 7, 19):
        K = 5
        x32 = (rng.standard_normal((T, K)) * 3.0).astype(np.float32)
        x = x32 if dtype == F32 else oracle.bf16_bits(x32)
        vals = x32 if dtype == F32 else _bf16_to_f32(x)
        got = oracle.act_absmean(x, dtype)
        for j in range(K):
            exact = sum(Fraction(abs(float(v))) for v in vals[:, j])
            # the fp64 running sum is exact for these few values...
            assert Fraction(float(np.sum(np.abs(vals[:, j]).astype(np.float64)))) == exact
            # ...so the oracle is the fp32 rounding of the correctly rounded fp64 mean
            want = np.float32(float(exact / T))
            assert got[j] == want, (T, j, got[j], want)


def test_absmean_one_token_is_magnitude():
    x = np.array([[-1.5, 0.0, -0.0, 3.25e-5, -7e30]], np.float32)
    assert np.array_equal(oracle.act_absmean(x, F32), np.abs(x[0]))


def test_absmean_power_of_two_scaling_is_exact():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 33)) * 0.1).astype(np.float32)
    base = oracle.act_absmean(x, F32)
    for s in (-6, 5):
        got = oracle.act_absmean((x * np.float32(2.0 ** s)).astype(np.float32), F32)
        assert np.array_equal(got, (base * np.float32(2.0 ** s)).astype(np.float32))


def test_absmean_constant_and_sign_alternating_channels():
    T = 37
    x = np.zeros((T, 3), np.float32)
    x[:, 0] = -0.3
    x[:, 1] = np.where(np.arange(T) % 2 == 0, 2.5, -2.5)
    x[:, 2] = 0.0
    got = oracle.act_absmean(x, F32)
    assert got[1] == np.float32(2.5) and got[2] == 0.0
    # 37 copies of fp32(0.3) summed in fp64 and divided by 37 round back to fp32(0.3)
    assert got[0] == np.float32(0.3)


def test_absmean_is_per_channel_not_per_token():
    x = np.array([[1.0, 100.0], [3.0, 300.0]], np.float32)
    assert np.array_equal(oracle.act_absmean(x, F32), np.array([2.0, 200.0], np.float32))


def test_absmean_rejects_empty():
    with pytest.raises(ValueError):
        oracle.act_absmean(np.zeros((0, 4), np.float32), F32)


# --- dequantization --------------------------------------------------------------------

def test_dequant_worked_example():
    """Eq. 4 by hand.  One row, K = 4, group 2, a 4-entry LUT:
    LUT = [0, 1, 2.5, 15]           fp16 bits 0x0000 0x3C00 0x4100 0x4B80
    group 0: alpha = 0.5, beta = -1.25  (0x3800, 0xBD00)
    group 1: alpha = 2,   beta = 3      (0x4000, 0x4200)
    codes q = [3, 1, 2, 0] -> bytes [0x13, 0x02] (even column in the low nibble)
    w_hat = [0.5*15 - 1.25, 0.5*1 - 1.25, 2*2.5 + 3, 2*0 + 3] = [6.25, -0.75, 8, 3]."""
    codes = np.array([[0x13, 0x02]], np.uint8)
    lut = np.array([[0x0000, 0x3C00, 0x4100, 0x4B80]], np.uint16)
    scale = np.array([[0x3800, 0x4000]], np.uint16)
    offset = np.array([[0xBD00, 0x4200]], np.uint16)
    got = oracle.dequantize(codes, lut, scale, offset, group=2, n_clusters=4)
    assert np.array_equal(got, np.array([[6.25, -0.75, 8.0, 3.0]], np.float32))


@pytest.mark.parametrize("k,g", [(16, 64), (8, 128), (4, 32)])
def test_dequant_reconstructs_exact_level_rows(k, g):
    K = 512
    w = exact_level_rows(5, K, g, k, 40 + k)
    act = np.random.default_rng(41).lognormal(0, 0.5, K).astype(np.float32)
    out = oracle.quantize(w, F32, act, g, k, iters=8)
    assert out["status"] == 0 and np.all(out["objective"] == 0.0)
    rec = oracle.dequantize(out["codes"], out["lut"], out["scale"], out["offset"], g, k)
    assert np.array_equal(rec, w)


def test_dequant_code_outside_lut_is_nan():
    codes = np.array([[0x50]], np.uint8)            # q = [0, 5] with a 4-entry LUT
    lut = np.array([[0x3C00, 0x4000, 0x4200, 0x4400]], np.uint16)
    one = np.array([[0x3C00]], np.uint16)
    zero = np.array([[0x0000]], np.uint16)
    got = oracle.dequantize(codes, lut, one, zero, group=2, n_clusters=4)
    assert got[0, 0] == 1.0 and np.isnan(got[0, 1])


def _int4_rtn(w32, group):
    """Uniform int4 with the same group scaling: codes = nearest integer level of the
    oracle's scaled values, LUT = the levels 0..15 (Section 2.5.2, round to nearest)."""
    N, K = w32.shape
    codes = np.zeros((N, K // 2), np.uint8)
    scale = np.zeros((N, K // group), np.uint16)
    offset = np.zeros((N, K // group), np.uint16)
    for i in range(N):
        ws, al, be, bad = oracle.scale_row(w32[i], group, 16)
        assert not bad
        q = np.clip(np.floor(ws.astype(np.float64) + 0.5), 0, 15).astype(np.uint8)
        codes[i] = oracle.pack_row(q)
        scale[i] = oracle.fp16_bits(al)
        offset[i] = oracle.fp16_bits(be)
    lut = np.tile(oracle.fp16_bits(np.arange(16, dtype=np.float32)), (N, 1))
    return codes, lut, scale, offset


def test_any4_output_error_below_int4_on_synthetic_activations():
    """The paper compares any4 against int4 at the same group size; on the heavy-tailed
    synthetic weights with outlier activation channels the learned LUT gives the lower
    relative output error ||X W_hat^T - X W^T|| / ||X W^T|| (fp64 products)."""
    m = make_matrix("err", 48, 512, F32, 55)
    g = 128
    out = oracle.quantize(m.w, F32, m.act, g, 16, iters=20)
    w_any4 = oracle.dequantize(out["codes"], out["lut"], out["scale"], out["offset"], g, 16)
    w_int4 = oracle.dequantize(*_int4_rtn(m.w, g), g, 16)
    x = draw_activations(np.random.default_rng(56), 256, m.act, F32).astype(np.float64)
    y = x @ m.w.astype(np.float64).T

    def rel(wh):
        return np.linalg.norm(x @ wh.astype(np.float64).T - y) / np.linalg.norm(y)

    e4, ei = rel(w_any4), rel(w_int4)
    assert e4 < ei, (e4, ei)
    assert e4 < 0.2


# --- LUT-dequantized matrix-vector products ----------------------------------------------

def test_gemv_worked_example():
    """The Eq. 4 example above (w_hat = [6.25, -0.75, 8, 3]) times x = [1, 2, -1, 0.5]:
    6.25 - 1.5 - 8 + 1.5 = -1.75; a second token [0, 0, 0.25, 4] gives 2 + 12 = 14."""
    codes = np.array([[0x13, 0x02]], np.uint8)
    lut = np.array([[0x0000, 0x3C00, 0x4100, 0x4B80]], np.uint16)
    scale = np.array([[0x3800, 0x4000]], np.uint16)
    offset = np.array([[0xBD00, 0x4200]], np.uint16)
    x = np.array([[1, 2, -1, 0.5], [0, 0, 0.25, 4]], np.float32)
    y, s = oracle.lut_gemv(codes, lut, scale, offset, 2, 4, x, F32)
    assert np.array_equal(y, np.array([[-1.75], [14.0]], np.float32))
    # magnitude scale: sum |x| (|alpha L| + |beta|) = 1*8.75 + 2*1.75 + 1*8 + 0.5*3
    assert s[0, 0] == 8.75 + 3.5 + 8 + 1.5


def test_gemv_matches_dequantize_times_x():
    m = make_matrix("gemv", 20, 512, BF16, 71)
    out = oracle.quantize(m.w, BF16, m.act, 128, 16, 6)
    w_hat = oracle.dequantize(out["codes"], out["lut"], out["scale"], out["offset"], 128, 16)
    x = draw_activations(np.random.default_rng(72), 3, m.act, BF16)
    y, _ = oracle.lut_gemv(out["codes"], out["lut"], out["scale"], out["offset"], 128, 16, x, BF16)
    ref = _bf16_to_f32(x).astype(np.float64) @ w_hat.astype(np.float64).T   # numpy fp64 product
    assert np.allclose(y, ref, rtol=1e-6, atol=1e-30)
    assert y.shape == (3, 20)


def test_gemv_is_linear_in_x():
    m = make_matrix("lin", 6, 256, F32, 73)
    out = oracle.quantize(m.w, F32, m.act, 64, 8, 4)
    rng = np.random.default_rng(74)
    x1 = (rng.integers(-8, 8, (2, 256)) * 0.25).astype(np.float32)   # sums stay exact
    x2 = (rng.integers(-8, 8, (2, 256)) * 0.5).astype(np.float32)
    args = (out["codes"], out["lut"], out["scale"], out["offset"], 64, 8)
    y1, _ = oracle.lut_gemv(*args, x1, F32)
    y2, _ = oracle.lut_gemv(*args, x2, F32)
    y12, _ = oracle.lut_gemv(*args, x1 + x2, F32)
    assert np.allclose(y12, y1 + y2, rtol=1e-6, atol=1e-6)

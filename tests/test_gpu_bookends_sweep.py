"""Randomized parity sweep of the bookend kernels against the oracle on seeded random
shapes: E|x| (any T and K, bf16/fp32; within one fp32 ulp), Eq. 4 dequantization (groups
2..256, 2..16 clusters, fp32/bf16 out; bit-exact, vector and scalar paths) and the LUT
matrix-vector product (1..8 tokens, K and group multiples of 16, bf16/fp32 x; within 1e-5
of the magnitude scale).
"""
import numpy as np
import pytest

import oracle
from parity_util import say
from workloads import BF16, F32, draw_act, draw_activations

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

BASE_SEED = 8000


def any4():
    import weight_only_bit_row_amd as mod
    return mod


def _dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def _fields(rng, N, K, g, k):
    codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    if rng.random() < 0.8:   # mostly codes inside the LUT; otherwise some NaN outputs
        codes &= np.uint8({2: 0x11, 4: 0x33, 8: 0x77, 16: 0xFF}[k])
    lut = (rng.standard_normal((N, k)) * 4).astype(np.float16).view(np.uint16)
    scale = rng.lognormal(-5, 1.5, (N, K // g)).astype(np.float16).view(np.uint16)
    offset = (rng.standard_normal((N, K // g)) * 0.05).astype(np.float16).view(np.uint16)
    q = any4().Quantized(codes=_dev(codes), lut=torch.from_numpy(lut.view(np.float16)).cuda(),
                         scale=torch.from_numpy(scale.view(np.float16)).cuda(),
                         offset=torch.from_numpy(offset.view(np.float16)).cuda(), objective=None)
    return q, codes, lut, scale, offset


def test_absmean_random_shapes():
    rng = np.random.default_rng(BASE_SEED)
    for i in range(60):
        T, K = int(rng.integers(1, 3000)), int(rng.integers(1, 5000))
        dtype = int(rng.choice([F32, BF16]))
        x = draw_activations(rng, T, draw_act(rng, K), dtype)
        got = any4().act_absmean(_dev(x)).cpu().numpy()
        ref = oracle.act_absmean(x, dtype)
        d = np.abs(got.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
        assert d.max() <= 1, (i, T, K, dtype, int(d.max()))


def test_dequantize_random_shapes():
    rng = np.random.default_rng(BASE_SEED + 1)
    for i in range(80):
        g = int(rng.choice([2, 4, 8, 16, 32, 64, 128, 256]))
        K = g * int(rng.integers(1, max(2, 4096 // g) + 1))
        K += K % 2
        if K % g:
            g = 2
        N, k = int(rng.integers(1, 40)), int(rng.choice([2, 4, 8, 16]))
        q, codes, lut, scale, offset = _fields(rng, N, K, g, k)
        ref = oracle.dequantize(codes, lut, scale, offset, g, k)
        f32 = any4().dequantize(q, g, k, out_dtype=torch.float32).cpu().numpy()
        assert np.array_equal(f32.view(np.uint32), ref.view(np.uint32)), (i, N, K, g, k)
        b16 = any4().dequantize(q, g, k).cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(b16, oracle.bf16_bits(ref)), (i, N, K, g, k)


def test_lut_gemv_random_shapes():
    rng = np.random.default_rng(BASE_SEED + 2)
    worst = 0.0
    for i in range(80):
        g = int(rng.choice([16, 32, 64, 128, 256]))
        K = g * int(rng.integers(1, max(2, 20000 // g) + 1))
        N, k, M = int(rng.integers(1, 70)), int(rng.choice([2, 4, 8, 16])), int(rng.integers(1, 9))
        dtype = int(rng.choice([F32, BF16]))
        q, codes, lut, scale, offset = _fields(rng, N, K, g, k)
        x = draw_activations(rng, M, draw_act(rng, K), dtype)
        got = any4().lut_gemv(q, _dev(x), g, k).cpu().numpy()
        ref, s = oracle.lut_gemv(codes, lut, scale, offset, g, k, x, dtype)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan), (i, N, K, g, k, M)
        err = np.abs(got[~nan].astype(np.float64) - ref[~nan])
        assert np.all(err <= 1e-5 * s[~nan] + 1e-30), (i, N, K, g, k, M)
        if err.size:
            worst = max(worst, float((err / np.maximum(s[~nan], 1e-300)).max()))
    say(f"LUT product sweep: worst error {worst:.2e} of the magnitude scale")

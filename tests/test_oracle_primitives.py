"""Pins for the oracle's primitives: Philox, fp16 emission, nibble packing, output sizes.

Each check ties the oracle to something outside itself: numpy's Philox4x64-10 stream
and float16 casts, the storage cost printed in the any4 paper (Section 2.4.1), and
the int4 range printed in Section 2.5.1.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --- Philox ------------------------------------------------------------------------

@pytest.mark.parametrize("key", [(0, 0), (1, 2), (0xDEADBEEFCAFEBABE, 0x0123456789ABCDEF)])
def test_philox4x64_matches_numpy(key):
    """numpy.random.Philox is Philox4x64-10; it increments its counter before each block.
    The oracle's 32-bit and 64-bit variants share one round macro, so this pins the
    round structure (products, xor with key, word order, key schedule)."""
    bg = np.random.Philox(key=np.array(key, np.uint64), counter=np.array([5, 0, 0, 0], np.uint64))
    raw = bg.random_raw(12)
    for blk in range(3):
        ours = oracle.philox4x64_10([6 + blk, 0, 0, 0], key)
        assert [int(x) for x in ours] == [int(x) for x in raw[4 * blk:4 * blk + 4]]


def test_philox4x64_counter_words_matter():
    """Every counter word and key word changes the block (catches a dropped word)."""
    base = oracle.philox4x64_10([1, 2, 3, 4], [5, 6])
    for i in range(4):
        c = [1, 2, 3, 4]
        c[i] += 1
        assert not np.array_equal(oracle.philox4x64_10(c, [5, 6]), base)
    for i in range(2):
        k = [5, 6]
        k[i] += 1
        assert not np.array_equal(oracle.philox4x64_10([1, 2, 3, 4], k), base)
    # numpy agrees for a counter with high words set
    bg = np.random.Philox(key=np.array([5, 6], np.uint64),
                         counter=np.array([2**64 - 1, 7, 0, 9], np.uint64))
    raw = bg.random_raw(4)  # counter wraps word 0 and carries into word 1
    ours = oracle.philox4x64_10([0, 8, 0, 9], [5, 6])
    assert [int(x) for x in ours] == [int(x) for x in raw]


def test_philox4x32_uniform_and_counter_sensitive():
    """Uniformity of the 64-bit draws the seeding uses, and every word of counter/key
    matters (the absolute stream is pinned against rocRAND in
    test_oracle_philox_rocrand.py)."""
    n = 20000
    u = np.array([oracle.philox4x32_10([i, 3, 1, 0], [7, 0])[0] for i in range(n)], np.float64)
    hist, _ = np.histogram(u / 2.0**32, bins=20, range=(0, 1))
    chi2 = ((hist - n / 20) ** 2 / (n / 20)).sum()
    assert chi2 < 45.0  # 19 dof, p ~ 1e-3
    bits = np.unpackbits(np.array([oracle.philox4x32_10([i, 0, 0, 0], [0, 0]) for i in range(2000)],
                                  np.uint32).view(np.uint8))
    assert abs(bits.mean() - 0.5) < 0.01
    base = oracle.philox4x32_10([1, 2, 3, 4], [5, 6])
    for i in range(4):
        c = [1, 2, 3, 4]
        c[i] += 1
        assert not np.array_equal(oracle.philox4x32_10(c, [5, 6]), base)
    for i in range(2):
        k = [5, 6]
        k[i] += 1
        assert not np.array_equal(oracle.philox4x32_10([1, 2, 3, 4], k), base)


# --- fp16 emission ---------------------------------------------------------------------

def test_fp16_rne_matches_numpy():
    rng = np.random.default_rng(0)
    parts = [
        rng.uniform(0, 15, 100000),                          # LUT values live in [0, Qr]
        rng.standard_normal(100000) * 0.05,                  # alpha, beta magnitudes
        rng.standard_normal(20000) * 1e-5,                   # fp16 subnormal range
        rng.standard_normal(20000) * 1e-8,                   # underflow to zero
        rng.standard_normal(20000) * 3e4,                    # near overflow
        np.array([65504, 65519.99, 65520, 70000, -65520, 0.0, -0.0, np.inf, -np.inf,
                  2.0**-24, 2.0**-25, 1.5 * 2.0**-25, 2.0**-14, 2.0**-14 - 2.0**-25]),
    ]
    x = np.concatenate(parts).astype(np.float32)
    # exact ties: fp32 values halfway between fp16 neighbours
    base = rng.integers(0, 0x7BFF, 20000).astype(np.uint16).view(np.float16).astype(np.float32)
    step = np.abs(base) * 2.0**-11
    x = np.concatenate([x, (base + step).astype(np.float32)])
    ours = oracle.fp16_bits(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_fp16_nan_stays_nan():
    out = oracle.fp16_bits(np.array([np.nan], np.float32))
    assert np.isnan(out.view(np.float16)[0])


# --- packing and sizes -----------------------------------------------------------------

def test_pack_low_nibble_first():
    rng = np.random.default_rng(1)
    q = rng.integers(0, 16, 4096).astype(np.uint8)
    packed = oracle.pack_row(q)
    assert np.array_equal(packed & 0xF, q[0::2])
    assert np.array_equal(packed >> 4, q[1::2])


def test_storage_cost_matches_paper():
    """Output byte counts give the bits/entry the paper prints for K=4096, g=128."""
    gold = json.load(open(os.path.join(GOLDEN, "storage_cost.json")))
    for case in gold["cases"]:
        K, g, k = case["n_cols"], case["group"], case["n_clusters"]
        N = 8
        w = np.random.default_rng(2).standard_normal((N, K)).astype(np.float32) * 0.02
        act = np.ones(K, np.float32)
        out = oracle.quantize(w, 0, act, g, k, iters=1)
        lut_bits = out["lut"].nbytes * 8 / (N * K)
        grp_bits = (out["scale"].nbytes + out["offset"].nbytes) * 8 / (N * K)
        code_bits = out["codes"].nbytes * 8 / (N * K)
        assert lut_bits == case["lut_bits_per_entry"]
        assert grp_bits == case["group_bits_per_entry"]
        assert code_bits + lut_bits + grp_bits == case["total_bits_per_entry"]
        assert code_bits + grp_bits == gold["int4_grouped_bits_per_entry"]


def test_scaled_range_is_int4_span():
    """Qmax - Qmin for 4 bits is the int4 span the paper prints (-7..+8): the scaled
    row spans [0, 15] exactly at a group's extremes."""
    gold = json.load(open(os.path.join(GOLDEN, "int4_range.json")))
    span = gold["q_max"] - gold["q_min"]
    w = np.array([-0.5, 0.125, 0.4375, -0.1875] * 2, np.float32)  # range 0.9375 = 15/16
    ws, al, be, bad = oracle.scale_row(w, 4, 1 << gold["bits"])
    assert not bad
    assert ws.min() == 0.0 and ws.max() == float(span)

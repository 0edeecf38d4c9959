"""Host check of the integer conversion the row kernel uses for its fixed-point Eq. 23
sums (rows of 2-16 waves): a term t with |t| < 2^51 plus 1.5 * 2^52 lands in
[2^52, 2^53), where doubles are spaced by 1, so the addition rounds t to the nearest
integer (ties to even); the bit pattern of the sum minus that of 1.5 * 2^52 is that
integer in two's complement, and the subtraction only touches the high 32 bits.  Also
checks the scale bound: with a * 2^sigma < 2^43 and |w_S| < 16, 2^15 terms of either sum
stay below 2^62."""
import numpy as np

BIAS = 6755399441055744.0  # 1.5 * 2^52
BIAS_BITS = 0x4338000000000000


def to_int(t):
    s = np.asarray(t, np.float64) + BIAS  # one IEEE addition, as the fused add with u*v exact
    bits = s.view(np.uint64)
    hi = (bits >> np.uint64(32)).astype(np.uint32) - np.uint32(BIAS_BITS >> 32)
    lo = (bits & np.uint64(0xFFFFFFFF)).astype(np.uint32)
    return ((hi.astype(np.uint64) << np.uint64(32)) | lo.astype(np.uint64)).view(np.int64)


def test_nearest_integer_both_signs():
    rng = np.random.default_rng(5)
    for scale in (1.0, 2.0 ** 20, 2.0 ** 40, 2.0 ** 50):
        t = rng.uniform(-scale, scale, 20000)
        assert np.array_equal(to_int(t), np.rint(t).astype(np.int64))


def test_ties_go_to_even_and_edges():
    t = np.array([0.5, 1.5, 2.5, -0.5, -1.5, 0.0, -0.0, 2.0 ** 51 - 1, -(2.0 ** 51) + 1, 3.25, -3.75])
    assert np.array_equal(to_int(t), np.rint(t).astype(np.int64))


def test_products_of_fp32_weights_and_scaled_values():
    # the kernel's terms: round(4 a) and round(a w) with a = fp32 sample weight * 2^sigma
    # (< 2^43) and w = fp32 scaled weight; a * w is exact in fp64 (48 significant bits)
    rng = np.random.default_rng(6)
    a = (rng.lognormal(0, 2, 50000) * 2.0 ** 30).astype(np.float32)
    a = np.minimum(a, np.float32(2.0 ** 43 * (1 - 2 ** -24)))
    w = rng.uniform(-8, 15.9, 50000).astype(np.float32)
    prod = a.astype(np.float64) * w.astype(np.float64)
    exact = [int(round(x)) for x in prod]  # Python ints: no overflow or rounding in the check
    got = to_int(prod)
    # round-half-even of an exact product equals Python's round() on the same double
    assert all(int(g) == e for g, e in zip(got, exact))
    assert np.array_equal(to_int(4.0 * a.astype(np.float64)), np.rint(4.0 * a.astype(np.float64)).astype(np.int64))
    # bounds: 2^15 terms below 2^47 (S1) and 2^45 (S0) stay below 2^62
    assert (2 ** 15) * (2 ** 47) <= 2 ** 62
    assert np.all(np.abs(prod) < 2.0 ** 47) and np.all(4.0 * a.astype(np.float64) < 2.0 ** 45)


def test_wraparound_differences_are_exact():
    # bins accumulate mod 2^64 over the rounds; a round's sum is the difference of the
    # totals, read as a signed 64-bit integer
    rng = np.random.default_rng(7)
    terms = rng.integers(-(2 ** 46), 2 ** 46, size=(30, 2 ** 10), dtype=np.int64)
    mask = 2 ** 64 - 1
    total = 0
    for r in range(terms.shape[0]):
        prev = total
        for t in terms[r]:
            total = (total + (int(t) & mask)) & mask
        d = (total - prev) & mask
        diff = d - 2 ** 64 if d >= 2 ** 63 else d
        assert diff == int(terms[r].sum())

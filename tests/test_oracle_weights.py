"""Pins for the oracle's Eq. 23 sample weights a_j = alpha_{g(j)} * E|x_j| ("any4:
Learned 4-bit Numeric Representation for LLMs", Section 4.1, Eq. 23; the group of
column j is the t with t*g <= j < (t+1)*g, Section 2.5.1).

The other weighting pins give every group the same alpha or pass a directly, so they
cannot see which group's alpha multiplies a column.  These can:
  * a hand-worked example: three groups with distinct power-of-two alphas and chosen
    E|x| values; every product is exact, so every a_j is known bit for bit;
  * permuting whole groups (of W, hence of alpha, and of E|x|) permutes a_j the same way;
  * through the scaling step: rows built so that each group's alpha is a distinct power
    of two give a_j = 2^s_t * E|x_j| exactly, per group;
  * end to end: a constant first group has alpha = 0, so its columns carry no weight and
    k-means++ never draws them, however large their E|x| is.
"""
import numpy as np

import oracle


def test_hand_worked_example_bit_exact():
    # K = 12, g = 4: columns 0-3 are group 0, 4-7 group 1, 8-11 group 2
    alpha = np.array([0.5, 4.0, 0.125], np.float32)
    act = np.array([1.0, 3.0, 0.25, 5.0,
                    2.0, 1.5, 0.5, 7.0,
                    4.0, 8.0, 0.75, 6.0], np.float32)
    expect = np.array([0.5, 1.5, 0.125, 2.5,
                       8.0, 6.0, 2.0, 28.0,
                       0.5, 1.0, 0.09375, 0.75], np.float32)
    a, bad = oracle.weights_row(alpha, act, 4)
    assert not bad
    assert np.array_equal(a.view(np.uint32), expect.view(np.uint32))


def test_group_permutation_permutes_weights():
    rng = np.random.default_rng(5)
    G, g = 6, 8
    alpha = (2.0 ** rng.integers(-6, 6, G)).astype(np.float32)   # distinct scales per group
    act = rng.lognormal(0, 0.5, G * g).astype(np.float32)
    a, _ = oracle.weights_row(alpha, act, g)
    for perm in (np.roll(np.arange(G), 1), rng.permutation(G), np.arange(G)[::-1]):
        act_p = act.reshape(G, g)[perm].reshape(-1)
        a_p, _ = oracle.weights_row(alpha[perm], act_p, g)
        assert np.array_equal(a_p.view(np.uint32), a.reshape(G, g)[perm].reshape(-1).view(np.uint32))
    # a column's weight follows its own group's alpha, not a neighbour's
    for t in range(G):
        cols = slice(t * g, (t + 1) * g)
        assert np.array_equal(a[cols], (alpha[t] * act[cols]).astype(np.float32))


def test_scaled_rows_with_power_of_two_alphas():
    """Group t spans [0, 15 * 2^s_t] (min 0, max 15 * 2^s_t), so Eq. 2 gives
    alpha_t = 2^s_t exactly and a_j = 2^s_t * E|x_j| exactly."""
    k, g = 16, 16
    shifts = np.array([-3, 2, 0, -7, 5, 1], int)
    rng = np.random.default_rng(6)
    w = np.empty(shifts.size * g, np.float32)
    for t, s in enumerate(shifts):
        lv = rng.integers(0, k, g).astype(np.float32)
        lv[0], lv[1] = 0.0, k - 1.0
        w[t * g:(t + 1) * g] = lv * np.float32(2.0 ** s)
    act = rng.lognormal(0, 0.5, w.size).astype(np.float32)
    ws, a, al, be, bad = oracle.prepare_row(w, 0, act, g, k)
    assert not bad
    assert np.array_equal(al, (2.0 ** shifts).astype(np.float32))
    assert np.array_equal(a, (np.repeat(2.0 ** shifts, g) * act).astype(np.float32))


def test_zero_alpha_group_is_never_drawn():
    """Group 0 is constant (alpha = 0): its a_j are 0 even though its E|x| is 1e6 times
    the rest, so no k-means++ draw of any row, key or restart lands there."""
    k, g, K = 16, 64, 256
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((8, K)) * 0.02).astype(np.float32)
    w[:, :g] = 0.125
    act = np.full(K, 1e-3, np.float32)
    act[:g] = 1e3
    for seed in range(4):
        out = oracle.quantize(w, 0, act, g, k, 0, seed=seed)
        assert out["status"] == 0
        picks = out["picks"]
        assert (picks >= g).all(), picks

"""Pin the oracle's Philox4x32-10 against rocRAND's engine.

The k-means++ draws (DESIGN reading R6) take one Philox4x32-10 block per (row, draw)
(Salmon, Moraes, Dror and Shaw, SC'11).  rocRAND ships its own implementation of that
generator as a host-callable header; `philox_ref/rocrand_philox_ref.cpp` exposes its
blocks for a given counter and key.  Agreement on random and extreme counters and keys
pins the oracle's round multipliers, Weyl constants, word order and key schedule.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(__file__)
SRC = os.path.join(HERE, "philox_ref", "rocrand_philox_ref.cpp")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
HEADER = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"


@pytest.fixture(scope="module")
def reference(tmp_path_factory):
    if not (os.path.exists(HIPCC) and os.path.exists(HEADER)):
        pytest.skip("hipcc or the rocRAND headers are not installed")
    exe = str(tmp_path_factory.mktemp("philox") / "philox_ref")
    subprocess.run([HIPCC, "-O1", "-std=c++17", "--offload-host-only", "-o", exe, SRC],
                   check=True, capture_output=True, timeout=300)

    def run(rows):
        text = "".join(" ".join(str(int(v)) for v in r) + "\n" for r in rows)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True, timeout=120)
        return np.array([[int(w) for w in line.split()] for line in out.stdout.splitlines()], np.uint64)
    return run


def _cases():
    rng = np.random.default_rng(20240707)
    m32 = 2**32 - 1
    rows = []
    # random counters and keys (word 1 below 2^30: the engine reaches it through an offset)
    for _ in range(3000):
        c = rng.integers(0, 2**32, 4, dtype=np.uint64)
        c[1] %= 2**30
        k = rng.integers(0, 2**32, 2, dtype=np.uint64)
        rows.append([*c, *k])
    # extremes of every word
    for c0 in (0, 1, m32):
        for c2 in (0, m32):
            for c3 in (0, m32):
                for k in ((0, 0), (m32, m32), (0, m32), (m32, 0)):
                    rows.append([c0, 2**30 - 1 if c0 == m32 else 0, c2, c3, *k])
    # the seeding's own layout: (lo32 row, draw + 16 restart, matrix index, hi32 row), key = seed
    for row in (0, 1, 14335, 2**32 + 5):
        for t in (0, 15, 16 + 3):
            for mat in (0, 6):
                for seed in (0, 0x0123456789ABCDEF):
                    rows.append([row & m32, t, mat, row >> 32, seed & m32, seed >> 32])
    return rows


def test_philox4x32_matches_rocrand(reference):
    rows = _cases()
    ref = reference(rows)
    assert ref.shape == (len(rows), 4)
    ours = np.array([oracle.philox4x32_10(r[:4], r[4:]) for r in rows], np.uint64)
    bad = np.nonzero((ours != ref).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} blocks differ, first at {rows[bad[0]]}"


def test_reference_tracks_every_word(reference):
    """The comparison would see a dropped counter or key word: the reference itself
    changes with each of them."""
    base = [1, 2, 3, 4, 5, 6]
    rows = [base]
    for i in range(6):
        r = list(base)
        r[i] += 1
        rows.append(r)
    ref = reference(rows)
    for i in range(1, 7):
        assert not np.array_equal(ref[i], ref[0])

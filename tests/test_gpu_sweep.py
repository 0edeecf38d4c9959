"""Randomized end-to-end parity sweep: the GPU path against the oracle on seeded random
configurations (row count, row length up to 32768, group 2..256, 2..16 clusters, fp32 and
bf16, 0..20 Lloyd rounds, every sample-weight / initialization / scaling variant, restarts),
each judged like T4: both report a good status, the matrix objective agrees within 1e-4,
the picks are identical, every row has identical codes (with centroids and LUT within
tolerance) or a first divergence that is an excused near-tie or an in-tolerance M-step
rounding (with restarts: identical rows only); scale and offset are bit-exact.
"""
import json

import numpy as np
import pytest

import oracle
from parity_util import OBJECTIVE_REL, check_rows, say, to_device
from workloads import BF16, F32, make_matrix

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

N_CASES = 300
BASE_SEED = 7000


def any4():
    import weight_only_bit_row_amd as mod
    return mod


def _cases():
    rng = np.random.default_rng(BASE_SEED)
    out = []
    for i in range(N_CASES):
        g = int(rng.choice([2, 4, 8, 16, 32, 64, 128, 256]))
        K = g * int(rng.integers(1, max(2, 8192 // g) + 1))
        if K % 2:
            K *= 2
        if rng.random() < 0.05:
            K = int(rng.choice([16384, 32768]))
        if K % g:
            g = 128
        variant = int(rng.integers(0, 3)) | (int(rng.integers(0, 4)) << 2) | (int(rng.random() < 0.3) << 4)
        if rng.random() < 0.15:
            variant |= int(rng.integers(1, 3)) << 8
        out.append(dict(i=i, N=int(rng.integers(1, 13)), K=K, g=g, k=int(rng.choice([2, 4, 8, 16])),
                        dtype=int(rng.choice([F32, BF16])), iters=int(rng.choice([0, 1, 5, 20])),
                        variant=variant, seed=int(rng.integers(0, 2 ** 31))))
    return out


def test_random_configurations_match_the_oracle():
    failures = []
    for c in _cases():
        m = make_matrix(f"sweep{c['i']}", c["N"], c["K"], c["dtype"], BASE_SEED + c["i"])
        w, act = to_device(m)
        out, c_final, picks, ws = any4().stage_full(w, act, c["g"], c["k"], c["iters"], seed=c["seed"],
                                                    variant=c["variant"])
        status = any4().read_status(ws)
        ref = oracle.quantize(m.w, m.dtype, m.act, c["g"], c["k"], c["iters"], seed=c["seed"],
                              variant=c["variant"])
        problems = []
        if status != 0 or ref["status"] != 0:
            problems.append(f"status {status}/{ref['status']}")
        J, Jr = out.objective.cpu().numpy().sum(), ref["objective"].sum()
        if not abs(J - Jr) <= OBJECTIVE_REL * max(Jr, 1e-30):
            problems.append(f"objective {J} vs {Jr}")
        if not np.array_equal(picks.cpu().numpy(), ref["picks"]):
            problems.append("picks")
        try:
            check_rows(any4(), m, c["g"], c["k"], c["iters"], c["seed"], out.codes.cpu().numpy(),
                       c_final.cpu().numpy(), out.lut.cpu().numpy().view(np.uint16), ref,
                       np.arange(c["N"]), variant=c["variant"])
        except AssertionError as e:
            problems.append(f"rows: {e}")
        if not np.array_equal(out.scale.cpu().numpy().view(np.uint16), ref["scale"]):
            problems.append("scale")
        if not np.array_equal(out.offset.cpu().numpy().view(np.uint16), ref["offset"]):
            problems.append("offset")
        if problems:
            failures.append((json.dumps(c), problems))
            say("FAIL", json.dumps(c), problems)
    say(f"sweep: {N_CASES} configurations, {len(failures)} failures")
    assert not failures, failures[:5]

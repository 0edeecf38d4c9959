"""Shared helpers for the GPU-vs-oracle parity tests (imported by tests only)."""
import sys

import numpy as np

# Tolerances (stated once, used by every parity test):
#   assignments: bit-exact, except where the two competing centroids' distances
#     |w_S - c| (fp64 from the fp32 operands) differ by less than 1e-6 relative
NEAR_TIE_REL = 1e-6
#   centroids after an M-step: |dc| <= 1e-5 * |c|, or at most one fp32 ulp of the top
#     of the scaled range (2^-20, the spacing of floats in [8, 16)) for centroids near 0
CENTROID_REL = 1e-5
CENTROID_ABS_FLOOR = 2.0 ** -20
#   final weighted objective of a matrix (fp64 sum over rows): 1e-4 relative
OBJECTIVE_REL = 1e-4


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def to_device(m, dev="cuda"):
    import torch
    if m.dtype == 1:
        w = torch.from_numpy(np.ascontiguousarray(m.w).view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        w = torch.from_numpy(np.ascontiguousarray(m.w)).to(dev)
    act = torch.from_numpy(np.ascontiguousarray(m.act)).to(dev)
    return w, act


def widen(w_row, dtype):
    if dtype == 1:
        return (np.asarray(w_row, np.uint16).astype(np.uint32) << 16).view(np.float32)
    return np.asarray(w_row, np.float32)


def excused_mismatch(ws, c_ref, q_ref, q_gpu):
    """Indices where assignments differ, and whether each difference is a near-tie."""
    diff = np.nonzero(q_ref != q_gpu)[0]
    if diff.size == 0:
        return diff, np.zeros(0, bool)
    x = ws[diff].astype(np.float64)
    da = np.abs(x - c_ref[q_ref[diff]].astype(np.float64))
    db = np.abs(x - c_ref[q_gpu[diff]].astype(np.float64))
    ok = np.abs(da - db) < NEAR_TIE_REL * np.maximum(da, db)
    return diff, ok


def centroid_close(c_gpu, c_ref):
    c_gpu = np.asarray(c_gpu).astype(np.float64)
    c_ref = np.asarray(c_ref).astype(np.float64)
    return np.abs(c_gpu - c_ref) <= np.maximum(CENTROID_REL * np.abs(c_ref), CENTROID_ABS_FLOOR)


def unpack_codes(codes):
    codes = np.asarray(codes)
    return np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(codes.shape[0], -1)


def identical_centroids(c_gpu, c_ref):
    return np.array_equal(np.asarray(c_gpu, np.float32).view(np.uint32),
                          np.asarray(c_ref, np.float32).view(np.uint32))


def explain_divergence(ws, a, c_trace, gpu_c_at, gpu_assign_at, gpu_final_q=None):
    """Why a GPU row differs from the oracle's, found by replaying the oracle's trajectory.

    ws, a:          the row's scaled weights and sample weights (oracle, fp32)
    c_trace:        the oracle's centroids c^0 .. c^iters of the row, [iters + 1, k]
    gpu_c_at(t):    the GPU path's centroids after t rounds (same row, same inputs)
    gpu_assign_at(c): the GPU E-step assignment of the row at centroids c (the stage
                    entry point that runs one round from given centroids)
    gpu_final_q:    the GPU's final codes of the row (unpacked), or None when only
                    centroids are compared

    Both trajectories start from the same c^0 (picks are compared bit-exactly elsewhere).
    At the first round t whose GPU centroids are not bit-identical to the oracle's, both
    sides started from the same c^(t-1); the divergence is allowed only if
      * every assignment that differs at c^(t-1) is an excused near-tie (the two
        distances differ by less than NEAR_TIE_REL relative), and
      * the GPU's c^t is within the centroid tolerance of the oracle's M-step evaluated
        on the GPU's assignment (what remains is fp64 summation order).
    If every round is bit-identical, the final assignments at c^iters may differ only at
    excused near-ties, and must differ somewhere (otherwise nothing diverged).
    Returns a one-line description; raises AssertionError when nothing explains the row.
    """
    iters = c_trace.shape[0] - 1
    for t in range(iters + 1):
        cg = np.asarray(gpu_c_at(t), np.float32)
        if identical_centroids(cg, c_trace[t]):
            continue
        assert t > 0, "initial centres differ"
        c_prev = c_trace[t - 1]
        q_ref = _oracle().estep_row(ws, c_prev)
        q_gpu = np.asarray(gpu_assign_at(c_prev), np.uint8)
        diff, ok = excused_mismatch(ws, c_prev, q_ref, q_gpu)
        assert ok.all(), f"round {t}: {int((~ok).sum())} assignments differ beyond a near-tie"
        c_ref = _oracle().mstep_row(ws, a, q_gpu, c_prev)
        assert centroid_close(cg, c_ref).all(), f"round {t}: centroids {cg} vs {c_ref}"
        what = f"{diff.size} excused near-ties" if diff.size else "M-step rounding only"
        dmax = float(np.max(np.abs(cg.astype(np.float64) - c_ref.astype(np.float64))))
        return f"first divergence in round {t}: {what}, max |dc| {dmax:.2e}"
    if gpu_final_q is None:
        raise AssertionError("no round diverged, yet the row differs")
    q_ref = _oracle().estep_row(ws, c_trace[iters])
    diff, ok = excused_mismatch(ws, c_trace[iters], q_ref, np.asarray(gpu_final_q, np.uint8))
    assert diff.size > 0, "trajectory and final assignment identical, yet the row differs"
    assert ok.all(), f"final E-step: {int((~ok).sum())} assignments differ beyond a near-tie"
    return f"final E-step: {diff.size} excused near-ties"


def _oracle():
    import oracle
    return oracle


def oracle_row_inputs(w_row, dtype, act, g, k, variant=0):
    """Scaled row and sample weights of one row under a variant (oracle)."""
    o = _oracle()
    ws, al, _, bad = o.scale_row(widen(w_row, dtype), g, k, symmetric=bool(variant & (1 << 4)))
    a, bad2 = o.weights_row(al, act, g, variant & 3)
    assert not bad and not bad2
    return ws, a


ALL_ROUNDS = 1 << 5  # the library's ANY4_ALL_ROUNDS: every Lloyd round, no stop at a fixed point


def explain_gpu_row(any4, w_row, dtype, act, g, k, iters, seed, row_offset, matrix_index, variant,
                    gpu_codes_row):
    """explain_divergence for one row of a GPU quantization: the row is re-run on its own
    (row_offset and matrix_index keep its Philox stream, so its bits are those of the
    whole-matrix call) once per round count to get the GPU trajectory."""
    import torch
    assert (variant >> 8) == 0, "with restarts every row must be identical"
    o = _oracle()
    w1 = np.ascontiguousarray(np.asarray(w_row)[None, :])
    # the oracle runs every round anyway: the no-early-stop bit is not a method variant
    ref = o.quantize(w1, dtype, act, g, k, iters, seed=seed, row_offset=row_offset,
                     matrix_index=matrix_index, trace=True, variant=variant & ~ALL_ROUNDS)
    ws, a = oracle_row_inputs(w_row, dtype, act, g, k, variant)

    class _M:
        pass
    m = _M()
    m.w, m.dtype, m.act = w1, dtype, act
    w, act_d = to_device(m)

    def c_at(t):
        _, c, _, _ = any4.stage_full(w, act_d, g, k, t, seed=seed, row_offset=row_offset,
                                     matrix_index=matrix_index, variant=variant)
        return c.cpu().numpy()[0]

    def assign_at(c):
        c_in = torch.from_numpy(np.asarray(c, np.float32)[None].copy()).to(w.device)
        q, _, _ = any4.stage_lloyd_step(w, act_d, c_in, g, k, variant=variant)
        return q.cpu().numpy()[0]

    q_final = unpack_codes(np.asarray(gpu_codes_row)[None])[0]
    return explain_divergence(ws, a, ref["c_trace"][0], c_at, assign_at, q_final)


def check_rows(any4, m, g, k, iters, seed, codes, cf, lut, ref, rows, ref_rows=None, matrix_index=0,
               variant=0):
    """Per GPU row i in `rows` (oracle row ref_rows[n], default the same index): identical
    codes, with centroids within tolerance and an fp16 LUT within one unit in the last
    place; or a divergence that explain_gpu_row accounts for.  With restarts every row must
    be identical.  Returns the per-row "identical codes" flags."""
    ref_rows = rows if ref_rows is None else ref_rows
    same = np.zeros(len(rows), bool)
    for n, (i, r) in enumerate(zip(rows, ref_rows)):
        same[n] = np.array_equal(codes[i], ref["codes"][r])
        if same[n]:
            assert centroid_close(cf[i], ref["c_final"][r]).all(), (m.name, i, cf[i], ref["c_final"][r])
            assert (np.abs(lut[i].astype(np.int32) - ref["lut"][r].astype(np.int32)) <= 1).all(), (m.name, i)
        else:
            why = explain_gpu_row(any4, m.w[i], m.dtype, m.act, g, k, iters, seed, int(i),
                                  matrix_index, variant, codes[i])
            say(f"  {m.name} row {i}: {why}")
    return same

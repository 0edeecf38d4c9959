"""Shared helpers for the GPU-vs-oracle parity tests (imported by tests only)."""
import sys

import numpy as np

# Tolerances (stated once, used by every parity test):
#   assignments: bit-exact, except where the two competing centroids' distances
#     |w_S - c| (fp64 from the fp32 operands) differ by less than 1e-6 relative
NEAR_TIE_REL = 1e-6
#   centroids after an M-step: |dc| <= 1e-5 * max(|c|, 1)   (scaled domain is [0, 2^n - 1])
CENTROID_REL = 1e-5
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
    return np.abs(c_gpu.astype(np.float64) - c_ref.astype(np.float64)) <= \
        CENTROID_REL * np.maximum(np.abs(c_ref.astype(np.float64)), 1.0)


def unpack_codes(codes):
    codes = np.asarray(codes)
    return np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(codes.shape[0], -1)

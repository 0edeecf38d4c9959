"""Python access to the any4 CPU oracle (test infrastructure only).

Only tests/, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of bench.py may
import this package.  It wraps ``liboracle_any4.so`` (plain C, built from
``any4_oracle.c`` with ``gcc -O2 -ffp-contract=off``) with ctypes and numpy.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "any4_oracle.c")
LIB = os.path.join(_HERE, "liboracle_any4.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc.  No fused multiply-add, no fast-math."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-o", tmp, SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        i32, i64, u32, u64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64
        L.oracle_philox4x32_10.argtypes = [P, P, P]
        L.oracle_philox4x64_10.argtypes = [P, P, P]
        L.oracle_fp16_rne_array.argtypes = [P, P, i64]
        L.oracle_scale_row.argtypes = [P, i64, i32, i32, P, P, P]
        L.oracle_scale_row.restype = ctypes.c_int
        L.oracle_weights_row.argtypes = [P, P, i64, i32, P]
        L.oracle_weights_row.restype = ctypes.c_int
        L.oracle_seed_row.argtypes = [P, P, i64, i32, u64, u64, u32, P, P]
        L.oracle_greedy_trials.argtypes = [i32]
        L.oracle_greedy_trials.restype = i32
        L.oracle_seed_row.restype = ctypes.c_int
        L.oracle_estep_row.argtypes = [P, i64, P, i32, P]
        L.oracle_mstep_row.argtypes = [P, P, P, i64, P, i32, P]
        L.oracle_objective_row.argtypes = [P, P, P, i64, P]
        L.oracle_objective_row.restype = ctypes.c_double
        L.oracle_pack_row.argtypes = [P, i64, P]
        L.oracle_any4_quantize.argtypes = [P, i32, i64, i64, P, i64, i32, i32, i32, i32, u64,
                                           P, P, P, P, P, P, P, P, P]
        L.oracle_any4_quantize.restype = ctypes.c_int
        L.oracle_any4_quantize_v.argtypes = [P, i32, i64, i64, P, i64, i32, i32, i32, i32, u64, i32,
                                             P, P, P, P, P, P, P, P, P]
        L.oracle_any4_quantize_v.restype = ctypes.c_int
        L.oracle_scale_row_mode.argtypes = [P, i64, i32, i32, i32, P, P, P]
        L.oracle_scale_row_mode.restype = ctypes.c_int
        L.oracle_weights_row_mode.argtypes = [P, P, i64, i32, i32, P]
        L.oracle_weights_row_mode.restype = ctypes.c_int
        L.oracle_seed_row_init.argtypes = [P, P, i64, i32, u64, u64, u32, i32, i32, ctypes.c_float, P, P]
        L.oracle_seed_row_init.restype = ctypes.c_int
        L.oracle_fp16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_fp16_to_f32.restype = ctypes.c_float
        L.oracle_bf16_rne_array.argtypes = [P, P, i64]
        L.oracle_act_absmean.argtypes = [P, i32, i64, i64, P]
        L.oracle_act_absmean.restype = ctypes.c_int
        L.oracle_dequantize.argtypes = [P, P, P, P, i64, i64, i32, i32, P]
        L.oracle_dequantize.restype = ctypes.c_int
        L.oracle_lut_gemv.argtypes = [P, P, P, P, i64, i64, i32, i32, P, i32, i64, P, P]
        L.oracle_lut_gemv.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


# --- primitives ----------------------------------------------------------------

def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, np.uint32)
    lib().oracle_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def philox4x64_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, dtype=np.uint64)
    k = np.ascontiguousarray(key, dtype=np.uint64)
    out = np.zeros(4, np.uint64)
    lib().oracle_philox4x64_10(_p(c), _p(k), _p(out))
    return out


def fp16_bits(x) -> np.ndarray:
    x = _f32(x).reshape(-1)
    out = np.zeros(x.shape, np.uint16)
    lib().oracle_fp16_rne_array(_p(x), _p(out), x.size)
    return out


def fp16_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16).reshape(-1)
    return np.array([lib().oracle_fp16_to_f32(int(v)) for v in b], np.float32)


def bf16_bits(x) -> np.ndarray:
    x = _f32(x)
    out = np.zeros(x.shape, np.uint16)
    lib().oracle_bf16_rne_array(_p(x), _p(out), x.size)
    return out


# --- bookends: the calibration statistic and dequantization -----------------------

def act_absmean(x: np.ndarray, dtype: int) -> np.ndarray:
    """E|x_j| over the rows of x ([T, K]; float32, or uint16 holding bfloat16 bits)."""
    x = np.ascontiguousarray(x)
    assert x.dtype == (np.float32 if dtype == 0 else np.uint16) and x.ndim == 2
    T, K = x.shape
    out = np.zeros(K, np.float32)
    st = lib().oracle_act_absmean(_p(x), dtype, T, K, _p(out))
    if st != 0:
        raise ValueError("oracle_act_absmean: invalid argument")
    return out


def dequantize(codes, lut, scale, offset, group: int, n_clusters: int) -> np.ndarray:
    """Eq. 4 dequantization to fp32 [N, K] from the emitted codes/LUT/scale/offset
    (fp16 arrays may be float16 or their uint16 bits)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    lut, scale, offset = (np.ascontiguousarray(np.asarray(a).view(np.uint16)) for a in (lut, scale, offset))
    N, K = codes.shape[0], codes.shape[1] * 2
    out = np.zeros((N, K), np.float32)
    st = lib().oracle_dequantize(_p(codes), _p(lut), _p(scale), _p(offset), N, K, group,
                                 n_clusters, _p(out))
    if st != 0:
        raise ValueError("oracle_dequantize: invalid argument")
    return out


def lut_gemv(codes, lut, scale, offset, group: int, n_clusters: int, x: np.ndarray, dtype: int):
    """y [M, N] fp32 = x [M, K] times the dequantized weight transposed (fp64 sums), and the
    magnitude scale s [M, N] (sum |x| (|alpha L| + |beta|)) for judging fp32 evaluations."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    lut, scale, offset = (np.ascontiguousarray(np.asarray(a).view(np.uint16)) for a in (lut, scale, offset))
    x = np.ascontiguousarray(x)
    assert x.dtype == (np.float32 if dtype == 0 else np.uint16) and x.ndim == 2
    N, K = codes.shape[0], codes.shape[1] * 2
    M = x.shape[0]
    y = np.zeros((M, N), np.float32)
    s = np.zeros((M, N), np.float64)
    st = lib().oracle_lut_gemv(_p(codes), _p(lut), _p(scale), _p(offset), N, K, group, n_clusters,
                               _p(x), dtype, M, _p(y), _p(s))
    if st != 0:
        raise ValueError("oracle_lut_gemv: invalid argument")
    return y, s


# --- row-level steps -------------------------------------------------------------

# variant word (the paper's ablations; 0 = defaults): bits 0-1 sample weights
# (0 alpha*E|x|, 1 E|x|, 2 none), bits 2-3 initialization (0 k-means++, 1 random,
# 2 uniform levels, 3 greedy k-means++), bit 4 symmetric scaling, bits 8-15 restarts - 1
WEIGHT_ALPHA_ACT, WEIGHT_ACT, WEIGHT_NONE = 0, 1, 2
INIT_KMEANSPP, INIT_RANDOM, INIT_UNIFORM, INIT_GREEDY = 0, 1 << 2, 2 << 2, 3 << 2


def greedy_trials(n_clusters: int) -> int:
    """Candidates per greedy k-means++ draw (2 + floor(ln k))."""
    return int(lib().oracle_greedy_trials(n_clusters))
SYMMETRIC = 1 << 4


def restarts(n: int) -> int:
    return (n - 1) << 8


def scale_row(w, group: int, n_clusters: int, symmetric: bool = False):
    w = _f32(w)
    K = w.size
    ws = np.zeros(K, np.float32)
    al = np.zeros(K // group, np.float32)
    be = np.zeros(K // group, np.float32)
    bad = lib().oracle_scale_row_mode(_p(w), K, group, n_clusters - 1, int(symmetric), _p(ws),
                                      _p(al), _p(be))
    return ws, al, be, bool(bad)


def weights_row(alpha, act, group: int, weighting: int = 0):
    alpha = _f32(alpha)
    act = _f32(act)
    a = np.zeros(act.size, np.float32)
    bad = lib().oracle_weights_row_mode(_p(alpha), _p(act), act.size, group, weighting, _p(a))
    return a, bool(bad)


def seed_row(ws, a, n_clusters: int, seed: int = 0, row_id: int = 0, matrix_index: int = 0,
             init: int = 0, restart: int = 0, level0: float = 0.0):
    """Initial centres; init 0 k-means++, 1 random, 2 uniform levels, 3 greedy k-means++
    (plain codes, not the shifted variant bits)."""
    ws, a = _f32(ws), _f32(a)
    c0 = np.zeros(n_clusters, np.float32)
    picks = np.zeros(n_clusters, np.int32)
    lib().oracle_seed_row_init(_p(ws), _p(a), ws.size, n_clusters, seed, row_id, matrix_index,
                               init, restart, level0, _p(c0), _p(picks))
    return c0, picks


def estep_row(ws, c) -> np.ndarray:
    ws, c = _f32(ws), _f32(c)
    q = np.zeros(ws.size, np.uint8)
    lib().oracle_estep_row(_p(ws), ws.size, _p(c), c.size, _p(q))
    return q


def mstep_row(ws, a, q, c_prev) -> np.ndarray:
    ws, a, c_prev = _f32(ws), _f32(a), _f32(c_prev)
    q = np.ascontiguousarray(q, dtype=np.uint8)
    cn = np.zeros(c_prev.size, np.float32)
    lib().oracle_mstep_row(_p(ws), _p(a), _p(q), ws.size, _p(c_prev), c_prev.size, _p(cn))
    return cn


def objective_row(ws, a, q, c) -> float:
    ws, a, c = _f32(ws), _f32(a), _f32(c)
    q = np.ascontiguousarray(q, dtype=np.uint8)
    return float(lib().oracle_objective_row(_p(ws), _p(a), _p(q), ws.size, _p(c)))


def pack_row(q) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    out = np.zeros(q.size // 2, np.uint8)
    lib().oracle_pack_row(_p(q), q.size, _p(out))
    return out


def lloyd_row(ws, a, c0, iters: int):
    """iters rounds of E then M from c0; returns (c_final, q_final, J trace)."""
    c = _f32(c0).copy()
    Js = []
    for _ in range(iters):
        q = estep_row(ws, c)
        Js.append(objective_row(ws, a, q, c))
        c = mstep_row(ws, a, q, c)
    q = estep_row(ws, c)
    Js.append(objective_row(ws, a, q, c))
    return c, q, np.array(Js)


# --- whole matrix ----------------------------------------------------------------

def quantize(w: np.ndarray, dtype: int, act: np.ndarray, group: int, n_clusters: int,
             iters: int, seed: int = 0, row_offset: int = 0, matrix_index: int = 0,
             trace: bool = False, variant: int = 0) -> dict:
    """Run the oracle over all rows of ``w`` ([N, K]; float32, or uint16 bf16 bits)."""
    w = np.ascontiguousarray(w)
    assert w.dtype == (np.float32 if dtype == 0 else np.uint16)
    N, K = w.shape
    act = _f32(act)
    G = K // group
    out = dict(
        codes=np.zeros((N, K // 2), np.uint8),
        lut=np.zeros((N, n_clusters), np.uint16),
        scale=np.zeros((N, G), np.uint16),
        offset=np.zeros((N, G), np.uint16),
        objective=np.zeros(N, np.float64),
        c_final=np.zeros((N, n_clusters), np.float32),
        picks=np.zeros((N, n_clusters), np.int32),
    )
    if trace:
        out["c_trace"] = np.zeros((N, iters + 1, n_clusters), np.float32)
        out["j_trace"] = np.zeros((N, iters + 1), np.float64)
    st = lib().oracle_any4_quantize_v(
        _p(w), dtype, N, K, _p(act), row_offset, matrix_index, group, n_clusters, iters, seed, variant,
        _p(out["codes"]), _p(out["lut"]), _p(out["scale"]), _p(out["offset"]),
        _p(out["objective"]), _p(out.get("c_trace")), _p(out.get("j_trace")),
        _p(out["picks"]), _p(out["c_final"]))
    out["status"] = st
    return out


def prepare_row(w_row: np.ndarray, dtype: int, act: np.ndarray, group: int, n_clusters: int):
    """Scaled row, alphas, betas and sample weights of one row (for staged checks)."""
    if dtype == 1:
        w_row = (np.asarray(w_row, np.uint16).astype(np.uint32) << 16).view(np.float32)
    ws, al, be, bad1 = scale_row(w_row, group, n_clusters)
    a, bad2 = weights_row(al, act, group)
    return ws, a, al, be, (bad1 or bad2)

"""Python binding of the MI355X any4 quantizer (libany4.so).

Argument marshalling only: every step of the quantizer runs in the gfx950 kernels
behind the C ABI declared in include/any4.h.  PyTorch supplies device memory and the
current HIP stream.  There is no CPU fallback: without the built library, or
without a GPU, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libany4.so")

ANY4_F32, ANY4_BF16 = 0, 1
# method variants (include/any4.h): OR them into `variant`
WEIGHT_ALPHA_ACT, WEIGHT_ACT, WEIGHT_NONE = 0, 1, 2
INIT_KMEANSPP, INIT_RANDOM, INIT_UNIFORM, INIT_GREEDY = 0, 1 << 2, 2 << 2, 3 << 2
SCALE_SYMMETRIC = 1 << 4
ALL_ROUNDS = 1 << 5   # every Lloyd round, no stop at an exact fixed point (same output bits)


def RESTARTS(n: int) -> int:
    return (n - 1) << 8
ANY4_OK = 0
ANY4_ERR_NONFINITE = 5
WORKSPACE_BYTES = 256
NOALLOC_SCRATCH_BYTES = 32 << 20   # ANY4_NOALLOC_SCRATCH_BYTES
NOALLOC_MAX_MATRICES = 64          # ANY4_NOALLOC_MAX_MATRICES

EXPORTED = [
    "any4_workspace_bytes", "any4_quantize", "any4_read_device_status", "any4_status_string",
    "any4_launch_geometry",
    "any4_stage_scale", "any4_stage_seed", "any4_stage_lloyd_step", "any4_stage_pack",
    "any4_stage_full", "any4_stage_lloyd_sorted", "any4_stage_lloyd_sorted_workspace_bytes",
    "any4_stage_quantize_batch",
    "any4_quantize_noalloc",
    "any4_act_absmean_workspace_bytes", "any4_act_absmean", "any4_dequantize", "any4_lut_gemv",
]


class Any4Matrix(ctypes.Structure):
    _fields_ = [
        ("w", ctypes.c_void_p),
        ("w_dtype", ctypes.c_int32),
        ("matrix_index", ctypes.c_int32),
        ("n_rows", ctypes.c_int64),
        ("n_cols", ctypes.c_int64),
        ("act_absmean", ctypes.c_void_p),
        ("row_offset", ctypes.c_int64),
        ("codes", ctypes.c_void_p),
        ("lut", ctypes.c_void_p),
        ("scale", ctypes.c_void_p),
        ("offset", ctypes.c_void_p),
        ("objective", ctypes.c_void_p),
    ]


class Any4Params(ctypes.Structure):
    _fields_ = [
        ("group", ctypes.c_int32),
        ("n_clusters", ctypes.c_int32),
        ("iters", ctypes.c_int32),
        ("variant", ctypes.c_int32),
        ("seed", ctypes.c_uint64),
    ]


class Any4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


_lib = None


def lib():
    """Load libany4.so (built in-tree by build.py / __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run python -m weight_only_bit_row_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, MP, PP = ctypes.c_void_p, ctypes.POINTER(Any4Matrix), ctypes.POINTER(Any4Params)
        L.any4_workspace_bytes.argtypes = [MP, ctypes.c_int32, PP, ctypes.POINTER(ctypes.c_size_t)]
        L.any4_quantize.argtypes = [MP, ctypes.c_int32, PP, P, ctypes.c_size_t, P]
        L.any4_quantize_noalloc.argtypes = [MP, ctypes.c_int32, PP, P, P]
        L.any4_read_device_status.argtypes = [P, P]
        L.any4_status_string.argtypes = [ctypes.c_int]
        L.any4_status_string.restype = ctypes.c_char_p
        L.any4_stage_scale.argtypes = [MP, PP, P, P, P, P, P]
        L.any4_stage_seed.argtypes = [MP, PP, P, P, P]
        L.any4_stage_lloyd_step.argtypes = [MP, PP, P, P, P, P, P]
        L.any4_stage_lloyd_sorted.argtypes = [MP, PP, P, P, P, P, P, ctypes.c_size_t, P]
        L.any4_stage_lloyd_sorted_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64,
                                                               ctypes.POINTER(ctypes.c_size_t)]
        L.any4_stage_pack.argtypes = [MP, PP, P, P, P, P, P]
        L.any4_stage_full.argtypes = [MP, PP, P, P, P, ctypes.c_size_t, P]
        L.any4_stage_quantize_batch.argtypes = [MP, ctypes.c_int32, PP, P, P, P, ctypes.c_size_t, P]
        L.any4_launch_geometry.argtypes = [ctypes.c_int64, ctypes.POINTER(ctypes.c_int32),
                                           ctypes.POINTER(ctypes.c_int32)]
        L.any4_act_absmean_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64,
                                                       ctypes.POINTER(ctypes.c_size_t)]
        L.any4_act_absmean.argtypes = [P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, P, P,
                                       ctypes.c_size_t, P]
        L.any4_dequantize.argtypes = [MP, PP, P, ctypes.c_int32, P]
        L.any4_lut_gemv.argtypes = [MP, PP, P, ctypes.c_int32, ctypes.c_int64, P, P]
        for name in EXPORTED:
            if name != "any4_status_string":
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def launch_geometry(n_cols: int) -> Tuple[int, int]:
    """(elements per lane, waves per row) of the row kernel for this row length."""
    e, nw = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib().any4_launch_geometry(n_cols, ctypes.byref(e), ctypes.byref(nw)), "any4_launch_geometry")
    return e.value, nw.value


def status_string(status: int) -> str:
    return lib().any4_status_string(status).decode()


def _check(status: int, what: str):
    if status != ANY4_OK:
        raise Any4Error(status, what)


# ---------------------------------------------------------------------------------
# torch glue

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _require_gpu(t):
    torch = _torch()
    if not torch.cuda.is_available():
        raise RuntimeError("the any4 quantizer needs a ROCm GPU; none is visible")
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")


def _dtype_code(w) -> Tuple[int, object]:
    torch = _torch()
    if w.dtype == torch.bfloat16:
        return ANY4_BF16, w
    if w.dtype == torch.float32:
        return ANY4_F32, w
    if w.dtype in (torch.int16, torch.uint16):   # raw bf16 bits
        return ANY4_BF16, w
    raise TypeError(f"W must be float32 or bfloat16, got {w.dtype}")


def params(group: int = 128, n_clusters: int = 16, iters: int = 20, seed: int = 0,
           variant: int = 0) -> Any4Params:
    return Any4Params(group, n_clusters, iters, variant, seed)


def workspace_bytes(mats, count: int, p: Any4Params) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().any4_workspace_bytes(mats, count, ctypes.byref(p), ctypes.byref(n)),
           "any4_workspace_bytes")
    return n.value


@dataclass
class Quantized:
    codes: object      # uint8 [N, K/2]
    lut: object        # fp16 [N, n_clusters]
    scale: object      # fp16 [N, K/group]
    offset: object     # fp16 [N, K/group]
    objective: object  # fp64 [N] or None


def _alloc_outputs(n, k_cols, group, n_clusters, device, with_objective):
    torch = _torch()
    return Quantized(
        codes=torch.empty((n, k_cols // 2), dtype=torch.uint8, device=device),
        lut=torch.empty((n, n_clusters), dtype=torch.float16, device=device),
        scale=torch.empty((n, k_cols // group), dtype=torch.float16, device=device),
        offset=torch.empty((n, k_cols // group), dtype=torch.float16, device=device),
        objective=(torch.empty((n,), dtype=torch.float64, device=device) if with_objective else None),
    )


def _matrix(w, act, out: Optional[Quantized], row_offset=0, matrix_index=0,
            group: Optional[int] = None, n_clusters: Optional[int] = None) -> Any4Matrix:
    torch = _torch()
    code, w = _dtype_code(w)
    if w.dim() != 2 or not w.is_contiguous():
        raise ValueError("W must be a contiguous [N, K] tensor")
    if (act.dim() != 1 or not act.is_contiguous() or act.dtype != torch.float32
            or act.numel() != w.shape[1] or act.device != w.device):
        raise ValueError("act_absmean must be a contiguous float32 [K] tensor on W's device")
    if out is not None and group is not None and n_clusters is not None:
        # caller-provided outputs: the kernels write exactly these extents
        N, K = int(w.shape[0]), int(w.shape[1])
        if group < 1 or K % group != 0 or K % 2 != 0:
            raise ValueError("group must divide K, and K must be even")
        want = [("codes", out.codes, (N, K // 2), torch.uint8),
                ("lut", out.lut, (N, n_clusters), torch.float16),
                ("scale", out.scale, (N, K // group), torch.float16),
                ("offset", out.offset, (N, K // group), torch.float16)]
        if out.objective is not None:
            want.append(("objective", out.objective, (N,), torch.float64))
        for name, t, shape, dt in want:
            if tuple(t.shape) != shape or t.dtype != dt or not t.is_contiguous() or t.device != w.device:
                raise ValueError(f"out.{name} must be a contiguous {list(shape)} {dt} tensor on W's device")
    m = Any4Matrix()
    m.w = _ptr(w)
    m.w_dtype = code
    m.matrix_index = matrix_index
    m.n_rows, m.n_cols = int(w.shape[0]), int(w.shape[1])
    m.act_absmean = _ptr(act)
    m.row_offset = row_offset
    if out is not None:
        m.codes, m.lut = _ptr(out.codes), _ptr(out.lut)
        m.scale, m.offset = _ptr(out.scale), _ptr(out.offset)
        m.objective = _ptr(out.objective)
    return m


def workspace(device=None, nbytes: int = WORKSPACE_BYTES):
    torch = _torch()
    return torch.empty((max(nbytes, WORKSPACE_BYTES),), dtype=torch.uint8, device=device or "cuda")


def quantize_batch(items: Sequence[Tuple[object, object]], group: int = 128, n_clusters: int = 16,
                   iters: int = 20, seed: int = 0, with_objective: bool = True,
                   outputs: Optional[List[Quantized]] = None, ws=None,
                   row_offsets: Optional[Sequence[int]] = None,
                   matrix_indices: Optional[Sequence[int]] = None,
                   variant: int = 0) -> List[Quantized]:
    """Quantize several (W [N,K], act_absmean [K]) pairs in one call."""
    if not items:
        return []
    w0 = items[0][0]
    _require_gpu(w0)
    device = w0.device
    p = params(group, n_clusters, iters, seed, variant)
    if outputs is None:
        outputs = [_alloc_outputs(w.shape[0], w.shape[1], group, n_clusters, device, with_objective)
                   for w, _ in items]
    mats = (Any4Matrix * len(items))()
    for i, (w, act) in enumerate(items):
        mats[i] = _matrix(w, act, outputs[i],
                          row_offset=(row_offsets[i] if row_offsets else 0),
                          matrix_index=(matrix_indices[i] if matrix_indices else i),
                          group=group, n_clusters=n_clusters)
    need = workspace_bytes(mats, len(items), p)
    if ws is None or ws.numel() < need:
        ws = workspace(device, need)
    _check(lib().any4_quantize(mats, len(items), ctypes.byref(p), _ptr(ws), ws.numel(),
                               _stream(device)), "any4_quantize")
    return outputs


def quantize(w, act, group: int = 128, n_clusters: int = 16, iters: int = 20, seed: int = 0,
             row_offset: int = 0, matrix_index: int = 0, with_objective: bool = True,
             out: Optional[Quantized] = None, ws=None, variant: int = 0) -> Quantized:
    """Quantize one matrix W [N,K] (bf16/fp32) with E|x| act [K] (fp32).  `variant`
    selects the paper's ablated variants (WEIGHT_*, INIT_*, SCALE_SYMMETRIC, RESTARTS(n))."""
    _require_gpu(w)
    p = params(group, n_clusters, iters, seed, variant)
    if out is None:
        out = _alloc_outputs(w.shape[0], w.shape[1], group, n_clusters, w.device, with_objective)
    m = _matrix(w, act, out, row_offset, matrix_index, group, n_clusters)
    need = WORKSPACE_BYTES if variant >> 8 == 0 else workspace_bytes(ctypes.byref(m), 1, p)
    if ws is None or ws.numel() < need:
        ws = workspace(w.device, need)
    _check(lib().any4_quantize(ctypes.byref(m), 1, ctypes.byref(p), _ptr(ws), ws.numel(),
                               _stream(w.device)), "any4_quantize")
    return out


def quantize_noalloc(items: Sequence[Tuple[object, object]], outputs: List[Quantized], group: int = 128,
                     n_clusters: int = 16, iters: int = 20, seed: int = 0, status_out=None,
                     matrix_indices: Optional[Sequence[int]] = None, variant: int = 0) -> List[Quantized]:
    """any4_quantize_noalloc: the batched quantizer with no workspace and no device
    allocation in the library (its scratch is a library-owned device array).  The caller
    passes preallocated outputs; status_out is an optional int32 [1] device tensor that
    receives the status word.  Calls that overlap on one GPU race on the scratch."""
    if not items:
        return []
    device = items[0][0].device
    _require_gpu(items[0][0])
    p = params(group, n_clusters, iters, seed, variant)
    mats = (Any4Matrix * len(items))()
    for i, (w, act) in enumerate(items):
        mats[i] = _matrix(w, act, outputs[i], matrix_index=(matrix_indices[i] if matrix_indices else i),
                          group=group, n_clusters=n_clusters)
    if status_out is not None:
        torch = _torch()
        if status_out.dtype != torch.int32 or status_out.numel() < 1 or status_out.device != device:
            raise ValueError("status_out must be an int32 tensor on W's device")
    _check(lib().any4_quantize_noalloc(mats, len(items), ctypes.byref(p), _ptr(status_out),
                                       _stream(device)), "any4_quantize_noalloc")
    return outputs


def read_status(ws) -> int:
    return lib().any4_read_device_status(_ptr(ws), _stream(ws.device))


# ---------------------------------------------------------------------------------
# bookends: E|x| of a calibration batch, and dequantization of the emitted codes

def act_absmean_workspace_bytes(n_tokens: int, n_cols: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().any4_act_absmean_workspace_bytes(n_tokens, n_cols, ctypes.byref(n)),
           "any4_act_absmean_workspace_bytes")
    return n.value


def act_absmean(x, out=None, ws=None):
    """E|x_j| [K] fp32 of activations x [T, K] (bf16 or fp32) on the GPU."""
    torch = _torch()
    _require_gpu(x)
    code, x = _dtype_code(x)
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [T, K] tensor")
    T, K = int(x.shape[0]), int(x.shape[1])
    if out is None:
        out = torch.empty((K,), dtype=torch.float32, device=x.device)
    elif tuple(out.shape) != (K,) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 [K] tensor")
    need = act_absmean_workspace_bytes(T, K)
    if ws is None or ws.numel() < need:
        ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=x.device)
    _check(lib().any4_act_absmean(_ptr(x), code, T, K, _ptr(out), _ptr(ws), ws.numel(),
                                  _stream(x.device)), "any4_act_absmean")
    return out


def _check_quantized(q: Quantized, group: int, n_clusters: int):
    """The C ABI takes bare pointers, so the extents it will read are checked here: codes
    [N, K/2] uint8, lut [N, n_clusters] fp16, scale and offset [N, K/group] fp16, all
    contiguous on one GPU."""
    torch = _torch()
    _require_gpu(q.codes)
    if q.codes.dim() != 2 or q.codes.dtype != torch.uint8:
        raise ValueError("codes must be a [N, K/2] uint8 tensor")
    N, K = int(q.codes.shape[0]), int(q.codes.shape[1]) * 2
    if group < 1 or K % group != 0:
        raise ValueError("group must divide K")
    want = {"lut": ((N, n_clusters), q.lut), "scale": ((N, K // group), q.scale),
            "offset": ((N, K // group), q.offset)}
    for name, (shape, t) in want.items():
        if tuple(t.shape) != shape or t.dtype != torch.float16:
            raise ValueError(f"{name} must be a {list(shape)} float16 tensor, got "
                             f"{list(t.shape)} {t.dtype}")
    for t in (q.codes, q.lut, q.scale, q.offset):
        if not t.is_contiguous() or t.device != q.codes.device:
            raise ValueError("codes, lut, scale and offset must be contiguous on one device")
    return N, K


def dequantize(q: Quantized, group: int = 128, n_clusters: int = 16, out_dtype=None, out=None):
    """Eq. 4 dequantization alpha * LUT[q] + beta of a quantized matrix to [N, K]
    bf16 (default) or fp32."""
    torch = _torch()
    N, K = _check_quantized(q, group, n_clusters)
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")
    if out is None:
        out = torch.empty((N, K), dtype=out_dtype, device=q.codes.device)
    elif tuple(out.shape) != (N, K) or out.dtype != out_dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [N, K] tensor of out_dtype")
    m = Any4Matrix()
    m.n_rows, m.n_cols = N, K
    m.w_dtype = ANY4_F32
    m.codes, m.lut, m.scale, m.offset = _ptr(q.codes), _ptr(q.lut), _ptr(q.scale), _ptr(q.offset)
    p = params(group, n_clusters, 0, 0)
    code = ANY4_BF16 if out_dtype == torch.bfloat16 else ANY4_F32
    _check(lib().any4_dequantize(ctypes.byref(m), ctypes.byref(p), _ptr(out), code,
                                 _stream(q.codes.device)), "any4_dequantize")
    return out


def lut_gemv(q: Quantized, x, group: int = 128, n_clusters: int = 16, out=None):
    """y [M, N] fp32 = x [M, K] (bf16/fp32, M <= 8) times the dequantized weight,
    transposed, without materializing it."""
    torch = _torch()
    N, K = _check_quantized(q, group, n_clusters)
    code, x = _dtype_code(x)
    if x.dim() != 2 or not x.is_contiguous() or x.device != q.codes.device:
        raise ValueError("x must be a contiguous [M, K] tensor on the codes' device")
    M = int(x.shape[0])
    if int(x.shape[1]) != K:
        raise ValueError("x has the wrong number of columns")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=q.codes.device)
    elif tuple(out.shape) != (M, N) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous [M, N] float32 tensor")
    m = Any4Matrix()
    m.n_rows, m.n_cols = N, K
    m.w_dtype = ANY4_F32
    m.codes, m.lut, m.scale, m.offset = _ptr(q.codes), _ptr(q.lut), _ptr(q.scale), _ptr(q.offset)
    p = params(group, n_clusters, 0, 0)
    _check(lib().any4_lut_gemv(ctypes.byref(m), ctypes.byref(p), _ptr(x), code, M, _ptr(out),
                               _stream(q.codes.device)), "any4_lut_gemv")
    return out


# ---------------------------------------------------------------------------------
# stage entry points (parity tests)

def stage_scale(w, act, group=128, n_clusters=16, row_offset=0, matrix_index=0, variant=0):
    torch = _torch()
    _require_gpu(w)
    N, K = w.shape
    dev = w.device
    ws_ = torch.empty((N, K), dtype=torch.float32, device=dev)
    al = torch.empty((N, K // group), dtype=torch.float32, device=dev)
    be = torch.empty((N, K // group), dtype=torch.float32, device=dev)
    a = torch.empty((N, K), dtype=torch.float32, device=dev)
    m = _matrix(w, act, None, row_offset, matrix_index)
    p = params(group, n_clusters, 0, 0, variant)
    _check(lib().any4_stage_scale(ctypes.byref(m), ctypes.byref(p), _ptr(ws_), _ptr(al), _ptr(be),
                                  _ptr(a), _stream(dev)), "any4_stage_scale")
    return ws_, al, be, a


def stage_seed(w, act, group=128, n_clusters=16, seed=0, row_offset=0, matrix_index=0, variant=0):
    torch = _torch()
    _require_gpu(w)
    N = w.shape[0]
    c0 = torch.empty((N, n_clusters), dtype=torch.float32, device=w.device)
    picks = torch.empty((N, n_clusters), dtype=torch.int32, device=w.device)
    m = _matrix(w, act, None, row_offset, matrix_index)
    p = params(group, n_clusters, 0, seed, variant)
    _check(lib().any4_stage_seed(ctypes.byref(m), ctypes.byref(p), _ptr(c0), _ptr(picks),
                                 _stream(w.device)), "any4_stage_seed")
    return c0, picks


def stage_lloyd_step(w, act, c_in, group=128, n_clusters=16, variant=0):
    torch = _torch()
    _require_gpu(w)
    N, K = w.shape
    assign = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    c_out = torch.empty((N, n_clusters), dtype=torch.float32, device=w.device)
    obj = torch.empty((N,), dtype=torch.float64, device=w.device)
    m = _matrix(w, act, None)
    p = params(group, n_clusters, 1, 0, variant)
    c_in = c_in.contiguous().to(torch.float32)
    _check(lib().any4_stage_lloyd_step(ctypes.byref(m), ctypes.byref(p), _ptr(c_in), _ptr(assign),
                                       _ptr(c_out), _ptr(obj), _stream(w.device)),
           "any4_stage_lloyd_step")
    return assign, c_out, obj


def stage_lloyd_sorted(w_s, a, c_in, n_clusters=16, iters=20, variant=0, group=128, ws=None):
    """Sorted-row Lloyd: ``iters`` rounds from c_in [N, n_clusters] on the scaled rows
    w_s and sample weights a ([N, K] fp32, K <= 32768); returns c_out [N, n_clusters].
    Rows over 16384 columns need a workspace (made here unless ``ws`` is given)."""
    torch = _torch()
    _require_gpu(w_s)
    N, K = w_s.shape
    w_s = w_s.contiguous().to(torch.float32)
    a = a.contiguous().to(torch.float32)
    c_in = c_in.contiguous().to(torch.float32)
    if a.shape != (N, K) or c_in.shape != (N, n_clusters):
        raise ValueError("a must be [N, K] and c_in [N, n_clusters]")
    if a.device != w_s.device or c_in.device != w_s.device:
        raise ValueError("w_s, a and c_in must be on one device")
    nbytes = ctypes.c_size_t(0)
    _check(lib().any4_stage_lloyd_sorted_workspace_bytes(N, K, ctypes.byref(nbytes)),
           "any4_stage_lloyd_sorted_workspace_bytes")
    if nbytes.value and ws is None:
        ws = torch.empty((nbytes.value,), dtype=torch.uint8, device=w_s.device)
    if ws is not None and (ws.device != w_s.device or ws.numel() * ws.element_size() < nbytes.value):
        raise ValueError("ws must be on w_s's device and hold the sorted stage's workspace")
    c_out = torch.empty((N, n_clusters), dtype=torch.float32, device=w_s.device)
    m = Any4Matrix()
    m.n_rows, m.n_cols = N, K
    p = params(group, n_clusters, iters, 0, variant)
    _check(lib().any4_stage_lloyd_sorted(ctypes.byref(m), ctypes.byref(p), _ptr(w_s), _ptr(a),
                                         _ptr(c_in), _ptr(c_out), _ptr(ws) if ws is not None else None,
                                         ws.numel() * ws.element_size() if ws is not None else 0,
                                         _stream(w_s.device)),
           "any4_stage_lloyd_sorted")
    return c_out


def stage_pack(n_rows, n_cols, assign, c, alpha, beta, group=128, n_clusters=16):
    _require_gpu(assign)
    out = _alloc_outputs(n_rows, n_cols, group, n_clusters, assign.device, False)
    m = Any4Matrix()
    m.n_rows, m.n_cols = n_rows, n_cols
    m.w_dtype = ANY4_F32
    m.w, m.act_absmean = _ptr(assign), _ptr(c)   # not read by the pack stage
    m.codes, m.lut, m.scale, m.offset = _ptr(out.codes), _ptr(out.lut), _ptr(out.scale), _ptr(out.offset)
    p = params(group, n_clusters, 0, 0)
    _check(lib().any4_stage_pack(ctypes.byref(m), ctypes.byref(p), _ptr(assign), _ptr(c),
                                 _ptr(alpha), _ptr(beta), _stream(assign.device)), "any4_stage_pack")
    return out


def stage_full(w, act, group=128, n_clusters=16, iters=20, seed=0, row_offset=0, matrix_index=0,
               variant=0):
    """Full path for one matrix plus the fp32 final centroids and the k-means++ picks."""
    torch = _torch()
    _require_gpu(w)
    N = w.shape[0]
    out = _alloc_outputs(N, w.shape[1], group, n_clusters, w.device, True)
    c_final = torch.empty((N, n_clusters), dtype=torch.float32, device=w.device)
    picks = torch.empty((N, n_clusters), dtype=torch.int32, device=w.device)
    m = _matrix(w, act, out, row_offset, matrix_index)
    p = params(group, n_clusters, iters, seed, variant)
    ws = workspace(w.device, workspace_bytes(ctypes.byref(m), 1, p))
    _check(lib().any4_stage_full(ctypes.byref(m), ctypes.byref(p), _ptr(c_final), _ptr(picks),
                                 _ptr(ws), ws.numel(), _stream(w.device)), "any4_stage_full")
    return out, c_final, picks, ws


def stage_quantize_batch(items, group=128, n_clusters=16, iters=20, seed=0, matrix_indices=None,
                         variant=0):
    """The batched path over several (W, act) pairs (one launch per row geometry, as
    quantize_batch) plus, per matrix, the fp32 final centroids and the k-means++ picks.
    Returns (outputs, c_finals, picks, ws)."""
    torch = _torch()
    if not items:
        return [], [], [], None
    device = items[0][0].device
    _require_gpu(items[0][0])
    p = params(group, n_clusters, iters, seed, variant)
    n = len(items)
    outputs = [_alloc_outputs(w.shape[0], w.shape[1], group, n_clusters, device, True) for w, _ in items]
    cfs = [torch.empty((w.shape[0], n_clusters), dtype=torch.float32, device=device) for w, _ in items]
    pks = [torch.empty((w.shape[0], n_clusters), dtype=torch.int32, device=device) for w, _ in items]
    mats = (Any4Matrix * n)()
    for i, (w, act) in enumerate(items):
        mats[i] = _matrix(w, act, outputs[i], matrix_index=(matrix_indices[i] if matrix_indices else i),
                          group=group, n_clusters=n_clusters)
    cptr = (ctypes.c_void_p * n)(*[_ptr(c) for c in cfs])
    pptr = (ctypes.c_void_p * n)(*[_ptr(q) for q in pks])
    ws = workspace(device, workspace_bytes(mats, n, p))
    _check(lib().any4_stage_quantize_batch(mats, n, ctypes.byref(p), cptr, pptr, _ptr(ws), ws.numel(),
                                           _stream(device)), "any4_stage_quantize_batch")
    return outputs, cfs, pks, ws

"""CPU-side checks of the C ABI: the library loads, exports every function that
include/any4.h declares, the ctypes structs match the header layout, and argument
validation rejects bad calls before anything is launched (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

import weight_only_bit_row_amd as any4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "any4.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(any4.LIB_PATH):
        from weight_only_bit_row_amd import build
        build.build()
    return any4.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(any4_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert len(names) >= 9
    out = subprocess.run(["nm", "-D", "--defined-only", any4.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(any4_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert sorted(any4.EXPORTED) == names


def test_struct_layout_matches_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "any4.h"\n'
        "int main(void){printf(\"%zu %zu %zu %zu %zu %zu\\n\", sizeof(any4_matrix),"
        " offsetof(any4_matrix, act_absmean), offsetof(any4_matrix, objective),"
        " sizeof(any4_params), offsetof(any4_params, seed), offsetof(any4_matrix, row_offset));"
        "return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    vals = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    assert vals == [ctypes.sizeof(any4.Any4Matrix), any4.Any4Matrix.act_absmean.offset,
                    any4.Any4Matrix.objective.offset, ctypes.sizeof(any4.Any4Params),
                    any4.Any4Params.seed.offset, any4.Any4Matrix.row_offset.offset]


def _mat(n=4, k=512, dtype=1):
    m = any4.Any4Matrix()
    m.w, m.act_absmean = 0x1000, 0x2000          # never dereferenced on these paths
    m.codes, m.lut, m.scale, m.offset = 0x3000, 0x4000, 0x5000, 0x6000
    m.w_dtype, m.n_rows, m.n_cols = dtype, n, k
    return m


def _ws_bytes(L, m, p):
    out = ctypes.c_size_t(0)
    st = L.any4_workspace_bytes(ctypes.byref(m), 1, ctypes.byref(p), ctypes.byref(out))
    return st, out.value


def test_workspace_query_and_validation(L):
    p = any4.params(128, 16, 20, 0)
    st, nbytes = _ws_bytes(L, _mat(), p)
    assert st == 0 and nbytes >= 4
    bad = [
        (dict(), dict(group=96)),          # not a power of two
        (dict(), dict(group=1)),
        (dict(), dict(n_clusters=3)),
        (dict(), dict(iters=-1)),
        (dict(k=500), dict()),             # K % group != 0
        (dict(k=129), dict(group=1)),
        (dict(n=-1), dict()),
        (dict(dtype=7), dict()),
    ]
    for mkw, pkw in bad:
        kw = dict(group=128, n_clusters=16, iters=20, seed=0)
        kw.update(pkw)
        st, _ = _ws_bytes(L, _mat(**mkw), any4.params(**kw))
        assert st == 1, (mkw, pkw)
    # variant word: unknown bits and unlisted field values are rejected
    for v in (3, 1 << 6, 1 << 7, 1 << 16, -1):
        assert _ws_bytes(L, _mat(), any4.params(128, 16, 20, 0, v))[0] == 1, v
    for v in (any4.WEIGHT_ACT, any4.WEIGHT_NONE | any4.INIT_RANDOM, any4.SCALE_SYMMETRIC,
              any4.INIT_UNIFORM | any4.SCALE_SYMMETRIC, any4.INIT_GREEDY, any4.ALL_ROUNDS,
              any4.ALL_ROUNDS | any4.WEIGHT_ACT):
        assert _ws_bytes(L, _mat(), any4.params(128, 16, 20, 0, v)) == (0, 256), v
    # restarts need room for one candidate set of outputs per matrix
    st, nbytes = _ws_bytes(L, _mat(n=4, k=512), any4.params(128, 16, 20, 0, any4.RESTARTS(3)))
    assert st == 0 and nbytes >= 256 + 4 * 256 + 4 * 16 * 2 + 2 * 4 * 8 + 2 * 4 * 16 * 4
    # too long for register residency
    assert _ws_bytes(L, _mat(k=65536), p)[0] == 2
    # missing product pointer
    m = _mat()
    m.lut = None
    assert _ws_bytes(L, m, p)[0] == 1
    # zero rows need no pointers
    m0 = any4.Any4Matrix()
    m0.n_rows, m0.n_cols, m0.w_dtype = 0, 256, 1
    assert _ws_bytes(L, m0, p)[0] == 0


def test_quantize_rejects_before_launch(L):
    """Errors are returned synchronously, before any HIP call."""
    p = any4.params(128, 16, 20, 0)
    m = _mat()
    # no workspace
    assert L.any4_quantize(ctypes.byref(m), 1, ctypes.byref(p), None, 0, None) == 3
    assert L.any4_quantize(ctypes.byref(m), 1, ctypes.byref(p), 0x7000, 8, None) == 3
    # invalid params win over the workspace check
    assert L.any4_quantize(ctypes.byref(m), 1, ctypes.byref(any4.params(100)), None, 0, None) == 1
    assert L.any4_quantize(None, 1, ctypes.byref(p), 0x7000, 256, None) == 1
    assert L.any4_quantize(ctypes.byref(m), 1, None, 0x7000, 256, None) == 1
    assert L.any4_quantize(ctypes.byref(m), -1, ctypes.byref(p), 0x7000, 256, None) == 1
    # stage entry points validate too
    assert L.any4_stage_seed(ctypes.byref(m), ctypes.byref(p), None, None, None) == 1
    assert L.any4_stage_lloyd_step(ctypes.byref(_mat(k=500)), ctypes.byref(p), 1, 1, 1, None, None) == 1
    assert L.any4_stage_full(ctypes.byref(m), ctypes.byref(p), None, None, None, 0, None) == 3


def test_noalloc_validates_before_launch(L):
    """The entry point that allocates nothing refuses bad batches, too many matrices and
    batches that need more than its scratch, all before any HIP call."""
    p = any4.params(128, 16, 20, 0)
    m = _mat()
    assert L.any4_quantize_noalloc(None, 1, ctypes.byref(p), None, None) == 1
    assert L.any4_quantize_noalloc(ctypes.byref(m), 1, ctypes.byref(any4.params(100)), None, None) == 1
    assert L.any4_quantize_noalloc(ctypes.byref(_mat(k=65536)), 1, ctypes.byref(p), None, None) == 2
    many = (any4.Any4Matrix * (any4.NOALLOC_MAX_MATRICES + 1))(*[_mat() for _ in range(any4.NOALLOC_MAX_MATRICES + 1)])
    assert L.any4_quantize_noalloc(many, any4.NOALLOC_MAX_MATRICES + 1, ctypes.byref(p), None, None) == 2
    # restarts on 20000 x 4096 need ~41 MB of candidates: more than the 32 MiB scratch
    big = _mat(n=20000, k=4096)
    pr = any4.params(128, 16, 20, 0, any4.RESTARTS(2))
    st, need = _ws_bytes(L, big, pr)
    assert st == 0 and need > any4.NOALLOC_SCRATCH_BYTES
    assert L.any4_quantize_noalloc(ctypes.byref(big), 1, ctypes.byref(pr), None, None) == 3
    # the headline matrix with restarts fits
    st, need = _ws_bytes(L, _mat(n=14336, k=4096), pr)
    assert st == 0 and need <= any4.NOALLOC_SCRATCH_BYTES


def test_bookends_validate_before_launch(L):
    """E|x| and dequantization reject bad arguments synchronously (no HIP call)."""
    n = ctypes.c_size_t(0)
    assert L.any4_act_absmean_workspace_bytes(1000, 4096, ctypes.byref(n)) == 0 and n.value > 0
    assert L.any4_act_absmean_workspace_bytes(0, 4096, ctypes.byref(n)) == 1
    assert L.any4_act_absmean_workspace_bytes(10, 0, ctypes.byref(n)) == 1
    assert L.any4_act_absmean_workspace_bytes(10, 8, None) == 1
    L.any4_act_absmean_workspace_bytes(262144, 4096, ctypes.byref(n))
    assert n.value <= 64 << 20           # fp64 partials stay small next to the batch
    assert L.any4_act_absmean(0x7000, 1, 10, 8, 0x8000, None, 0, None) == 3
    assert L.any4_act_absmean(None, 1, 10, 8, 0x8000, 0x9000, 1 << 20, None) == 1
    assert L.any4_act_absmean(0x7000, 3, 10, 8, 0x8000, 0x9000, 1 << 20, None) == 1
    assert L.any4_act_absmean(0x7000, 1, 0, 8, 0x8000, 0x9000, 1 << 20, None) == 1
    p = any4.params(128, 16, 20, 0)
    m = _mat()
    assert L.any4_dequantize(ctypes.byref(m), ctypes.byref(p), None, 1, None) == 1
    assert L.any4_dequantize(ctypes.byref(m), ctypes.byref(p), 0x7000, 5, None) == 1
    assert L.any4_dequantize(ctypes.byref(m), ctypes.byref(any4.params(96)), 0x7000, 1, None) == 1
    assert L.any4_dequantize(ctypes.byref(_mat(k=500)), ctypes.byref(p), 0x7000, 1, None) == 1
    assert L.any4_dequantize(None, ctypes.byref(p), 0x7000, 1, None) == 1
    m0 = any4.Any4Matrix()
    m0.n_rows, m0.n_cols = 0, 256
    assert L.any4_dequantize(ctypes.byref(m0), ctypes.byref(p), None, 1, None) == 0



def test_lut_gemv_validates_before_launch(L):
    """The LUT matrix-vector product rejects bad arguments, and reports shapes outside
    its kernel (more than 8 tokens, K or group not a multiple of 16, codes not 8-byte or
    x not 16-byte aligned) as unsupported, without a HIP call."""
    p = any4.params(128, 16, 20, 0)
    m = _mat()
    y = 0x9000
    gemv = L.any4_lut_gemv
    assert gemv(ctypes.byref(m), ctypes.byref(p), None, 1, 1, y, None) == 1
    assert gemv(ctypes.byref(m), ctypes.byref(p), 0x7000, 1, 1, None, None) == 1
    assert gemv(ctypes.byref(m), ctypes.byref(p), 0x7000, 5, 1, y, None) == 1
    assert gemv(ctypes.byref(m), ctypes.byref(p), 0x7000, 1, 0, y, None) == 1
    assert gemv(ctypes.byref(m), ctypes.byref(any4.params(96)), 0x7000, 1, 1, y, None) == 1
    assert gemv(ctypes.byref(_mat(k=500)), ctypes.byref(p), 0x7000, 1, 1, y, None) == 1
    assert gemv(None, ctypes.byref(p), 0x7000, 1, 1, y, None) == 1
    assert gemv(ctypes.byref(m), ctypes.byref(p), 0x7000, 1, 9, y, None) == 2
    assert gemv(ctypes.byref(m), ctypes.byref(any4.params(8)), 0x7000, 1, 1, y, None) == 2
    assert gemv(ctypes.byref(_mat(k=520)), ctypes.byref(any4.params(8)), 0x7000, 1, 1, y, None) == 2
    odd = _mat()
    odd.codes = 0x3004
    assert gemv(ctypes.byref(odd), ctypes.byref(p), 0x7000, 1, 1, y, None) == 2
    assert gemv(ctypes.byref(m), ctypes.byref(p), 0x7008, 1, 1, y, None) == 2   # x alignment
    assert gemv(ctypes.byref(_mat(k=1 << 31)), ctypes.byref(p), 0x7000, 1, 1, y, None) == 2
    m0 = any4.Any4Matrix()
    m0.n_rows, m0.n_cols = 0, 256
    assert gemv(ctypes.byref(m0), ctypes.byref(p), None, 1, 1, None, None) == 0

def test_sorted_lloyd_validates_before_launch(L):
    """any4_stage_lloyd_sorted rejects bad params, missing buffers and odd or short rows
    (invalid argument), rows over 16384 columns without their workspace (workspace) and
    rows over 32768 columns (unsupported), all without a HIP call; an empty matrix is a
    no-op."""
    p = any4.params(128, 16, 20, 0)
    f = L.any4_stage_lloyd_sorted
    buf = 0x8000
    assert f(ctypes.byref(_mat(k=4096)), ctypes.byref(p), None, buf, buf, buf, None, 0, None) == 1
    assert f(ctypes.byref(_mat(k=4096)), ctypes.byref(p), buf, buf, buf, None, None, 0, None) == 1
    assert f(ctypes.byref(_mat(k=511)), ctypes.byref(p), buf, buf, buf, buf, None, 0, None) == 1
    assert f(ctypes.byref(_mat(k=0)), ctypes.byref(p), buf, buf, buf, buf, None, 0, None) == 1
    assert f(None, ctypes.byref(p), buf, buf, buf, buf, None, 0, None) == 1
    assert f(ctypes.byref(_mat(k=512)), ctypes.byref(any4.params(128, 5)), buf, buf, buf, buf, None, 0,
             None) == 1
    need = ctypes.c_size_t(0)
    assert L.any4_stage_lloyd_sorted_workspace_bytes(4, 16386, ctypes.byref(need)) == 0
    assert need.value == 4 * 3 * 16384 * 4
    g2 = any4.params(2, 16, 20, 0)
    assert f(ctypes.byref(_mat(k=16386)), ctypes.byref(g2), buf, buf, buf, buf, None, 0, None) == 3
    assert f(ctypes.byref(_mat(k=16386)), ctypes.byref(g2), buf, buf, buf, buf, 0x9000,
             need.value - 1, None) == 3
    assert f(ctypes.byref(_mat(k=16386)), ctypes.byref(g2), buf, buf, buf, buf, 0x9008,
             need.value, None) == 3   # misaligned
    assert f(ctypes.byref(_mat(k=32770)), ctypes.byref(g2), buf, buf, buf, buf, 0x9000,
             need.value, None) == 2
    assert L.any4_stage_lloyd_sorted_workspace_bytes(4, 32770, ctypes.byref(need)) == 2
    assert L.any4_stage_lloyd_sorted_workspace_bytes(4, 4096, ctypes.byref(need)) == 0
    assert need.value == 0
    assert L.any4_stage_lloyd_sorted_workspace_bytes(4, 4095, ctypes.byref(need)) == 1
    m0 = any4.Any4Matrix()
    m0.n_rows, m0.n_cols = 0, 256
    assert f(ctypes.byref(m0), ctypes.byref(p), None, None, None, None, None, 0, None) == 0


def test_launch_geometry(L):
    assert any4.launch_geometry(4096) == (32, 2)
    assert any4.launch_geometry(512) == (8, 1)
    assert any4.launch_geometry(28672) == (32, 14)
    assert any4.launch_geometry(32768) == (32, 16)
    for k in [2, 100, 1000, 2048, 14336, 32768]:
        e, nw = any4.launch_geometry(k)
        assert e * nw * 64 >= k
    with pytest.raises(any4.Any4Error):
        any4.launch_geometry(65536)


def test_status_strings(L):
    for s in range(6):
        assert any4.status_string(s)
    assert any4.status_string(0) == "ok"
    assert "unknown" in any4.status_string(99)


def test_no_gpu_fails_loudly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("GPU present")
    w = torch.zeros((2, 256), dtype=torch.bfloat16)
    with pytest.raises(RuntimeError):
        any4.quantize(w, torch.ones(256))

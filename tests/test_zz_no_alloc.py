"""any4_quantize_noalloc, the entry point for callers that cannot allocate (graph capture,
serving loops): through the C ABI, its outputs equal any4_quantize's bit for bit, on two
calls in a row with the second smaller (the library-owned scratch keeps the first call's
contents), with and without restarts (whose candidates live in the scratch); its status
word reaches status_out and is cleared between calls; batches that would need more
scratch than it has are refused before any launch."""
import numpy as np
import pytest

from parity_util import say, to_device
from workloads import BF16, F32, make_matrix

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def any4():
    import weight_only_bit_row_amd as mod
    return mod


FIELDS = ["codes", "lut", "scale", "offset", "objective"]


def _alloc(items, g, k):
    return [any4()._alloc_outputs(w.shape[0], w.shape[1], g, k, w.device, True) for w, _ in items]


def _same(a, b):
    for qa, qb in zip(a, b):
        for f in FIELDS:
            x, y = getattr(qa, f).cpu().view(torch.uint8), getattr(qb, f).cpu().view(torch.uint8)
            assert torch.equal(x, y), f


@pytest.mark.parametrize("variant", [0, 2 << 8], ids=["default", "restarts3"])
def test_noalloc_matches_quantize_on_two_calls(variant):
    g, k, iters = 128, 16, 12
    calls = [
        [make_matrix("na0", 1200, 4096, BF16, 501), make_matrix("na1", 64, 14336, BF16, 502)],
        [make_matrix("na2", 300, 1024, F32, 503)],            # smaller than the first
    ]
    for n, mats in enumerate(calls):
        items = [to_device(m) for m in mats]
        say(f"noalloc variant={variant} call {n}: {[m.w.shape for m in mats]}")
        ref = any4().quantize_batch(items, group=g, n_clusters=k, iters=iters, seed=3, variant=variant)
        st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        got = any4().quantize_noalloc(items, _alloc(items, g, k), group=g, n_clusters=k, iters=iters,
                                      seed=3, status_out=st, variant=variant)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        _same(got, ref)


def test_noalloc_status_word_is_reported_and_cleared():
    g, k = 128, 16
    m = make_matrix("nb", 8, 1024, F32, 504)
    w = m.w.copy()
    w[3, 5] = np.nan
    bad = [(torch.from_numpy(w).cuda(), torch.from_numpy(m.act).cuda())]
    st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    say("noalloc non-finite row, then a clean call")
    out = any4().quantize_noalloc(bad, _alloc(bad, g, k), group=g, n_clusters=k, iters=4, status_out=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 5
    obj = out[0].objective.cpu().numpy()
    assert np.isnan(obj[3]) and np.isfinite(obj[[0, 1, 2, 4, 5, 6, 7]]).all()
    good = [to_device(m)]
    any4().quantize_noalloc(good, _alloc(good, g, k), group=g, n_clusters=k, iters=4, status_out=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0


def test_noalloc_refuses_batches_beyond_its_scratch():
    say("noalloc size limits")
    A = any4()
    w = torch.zeros((20000, 4096), dtype=torch.bfloat16, device="cuda")   # restarts need ~41 MB
    act = torch.ones(4096, device="cuda")
    items = [(w, act)]
    with pytest.raises(A.Any4Error) as e:
        A.quantize_noalloc(items, _alloc(items, 128, 16), variant=A.RESTARTS(2))
    assert e.value.status == 3
    small = [(torch.zeros((1, 64), device="cuda"), torch.ones(64, device="cuda"))] * (A.NOALLOC_MAX_MATRICES + 1)
    with pytest.raises(A.Any4Error) as e:
        A.quantize_noalloc(small, _alloc(small, 64, 16), group=64)
    assert e.value.status == 2

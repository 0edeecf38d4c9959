"""GPU parity of the k-means++ sampling at the edges of its fixed-point scale.

The integer CDF scales the sampling weights by 2^s, s = 40 - floor(log2 B) (reading R7 of
the any4 paper's k-means++ initialization, Appendix C.2).  From the second draw on the
sample weights carry that scale when s >= 0; a bound above 2^40 (s < 0) scales each product
instead.  The synthetic rows never leave the first regime, so these cases push E|x| by
2^40 (s < 0) and by 2^-110 (s near 150, products a_j * D_j below the fp32 normal range),
on every row geometry and for plain, greedy and random initialization:

- the GPU's picks and initial centres equal the oracle's bit for bit;
- the picks do not depend on the power of two (D^2 sampling is scale-free in the weights,
  and both scalings of E|x| are exact here);
- end to end, codes and LUT equal those of the unscaled row and the objective scales by
  exactly the same power of two.
"""
import numpy as np
import pytest

import oracle
from parity_util import say, to_device
from workloads import BF16, F32, make_matrix

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def any4():
    import weight_only_bit_row_amd as mod
    return mod


# (name, N, K, dtype, group, n_clusters, seed): one case per row geometry
SHAPES = [
    ("e8_k512", 16, 512, F32, 128, 16, 201),
    ("e16_k1024", 12, 1024, BF16, 64, 16, 202),
    ("one_wave_k2048", 10, 2048, BF16, 128, 16, 203),
    ("two_waves_k4096", 8, 4096, BF16, 128, 16, 204),
    ("two_waves_narrow_g16", 6, 4096, BF16, 16, 16, 205),
    ("seven_waves_k14336", 4, 14336, BF16, 128, 16, 206),
    ("fourteen_waves_k28672", 2, 28672, BF16, 128, 8, 207),
]
SCALES = [("x2^40", 40), ("x2^-110", -110)]
# (name, GPU variant word, oracle init code)
INITS = [("kmeanspp", 0, 0), ("greedy", 3 << 2, 3), ("random", 1 << 2, 1)]


@pytest.fixture(scope="module", params=SHAPES, ids=[s[0] for s in SHAPES])
def case(request):
    name, N, K, dtype, g, k, seed = request.param
    return name, make_matrix(name, N, K, dtype, seed), g, k


def scaled_act(m, e):
    act = (m.act.astype(np.float64) * 2.0 ** e).astype(np.float32)
    assert np.array_equal(act.astype(np.float64) * 2.0 ** -e, m.act.astype(np.float64))  # exact
    return act


@pytest.mark.parametrize("scale", SCALES, ids=[s[0] for s in SCALES])
@pytest.mark.parametrize("init", INITS, ids=[i[0] for i in INITS])
def test_seed_at_scale_edges(case, scale, init):
    name, m, g, k = case
    sname, e = scale
    iname, variant, init_code = init
    say(f"seed scales {name} {sname} {iname}")
    act2 = scaled_act(m, e)
    w, act_d = to_device(m)
    act2_d = torch.from_numpy(act2).cuda()
    c0, picks = any4().stage_seed(w, act2_d, group=g, n_clusters=k, seed=7, variant=variant)
    _, picks_1 = any4().stage_seed(w, act_d, group=g, n_clusters=k, seed=7, variant=variant)
    torch.cuda.synchronize()
    c0, picks, picks_1 = c0.cpu().numpy(), picks.cpu().numpy(), picks_1.cpu().numpy()
    for i in range(m.w.shape[0]):
        ws, a, _, _, bad = oracle.prepare_row(m.w[i], m.dtype, act2, g, k)
        assert not bad
        rc, rp = oracle.seed_row(ws, a, k, 7, i, 0, init=init_code)
        assert np.array_equal(picks[i], rp), (name, sname, iname, i, picks[i], rp)
        assert np.array_equal(c0[i].view(np.uint32), rc.view(np.uint32)), (name, sname, iname, i)
    assert np.array_equal(picks, picks_1), (name, sname, iname)


@pytest.mark.parametrize("scale", SCALES, ids=[s[0] for s in SCALES])
def test_quantize_is_scale_free_in_act(case, scale):
    name, m, g, k = case
    sname, e = scale
    say(f"scale-free quantize {name} {sname}")
    act2 = scaled_act(m, e)
    w, act_d = to_device(m)
    out1 = any4().quantize(w, act_d, group=g, n_clusters=k, iters=20)
    out2 = any4().quantize(w, torch.from_numpy(act2).cuda(), group=g, n_clusters=k, iters=20)
    torch.cuda.synchronize()
    assert np.array_equal(out1.codes.cpu().numpy(), out2.codes.cpu().numpy()), (name, sname)
    assert np.array_equal(out1.lut.cpu().numpy(), out2.lut.cpu().numpy()), (name, sname)
    j1 = out1.objective.cpu().numpy()
    j2 = out2.objective.cpu().numpy()
    assert np.array_equal(j2, j1 * 2.0 ** e), (name, sname, j1[:3], j2[:3])

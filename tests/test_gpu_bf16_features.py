"""bfloat16 node features (x_dtype = EQTP_BF16) in the node-factored
convolution and in the per-edge kernel (edges in any order with fp32 atomics,
radial weights, the per-edge walk on request): parity with the fp64 oracle
evaluated on the same bf16 values (widened exactly), and bit-identity with the
fp32 path fed those values where the summation order is fixed."""
import numpy as np
import pytest

import oracle
from spherical_harmonic_cg_amd import synth
from test_gpu_parity import TOL, _assert_close, _eq, _np, _say, _t

pytestmark = pytest.mark.gpu


def _bf16(x):
    import torch

    xb = _t(x).to(torch.bfloat16)
    return xb, xb.float().cpu().numpy()


@pytest.mark.parametrize("lmax", [0, 1, 2, 3])
@pytest.mark.parametrize("ps", [0, 1])
@pytest.mark.parametrize("C", [8, 16, 32, 64, 128])
def test_bf16_features_small(lmax, ps, C):
    eq = _eq()
    wl = synth.small_graph(33, 9, C, lmax, 1100 + lmax * 10 + C, path_set=ps, empty_rows=(2,), long_rows=(4,),
                           long_len=90, zero_vec_edges=1)
    xb, xr = _bf16(wl.x)
    _say("bf16 features lmax=%d ps=%d C=%d" % (lmax, ps, C))
    got = _np(eq.eqtp_conv_fused(_t(wl.vec), _t(wl.src), xb, _t(wl.w), lmax, row_ptr=_t(wl.row_ptr), path_set=ps))
    ref = oracle.conv(wl.N, wl.vec, wl.src, wl.dst, xr, wl.w, lmax, path_set=ps)
    _assert_close(got, ref, TOL, "bf16 features L%d ps%d C%d" % (lmax, ps, C))
    same = _np(eq.eqtp_conv_fused(_t(wl.vec), _t(wl.src), _t(xr), _t(wl.w), lmax, row_ptr=_t(wl.row_ptr),
                                  path_set=ps))
    assert np.array_equal(got, same), "bf16 path differs from the fp32 path on the same values"


def test_bf16_features_mid_workload():
    eq = _eq()
    wl = synth.make_config("mid")
    xb, xr = _bf16(wl.x)
    _say("bf16 features mid")
    got = _np(eq.eqtp_conv_fused(_t(wl.vec), _t(wl.src), xb, _t(wl.w), 3, row_ptr=_t(wl.row_ptr)))
    ref = oracle.conv(wl.N, wl.vec, wl.src, wl.dst, xr, wl.w, 3)
    _assert_close(got, ref, TOL, "bf16 features mid")


@pytest.mark.parametrize("lmax", [0, 1, 2, 3])
@pytest.mark.parametrize("C", [8, 16, 32, 64, 128])
def test_bf16_features_edge_kernel(lmax, C):
    """Unsorted edges (atomics), the sorted per-edge walk (algo 2) and radial weights with bf16 x."""
    eq = _eq()
    wl = synth.small_graph(31, 10, C, lmax, 1300 + lmax * 10 + C, empty_rows=(0,), long_rows=(5,), long_len=80,
                           zero_vec_edges=1, radial=True, r_cut=5.0)
    wl.vec[7:10] *= 1.7  # beyond the cut-off for the radial case
    xb, xr = _bf16(wl.x)
    pvec, psrc, pdst = synth.random_permutation(wl)
    ref = oracle.conv(wl.N, wl.vec, wl.src, wl.dst, xr, wl.w, lmax)
    _say("bf16 features unsorted lmax=%d C=%d" % (lmax, C))
    got = _np(eq.eqtp_conv_fused(_t(pvec), _t(psrc), xb, _t(wl.w), lmax, dst=_t(pdst)))
    _assert_close(got, ref, TOL, "bf16 unsorted L%d C%d" % (lmax, C))
    _say("bf16 features sorted per-edge walk lmax=%d C=%d" % (lmax, C))
    got2 = _np(eq.eqtp_conv_fused(_t(wl.vec), _t(wl.src), xb, _t(wl.w), lmax, row_ptr=_t(wl.row_ptr), algo=2))
    _assert_close(got2, ref, TOL, "bf16 per-edge walk L%d C%d" % (lmax, C))
    same = _np(eq.eqtp_conv_fused(_t(wl.vec), _t(wl.src), _t(xr), _t(wl.w), lmax, row_ptr=_t(wl.row_ptr), algo=2))
    assert np.array_equal(got2, same), "bf16 per-edge walk differs from the fp32 walk on the same values"
    refr = oracle.conv(wl.N, wl.vec, wl.src, wl.dst, xr, wl.w_rad, lmax, weight_mode=1, r_cut=5.0)
    _say("bf16 features radial sorted / unsorted lmax=%d C=%d" % (lmax, C))
    kw = dict(weight_mode=1, r_cut=5.0)
    gr = _np(eq.eqtp_conv_fused(_t(wl.vec), _t(wl.src), xb, _t(wl.w_rad), lmax, row_ptr=_t(wl.row_ptr), **kw))
    _assert_close(gr, refr, TOL, "bf16 radial sorted L%d C%d" % (lmax, C))
    gu = _np(eq.eqtp_conv_fused(_t(pvec), _t(psrc), xb, _t(wl.w_rad), lmax, dst=_t(pdst), **kw))
    _assert_close(gu, refr, TOL, "bf16 radial unsorted L%d C%d" % (lmax, C))


def test_bf16_features_large_unsorted():
    """The large workload (5.2M edges) in random order with bf16 features: every row against the oracle
    on the same bf16 values."""
    eq = _eq()
    wl = synth.make_config("large")
    xb, xr = _bf16(wl.x)
    pvec, psrc, pdst = synth.random_permutation(wl)
    _say("bf16 features large unsorted E=%d" % wl.E)
    got = _np(eq.eqtp_conv_fused(_t(pvec), _t(psrc), xb, _t(wl.weights), 3, dst=_t(pdst)))
    ref = oracle.conv(wl.N, wl.vec, wl.src, wl.dst, xr, wl.weights, 3)
    _assert_close(got, ref, TOL, "bf16 large unsorted")


def test_bf16_features_rejected_where_unsupported():
    eq = _eq()
    wl = synth.small_graph(8, 4, 16, 3, 1200)
    xb, _ = _bf16(wl.x)
    _say("bf16 features unsupported paths")
    with pytest.raises(eq.EqtpError):  # the edge-aligned form takes fp32 features only
        eq.eqtp_conv_fused(_t(wl.vec), _t(wl.src), xb, _t(wl.w), 3, row_ptr=_t(wl.row_ptr), algo=3)

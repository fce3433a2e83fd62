"""bfloat16 node features in the node-factored convolution (x_dtype =
EQTP_BF16): parity with the fp64 oracle evaluated on the same bf16 values
(widened exactly), and bit-identity with the fp32 path fed those values."""
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


def test_bf16_features_rejected_where_unsupported():
    eq = _eq()
    wl = synth.small_graph(8, 4, 16, 3, 1200)
    xb, _ = _bf16(wl.x)
    _say("bf16 features unsupported paths")
    with pytest.raises(eq.EqtpError):
        eq.eqtp_conv_fused(_t(wl.vec), _t(wl.src), xb, _t(wl.w), 3, dst=_t(wl.dst))
    with pytest.raises(eq.EqtpError):
        eq.eqtp_conv_fused(_t(wl.vec), _t(wl.src), xb, _t(wl.w), 3, row_ptr=_t(wl.row_ptr), algo=2)

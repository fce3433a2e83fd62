"""eqtp_conv_fused_noalloc (through the C ABI): the workspace path with the
library's static per-device scratch instead of a caller-given workspace must
give the same output as eqtp_conv_fused_ws, bit for bit, on consecutive calls
of decreasing size (the scratch keeps the previous call's contents, so
anything that must start from zero is cleared by the call itself); requests
beyond the scratch are refused before any launch."""
import ctypes

import numpy as np
import pytest

import oracle
from spherical_harmonic_cg_amd import synth
from test_gpu_parity import TOL, _assert_close, _eq, _np, _oracle_full, _say, _t, _wl

pytestmark = pytest.mark.gpu


def _desc(eq, wl, order):
    return eq.eqtp.__dict__["_ConvDesc"](ctypes.sizeof(eq.eqtp._ConvDesc), wl.lmax, wl.C, wl.path_set,
                                         wl.weight_mode, order, 0, float(wl.r_cut), 8, 0)


def test_noalloc_matches_workspace_path_on_shrinking_calls():
    import torch

    eq = _eq()
    lib = eq.load_library()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    for name in ("large", "mid", "typical"):  # each call smaller than the one before
        wl = _wl(name)
        pvec, psrc, pdst = synth.random_permutation(wl, seed=11)
        vec, src, dst, x, w = _t(pvec), _t(psrc), _t(pdst), _t(wl.x), _t(wl.weights)
        _say("noalloc %s E=%d" % (name, wl.E))
        ref = eq.eqtp_conv_fused_ws(vec, src, x, w, wl.lmax, dst=dst, path_set=wl.path_set)
        out = torch.full_like(ref, 7.0)
        d = _desc(eq, wl, eq.EQTP_EDGES_UNSORTED)
        rc = lib.eqtp_conv_fused_noalloc(ctypes.byref(d), wl.N, wl.E, p(vec), p(src), p(dst), None, p(x), p(w),
                                         p(out), stream)
        assert rc == 0, eq.eqtp_status_string(rc)
        got, want = _np(out), _np(ref)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), name + ": differs from the workspace path"
        _assert_close(got, _oracle_full(name), TOL, name + " noalloc")


def test_noalloc_dst_sorted_and_too_large():
    import torch

    eq = _eq()
    lib = eq.load_library()
    wl = synth.small_graph(30, 8, 64, 3, 4100)
    _say("noalloc dst-sorted")
    got = _np(eq.eqtp_conv_fused_noalloc(_t(wl.vec), _t(wl.src), _t(wl.x), _t(wl.w), 3, row_ptr=_t(wl.row_ptr)))
    want = _np(eq.eqtp_conv_fused(_t(wl.vec), _t(wl.src), _t(wl.x), _t(wl.w), 3, row_ptr=_t(wl.row_ptr)))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # 10 million edges in any order need about 200 MB of workspace: refused before anything is read or launched
    d = eq.eqtp._ConvDesc(ctypes.sizeof(eq.eqtp._ConvDesc), 3, 64, 0, 0, eq.EQTP_EDGES_UNSORTED, 0, 0.0, 8, 0)
    fake = ctypes.c_void_p(0x10000)
    assert lib.eqtp_conv_fused_noalloc(ctypes.byref(d), 100000, 10000000, fake, fake, fake, None, fake, fake, fake,
                                       None) == eq.EQTP_ETOOLARGE

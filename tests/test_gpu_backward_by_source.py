"""GPU parity of the gradients from edges grouped by source node
(eqtp_conv_backward_by_source, through the C ABI) in every mode it has:
fixed weights at lmax <= 3 (node-factored adjoint, grad_vec by the edge-frame
walk), fixed weights at lmax 4..6 and radial weights (one walk in each edge's
frame with grad_x summed per source row, no atomics).  Reference: the fp64
oracle's gradients on the same seeded inputs.

Bar: max|gpu - oracle| <= 2e-4 * max|oracle| per gradient tensor; grad_x is
written once per source row, so it is also checked to be bit-identical from
run to run.  The grouping comes from the host (a stable argsort) and from the
GPU sort (eqtp_edge_rows + eqtp_sort_edges, whose order within a source is
not unique: the gradients must not depend on it beyond rounding).
"""
import numpy as np
import pytest

import oracle
from spherical_harmonic_cg_amd import synth
from test_gpu_parity import TOL, _assert_close, _eq, _np, _say, _t

pytestmark = pytest.mark.gpu

RAD = 1  # EQTP_W_RADIAL
SO2 = 3  # EQTP_ALGO_EDGE_SO2


def _gout(wl, seed):
    return np.random.default_rng(seed).standard_normal((wl.N, wl.C, (wl.lmax + 1) ** 2)).astype(np.float32)


def _group_host(wl, vec=None):
    vec = wl.vec if vec is None else vec
    order = np.argsort(wl.src, kind="stable")
    src_ptr = np.concatenate([[0], np.cumsum(np.bincount(wl.src, minlength=wl.N))]).astype(np.int32)
    return _t(src_ptr), _t(vec[order]), _t(wl.dst[order].astype(np.int32)), _t(order.astype(np.int32))


def _group_gpu(eq, wl, vec=None):
    vec = wl.vec if vec is None else vec
    rows = eq.eqtp_edge_rows(_t(wl.row_ptr), wl.src.shape[0])
    src_ptr, perm, vec_s, dst_s = eq.eqtp_sort_edges(_t(wl.src), wl.N, vec=_t(vec), src=rows)
    return src_ptr, vec_s, dst_s, perm


def _run(eq, wl, grp, gout, need=(True, True, True), radial=False, algo=0):
    src_ptr, vec_s, dst_s, perm = grp
    kw = dict(weight_mode=RAD, r_cut=wl.r_cut) if radial else {}
    return eq.eqtp_conv_backward_by_source(vec_s, dst_s, src_ptr, _t(wl.x), _t(wl.w_rad if radial else wl.w),
                                           _t(gout), wl.lmax, path_set=wl.path_set, need_x=need[0], need_w=need[1],
                                           need_vec=need[2], perm=perm if need[2] else None, algo=algo, **kw)


def _ref(wl, gout, radial, vec=None):
    vec = wl.vec if vec is None else vec
    if radial:
        return oracle.conv_backward_radial(wl.N, vec, wl.src, wl.dst, wl.x, wl.w_rad, gout, wl.lmax, wl.r_cut,
                                           wl.path_set)
    return oracle.conv_backward(wl.N, vec, wl.src, wl.dst, wl.x, wl.w, gout, wl.lmax, wl.path_set)


def _compare(got, ref, need, what):
    errs = []
    for g, r, name, want in zip(got, ref, ("grad_x", "grad_w", "grad_vec"), need):
        if not want:
            assert g is None
            continue
        errs.append(_assert_close(_np(g), r, TOL, what + " " + name))
    return errs


@pytest.mark.parametrize("lmax", [0, 1, 2, 3])
@pytest.mark.parametrize("ps", [0, 1])
@pytest.mark.parametrize("C", [16, 64, 128])
def test_radial_by_source_small(lmax, ps, C):
    eq = _eq()
    wl = synth.small_graph(37, 9, C, lmax, 3000 + lmax * 10 + C + ps, path_set=ps, radial=True, r_cut=5.0,
                           empty_rows=(3,), long_rows=(5,), long_len=70, zero_vec_edges=1)
    gout = _gout(wl, 7)
    _say("radial by source lmax=%d ps=%d C=%d E=%d" % (lmax, ps, C, wl.src.shape[0]))
    _compare(_run(eq, wl, _group_host(wl), gout, radial=True), _ref(wl, gout, True), (True, True, True),
             "radial by source L%d ps%d C%d" % (lmax, ps, C))


@pytest.mark.parametrize("L,ps,C", [(4, 0, 32), (4, 1, 128), (5, 1, 16), (6, 0, 64), (6, 1, 8), (5, 0, 128),
                                    (6, 1, 128), (3, 0, 64), (2, 1, 32), (0, 0, 16)])
def test_so2_by_source_small(L, ps, C):
    """Fixed weights in the edge-aligned form (lmax 4..6, and lmax <= 3 with EQTP_ALGO_EDGE_SO2)."""
    eq = _eq()
    wl = synth.small_graph(31, 8, C, L, 3100 + 10 * L + C + ps, path_set=ps, empty_rows=(2,), long_rows=(6,),
                           long_len=70, zero_vec_edges=2)
    wl.vec[3] = (0.0, 0.0, 1.4)
    wl.vec[4] = (0.0, 0.0, -0.8)
    gout = _gout(wl, 8)
    _say("so2 by source L=%d ps=%d C=%d E=%d" % (L, ps, C, wl.src.shape[0]))
    _compare(_run(eq, wl, _group_host(wl), gout, algo=SO2 if L <= 3 else 0), _ref(wl, gout, False),
             (True, True, True), "so2 by source L%d ps%d C%d" % (L, ps, C))


@pytest.mark.parametrize("L,ps,C", [(3, 0, 64), (3, 1, 128), (2, 0, 8), (1, 1, 32)])
def test_fixed_by_source_with_grad_vec(L, ps, C):
    """lmax <= 3, fixed weights: grad_x and grad_w by the node-factored adjoint, grad_vec by the
    edge-frame walk over the same grouped edges, back in the caller's order."""
    eq = _eq()
    wl = synth.small_graph(33, 9, C, L, 3200 + L + C + ps, path_set=ps, empty_rows=(1,), zero_vec_edges=1)
    gout = _gout(wl, 9)
    _say("fixed by source with grad_vec L=%d ps=%d C=%d" % (L, ps, C))
    _compare(_run(eq, wl, _group_host(wl), gout), _ref(wl, gout, False), (True, True, True),
             "fixed by source L%d ps%d C%d" % (L, ps, C))


@pytest.mark.parametrize("radial", [False, True])
@pytest.mark.parametrize("need", [(True, False, False), (False, True, False), (False, False, True),
                                  (True, False, True)])
def test_by_source_partial_requests(radial, need):
    eq = _eq()
    wl = synth.small_graph(23, 8, 32, 3 if radial else 5, 3301, radial=radial, r_cut=5.0)
    gout = _gout(wl, 10)
    _say("by source partial radial=%s need=%s" % (radial, need))
    _compare(_run(eq, wl, _group_host(wl), gout, need=need, radial=radial), _ref(wl, gout, radial), need,
             "by source partial")


@pytest.mark.parametrize("radial", [False, True])
def test_by_source_gpu_grouping_and_determinism(radial):
    """The GPU sort's grouping gives the same gradients (to rounding); grad_x written once per row is
    bit-identical from run to run on one grouping."""
    eq = _eq()
    wl = synth.small_graph(61, 14, 64, 3 if radial else 4, 3401, radial=radial, r_cut=5.0, long_rows=(9,),
                           long_len=120, zero_vec_edges=1)
    gout = _gout(wl, 11)
    _say("by source gpu grouping radial=%s" % radial)
    grp = _group_gpu(eq, wl)
    a = _run(eq, wl, grp, gout, radial=radial)
    _compare(a, _ref(wl, gout, radial), (True, True, True), "by source gpu grouping")
    b = _run(eq, wl, grp, gout, radial=radial)
    assert np.array_equal(_np(a[0]), _np(b[0]))


@pytest.mark.parametrize("radial,L", [(True, 3), (False, 3), (False, 5)])
def test_by_source_stable_grouping_deterministic(radial, L):
    """The stable GPU grouping (eqtp_sort_edges_stable) equals the host's stable argsort exactly, so two
    groupings and backward passes give bit-identical grad_x (summed per source row in the grouped order and
    written once); grad_w and grad_vec, whose partial sums meet in fp32 atomics, agree with the oracle."""
    eq = _eq()
    wl = synth.small_graph(67, 15, 64, L, 3451 + L, radial=radial, r_cut=5.0, long_rows=(5,), long_len=150,
                           zero_vec_edges=1)
    gout = _gout(wl, 13)
    _say("by source stable grouping radial=%s L=%d" % (radial, L))
    runs = []
    for _ in range(2):
        rows = eq.eqtp_edge_rows(_t(wl.row_ptr), wl.src.shape[0])
        src_ptr, perm, vec_s, dst_s = eq.eqtp_sort_edges_stable(_t(wl.src), wl.N, vec=_t(wl.vec), src=rows)
        assert np.array_equal(_np(perm), np.argsort(wl.src, kind="stable").astype(np.int32))
        runs.append(_run(eq, wl, (src_ptr, vec_s, dst_s, perm), gout, radial=radial))
    _compare(runs[0], _ref(wl, gout, radial), (True, True, True), "by source stable grouping")
    assert np.array_equal(_np(runs[0][0]), _np(runs[1][0]))


def test_by_source_no_edges():
    eq = _eq()
    for radial, L in ((True, 3), (False, 5)):
        wl = synth.small_graph(6, 0, 16, L, 3501, radial=radial, r_cut=5.0, empty_rows=range(6))
        gout = _gout(wl, 12)
        _say("by source no edges radial=%s" % radial)
        gx, gw, gv = _run(eq, wl, _group_host(wl), gout, radial=radial)
        assert np.all(_np(gx) == 0.0) and np.all(_np(gw) == 0.0) and _np(gv).shape == (0, 3)


def test_radial_by_source_workload_full():
    """The radial workload (50k atoms, r_c = 5 A, 2.6M edges, L = 3, C = 128) grouped by source on the
    GPU: every entry of the three gradients against the oracle."""
    eq = _eq()
    wl = synth.make_config("radial")
    gout = _gout(wl, 14)
    _say("radial by source radial workload E=%d" % wl.src.shape[0])
    errs = _compare(_run(eq, wl, _group_gpu(eq, wl), gout, radial=True), _ref(wl, gout, True),
                    (True, True, True), "radial workload by source")
    _say("radial workload by source rel errors %s" % (errs,))


@pytest.mark.parametrize("radial,L", [(True, 3), (False, 4), (False, 6)])
def test_autograd_by_source_walk(radial, L):
    """equivariant_conv's default backward for radial weights and above lmax 3: grouped by source,
    all three gradients from one walk."""
    import torch

    eq = _eq()
    from spherical_harmonic_cg_amd.autograd import equivariant_conv

    wl = synth.small_graph(21, 7, 32, L, 3600 + L, radial=radial, r_cut=5.0, zero_vec_edges=1)
    gout = _gout(wl, 16)
    vec = _t(wl.vec).requires_grad_(True)
    x = _t(wl.x).requires_grad_(True)
    w = _t(wl.w_rad if radial else wl.w).requires_grad_(True)
    kw = dict(weight_mode=RAD, r_cut=wl.r_cut) if radial else {}
    _say("autograd by source radial=%s L=%d" % (radial, L))
    out = equivariant_conv(vec, x, w, _t(wl.src), L, row_ptr=_t(wl.row_ptr), **kw)
    (out * _t(gout)).sum().backward()
    torch.cuda.synchronize()
    _compare((x.grad, w.grad, vec.grad), _ref(wl, gout, radial), (True, True, True), "autograd by source")

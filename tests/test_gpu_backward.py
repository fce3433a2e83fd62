"""GPU parity of the convolution's gradients (eqtp_conv_backward, through the
C ABI) against the fp64 oracle's gradients on the same seeded inputs.

Bar: max|gpu - oracle| <= 2e-4 * max|oracle| per gradient tensor (grad_x,
grad_w, grad_vec), as for the forward.
"""
import numpy as np
import pytest

import oracle
from spherical_harmonic_cg_amd import synth
from test_gpu_parity import TOL, _assert_close, _eq, _np, _say, _t

pytestmark = pytest.mark.gpu


def _gout(wl, seed):
    K = (wl.lmax + 1) ** 2
    return np.random.default_rng(seed).standard_normal((wl.N, wl.C, K)).astype(np.float32)


def _check(eq, wl, gout, unsorted=False, perm_seed=2026, need=(True, True, True), what="", algo=0):
    ref = oracle.conv_backward(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w, gout, wl.lmax, wl.path_set)
    if unsorted:
        rng = np.random.default_rng(perm_seed)
        perm = rng.permutation(wl.src.shape[0])
        vec, src, dst = wl.vec[perm], wl.src[perm], wl.dst[perm]
        gx, gw, gv = eq.eqtp_conv_backward(_t(vec), _t(src), _t(wl.x), _t(wl.w), _t(gout), wl.lmax, dst=_t(dst),
                                           path_set=wl.path_set, need_x=need[0], need_w=need[1], need_vec=need[2],
                                           algo=algo)
        inv = np.empty_like(perm)
        inv[perm] = np.arange(perm.shape[0])
        gv_np = _np(gv)[inv] if gv is not None else None
    else:
        gx, gw, gv = eq.eqtp_conv_backward(_t(wl.vec), _t(wl.src), _t(wl.x), _t(wl.w), _t(gout), wl.lmax,
                                           row_ptr=_t(wl.row_ptr), path_set=wl.path_set, need_x=need[0],
                                           need_w=need[1], need_vec=need[2], algo=algo)
        gv_np = _np(gv) if gv is not None else None
    for got, r, name, want in ((gx, ref[0], "grad_x", need[0]), (gw, ref[1], "grad_w", need[1]),
                               (gv_np, ref[2], "grad_vec", need[2])):
        if not want:
            assert got is None
            continue
        got = got if isinstance(got, np.ndarray) else _np(got)
        _assert_close(got, r, TOL, what + " " + name)


# algo 0: the default (the edge-aligned form when grad_x or grad_w is wanted); 1: the coupling walk with
# grad_vec on the matrix cores
@pytest.mark.parametrize("algo", [0, 1])
@pytest.mark.parametrize("lmax", [0, 1, 2, 3])
@pytest.mark.parametrize("ps", [0, 1])
@pytest.mark.parametrize("C", [8, 16, 32, 64, 128])
def test_backward_small_sorted(lmax, ps, C, algo):
    eq = _eq()
    wl = synth.small_graph(37, 9, C, lmax, 300 + lmax * 10 + C, path_set=ps, empty_rows=(3,), long_rows=(5,),
                           long_len=70, zero_vec_edges=1)
    _say("backward sorted lmax=%d ps=%d C=%d algo=%d E=%d" % (lmax, ps, C, algo, wl.src.shape[0]))
    _check(eq, wl, _gout(wl, 7), what="sorted L%d ps%d C%d algo%d" % (lmax, ps, C, algo), algo=algo)


@pytest.mark.parametrize("algo", [0, 1])
@pytest.mark.parametrize("lmax,ps,C", [(3, 0, 64), (3, 1, 32), (2, 0, 8), (1, 0, 128), (3, 0, 128)])
def test_backward_small_unsorted(lmax, ps, C, algo):
    eq = _eq()
    wl = synth.small_graph(41, 10, C, lmax, 500 + lmax + C, path_set=ps, empty_rows=(0,), zero_vec_edges=2)
    _say("backward unsorted lmax=%d ps=%d C=%d algo=%d E=%d" % (lmax, ps, C, algo, wl.src.shape[0]))
    _check(eq, wl, _gout(wl, 8), unsorted=True, what="unsorted L%d ps%d C%d algo%d" % (lmax, ps, C, algo),
           algo=algo)


@pytest.mark.parametrize("need", [(True, False, False), (False, True, False), (False, False, True),
                                  (True, False, True)])
@pytest.mark.parametrize("lmax,unsorted", [(3, False), (1, False), (2, True)])
def test_backward_partial_requests(need, lmax, unsorted):
    """Each subset of outputs under the default algorithm (grad_vec alone goes to the coupling walk)."""
    eq = _eq()
    wl = synth.small_graph(23, 8, 32, lmax, 77 + lmax)
    _say("backward partial %s lmax=%d unsorted=%s" % (need, lmax, unsorted))
    _check(eq, wl, _gout(wl, 9), unsorted=unsorted, need=need, what="partial L%d" % lmax)


def test_backward_typical_workload():
    eq = _eq()
    wl = synth.make_config("typical")
    _say("backward typical E=%d" % wl.src.shape[0])
    _check(eq, wl, _gout(wl, 10), what="typical")


def test_backward_zero_length_edges_give_zero_grad_vec():
    eq = _eq()
    wl = synth.small_graph(12, 6, 16, 3, 88, zero_vec_edges=4)
    _say("backward zero-length edges")
    _, _, gv = eq.eqtp_conv_backward(_t(wl.vec), _t(wl.src), _t(wl.x), _t(wl.w), _t(_gout(wl, 11)), 3,
                                     row_ptr=_t(wl.row_ptr))
    assert np.all(_np(gv)[:4] == 0.0)


def test_backward_no_edges():
    eq = _eq()
    import torch

    N, C = 5, 16
    x = torch.randn(N, C, 16, device="cuda")
    w = torch.randn(23, C, device="cuda")
    g = torch.randn(N, C, 16, device="cuda")
    rp = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
    vec = torch.zeros(0, 3, device="cuda")
    src = torch.zeros(0, dtype=torch.int32, device="cuda")
    _say("backward no edges")
    gx, gw, gv = eq.eqtp_conv_backward(vec, src, x, w, g, 3, row_ptr=rp)
    assert float(_np(gx).__abs__().max()) == 0.0 and float(_np(gw).__abs__().max()) == 0.0
    assert gv.shape == (0, 3)


def test_autograd_function_matches_backward_and_oracle():
    import torch

    eq = _eq()
    from spherical_harmonic_cg_amd.autograd import equivariant_conv

    wl = synth.small_graph(19, 7, 32, 3, 99, zero_vec_edges=1)
    gout = _gout(wl, 12)
    vec = _t(wl.vec).requires_grad_(True)
    x = _t(wl.x).requires_grad_(True)
    w = _t(wl.w).requires_grad_(True)
    _say("autograd function")
    out = equivariant_conv(vec, x, w, _t(wl.src), 3, row_ptr=_t(wl.row_ptr))
    ref_out = oracle.conv(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w, 3)
    _assert_close(_np(out.detach()), ref_out, TOL, "autograd forward")
    (out * _t(gout)).sum().backward()
    ref = oracle.conv_backward(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w, gout, 3)
    _assert_close(_np(x.grad), ref[0], TOL, "autograd grad_x")
    _assert_close(_np(w.grad), ref[1], TOL, "autograd grad_w")
    _assert_close(_np(vec.grad), ref[2], TOL, "autograd grad_vec")
    # only the edge vectors (forces)
    vec2 = _t(wl.vec).requires_grad_(True)
    out2 = equivariant_conv(vec2, _t(wl.x), _t(wl.w), _t(wl.src), 3, row_ptr=_t(wl.row_ptr))
    (out2 * _t(gout)).sum().backward()
    _assert_close(_np(vec2.grad), ref[2], TOL, "autograd grad_vec only")


# ---------------------------------------------------------------------------
# grad_x and grad_w from the edges grouped by source (eqtp_conv_backward_by_source)
# ---------------------------------------------------------------------------

def _by_source_numpy(wl):
    """Source grouping built on the host (stable order), as test input."""
    order = np.argsort(wl.src, kind="stable")
    src_ptr = np.concatenate([[0], np.cumsum(np.bincount(wl.src, minlength=wl.N))]).astype(np.int32)
    return src_ptr, wl.vec[order], wl.dst[order].astype(np.int32)


def _check_by_source(eq, wl, gout, grouping, need=(True, True), what=""):
    ref = oracle.conv_backward(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w, gout, wl.lmax, wl.path_set)
    sp, vs, ds = grouping
    gx, gw, _ = eq.eqtp_conv_backward_by_source(vs if not isinstance(vs, np.ndarray) else _t(vs),
                                             ds if not isinstance(ds, np.ndarray) else _t(ds),
                                             sp if not isinstance(sp, np.ndarray) else _t(sp),
                                             _t(wl.x), _t(wl.w), _t(gout), wl.lmax, path_set=wl.path_set,
                                             need_x=need[0], need_w=need[1])
    if need[0]:
        _assert_close(_np(gx), ref[0], TOL, what + " grad_x")
    else:
        assert gx is None
    if need[1]:
        _assert_close(_np(gw), ref[1], TOL, what + " grad_w")
    else:
        assert gw is None


@pytest.mark.parametrize("lmax", [0, 1, 2, 3])
@pytest.mark.parametrize("ps", [0, 1])
@pytest.mark.parametrize("C", [8, 16, 32, 64, 128])
def test_backward_by_source_small(lmax, ps, C):
    eq = _eq()
    wl = synth.small_graph(37, 9, C, lmax, 900 + lmax * 10 + C, path_set=ps, empty_rows=(3,), long_rows=(5,),
                           long_len=70, zero_vec_edges=1)
    # a source with many outgoing edges (> 64: several staging chunks) and one with none
    wl.src[: 80] = 11
    wl.src[wl.src == 2] = 12
    _say("backward by source lmax=%d ps=%d C=%d E=%d" % (lmax, ps, C, wl.src.shape[0]))
    _check_by_source(eq, wl, _gout(wl, 17), _by_source_numpy(wl), what="by source L%d ps%d C%d" % (lmax, ps, C))


@pytest.mark.parametrize("need", [(True, False), (False, True)])
def test_backward_by_source_partial(need):
    eq = _eq()
    wl = synth.small_graph(23, 8, 32, 3, 78)
    _say("backward by source partial %s" % (need,))
    _check_by_source(eq, wl, _gout(wl, 18), _by_source_numpy(wl), need=need, what="by source partial")


@pytest.mark.parametrize("from_rows", [True, False])
def test_backward_by_source_gpu_grouping(from_rows):
    """Grouping built on the GPU: eqtp_edge_rows (from the dst-sorted CSR) or
    the dst array, then eqtp_sort_edges keyed by source."""
    eq = _eq()
    from spherical_harmonic_cg_amd.autograd import group_by_source

    wl = synth.make_config("typical")
    _say("backward by source, GPU grouping (from_rows=%s) E=%d" % (from_rows, wl.src.shape[0]))
    if from_rows:
        rows = eq.eqtp_edge_rows(_t(wl.row_ptr), wl.src.shape[0])
        assert np.array_equal(_np(rows), wl.dst)
        grouping = group_by_source(wl.N, _t(wl.src), _t(wl.vec), row_ptr=_t(wl.row_ptr))
    else:
        grouping = group_by_source(wl.N, _t(wl.src), _t(wl.vec), dst=_t(wl.dst))
    _check_by_source(eq, wl, _gout(wl, 19), grouping, what="by source typical")


def test_backward_by_source_mid():
    eq = _eq()
    from spherical_harmonic_cg_amd.autograd import group_by_source

    wl = synth.make_config("mid")
    _say("backward by source mid E=%d" % wl.src.shape[0])
    grouping = group_by_source(wl.N, _t(wl.src), _t(wl.vec), row_ptr=_t(wl.row_ptr))
    _check_by_source(eq, wl, _gout(wl, 20), grouping, what="by source mid")


def test_backward_by_source_no_edges():
    eq = _eq()
    import torch

    N, C = 6, 32
    g = torch.randn(N, C, 16, device="cuda")
    x = torch.randn(N, C, 16, device="cuda")
    w = torch.randn(23, C, device="cuda")
    _say("backward by source, no edges")
    gx, gw, _ = eq.eqtp_conv_backward_by_source(torch.zeros(0, 3, device="cuda"),
                                             torch.zeros(0, dtype=torch.int32, device="cuda"),
                                             torch.zeros(N + 1, dtype=torch.int32, device="cuda"), x, w, g, 3)
    assert float(_np(gx).__abs__().max()) == 0.0 and float(_np(gw).__abs__().max()) == 0.0


def test_edge_rows_exact():
    eq = _eq()
    wl = synth.small_graph(300, 7, 8, 1, 5, empty_rows=(0, 17, 299), long_rows=(40,), long_len=200)
    _say("edge rows")
    assert np.array_equal(_np(eq.eqtp_edge_rows(_t(wl.row_ptr), wl.src.shape[0])), wl.dst)


@pytest.mark.parametrize("mode", ["by_source", "edge"])
@pytest.mark.parametrize("csr", [True, False])
def test_autograd_modes(mode, csr):
    import torch

    eq = _eq()
    from spherical_harmonic_cg_amd.autograd import equivariant_conv

    wl = synth.small_graph(29, 9, 64, 3, 123, zero_vec_edges=1)
    gout = _gout(wl, 21)
    kw = dict(row_ptr=_t(wl.row_ptr)) if csr else dict(dst=_t(wl.dst))
    vec = _t(wl.vec).requires_grad_(True)
    x = _t(wl.x).requires_grad_(True)
    w = _t(wl.w).requires_grad_(True)
    _say("autograd mode=%s csr=%s" % (mode, csr))
    out = equivariant_conv(vec, x, w, _t(wl.src), 3, grad_x_mode=mode, **kw)
    (out * _t(gout)).sum().backward()
    ref = oracle.conv_backward(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w, gout, 3)
    _assert_close(_np(x.grad), ref[0], TOL, "autograd %s grad_x" % mode)
    _assert_close(_np(w.grad), ref[1], TOL, "autograd %s grad_w" % mode)
    _assert_close(_np(vec.grad), ref[2], TOL, "autograd %s grad_vec" % mode)


@pytest.mark.parametrize("lmax,ps,C", [(3, 0, 64), (3, 1, 128), (2, 0, 16), (1, 1, 8), (0, 0, 32), (3, 0, 8)])
def test_grad_vec_both_walks(lmax, ps, C):
    """grad_vec alone of dst-sorted edges: the default (the vector-ALU walk below lmax 3,
    the matrix cores at 3), the matrix-core kernel (algo = NODE_MFMA), the vector-ALU walk
    (algo = EDGE_VALU) and the edge-aligned form (algo = EDGE_SO2), all against the oracle;
    rows longer than 64 edges (several chunks) and empty rows included."""
    eq = _eq()
    wl = synth.small_graph(31, 12, C, lmax, 610 + lmax + C + ps, path_set=ps, empty_rows=(1, 2), long_rows=(7, 8),
                           long_len=150, zero_vec_edges=2)
    gout = _gout(wl, 33)
    ref = oracle.conv_backward(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w, gout, lmax, ps)[2]
    for algo in (0, 1, 2, 3):
        _say("grad_vec walk algo=%d lmax=%d ps=%d C=%d" % (algo, lmax, ps, C))
        _, _, gv = eq.eqtp_conv_backward(_t(wl.vec), _t(wl.src), _t(wl.x), _t(wl.w), _t(gout), lmax,
                                         row_ptr=_t(wl.row_ptr), path_set=ps, need_x=False, need_w=False,
                                         algo=algo)
        _assert_close(_np(gv), ref, TOL, "grad_vec algo %d" % algo)


def test_grad_vec_mid_workload():
    eq = _eq()
    wl = synth.make_config("mid")
    gout = _gout(wl, 34)
    _say("grad_vec mid E=%d" % wl.src.shape[0])
    ref = oracle.conv_backward(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w, gout, 3)[2]
    for algo in (0, 1):
        _, _, gv = eq.eqtp_conv_backward(_t(wl.vec), _t(wl.src), _t(wl.x), _t(wl.w), _t(gout), 3,
                                         row_ptr=_t(wl.row_ptr), need_x=False, need_w=False, algo=algo)
        _assert_close(_np(gv), ref, TOL, "grad_vec mid algo %d" % algo)

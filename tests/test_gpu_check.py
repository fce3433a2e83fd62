"""GPU tests of the graph checks (eqtp_check_graph) and of debug mode
(eqtp_set_debug): the report is compared word for word with a plain numpy
statement of the same checks on the same arrays, for clean graphs, for faults
planted at chosen and at random places (many workgroups, so the counts and
first indices go through the kernel's cross-wave reduction), and for the
degenerate sizes.  In debug mode every entry point that takes a graph refuses
a faulty one with EQTP_EGRAPH before launching anything (its output buffer is
left as it was) and gives bit-identical results on a clean one.

The faulty arrays are only ever given to the check itself or to an entry
point in debug mode, which stops before its kernels run."""
import numpy as np
import pytest

from spherical_harmonic_cg_amd import synth
from test_gpu_parity import _eq, _np, _say, _t

pytestmark = pytest.mark.gpu


def _expected(N, E, row_ptr=None, src=None, dst=None, vec=None):
    """The report's definition (include/eqtp.h, eqtp_check_graph), written out with numpy."""
    rep = np.zeros(8, dtype=np.int64)
    bad_e = np.zeros(E, dtype=bool)
    if E > 0 and src is not None:
        b = (src < 0) | (src >= N)
        rep[0] = b.sum()
        bad_e |= b
    if E > 0 and dst is not None:
        b = (dst < 0) | (dst >= N)
        rep[1] = b.sum()
        bad_e |= b
        if row_ptr is not None and N > 0:
            # row of edge e: the largest r in [0, N) with row_ptr[r] <= e (rows monotone here)
            r = np.maximum(np.searchsorted(row_ptr[:N], np.arange(E), side="right") - 1, 0)
            b = dst != r
            rep[4] = b.sum()
            bad_e |= b
    if E > 0 and vec is not None:
        b = ~np.isfinite(vec).all(axis=1)
        rep[5] = b.sum()
        bad_e |= b
    rep[6] = int(np.flatnonzero(bad_e)[0]) if bad_e.any() else -1
    rep[7] = -1
    if row_ptr is not None:
        dec = np.flatnonzero(row_ptr[1:N + 1] < row_ptr[:N])
        rep[2] = dec.size
        rep[7] = int(dec[0]) if dec.size else -1
        rep[3] = int(row_ptr[0] != 0) + int(row_ptr[N] != E)
    return rep.astype(np.int32)


def _report(eq, N, E, row_ptr=None, src=None, dst=None, vec=None):
    g = lambda a: None if a is None else _t(a)
    return _np(eq.eqtp_check_graph(N, E, row_ptr=g(row_ptr), src=g(src), dst=g(dst), vec=g(vec)))


def _both(eq, what, N, E, **arrs):
    _say("check graph: %s N=%d E=%d" % (what, N, E))
    got = _report(eq, N, E, **arrs)
    want = _expected(N, E, **arrs)
    np.testing.assert_array_equal(got, want, err_msg=what)
    return got


@pytest.mark.parametrize("name", ["tiny", "mid"])
def test_clean_workloads(name):
    eq = _eq()
    wl = synth.make_config(name)
    got = _both(eq, "clean " + name, wl.N, wl.E, row_ptr=wl.row_ptr, src=wl.src, dst=wl.dst, vec=wl.vec)
    np.testing.assert_array_equal(got, [0, 0, 0, 0, 0, 0, -1, -1])


def test_planted_faults_one_at_a_time():
    eq = _eq()
    wl = synth.small_graph(53, 9, 16, 2, 4101, empty_rows=(0, 7, 52), long_rows=(11,), long_len=90)
    N, E = wl.N, wl.E
    base = dict(row_ptr=wl.row_ptr, src=wl.src, dst=wl.dst, vec=wl.vec)

    def case(what, **over):
        arrs = {k: (v.copy() if v is not None else None) for k, v in base.items()}
        for k, f in over.items():
            if callable(f):
                f(arrs[k])
            else:
                arrs[k] = f
        got = _both(eq, what, N, E, **arrs)
        assert got[:6].any(), what  # every planted fault is seen

    case("src = N", src=lambda a: a.__setitem__(17, N))
    case("src negative at 0 and E-1", src=lambda a: (a.__setitem__(0, -1), a.__setitem__(E - 1, -5)))
    case("dst out of range", dst=lambda a: a.__setitem__(40, N + 3))
    case("dst in the wrong row", dst=lambda a: a.__setitem__(60, (a[60] + 1) % N))
    case("NaN vector", vec=lambda a: a.__setitem__((33, 1), np.nan))
    case("inf vector", vec=lambda a: a.__setitem__((E - 1, 2), np.inf))
    case("row_ptr[0] != 0", row_ptr=lambda a: a.__setitem__(0, 1), dst=None)
    case("row_ptr[N] != E", row_ptr=lambda a: a.__setitem__(N, E - 1), dst=None)

    def dec(a):
        a[20] = a[21] + 2
    case("row_ptr decreasing", row_ptr=dec, dst=None)


def test_random_faults_on_the_mid_graph():
    """Faults at 1,000 random places of a 266 k-edge graph: exact counts and first indices."""
    eq = _eq()
    wl = synth.make_config("mid")
    N, E = wl.N, wl.E
    rng = np.random.default_rng(4102)
    src = wl.src.copy()
    src[rng.choice(E, 400, replace=False)] = rng.integers(N, 2 * N, 400)
    dst = wl.dst.copy()
    dst[rng.choice(E, 300, replace=False)] = rng.integers(-N, 0, 300)
    vec = wl.vec.copy()
    vec[rng.choice(E, 300, replace=False), rng.integers(0, 3, 300)] = np.nan
    got = _both(eq, "random faults", N, E, row_ptr=wl.row_ptr, src=src, dst=dst, vec=vec)
    assert got[0] == 400 and got[1] == 300
    rp = wl.row_ptr.copy()
    rows = rng.choice(np.arange(1, N - 1), 50, replace=False)
    rp[rows] = rp[rows + 1] + 1  # each makes row_ptr drop right after
    _both(eq, "random decreasing rows", N, E, row_ptr=rp, src=wl.src)


def test_degenerate_sizes():
    eq = _eq()
    _both(eq, "no nodes, no edges", 0, 0, row_ptr=np.zeros(1, np.int32))
    _both(eq, "no edges", 5, 0, row_ptr=np.zeros(6, np.int32))
    _both(eq, "no edges, bad end", 5, 0, row_ptr=np.array([0, 0, 1, 1, 1, 1], np.int32))
    _both(eq, "one node", 1, 3, row_ptr=np.array([0, 3], np.int32), src=np.zeros(3, np.int32),
          dst=np.zeros(3, np.int32), vec=np.ones((3, 3), np.float32))
    _both(eq, "src only", 4, 6, src=np.array([0, 1, 2, 3, 4, -1], np.int32))
    _both(eq, "nothing given", 4, 6)


def _conv_setup(wl):
    import torch

    out = torch.full((wl.N, wl.C, (wl.lmax + 1) ** 2), 7.25, dtype=torch.float32, device="cuda")
    return out


def test_debug_mode_refuses_faulty_graphs():
    import torch

    eq = _eq()
    wl = synth.small_graph(41, 8, 32, 3, 4103, empty_rows=(4,))
    bad_src = wl.src.copy()
    bad_src[5] = wl.N
    bad_rp = wl.row_ptr.copy()
    bad_rp[-1] = wl.E + 1
    was = eq.eqtp_set_debug(True)
    try:
        _say("debug mode: fused conv with src out of range")
        out = _conv_setup(wl)
        with pytest.raises(eq.EqtpError) as ei:
            eq.eqtp_conv_fused(_t(wl.vec), _t(bad_src), _t(wl.x), _t(wl.w), wl.lmax, row_ptr=_t(wl.row_ptr), out=out)
        assert ei.value.status == eq.EQTP_EGRAPH
        assert bool((out == 7.25).all())
        _say("debug mode: fused conv with a bad row_ptr end")
        with pytest.raises(eq.EqtpError) as ei:
            eq.eqtp_conv_fused(_t(wl.vec), _t(wl.src), _t(wl.x), _t(wl.w), wl.lmax, row_ptr=_t(bad_rp), out=out)
        assert ei.value.status == eq.EQTP_EGRAPH and bool((out == 7.25).all())
        _say("debug mode: unsorted edges with dst out of range (atomic path and workspace path)")
        bad_dst = wl.dst.copy()
        bad_dst[9] = -2
        for fn in (eq.eqtp_conv_fused, eq.eqtp_conv_fused_ws):
            with pytest.raises(eq.EqtpError) as ei:
                fn(_t(wl.vec), _t(wl.src), _t(wl.x), _t(wl.w), wl.lmax, dst=_t(bad_dst), out=out)
            assert ei.value.status == eq.EQTP_EGRAPH and bool((out == 7.25).all())
        _say("debug mode: backward and messages with a NaN vector")
        bad_vec = wl.vec.copy()
        bad_vec[3, 0] = np.nan
        gout = _t(np.ones((wl.N, wl.C, 16), np.float32))
        with pytest.raises(eq.EqtpError) as ei:
            eq.eqtp_conv_backward(_t(bad_vec), _t(wl.src), _t(wl.x), _t(wl.w), gout, wl.lmax,
                                  row_ptr=_t(wl.row_ptr))
        assert ei.value.status == eq.EQTP_EGRAPH
        with pytest.raises(eq.EqtpError) as ei:
            eq.eqtp_conv_messages(_t(bad_vec), _t(wl.src), _t(wl.x), _t(wl.w), wl.lmax)
        assert ei.value.status == eq.EQTP_EGRAPH
        _say("debug mode: source-grouped gradients with perm out of range")
        order = np.argsort(wl.src, kind="stable")
        src_ptr = np.concatenate([[0], np.cumsum(np.bincount(wl.src, minlength=wl.N))]).astype(np.int32)
        perm = order.astype(np.int32)
        perm[2] = wl.E
        with pytest.raises(eq.EqtpError) as ei:
            eq.eqtp_conv_backward_by_source(_t(wl.vec[order]), _t(wl.dst[order].astype(np.int32)), _t(src_ptr),
                                            _t(wl.x), _t(wl.w), gout, wl.lmax, need_vec=True, perm=_t(perm))
        assert ei.value.status == eq.EQTP_EGRAPH
        _say("debug mode: edge grouping with dst out of range")
        with pytest.raises(eq.EqtpError) as ei:
            eq.eqtp_sort_edges(_t(bad_dst), wl.N)
        assert ei.value.status == eq.EQTP_EGRAPH
        torch.cuda.synchronize()
    finally:
        eq.eqtp_set_debug(was)


def test_debug_mode_same_results_on_clean_graphs():
    eq = _eq()
    wl = synth.small_graph(47, 10, 64, 3, 4104, empty_rows=(3,), long_rows=(8,), long_len=80)
    _say("debug mode: clean graph, results with and without")
    args = (_t(wl.vec), _t(wl.src), _t(wl.x), _t(wl.w), wl.lmax)
    ref = _np(eq.eqtp_conv_fused(*args, row_ptr=_t(wl.row_ptr)))
    ref_u = _np(eq.eqtp_conv_fused_ws(*args, dst=_t(wl.dst)))
    was = eq.eqtp_set_debug(True)
    try:
        got = _np(eq.eqtp_conv_fused(*args, row_ptr=_t(wl.row_ptr)))
        got_u = _np(eq.eqtp_conv_fused_ws(*args, dst=_t(wl.dst)))
    finally:
        eq.eqtp_set_debug(was)
    assert np.array_equal(got, ref) and np.array_equal(got_u, ref_u)


def test_debug_mode_other_entry_points():
    """Debug mode in the interaction layer, eqtp_edge_rows, eqtp_sort_edges_stable and
    eqtp_conv_fused_noalloc: a faulty graph is refused with EQTP_EGRAPH and nothing written."""
    import torch

    eq = _eq()
    wl = synth.small_graph(39, 8, 32, 3, 4105, empty_rows=(6,))
    iw = synth.interaction_weights(3, 32)
    bad_src = wl.src.copy()
    bad_src[11] = wl.N + 4
    bad_rp = wl.row_ptr.copy()
    bad_rp[10] = bad_rp[11] + 1  # decreasing
    was = eq.eqtp_set_debug(True)
    try:
        _say("debug mode: interaction layer with src out of range")
        out = torch.full((wl.N, 32, 16), 3.5, dtype=torch.float32, device="cuda")
        with pytest.raises(eq.EqtpError) as ei:
            eq.eqtp_interaction(_t(wl.vec), _t(bad_src), _t(wl.row_ptr), _t(wl.x), _t(iw.W_up), _t(iw.W1),
                                _t(iw.W2), _t(iw.W3), _t(iw.W_out), 3, r_cut=5.0, norm=8.0, out=out)
        assert ei.value.status == eq.EQTP_EGRAPH and bool((out == 3.5).all())
        _say("debug mode: edge rows with a decreasing row_ptr")
        rows = torch.full((wl.E,), -7, dtype=torch.int32, device="cuda")
        with pytest.raises(eq.EqtpError) as ei:
            eq.eqtp_edge_rows(_t(bad_rp), wl.E, out=rows)
        assert ei.value.status == eq.EQTP_EGRAPH and bool((rows == -7).all())
        _say("debug mode: stable sort with a key out of range")
        bad_dst = wl.dst.copy()
        bad_dst[0] = -1
        with pytest.raises(eq.EqtpError) as ei:
            eq.eqtp_sort_edges_stable(_t(bad_dst), wl.N)
        assert ei.value.status == eq.EQTP_EGRAPH
        _say("debug mode: no-alloc convolution with a NaN vector")
        bad_vec = wl.vec.copy()
        bad_vec[2, 1] = np.inf
        out2 = torch.full((wl.N, 32, 16), 1.25, dtype=torch.float32, device="cuda")
        with pytest.raises(eq.EqtpError) as ei:
            eq.eqtp_conv_fused_noalloc(_t(bad_vec), _t(wl.src), _t(wl.x), _t(wl.w), 3, dst=_t(wl.dst), out=out2)
        assert ei.value.status == eq.EQTP_EGRAPH and bool((out2 == 1.25).all())
        _say("debug mode: the same calls on the clean graph succeed")
        eq.eqtp_interaction(_t(wl.vec), _t(wl.src), _t(wl.row_ptr), _t(wl.x), _t(iw.W_up), _t(iw.W1), _t(iw.W2),
                            _t(iw.W3), _t(iw.W_out), 3, r_cut=5.0, norm=8.0, out=out)
        eq.eqtp_edge_rows(_t(wl.row_ptr), wl.E, out=rows)
        eq.eqtp_sort_edges_stable(_t(wl.dst), wl.N)
        eq.eqtp_conv_fused_noalloc(_t(wl.vec), _t(wl.src), _t(wl.x), _t(wl.w), 3, dst=_t(wl.dst), out=out2)
        torch.cuda.synchronize()
        assert np.array_equal(_np(rows), wl.dst.astype(np.int32))
    finally:
        eq.eqtp_set_debug(was)

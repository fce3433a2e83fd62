"""GPU counting sort of edges by destination (eqtp_sort_edges, through the C
ABI) and the dst-sorted convolution run on its output.

Unique results are compared exactly: row_ptr against numpy's bincount +
cumsum, and vec[perm] / src[perm] against numpy gathers with the GPU's perm.
The order of edges inside a row is not unique (it follows the hardware
atomics), so perm is checked for validity: a permutation of 0..E-1 that puts
row n's edges, and only those, in [row_ptr[n], row_ptr[n+1]).  The
convolution on the sorted edges is compared with the fp64 oracle on the
original order to the usual 2e-4 * max|oracle| bar.
"""
import numpy as np
import pytest

import oracle
from spherical_harmonic_cg_amd import synth
from test_gpu_parity import TOL, _assert_close, _eq, _np, _oracle_full, _say, _t, _wl

pytestmark = pytest.mark.gpu


def _check_sort(eq, N, dst, vec=None, src=None):
    E = dst.shape[0]
    rp, perm, vs, ss = eq.eqtp_sort_edges(_t(dst), N, vec=_t(vec) if vec is not None else None,
                                         src=_t(src) if src is not None else None)
    rp, perm = _np(rp), _np(perm)
    want_rp = np.concatenate([[0], np.cumsum(np.bincount(dst, minlength=N))]).astype(np.int32)
    assert rp.dtype == np.int32 and np.array_equal(rp, want_rp), "row_ptr differs"
    assert perm.shape == (E,)
    assert np.array_equal(np.sort(perm), np.arange(E, dtype=np.int32)), "perm is not a permutation"
    deg = np.diff(want_rp)
    assert np.array_equal(dst[perm], np.repeat(np.arange(N, dtype=np.int32), deg)), "rows hold foreign edges"
    if vec is not None:
        assert np.array_equal(_np(vs), vec[perm])
    if src is not None:
        assert np.array_equal(_np(ss), src[perm])
    return rp, perm, vs, ss


@pytest.mark.parametrize("N,E,seed", [(1, 1, 0), (1, 500, 1), (7, 3, 2), (100, 1000, 3), (1023, 5000, 4),
                                      (1024, 4096, 5), (1025, 777, 6), (5000, 2, 7), (40000, 300001, 8)])
def test_sort_random_destinations(N, E, seed):
    eq = _eq()
    rng = np.random.default_rng(seed)
    dst = rng.integers(0, N, size=E).astype(np.int32)
    vec = rng.standard_normal((E, 3)).astype(np.float32)
    src = rng.integers(0, N, size=E).astype(np.int32)
    _say("sort N=%d E=%d" % (N, E))
    _check_sort(eq, N, dst, vec, src)


def test_sort_skewed_rows():
    """One hot row with half the edges, many empty rows, first and last rows used."""
    eq = _eq()
    rng = np.random.default_rng(11)
    N, E = 3000, 60000
    dst = np.where(rng.random(E) < 0.5, 1234, rng.integers(0, N, size=E) // 7 * 7).astype(np.int32)
    dst[:2] = (0, N - 1)
    _say("sort skewed N=%d E=%d" % (N, E))
    _check_sort(eq, N, dst, rng.standard_normal((E, 3)).astype(np.float32), rng.integers(0, N, E).astype(np.int32))


def test_sort_without_vec_and_src():
    eq = _eq()
    dst = np.random.default_rng(12).integers(0, 50, size=999).astype(np.int32)
    _say("sort perm only")
    _, _, vs, ss = _check_sort(eq, 50, dst)
    assert vs is None and ss is None


def test_sort_no_edges():
    eq = _eq()
    import torch

    _say("sort no edges")
    for N in (0, 1, 5000):
        rp, perm, _, _ = eq.eqtp_sort_edges(torch.zeros(0, dtype=torch.int32, device="cuda"), N)
        assert np.array_equal(_np(rp), np.zeros(N + 1, dtype=np.int32)) and perm.numel() == 0


def test_sort_repeated_calls_reuse_outputs():
    """The outputs double as the counters: a second call into the same buffers,
    on different edges, must not see the first call's values."""
    eq = _eq()
    rng = np.random.default_rng(13)
    N = 300
    d1 = rng.integers(0, N, size=4000).astype(np.int32)
    d2 = rng.integers(0, N // 2, size=4000).astype(np.int32)
    _say("sort repeated")
    rp, perm, _, _ = eq.eqtp_sort_edges(_t(d1), N)
    eq.eqtp_sort_edges(_t(d2), N, out=(rp, perm, None, None))
    rp, perm = _np(rp), _np(perm)
    assert np.array_equal(rp, np.concatenate([[0], np.cumsum(np.bincount(d2, minlength=N))]))
    assert np.array_equal(d2[perm], np.sort(d2))


@pytest.mark.parametrize("lmax,ps,C", [(3, 0, 64), (3, 1, 32), (2, 0, 16), (1, 0, 128), (0, 0, 8)])
def test_sort_then_conv_small(lmax, ps, C):
    eq = _eq()
    wl = synth.small_graph(57, 11, C, lmax, 700 + lmax + C, path_set=ps, empty_rows=(0, 9), long_rows=(4,),
                           long_len=90, zero_vec_edges=2)
    pvec, psrc, pdst = synth.random_permutation(wl, seed=5)
    _say("sort+conv lmax=%d ps=%d C=%d E=%d" % (lmax, ps, C, wl.E))
    rp, _, vs, ss = _check_sort(eq, wl.N, pdst, pvec, psrc)
    out = eq.eqtp_conv_fused(vs, ss, _t(wl.x), _t(wl.w), lmax, row_ptr=_t(rp), path_set=ps)
    ref = oracle.conv(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w, lmax, path_set=ps)
    _assert_close(_np(out), ref, TOL, "sort+conv")


@pytest.mark.parametrize("name", ["mid", "large"])
def test_sort_then_conv_workload(name):
    """Full-size workloads in random edge order: sort exact, conv on every row against the oracle."""
    eq = _eq()
    wl = _wl(name)
    pvec, psrc, pdst = synth.random_permutation(wl)
    _say("sort+conv %s E=%d" % (name, wl.E))
    rp, _, vs, ss = _check_sort(eq, wl.N, pdst, pvec, psrc)
    assert np.array_equal(rp, wl.row_ptr)
    out = _np(eq.eqtp_conv_fused(vs, ss, _t(wl.x), _t(wl.weights), wl.lmax, row_ptr=_t(rp), path_set=wl.path_set,
                                 weight_mode=wl.weight_mode, r_cut=wl.r_cut))
    _assert_close(out, _oracle_full(name), TOL, name + " sort+conv")


# ----------------------------------------------------------------------------
# eqtp_conv_fused_ws: edges in any order, grouped in a workspace (rows in input
# order), then the dst-sorted kernels
# ----------------------------------------------------------------------------

def _interleave_rows(wl, seed):
    """A random interleaving of the rows that keeps every row's edges in their sorted order: the grouping
    must then give back exactly the dst-sorted edge list."""
    rng = np.random.default_rng(seed)
    pos = rng.permutation(wl.E)             # edge i of the sorted list would land at pos[i] ...
    order = np.empty(wl.E, dtype=np.int64)
    for r in range(wl.N):                    # ... but each row's slots are refilled in sorted order
        b, e = wl.row_ptr[r], wl.row_ptr[r + 1]
        order[np.sort(pos[b:e])] = np.arange(b, e)
    return wl.vec[order].copy(), wl.src[order].copy(), wl.dst[order].copy()


@pytest.mark.parametrize("C,L,radial", [(8, 2, False), (16, 1, False), (32, 3, False), (64, 3, False),
                                        (128, 3, False), (64, 0, False), (32, 3, True), (128, 3, True),
                                        (8, 2, True)])
def test_conv_ws_matches_sorted_bitwise(C, L, radial):
    """Rows interleaved at random but each in sorted order: the workspace path gives the dst-sorted
    convolution bit for bit (the grouping restores the sorted list exactly), and two calls agree."""
    eq = _eq()
    wl = synth.small_graph(45, 9, C, L, 2000 + C + L, radial=radial, r_cut=5.0, empty_rows=(0, 44),
                           long_rows=(3,), long_len=150, zero_vec_edges=1)
    w = wl.w_rad if radial else wl.w
    kw = dict(weight_mode=1, r_cut=5.0) if radial else {}
    pvec, psrc, pdst = _interleave_rows(wl, 17)
    _say("conv ws interleaved C=%d L=%d radial=%d" % (C, L, radial))
    ref = _np(eq.eqtp_conv_fused(_t(wl.vec), _t(wl.src), _t(wl.x), _t(w), L, row_ptr=_t(wl.row_ptr), **kw))
    got = _np(eq.eqtp_conv_fused_ws(_t(pvec), _t(psrc), _t(wl.x), _t(w), L, dst=_t(pdst), **kw))
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), "grouped result differs from the sorted one"
    again = _np(eq.eqtp_conv_fused_ws(_t(pvec), _t(psrc), _t(wl.x), _t(w), L, dst=_t(pdst), **kw))
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32))
    orc = oracle.conv(wl.N, wl.vec, wl.src, wl.dst, wl.x, w, L, weight_mode=1 if radial else 0, r_cut=5.0)
    _assert_close(got, orc, TOL, "conv ws C%d L%d" % (C, L))


@pytest.mark.parametrize("C,L,ps", [(C, L, ps) for C in (8, 32, 64, 128) for L in (0, 1, 2, 3) for ps in (0, 1)])
def test_conv_ws_random_order(C, L, ps):
    """Edges in a random order: against the oracle, deterministic from call to call, fp32 and bf16 x."""
    import torch

    eq = _eq()
    wl = synth.small_graph(40, 11, C, L, 2100 + C + 10 * L + 100 * ps, path_set=ps, empty_rows=(5,),
                           long_rows=(6, 7), long_len=200, zero_vec_edges=2)
    pvec, psrc, pdst = synth.random_permutation(wl, seed=3)
    ref = oracle.conv(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w, L, path_set=ps)
    _say("conv ws random order C=%d L=%d ps=%d" % (C, L, ps))
    ws = torch.empty(eq.eqtp_conv_workspace_bytes(wl.N, wl.E, L, C), dtype=torch.uint8, device="cuda")
    a = _np(eq.eqtp_conv_fused_ws(_t(pvec), _t(psrc), _t(wl.x), _t(wl.w), L, dst=_t(pdst), path_set=ps,
                                  workspace=ws))
    _assert_close(a, ref, TOL, "conv ws random order")
    b = _np(eq.eqtp_conv_fused_ws(_t(pvec), _t(psrc), _t(wl.x), _t(wl.w), L, dst=_t(pdst), path_set=ps,
                                  workspace=ws))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "not deterministic"
    xb = _t(wl.x).to(torch.bfloat16)
    xr = xb.float().cpu().numpy()
    got = _np(eq.eqtp_conv_fused_ws(_t(pvec), _t(psrc), xb, _t(wl.w), L, dst=_t(pdst), path_set=ps))
    _assert_close(got, oracle.conv(wl.N, wl.vec, wl.src, wl.dst, xr, wl.w, L, path_set=ps), TOL, "conv ws bf16 x")


def test_conv_ws_no_edges_and_sorted_passthrough():
    import torch

    eq = _eq()
    N, C = 9, 32
    x = torch.randn(N, C, 16, device="cuda")
    w = torch.randn(23, C, device="cuda")
    _say("conv ws no edges")
    out = torch.full_like(x, 7.0)
    eq.eqtp_conv_fused_ws(torch.zeros((0, 3), device="cuda"), torch.zeros(0, dtype=torch.int32, device="cuda"), x, w,
                          3, dst=torch.zeros(0, dtype=torch.int32, device="cuda"), out=out)
    assert np.all(_np(out) == 0.0)
    assert eq.eqtp_conv_workspace_bytes(N, 100, 3, C, edge_order=eq.EQTP_EDGES_DST_SORTED) == 0
    wl = synth.small_graph(20, 7, 64, 3, 2200)
    _say("conv ws sorted pass-through")
    a = _np(eq.eqtp_conv_fused_ws(_t(wl.vec), _t(wl.src), _t(wl.x), _t(wl.w), 3, row_ptr=_t(wl.row_ptr)))
    b = _np(eq.eqtp_conv_fused(_t(wl.vec), _t(wl.src), _t(wl.x), _t(wl.w), 3, row_ptr=_t(wl.row_ptr)))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("name", ["mid", "large", "radial"])
def test_conv_ws_workloads(name):
    """Full-size workloads in random edge order through the workspace path: every row against the oracle."""
    eq = _eq()
    wl = _wl(name)
    pvec, psrc, pdst = synth.random_permutation(wl)
    _say("conv ws %s E=%d" % (name, wl.E))
    out = _np(eq.eqtp_conv_fused_ws(_t(pvec), _t(psrc), _t(wl.x), _t(wl.weights), wl.lmax, dst=_t(pdst),
                                    path_set=wl.path_set, weight_mode=wl.weight_mode, r_cut=wl.r_cut))
    _assert_close(out, _oracle_full(name), TOL, name + " conv ws")


# ---- eqtp_sort_edges_stable: every output unique, so all of them are compared exactly ----

def _check_stable(eq, N, dst, vec=None, src=None, reuse=None):
    E = dst.shape[0]
    key = np.clip(dst, 0, max(N - 1, 0))  # out-of-range keys are clamped, as the kernels do
    order = np.argsort(key, kind="stable").astype(np.int32)
    got = eq.eqtp_sort_edges_stable(_t(dst), N, vec=_t(vec) if vec is not None else None,
                                    src=_t(src) if src is not None else None, out=reuse)
    rp, perm = _np(got[0]), _np(got[1])
    want_rp = np.concatenate([[0], np.cumsum(np.bincount(key, minlength=N))]).astype(np.int32)
    assert np.array_equal(rp, want_rp), "row_ptr differs"
    assert np.array_equal(perm, order), "perm differs from the stable order"
    if vec is not None:
        assert np.array_equal(_np(got[2]), vec[order])
    if src is not None:
        assert np.array_equal(_np(got[3]), src[order])
    return got


@pytest.mark.parametrize("N,E,seed", [(1, 1, 20), (1, 500, 21), (7, 3, 22), (512, 5000, 23), (513, 5000, 24),
                                      (10000, 266116, 25), (262144, 40000, 26), (300000, 50000, 27),
                                      (5000, 2, 28)])
def test_stable_sort_random(N, E, seed):
    """One, two and three radix passes (keys of up to 9, 18 and 27 bits), tiny and mid-sized inputs."""
    eq = _eq()
    rng = np.random.default_rng(seed)
    dst = rng.integers(0, N, size=E).astype(np.int32)
    _say("stable sort N=%d E=%d" % (N, E))
    _check_stable(eq, N, dst, rng.standard_normal((E, 3)).astype(np.float32),
                  rng.integers(0, N, size=E).astype(np.int32))


def test_stable_sort_skewed_clamped_and_repeated():
    eq = _eq()
    rng = np.random.default_rng(29)
    N, E = 3000, 60000
    dst = np.where(rng.random(E) < 0.5, 1234, rng.integers(0, N, size=E) // 7 * 7).astype(np.int32)
    dst[:4] = (0, N - 1, -5, N + 9)  # the last two are clamped to rows 0 and N - 1
    vec = rng.standard_normal((E, 3)).astype(np.float32)
    _say("stable sort skewed + clamped")
    first = _check_stable(eq, N, dst, vec, None)
    again = _check_stable(eq, N, dst, vec, None)
    assert np.array_equal(_np(first[1]), _np(again[1]))
    d2 = rng.integers(0, N // 3, size=E).astype(np.int32)  # same buffers, other edges
    _check_stable(eq, N, d2, None, None, reuse=(first[0], first[1], None, None))


def test_stable_sort_no_edges_and_validation():
    import torch

    eq = _eq()
    _say("stable sort no edges")
    for N in (0, 1, 777):
        rp, perm, _, _ = eq.eqtp_sort_edges_stable(torch.zeros(0, dtype=torch.int32, device="cuda"), N)
        assert np.array_equal(_np(rp), np.zeros(N + 1, dtype=np.int32)) and perm.numel() == 0
    dst = _t(np.zeros(100, np.int32))
    short = torch.empty(eq.eqtp_sort_workspace_bytes(10, 100) - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(eq.EqtpError):
        eq.eqtp_sort_edges_stable(dst, 10, workspace=short)

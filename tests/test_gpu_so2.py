"""GPU parity of the edge-aligned (SO(2)) convolution (eqtp_conv_fused with
EQTP_ALGO_EDGE_SO2, through the C ABI) against the fp64 oracle, which
evaluates the Clebsch-Gordan definition directly: the two routes share no
arithmetic (the kernel never evaluates a harmonic or a full coupling block).

Bar: max|gpu - oracle| <= 2e-4 * max|oracle| per output tensor.  Cases: every
lmax 0..6, both path sets, every supported channel count, dst-sorted and
unsorted edges, zero-length edges, edges along +z / -z and nearly along z
(the frame's special cases), empty and long rows.
"""
import numpy as np
import pytest

import oracle
from spherical_harmonic_cg_amd import synth
from test_gpu_parity import TOL, _assert_close, _eq, _np, _oracle_full, _say, _t, _wl

pytestmark = pytest.mark.gpu

SO2 = 3


def _graph(L, ps, C, seed, n=23, deg=7):
    wl = synth.small_graph(n, deg, C, L, seed, path_set=ps, empty_rows=(2,), long_rows=(5,), long_len=70,
                           zero_vec_edges=2)
    wl.vec[2] = (0.0, 0.0, 1.7)
    wl.vec[3] = (0.0, 0.0, -0.9)
    wl.vec[4] = (1e-4, -2e-4, 1.3)
    wl.vec[5] = (3e-4, 1e-4, -2.2)
    return wl


def _run(eq, wl, unsorted, algo=SO2, perm_seed=3):
    kw = dict(path_set=wl.path_set, algo=algo)
    if unsorted:
        perm = np.random.default_rng(perm_seed).permutation(wl.src.shape[0])
        return eq.eqtp_conv_fused(_t(wl.vec[perm]), _t(wl.src[perm]), _t(wl.x), _t(wl.w), wl.lmax,
                                  dst=_t(wl.dst[perm]), **kw)
    return eq.eqtp_conv_fused(_t(wl.vec), _t(wl.src), _t(wl.x), _t(wl.w), wl.lmax, row_ptr=_t(wl.row_ptr), **kw)


# C = 128 above lmax 4 runs as two launches over 64-channel halves
CASES = [(L, ps, C) for L in range(7) for ps in (0, 1) for C in (8, 16, 32, 64, 128)]


@pytest.mark.parametrize("L,ps,C", CASES)
@pytest.mark.parametrize("unsorted", [False, True])
def test_so2_small(L, ps, C, unsorted):
    eq = _eq()
    wl = _graph(L, ps, C, 1000 + 10 * L + C + ps)
    _say("so2 L=%d ps=%d C=%d unsorted=%s E=%d" % (L, ps, C, unsorted, wl.src.shape[0]))
    ref = oracle.conv(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w, L, path_set=ps)
    _assert_close(_np(_run(eq, wl, unsorted)), ref, TOL, "so2 L%d ps%d C%d u%d" % (L, ps, C, unsorted))


@pytest.mark.parametrize("L", [4, 5, 6])
def test_so2_auto_selects_for_high_lmax(L):
    eq = _eq()
    wl = _graph(L, 0, 32, 77 + L)
    _say("so2 auto L=%d" % L)
    ref = oracle.conv(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w, L)
    _assert_close(_np(_run(eq, wl, False, algo=0)), ref, TOL, "auto L%d" % L)


def test_so2_rejects_unsupported():
    import torch

    eq = _eq()
    _say("so2 unsupported combinations")
    wl = _graph(4, 0, 32, 6)
    with pytest.raises(eq.EqtpError):
        _run(eq, wl, False, algo=1)              # lmax 4 has no node-factored form
    with pytest.raises(eq.EqtpError):
        eq.eqtp_conv_fused(_t(wl.vec), _t(wl.src), _t(wl.x).to(torch.bfloat16), _t(wl.w), 4,
                           row_ptr=_t(wl.row_ptr), algo=SO2)


def test_so2_sorted_deterministic():
    eq = _eq()
    wl = _graph(6, 0, 64, 9)
    _say("so2 deterministic")
    a = _np(_run(eq, wl, False))
    b = _np(_run(eq, wl, False))
    assert np.array_equal(a, b)


def test_so2_mid_lmax3_full():
    """The mid workload (266 k edges, C = 64, lmax 3) through the edge-aligned
    kernel, every output against the oracle."""
    eq = _eq()
    from test_gpu_parity import _gpu_inputs, _oracle_full

    wl = _wl("mid")
    g = _gpu_inputs(wl)
    _say("so2 mid lmax 3 E=%d" % wl.E)
    out = eq.eqtp_conv_fused(g["vec"], g["src"], g["x"], g["w"], 3, row_ptr=g["row_ptr"], algo=SO2)
    _assert_close(_np(out), _oracle_full("mid"), TOL, "so2 mid")


def test_so2_lmax6_graph_full():
    """A 2,000-atom radius graph at lmax 6 (C = 32): sorted and unsorted outputs, every row
    against the oracle."""
    eq = _eq()
    wl = synth.lmax_graph(6, 32, seed=11)
    ref = oracle.conv(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.weights, 6, path_set=wl.path_set)
    _say("so2 lmax 6 graph E=%d" % wl.E)
    out = _np(_run(eq, wl, False))
    _assert_close(out, ref, TOL, "so2 L6 sorted")
    outu = _np(_run(eq, wl, True))
    _assert_close(outu, ref, TOL, "so2 L6 unsorted")


@pytest.mark.parametrize("L,ps,C", [(4, 0, 32), (5, 1, 16), (6, 0, 64), (6, 1, 8), (4, 1, 128), (5, 1, 128), (6, 0, 128),
                                    (3, 0, 64), (2, 1, 32)])
def test_so2_messages(L, ps, C):
    """Per-edge messages [E, C, K] in the edge-aligned form (lmax > 3, or
    algo = EDGE_SO2 at lmax <= 3) against the oracle's messages."""
    eq = _eq()
    wl = _graph(L, ps, C, 400 + 10 * L + C + ps, n=11, deg=5)
    _say("so2 messages L=%d ps=%d C=%d E=%d" % (L, ps, C, wl.src.shape[0]))
    ref = oracle.messages(wl.N, wl.vec, wl.src, wl.x, wl.w, L, path_set=ps)
    got = eq.eqtp_conv_messages(_t(wl.vec), _t(wl.src), _t(wl.x), _t(wl.w), L, path_set=ps, algo=SO2)
    _assert_close(_np(got), ref, TOL, "so2 messages L%d ps%d C%d" % (L, ps, C))
    if L > 3:  # the default choice at high degree
        got2 = eq.eqtp_conv_messages(_t(wl.vec), _t(wl.src), _t(wl.x), _t(wl.w), L, path_set=ps)
        assert np.array_equal(_np(got2), _np(got))


@pytest.mark.parametrize("L", [4, 5, 6])
@pytest.mark.parametrize("E", [1, 255, 256, 257, 5000])
def test_sh_high_degree(L, E):
    """Standalone harmonics at degree 4..6 (recurrence) against the oracle's,
    with zero vectors, the +-z axis and tiny / huge lengths."""
    eq = _eq()
    rng = np.random.default_rng(E + 10 * L)
    v = (rng.standard_normal((E, 3)) * rng.uniform(0.01, 50.0, (E, 1))).astype(np.float32)
    special = np.array([[0, 0, 0], [0, 0, 3.0], [0, 0, -0.2], [1e-3, 0, 0], [0, -7.0, 0]], np.float32)
    v[: min(E, 5)] = special[: min(E, 5)]
    _say("sh high degree L=%d E=%d" % (L, E))
    got = _np(eq.eqtp_sh(_t(v), L))
    ref = oracle.sh(v, L)
    assert np.abs(got - ref).max() <= 2e-5 * max(1.0, np.abs(ref).max())
    if E >= 1:
        assert got[0, 0] == np.float32(0.28209479177387814) and np.all(got[0, 1:] == 0.0)


@pytest.mark.parametrize("L", [4, 5, 6])
@pytest.mark.parametrize("C", [8, 16, 32, 64, 128])
def test_linear_high_degree(L, C):
    """The per-l channel linear at lmax 4..6 (column-tiled kernel), fp32 and
    bf16 operands, node counts that are not multiples of the tile."""
    eq = _eq()
    rng = np.random.default_rng(C * 11 + L)
    N = 37
    K = (L + 1) ** 2
    h = rng.standard_normal((N, C, K)).astype(np.float32)
    W = (rng.standard_normal((L + 1, C, C)) / np.sqrt(C)).astype(np.float32)
    _say("linear fp32 L=%d C=%d" % (L, C))
    _assert_close(_np(eq.eqtp_linear(_t(h), _t(W), L, eq.EQTP_F32)), oracle.linear(h, W, L), TOL, "linear fp32")
    _say("linear bf16 L=%d C=%d" % (L, C))
    outb = _np(eq.eqtp_linear(_t(h), _t(W), L, eq.EQTP_BF16))
    _assert_close(outb, oracle.linear(h, W, L, bf16=True), 2e-5, "linear bf16 vs rounded inputs")

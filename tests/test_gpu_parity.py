"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle on
the same seeded inputs.

Bar: max|gpu - oracle| <= 2e-4 * max|oracle| per output tensor for fp32 work;
bit-exact for the integer segment probe; bf16 linear within 1e-2 of the
unrounded fp64 product (and 2e-5 of the product of the bf16-rounded inputs).
"""
import functools
import sys

import numpy as np
import pytest

import oracle
from spherical_harmonic_cg_amd import synth

pytestmark = pytest.mark.gpu

TOL = 2e-4


def _eq():
    import spherical_harmonic_cg_amd as eq

    eq.load_library()
    return eq


def _t(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _np(t):
    import torch

    torch.cuda.synchronize()
    return t.cpu().numpy()


def _say(msg):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


def _assert_close(got, ref, tol=TOL, what=""):
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    err = float(np.abs(got.astype(np.float64) - ref).max()) if ref.size else 0.0
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    assert err <= tol * max(scale, 1e-30), "%s: max|d| %.3e > %.1e * %.3e" % (what, err, tol, scale)
    return err / max(scale, 1e-30)


@functools.lru_cache(maxsize=None)
def _wl(name):
    return synth.make_config(name)


@functools.lru_cache(maxsize=2)
def _oracle_full(name):
    """The oracle over every destination row of the workload (its rows shared out over the host's
    threads; the result does not depend on the thread count)."""
    wl = _wl(name)
    return oracle.conv(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.weights, wl.lmax, path_set=wl.path_set,
                       weight_mode=wl.weight_mode, r_cut=wl.r_cut)


def _gpu_inputs(wl):
    return dict(vec=_t(wl.vec), src=_t(wl.src), dst=_t(wl.dst), row_ptr=_t(wl.row_ptr), x=_t(wl.x),
                w=_t(wl.weights))


def _run_conv(eq, wl, g, algo, unsorted=False, perm=None):
    kw = dict(lmax=wl.lmax, path_set=wl.path_set, weight_mode=wl.weight_mode, r_cut=wl.r_cut, algo=algo)
    if unsorted:
        vec, src, dst = perm
        return eq.eqtp_conv_fused(_t(vec), _t(src), g["x"], g["w"], dst=_t(dst), **kw)
    return eq.eqtp_conv_fused(g["vec"], g["src"], g["x"], g["w"], row_ptr=g["row_ptr"], **kw)


# ----------------------------------------------------------------------------
# spherical harmonics
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "typical", "mid"])
def test_sh_workloads(name):
    eq = _eq()
    wl = _wl(name)
    for lmax in (wl.lmax, 3):
        _say("sh %s lmax=%d E=%d" % (name, lmax, wl.E))
        Y = _np(eq.eqtp_sh(_t(wl.vec), lmax))
        _assert_close(Y, oracle.sh(wl.vec, lmax), what="sh " + name)


@pytest.mark.parametrize("E", [1, 3, 255, 256, 257, 1000])
@pytest.mark.parametrize("lmax", [0, 1, 2, 3])
def test_sh_ragged_and_zero(E, lmax):
    eq = _eq()
    rng = np.random.default_rng(E * 10 + lmax)
    vec = (rng.standard_normal((E, 3)) * rng.uniform(0.1, 10, size=(E, 1))).astype(np.float32)
    vec[0] = 0.0
    _say("sh ragged E=%d lmax=%d" % (E, lmax))
    Y = _np(eq.eqtp_sh(_t(vec), lmax))
    ref = oracle.sh(vec, lmax)
    assert np.abs(Y - ref).max() < 2e-6
    assert Y[0, 0] == np.float32(0.28209479177387814) and np.all(Y[0, 1:] == 0)


def test_sh_empty():
    import torch

    eq = _eq()
    Y = eq.eqtp_sh(torch.zeros((0, 3), dtype=torch.float32, device="cuda"), 3)
    assert tuple(Y.shape) == (0, 16)


# ----------------------------------------------------------------------------
# fused convolution on the named workloads
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "typical", "mid"])
@pytest.mark.parametrize("algo", [1, 2])
def test_conv_sorted_full(name, algo):
    eq = _eq()
    wl = _wl(name)
    g = _gpu_inputs(wl)
    _say("conv sorted %s algo=%d E=%d" % (name, algo, wl.E))
    out = _np(_run_conv(eq, wl, g, algo))
    _assert_close(out, _oracle_full(name), what="conv %s algo %d" % (name, algo))


@pytest.mark.parametrize("name", ["tiny", "typical"])
def test_conv_unsorted_full(name):
    eq = _eq()
    wl = _wl(name)
    g = _gpu_inputs(wl)
    perm = synth.random_permutation(wl)
    _say("conv unsorted %s E=%d" % (name, wl.E))
    out = _np(_run_conv(eq, wl, g, 0, unsorted=True, perm=perm))
    _assert_close(out, _oracle_full(name), what="conv unsorted " + name)


def test_conv_large_sorted_full():
    """Large workload (100k atoms, 5.2M edges, C = 32), dst-sorted edges through the
    node kernel: the whole output tensor against the oracle over every row."""
    eq = _eq()
    wl = _wl("large")
    g = _gpu_inputs(wl)
    _say("conv large sorted node E=%d" % wl.E)
    out = _np(_run_conv(eq, wl, g, 0))
    _assert_close(out, _oracle_full("large"), what="large sorted")


def test_conv_large_unsorted_full():
    """Large workload with the edges in a seeded random order (fp32 atomics): the whole output
    tensor against the oracle."""
    eq = _eq()
    wl = _wl("large")
    g = _gpu_inputs(wl)
    _say("conv large unsorted (atomic) E=%d" % wl.E)
    outu = _np(_run_conv(eq, wl, g, 0, unsorted=True, perm=synth.random_permutation(wl)))
    _assert_close(outu, _oracle_full("large"), what="large atomic")


def test_conv_radial_sorted_full():
    """Radial workload (50k atoms, C = 128, per-edge radial weights), dst-sorted edges through the
    edge-aligned kernel with the radial products on the matrix cores: the whole output tensor."""
    eq = _eq()
    wl = _wl("radial")
    g = _gpu_inputs(wl)
    _say("conv radial sorted E=%d" % wl.E)
    out = _np(_run_conv(eq, wl, g, 0))
    _assert_close(out, _oracle_full("radial"), what="radial sorted")


def test_conv_radial_unsorted_full():
    """Radial workload with the edges in a seeded random order (per-edge walk, fp32 atomics): the
    whole output tensor."""
    eq = _eq()
    wl = _wl("radial")
    g = _gpu_inputs(wl)
    _say("conv radial unsorted E=%d" % wl.E)
    outu = _np(_run_conv(eq, wl, g, 0, unsorted=True, perm=synth.random_permutation(wl)))
    _assert_close(outu, _oracle_full("radial"), what="radial atomic")


# ----------------------------------------------------------------------------
# every (C, lmax, path set, algorithm, mode) on small ragged graphs
# ----------------------------------------------------------------------------

CASES = [(C, L, ps) for C in (8, 16, 32, 64, 128) for L in (0, 1, 2, 3) for ps in (0, 1)]


@pytest.mark.parametrize("C,L,ps", CASES)
def test_conv_small_all_variants(C, L, ps):
    eq = _eq()
    wl = synth.small_graph(n=37, e_per_row=9, C=C, lmax=L, seed=C + 10 * L + 100 * ps, path_set=ps,
                           empty_rows=(3, 4, 36), long_rows=(5,), long_len=70, zero_vec_edges=2)
    g = _gpu_inputs(wl)
    ref = oracle.conv(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w, L, path_set=ps)
    perm = synth.random_permutation(wl)
    for algo in (1, 2):
        _say("small C=%d L=%d ps=%d algo=%d" % (C, L, ps, algo))
        out = _np(_run_conv(eq, wl, g, algo))
        _assert_close(out, ref, what="small C%d L%d ps%d algo%d" % (C, L, ps, algo))
        assert np.all(out[[3, 4, 36]] == 0.0)
    _say("small C=%d L=%d ps=%d unsorted" % (C, L, ps))
    outu = _np(_run_conv(eq, wl, g, 0, unsorted=True, perm=perm))
    _assert_close(outu, ref, what="small unsorted")


@pytest.mark.parametrize("C,L", [(8, 2), (32, 3), (128, 3), (64, 1)])
def test_conv_small_radial(C, L):
    eq = _eq()
    wl = synth.small_graph(n=29, e_per_row=11, C=C, lmax=L, seed=5 + C + L, radial=True, r_cut=5.0,
                           empty_rows=(0,), long_rows=(7,), long_len=130, zero_vec_edges=1)
    # some edges beyond the cut-off contribute nothing
    wl.vec[5:9] *= 1.6
    g = _gpu_inputs(wl)
    ref = oracle.conv(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w_rad, L, weight_mode=1, r_cut=5.0)
    _say("small radial C=%d L=%d sorted" % (C, L))
    _assert_close(_np(_run_conv(eq, wl, g, 0)), ref, what="radial sorted")
    _say("small radial C=%d L=%d unsorted" % (C, L))
    _assert_close(_np(_run_conv(eq, wl, g, 0, unsorted=True, perm=synth.random_permutation(wl))), ref,
                  what="radial unsorted")


RADIAL_CASES = [(C, L, ps) for C in (8, 16, 32, 64, 128) for L in (0, 1, 2, 3) for ps in (0, 1)]


@pytest.mark.parametrize("C,L,ps", RADIAL_CASES)
def test_conv_radial_all_variants(C, L, ps):
    """Radial weights on dst-sorted edges for every channel count, degree and path set: the edge-aligned
    kernel with the weights on the matrix cores (algo 0 and 3; C = 8 takes the per-edge walk) and the
    per-edge walk (algo 2).  Rows of 0, 1, 16, 17 and 70 edges cover empty, full and ragged 16-edge
    batches; zero vectors and edges beyond the cut-off are mixed in."""
    eq = _eq()
    wl = synth.small_graph(n=31, e_per_row=9, C=C, lmax=L, seed=300 + C + 10 * L + 100 * ps, path_set=ps,
                           radial=True, r_cut=5.0, empty_rows=(0, 30), long_rows=(7,), long_len=70,
                           zero_vec_edges=2)
    wl.vec[12:16] *= 1.7  # beyond the cut-off: no contribution
    g = _gpu_inputs(wl)
    ref = oracle.conv(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w_rad, L, path_set=ps, weight_mode=1, r_cut=5.0)
    for algo in (0, 2, 3):
        if algo == 3 and C % 16:
            continue
        _say("radial C=%d L=%d ps=%d algo=%d" % (C, L, ps, algo))
        out = _np(_run_conv(eq, wl, g, algo))
        _assert_close(out, ref, what="radial C%d L%d ps%d algo%d" % (C, L, ps, algo))
        assert np.all(out[[0, 30]] == 0.0)


def test_conv_radial_batch_edges():
    """Rows of exactly 1, 15, 16, 17, 31, 32 and 33 edges: around the 16-edge batch of the radial
    edge-aligned kernel."""
    eq = _eq()
    for n_e in (1, 15, 16, 17, 31, 32, 33):
        wl = synth.small_graph(n=4, e_per_row=n_e, C=32, lmax=3, seed=900 + n_e, radial=True, r_cut=5.0,
                               long_rows=(0, 1, 2, 3), long_len=n_e)
        g = _gpu_inputs(wl)
        ref = oracle.conv(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w_rad, 3, weight_mode=1, r_cut=5.0)
        _say("radial batch edges %d" % n_e)
        _assert_close(_np(_run_conv(eq, wl, g, 0)), ref, what="radial %d edges per row" % n_e)


@pytest.mark.parametrize("n", [1, 2, 3, 5])
def test_conv_radial_few_nodes(n):
    """Fewer nodes than a workgroup's four rows (one row group per channel block in the radial
    edge-aligned kernel's block-major grid), C = 128 (eight channel blocks)."""
    eq = _eq()
    wl = synth.small_graph(n=n, e_per_row=19, C=128, lmax=3, seed=1200 + n, radial=True, r_cut=5.0)
    g = _gpu_inputs(wl)
    ref = oracle.conv(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w_rad, 3, weight_mode=1, r_cut=5.0)
    _say("radial few nodes n=%d" % n)
    _assert_close(_np(_run_conv(eq, wl, g, 0)), ref, what="radial n=%d" % n)


def test_conv_radial_deterministic():
    eq = _eq()
    wl = synth.small_graph(n=40, e_per_row=23, C=64, lmax=3, seed=41, radial=True, r_cut=5.0)
    g = _gpu_inputs(wl)
    _say("radial determinism")
    a = _np(_run_conv(eq, wl, g, 0))
    b = _np(_run_conv(eq, wl, g, 0))
    np.testing.assert_array_equal(a, b)


def test_conv_long_rows_and_single_node():
    """Rows longer than 64 and 256 edges (several staging chunks), and N = 1."""
    eq = _eq()
    wl = synth.small_graph(n=6, e_per_row=3, C=64, lmax=3, seed=77, long_rows=(1, 4), long_len=300)
    g = _gpu_inputs(wl)
    ref = oracle.conv(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w, 3)
    for algo in (1, 2):
        _say("long rows algo=%d" % algo)
        _assert_close(_np(_run_conv(eq, wl, g, algo)), ref, what="long rows")
    one = synth.small_graph(n=1, e_per_row=5, C=32, lmax=3, seed=78)
    g1 = _gpu_inputs(one)
    ref1 = oracle.conv(1, one.vec, one.src, one.dst, one.x, one.w, 3)
    for algo in (1, 2):
        _say("single node algo=%d" % algo)
        _assert_close(_np(_run_conv(eq, one, g1, algo)), ref1, what="single node")


def test_conv_no_edges():
    import torch

    eq = _eq()
    N, C = 9, 32
    x = torch.randn(N, C, 16, device="cuda")
    w = torch.randn(23, C, device="cuda")
    vec = torch.zeros((0, 3), device="cuda")
    src = torch.zeros(0, dtype=torch.int32, device="cuda")
    rp = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
    for algo in (1, 2):
        _say("no edges algo=%d" % algo)
        out = torch.full_like(x, 7.0)
        eq.eqtp_conv_fused(vec, src, x, w, 3, row_ptr=rp, algo=algo, out=out)
        assert np.all(_np(out) == 0.0)
    out = torch.full_like(x, 7.0)
    eq.eqtp_conv_fused(vec, src, x, w, 3, dst=torch.zeros(0, dtype=torch.int32, device="cuda"), out=out)
    assert np.all(_np(out) == 0.0)


def test_conv_sorted_deterministic():
    eq = _eq()
    wl = _wl("mid")
    g = _gpu_inputs(wl)
    for algo in (1, 2):
        _say("determinism algo=%d" % algo)
        a = _np(_run_conv(eq, wl, g, algo))
        for _ in range(2):
            b = _np(_run_conv(eq, wl, g, algo))
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ----------------------------------------------------------------------------
# bit-exact indexing: the conv kernels' walk, counting edges per node
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "typical", "mid", "large"])
def test_segment_probe_exact(name):
    eq = _eq()
    wl = _wl(name)
    want_cnt = np.bincount(wl.dst, minlength=wl.N)
    want_sum = np.bincount(wl.dst, weights=wl.src.astype(np.float64), minlength=wl.N).astype(np.int64)
    rp, src = _t(wl.row_ptr), _t(wl.src)
    for algo in (1, 2):
        _say("probe %s algo=%d" % (name, algo))
        cnt, s = eq.eqtp_test_segment_probe(rp, src, wl.C, wl.lmax, algo)
        np.testing.assert_array_equal(_np(cnt), want_cnt)
        np.testing.assert_array_equal(_np(s), want_sum)


def test_segment_probe_ragged():
    eq = _eq()
    for C in (8, 16, 32, 64, 128):
        wl = synth.small_graph(n=50, e_per_row=13, C=C, lmax=3, seed=C, empty_rows=(0, 49),
                               long_rows=(10, 11), long_len=257)
        for algo in (1, 2):
            _say("probe ragged C=%d algo=%d" % (C, algo))
            cnt, s = eq.eqtp_test_segment_probe(_t(wl.row_ptr), _t(wl.src), C, 3, algo)
            np.testing.assert_array_equal(_np(cnt), np.diff(wl.row_ptr))
            np.testing.assert_array_equal(
                _np(s), np.bincount(wl.dst, weights=wl.src.astype(np.float64), minlength=wl.N).astype(np.int64))


# ----------------------------------------------------------------------------
# per-l linear
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("C", [8, 16, 32, 64, 128])
@pytest.mark.parametrize("L", [0, 2, 3])
def test_linear(C, L):
    eq = _eq()
    rng = np.random.default_rng(C * 7 + L)
    N = 53  # not a multiple of the 16-node tile
    K = (L + 1) ** 2
    h = rng.standard_normal((N, C, K)).astype(np.float32)
    W = (rng.standard_normal((L + 1, C, C)) / np.sqrt(C)).astype(np.float32)
    _say("linear fp32 C=%d L=%d" % (C, L))
    out = _np(eq.eqtp_linear(_t(h), _t(W), L, eq.EQTP_F32))
    _assert_close(out, oracle.linear(h, W, L), what="linear fp32")
    _say("linear bf16 C=%d L=%d" % (C, L))
    outb = _np(eq.eqtp_linear(_t(h), _t(W), L, eq.EQTP_BF16))
    _assert_close(outb, oracle.linear(h, W, L, bf16=True), tol=2e-5, what="linear bf16 vs rounded inputs")
    _assert_close(outb, oracle.linear(h, W, L), tol=1e-2, what="linear bf16 vs fp64")


@pytest.mark.parametrize("C,L", [(32, 3), (64, 3), (64, 1), (128, 3)])
def test_linear_many_tiles(C, L):
    """Enough nodes that every persistent workgroup walks several 16-node tiles (prefetching the
    next one), with a ragged last tile."""
    eq = _eq()
    rng = np.random.default_rng(1000 + C + L)
    N = 40009 if C <= 64 else 5009  # C = 128 takes one tile per workgroup
    K = (L + 1) ** 2
    h = rng.standard_normal((N, C, K)).astype(np.float32)
    W = (rng.standard_normal((L + 1, C, C)) / np.sqrt(C)).astype(np.float32)
    for dt, name in ((eq.EQTP_F32, "fp32"), (eq.EQTP_BF16, "bf16")):
        _say("linear many tiles %s C=%d L=%d N=%d" % (name, C, L, N))
        out = _np(eq.eqtp_linear(_t(h), _t(W), L, dt))
        ref = oracle.linear(h, W, L, bf16=(dt == eq.EQTP_BF16))
        _assert_close(out, ref, tol=2e-4 if dt == eq.EQTP_F32 else 2e-5, what="linear %s many tiles" % name)


def test_linear_identity_exact():
    eq = _eq()
    rng = np.random.default_rng(3)
    h = rng.standard_normal((40, 64, 16)).astype(np.float32)
    W = np.stack([np.eye(64, dtype=np.float32)] * 4)
    _say("linear identity")
    out = _np(eq.eqtp_linear(_t(h), _t(W), 3, eq.EQTP_F32))
    np.testing.assert_array_equal(out, h)


@pytest.mark.parametrize("name", ["typical", "mid"])
def test_linear_workloads(name):
    eq = _eq()
    wl = _wl(name)
    dtype = eq.EQTP_BF16 if wl.linear_bf16 else eq.EQTP_F32
    h = _oracle_full(name).astype(np.float32)
    _say("linear %s" % name)
    out = _np(eq.eqtp_linear(_t(h), _t(wl.w_lin), wl.lmax, dtype))
    ref = oracle.linear(h, wl.w_lin, wl.lmax)
    _assert_close(out, ref, tol=1e-2 if wl.linear_bf16 else TOL, what="linear " + name)


def _bf16_pair(rng, shape, scale=1.0):
    """A bfloat16 CUDA tensor and the exact float32 values it holds."""
    import torch

    t = (torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32))).to(torch.bfloat16)
    return t.cuda(), t.float().numpy()


@pytest.mark.parametrize("C", [8, 16, 32, 64, 128])
@pytest.mark.parametrize("L", [0, 1, 2, 3, 4, 6])
def test_linear_bf16_storage(C, L):
    """h and W held as bfloat16 in memory (EQTP_BF16): against the oracle on the same bf16 values."""
    eq = _eq()
    rng = np.random.default_rng(500 + 7 * C + L)
    N = 53
    K = (L + 1) ** 2
    h, h32 = _bf16_pair(rng, (N, C, K))
    W, W32 = _bf16_pair(rng, (L + 1, C, C), 1.0 / np.sqrt(C))
    _say("linear bf16 storage C=%d L=%d" % (C, L))
    out = _np(eq.eqtp_linear(h, W, L, eq.EQTP_BF16))
    _assert_close(out, oracle.linear(h32, W32, L), tol=2e-5, what="linear bf16 storage")


@pytest.mark.parametrize("C,L", [(64, 3), (32, 3), (128, 3), (64, 2), (16, 1)])
def test_linear_bf16_many_tiles(C, L):
    """Enough nodes that every persistent workgroup of the bf16-product kernel walks many 4-node tiles
    (both register sets of its load ring), a ragged last tile; fp32 storage rounded on load and bf16
    storage."""
    eq = _eq()
    rng = np.random.default_rng(900 + C + L)
    N = 40009
    K = (L + 1) ** 2
    h, h32 = _bf16_pair(rng, (N, C, K))
    W, W32 = _bf16_pair(rng, (L + 1, C, C), 1.0 / np.sqrt(C))
    ref = oracle.linear(h32, W32, L)
    _say("linear bf16 storage many tiles C=%d L=%d" % (C, L))
    _assert_close(_np(eq.eqtp_linear(h, W, L, eq.EQTP_BF16)), ref, tol=2e-5, what="bf16 storage many tiles")
    hf = rng.standard_normal((N, C, K)).astype(np.float32)
    _say("linear fp32 storage bf16 products many tiles C=%d L=%d" % (C, L))
    out = _np(eq.eqtp_linear(_t(hf), _t(W32), L, eq.EQTP_F32_BF16))
    _assert_close(out, oracle.linear(hf, W32, L, bf16=True), tol=2e-5, what="fp32 storage bf16 products")

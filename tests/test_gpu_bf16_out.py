"""bfloat16 output with packed bf16 atomics (eqtp_conv_fused with
desc.out_dtype = EQTP_BF16, edges in any order): parity with the fp64 oracle
to a bound derived from the rounding the path performs.

Every message element m_e (fp32, error ~1e-6 relative) is rounded to bf16
and added into out[dst_e] by an atomic whose result is bf16 again.  With
unit roundoff u = 2^-8 for bf16's 8-bit significand, and one ulp = 2u per
operation (so the bound holds whatever rounding the atomic unit applies), the
error of a node receiving d messages in any order is at most
    2u * (d + 1) * (1 + 2u d) * S,   S = sum_e |m_e|
(one rounding of each message, d - 1 roundings of partial sums bounded by S,
and the second-order term).  The checks compare every element with that
bound, and also on graphs of in-degree <= 1 (a single rounding: |error| <=
2u |m|) and <= 3, where dropping or doubling one message breaks the bound by
an order of magnitude."""
import numpy as np
import pytest

import oracle
from spherical_harmonic_cg_amd import synth
from test_gpu_parity import _eq, _np, _say, _t

pytestmark = pytest.mark.gpu

ULP = 2.0 ** -7  # one bf16 ulp relative to the value, 2u


def _abs_sum_and_degree(wl, x, w, weight_mode=0, r_cut=0.0, block=20000):
    """S[n, c, k] = sum over edges into n of |message| (fp64 oracle), and the in-degree of every node."""
    S = np.zeros((wl.N, wl.C, (wl.lmax + 1) ** 2))
    for b in range(0, wl.E, block):
        m = oracle.messages(wl.N, wl.vec[b:b + block], wl.src[b:b + block], x, w, wl.lmax, wl.path_set,
                            weight_mode=weight_mode, r_cut=r_cut)
        db = wl.dst[b:b + block]  # dst-sorted: one run per destination
        starts = np.flatnonzero(np.r_[True, db[1:] != db[:-1]])
        S[db[starts]] += np.add.reduceat(np.abs(m), starts, axis=0)
    deg = np.bincount(wl.dst, minlength=wl.N)
    return S, deg


def _check(got, ref, S, deg, what):
    d = deg.astype(np.float64)[:, None, None]
    bound = ULP * (d + 1.0) * (1.0 + ULP * d) * S + 1e-6 * max(float(np.abs(ref).max()), 1e-30)
    err = np.abs(got.astype(np.float64) - ref)
    worst = float((err / bound).max()) if err.size else 0.0
    _say("%s: worst error / bound = %.3f, mean |error| / mean S = %.2e" % (
        what, worst, float(err.mean() / max(S.mean(), 1e-30)) if err.size else 0.0))
    assert worst <= 1.0, what
    # nodes with no incoming edge are exact zeros
    assert np.all(got[deg == 0] == 0.0), what


def _run(eq, wl, x, w, perm_seed=1, **kw):
    import torch

    rng = np.random.default_rng(perm_seed)
    p = rng.permutation(wl.E)
    out = eq.eqtp_conv_fused(_t(wl.vec[p]), _t(wl.src[p]), x, _t(w), wl.lmax, dst=_t(wl.dst[p].astype(np.int32)),
                             path_set=wl.path_set, out_dtype=eq.EQTP_BF16, **kw)
    assert out.dtype == torch.bfloat16
    return _np(out.float())


@pytest.mark.parametrize("lmax", [0, 1, 2, 3])
@pytest.mark.parametrize("ps", [0, 1])
@pytest.mark.parametrize("C", [8, 16, 32, 64, 128])
def test_bf16_out_small(lmax, ps, C):
    eq = _eq()
    wl = synth.small_graph(29, 8, C, lmax, 5100 + 10 * lmax + C + ps, path_set=ps, empty_rows=(1, 7),
                           long_rows=(4,), long_len=60, zero_vec_edges=1)
    _say("bf16 out lmax=%d ps=%d C=%d E=%d" % (lmax, ps, C, wl.E))
    got = _run(eq, wl, _t(wl.x), wl.w)
    ref = oracle.conv(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w, lmax, path_set=ps)
    S, deg = _abs_sum_and_degree(wl, wl.x, wl.w)
    _check(got, ref, S, deg, "bf16 out L%d ps%d C%d" % (lmax, ps, C))


@pytest.mark.parametrize("max_deg", [1, 3])
@pytest.mark.parametrize("C", [16, 64])
def test_bf16_out_low_degree(max_deg, C):
    """In-degree <= 1: each element is one rounding of the message; <= 3: a dropped message fails."""
    eq = _eq()
    rng = np.random.default_rng(5200 + max_deg + C)
    wl = synth.small_graph(64, 0, C, 3, 5201 + C, empty_rows=range(64))
    deg = rng.integers(0, max_deg + 1, size=wl.N)
    dst = np.repeat(np.arange(wl.N), deg).astype(np.int32)
    E = dst.shape[0]
    wl.dst = dst
    wl.src = rng.integers(0, wl.N, size=E).astype(np.int32)
    wl.vec = rng.normal(size=(E, 3)).astype(np.float32)
    wl.row_ptr = np.concatenate([[0], np.cumsum(deg)]).astype(np.int32)
    _say("bf16 out low degree max_deg=%d C=%d E=%d" % (max_deg, C, E))
    got = _run(eq, wl, _t(wl.x), wl.w)
    ref = oracle.conv(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w, 3)
    S, d = _abs_sum_and_degree(wl, wl.x, wl.w)
    _check(got, ref, S, d, "bf16 out low degree %d" % max_deg)
    if max_deg == 1:
        one = d == 1
        assert np.all(np.abs(got[one] - ref[one]) <= ULP * np.abs(ref[one]) + 1e-6 * np.abs(ref).max())


def test_bf16_out_radial_and_bf16_features():
    import torch

    eq = _eq()
    wl = synth.small_graph(37, 9, 32, 3, 5301, radial=True, r_cut=5.0, empty_rows=(3,), zero_vec_edges=1)
    wl.vec[5:8] *= 1.8  # some edges beyond the cut-off
    _say("bf16 out radial weights E=%d" % wl.E)
    got = _run(eq, wl, _t(wl.x), wl.w_rad, weight_mode=eq.EQTP_W_RADIAL, r_cut=wl.r_cut)
    ref = oracle.conv(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w_rad, 3, weight_mode=1, r_cut=wl.r_cut)
    S, deg = _abs_sum_and_degree(wl, wl.x, wl.w_rad, weight_mode=1, r_cut=wl.r_cut)
    _check(got, ref, S, deg, "bf16 out radial")
    _say("bf16 out with bf16 features")
    xb = _t(wl.x).to(torch.bfloat16)
    xr = xb.float().cpu().numpy()
    got = _run(eq, wl, xb, wl.w)
    ref = oracle.conv(wl.N, wl.vec, wl.src, wl.dst, xr, wl.w, 3)
    S, deg = _abs_sum_and_degree(wl, xr, wl.w)
    _check(got, ref, S, deg, "bf16 out, bf16 x")


def test_bf16_out_mid_workload():
    """The mid graph (10k atoms, 266 k edges, C = 64, lmax 3) in random order: every element within its bound."""
    eq = _eq()
    wl = synth.make_config("mid")
    _say("bf16 out mid E=%d" % wl.E)
    got = _run(eq, wl, _t(wl.x), wl.w, perm_seed=3)
    ref = oracle.conv(wl.N, wl.vec, wl.src, wl.dst, wl.x, wl.w, 3)
    S, deg = _abs_sum_and_degree(wl, wl.x, wl.w)
    _check(got, ref, S, deg, "bf16 out mid")


def test_bf16_out_no_edges():
    eq = _eq()
    wl = synth.small_graph(9, 0, 16, 2, 5401, empty_rows=range(9))
    _say("bf16 out no edges")
    got = _run(eq, wl, _t(wl.x), wl.w)
    assert got.shape == (9, 16, 9) and np.all(got == 0.0)

"""Features past 4 GiB.  The dst-sorted matrix-core kernel (and its adjoint,
grouped by source) reads the features through buffer loads with 32-bit byte
offsets while they fit in 4 GiB, and through plain 64-bit loads beyond that.
These tests run the second form (and the other fixed-weight forward
kernels, which index with 64-bit offsets throughout, at the same size):
600,000 nodes x 128 channels x 16
components (lmax 3) is 4.9 GB of fp32, with sources spread over all nodes so
that about an eighth of the gathers land past the 4 GiB mark.  The features
come from a seeded generator on the GPU; the fp64 oracle checks the sampled
rows (every row whose sources reach past the mark among them) on the same
values, to the tolerance of the other parity tests (2e-4 of the largest
oracle value)."""
import numpy as np
import pytest

import oracle
from test_gpu_parity import TOL, _assert_close, _eq, _np, _say, _t

pytestmark = pytest.mark.gpu

N, C, L = 600_000, 128, 3
K = (L + 1) ** 2
PAST = (1 << 32) // (C * K * 4)  # first node whose features start past 4 GiB


def _graph(seed):
    rng = np.random.default_rng(seed)
    deg = rng.integers(0, 4, size=N)
    deg[-1] = 3
    E = int(deg.sum())
    src = rng.integers(0, N, size=E).astype(np.int32)
    src[-3:] = [N - 1, PAST, PAST - 1]  # the last feature row, and either side of the mark
    vec = rng.normal(size=(E, 3)).astype(np.float32)
    row_ptr = np.concatenate([[0], np.cumsum(deg)]).astype(np.int32)
    dst = np.repeat(np.arange(N, dtype=np.int32), deg)
    return rng, deg, src, dst, vec, row_ptr


def _features(seed):
    import torch

    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    return torch.randn((N, C, K), generator=gen, device="cuda", dtype=torch.float32)


def _take_rows(t, rows):
    import torch

    return _np(t.index_select(0, torch.from_numpy(np.asarray(rows, dtype=np.int64)).cuda()))


# node: the dst-sorted matrix-core kernel (plain loads past 4 GiB); edge: edges in random order, fp32
# atomics; so2: the edge-aligned form on dst-sorted edges
@pytest.mark.parametrize("form", ["node", "edge", "so2"])
def test_conv_features_past_4gib(form):
    eq = _eq()
    assert N * C * K * 4 > (1 << 32)
    rng, deg, src, dst, vec, row_ptr = _graph(9100)
    w = rng.normal(size=(eq.eqtp_num_paths(L), C)).astype(np.float32)
    x = _features(9101)
    _say("conv (%s), features past 4 GiB: N=%d C=%d E=%d" % (form, N, C, src.shape[0]))
    if form == "edge":
        p = np.random.default_rng(9102).permutation(src.shape[0])
        out = eq.eqtp_conv_fused(_t(vec[p]), _t(src[p]), x, _t(w), L, dst=_t(dst[p]))
    else:
        out = eq.eqtp_conv_fused(_t(vec), _t(src), x, _t(w), L, row_ptr=_t(row_ptr),
                                 algo=eq.EQTP_ALGO_EDGE_SO2 if form == "so2" else eq.EQTP_ALGO_AUTO)
    # sampled rows: random ones, rows with a source past the mark, the last row
    far_rows = np.unique(dst[src >= PAST])
    rows = np.unique(np.concatenate([rng.choice(N, 120, replace=False), rng.choice(far_rows, 60, replace=False),
                                     [N - 1]]))
    sel = np.concatenate([np.arange(row_ptr[r], row_ptr[r + 1]) for r in rows])
    uniq, local = np.unique(src[sel], return_inverse=True)
    assert uniq.max() >= PAST
    n_sub = max(len(uniq), len(rows))
    x_sub = np.zeros((n_sub, C, K), dtype=np.float32)
    x_sub[:len(uniq)] = _take_rows(x, uniq)
    dst_local = np.searchsorted(rows, dst[sel]).astype(np.int32)
    ref = oracle.conv(n_sub, vec[sel], local.astype(np.int32), dst_local, x_sub, w, L)[:len(rows)]
    got = _take_rows(out, rows)
    _assert_close(got, ref, TOL, "conv (%s) past 4 GiB" % form)
    # rows without edges are exact zeros
    empty = np.flatnonzero(deg == 0)[:50]
    assert np.all(_take_rows(out, empty) == 0.0)


def test_backward_by_source_features_past_4gib():
    """grad_x on the matrix cores from edges grouped by source, grad_out of 4.9 GB
    (the adjoint gathers grad_out through dst), and grad_vec per edge."""
    eq = _eq()
    rng, deg, src, dst, vec, row_ptr = _graph(9200)
    w = rng.normal(size=(eq.eqtp_num_paths(L), C)).astype(np.float32)
    # group by source (stable: each source's edges in input order)
    order = np.argsort(src, kind="stable")
    src_ptr = np.concatenate([[0], np.cumsum(np.bincount(src, minlength=N))]).astype(np.int32)
    x = _features(9201)
    gout = _features(9202)
    _say("backward by source, grad_out past 4 GiB: N=%d C=%d E=%d" % (N, C, src.shape[0]))
    gx, _, gv = eq.eqtp_conv_backward_by_source(_t(vec[order]), _t(dst[order]), _t(src_ptr), x, _t(w), gout, L,
                                                need_w=False, need_vec=True, perm=_t(order.astype(np.int32)))
    # sampled sources: random ones and ones whose destinations reach past the mark
    far_srcs = np.unique(src[dst >= PAST])
    srcs = np.unique(np.concatenate([rng.choice(np.unique(src), 80, replace=False),
                                     rng.choice(far_srcs, 40, replace=False)]))
    sel = np.flatnonzero(np.isin(src, srcs))
    nodes = np.unique(np.concatenate([srcs, dst[sel]]))
    assert nodes.max() >= PAST
    n_sub = len(nodes)
    src_l = np.searchsorted(nodes, src[sel]).astype(np.int32)
    dst_l = np.searchsorted(nodes, dst[sel]).astype(np.int32)
    x_sub = _take_rows(x, nodes)
    g_sub = _take_rows(gout, nodes)
    ref_gx, _, ref_gv = oracle.conv_backward(n_sub, vec[sel], src_l, dst_l, x_sub, w, g_sub, L)
    s_l = np.searchsorted(nodes, srcs)
    _assert_close(_take_rows(gx, srcs), ref_gx[s_l], TOL, "grad_x past 4 GiB")
    _assert_close(_np(gv)[sel], ref_gv, TOL, "grad_vec past 4 GiB")

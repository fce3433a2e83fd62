"""Host-side checks of the seeded synthetic workloads (CPU only)."""
import numpy as np

from spherical_harmonic_cg_amd import synth


def test_radius_graph_matches_bruteforce_periodic():
    rng = np.random.default_rng(1)
    box = 12.0
    pos = rng.uniform(0, box, size=(300, 3))
    s1, d1 = synth.radius_edges(pos, 3.0, box)
    s2, d2 = synth.radius_edges_bruteforce(pos, 3.0, box)
    a = sorted(zip(d1.tolist(), s1.tolist()))
    b = sorted(zip(d2.tolist(), s2.tolist()))
    assert a == b


def test_knn_in_degree_and_distances():
    rng = np.random.default_rng(2)
    box = 10.0
    pos = rng.uniform(0, box, size=(200, 3))
    src, dst = synth.knn_edges(pos, 20, box)
    assert np.all(np.bincount(dst, minlength=200) == 20)
    d = pos[None, :, :] - pos[:, None, :]
    d -= box * np.round(d / box)
    r = np.linalg.norm(d, axis=2)
    np.fill_diagonal(r, np.inf)
    kth = np.sort(r, axis=1)[:, 19]
    got = np.linalg.norm(synth.edge_vectors(pos, src, dst, box).astype(np.float64), axis=1).reshape(200, 20)
    np.testing.assert_allclose(got.max(axis=1), kth, rtol=1e-6)


def test_tiny_and_typical_structure():
    for name in ("tiny", "typical"):
        wl = synth.make_config(name)
        assert wl.row_ptr[0] == 0 and wl.row_ptr[-1] == wl.E
        assert np.all(np.diff(wl.row_ptr) >= 0)
        assert np.all(np.diff(wl.dst) >= 0)
        assert np.all(wl.src != wl.dst)
        np.testing.assert_array_equal(np.repeat(np.arange(wl.N), np.diff(wl.row_ptr)), wl.dst)
        assert wl.x.shape == (wl.N, wl.C, wl.K) and wl.x.dtype == np.float32
        assert wl.w.shape == (wl.P, wl.C)
    assert synth.make_config("typical").E == 20000


def test_deterministic():
    a = synth.make_config("typical")
    b = synth.make_config("typical")
    np.testing.assert_array_equal(a.vec, b.vec)
    np.testing.assert_array_equal(a.x, b.x)
    np.testing.assert_array_equal(a.w_lin, b.w_lin)


def test_num_paths():
    assert synth.num_paths(0, 0) == 1 and synth.num_paths(1, 0) == 4
    assert synth.num_paths(3, 0) == 23 and synth.num_paths(3, 1) == 34
    assert synth.num_paths(2, 0) == 11 and synth.num_paths(2, 1) == 15


def test_cell_order_is_a_renumbering():
    """The cell-sorted numbering is a permutation of the same atoms: same edge
    count and the same sorted multiset of edge lengths."""
    a = synth.make_config("typical")
    b = synth.make_config("typical", atom_order="cell")
    assert a.E == b.E
    la = np.sort(np.linalg.norm(a.vec.astype(np.float64), axis=1))
    lb = np.sort(np.linalg.norm(b.vec.astype(np.float64), axis=1))
    np.testing.assert_allclose(la, lb, rtol=1e-6)
    assert np.abs(b.src.astype(int) - b.dst).mean() < np.abs(a.src.astype(int) - a.dst).mean()

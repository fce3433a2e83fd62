"""Seeded synthetic workloads for the equivariant convolution.

This module only builds inputs: atom positions, neighbour lists, edge vectors,
CSR row pointers, node features and weights.  It holds none of the method's
arithmetic (no spherical harmonics, coupling coefficients or tensor
products), so both the HIP path and the fp64 oracle may consume what it
produces.

Workload shapes follow the Batmobile page (section "equivariant GNN compute
bottleneck": 1000 atoms, 32 channels, about 20 neighbours per atom; section
"monitoring and tuning": 1000-5000 atoms per batch, cut-offs of 4-6 Angstrom,
32-128 channels) plus three larger radius graphs.  Recipe:

* seeds: ``np.random.SeedSequence([2026, k]).spawn(4)`` for config index k,
  the four children drawing (positions, features, path weights,
  radial/linear weights) in that order;
* positions uniform in the box (float64); periodic boxes use the minimum
  image, every cut-off is below half the box side;
* edges are directed src -> dst with ``vec = pos[src] - pos[dst]`` computed in
  float64 and stored as float32; self edges are excluded;
* radius graphs contain both directions of every pair within the cut-off;
  the k-nearest graph gives every atom exactly k incoming edges;
* edges are sorted by (dst, src) and compressed into CSR row pointers;
* features are N(0, 1) float32 with layout [N, C, (L+1)^2];
* path weights are N(0, 1/P) float32 with layout [P, C];
* radial weights are N(0, 1/8) float32 with layout [8, P*C];
* linear weights are N(0, 1/C) float32 with layout [L+1, C_out, C_in];
* interaction-layer weights (``interaction_weights``): W_up and W_out as the
  linear weights, radial MLP W1 [8, H] N(0, 1/8), W2 [H, H] N(0, 1/H) and
  W3 [H, P*C] N(0, 1/H), float32, from their own seed.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

DENSITY = 0.1  # atoms per cubic Angstrom


def num_paths(lmax: int, path_set: int = 0) -> int:
    count = 0
    for l1 in range(lmax + 1):
        for l2 in range(lmax + 1):
            for l3 in range(lmax + 1):
                if abs(l1 - l2) <= l3 <= l1 + l2 and (path_set == 1 or (l1 + l2 + l3) % 2 == 0):
                    count += 1
    return count


@dataclasses.dataclass
class Workload:
    name: str
    N: int
    lmax: int
    C: int
    pos: np.ndarray          # [N, 3] float64
    box: Optional[float]     # periodic side length, None for open boundaries
    src: np.ndarray          # [E] int32, sorted by (dst, src)
    dst: np.ndarray          # [E] int32
    vec: np.ndarray          # [E, 3] float32
    row_ptr: np.ndarray      # [N+1] int32
    x: np.ndarray            # [N, C, K] float32
    w: np.ndarray            # [P, C] float32 (fixed path weights)
    path_set: int = 0
    weight_mode: int = 0     # 0 fixed weights, 1 radial weights
    r_cut: float = 0.0
    n_basis: int = 8
    w_rad: Optional[np.ndarray] = None   # [n_basis, P*C] float32
    w_lin: Optional[np.ndarray] = None   # [L+1, C, C] float32
    linear_bf16: bool = False

    @property
    def E(self) -> int:
        return int(self.src.shape[0])

    @property
    def K(self) -> int:
        return (self.lmax + 1) ** 2

    @property
    def P(self) -> int:
        return num_paths(self.lmax, self.path_set)

    @property
    def weights(self) -> np.ndarray:
        return self.w_rad if self.weight_mode == 1 else self.w


def _min_image(d: np.ndarray, box: Optional[float]) -> np.ndarray:
    if box is None:
        return d
    return d - box * np.round(d / box)


def radius_edges_bruteforce(pos: np.ndarray, r_cut: float, box: Optional[float]):
    """All ordered pairs (src, dst), src != dst, with |pos[src]-pos[dst]| < r_cut."""
    n = pos.shape[0]
    d = pos[None, :, :] - pos[:, None, :]          # d[i, j] = pos[j] - pos[i]
    d = _min_image(d, box)
    r2 = np.einsum("ijk,ijk->ij", d, d)
    mask = r2 < r_cut * r_cut
    np.fill_diagonal(mask, False)
    dst, src = np.nonzero(mask)
    return src.astype(np.int64), dst.astype(np.int64)


def radius_edges(pos: np.ndarray, r_cut: float, box: Optional[float]):
    """Radius graph via a k-d tree (periodic when ``box`` is given)."""
    from scipy.spatial import cKDTree

    if box is not None:
        p = np.mod(pos, box)
        p[p >= box] = 0.0
        tree = cKDTree(p, boxsize=box)
    else:
        p = pos
        tree = cKDTree(p)
    pairs = tree.query_pairs(r_cut, output_type="ndarray")
    i, j = pairs[:, 0].astype(np.int64), pairs[:, 1].astype(np.int64)
    src = np.concatenate([i, j])
    dst = np.concatenate([j, i])
    return src, dst


def knn_edges(pos: np.ndarray, k: int, box: Optional[float]):
    """Directed edges neighbour -> atom for the k nearest neighbours of every atom."""
    from scipy.spatial import cKDTree

    p = np.mod(pos, box) if box is not None else pos
    if box is not None:
        p[p >= box] = 0.0
    tree = cKDTree(p, boxsize=box) if box is not None else cKDTree(p)
    dist, idx = tree.query(p, k=k + 1)
    n = pos.shape[0]
    dst = np.repeat(np.arange(n, dtype=np.int64), k)
    nb = idx[:, 1:]
    # drop self if it is not in column 0 (exact coincidences only)
    selfcol = idx[:, 0] != np.arange(n)
    if np.any(selfcol):
        raise RuntimeError("coincident atoms in k-NN graph")
    return nb.reshape(-1).astype(np.int64), dst


def sort_and_compress(src, dst, n):
    """Sort edges by (dst, src); return permutation and CSR row pointers."""
    order = np.lexsort((src, dst))
    counts = np.bincount(dst[order], minlength=n)
    row_ptr = np.zeros(n + 1, dtype=np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    return order, row_ptr


def edge_vectors(pos, src, dst, box):
    d = pos[src] - pos[dst]
    return _min_image(d, box).astype(np.float32)


def _finish(name, pos, box, src, dst, lmax, C, rng_feat, rng_w, rng_extra, path_set=0, r_cut=0.0,
            radial=False, linear=False, linear_bf16=False):
    n = pos.shape[0]
    order, row_ptr = sort_and_compress(src, dst, n)
    src = src[order]
    dst = dst[order]
    vec = edge_vectors(pos, src, dst, box)
    K = (lmax + 1) ** 2
    P = num_paths(lmax, path_set)
    x = rng_feat.standard_normal((n, C, K), dtype=np.float64).astype(np.float32)
    w = (rng_w.standard_normal((P, C)) / np.sqrt(P)).astype(np.float32)
    w_rad = None
    w_lin = None
    if radial:
        w_rad = (rng_extra.standard_normal((8, P * C)) / np.sqrt(8.0)).astype(np.float32)
    if linear:
        w_lin = (rng_extra.standard_normal((lmax + 1, C, C)) / np.sqrt(C)).astype(np.float32)
    if src.shape[0] >= 2 ** 31 or n >= 2 ** 31:
        raise ValueError("workload too large for int32 indices")
    return Workload(name=name, N=n, lmax=lmax, C=C, pos=pos, box=box, src=src.astype(np.int32),
                    dst=dst.astype(np.int32), vec=vec, row_ptr=row_ptr.astype(np.int32), x=x, w=w,
                    path_set=path_set, weight_mode=1 if radial else 0, r_cut=r_cut, w_rad=w_rad,
                    w_lin=w_lin, linear_bf16=linear_bf16)


CONFIG_NAMES = ("tiny", "typical", "mid", "large", "radial")


def cell_order(pos: np.ndarray, box: float, cell: float) -> np.ndarray:
    """Permutation that numbers atoms by the Morton (Z-order) index of their
    cubic cell of side ~``cell`` -- a spatially coherent numbering."""
    n_side = max(1, int(box // cell))
    ijk = np.clip(np.floor(np.mod(pos, box) / (box / n_side)).astype(np.int64), 0, n_side - 1)
    code = np.zeros(pos.shape[0], dtype=np.int64)
    for bit in range(21):
        for d in range(3):
            code |= ((ijk[:, d] >> bit) & 1) << (3 * bit + d)
    return np.argsort(code, kind="stable")


def make_config(name: str, seed: int = 2026, atom_order: str = "generation", path_set: int = 0) -> Workload:
    """Build one of the five named workloads (see the module docstring).

    ``atom_order="cell"`` renumbers the atoms of a periodic workload along a
    Morton curve over cells of side 2 A before the graph is built (a
    spatially coherent numbering, for comparison only); the default keeps the
    generation order, in which atom numbers carry no spatial information.
    ``path_set=1`` draws the path weights for the 34-path SO(3) set instead of
    the 23 parity-respecting paths (lmax 3; same graph and features)."""
    k = CONFIG_NAMES.index(name) + 1
    ss = np.random.SeedSequence([seed, k]).spawn(4)
    rng_pos, rng_feat, rng_w, rng_extra = (np.random.default_rng(s) for s in ss)
    if atom_order not in ("generation", "cell"):
        raise ValueError(atom_order)

    def place(n, box):
        pos = rng_pos.uniform(0.0, box, size=(n, 3))
        if atom_order == "cell":
            pos = pos[cell_order(pos, box, 2.0)]
        return pos
    if name == "tiny":
        n, box_side = 64, 6.0
        pos = rng_pos.uniform(0.0, box_side, size=(n, 3))
        src, dst = radius_edges_bruteforce(pos, 3.0, None)
        return _finish(name, pos, None, src, dst, 2, 8, rng_feat, rng_w, rng_extra, r_cut=3.0, path_set=path_set)
    if name == "typical":
        n = 1000
        box = (n / DENSITY) ** (1.0 / 3.0)
        pos = place(n, box)
        src, dst = knn_edges(pos, 20, box)
        return _finish(name, pos, box, src, dst, 3, 32, rng_feat, rng_w, rng_extra, linear=True, path_set=path_set)
    if name == "mid":
        n = 10000
        box = (n / DENSITY) ** (1.0 / 3.0)
        pos = place(n, box)
        src, dst = radius_edges(pos, 4.0, box)
        return _finish(name, pos, box, src, dst, 3, 64, rng_feat, rng_w, rng_extra, r_cut=4.0, linear=True,
                       linear_bf16=True, path_set=path_set)
    if name == "large":
        n = 100000
        box = (n / DENSITY) ** (1.0 / 3.0)
        pos = place(n, box)
        src, dst = radius_edges(pos, 5.0, box)
        return _finish(name, pos, box, src, dst, 3, 32, rng_feat, rng_w, rng_extra, r_cut=5.0, path_set=path_set)
    if name == "radial":
        n = 50000
        box = (n / DENSITY) ** (1.0 / 3.0)
        pos = place(n, box)
        src, dst = radius_edges(pos, 5.0, box)
        return _finish(name, pos, box, src, dst, 3, 128, rng_feat, rng_w, rng_extra, r_cut=5.0, radial=True,
                       path_set=path_set)
    raise KeyError(name)


def lmax_graph(lmax: int, C: int, seed: int = 2026, n: int = 2000, r_cut: float = 4.0, path_set: int = 0) -> Workload:
    """A periodic radius graph like the mid workload (density 0.1 / A^3, r_c =
    4 A: about 27 neighbours per atom) with n atoms and features of degree up
    to ``lmax`` (any lmax; for the edge-aligned form above 3)."""
    ss = np.random.SeedSequence([seed, 100 + lmax, C, n]).spawn(4)
    rng_pos, rng_feat, rng_w, rng_extra = (np.random.default_rng(s) for s in ss)
    box = (n / DENSITY) ** (1.0 / 3.0)
    pos = rng_pos.uniform(0.0, box, size=(n, 3))
    src, dst = radius_edges(pos, r_cut, box)
    return _finish("lmax%d" % lmax, pos, box, src, dst, lmax, C, rng_feat, rng_w, rng_extra, r_cut=r_cut,
                   path_set=path_set)


def random_permutation(wl: Workload, seed: int = 2026):
    """A seeded random edge order (for the unsorted / atomic path): returns
    (vec, src, dst) permuted, in the argument order of the convolution."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 99]))
    perm = rng.permutation(wl.E)
    return wl.vec[perm].copy(), wl.src[perm].copy(), wl.dst[perm].copy()


def small_graph(n: int, e_per_row: int, C: int, lmax: int, seed: int, path_set: int = 0,
                radial: bool = False, r_cut: float = 5.0, empty_rows=(), long_rows=(), long_len: int = 0,
                zero_vec_edges: int = 0) -> Workload:
    """A random ragged test graph: degrees vary around ``e_per_row``; rows in
    ``empty_rows`` get no edges, rows in ``long_rows`` get ``long_len`` edges;
    the first ``zero_vec_edges`` edges get a zero vector."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, n, C, lmax]))
    deg = rng.integers(max(0, e_per_row - 5), e_per_row + 6, size=n)
    for r in empty_rows:
        deg[r] = 0
    for r in long_rows:
        deg[r] = long_len
    dst = np.repeat(np.arange(n, dtype=np.int64), deg)
    src = rng.integers(0, n, size=dst.shape[0]).astype(np.int64)
    order, row_ptr = sort_and_compress(src, dst, n)
    src, dst = src[order], dst[order]
    E = src.shape[0]
    r = rng.uniform(0.5, 0.95 * r_cut, size=E)
    u = rng.standard_normal((E, 3))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    vec = (u * r[:, None]).astype(np.float32)
    vec[:zero_vec_edges] = 0.0
    K = (lmax + 1) ** 2
    P = num_paths(lmax, path_set)
    x = rng.standard_normal((n, C, K)).astype(np.float32)
    w = (rng.standard_normal((P, C)) / np.sqrt(P)).astype(np.float32)
    w_rad = (rng.standard_normal((8, P * C)) / np.sqrt(8.0)).astype(np.float32) if radial else None
    w_lin = (rng.standard_normal((lmax + 1, C, C)) / np.sqrt(C)).astype(np.float32)
    return Workload(name="small", N=n, lmax=lmax, C=C, pos=np.zeros((n, 3)), box=None, src=src.astype(np.int32),
                    dst=dst.astype(np.int32), vec=vec, row_ptr=row_ptr.astype(np.int32), x=x, w=w,
                    path_set=path_set, weight_mode=1 if radial else 0, r_cut=r_cut, w_rad=w_rad, w_lin=w_lin)


@dataclasses.dataclass
class InteractionWeights:
    W_up: np.ndarray    # [L+1, C, C]
    W1: np.ndarray      # [n_basis, H]
    W2: np.ndarray      # [H, H]
    W3: np.ndarray      # [H, P*C]
    W_out: np.ndarray   # [L+1, C, C]


def interaction_weights(lmax: int, C: int, path_set: int = 0, H: int = 64, n_basis: int = 8,
                        seed: int = 2026) -> InteractionWeights:
    """Seeded weights of one interaction layer (see the module docstring)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 7000 + lmax, C, H, path_set]))
    P = num_paths(lmax, path_set)
    f = lambda shape, var: (rng.standard_normal(shape) * np.sqrt(var)).astype(np.float32)
    return InteractionWeights(W_up=f((lmax + 1, C, C), 1.0 / C), W1=f((n_basis, H), 1.0 / n_basis),
                              W2=f((H, H), 1.0 / H), W3=f((H, P * C), 1.0 / H), W_out=f((lmax + 1, C, C), 1.0 / C))

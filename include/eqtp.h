/*
 * eqtp.h -- C ABI of the MI355X (gfx950) equivariant convolution library.
 *
 * The library computes, on one GPU, the hot path of an equivariant
 * message-passing convolution as the Batmobile page describes it ("Batmobile
 * CUDA kernel optimisation: a 10-20x acceleration strategy for equivariant
 * graph neural networks"):
 *   section "equivariant GNN compute bottleneck" -- real spherical harmonics
 *     of each edge direction, a Clebsch-Gordan tensor product with the source
 *     node's features, and message passing into the destination node;
 *   section "2. register intermediate computation" -- the harmonics for
 *     l <= 3 of the normalised edge vector, components per l in the order
 *     l0, l1c, l1s, l2c, l2s, ... (Y00, Y10, Y11c, Y11s first);
 *   section "1. compile-time constants" -- coupling coefficients compiled
 *     into the kernels, indexed by path;
 *   section "3. operator fusion" -- edge vectors [E,3], node features
 *     [N,C,16], source indices [E]; every edge vector read once.
 *
 * Conventions shared by every entry point
 *   - All pointers not marked "host" are device pointers allocated and owned
 *     by the caller.  The library allocates no device memory, performs no
 *     host<->device copies and never synchronises (debug mode, below
 *     eqtp_check_graph, is the one exception).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on it and the call returns immediately.
 *   - Return value: EQTP_OK (0) or an error code.  Argument errors are
 *     detected on the host before anything is launched (no partial writes).
 *     A failed launch returns EQTP_EHIP.  Device faults surface at the
 *     caller's next synchronisation.
 *   - Functions are thread-safe; the only mutable state is a per-device cache
 *     of the compute-unit count, read once through the HIP runtime, and the
 *     debug-mode switch.
 *   - Feature vectors use layout [N, C, K] with K = (lmax+1)^2: each
 *     channel's K components are contiguous, in the component order above.
 *   - Indices (src, dst, row_ptr) are int32.  Out-of-range index values are
 *     clamped inside the kernels so that no access leaves the buffers; the
 *     result for such inputs is unspecified.
 */
#ifndef EQTP_H
#define EQTP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define EQTP_OK 0
#define EQTP_EINVAL 1       /* bad argument (null pointer, size, alignment, enum) */
#define EQTP_EUNSUPPORTED 2 /* valid request this build does not implement */
#define EQTP_EHIP 3         /* the HIP runtime reported an error at launch */
#define EQTP_ETOOLARGE 4    /* eqtp_conv_fused_noalloc: the call needs more than the static scratch */
#define EQTP_EGRAPH 5       /* debug mode: the graph arrays fail eqtp_check_graph (nothing else launched) */

/* coupling path sets (paths are (l1 = feature l, l2 = harmonic l, l3 = output l)) */
#define EQTP_PATHS_PARITY 0 /* l1+l2+l3 even: 23 paths at lmax 3, 11 at lmax 2 */
#define EQTP_PATHS_SO3 1    /* every triangle-allowed triple: 34 at lmax 3, 15 at lmax 2 */

/* how the per-path, per-channel weights are given */
#define EQTP_W_FIXED 0  /* weights fp32 [P, C], shared by every edge */
#define EQTP_W_RADIAL 1 /* weights fp32 [n_basis, P*C]; per edge w_e[p,c] = sum_n R_n(r_e) W[n, p*C+c] */

/* edge order */
#define EQTP_EDGES_DST_SORTED 0 /* edges grouped by dst; row_ptr[N+1] gives each node's range */
#define EQTP_EDGES_UNSORTED 1   /* any order; dst[E] given; results summed with atomics */

/* algorithm of eqtp_conv_fused.  AUTO: NODE_MFMA for dst-sorted edges with
   fixed weights and lmax <= 3; EDGE_SO2 for dst-sorted edges with radial
   weights, fp32 features, lmax <= 3 and C a multiple of 16 (the radial
   products 8 -> P*C on the matrix cores, 16 edges at a time); EDGE_VALU for
   other lmax <= 3 cases; EDGE_SO2 for lmax 4..6. */
#define EQTP_ALGO_AUTO 0
#define EQTP_ALGO_NODE_MFMA 1 /* per node: outer-product sums on matrix cores, then the coupling */
#define EQTP_ALGO_EDGE_VALU 2 /* per edge: harmonics, coupling and product on the vector ALUs */
#define EQTP_ALGO_EDGE_SO2 3  /* per edge in the edge-aligned frame (E2Former-V2 page, section 2.1,
                                 "EAAS"): rotate x[src] so that the edge is the z axis, where the
                                 harmonics keep only m = 0 and the coupling is a sparse re-indexing,
                                 rotate back; vector ALUs; fixed weights, fp32 features; lmax 0..6
                                 (C = 128 above lmax 4 as two 64-channel halves).  Same result as
                                 the coupling form. */

/* element types: node features (eqtp_conv_desc.x_dtype) and the channel
   linear's operands (eqtp_linear's dtype) */
#define EQTP_F32 0      /* fp32 in memory, fp32 arithmetic */
#define EQTP_BF16 1     /* bfloat16 in memory */
#define EQTP_F32_BF16 2 /* eqtp_linear only: fp32 in memory, rounded to bfloat16 (nearest even) for the
                           matrix-core products */

/*
 * Number of coupling paths P for (lmax, path_set), or a negative status.
 * lmax in [0, 6] (above 3 only eqtp_conv_fused with EQTP_ALGO_EDGE_SO2 or
 * EQTP_ALGO_AUTO takes it).
 */
int eqtp_num_paths(int lmax, int path_set);

/*
 * Writes the path list in canonical order (lexicographic in (l1, l2, l3)) to
 * the host array l1l2l3 [P, 3].  Returns P or a negative status.  The weight
 * rows of eqtp_conv_fused follow this order.
 */
int eqtp_path_table(int lmax, int path_set, int32_t* l1l2l3 /* host */);

/*
 * Real spherical harmonics of edge vectors (Batmobile page, section
 * "2. register intermediate computation").
 *   vec [E, 3] fp32, any length; a zero vector gives (Y00, 0, ..., 0).
 *   Y   [E, (lmax+1)^2] fp32 output, 16-byte aligned; fully overwritten.
 *   lmax in [0, 6]; 0 <= E < 2^31.  lmax <= 3: closed-form polynomials;
 *   4..6: the Legendre-derivative recurrence in z times Re/Im (x + i y)^m.
 * Orthonormal harmonics with the Condon-Shortley phase:
 *   Y00 = 0.28209479177387814, Y10 = 0.4886025119029199 z,
 *   Y11c = -0.4886025119029199 x, Y11s = -0.4886025119029199 y (unit vector),
 *   Y_lm,c / Y_lm,s = sqrt2 Re / Im of the complex harmonic.
 */
int eqtp_sh(const float* vec, int64_t E, int lmax, float* Y, void* stream);

typedef struct eqtp_conv_desc {
  int32_t struct_size; /* = sizeof(eqtp_conv_desc) */
  int32_t lmax;        /* 0..3; 4..6 with EQTP_ALGO_EDGE_SO2 / EQTP_ALGO_AUTO */
  int32_t C;           /* channels: 8, 16, 32, 64 or 128 */
  int32_t path_set;    /* EQTP_PATHS_* */
  int32_t weight_mode; /* EQTP_W_* */
  int32_t edge_order;  /* EQTP_EDGES_* */
  int32_t algo;        /* EQTP_ALGO_* */
  float r_cut;         /* radial mode: cut-off radius (> 0) */
  int32_t n_basis;     /* radial mode: number of radial functions, must be 8 */
  int32_t x_dtype;     /* EQTP_F32 (default) or EQTP_BF16: x holds bfloat16 features,
                          same [N, C, K] layout, 2 bytes each (eqtp_conv_fused at
                          lmax <= 3).  A descriptor whose struct_size ends before
                          this field is read as EQTP_F32. */
  int32_t out_dtype;   /* EQTP_F32 (default) or EQTP_BF16: eqtp_conv_fused writes a
                          bfloat16 out, summed with packed bf16 atomics (edges in
                          any order, lmax <= 3; see eqtp_conv_fused).  A descriptor
                          whose struct_size ends before this field is read as
                          EQTP_F32. */
} eqtp_conv_desc;

/* struct_size of a descriptor without the x_dtype field (still accepted) */
#define EQTP_CONV_DESC_SIZE_V1 36
/* struct_size of a descriptor without the out_dtype field (still accepted) */
#define EQTP_CONV_DESC_SIZE_V2 40

/*
 * Fused convolution: spherical harmonics -> coupling with the source
 * features -> sum into the destination node (Batmobile page, sections
 * "2." and "3."):
 *   out[n, c, l3 m3] = sum_{e : dst_e = n} sum_{p = (l1,l2,l3)} w_e[p, c]
 *                      sum_{m1, m2} C^p[m1, m2, m3] x[src_e, c, l1 m1] Y_{l2 m2}(vec_e)
 * with real-basis coupling coefficients C^p (odd l1+l2+l3 paths of the SO3
 * set use the imaginary part of the purely imaginary real-basis block).
 *   d        host descriptor (read during the call only).
 *   N, E     nodes and edges, 0 <= N, E < 2^31 (E > 0 requires N > 0).
 *   vec      [E, 3] fp32 edge vectors.
 *   src      [E] int32 source node of each edge.
 *   dst      [E] int32 destination node; required for EQTP_EDGES_UNSORTED,
 *            ignored (may be NULL) for EQTP_EDGES_DST_SORTED.
 *   row_ptr  [N+1] int32 CSR row pointers over dst-sorted edges
 *            (row_ptr[0] = 0, row_ptr[N] = E, non-decreasing); required for
 *            EQTP_EDGES_DST_SORTED, ignored for EQTP_EDGES_UNSORTED.
 *   x        [N, C, K] node features, 16-byte aligned: fp32, or bfloat16 when
 *            d->x_dtype = EQTP_BF16 (lmax <= 3; either edge order, fixed or
 *            radial weights; EQTP_ALGO_EDGE_SO2 gives EQTP_EUNSUPPORTED).  The
 *            bf16 values are widened exactly; every product, sum and atomic
 *            add is fp32 either way (out stays fp32).
 *   weights  EQTP_W_FIXED: [P, C] fp32; EQTP_W_RADIAL: [8, P*C] fp32 with
 *            R_n(r) = sin(n pi r / r_cut) / r * u(r / r_cut), n = 1..8,
 *            u(d) = 1 - 28 d^6 + 48 d^7 - 21 d^8 for d < 1, else 0
 *            (limit n pi / r_cut at r = 0).
 *   out      [N, C, K] fp32, 16-byte aligned, fully overwritten (nodes with
 *            no incoming edge get zeros); must not alias any input.
 *            d->out_dtype = EQTP_BF16 (EQTP_EDGES_UNSORTED, lmax <= 3,
 *            EQTP_ALGO_AUTO or EQTP_ALGO_EDGE_VALU; EQTP_EUNSUPPORTED
 *            otherwise): out is [N, C, K] bfloat16, zero-filled, and every
 *            edge's message -- computed in fp32 -- is rounded to bf16 (nearest
 *            even) and added with packed two-element bf16 atomics, so each
 *            partial sum is rounded to bf16 as well: half the atomic
 *            operations and output bytes, at bf16 accuracy (the Batmobile
 *            page's extensions, mixed precision).
 * Sorted edges: deterministic (bit-identical from run to run).  Unsorted
 * edges: summation order varies from run to run.
 * lmax 4..6 (EQTP_ALGO_EDGE_SO2): fixed weights and fp32 features only
 * (EQTP_EUNSUPPORTED otherwise), any C (C = 128 above lmax 4 runs as two
 * launches over 64-channel halves); both edge orders.
 * EQTP_ALGO_EDGE_SO2 with radial weights: dst-sorted edges, fp32 features,
 * lmax <= 3 and C a multiple of 16 only.
 */
int eqtp_conv_fused(const eqtp_conv_desc* d, int64_t N, int64_t E, const float* vec, const int32_t* src,
                    const int32_t* dst, const int32_t* row_ptr, const void* x, const float* weights, void* out,
                    void* stream);

/*
 * Bytes of device workspace eqtp_conv_fused_ws needs for (d, N, E): for
 * EQTP_EDGES_UNSORTED with N > 0, 256-byte aligned regions for row pointers
 * [N+1], five int arrays [E] (the sort's keys and edge indices, later the
 * grouped vectors [E,3] and sources [E]) and the sort's digit counts (about
 * 20.5 bytes per edge); 0 for dst-sorted edges.  Negative status for a bad
 * descriptor or sizes.
 */
int64_t eqtp_conv_workspace_bytes(const eqtp_conv_desc* d, int64_t N, int64_t E);

/*
 * The fused convolution of eqtp_conv_fused with a caller-given workspace.
 * Dst-sorted edges: exactly eqtp_conv_fused (the workspace is not touched).
 * Edges in any order (d->edge_order = EQTP_EDGES_UNSORTED, dst given): the
 * edges are first grouped by destination in the workspace -- a stable radix
 * sort on the GPU, so every row keeps its edges' input order and the grouping
 * does not depend on the order of hardware atomics -- and the call then runs as for
 * dst-sorted edges (d->algo as there; row_ptr is ignored).  The result is
 * deterministic (bit-identical from call to call) and no atomics touch out.
 * The grouping is layout preparation for the destination sum of the
 * Batmobile page's section "3. operator fusion"; the page has no sort.
 *   workspace        device memory of at least eqtp_conv_workspace_bytes(d,
 *                    N, E) bytes, 16-byte aligned, owned by the caller; its
 *                    contents on entry do not matter and are overwritten.
 *   workspace_bytes  its size.
 * Other arguments, layouts and errors as for eqtp_conv_fused; a missing or
 * short workspace gives EQTP_EINVAL before any launch.  Asynchronous on
 * stream; the workspace must not be reused by another call before this one
 * has finished on the stream.
 */
int eqtp_conv_fused_ws(const eqtp_conv_desc* d, int64_t N, int64_t E, const float* vec, const int32_t* src,
                       const int32_t* dst, const int32_t* row_ptr, const void* x, const float* weights, float* out,
                       void* workspace, int64_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): exactly
 * eqtp_conv_fused_ws, with the workspace taken from a static array of the
 * library (128 MiB per device, reserved while the process runs) instead of
 * the caller.  The call allocates nothing.  A request whose workspace
 * (eqtp_conv_workspace_bytes) exceeds 128 MiB -- e.g. more than about six
 * million edges in any order -- returns EQTP_ETOOLARGE before any launch;
 * dst-sorted edges need none.  Every call on a device shares that device's
 * array, so calls that overlap on one device (other streams, other threads)
 * race and must be serialised by the caller; consecutive calls on one stream
 * are safe.  The first call on a device looks up the array's address there.
 * Arguments, layouts, results and other errors as for eqtp_conv_fused_ws.
 */
int eqtp_conv_fused_noalloc(const eqtp_conv_desc* d, int64_t N, int64_t E, const float* vec, const int32_t* src,
                            const int32_t* dst, const int32_t* row_ptr, const void* x, const float* weights,
                            float* out, void* stream);

/*
 * Per-edge messages, without the destination sum (the page's fused kernel,
 * section "3. operator fusion": edge vectors [E,3], node features [N,C,16],
 * source indices [E] in, messages [E,C,16] out):
 *   messages[e, c, l3 m3] = sum_p w_e[p, c] sum_{m1, m2} C^p[m1, m2, m3] x[src_e, c, l1 m1] Y_{l2 m2}(vec_e)
 * d: lmax, C, path_set, weight_mode, r_cut, n_basis as for eqtp_conv_fused
 * (edge_order is ignored); N, E, vec, src, x, weights as there.  Fixed
 * weights use the edge-aligned form (any C) unless d->algo =
 * EQTP_ALGO_EDGE_VALU asks for the coupling form (lmax <= 3); radial weights
 * use the coupling form (lmax <= 3; EQTP_ALGO_EDGE_SO2 gives
 * EQTP_EUNSUPPORTED).  Both forms give the same messages to rounding.
 *   messages [E, C, K] fp32, 16-byte aligned, fully overwritten; must not
 *            alias an input (d->out_dtype must be EQTP_F32).  Deterministic.
 */
int eqtp_conv_messages(const eqtp_conv_desc* d, int64_t N, int64_t E, const float* vec, const int32_t* src,
                       const float* x, const float* weights, float* messages, void* stream);

/*
 * Gradients of the fused convolution: for a scalar loss L with
 * grad_out = dL/dout, with fixed weights,
 *   grad_x[s, c, l1 m1] = sum_{e: src_e = s} sum_p w[p, c] sum_{m2, m3} C^p[m1, m2, m3] Y_{l2 m2}(vec_e)
 *                         grad_out[dst_e, c, l3 m3]
 *   grad_w[p, c]        = sum_e sum_{m1, m2, m3} C^p x[src_e, c, l1 m1] Y_{l2 m2}(vec_e) grad_out[dst_e, c, l3 m3]
 *   grad_vec[e]         = sum_{l2 m2} dL/dY_{l2 m2}(vec_e) * dY_{l2 m2}/dvec_e
 * (the forces of an interatomic potential are built from grad_vec; the page
 * names a PyTorch autograd function with a backward as the integration path,
 * section "extension possibilities").  With radial weights
 * (d->weight_mode = EQTP_W_RADIAL, w_e[p,c] = sum_b R_b(|vec_e|) W[b, p*C+c]
 * as in eqtp_conv_fused) w becomes w_e in grad_x and dL/dY, and
 *   grad_W[b, p*C + c] = sum_e R_b(r_e) T_e[p, c],
 *   T_e[p, c] = sum C^p x[src_e, c, l1 m1] Y_{l2 m2}(vec_e) grad_out[dst_e, c, l3 m3],
 *   grad_vec[e] += (sum_b R_b'(r_e) sum_{p,c} W[b, p*C+c] T_e[p, c]) vec_e / r_e
 * (the product and chain rule through the radial basis; R_b' = dR_b/dr).
 * A zero-length edge vector has grad_vec = 0.
 * Fixed weights (d->algo = EQTP_ALGO_AUTO -- see below -- or
 * EQTP_ALGO_EDGE_SO2, and always at lmax 4..6): the edge-aligned form
 * (E2Former-V2 page, section 2.1), where grad_x
 * and grad_w come from the sparse coupling in each edge's frame and grad_vec
 * from the generators of rotations about the frame's x and y axes acting on
 * the rotated features (same formulas as above, to rounding); C = 128 above
 * lmax 4 runs as two launches over 64-channel halves (the second adds its
 * channels' share of grad_vec).
 *   d, N, E, vec, src, dst, row_ptr, x, weights: as for eqtp_conv_fused
 *            (x fp32, 16-byte aligned; lmax 0..6).  Radial weights: lmax
 *            0..3, C a multiple of 16, n_basis 8, r_cut > 0 (else
 *            EQTP_EUNSUPPORTED / EQTP_EINVAL); weights [8, P*C] fp32.
 *   grad_out [N, C, K] fp32, 16-byte aligned.
 *   grad_x   [N, C, K] fp32, 16-byte aligned, or NULL (not computed).
 *   grad_w   [P, C] fp32 (fixed weights) or [8, P*C] (radial), or NULL.
 *   grad_vec [E, 3] fp32, or NULL.
 * Each requested output is fully overwritten; outputs must not alias inputs
 * or each other.  grad_x and grad_w are sums of fp32 atomics (their
 * summation order varies from run to run); with fixed weights grad_vec is
 * written once per edge, with radial weights it is a sum of fp32 atomics
 * (two per 16-channel block).  Errors as for eqtp_conv_fused.  d->algo
 * (fixed weights, lmax <= 3): EQTP_ALGO_AUTO takes the edge-aligned form
 * when grad_x or grad_w is requested (it is the faster one there at every
 * lmax and channel count), and the coupling form for grad_vec alone (the
 * faster one there: for dst-sorted edges the per-edge walk below lmax 3 and
 * the matrix cores at lmax 3).  EQTP_ALGO_NODE_MFMA and EQTP_ALGO_EDGE_VALU
 * always select the coupling form -- grad_x and grad_w by a walk of the
 * coupling per edge on the vector ALUs, and grad_vec, for dst-sorted edges,
 * on the matrix cores (dL/dY_e = x[src_e] contracted with a per-node B_d
 * built from grad_out; EQTP_ALGO_NODE_MFMA) or by the same per-edge walk
 * (EQTP_ALGO_EDGE_VALU, and for edges in any order).  Radial weights ignore
 * d->algo.  d->x_dtype and d->out_dtype must
 * be EQTP_F32 (EQTP_EUNSUPPORTED for EQTP_BF16).
 */
int eqtp_conv_backward(const eqtp_conv_desc* d, int64_t N, int64_t E, const float* vec, const int32_t* src,
                       const int32_t* dst, const int32_t* row_ptr, const float* x, const float* weights,
                       const float* grad_out, float* grad_x, float* grad_w, float* grad_vec, void* stream);

/*
 * The gradients of eqtp_conv_backward (same formulas) from a copy of the edges
 * grouped by SOURCE node, so that grad_x[s] is summed over the source's edges
 * in one place and written once: no atomics on grad_x, deterministic.
 *   src_ptr [N+1] int32: CSR over source nodes (src_ptr[N] = E);
 *   vec_s   [E, 3] fp32 and dst_s [E] int32: each edge's vector (pointing
 *           from its source to its destination, as in the forward) and its
 *           destination, in source-grouped order;
 *   perm    [E] int32: perm[i] = the index, in the caller's edge order, of
 *           grouped edge i (needed with grad_vec only, else may be NULL).
 *   eqtp_sort_edges(N, E, src, vec, dst, src_ptr, perm, vec_s, dst_s, ...)
 *   produces all four from the forward's arrays (eqtp_edge_rows gives dst from
 *   a dst-sorted CSR).
 *   x [N, C, K] fp32 16-byte aligned (needed for grad_w and grad_vec, and
 *   always with radial weights or the edge-aligned form; else may be NULL);
 *   grad_out [N, C, K] fp32 16-byte aligned; weights [P, C] fp32 (fixed) or
 *   [8, P*C] (radial).
 *   grad_x   [N, C, K] fp32 16-byte aligned, fully overwritten (zeros for nodes
 *            that are no edge's source), deterministic; or NULL.
 *   grad_w   [P, C] or [8, P*C] fp32, a sum of fp32 atomics; or NULL.
 *   grad_vec [E, 3] fp32 in the caller's edge order (entry perm[i] for grouped
 *            edge i), fully overwritten; or NULL.  Not all three NULL.
 * How: fixed weights at lmax <= 3 (the default): grad_x and grad_w by the
 * adjoint of the node-factored forward on the matrix cores,
 *   H_s[c, m3, m2] = sum_{e: src_e = s} grad_out[dst_e, c, m3] Y_m2(vec_e),
 *   grad_x[s, c, m1] = sum_p w[p, c] sum_{m2, m3} C^p[m1, m2, m3] H_s[c, m3, m2],
 *   grad_w[p, c] = sum_s sum_{m1} x[s, c, m1] sum_{m2, m3} C^p[m1, m2, m3] H_s[c, m3, m2],
 * and grad_vec by a walk in the edge frame; fixed weights at lmax 4..6 (or
 * d->algo = EQTP_ALGO_EDGE_SO2): all three by one walk in the edge frame (C =
 * 128 above lmax 4 as two 64-channel halves); radial weights (lmax 0..3, C a multiple of 16,
 * n_basis 8, r_cut > 0): all three by one walk in the edge frame.
 * d: lmax, C, path_set, weight_mode, r_cut, n_basis, algo, x_dtype and
 * out_dtype (both must be EQTP_F32); edge_order is ignored.  Errors as for
 * eqtp_conv_backward.
 */
int eqtp_conv_backward_by_source(const eqtp_conv_desc* d, int64_t N, int64_t E, const float* vec_s,
                                 const int32_t* dst_s, const int32_t* src_ptr, const float* x, const float* weights,
                                 const float* grad_out, float* grad_x, float* grad_w, const int32_t* perm,
                                 float* grad_vec, void* stream);

/*
 * rows[e] = the row n with row_ptr[n] <= e < row_ptr[n+1] (the destination of
 * each edge of a dst-sorted CSR), for 0 <= e < E.  row_ptr [N+1] int32 as for
 * eqtp_conv_fused; rows [E] int32 out.  EQTP_EINVAL for bad sizes or
 * NULL / misaligned pointers when E > 0; asynchronous on stream.
 */
int eqtp_edge_rows(int64_t N, int64_t E, const int32_t* row_ptr, int32_t* rows, void* stream);

/*
 * Groups edges given in any order by destination node (a counting sort on the
 * GPU), producing what the dst-sorted convolution takes.  Layout preparation
 * for the message-passing step that the Batmobile page, section "3. operator
 * fusion", chains after the tensor product; the sort itself is not on the
 * page (a plain counting sort by destination).  Outputs:
 *   row_ptr    [N+1] int32 out: CSR row pointers (row_ptr[N] = E);
 *   perm       [E] int32 out: perm[i] = index (in the input order) of the
 *              edge placed at sorted position i;
 *   vec_sorted [E, 3] fp32 out = vec[perm], or NULL (then vec may be NULL);
 *   src_sorted [E] int32 out = src[perm], or NULL (then src may be NULL).
 *   dst        [E] int32 in, 0 <= dst < N (values outside are clamped).
 * The order of the edges inside a row is unspecified and may differ from call
 * to call (it follows the order of hardware atomics); everything else is
 * unique.  No scratch memory: row_ptr serves as the counter array.
 * 0 <= N < 2^31 - 1, 0 <= E < 2^31, E > 0 requires N > 0; row_ptr is never
 * NULL (N = 0 writes row_ptr[0] = 0).  dst and perm may be NULL when E = 0.
 * Returns EQTP_EINVAL for bad sizes, NULL or misaligned pointers (checked
 * before anything is launched), else the launch status.  Asynchronous on
 * stream; the caller owns every buffer.
 */
int eqtp_sort_edges(int64_t N, int64_t E, const int32_t* dst, const float* vec, const int32_t* src, int32_t* row_ptr,
                    int32_t* perm, float* vec_sorted, int32_t* src_sorted, void* stream);

/*
 * eqtp_sort_edges with every row in input order: a stable LSD radix sort of
 * (key, edge index) on the GPU (digits of up to 9 bits, per-tile digit
 * counts in LDS, one scan per digit, ranks from wave ballots), so all
 * outputs, perm included, are unique and the same from call to call -- what
 * makes sums taken in the grouped order deterministic (grad_x of
 * eqtp_conv_backward_by_source, which sums each source row's edges in that
 * order and writes it once).  Same arguments, layouts
 * and errors as eqtp_sort_edges, plus:
 *   workspace        device memory of at least eqtp_sort_workspace_bytes(N, E)
 *                    bytes (about 12 bytes per edge plus the digit counts),
 *                    16-byte aligned, owned by the caller; its contents on
 *                    entry do not matter.  May be NULL when E = 0.
 *   workspace_bytes  its size (EQTP_EINVAL when short).
 */
int64_t eqtp_sort_workspace_bytes(int64_t N, int64_t E);
int eqtp_sort_edges_stable(int64_t N, int64_t E, const int32_t* dst, const float* vec, const int32_t* src,
                           int32_t* row_ptr, int32_t* perm, float* vec_sorted, int32_t* src_sorted, void* workspace,
                           int64_t workspace_bytes, void* stream);

/*
 * Per-l channel linear (channel mixing inside each irrep, no bias), the
 * channel-wise mixing that follows the convolution: the Batmobile page names
 * no such layer; its form (a C x C matrix per degree l, applied to every m of
 * that degree, "bf16 in, fp32 accumulate" on the matrix cores) is this
 * library's reading of the workload it is measured on.
 *   out[n, c', l m] = sum_c W[l, c', c] h[n, c, l m]
 *   dtype    EQTP_F32:      h, W fp32; fp32 matrix-core products.
 *            EQTP_BF16:     h, W bfloat16 in memory; bf16 matrix-core products,
 *                           fp32 accumulation.
 *            EQTP_F32_BF16: h, W fp32 in memory, each value rounded to bf16
 *                           (nearest even) as it is loaded; bf16 products,
 *                           fp32 accumulation (for an fp32 h straight from
 *                           eqtp_conv_fused).
 *   h    [N, C, K] in the dtype's storage type, 16-byte aligned (read only).
 *   W    [lmax+1, C, C] (output-channel major) in the same storage type,
 *        16-byte aligned (read only).
 *   out  [N, C, K] fp32, 16-byte aligned, fully overwritten; must not alias
 *        h or W.
 *   C in {8, 16, 32, 64, 128}, lmax in [0, 6], 0 <= N < 2^31.  Caller-owned
 *   device buffers; asynchronous on stream; deterministic.  EQTP_EINVAL for
 *   bad sizes, enums, NULL or misaligned pointers (before any launch).
 */
int eqtp_linear(int64_t N, int C, int lmax, int dtype, const void* h, const void* W, float* out, void* stream);

/*
 * One interaction layer of an equivariant interatomic potential on node
 * features h, around the fused convolution.  The page names an end-to-end
 * layer benchmark (section "deployment", benchmark of an end-to-end MACE
 * layer) but not its parts; this is the plainest layer built from what the
 * page and this library define, in this order:
 *   h1  = linear(h, W_up)                 per-l channel linear (eqtp_linear), W_up [lmax+1, C, C]
 *   R_b = radial basis of |vec_e|         the 8 functions of the radial weights (cut-off r_cut)
 *   a   = SiLU(R W1),  phi_e = SiLU(a W2) radial network, W1 [8, H], W2 [H, H], no bias,
 *                                         SiLU(t) = t / (1 + exp(-t))
 *   w_e = phi_e W3                        per-edge path weights, W3 [H, P*C]
 *   m   = conv(h1; w_e)                   the fused convolution with the per-edge weights w_e
 *   out = linear(m, W_out) / norm         W_out [lmax+1, C, C]; norm > 0 (e.g. the mean degree)
 * H = 64.  Edges dst-sorted (row_ptr), lmax 0..3, C 16, 32, 64 or 128,
 * any path set.  The last network layer (w_e) is applied on the matrix cores
 * inside the convolution kernel; w_e never reaches memory.
 *   d          lmax, C, path_set, r_cut (> 0), n_basis (must be 8), hidden
 *              (must be 64), norm (> 0).
 *   vec, src, row_ptr  as for eqtp_conv_fused with dst-sorted edges.
 *   h, out     [N, C, K] fp32, 16-byte aligned; out must not alias an input.
 *   W_up, W_out [lmax+1, C, C] fp32, 16-byte aligned (output channel major).
 *   W1 [8, 64], W2 [64, 64], W3 [64, P*C] fp32, 4-byte aligned.
 *   workspace  device memory of at least eqtp_interaction_workspace_bytes
 *              bytes, 16-byte aligned, owned by the caller (h1, m and phi).
 * Errors as for eqtp_conv_fused (EQTP_EINVAL / EQTP_EUNSUPPORTED before any
 * launch, EQTP_EHIP at launch).  Asynchronous on stream; deterministic.
 */
typedef struct eqtp_interaction_desc {
  int32_t struct_size; /* = sizeof(eqtp_interaction_desc) */
  int32_t lmax;        /* 0..3 */
  int32_t C;           /* 16, 32, 64 or 128 */
  int32_t path_set;    /* EQTP_PATHS_* */
  float r_cut;         /* cut-off radius of the radial basis (> 0) */
  int32_t n_basis;     /* must be 8 */
  int32_t hidden;      /* must be 64 */
  float norm;          /* the output is divided by it (> 0) */
} eqtp_interaction_desc;

/* Workspace bytes of eqtp_interaction for N nodes and E edges (a negative
 * status for invalid arguments). */
int64_t eqtp_interaction_workspace_bytes(const eqtp_interaction_desc* d, int64_t N, int64_t E);

int eqtp_interaction(const eqtp_interaction_desc* d, int64_t N, int64_t E, const float* vec, const int32_t* src,
                     const int32_t* row_ptr, const float* h, const float* W_up, const float* W1, const float* W2,
                     const float* W3, const float* W_out, float* out, void* workspace, int64_t workspace_bytes,
                     void* stream);

/* Static description of a status code (never NULL). */
const char* eqtp_status_string(int status);

/*
 * Graph checks, the debugging aid for the index arrays every kernel trusts
 * (the PyTorch custom-operator tutorial page, chapter 5, debugging and best
 * practices: look at the last launch error, run a memory checker, synchronise
 * to find which launch went wrong).  The kernels clamp out-of-range indices
 * so that no access leaves the buffers; this call says whether any clamp
 * would act, and where.  Each array may be NULL (its checks are skipped):
 *   row_ptr  [N+1] int32: CSR rows (row_ptr[0] = 0, non-decreasing,
 *            row_ptr[N] = E); for edges grouped by source pass src_ptr here.
 *   src      [E] int32, each in [0, N).
 *   dst      [E] int32, each in [0, N); with row_ptr also given, each edge e
 *            must lie in row dst[e] of the CSR.
 *   vec      [E, 3] fp32, every component finite.
 *   report   [EQTP_CHECK_WORDS] int32, device, out (the caller's; 4-byte
 *            aligned); fully written:
 *     [0] edges with src outside [0, N)       [1] edges with dst outside [0, N)
 *     [2] rows with row_ptr[r+1] < row_ptr[r]  [3] endpoint faults (row_ptr[0]
 *         != 0 and row_ptr[N] != E count one each)
 *     [4] edges outside the row their dst names  [5] edges with a non-finite
 *         vector component
 *     [6] smallest edge index counted in [0], [1], [4] or [5], or -1
 *     [7] smallest row index counted in [2], or -1
 * The report is a set of counts, so it is the same from run to run.
 * 0 <= N, E < 2^31.  EQTP_EINVAL for bad sizes or a NULL / misaligned report
 * or array (before any launch), else the launch status.  Asynchronous on
 * stream; reads only the arrays given.
 */
#define EQTP_CHECK_WORDS 8
int eqtp_check_graph(int64_t N, int64_t E, const int32_t* row_ptr, const int32_t* src, const int32_t* dst,
                     const float* vec, int32_t* report, void* stream);

/*
 * Debug mode.  When on, every entry point that takes a graph (the
 * convolutions, messages, gradients, edge grouping and the interaction layer)
 * first runs eqtp_check_graph on the arrays it will read (and on perm for the
 * source-grouped gradients), waits for the report on its stream and returns
 * EQTP_EGRAPH, with nothing else launched, if any count is non-zero.  Debug
 * calls synchronise the stream and share one small static report per device
 * (calls are serialised by a host lock), so they are for finding bad inputs,
 * not for graph capture or timing.  The initial setting comes from the
 * environment variable EQTP_DEBUG when the library is loaded (set and not
 * "0" = on).  eqtp_set_debug(on) sets it for the whole process (on = 0 or 1;
 * any other value leaves it unchanged) and returns the previous setting.
 */
int eqtp_set_debug(int on);

/*
 * Test-only: walks the dst-sorted edges with exactly the row -> wave ->
 * lane -> step schedule that eqtp_conv_fused uses for the given (C, lmax,
 * algo) and, instead of the tensor product, counts the edges each node
 * receives and sums their src indices:
 *   count   [N] int32 output, src_sum [N] int64 output (fully overwritten).
 * algo: EQTP_ALGO_NODE_MFMA or EQTP_ALGO_EDGE_VALU.  Other arguments as in
 * eqtp_conv_fused.
 */
int eqtp_test_segment_probe(const int32_t* row_ptr, const int32_t* src, int64_t N, int64_t E, int C, int lmax,
                            int algo, int32_t* count, int64_t* src_sum, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* EQTP_H */

// abi.hip -- the extern "C" entry points declared in include/eqtp.h:
// argument validation, kernel selection and launch on the caller's stream.
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/eqtp.h"
#include "eqtp_device.hpp"
#include "eqtp_kernels.hpp"
#include "generated/so2_tables.inc"

// The static scratch of eqtp_conv_fused_noalloc: the workspace of the grouping
// by destination, one array per device (each GPU holds its own copy for the
// life of the process).  Host code never uses this name as an address: the
// device address comes from hipGetSymbolAddress, once per device.
constexpr int64_t kScratchBytes = (int64_t)128 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Debug mode's report: the graph check's words, then those of the check of a
// permutation (source-grouped gradients); one array per device, used under
// g_debug_mu only, addressed like the scratch above.
static __device__ __align__(16) int32_t debug_report[2 * eqtp::kCheckWords];

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool valid_c(int C) { return C == 8 || C == 16 || C == 32 || C == 64 || C == 128; }

static_assert(offsetof(eqtp_conv_desc, x_dtype) == EQTP_CONV_DESC_SIZE_V1, "descriptor layout");
static_assert(offsetof(eqtp_conv_desc, out_dtype) == EQTP_CONV_DESC_SIZE_V2, "descriptor layout");

// descriptor version check: the current size, or the size before out_dtype, or before x_dtype
bool desc_ok(const eqtp_conv_desc* d) {
  return d && (d->struct_size == (int32_t)sizeof(eqtp_conv_desc) || d->struct_size == EQTP_CONV_DESC_SIZE_V2 ||
               d->struct_size == EQTP_CONV_DESC_SIZE_V1);
}
int desc_x_dtype(const eqtp_conv_desc* d) {
  return d->struct_size >= EQTP_CONV_DESC_SIZE_V2 ? d->x_dtype : EQTP_F32;
}
int desc_out_dtype(const eqtp_conv_desc* d) {
  return d->struct_size >= (int32_t)sizeof(eqtp_conv_desc) ? d->out_dtype : EQTP_F32;
}
// status for the entry points whose outputs are fp32 only
int out_f32_only(const eqtp_conv_desc* d) {
  const int o = desc_out_dtype(d);
  return o == EQTP_F32 ? EQTP_OK : (o == EQTP_BF16 ? EQTP_EUNSUPPORTED : EQTP_EINVAL);
}
constexpr int64_t kMaxIndex = (int64_t(1) << 31) - 1;

// path counts and lists for lmax 0..6 (the same canonical order in both
// generated tables; lmax <= 3 also has the coupling-form tables)
int num_paths_host(int lmax, int path_set) {
  static const int parity[7] = {eqtp_gen::kSo2NumPaths_L0_parity, eqtp_gen::kSo2NumPaths_L1_parity,
                                eqtp_gen::kSo2NumPaths_L2_parity, eqtp_gen::kSo2NumPaths_L3_parity,
                                eqtp_gen::kSo2NumPaths_L4_parity, eqtp_gen::kSo2NumPaths_L5_parity,
                                eqtp_gen::kSo2NumPaths_L6_parity};
  static const int so3[7] = {eqtp_gen::kSo2NumPaths_L0_so3, eqtp_gen::kSo2NumPaths_L1_so3,
                             eqtp_gen::kSo2NumPaths_L2_so3, eqtp_gen::kSo2NumPaths_L3_so3,
                             eqtp_gen::kSo2NumPaths_L4_so3, eqtp_gen::kSo2NumPaths_L5_so3,
                             eqtp_gen::kSo2NumPaths_L6_so3};
  static_assert(eqtp_gen::kSo2NumPaths_L3_parity == eqtp_gen::kNumPaths_L3_parity, "path tables");
  static_assert(eqtp_gen::kSo2NumPaths_L3_so3 == eqtp_gen::kNumPaths_L3_so3, "path tables");
  if (lmax < 0 || lmax > eqtp::kSo2MaxL) return -EQTP_EUNSUPPORTED;
  if (path_set == EQTP_PATHS_PARITY) return parity[lmax];
  if (path_set == EQTP_PATHS_SO3) return so3[lmax];
  return -EQTP_EINVAL;
}

const eqtp_gen::PathLs* path_list(int lmax, int path_set) {
  static const eqtp_gen::PathLs* parity[7] = {eqtp_gen::kSo2Paths_L0_parity, eqtp_gen::kSo2Paths_L1_parity,
                                              eqtp_gen::kSo2Paths_L2_parity, eqtp_gen::kSo2Paths_L3_parity,
                                              eqtp_gen::kSo2Paths_L4_parity, eqtp_gen::kSo2Paths_L5_parity,
                                              eqtp_gen::kSo2Paths_L6_parity};
  static const eqtp_gen::PathLs* so3[7] = {eqtp_gen::kSo2Paths_L0_so3, eqtp_gen::kSo2Paths_L1_so3,
                                           eqtp_gen::kSo2Paths_L2_so3, eqtp_gen::kSo2Paths_L3_so3,
                                           eqtp_gen::kSo2Paths_L4_so3, eqtp_gen::kSo2Paths_L5_so3,
                                           eqtp_gen::kSo2Paths_L6_so3};
  return path_set == EQTP_PATHS_PARITY ? parity[lmax] : so3[lmax];
}

int status_of(hipError_t e) { return e == hipSuccess ? EQTP_OK : EQTP_EHIP; }

// ---- debug mode: graph checks before each launch (see eqtp_set_debug) ----
int debug_from_env() {
  const char* v = getenv("EQTP_DEBUG");
  return (v != nullptr && v[0] != '\0' && strcmp(v, "0") != 0) ? 1 : 0;
}
std::atomic<int> g_debug{debug_from_env()};
std::mutex g_debug_mu;
constexpr int kMaxDebugDevices = 64;
int32_t* g_debug_report[kMaxDebugDevices] = {};

// Runs the graph check (and, with perm, the check that perm holds edge
// indices in [0, E)) on the stream, waits for the report and returns
// EQTP_EGRAPH if any count is non-zero.  A no-op returning EQTP_OK when debug
// mode is off.  Arrays may be NULL (their checks are skipped).
int debug_check(int64_t N, int64_t E, const int32_t* row_ptr, const int32_t* src, const int32_t* dst,
                const float* vec, const int32_t* perm, void* stream) {
  if (!g_debug.load(std::memory_order_relaxed)) return EQTP_OK;
  if (N == 0 && E == 0) return EQTP_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return EQTP_EHIP;
  if (dev < 0 || dev >= kMaxDebugDevices) return EQTP_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_debug_mu);
  if (g_debug_report[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(debug_report)) != hipSuccess || p == nullptr) return EQTP_EHIP;
    g_debug_report[dev] = static_cast<int32_t*>(p);
  }
  int32_t* rep = g_debug_report[dev];
  const hipStream_t st = (hipStream_t)stream;
  if (E == 0) src = dst = perm = nullptr, vec = nullptr;
  if (eqtp::launch_check_graph(N, E, row_ptr, src, dst, vec, rep, st) != hipSuccess) return EQTP_EHIP;
  if (perm && eqtp::launch_check_graph(E, E, nullptr, perm, nullptr, nullptr, rep + eqtp::kCheckWords, st) !=
                  hipSuccess)
    return EQTP_EHIP;
  int32_t host[2 * eqtp::kCheckWords] = {};
  const int words = perm ? 2 * eqtp::kCheckWords : eqtp::kCheckWords;
  if (hipMemcpyAsync(host, rep, words * sizeof(int32_t), hipMemcpyDeviceToHost, st) != hipSuccess) return EQTP_EHIP;
  if (hipStreamSynchronize(st) != hipSuccess) return EQTP_EHIP;
  for (int k = 0; k < words; ++k)
    if (k % eqtp::kCheckWords < 6 && host[k] != 0) return EQTP_EGRAPH;
  return EQTP_OK;
}

}  // namespace

namespace {
struct IxLayout {
  size_t m, phi, total;
};
IxLayout ix_layout(int64_t N, int64_t E, int lmax, int C) {
  auto al = [](int64_t b) { return (size_t)((b + 255) & ~(int64_t)255); };
  const int64_t nodes = N * C * (int64_t)(lmax + 1) * (lmax + 1) * 4;
  IxLayout w;
  w.m = al(nodes);
  w.phi = w.m + al(nodes);
  w.total = w.phi + al(E * 64 * 4);
  return w;
}
bool ix_desc_ok(const eqtp_interaction_desc* d) {
  return d && d->struct_size >= (int32_t)sizeof(eqtp_interaction_desc);
}
// EQTP_OK, or the status of an invalid / unsupported descriptor
int ix_check(const eqtp_interaction_desc* d, int64_t N, int64_t E) {
  if (!ix_desc_ok(d)) return EQTP_EINVAL;
  if (d->lmax < 0 || d->C <= 0 || !(d->r_cut > 0.0f) || !(d->norm > 0.0f)) return EQTP_EINVAL;
  if (d->path_set != EQTP_PATHS_PARITY && d->path_set != EQTP_PATHS_SO3) return EQTP_EINVAL;
  if (d->lmax > 3 || d->C % 16 != 0 || !valid_c(d->C) || d->n_basis != 8 || d->hidden != 64)
    return EQTP_EUNSUPPORTED;
  if (N < 0 || E < 0 || N > kMaxIndex || E > kMaxIndex || (E > 0 && N == 0)) return EQTP_EINVAL;
  return EQTP_OK;
}
}  // namespace

extern "C" {

int eqtp_num_paths(int lmax, int path_set) { return num_paths_host(lmax, path_set); }

int eqtp_path_table(int lmax, int path_set, int32_t* l1l2l3) {
  const int P = num_paths_host(lmax, path_set);
  if (P < 0) return P;
  if (!l1l2l3) return -EQTP_EINVAL;
  const eqtp_gen::PathLs* pl = path_list(lmax, path_set);
  for (int p = 0; p < P; ++p) {
    l1l2l3[3 * p] = pl[p].l1;
    l1l2l3[3 * p + 1] = pl[p].l2;
    l1l2l3[3 * p + 2] = pl[p].l3;
  }
  return P;
}

int eqtp_sh(const float* vec, int64_t E, int lmax, float* Y, void* stream) {
  if (lmax < 0 || lmax > eqtp::kSo2MaxL) return lmax < 0 ? EQTP_EINVAL : EQTP_EUNSUPPORTED;
  if (E < 0 || E > kMaxIndex) return EQTP_EINVAL;
  if (E == 0) return EQTP_OK;
  if (!vec || !Y || !aligned4(vec) || !aligned16(Y)) return EQTP_EINVAL;
  return status_of(eqtp::launch_sh(vec, E, lmax, Y, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Validation and dispatch of the fused convolution; nothing is launched when launch is false.
int conv_impl(const eqtp_conv_desc* d, int64_t N, int64_t E, const float* vec, const int32_t* src,
              const int32_t* dst, const int32_t* row_ptr, const void* x, const float* weights, void* out,
              void* stream, bool launch) {
  if (!desc_ok(d)) return EQTP_EINVAL;
  const int x_dtype = desc_x_dtype(d);
  if (x_dtype != EQTP_F32 && x_dtype != EQTP_BF16) return EQTP_EINVAL;
  const int out_dtype = desc_out_dtype(d);
  if (out_dtype != EQTP_F32 && out_dtype != EQTP_BF16) return EQTP_EINVAL;
  if (d->lmax < 0) return EQTP_EINVAL;
  if (d->lmax > eqtp::kSo2MaxL) return EQTP_EUNSUPPORTED;
  if (d->path_set != EQTP_PATHS_PARITY && d->path_set != EQTP_PATHS_SO3) return EQTP_EINVAL;
  if (d->weight_mode != EQTP_W_FIXED && d->weight_mode != EQTP_W_RADIAL) return EQTP_EINVAL;
  if (d->edge_order != EQTP_EDGES_DST_SORTED && d->edge_order != EQTP_EDGES_UNSORTED) return EQTP_EINVAL;
  if (d->algo != EQTP_ALGO_AUTO && d->algo != EQTP_ALGO_NODE_MFMA && d->algo != EQTP_ALGO_EDGE_VALU &&
      d->algo != EQTP_ALGO_EDGE_SO2)
    return EQTP_EINVAL;
  if (d->C <= 0) return EQTP_EINVAL;
  if (!valid_c(d->C)) return EQTP_EUNSUPPORTED;
  // radial weights on dst-sorted edges (lmax <= 3, C a multiple of 16): the edge-aligned form with the
  // per-edge weights on the matrix cores, unless the per-edge walk (EQTP_ALGO_EDGE_VALU) is asked for
  const bool radial_so2_ok = d->weight_mode == EQTP_W_RADIAL && d->edge_order == EQTP_EDGES_DST_SORTED &&
                             d->lmax >= 0 && d->lmax <= 3 && d->C % 16 == 0 && x_dtype == EQTP_F32;
  const bool use_radial_so2 = radial_so2_ok && (d->algo == EQTP_ALGO_AUTO || d->algo == EQTP_ALGO_EDGE_SO2);
  // lmax above 3 exists only in the edge-aligned form
  const bool use_so2 =
      !use_radial_so2 && (d->algo == EQTP_ALGO_EDGE_SO2 || (d->algo == EQTP_ALGO_AUTO && d->lmax > 3));
  if (d->lmax > 3 && !use_so2) return EQTP_EUNSUPPORTED;
  if (use_so2 && (d->weight_mode != EQTP_W_FIXED || x_dtype != EQTP_F32)) return EQTP_EUNSUPPORTED;
  // bf16 output: packed bf16 atomics of the per-edge walk, edges in any order
  if (out_dtype == EQTP_BF16 &&
      (d->edge_order != EQTP_EDGES_UNSORTED || use_so2 || use_radial_so2 ||
       (d->algo != EQTP_ALGO_AUTO && d->algo != EQTP_ALGO_EDGE_VALU)))
    return EQTP_EUNSUPPORTED;
  if (d->weight_mode == EQTP_W_RADIAL) {
    if (!(d->r_cut > 0.0f)) return EQTP_EINVAL;
    if (d->n_basis != 8) return EQTP_EUNSUPPORTED;
  }
  if (N < 0 || E < 0 || N > kMaxIndex || E > kMaxIndex) return EQTP_EINVAL;
  if (E > 0 && N == 0) return EQTP_EINVAL;
  // the node-factored algorithm needs per-node sums of edge-independent weights
  const bool node_ok = d->edge_order == EQTP_EDGES_DST_SORTED && d->weight_mode == EQTP_W_FIXED;
  if (d->algo == EQTP_ALGO_NODE_MFMA && !node_ok) return EQTP_EUNSUPPORTED;
  if (N == 0) return EQTP_OK;
  if (!x || !out || !weights || !aligned16(x) || !aligned16(out) || !aligned4(weights)) return EQTP_EINVAL;
  if (E > 0) {
    if (!vec || !src || !aligned4(vec) || !aligned4(src)) return EQTP_EINVAL;
  }
  if (d->edge_order == EQTP_EDGES_DST_SORTED) {
    if (!row_ptr || !aligned4(row_ptr)) return EQTP_EINVAL;
  } else if (E > 0) {
    if (!dst || !aligned4(dst)) return EQTP_EINVAL;
  }
  eqtp::ConvArgs a;
  a.N = N;
  a.E = E;
  a.lmax = d->lmax;
  a.C = d->C;
  a.path_set = d->path_set;
  a.weight_mode = d->weight_mode;
  a.edge_order = d->edge_order;
  a.r_cut = d->r_cut;
  a.vec = vec;
  a.src = src;
  a.dst = dst;
  a.row_ptr = row_ptr;
  a.x = static_cast<const float*>(x);
  a.x_bf16 = x_dtype == EQTP_BF16;
  a.w = weights;
  a.out = static_cast<float*>(out);
  a.out_bf16 = out_dtype == EQTP_BF16;
  a.stream = (hipStream_t)stream;
  if (!launch) return EQTP_OK;
  if (use_radial_so2) return status_of(eqtp::launch_conv_so2_radial(a));
  if (use_so2) return status_of(eqtp::launch_conv_so2(a));
  const bool use_node = node_ok && d->algo != EQTP_ALGO_EDGE_VALU;
  return status_of(use_node ? eqtp::launch_conv_node(a) : eqtp::launch_conv_edge(a));
}

// conv_impl with debug mode's graph check between validation and launch
int conv_checked(const eqtp_conv_desc* d, int64_t N, int64_t E, const float* vec, const int32_t* src,
                 const int32_t* dst, const int32_t* row_ptr, const void* x, const float* weights, void* out,
                 void* stream) {
  int rc = conv_impl(d, N, E, vec, src, dst, row_ptr, x, weights, out, stream, false);
  if (rc != EQTP_OK || N == 0) return rc;
  const bool sorted = d->edge_order == EQTP_EDGES_DST_SORTED;
  rc = debug_check(N, E, sorted ? row_ptr : nullptr, src, sorted ? nullptr : dst, vec, nullptr, stream);
  if (rc != EQTP_OK) return rc;
  return conv_impl(d, N, E, vec, src, dst, row_ptr, x, weights, out, stream, true);
}

// Workspace of the grouping by destination: row pointers [N+1]; five regions of
// E ints R0..R4 (the radix sort's keys and edge indices: the last pass leaves
// them in R0 and R4); the sort's digit counts.  After the sort the grouped
// vectors [E,3] overwrite R0..R2 (contiguous, 12 E bytes) and the grouped
// sources R3.  Every region 256-byte aligned.
struct WsLayout {
  size_t r[5], hist, total;
};
WsLayout ws_layout(int64_t N, int64_t E) {
  auto al = [](int64_t b) { return (size_t)((b + 255) & ~(int64_t)255); };
  WsLayout w;
  size_t o = al((N + 1) * 4);
  for (int i = 0; i < 5; ++i) {
    w.r[i] = o;
    o += al(E * 4);
  }
  w.hist = o;
  w.total = o + al(eqtp::radix_hist_entries(E) * 4);
  return w;
}

bool groups_edges(const eqtp_conv_desc* d, int64_t N) { return d->edge_order == EQTP_EDGES_UNSORTED && N > 0; }

// eqtp_conv_fused_ws on a given workspace (see include/eqtp.h)
int conv_ws_impl(const eqtp_conv_desc* d, int64_t N, int64_t E, const float* vec, const int32_t* src,
                 const int32_t* dst, const int32_t* row_ptr, const void* x, const float* weights, float* out,
                 void* workspace, int64_t workspace_bytes, void* stream) {
  if (!desc_ok(d)) return EQTP_EINVAL;
  if (!groups_edges(d, N)) return conv_checked(d, N, E, vec, src, dst, row_ptr, x, weights, out, stream);
  if (N < 0 || E < 0 || N > kMaxIndex || E > kMaxIndex) return EQTP_EINVAL;
  const WsLayout L = ws_layout(N, E);
  if (!workspace || !aligned16(workspace) || workspace_bytes < (int64_t)L.total) return EQTP_EINVAL;
  if (E > 0 && (!dst || !aligned4(dst))) return EQTP_EINVAL;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  int32_t* rp = reinterpret_cast<int32_t*>(ws);
  int32_t* R[5];
  for (int i = 0; i < 5; ++i) R[i] = reinterpret_cast<int32_t*>(ws + L.r[i]);
  int32_t* hist = reinterpret_cast<int32_t*>(ws + L.hist);
  float* vec_s = reinterpret_cast<float*>(R[0]);  // spans R0..R2
  int32_t* src_s = R[3];
  // the call as it runs after the grouping: dst-sorted edges
  eqtp_conv_desc ds{};
  memcpy(&ds, d, (size_t)d->struct_size);  // a descriptor of an earlier size ends before x_dtype or out_dtype
  ds.struct_size = (int32_t)sizeof(eqtp_conv_desc);
  ds.x_dtype = desc_x_dtype(d);
  ds.out_dtype = desc_out_dtype(d);
  ds.edge_order = EQTP_EDGES_DST_SORTED;
  int rc = conv_impl(&ds, N, E, vec, src, nullptr, rp, x, weights, out, stream, false);
  if (rc != EQTP_OK) return rc;
  rc = debug_check(N, E, nullptr, src, dst, vec, nullptr, stream);
  if (rc != EQTP_OK) return rc;
  rc = status_of(eqtp::launch_sort_edges_stable(N, E, dst, vec, src, rp, R[0], R[4], R[1], R[2], hist, vec_s, src_s,
                                                (hipStream_t)stream));
  if (rc != EQTP_OK) return rc;
  return conv_impl(&ds, N, E, vec_s, src_s, nullptr, rp, x, weights, out, stream, true);
}

}  // namespace

extern "C" {

int eqtp_conv_fused(const eqtp_conv_desc* d, int64_t N, int64_t E, const float* vec, const int32_t* src,
                    const int32_t* dst, const int32_t* row_ptr, const void* x, const float* weights, void* out,
                    void* stream) {
  return conv_checked(d, N, E, vec, src, dst, row_ptr, x, weights, out, stream);
}

int64_t eqtp_conv_workspace_bytes(const eqtp_conv_desc* d, int64_t N, int64_t E) {
  if (!desc_ok(d) || N < 0 || E < 0 || N > kMaxIndex || E > kMaxIndex) return -EQTP_EINVAL;
  return groups_edges(d, N) ? (int64_t)ws_layout(N, E).total : 0;
}

int eqtp_conv_fused_ws(const eqtp_conv_desc* d, int64_t N, int64_t E, const float* vec, const int32_t* src,
                       const int32_t* dst, const int32_t* row_ptr, const void* x, const float* weights, float* out,
                       void* workspace, int64_t workspace_bytes, void* stream) {
  return conv_ws_impl(d, N, E, vec, src, dst, row_ptr, x, weights, out, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// device address of the current device's scratch array, looked up on the first call on that device
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return EQTP_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return EQTP_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return EQTP_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return EQTP_OK;
}

}  // namespace

extern "C" {

int eqtp_conv_fused_noalloc(const eqtp_conv_desc* d, int64_t N, int64_t E, const float* vec, const int32_t* src,
                            const int32_t* dst, const int32_t* row_ptr, const void* x, const float* weights,
                            float* out, void* stream) {
  const int64_t need = eqtp_conv_workspace_bytes(d, N, E);
  if (need < 0) return (int)-need;
  if (need > kScratchBytes) return EQTP_ETOOLARGE;
  void* ws = nullptr;
  if (need > 0) {
    const int rc = scratch_address(&ws);
    if (rc != EQTP_OK) return rc;
  }
  return conv_ws_impl(d, N, E, vec, src, dst, row_ptr, x, weights, out, ws, kScratchBytes, stream);
}

int eqtp_conv_messages(const eqtp_conv_desc* d, int64_t N, int64_t E, const float* vec, const int32_t* src,
                       const float* x, const float* weights, float* messages, void* stream) {
  if (!desc_ok(d)) return EQTP_EINVAL;
  if (desc_x_dtype(d) != EQTP_F32) return desc_x_dtype(d) == EQTP_BF16 ? EQTP_EUNSUPPORTED : EQTP_EINVAL;
  if (out_f32_only(d) != EQTP_OK) return out_f32_only(d);
  if (d->lmax < 0) return EQTP_EINVAL;
  if (d->lmax > eqtp::kSo2MaxL) return EQTP_EUNSUPPORTED;
  // fixed weights: the edge-aligned form unless the per-edge coupling walk (EQTP_ALGO_EDGE_VALU) is asked for
  // (the same messages with fewer operations per edge); radial weights at lmax <= 3: the coupling walk
  const bool use_so2 = d->lmax > 3 || d->algo == EQTP_ALGO_EDGE_SO2 ||
                       (d->algo != EQTP_ALGO_EDGE_VALU && d->weight_mode == EQTP_W_FIXED);
  if (use_so2 && d->weight_mode != EQTP_W_FIXED) return EQTP_EUNSUPPORTED;
  if (d->path_set != EQTP_PATHS_PARITY && d->path_set != EQTP_PATHS_SO3) return EQTP_EINVAL;
  if (d->weight_mode != EQTP_W_FIXED && d->weight_mode != EQTP_W_RADIAL) return EQTP_EINVAL;
  if (d->C <= 0) return EQTP_EINVAL;
  if (!valid_c(d->C)) return EQTP_EUNSUPPORTED;
  if (d->weight_mode == EQTP_W_RADIAL) {
    if (!(d->r_cut > 0.0f)) return EQTP_EINVAL;
    if (d->n_basis != 8) return EQTP_EUNSUPPORTED;
  }
  if (N < 0 || E < 0 || N > kMaxIndex || E > kMaxIndex) return EQTP_EINVAL;
  if (E > 0 && N == 0) return EQTP_EINVAL;
  if (E == 0) return EQTP_OK;
  if (!vec || !src || !x || !weights || !messages) return EQTP_EINVAL;
  if (!aligned4(vec) || !aligned4(src) || !aligned4(weights) || !aligned16(x) || !aligned16(messages))
    return EQTP_EINVAL;
  eqtp::ConvArgs a;
  a.N = N;
  a.E = E;
  a.lmax = d->lmax;
  a.C = d->C;
  a.path_set = d->path_set;
  a.weight_mode = d->weight_mode;
  a.edge_order = EQTP_EDGES_UNSORTED;
  a.r_cut = d->r_cut;
  a.vec = vec;
  a.src = src;
  a.dst = nullptr;
  a.row_ptr = nullptr;
  a.x = x;
  a.w = weights;
  a.out = messages;
  a.stream = (hipStream_t)stream;
  const int chk = debug_check(N, E, nullptr, src, nullptr, vec, nullptr, stream);
  if (chk != EQTP_OK) return chk;
  if (use_so2) {
    a.messages = 1;
    return status_of(eqtp::launch_conv_so2(a));
  }
  return status_of(eqtp::launch_conv_messages(a));
}

int eqtp_conv_backward(const eqtp_conv_desc* d, int64_t N, int64_t E, const float* vec, const int32_t* src,
                       const int32_t* dst, const int32_t* row_ptr, const float* x, const float* weights,
                       const float* grad_out, float* grad_x, float* grad_w, float* grad_vec, void* stream) {
  if (!desc_ok(d)) return EQTP_EINVAL;
  if (desc_x_dtype(d) != EQTP_F32) return desc_x_dtype(d) == EQTP_BF16 ? EQTP_EUNSUPPORTED : EQTP_EINVAL;
  if (out_f32_only(d) != EQTP_OK) return out_f32_only(d);
  if (d->lmax < 0) return EQTP_EINVAL;
  if (d->lmax > eqtp::kSo2MaxL) return EQTP_EUNSUPPORTED;
  if (d->path_set != EQTP_PATHS_PARITY && d->path_set != EQTP_PATHS_SO3) return EQTP_EINVAL;
  if (d->weight_mode != EQTP_W_FIXED && d->weight_mode != EQTP_W_RADIAL) return EQTP_EINVAL;
  if (d->edge_order != EQTP_EDGES_DST_SORTED && d->edge_order != EQTP_EDGES_UNSORTED) return EQTP_EINVAL;
  if (d->algo != EQTP_ALGO_AUTO && d->algo != EQTP_ALGO_NODE_MFMA && d->algo != EQTP_ALGO_EDGE_VALU &&
      d->algo != EQTP_ALGO_EDGE_SO2)
    return EQTP_EINVAL;
  if (d->C <= 0) return EQTP_EINVAL;
  if (!valid_c(d->C)) return EQTP_EUNSUPPORTED;
  const bool radial = d->weight_mode == EQTP_W_RADIAL;
  // fixed weights, lmax <= 3, EQTP_ALGO_AUTO: the edge-aligned form when grad_x or grad_w is wanted (faster
  // than the coupling walk at every lmax and channel count measured); grad_vec alone by the coupling walk,
  // which is faster there (dst-sorted edges: the vector-ALU walk below lmax 3, the matrix cores at 3)
  const bool vec_only = !grad_x && !grad_w;
  const bool use_so2 = !radial && (d->lmax > 3 || d->algo == EQTP_ALGO_EDGE_SO2 ||
                                   (d->algo == EQTP_ALGO_AUTO && !vec_only));
  if (d->lmax > 3 && !use_so2) return EQTP_EUNSUPPORTED;
  if (radial) {
    if (!(d->r_cut > 0.0f)) return EQTP_EINVAL;
    if (d->n_basis != 8 || d->C % 16 != 0) return EQTP_EUNSUPPORTED;
  }
  if (N < 0 || E < 0 || N > kMaxIndex || E > kMaxIndex) return EQTP_EINVAL;
  if (E > 0 && N == 0) return EQTP_EINVAL;
  if (!grad_x && !grad_w && !grad_vec) return EQTP_EINVAL;
  if (grad_x && !aligned16(grad_x)) return EQTP_EINVAL;
  if ((grad_w && !aligned4(grad_w)) || (grad_vec && !aligned4(grad_vec))) return EQTP_EINVAL;
  if (!weights || !aligned4(weights)) return EQTP_EINVAL;
  if (N > 0 && (!x || !grad_out || !aligned16(x) || !aligned16(grad_out))) return EQTP_EINVAL;
  if (E > 0) {
    if (!vec || !src || !aligned4(vec) || !aligned4(src)) return EQTP_EINVAL;
    if (d->edge_order == EQTP_EDGES_UNSORTED && (!dst || !aligned4(dst))) return EQTP_EINVAL;
  }
  if (d->edge_order == EQTP_EDGES_DST_SORTED && N > 0 && (!row_ptr || !aligned4(row_ptr))) return EQTP_EINVAL;
  eqtp::BwdArgs a;
  a.N = N;
  a.E = E;
  a.lmax = d->lmax;
  a.C = d->C;
  a.path_set = d->path_set;
  a.vec = vec;
  a.src = src;
  a.dst = d->edge_order == EQTP_EDGES_UNSORTED ? dst : nullptr;
  a.row_ptr = d->edge_order == EQTP_EDGES_DST_SORTED ? row_ptr : nullptr;
  a.x = x;
  a.w = weights;
  a.gout = grad_out;
  a.gx = grad_x;
  a.gw = grad_w;
  a.gvec = grad_vec;
  a.algo = d->algo == EQTP_ALGO_AUTO && vec_only && d->lmax < 3 ? EQTP_ALGO_EDGE_VALU : d->algo;
  a.r_cut = d->r_cut;
  a.stream = (hipStream_t)stream;
  if (N > 0) {
    const int chk = debug_check(N, E, a.row_ptr, src, a.dst, vec, nullptr, stream);
    if (chk != EQTP_OK) return chk;
  }
  return status_of(radial    ? eqtp::launch_conv_backward_radial(a)
                   : use_so2 ? eqtp::launch_conv_backward_so2(a)
                             : eqtp::launch_conv_backward(a));
}

int eqtp_conv_backward_by_source(const eqtp_conv_desc* d, int64_t N, int64_t E, const float* vec_s,
                                 const int32_t* dst_s, const int32_t* src_ptr, const float* x, const float* weights,
                                 const float* grad_out, float* grad_x, float* grad_w, const int32_t* perm,
                                 float* grad_vec, void* stream) {
  if (!desc_ok(d)) return EQTP_EINVAL;
  if (desc_x_dtype(d) != EQTP_F32) return desc_x_dtype(d) == EQTP_BF16 ? EQTP_EUNSUPPORTED : EQTP_EINVAL;
  if (out_f32_only(d) != EQTP_OK) return out_f32_only(d);
  if (d->lmax < 0) return EQTP_EINVAL;
  if (d->lmax > eqtp::kSo2MaxL) return EQTP_EUNSUPPORTED;
  if (d->path_set != EQTP_PATHS_PARITY && d->path_set != EQTP_PATHS_SO3) return EQTP_EINVAL;
  if (d->weight_mode != EQTP_W_FIXED && d->weight_mode != EQTP_W_RADIAL) return EQTP_EINVAL;
  if (d->algo != EQTP_ALGO_AUTO && d->algo != EQTP_ALGO_NODE_MFMA && d->algo != EQTP_ALGO_EDGE_VALU &&
      d->algo != EQTP_ALGO_EDGE_SO2)
    return EQTP_EINVAL;
  if (d->C <= 0) return EQTP_EINVAL;
  if (!valid_c(d->C)) return EQTP_EUNSUPPORTED;
  const bool radial = d->weight_mode == EQTP_W_RADIAL;
  // fixed weights: the node-factored adjoint (lmax <= 3) unless the edge-aligned form is asked for or needed
  const bool use_so2 = !radial && (d->lmax > 3 || d->algo == EQTP_ALGO_EDGE_SO2);
  if (d->lmax > 3 && !use_so2) return EQTP_EUNSUPPORTED;
  if (radial) {
    if (!(d->r_cut > 0.0f)) return EQTP_EINVAL;
    if (d->n_basis != 8 || d->C % 16 != 0) return EQTP_EUNSUPPORTED;
  }
  if (N < 0 || E < 0 || N > kMaxIndex || E > kMaxIndex) return EQTP_EINVAL;
  if (E > 0 && N == 0) return EQTP_EINVAL;
  if (!grad_x && !grad_w && !grad_vec) return EQTP_EINVAL;
  if ((grad_x && !aligned16(grad_x)) || (grad_w && !aligned4(grad_w)) || (grad_vec && !aligned4(grad_vec)))
    return EQTP_EINVAL;
  if (!weights || !aligned4(weights)) return EQTP_EINVAL;
  const bool edge_walk = radial || use_so2 || grad_vec;  // a walk over the edges reads x for every output
  if (N > 0) {
    if (!grad_out || !aligned16(grad_out) || !src_ptr || !aligned4(src_ptr)) return EQTP_EINVAL;
    if ((grad_w || edge_walk) && (!x || !aligned16(x))) return EQTP_EINVAL;
  }
  if (E > 0 && (!vec_s || !dst_s || !aligned4(vec_s) || !aligned4(dst_s))) return EQTP_EINVAL;
  if (E > 0 && grad_vec && (!perm || !aligned4(perm))) return EQTP_EINVAL;
  eqtp::BwdArgs a;
  a.N = N;
  a.E = E;
  a.lmax = d->lmax;
  a.C = d->C;
  a.path_set = d->path_set;
  a.vec = vec_s;
  a.src = nullptr;
  a.dst = dst_s;
  a.row_ptr = src_ptr;
  a.x = x;
  a.w = weights;
  a.gout = grad_out;
  a.gx = grad_x;
  a.gw = grad_w;
  a.gvec = grad_vec;
  a.r_cut = d->r_cut;
  a.by_src = true;
  a.perm = perm;
  a.stream = (hipStream_t)stream;
  if (N > 0) {
    // rows are sources here: src_ptr is the CSR, dst_s is range-checked as an index array
    const int chk = debug_check(N, E, src_ptr, dst_s, nullptr, vec_s, grad_vec ? perm : nullptr, stream);
    if (chk != EQTP_OK) return chk;
  }
  if (radial) return status_of(eqtp::launch_conv_backward_radial(a));
  if (use_so2) return status_of(eqtp::launch_conv_backward_so2(a));
  // lmax <= 3, fixed weights: grad_x and grad_w by the node-factored adjoint, grad_vec by a walk in the edge
  // frame over the same grouped edges
  if (grad_x || grad_w) {
    eqtp::BwdArgs b = a;
    b.gvec = nullptr;
    b.by_src = false;
    b.perm = nullptr;
    const int st = status_of(eqtp::launch_conv_backward_by_source(b));
    if (st != EQTP_OK || !grad_vec) return st;
  }
  a.gx = nullptr;
  a.gw = nullptr;
  return status_of(eqtp::launch_conv_backward_so2(a));
}

int eqtp_edge_rows(int64_t N, int64_t E, const int32_t* row_ptr, int32_t* rows, void* stream) {
  if (N < 0 || E < 0 || N > kMaxIndex || E > kMaxIndex) return EQTP_EINVAL;
  if (E > 0 && (N == 0 || !row_ptr || !rows || !aligned4(row_ptr) || !aligned4(rows))) return EQTP_EINVAL;
  if (E > 0) {
    const int chk = debug_check(N, E, row_ptr, nullptr, nullptr, nullptr, nullptr, stream);
    if (chk != EQTP_OK) return chk;
  }
  return status_of(eqtp::launch_edge_rows(N, E, row_ptr, rows, (hipStream_t)stream));
}

int eqtp_sort_edges(int64_t N, int64_t E, const int32_t* dst, const float* vec, const int32_t* src, int32_t* row_ptr,
                    int32_t* perm, float* vec_sorted, int32_t* src_sorted, void* stream) {
  if (N < 0 || E < 0 || N > kMaxIndex - 1 || E > kMaxIndex) return EQTP_EINVAL;
  if (E > 0 && N == 0) return EQTP_EINVAL;
  if (!row_ptr || !aligned4(row_ptr)) return EQTP_EINVAL;  // N + 1 >= 1 entries, row_ptr[N] = E is always written
  if (E > 0) {
    if (!dst || !perm || !aligned4(dst) || !aligned4(perm)) return EQTP_EINVAL;
    if (vec_sorted && (!vec || !aligned4(vec) || !aligned4(vec_sorted))) return EQTP_EINVAL;
    if (src_sorted && (!src || !aligned4(src) || !aligned4(src_sorted))) return EQTP_EINVAL;
    const int chk = debug_check(N, E, nullptr, src_sorted ? src : nullptr, dst, vec_sorted ? vec : nullptr, nullptr,
                                stream);
    if (chk != EQTP_OK) return chk;
  }
  return status_of(eqtp::launch_sort_edges(N, E, dst, vec, src, row_ptr, perm, vec_sorted, src_sorted,
                                           (hipStream_t)stream));
}

}  // extern "C"

namespace {
// Workspace of eqtp_sort_edges_stable: the radix sort's second key buffer, both ping-pong buffers of the
// other pass and its digit counts, each region 256-byte aligned (the caller's perm receives the edge
// indices of the last pass)
struct SortWs {
  size_t keys_a, keys_b, vals_b, hist, total;
};
SortWs sort_ws_layout(int64_t E) {
  auto al = [](int64_t b) { return (size_t)((b + 255) & ~(int64_t)255); };
  SortWs w;
  w.keys_a = 0;
  w.keys_b = al(E * 4);
  w.vals_b = w.keys_b + al(E * 4);
  w.hist = w.vals_b + al(E * 4);
  w.total = w.hist + al(eqtp::radix_hist_entries(E) * 4);
  return w;
}
}  // namespace

extern "C" {

int64_t eqtp_sort_workspace_bytes(int64_t N, int64_t E) {
  if (N < 0 || E < 0 || N > kMaxIndex - 1 || E > kMaxIndex) return -EQTP_EINVAL;
  return (int64_t)sort_ws_layout(E).total;
}

int eqtp_sort_edges_stable(int64_t N, int64_t E, const int32_t* dst, const float* vec, const int32_t* src,
                           int32_t* row_ptr, int32_t* perm, float* vec_sorted, int32_t* src_sorted, void* workspace,
                           int64_t workspace_bytes, void* stream) {
  if (N < 0 || E < 0 || N > kMaxIndex - 1 || E > kMaxIndex) return EQTP_EINVAL;
  if (E > 0 && N == 0) return EQTP_EINVAL;
  if (!row_ptr || !aligned4(row_ptr)) return EQTP_EINVAL;
  const SortWs L = sort_ws_layout(E);
  if (E > 0) {
    if (!dst || !perm || !aligned4(dst) || !aligned4(perm)) return EQTP_EINVAL;
    if (vec_sorted && (!vec || !aligned4(vec) || !aligned4(vec_sorted))) return EQTP_EINVAL;
    if (src_sorted && (!src || !aligned4(src) || !aligned4(src_sorted))) return EQTP_EINVAL;
    if (!workspace || !aligned16(workspace) || workspace_bytes < (int64_t)L.total) return EQTP_EINVAL;
    const int chk = debug_check(N, E, nullptr, src_sorted ? src : nullptr, dst, vec_sorted ? vec : nullptr, nullptr,
                                stream);
    if (chk != EQTP_OK) return chk;
  }
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  int32_t* keys_a = E > 0 ? reinterpret_cast<int32_t*>(ws + L.keys_a) : nullptr;
  int32_t* keys_b = E > 0 ? reinterpret_cast<int32_t*>(ws + L.keys_b) : nullptr;
  int32_t* vals_b = E > 0 ? reinterpret_cast<int32_t*>(ws + L.vals_b) : nullptr;
  int32_t* hist = E > 0 ? reinterpret_cast<int32_t*>(ws + L.hist) : nullptr;
  return status_of(eqtp::launch_sort_edges_stable(N, E, dst, vec, src, row_ptr, keys_a, perm, keys_b, vals_b, hist,
                                                  vec_sorted, src_sorted, (hipStream_t)stream));
}

int eqtp_linear(int64_t N, int C, int lmax, int dtype, const void* h, const void* W, float* out, void* stream) {
  if (lmax < 0 || C <= 0 || N < 0 || N > kMaxIndex) return EQTP_EINVAL;
  if (lmax > eqtp::kSo2MaxL || !valid_c(C)) return EQTP_EUNSUPPORTED;
  if (dtype != EQTP_F32 && dtype != EQTP_BF16 && dtype != EQTP_F32_BF16) return EQTP_EINVAL;
  if (N == 0) return EQTP_OK;
  if (!h || !W || !out || !aligned16(h) || !aligned16(W) || !aligned16(out)) return EQTP_EINVAL;
  const int mode = dtype == EQTP_F32 ? 0 : (dtype == EQTP_BF16 ? 1 : 2);
  return status_of(eqtp::launch_linear(N, C, lmax, mode, h, W, out, (hipStream_t)stream));
}


int64_t eqtp_interaction_workspace_bytes(const eqtp_interaction_desc* d, int64_t N, int64_t E) {
  const int rc = ix_check(d, N, E);
  if (rc != EQTP_OK) return -rc;
  return (int64_t)ix_layout(N, E, d->lmax, d->C).total;
}

int eqtp_interaction(const eqtp_interaction_desc* d, int64_t N, int64_t E, const float* vec, const int32_t* src,
                     const int32_t* row_ptr, const float* h, const float* W_up, const float* W1, const float* W2,
                     const float* W3, const float* W_out, float* out, void* workspace, int64_t workspace_bytes,
                     void* stream) {
  const int rc = ix_check(d, N, E);
  if (rc != EQTP_OK) return rc;
  if (N == 0) return EQTP_OK;
  const IxLayout L = ix_layout(N, E, d->lmax, d->C);
  if (!workspace || !aligned16(workspace) || workspace_bytes < (int64_t)L.total) return EQTP_EINVAL;
  if (!h || !out || !W_up || !W_out || !aligned16(h) || !aligned16(out) || !aligned16(W_up) || !aligned16(W_out))
    return EQTP_EINVAL;
  if (!W1 || !W2 || !W3 || !aligned4(W1) || !aligned4(W2) || !aligned4(W3)) return EQTP_EINVAL;
  if (!row_ptr || !aligned4(row_ptr)) return EQTP_EINVAL;
  if (E > 0 && (!vec || !src || !aligned4(vec) || !aligned4(src))) return EQTP_EINVAL;
  const int chk = debug_check(N, E, row_ptr, src, nullptr, vec, nullptr, stream);
  if (chk != EQTP_OK) return chk;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  float* h1 = reinterpret_cast<float*>(ws);
  float* m = reinterpret_cast<float*>(ws + L.m);
  float* phi = reinterpret_cast<float*>(ws + L.phi);
  const hipStream_t st = (hipStream_t)stream;
  int s = status_of(eqtp::launch_linear(N, d->C, d->lmax, 0, h, W_up, h1, st));
  if (s != EQTP_OK) return s;
  s = status_of(eqtp::launch_radial_mlp(E, vec, d->r_cut, W1, W2, phi, 1.0f / d->norm, st));
  if (s != EQTP_OK) return s;
  eqtp::ConvArgs a;
  a.N = N;
  a.E = E;
  a.lmax = d->lmax;
  a.C = d->C;
  a.path_set = d->path_set;
  a.weight_mode = EQTP_W_RADIAL;
  a.edge_order = EQTP_EDGES_DST_SORTED;
  a.r_cut = d->r_cut;
  a.vec = vec;
  a.src = src;
  a.dst = nullptr;
  a.row_ptr = row_ptr;
  a.x = h1;
  a.w = W3;
  a.out = m;
  a.stream = st;
  a.phi = phi;
  s = status_of(eqtp::launch_conv_so2_radial(a));
  if (s != EQTP_OK) return s;
  return status_of(eqtp::launch_linear(N, d->C, d->lmax, 0, m, W_out, out, st));
}

const char* eqtp_status_string(int status) {
  switch (status) {
    case EQTP_OK: return "EQTP_OK: success";
    case EQTP_EINVAL: return "EQTP_EINVAL: invalid argument";
    case EQTP_EUNSUPPORTED: return "EQTP_EUNSUPPORTED: request not supported by this build";
    case EQTP_EHIP: return "EQTP_EHIP: HIP runtime error at launch";
    case EQTP_ETOOLARGE: return "EQTP_ETOOLARGE: the request needs more than the library's static scratch";
    case EQTP_EGRAPH: return "EQTP_EGRAPH: the graph arrays fail the debug-mode checks";
    default: return "unknown status";
  }
}

int eqtp_check_graph(int64_t N, int64_t E, const int32_t* row_ptr, const int32_t* src, const int32_t* dst,
                     const float* vec, int32_t* report, void* stream) {
  if (N < 0 || E < 0 || N > kMaxIndex || E > kMaxIndex) return EQTP_EINVAL;
  if (!report || !aligned4(report)) return EQTP_EINVAL;
  if ((row_ptr && !aligned4(row_ptr)) || (src && !aligned4(src)) || (dst && !aligned4(dst)) ||
      (vec && !aligned4(vec)))
    return EQTP_EINVAL;
  if (E == 0) src = dst = nullptr, vec = nullptr;
  return status_of(eqtp::launch_check_graph(N, E, row_ptr, src, dst, vec, report, (hipStream_t)stream));
}

int eqtp_set_debug(int on) {
  if (on != 0 && on != 1) return g_debug.load();
  return g_debug.exchange(on);
}

int eqtp_test_segment_probe(const int32_t* row_ptr, const int32_t* src, int64_t N, int64_t E, int C, int lmax,
                            int algo, int32_t* count, int64_t* src_sum, void* stream) {
  if (N < 0 || E < 0 || N > kMaxIndex || E > kMaxIndex || (E > 0 && N == 0)) return EQTP_EINVAL;
  if (lmax < 0 || lmax > 3 || !valid_c(C)) return EQTP_EUNSUPPORTED;
  if (algo != EQTP_ALGO_NODE_MFMA && algo != EQTP_ALGO_EDGE_VALU) return EQTP_EINVAL;
  if (N == 0) return EQTP_OK;
  if (!row_ptr || !count || !src_sum || (E > 0 && !src)) return EQTP_EINVAL;
  eqtp::ProbeArgs a;
  a.N = N;
  a.E = E;
  a.C = C;
  a.lmax = lmax;
  a.row_ptr = row_ptr;
  a.src = src;
  a.count = count;
  a.src_sum = reinterpret_cast<long long*>(src_sum);
  a.stream = (hipStream_t)stream;
  return status_of(algo == EQTP_ALGO_NODE_MFMA ? eqtp::launch_probe_node(a) : eqtp::launch_probe_edge(a));
}

}  // extern "C"

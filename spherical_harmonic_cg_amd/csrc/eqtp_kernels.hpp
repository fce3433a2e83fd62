// eqtp_kernels.hpp -- host-side launch interface between the C ABI and the
// kernels.  Arguments are validated by the ABI layer before these are called.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace eqtp {

struct ConvArgs {
  int64_t N, E;
  int lmax, C, path_set, weight_mode, edge_order;
  int x_bf16 = 0;     // x holds bfloat16 features
  int messages = 0;   // edge-aligned kernel: per-edge messages [E, C, K] into out instead of the sum
  bool out_bf16 = false;  // out holds bfloat16 (edges in any order: packed bf16 atomics)
  float r_cut;
  const float* vec;
  const int32_t* src;
  const int32_t* dst;
  const int32_t* row_ptr;
  const float* x;
  const float* w;
  float* out;
  hipStream_t stream;
  // radial edge-aligned kernel: a per-edge basis [E, 64] (stored [E][4][16], hidden unit 4 i + q at
  // q * 16 + i) in place of the radial functions, with w [64, P*C]; else nullptr
  const float* phi = nullptr;
};

struct ProbeArgs {
  int64_t N, E;
  int C, lmax;
  const int32_t* row_ptr;
  const int32_t* src;
  int32_t* count;
  long long* src_sum;
  hipStream_t stream;
};

struct BwdArgs {
  int64_t N, E;
  int lmax, C, path_set;
  const float* vec;
  const int32_t* src;
  const int32_t* dst;      // unsorted edges (row_ptr == nullptr)
  const int32_t* row_ptr;  // dst-sorted edges
  const float* x;
  const float* w;
  const float* gout;
  float* gx;    // or nullptr
  float* gw;    // or nullptr
  float* gvec;  // or nullptr
  int algo = 0;  // grad_vec of sorted edges: 2 = vector-ALU walk, else matrix cores
  float r_cut = 0.0f;  // radial weights: w is [8, P*C] and gw [8, P*C]
  hipStream_t stream;
  // edges grouped by source: row_ptr is the CSR over sources, dst the destinations in that order,
  // perm[i] the input index of grouped edge i (grad_vec is written there)
  bool by_src = false;
  const int32_t* perm = nullptr;
};

hipError_t launch_sh(const float* vec, int64_t E, int lmax, float* Y, hipStream_t stream);
hipError_t launch_conv_node(const ConvArgs& a);   // sorted edges, fixed weights, matrix cores
hipError_t launch_conv_edge(const ConvArgs& a);   // any order / weights, vector ALUs
hipError_t launch_conv_messages(const ConvArgs& a);  // per-edge messages into out [E, C, K]
hipError_t launch_probe_node(const ProbeArgs& a);
hipError_t launch_probe_edge(const ProbeArgs& a);
// mode 0: fp32 storage and products; 1: bf16 storage and products; 2: fp32 storage, bf16 products
hipError_t launch_linear(int64_t N, int C, int lmax, int mode, const void* h, const void* W, float* out,
                         hipStream_t stream);
// compute units of the current device (cached per device)
int num_cus();
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream);
// graph checks: kCheckWords int32 of counts and first offending indices into report (check.hip)
constexpr int kCheckWords = 8;
hipError_t launch_check_graph(int64_t N, int64_t E, const int32_t* row_ptr, const int32_t* src, const int32_t* dst,
                              const float* vec, int32_t* report, hipStream_t stream);
hipError_t launch_conv_backward(const BwdArgs& a);   // fixed weights, vector ALUs
hipError_t launch_conv_backward_radial(const BwdArgs& a);  // radial weights, lmax <= 3, C a multiple of 16
// the interaction layer's radial network: phi [E][4][16] (scaled by scale) from the edge lengths
hipError_t launch_radial_mlp(int64_t E, const float* vec, float r_cut, const float* W1, const float* W2, float* phi,
                             float scale, hipStream_t stream);
// edge-aligned (SO(2)) form, lmax 0..6, fixed fp32 weights, any C; C = 128 runs as two 64-channel halves from
// lmax 4 (forward, messages) or lmax 3 (gradients)
constexpr int kSo2MaxL = 6;
hipError_t launch_conv_so2(const ConvArgs& a);
// gradients in the edge-aligned form: fixed weights, lmax 0..6, any edge order (row_ptr or dst)
hipError_t launch_conv_backward_so2(const BwdArgs& a);
// edge-aligned form with radial weights on dst-sorted edges: lmax 0..3, C = 16, 32, 64 or 128
hipError_t launch_conv_so2_radial(const ConvArgs& a);
// grad_x / grad_w on the matrix cores from edges grouped by source: row_ptr =
// CSR over sources, vec / dst in that order (src unused)
hipError_t launch_conv_backward_by_source(const BwdArgs& a);
hipError_t launch_edge_rows(int64_t N, int64_t E, const int32_t* row_ptr, int32_t* rows, hipStream_t stream);
hipError_t launch_sort_edges(int64_t N, int64_t E, const int32_t* dst, const float* vec, const int32_t* src,
                             int32_t* row_ptr, int32_t* perm, float* vec_out, int32_t* src_out, hipStream_t stream);
// grouping by destination with each row in input order: staged [E] int32 scratch; vec_out, src_out required
// stable grouping by destination (LSD radix sort) for the workspace convolution: row_ptr [N+1], the sorted
// keys and edge indices end in keys_a / vals_a (keys_b / vals_b: the other buffers of the passes, hist:
// radix_hist_entries(E) ints); vec_out [E,3] / src_out [E] in that order, each may be null (vec_out may
// span keys_a..vals_b when they are laid out in that order and hold 12 E bytes; it must not overlap vals_a)
int64_t radix_hist_entries(int64_t E);
hipError_t launch_sort_edges_stable(int64_t N, int64_t E, const int32_t* dst, const float* vec, const int32_t* src,
                                    int32_t* row_ptr, int32_t* keys_a, int32_t* vals_a, int32_t* keys_b,
                                    int32_t* vals_b, int32_t* hist, float* vec_out, int32_t* src_out,
                                    hipStream_t stream);

}  // namespace eqtp

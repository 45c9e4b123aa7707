// Bi-directional channel reordering from a per-weight saliency map: rows and
// columns ordered by their total saliency, descending, so that salient
// weights gather into the leading block rows and block columns ("ScaleBITS"
// summary page, sections Approach and Limitations: both directions, Q and K
// projections left out of the row reordering; "SFMP" abstract: row-column
// reordering aggregates salient weights).
//
//   k_reorder_sums   one pass over S: workgroup = a slice of rows x all
//                    columns; each thread owns 4-column groups (accumulated
//                    in LDS, no sharing) and adds its part of each row; row
//                    sums reduced in a fixed order (thread, wavefront tree,
//                    wavefronts in order); column partials per slice to the
//                    workspace;
//   k_reorder_cols   column sums over the slices (16 slice groups per
//                    column, each in slice order, then the groups in order);
//   k_reorder_keys   order-preserving keys and indices;
//   radix sort       keys descending, indices as values (stable: ties keep
//                    ascending index) -> perm_row, perm_col.
// Every sum has a fixed order, so the permutations are reproducible.
#include <hip/hip_runtime.h>
#include <hipcub/hipcub.hpp>

#include <algorithm>
#include <cstdint>

#include "msq.h"

namespace msq {
namespace {

extern __shared__ __align__(16) unsigned char smem_reorder[];

constexpr int kSumThreads = 256;
constexpr int kSlicesMax = 1024;

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Slice blockIdx.x: rows [r0, r1).  Dynamic LDS: K floats (column
// accumulators) + rows-per-slice x 4 floats (wavefront row partials).
__global__ __launch_bounds__(kSumThreads) void k_reorder_sums(const float* __restrict__ S, int64_t N,
                                                              int64_t K, int64_t rows_per_slice,
                                                              float* __restrict__ row_sum,
                                                              float* __restrict__ col_part) {
  float* acc = reinterpret_cast<float*>(smem_reorder);
  float* rpart = acc + K;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_slice;
  const int64_t r1 = min(N, r0 + rows_per_slice);
  const int64_t k4 = K / 4;
  for (int64_t c = t; c < k4; c += kSumThreads)
    reinterpret_cast<float4*>(acc)[c] = float4{0.f, 0.f, 0.f, 0.f};
  for (int64_t r = r0; r < r1; ++r) {
    const float4* row = reinterpret_cast<const float4*>(S + r * K);
    float s = 0.f;
    for (int64_t c = t; c < k4; c += kSumThreads) {
      const float4 v = row[c];
      float4& a = reinterpret_cast<float4*>(acc)[c];
      a.x += v.x;
      a.y += v.y;
      a.z += v.z;
      a.w += v.w;
      s += (v.x + v.y) + (v.z + v.w);
    }
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    if (lane == 0) rpart[(r - r0) * 4 + wave] = s;
  }
  __syncthreads();
  for (int64_t r = r0 + t; r < r1; r += kSumThreads) {
    const float* p = rpart + (r - r0) * 4;
    row_sum[r] = (p[0] + p[1]) + (p[2] + p[3]);
  }
  for (int64_t c = t; c < k4; c += kSumThreads)
    reinterpret_cast<float4*>(col_part + (int64_t)blockIdx.x * K)[c] = reinterpret_cast<float4*>(acc)[c];
}

// Column sums over the slices: workgroup = 16 columns x 16 slice groups;
// group g adds slices g, g + 16, ... in order, then the 16 group sums are
// added in group order (a fixed order: reproducible).
constexpr int kColGroups = 16;
__global__ __launch_bounds__(256) void k_reorder_cols(const float* __restrict__ col_part,
                                                      int slices, int64_t K,
                                                      float* __restrict__ col_sum) {
  __shared__ float part[kColGroups][16];
  const int cl = threadIdx.x & 15, g = threadIdx.x >> 4;
  const int64_t c = (int64_t)blockIdx.x * 16 + cl;
  float s = 0.f;
  if (c < K)
    for (int k = g; k < slices; k += kColGroups) s += col_part[(int64_t)k * K + c];
  part[g][cl] = s;
  __syncthreads();
  if (g == 0 && c < K) {
    float t = 0.f;
    for (int k = 0; k < kColGroups; ++k) t += part[k][cl];
    col_sum[c] = t;
  }
}

__global__ __launch_bounds__(256) void k_reorder_keys(const float* __restrict__ score, int64_t n,
                                                      uint32_t* __restrict__ key,
                                                      int32_t* __restrict__ idx) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  key[i] = order_key(score[i]);
  idx[i] = (int32_t)i;
}

__global__ __launch_bounds__(256) void k_reorder_iota(int32_t* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = (int32_t)i;
}

constexpr size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct ReorderPlan {
  int slices;
  int64_t rows_per_slice;
  size_t row_sum, col_sum, col_part, key_in, key_out, idx_in, temp, temp_bytes, total;
  bool ok;  // false when hipCUB could not size its temporary storage
};

ReorderPlan reorder_plan(int64_t N, int64_t K) {
  ReorderPlan p{};
  p.slices = (int)std::min<int64_t>(N, kSlicesMax);
  p.rows_per_slice = (N + p.slices - 1) / p.slices;
  p.slices = (int)((N + p.rows_per_slice - 1) / p.rows_per_slice);
  const int64_t n = std::max(N, K);
  size_t sort_temp = 0;
  p.ok = hipcub::DeviceRadixSort::SortPairsDescending(nullptr, sort_temp, (const uint32_t*)nullptr,
                                                      (uint32_t*)nullptr, (const int32_t*)nullptr,
                                                      (int32_t*)nullptr, (int)n) == hipSuccess;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(bytes);
    return at;
  };
  p.row_sum = take(4 * (size_t)N);
  p.col_sum = take(4 * (size_t)K);
  p.col_part = take(4 * (size_t)K * p.slices);
  p.key_in = take(4 * (size_t)n);
  p.key_out = take(4 * (size_t)n);
  p.idx_in = take(4 * (size_t)n);
  p.temp_bytes = sort_temp;
  p.temp = take(sort_temp);
  p.total = o;
  return p;
}

bool reorder_shape_ok(int64_t N, int64_t K) {
  return N > 0 && K > 0 && N % 64 == 0 && K % 128 == 0 && N <= MSQ_REORDER_MAX_N &&
         K <= MSQ_REORDER_MAX_K;
}

}  // namespace
}  // namespace msq

using namespace msq;

extern "C" size_t msq_reorder_workspace_bytes(int64_t N, int64_t K) {
  if (!reorder_shape_ok(N, K)) return 0;
  const ReorderPlan p = reorder_plan(N, K);
  return p.ok ? p.total : 0;
}

extern "C" msq_status msq_reorder_channels(const float* saliency, int64_t N, int64_t K,
                                           int reorder_rows, int32_t* perm_row, int32_t* perm_col,
                                           void* workspace, size_t workspace_bytes,
                                           hipStream_t stream) {
  if (!saliency || !perm_row || !perm_col || !workspace ||
      (reinterpret_cast<uintptr_t>(saliency) & 15) || (reinterpret_cast<uintptr_t>(workspace) & 255) ||
      (reinterpret_cast<uintptr_t>(perm_row) & 3) || (reinterpret_cast<uintptr_t>(perm_col) & 3))
    return MSQ_ERR_INVALID_ARG;
  if (!reorder_shape_ok(N, K)) return MSQ_ERR_SHAPE;
  const ReorderPlan p = reorder_plan(N, K);
  if (!p.ok) return MSQ_ERR_HIP;
  if (workspace_bytes < p.total) return MSQ_ERR_BUFFER_TOO_SMALL;
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  float* row_sum = reinterpret_cast<float*>(ws + p.row_sum);
  float* col_sum = reinterpret_cast<float*>(ws + p.col_sum);
  float* col_part = reinterpret_cast<float*>(ws + p.col_part);
  uint32_t* key_in = reinterpret_cast<uint32_t*>(ws + p.key_in);
  uint32_t* key_out = reinterpret_cast<uint32_t*>(ws + p.key_out);
  int32_t* idx_in = reinterpret_cast<int32_t*>(ws + p.idx_in);

  const size_t lds = 4 * (size_t)K + 16 * (size_t)p.rows_per_slice;
  hipLaunchKernelGGL(k_reorder_sums, dim3((unsigned)p.slices), dim3(kSumThreads), lds, stream,
                     saliency, N, K, p.rows_per_slice, row_sum, col_part);
  hipLaunchKernelGGL(k_reorder_cols, dim3((unsigned)((K + 15) / 16)), dim3(256), 0, stream,
                     col_part, p.slices, K, col_sum);
  auto sort = [&](const float* score, int64_t n, int32_t* out) {
    hipLaunchKernelGGL(k_reorder_keys, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       score, n, key_in, idx_in);
    size_t tb = p.temp_bytes;
    return hipcub::DeviceRadixSort::SortPairsDescending(ws + p.temp, tb, key_in, key_out, idx_in,
                                                        out, (int)n, 0, 32, stream);
  };
  if (reorder_rows) {
    if (sort(row_sum, N, perm_row) != hipSuccess) return MSQ_ERR_HIP;
  } else {
    hipLaunchKernelGGL(k_reorder_iota, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, stream,
                       perm_row, N);
  }
  if (sort(col_sum, K, perm_col) != hipSuccess) return MSQ_ERR_HIP;
  return hipGetLastError() == hipSuccess ? MSQ_OK : MSQ_ERR_HIP;
}

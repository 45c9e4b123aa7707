// Bitwidth allocation per 64x128 block under a memory budget: the batched
// greedy knapsack ("ScaleBITS" summary page, sections Approach and Key
// results: a batched approximation to classic greedy, 16 to 36 iterations).
//
// Every iteration, for every block that can still move up a level:
//   k_alloc_keys   the cost d of its next step and the fp32 ratio
//                  (u[l+1] - u[l]) / d as an order-preserving 32-bit key;
//   radix sort     keys descending with 8 x block index + step cost as value
//                  (the sort is stable, so equal ratios keep ascending block
//                  order);
//   k_alloc_costs  the step costs in sorted order, then an inclusive scan;
//   k_alloc_select the longest sorted prefix whose cost is at most half the
//                  remaining budget R (binary search over the scan), or, when
//                  that is empty, k_alloc_first / k_alloc_finish: the first
//                  sorted step that fits R (atomic minimum over the grid); R
//                  and the iteration's status updated on the device;
//   k_alloc_apply  the chosen blocks move up one level.
// The host reads the status back after each iteration and stops when an
// iteration takes nothing.  Blocks that cannot move (already at 8 bits) get
// key 0 and cost 0: they sort after every real step and are never moved.
#include <hip/hip_runtime.h>
#include <hipcub/hipcub.hpp>

#include <algorithm>
#include <cstdint>

#include "msq.h"

namespace msq {
namespace {

constexpr int kLevels = 6;
__constant__ int kLevelBits[kLevels] = {0, 1, 2, 3, 4, 8};

struct AllocStatus {
  int64_t remaining;  // budget left, bits
  int64_t taken;      // bits spent by the last iteration
  int32_t count;      // sorted positions [0, count) move up (count = -1: none)
  int32_t single;     // or just this sorted position (-1: none)
  int32_t first;      // first-fit search: smallest qualifying position (INT32_MAX: none)
  int32_t pending;    // the prefix was empty: the first-fit search decides
};

// IEEE float -> uint32 with the same order (no NaNs: the inputs are checked).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);  // -0 -> +0: equal ratios get equal keys
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(256) void k_alloc_init(uint8_t* __restrict__ lev, int64_t n,
                                                    AllocStatus* st, int64_t budget) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) lev[i] = 0;
  if (i == 0) *st = AllocStatus{budget, 0, 0, -1, INT32_MAX, 0};
}

// The sort value carries the block index and the step cost: 8 i + d.
__global__ __launch_bounds__(256) void k_alloc_keys(const float* __restrict__ u,
                                                    const uint8_t* __restrict__ lev, int64_t n,
                                                    uint32_t* __restrict__ key,
                                                    int32_t* __restrict__ val) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int l = lev[i];
  uint32_t k = 0u;
  int d = 0;
  if (l < kLevels - 1) {
    d = kLevelBits[l + 1] - kLevelBits[l];
    const float gain = u[i * kLevels + l + 1] - u[i * kLevels + l];
    k = order_key(gain / (float)d);
  }
  key[i] = k;
  val[i] = (int32_t)(8 * i + d);
}

__global__ __launch_bounds__(256) void k_alloc_costs(const int32_t* __restrict__ sorted_val,
                                                     int64_t n, int32_t* __restrict__ sorted_cost) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p < n) sorted_cost[p] = sorted_val[p] & 7;
}

// One thread: the longest sorted prefix within floor(R / 2) (binary search
// over the non-decreasing scan).  When it takes nothing, the first-fit
// search (k_alloc_first, k_alloc_finish) decides.
__global__ __launch_bounds__(64) void k_alloc_select(const int32_t* __restrict__ scan, int64_t n,
                                                    AllocStatus* st) {
  if (threadIdx.x != 0) return;
  const int64_t R = st->remaining;
  const int64_t half = R / 2;
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = (lo + hi) / 2;
    if ((int64_t)scan[mid] <= half) lo = mid + 1; else hi = mid;
  }
  const int32_t count = (int32_t)lo;
  // a prefix of only blocks that cannot move takes nothing
  const int64_t prefix_bits = count > 0 ? (int64_t)scan[count - 1] : 0;
  st->first = INT32_MAX;
  if (prefix_bits > 0) {
    st->remaining = R - prefix_bits;
    st->taken = prefix_bits;
    st->count = count;
    st->single = -1;
    st->pending = 0;
  } else {
    st->count = -1;
    st->single = -1;
    st->pending = 1;
  }
}

// First sorted step that fits R (only when the prefix was empty).
__global__ __launch_bounds__(256) void k_alloc_first(const int32_t* __restrict__ sorted_cost,
                                                     int64_t n, AllocStatus* st) {
  if (!st->pending) return;
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t R = st->remaining;
  const bool fits = p < n && sorted_cost[p] > 0 && sorted_cost[p] <= R;
  // one atomic per wavefront: its lowest qualifying position
  const uint64_t m = __ballot(fits);
  if (m != 0 && (threadIdx.x & 63) == 0) {
    const int64_t q = (p & ~(int64_t)63) + __builtin_ctzll(m);
    atomicMin(&st->first, (int32_t)q);
  }
}

__global__ __launch_bounds__(64) void k_alloc_finish(const int32_t* __restrict__ sorted_cost,
                                                     AllocStatus* st) {
  if (threadIdx.x != 0 || !st->pending) return;
  const int32_t f = st->first;
  if (f == INT32_MAX) {
    st->taken = 0;
  } else {
    const int32_t d = sorted_cost[f];
    st->remaining -= d;
    st->taken = d;
    st->single = f;
  }
}

__global__ __launch_bounds__(256) void k_alloc_apply(const int32_t* __restrict__ sorted_val,
                                                     int64_t n, const AllocStatus* st,
                                                     uint8_t* __restrict__ lev) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= n) return;
  const bool move = p < st->count || p == st->single;
  const int32_t v = sorted_val[p];
  if (move && (v & 7) > 0) lev[v >> 3] += 1;
}

__global__ __launch_bounds__(256) void k_alloc_bits(const uint8_t* __restrict__ lev, int64_t n,
                                                    uint8_t* __restrict__ bits) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) bits[i] = (uint8_t)kLevelBits[lev[i]];
}

// Finite utilities only: a NaN has no place in the order.
__global__ __launch_bounds__(256) void k_alloc_check(const float* __restrict__ u, int64_t total,
                                                     int32_t* __restrict__ bad) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < total && !isfinite(u[i])) atomicOr(bad, 1);
}

constexpr size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct AllocLayout {
  size_t key_in, key_out, val_in, val_out, sorted_cost, scan, lev, status, bad, temp, temp_bytes,
      total;
  bool ok;  // false when hipCUB could not size its temporary storage
};

AllocLayout alloc_layout(int64_t n) {
  AllocLayout L{};
  size_t sort_temp = 0, scan_temp = 0;
  L.ok = hipcub::DeviceRadixSort::SortPairsDescending(nullptr, sort_temp, (const uint32_t*)nullptr,
                                                      (uint32_t*)nullptr, (const int32_t*)nullptr,
                                                      (int32_t*)nullptr, (int)n) == hipSuccess &&
         hipcub::DeviceScan::InclusiveSum(nullptr, scan_temp, (const int32_t*)nullptr,
                                          (int32_t*)nullptr, (int)n) == hipSuccess;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(bytes);
    return at;
  };
  L.key_in = take(4 * (size_t)n);
  L.key_out = take(4 * (size_t)n);
  L.val_in = take(4 * (size_t)n);
  L.val_out = take(4 * (size_t)n);
  L.sorted_cost = take(4 * (size_t)n);
  L.scan = take(4 * (size_t)n);
  L.lev = take((size_t)n);
  L.status = take(sizeof(AllocStatus));
  L.bad = take(4);
  L.temp_bytes = std::max(sort_temp, scan_temp);
  L.temp = take(L.temp_bytes);
  L.total = o;
  return L;
}

}  // namespace
}  // namespace msq

using namespace msq;

extern "C" size_t msq_alloc_workspace_bytes(int64_t n_blocks) {
  if (n_blocks <= 0 || n_blocks > MSQ_ALLOC_MAX_BLOCKS) return 0;
  const AllocLayout L = alloc_layout(n_blocks);
  return L.ok ? L.total : 0;
}

extern "C" msq_status msq_allocate_bits(const float* utility, int64_t n_blocks, int64_t budget_bits,
                                        uint8_t* bits, void* workspace, size_t workspace_bytes,
                                        int32_t* iterations, hipStream_t stream) {
  if (!utility || !bits || !workspace || (reinterpret_cast<uintptr_t>(utility) & 3) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255))
    return MSQ_ERR_INVALID_ARG;
  if (n_blocks <= 0 || n_blocks > MSQ_ALLOC_MAX_BLOCKS || budget_bits < 0) return MSQ_ERR_SHAPE;
  const AllocLayout L = alloc_layout(n_blocks);
  if (!L.ok) return MSQ_ERR_HIP;
  if (workspace_bytes < L.total) return MSQ_ERR_BUFFER_TOO_SMALL;
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  auto at = [&](size_t off) { return ws + off; };
  uint32_t* key_in = reinterpret_cast<uint32_t*>(at(L.key_in));
  uint32_t* key_out = reinterpret_cast<uint32_t*>(at(L.key_out));
  int32_t* val_in = reinterpret_cast<int32_t*>(at(L.val_in));
  int32_t* val_out = reinterpret_cast<int32_t*>(at(L.val_out));
  int32_t* sorted_cost = reinterpret_cast<int32_t*>(at(L.sorted_cost));
  int32_t* scan = reinterpret_cast<int32_t*>(at(L.scan));
  uint8_t* lev = at(L.lev);
  AllocStatus* st = reinterpret_cast<AllocStatus*>(at(L.status));
  int32_t* bad = reinterpret_cast<int32_t*>(at(L.bad));
  void* temp = at(L.temp);
  const int n = (int)n_blocks;
  const unsigned grid = (unsigned)((n_blocks + 255) / 256);
  const int64_t total = n_blocks * kLevels;

  // utilities must be finite
  int32_t h_bad = 0;
  if (hipMemcpyAsync(bad, &h_bad, 4, hipMemcpyHostToDevice, stream) != hipSuccess)
    return MSQ_ERR_HIP;
  hipLaunchKernelGGL(k_alloc_check, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                     utility, total, bad);
  if (hipMemcpyAsync(&h_bad, bad, 4, hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return MSQ_ERR_HIP;
  if (h_bad) return MSQ_ERR_INVALID_ARG;

  hipLaunchKernelGGL(k_alloc_init, dim3(grid), dim3(256), 0, stream, lev, n_blocks, st, budget_bits);
  int32_t iters = 0;
  // every iteration moves at least one block up a level: at most 5 n iterations
  for (int64_t guard = 0; guard <= 5 * n_blocks; ++guard) {
    hipLaunchKernelGGL(k_alloc_keys, dim3(grid), dim3(256), 0, stream, utility, lev, n_blocks,
                       key_in, val_in);
    size_t tb = L.temp_bytes;
    if (hipcub::DeviceRadixSort::SortPairsDescending(temp, tb, key_in, key_out, val_in, val_out, n,
                                                     0, 32, stream) != hipSuccess)
      return MSQ_ERR_HIP;
    hipLaunchKernelGGL(k_alloc_costs, dim3(grid), dim3(256), 0, stream, val_out, n_blocks,
                       sorted_cost);
    tb = L.temp_bytes;
    if (hipcub::DeviceScan::InclusiveSum(temp, tb, sorted_cost, scan, n, stream) != hipSuccess)
      return MSQ_ERR_HIP;
    hipLaunchKernelGGL(k_alloc_select, dim3(1), dim3(64), 0, stream, scan, n_blocks, st);
    hipLaunchKernelGGL(k_alloc_first, dim3(grid), dim3(256), 0, stream, sorted_cost, n_blocks, st);
    hipLaunchKernelGGL(k_alloc_finish, dim3(1), dim3(64), 0, stream, sorted_cost, st);
    hipLaunchKernelGGL(k_alloc_apply, dim3(grid), dim3(256), 0, stream, val_out, n_blocks, st,
                       lev);
    AllocStatus h{};
    if (hipGetLastError() != hipSuccess ||
        hipMemcpyAsync(&h, st, sizeof(h), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
      return MSQ_ERR_HIP;
    if (h.taken == 0) break;
    ++iters;
  }
  hipLaunchKernelGGL(k_alloc_bits, dim3(grid), dim3(256), 0, stream, lev, n_blocks, bits);
  if (hipGetLastError() != hipSuccess) return MSQ_ERR_HIP;
  if (iterations) *iterations = iters;
  return MSQ_OK;
}

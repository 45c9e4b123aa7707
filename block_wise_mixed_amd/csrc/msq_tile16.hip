// 16-bit (passthrough) blocks: tiles kept at bf16 beside quantized ones
// ("TileQuant" abstract, fugumt.com page: the highest-scoring tiles stay at
// 16 bits, the kernel computes natively on 16-bit values).  The quantized
// kernels treat these blocks as pruned (scale 0); this pass adds their exact
// products afterwards:
//     y[m][perm_row[n]] += sum over 16-bit blocks (r, c) of row n of
//                          sum_k x[m][perm_col[128 c + k]] W[n][k].
// The packed block is the bf16 weight in the format's b-bit layout with one
// fragment per chunk, so chunk F = 4 rt + kt at lane l is already the matrix
// instruction's B operand for row tile rt, k-step kt: no unpacking.
//
// Workgroup (block row r, 16 or 64 rows of M); wavefront rt owns rows
// 16 rt .. 16 rt + 15 of the block row.  Per 16-bit block: x's slice is
// staged in LDS (from the reordered x the gather kernel left in the
// workspace, or gathered through perm_col at M == 1), each wavefront loads
// its four chunks and issues (m tiles) x 4 (k-steps) matrix instructions.  Every output is
// owned by one thread, which adds its sum to y once (no atomics; the pass
// runs after the quantized kernels on the same stream).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "msq_dequant.h"
#include "msq_internal.h"

namespace msq {
namespace {

extern __shared__ __align__(16) unsigned char smem_t16[];

constexpr int kT16Threads = 256;
constexpr int kT16Stride = kBlockCols + 8;  // LDS row of x, bf16 (+16 bytes against conflicts)

// kMT m tiles of 16 rows per workgroup (4: M > 16).  xr: x
// already reordered along K ([M][K], the gather kernel's output in the
// caller's workspace), read with 16-byte loads; null: x gathered through
// perm_col here.
template <int kMT>
__global__ __launch_bounds__(kT16Threads) void k_tile16(const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ xr, int M,
                                                        WeightView w, float* __restrict__ y) {
  constexpr int kRows = 16 * kMT;
  __shared__ __align__(16) uint16_t xs[kRows * kT16Stride];
  __shared__ int pc[kBlockCols];
  const int r = blockIdx.x;
  const int64_t m0 = (int64_t)blockIdx.y * kRows;
  const int t = threadIdx.x, lane = t & 63;
  const int rt = __builtin_amdgcn_readfirstlane(t >> 6);
  const int kk = (int)w.K - 1;
  f32x4 acc[kMT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  bool any = false;
  for (int c = 0; c < w.NBc; ++c) {
    const int64_t blk = (int64_t)r * w.NBc + c;
    if (w.bits[blk] != 16) continue;
    any = true;
    __syncthreads();  // the previous block's readers of xs and pc are done
    if (xr) {
      // rows past M repeat row M - 1 (their outputs are never stored)
      for (int e = t; e < kRows * 16; e += kT16Threads) {
        const int mm = e >> 4, q = e & 15;
        const int64_t m = min(m0 + mm, (int64_t)M - 1);
        *reinterpret_cast<uint4*>(xs + mm * kT16Stride + 8 * q) =
            *reinterpret_cast<const uint4*>(xr + m * w.K + (int64_t)c * kBlockCols + 8 * q);
      }
    } else {
      if (t < kBlockCols) {
        const int p = w.perm_col[(int64_t)c * kBlockCols + t];
        pc[t] = p < 0 ? 0 : (p > kk ? kk : p);
      }
      __syncthreads();
      for (int e = t; e < kRows * kBlockCols; e += kT16Threads) {
        const int mm = e >> 7, k = e & (kBlockCols - 1);
        const int64_t m = min(m0 + mm, (int64_t)M - 1);
        xs[mm * kT16Stride + k] = x[m * w.K + pc[k]];
      }
    }
    const uint8_t* cb = w.codes + (int64_t)w.block_offset[blk] * 1024 + 16 * lane;
    uint4 b[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) b[kt] = *reinterpret_cast<const uint4*>(cb + 1024 * (4 * rt + kt));
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        // A fragment: row 16 mt + (lane & 15), columns 32 kt + 8 (lane >> 4) .. + 7
        const uint4 a = *reinterpret_cast<const uint4*>(
            xs + (16 * mt + (lane & 15)) * kT16Stride + 32 * kt + 8 * (lane >> 4));
        acc[mt] = mfma_bf16(as_bf16x8(a), as_bf16x8(b[kt]), acc[mt]);
      }
  }
  if (!any) return;
  // output (m, n): m = m0 + 16 mt + 4 (lane >> 4) + i, n = 64 r + 16 rt + (lane & 15)
  const int64_t n = (int64_t)r * kBlockRows + 16 * rt + (lane & 15);
  int64_t on = w.perm_row[n];
  on = on < 0 ? 0 : (on >= w.N ? w.N - 1 : on);
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + 16 * mt + 4 * (lane >> 4) + i;
      if (m < M) y[m * w.N + on] += acc[mt][i];
    }
}

// M <= 16: the four wavefronts of a workgroup (one block row) take the
// row's 16-bit blocks c with c % 4 == wave independently, each computing
// all 64 rows of its blocks (16 chunks, 16 matrix instructions per block),
// with no barrier per block; their sums are added through LDS in wavefront
// order at the end.  A operands straight from the reordered x (M > 1) or,
// at M == 1, from x gathered once per workgroup into LDS (row 0 of the
// operand; the other rows zero).
__global__ __launch_bounds__(kT16Threads) void k_tile16_small(const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ xr,
                                                              int M, WeightView w,
                                                              float* __restrict__ y) {
  __shared__ f32x4 red[4][4][64];
  uint16_t* xg = reinterpret_cast<uint16_t*>(smem_t16);  // M == 1: x reordered, [K]
  const int r = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kk = (int)w.K - 1;
  if (!xr) {
    for (int64_t j = threadIdx.x; j < w.K; j += kT16Threads) {
      const int p = w.perm_col[j];
      xg[j] = x[p < 0 ? 0 : (p > kk ? kk : p)];
    }
    __syncthreads();
  }
  const int arow = lane & 15, acol = 8 * (lane >> 4);  // A fragment: row, first column
  f32x4 acc[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the row's bit map and offsets 64 columns at a time (lane = column); this
  // wavefront's 16-bit blocks are the set bits of a ballot
  for (int c0 = 0; c0 < w.NBc; c0 += 64) {
    const int64_t rb = (int64_t)r * w.NBc + c0;
    const bool in = c0 + lane < w.NBc;
    const int bl = in ? w.bits[rb + lane] : 0;
    const uint32_t ol = in ? w.block_offset[rb + lane] : 0u;
    uint64_t todo = __ballot(bl == 16) & (0x1111111111111111ull << wave);
    while (todo) {
      const int p = __builtin_ctzll(todo);
      todo &= todo - 1;
      const int c = c0 + p;
      const uint32_t off = __builtin_amdgcn_readlane(ol, p);
      const uint8_t* cb = w.codes + (int64_t)off * 1024 + 16 * lane;
      uint4 b[16];
#pragma unroll
      for (int f = 0; f < 16; ++f) b[f] = *reinterpret_cast<const uint4*>(cb + 1024 * f);
      uint4 a[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const int64_t col = (int64_t)c * kBlockCols + 32 * kt + acol;
        if (xr) {
          const int64_t m = min(arow, M - 1);  // rows past M are never stored
          a[kt] = *reinterpret_cast<const uint4*>(xr + m * w.K + col);
        } else {
          // row 0 from the LDS copy; the other rows of the operand are zero
          const uint4 v = *reinterpret_cast<const uint4*>(xg + col);
          a[kt] = arow == 0 ? v : uint4{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          acc[rt] = mfma_bf16(as_bf16x8(a[kt]), as_bf16x8(b[4 * rt + kt]), acc[rt]);
    }
  }
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) red[wave][rt][lane] = acc[rt];
  __syncthreads();
  if (wave != 0) return;
  // output (m, n): m = 4 (lane >> 4) + i, n = 64 r + 16 rt + (lane & 15)
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    f32x4 s = red[0][rt][lane];
#pragma unroll
    for (int k = 1; k < 4; ++k) {
      const f32x4 t = red[k][rt][lane];
      s = f32x4{s[0] + t[0], s[1] + t[1], s[2] + t[2], s[3] + t[3]};
    }
    const int64_t n = (int64_t)r * kBlockRows + 16 * rt + (lane & 15);
    int64_t on = w.perm_row[n];
    on = on < 0 ? 0 : (on >= w.N ? w.N - 1 : on);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * (lane >> 4) + i;
      if (m < M) y[(int64_t)m * w.N + on] += s[i];
    }
  }
}

// M > 16: workgroup (block row r, 64 rows of M); as the small-M kernel, each
// wavefront takes the 16-bit blocks c = wave (mod 4) of the row from a
// ballot, with no barrier per block, and computes all 64 x 64 outputs of its
// blocks: A fragments (4 m tiles x 4 k-steps) straight from the reordered x
// in the workspace, B = the block's 16 chunks, 64 matrix instructions.  The
// four wavefronts' sums are added through LDS in wavefront order at the end.
__global__ __launch_bounds__(kT16Threads) void k_tile16_large(const uint16_t* __restrict__ xr,
                                                              int M, WeightView w,
                                                              float* __restrict__ y) {
  f32x4* red = reinterpret_cast<f32x4*>(smem_t16);  // [3][16][64]: wavefronts 1..3
  const int r = blockIdx.x;
  const int64_t m0 = (int64_t)blockIdx.y * 64;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int arow = lane & 15, acol = 8 * (lane >> 4);
  f32x4 acc[4][4];  // [mt][rt]
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[mt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < w.NBc; c0 += 64) {
    const int64_t rb = (int64_t)r * w.NBc + c0;
    const bool in = c0 + lane < w.NBc;
    const int bl = in ? w.bits[rb + lane] : 0;
    const uint32_t ol = in ? w.block_offset[rb + lane] : 0u;
    uint64_t todo = __ballot(bl == 16) & (0x1111111111111111ull << wave);
    while (todo) {
      const int p = __builtin_ctzll(todo);
      todo &= todo - 1;
      const int c = c0 + p;
      const uint32_t off = __builtin_amdgcn_readlane(ol, p);
      const uint8_t* cb = w.codes + (int64_t)off * 1024 + 16 * lane;
      uint4 b[16];
#pragma unroll
      for (int f = 0; f < 16; ++f) b[f] = *reinterpret_cast<const uint4*>(cb + 1024 * f);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        // rows past M repeat row M - 1 (their outputs are never stored)
        const int64_t m = min(m0 + 16 * mt + arow, (int64_t)M - 1);
        const uint16_t* src = xr + m * w.K + (int64_t)c * kBlockCols + acol;
        uint4 a[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) a[kt] = *reinterpret_cast<const uint4*>(src + 32 * kt);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
            acc[mt][rt] = mfma_bf16(as_bf16x8(a[kt]), as_bf16x8(b[4 * rt + kt]), acc[mt][rt]);
      }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) red[((wave - 1) * 16 + 4 * mt + rt) * 64 + lane] = acc[mt][rt];
  }
  __syncthreads();
  if (wave != 0) return;
  // output (m, n): m = m0 + 16 mt + 4 (lane >> 4) + i, n = 64 r + 16 rt + (lane & 15)
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int64_t n = (int64_t)r * kBlockRows + 16 * rt + (lane & 15);
    int64_t on = w.perm_row[n];
    on = on < 0 ? 0 : (on >= w.N ? w.N - 1 : on);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 s = acc[mt][rt];
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const f32x4 t = red[(k * 16 + 4 * mt + rt) * 64 + lane];
        s = f32x4{s[0] + t[0], s[1] + t[1], s[2] + t[2], s[3] + t[3]};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + 16 * mt + 4 * (lane >> 4) + i;
        if (m < M) y[m * w.N + on] += s[i];
      }
    }
  }
}

}  // namespace

hipError_t launch_tile16(const uint16_t* x, const uint16_t* xr, int64_t M, const WeightView& w,
                         float* y, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  // the small-M kernel keeps x's reordered row in LDS when it has no xr
  if (M <= 16 && (xr || w.K <= 32768)) {
    const size_t lds = xr ? 0 : (size_t)w.K * 2;  // M == 1: the reordered x row
    hipLaunchKernelGGL(k_tile16_small, dim3((unsigned)w.NBr), dim3(kT16Threads), lds, stream, x, xr,
                       (int)M, w, y);
  } else if (xr) {
    const dim3 grid((unsigned)w.NBr, (unsigned)((M + 63) / 64));
    hipLaunchKernelGGL(k_tile16_large, grid, dim3(kT16Threads), (size_t)3 * 16 * 64 * 16, stream,
                       xr, (int)M, w, y);
  } else {
    const dim3 grid((unsigned)w.NBr, (unsigned)((M + 63) / 64));
    hipLaunchKernelGGL(k_tile16<4>, grid, dim3(kT16Threads), 0, stream, x, xr, (int)M, w, y);
  }
  return hipGetLastError();
}

}  // namespace msq

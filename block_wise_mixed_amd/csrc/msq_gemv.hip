// Decode GEMV for gfx950: y = x . W^T for M <= 64, W dequantized block by
// block from packed format v1 in registers.  Memory-bound: every byte of the
// packed codes is read once, with one 16-byte load per lane per 1 KiB chunk.
//
// Work split.  A workgroup of NW wavefronts owns one block row r (64 output
// rows) and a range of at most 64 block columns [c0, c0 + ncl) (a K split).
//  1. Every wavefront reads the range's bit map with one lane per column and
//     forms, per bitwidth, a 64-bit mask of the columns holding it (wave
//     ballots).  Walking bitwidths 1, 2, 3, 4, 8 and columns in order gives
//     the blocks in packed order; the wavefronts cut that list into NW pieces
//     of equal packed size, so each wavefront gets at most a few runs of
//     same-bitwidth blocks.
//  2. The workgroup gathers its slice of the activations through perm_col
//     into LDS (the activation reordering of the "SFMP" abstract), with the
//     per-group sums of x used to fold the zero point.
//  3. Each wavefront walks its runs.  Inside a run the bitwidth is a
//     compile-time constant, so the next block's b chunk loads (and its
//     scales and zero points) are issued before the current block is
//     unpacked and multiplied: two blocks in flight per wavefront with
//     static wait counts.  Each 16x32 fragment is unpacked into exact bf16
//     operands and fed to v_mfma_f32_16x16x32_bf16 (M padded to 16), then
//     scale and zero point are folded per row:
//         y[row] += s * (sum_k (bias + q_k) x_k - (bias + z) * sum_k x_k).
//  4. The wavefronts reduce through LDS in a fixed order.  One K split writes
//     y directly (scattered to original rows through perm_row); several
//     splits write fp32 partials that k_gemv_reduce sums in split order, so
//     results are bitwise reproducible.
//
// Per-block precision and block layout: "ScaleBITS" summary page, section
// Approach; RTN-g128 dequantization s * (q - z): section Limitations.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdlib>
#include <utility>

#include "msq_dequant.h"
#include "msq_internal.h"

namespace msq {
namespace {

constexpr int kMaxCols = 64;  // block columns per workgroup: one wave ballot
constexpr size_t kLdsBudget = 64 * 1024;

__device__ __forceinline__ float bf16f(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

__device__ __forceinline__ int64_t orig_row(const int32_t* perm_row, int64_t i, int64_t N) {
  const int64_t v = perm_row[i];
  return v < 0 ? 0 : (v >= N ? N - 1 : v);
}

__device__ __forceinline__ int clampi(int v, int hi) { return v < 0 ? 0 : (v > hi ? hi : v); }

struct Ctx {
  const uint8_t* codes;
  const uint32_t* block_offset;
  const float* scale;
  const uint8_t* zero;
  int64_t rowbase;       // r * NBc + c0: block index of the range's first column
  const uint16_t* xs;    // LDS x slice [M][xs_stride]
  const float* xsum;     // LDS group sums [M][kmax]
  int xs_stride;         // bf16 elements per LDS row
  int kmax;              // block columns per workgroup (row length of xsum)
  int M;
  const float* corr;     // M == 1: LDS [kmax][16] bias corrections per (column, bitwidth, row tile)
  const unsigned char* lds;  // LDS base
  uint32_t a_lane;       // M == 1: LDS byte offset of this lane's A operand (zero area if dead)
  uint32_t a_step;       // M == 1: bytes per block column for live lanes, 0 for dead lanes
};

// ---- one block: unpack + matrix-core product into acc[mt][rt] ----------------------------
template <int B, int MT>
__device__ __forceinline__ void block_product(const uint4 (&ch)[B], const bf16x8 (&A)[MT][4],
                                              f32x4 (&acc)[MT][4]) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[mt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // kt outer, rt inner: consecutive instructions feed four independent accumulators
  auto step = [&](auto Ic) {
    constexpr int I = decltype(Ic)::value;
    constexpr int kt = I / 4, rt = I % 4;
    constexpr int F = 4 * rt + kt;
    const bf16x8 bop = block_operand<B, F>(ch);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt][rt] = mfma_bf16(A[mt][kt], bop, acc[mt][rt]);
    if constexpr (B == 3) {
      const bf16x8 hop = hi3_operand<F>(ch);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt][rt] = mfma_bf16(A[mt][kt], hop, acc[mt][rt]);
    }
  };
  [&]<int... Fs>(std::integer_sequence<int, Fs...>) {
    (step(std::integral_constant<int, Fs>{}), ...);
  }(std::make_integer_sequence<int, 16>{});
}

// M == 1 variant: shift-minimizing unpack (biases removed by the correction table).
template <int B>
__device__ __forceinline__ void block_product_m1(const uint4 (&ch)[B], const bf16x8 (&A)[4],
                                                 f32x4 (&acc)[4]) {
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto step = [&](auto Ic) {
    constexpr int I = decltype(Ic)::value;
    constexpr int kt = I / 4, rt = I % 4;
    constexpr int F = 4 * rt + kt;
    if constexpr (B == 8) {
      acc[rt] = mfma_bf16(A[kt], block_operand<8, F>(ch), acc[rt]);
    } else {
      acc[rt] = mfma_bf16(A[kt], exp_operand<B, F>(ch), acc[rt]);
      if constexpr (B == 3) acc[rt] = mfma_bf16(A[kt], exp_hi3_operand<F>(ch), acc[rt]);
    }
  };
  [&]<int... Is>(std::integer_sequence<int, Is...>) {
    (step(std::integral_constant<int, Is>{}), ...);
  }(std::make_integer_sequence<int, 16>{});
}

// A operands of block column cl: x rows 16*mt + (l & 15), columns 32*kt + 8*(l >> 4) .. +7.
// With M1 only row 0 exists and lanes with (l & 15) != 0 carry zeros.
template <int MT, bool M1>
__device__ __forceinline__ void load_a(const Ctx& cx, int cl, bf16x8 (&A)[MT][4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = 16 * mt + (lane & 15);
    const bool live = M1 ? ((lane & 15) == 0) : (m < cx.M);
    const uint16_t* row = cx.xs + (size_t)(M1 ? 0 : m) * cx.xs_stride + cl * kBlockCols + 8 * (lane >> 4);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      uint4 v = {0u, 0u, 0u, 0u};
      if (live) v = *reinterpret_cast<const uint4*>(row + 32 * kt);
      A[mt][kt] = as_bf16x8(v);
    }
  }
}

// Route acc[0][rt][0] of lanes 0..15 (rows 16*rt + l when only x row 0 is
// live) to lane 16*rt + l: two 16-lane-row swaps and one half swap.
__device__ __forceinline__ float rows_to_lanes(const f32x4 (&acc)[1][4]) {
  const uint32_t v0 = __float_as_uint(acc[0][0][0]), v1 = __float_as_uint(acc[0][1][0]);
  const uint32_t v2 = __float_as_uint(acc[0][2][0]), v3 = __float_as_uint(acc[0][3][0]);
  auto p01 = __builtin_amdgcn_permlane16_swap(v0, v1, false, false);
  auto p23 = __builtin_amdgcn_permlane16_swap(v2, v3, false, false);
  auto q = __builtin_amdgcn_permlane32_swap(p01[0], p23[0], false, false);
  return __uint_as_float(q[0]);
}

// Per-block operands that live in registers while the block is in flight.
template <int B>
struct BlockRegs {
  uint4 ch[B];
  float s;     // scale of row `lane`
  uint32_t z;  // zero point of row `lane`
};

// Issue the loads of one block: its b chunks at `base` (this lane's 16 bytes
// of the block's first chunk) and the scale / zero point of row `lane`.
template <int B>
__device__ __forceinline__ void issue_block(const Ctx& cx, const uint8_t* base, int cl,
                                            BlockRegs<B>& br) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = cx.rowbase + cl;
#pragma unroll
  for (int t = 0; t < B; ++t) br.ch[t] = *reinterpret_cast<const uint4*>(base + 1024 * t);
  br.s = cx.scale[blk * kBlockRows + lane];
  br.z = cx.zero[blk * kBlockRows + lane];
}

template <int B, int MT, bool M1>
__device__ __forceinline__ void consume_block(const Ctx& cx, int cl, const BlockRegs<B>& br,
                                              float& y1, f32x4 (&yacc)[MT][4]) {
  const int lane = threadIdx.x & 63;
  if constexpr (M1) {
    // A operands: lanes 0, 16, 32, 48 read x; the others read the zero area
    bf16x8 A[4];
    const unsigned char* a = cx.lds + cx.a_lane + (uint32_t)cl * cx.a_step;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) A[kt] = as_bf16x8(*reinterpret_cast<const uint4*>(a + 64 * kt));
    f32x4 acc[1][4];
    block_product_m1<B>(br.ch, A, acc[0]);
    const float v = rows_to_lanes(acc);
    constexpr int kidx = B == 1 ? 0 : (B == 2 ? 1 : (B == 3 ? 2 : 3));
    const float corr = B == 8 ? 0.f : cx.corr[cl * 16 + kidx * 4 + (lane >> 4)];
    y1 += br.s * ((v - corr) - (float)br.z * cx.xsum[cl]);
    return;
  }
  bf16x8 A[MT][4];
  load_a<MT, M1>(cx, cl, A);
  f32x4 acc[MT][4];
  block_product<B, MT>(br.ch, A, acc);
  constexpr float bias = (float)unpack_bias(B);
  {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int src = 16 * rt + (lane & 15);
      const float s = __shfl(br.s, src, 64);
      const float zz = bias + (float)__shfl((int)br.z, src, 64);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 16 * mt + 4 * (lane >> 4) + i;
          const float sx = m < cx.M ? cx.xsum[m * cx.kmax + cl] : 0.f;
          yacc[mt][rt][i] += s * (acc[mt][rt][i] - zz * sx);
        }
    }
  }
}

// Blocks per batch of a B-bit run: 4 to 8 KiB of chunks in flight per
// wavefront, within a register budget that keeps 4 wavefronts per SIMD.
// Larger M keeps more accumulators live, so its batches are smaller.
template <int B, int MT, bool M1>
constexpr int batch_of() {
  if constexpr (M1) return B == 1 ? 4 : (B == 2 ? 4 : (B == 3 ? 2 : (B == 4 ? 2 : 1)));
  else if constexpr (MT == 1) return B <= 2 ? 2 : 1;
  else return 1;
}

// CNT consecutive blocks of a run (run indices i .. i+CNT-1, columns taken
// from `cols` in order): issue all their loads, then consume them in order.
// Straight-line code in which every load is consumed, so the wait counts are
// static and no load stays in flight past the section.
template <int B, int CNT, int MT, bool M1>
__device__ __forceinline__ void run_batch(const Ctx& cx, const uint8_t* base, int i, uint64_t& cols,
                                          float& y1, f32x4 (&yacc)[MT][4]) {
  BlockRegs<B> br[CNT];
  int cc[CNT];
#pragma unroll
  for (int j = 0; j < CNT; ++j) {
    cc[j] = __builtin_amdgcn_readfirstlane(__builtin_ctzll(cols));
    cols &= cols - 1;
    issue_block<B>(cx, base + (int64_t)(i + j) * (1024 * B), cc[j], br[j]);
  }
#pragma unroll
  for (int j = 0; j < CNT; ++j) consume_block<B, MT, M1>(cx, cc[j], br[j], y1, yacc);
}

// A run of n blocks of bitwidth B whose columns are the lowest n set bits of
// `cols`.  Blocks of one bitwidth in one block row are consecutive in packed
// order, so block i of the run starts b * i KiB after the first, at `base`
// (this lane's 16 bytes of the run's first chunk).  Full batches first, then
// the remainder in batches of 4, 2 and 1 blocks.
template <int B, int MT, bool M1>
__device__ __forceinline__ void run_blocks(const Ctx& cx, const uint8_t* base, uint64_t cols, int n,
                                           float& y1, f32x4 (&yacc)[MT][4]) {
  constexpr int BATCH = batch_of<B, MT, M1>();
  int i = 0;
  for (; i + BATCH <= n; i += BATCH) run_batch<B, BATCH, MT, M1>(cx, base, i, cols, y1, yacc);
  if constexpr (BATCH > 4) {
    if (n - i >= 4) {
      run_batch<B, 4, MT, M1>(cx, base, i, cols, y1, yacc);
      i += 4;
    }
  }
  if constexpr (BATCH > 2) {
    if (n - i >= 2) {
      run_batch<B, 2, MT, M1>(cx, base, i, cols, y1, yacc);
      i += 2;
    }
  }
  if constexpr (BATCH > 1) {
    if (n - i >= 1) run_batch<B, 1, MT, M1>(cx, base, i, cols, y1, yacc);
  }
}

// This lane's pointer into the first chunk of the block at run column c.
__device__ __forceinline__ const uint8_t* run_base(const Ctx& cx, uint32_t off_kib) {
  return cx.codes + (int64_t)off_kib * 1024 + 16 * (threadIdx.x & 63);
}

__constant__ int kSegBits[5] = {1, 2, 3, 4, 8};

// Gather x[m][perm_col[128*(c0+cl) + j]] into LDS xs[m][cl*128 + j] and the
// per-group sums into xsum[m][cl].  Item = (m, 8-column chunk); 16 chunks
// make a group and sit in 16 consecutive lanes, reduced with shuffles.
__device__ __forceinline__ void gather_x(const uint16_t* __restrict__ x, int M, int64_t K,
                                         const int32_t* __restrict__ perm_col, int c0, int ncl,
                                         uint16_t* xs, int xs_stride, float* xsum, int kmax,
                                         int nthreads) {
  const int chunks = ncl * 16;
  const int items = M * chunks;
  const int kk = (int)K - 1;
  for (int base = 0; base < items; base += nthreads) {
    const int it = base + (int)threadIdx.x;
    float part = 0.f;
    int m = 0, q = 0;
    if (it < items) {
      m = it / chunks;
      q = it - m * chunks;
      const int4* pc = reinterpret_cast<const int4*>(perm_col + (int64_t)c0 * kBlockCols + 8 * q);
      const int4 p0 = pc[0], p1 = pc[1];
      const uint16_t* xr = x + (int64_t)m * K;
      const uint16_t u0 = xr[clampi(p0.x, kk)], u1 = xr[clampi(p0.y, kk)];
      const uint16_t u2 = xr[clampi(p0.z, kk)], u3 = xr[clampi(p0.w, kk)];
      const uint16_t u4 = xr[clampi(p1.x, kk)], u5 = xr[clampi(p1.y, kk)];
      const uint16_t u6 = xr[clampi(p1.z, kk)], u7 = xr[clampi(p1.w, kk)];
      uint4 v;
      v.x = (uint32_t)u0 | ((uint32_t)u1 << 16);
      v.y = (uint32_t)u2 | ((uint32_t)u3 << 16);
      v.z = (uint32_t)u4 | ((uint32_t)u5 << 16);
      v.w = (uint32_t)u6 | ((uint32_t)u7 << 16);
      *reinterpret_cast<uint4*>(xs + (size_t)m * xs_stride + 8 * q) = v;
      part = ((bf16f(u0) + bf16f(u1)) + (bf16f(u2) + bf16f(u3))) +
             ((bf16f(u4) + bf16f(u5)) + (bf16f(u6) + bf16f(u7)));
    }
    // items of one group are 16 consecutive threads (chunks is a multiple of 16)
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) part += __shfl_xor(part, d, 64);
    if (it < items && (q & 15) == 0) xsum[m * kmax + (q >> 4)] = part;
  }
}

// M == 1 gather: as gather_x, plus for every block column the sums of x over
// each 32-column k-step, from which the bias correction of every (bitwidth,
// row tile) is tabulated: corr[cl][4*k + rt] = sum_kt bias(b_k, 4*rt + kt) * Sx[kt]
// for b_k = 1, 2, 3, 4 (8-bit blocks carry no bias).
__device__ __forceinline__ void gather_x_m1(const uint16_t* __restrict__ x, int64_t K,
                                            const int32_t* __restrict__ perm_col, int c0, int ncl,
                                            uint16_t* xs, float* xsum, float* corr, int nthreads) {
  const int lane = threadIdx.x & 63;
  const int items = ncl * 16;
  const int kk = (int)K - 1;
  for (int base = 0; base < items; base += nthreads) {
    const int q = base + (int)threadIdx.x;
    float part = 0.f;
    if (q < items) {
      const int4* pc = reinterpret_cast<const int4*>(perm_col + (int64_t)c0 * kBlockCols + 8 * q);
      const int4 p0 = pc[0], p1 = pc[1];
      const uint16_t u0 = x[clampi(p0.x, kk)], u1 = x[clampi(p0.y, kk)];
      const uint16_t u2 = x[clampi(p0.z, kk)], u3 = x[clampi(p0.w, kk)];
      const uint16_t u4 = x[clampi(p1.x, kk)], u5 = x[clampi(p1.y, kk)];
      const uint16_t u6 = x[clampi(p1.z, kk)], u7 = x[clampi(p1.w, kk)];
      uint4 v;
      v.x = (uint32_t)u0 | ((uint32_t)u1 << 16);
      v.y = (uint32_t)u2 | ((uint32_t)u3 << 16);
      v.z = (uint32_t)u4 | ((uint32_t)u5 << 16);
      v.w = (uint32_t)u6 | ((uint32_t)u7 << 16);
      *reinterpret_cast<uint4*>(xs + 8 * q) = v;
      part = ((bf16f(u0) + bf16f(u1)) + (bf16f(u2) + bf16f(u3))) +
             ((bf16f(u4) + bf16f(u5)) + (bf16f(u6) + bf16f(u7)));
    }
    // k-step sums: 4 consecutive chunks (32 columns)
    part += __shfl_xor(part, 1, 64);
    part += __shfl_xor(part, 2, 64);
    const int g0 = lane & ~15;
    const float s0 = __shfl(part, g0, 64), s1 = __shfl(part, g0 + 4, 64);
    const float s2 = __shfl(part, g0 + 8, 64), s3 = __shfl(part, g0 + 12, 64);
    if (q < items) {
      const int j = q & 15, k = j >> 2, rt = j & 3;
      const int b = k + 1;  // bitwidths 1, 2, 3, 4
      const float c = exp_bias(b, 4 * rt) * s0 + exp_bias(b, 4 * rt + 1) * s1 +
                      exp_bias(b, 4 * rt + 2) * s2 + exp_bias(b, 4 * rt + 3) * s3;
      corr[(q >> 4) * 16 + j] = c;
      if (j == 0) xsum[q >> 4] = (s0 + s1) + (s2 + s3);
    }
  }
}

template <int NW, int MT, bool M1>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(M1 ? 4 : 1))) void k_gemv(const uint16_t* __restrict__ x, int M,
                                                  WeightView w, int split, int kmax, int xs_stride,
                                                  float* __restrict__ out, int direct) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = blockIdx.x / split, sp = blockIdx.x - (blockIdx.x / split) * split;
  const int c0 = sp * kmax;
  const int ncl = min(w.NBc, c0 + kmax) - c0;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  float* xsum = reinterpret_cast<float*>(smem + (size_t)M * xs_stride * 2);
  // M == 1 extras after xsum: corr [kmax][16], then a 256-byte zero area
  float* corr = xsum + kmax;
  const uint32_t zero_off = (uint32_t)(((size_t)M * xs_stride * 2 + (size_t)kmax * 4 * 17 + 15) & ~(size_t)15);

  // 1. this wavefront's share of the range's blocks, in packed order
  const int64_t rowbase = (int64_t)r * w.NBc + c0;
  const int bl = lane < ncl ? (int)w.bits[rowbase + lane] : 0;
  uint64_t mask[5];
  int cnt[5], start[5];
  int tot = 0;
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    mask[k] = __ballot(bl == kSegBits[k]);
    cnt[k] = __popcll(mask[k]);
    start[k] = tot;
    tot += cnt[k] * kSegBits[k];
  }
  const int lo = (wave * tot + NW - 1) / NW, hi = ((wave + 1) * tot + NW - 1) / NW;

  // 2. activation slice
  Ctx cx{w.codes, w.block_offset, w.scale, w.zero, rowbase, xs, xsum, xs_stride, kmax, M, corr, smem,
         0u, 0u};
  if constexpr (M1) {
    if (threadIdx.x < 64) reinterpret_cast<uint32_t*>(smem + zero_off)[threadIdx.x] = 0u;
    gather_x_m1(x, w.K, w.perm_col, c0, ncl, xs, xsum, corr, NW * 64);
    const bool live = (lane & 15) == 0;
    cx.a_lane = live ? (uint32_t)(16 * (lane >> 4)) : zero_off;
    cx.a_step = live ? (uint32_t)(kBlockCols * 2) : 0u;
  } else {
    gather_x(x, M, w.K, w.perm_col, c0, ncl, xs, xs_stride, xsum, kmax, NW * 64);
  }
  __syncthreads();

  float y1 = 0.f;
  f32x4 yacc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) yacc[mt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // 3. runs
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    const int b = kSegBits[k];
    const int a0 = lo - start[k], a1 = hi - start[k];
    int j0 = a0 <= 0 ? 0 : (a0 + b - 1) / b;
    int j1 = a1 <= 0 ? 0 : (a1 + b - 1) / b;
    j0 = min(j0, cnt[k]);
    j1 = min(j1, cnt[k]);
    if (j1 <= j0) continue;
    uint64_t cols = mask[k];
    for (int j = 0; j < j0; ++j) cols &= cols - 1;
    const int n = j1 - j0;
    const int c_first = __builtin_amdgcn_readfirstlane(__builtin_ctzll(cols));
    const uint8_t* base =
        run_base(cx, __builtin_amdgcn_readfirstlane(cx.block_offset[cx.rowbase + c_first]));
    switch (k) {
      case 0: run_blocks<1, MT, M1>(cx, base, cols, n, y1, yacc); break;
      case 1: run_blocks<2, MT, M1>(cx, base, cols, n, y1, yacc); break;
      case 2: run_blocks<3, MT, M1>(cx, base, cols, n, y1, yacc); break;
      case 3: run_blocks<4, MT, M1>(cx, base, cols, n, y1, yacc); break;
      default: run_blocks<8, MT, M1>(cx, base, cols, n, y1, yacc); break;
    }
  }

  // 4. reduce the wavefronts in a fixed order and write out
  __syncthreads();  // LDS is reused below
  float* red = reinterpret_cast<float*>(smem);
  if constexpr (M1) {
    if (wave > 0) red[(wave - 1) * 64 + lane] = y1;
    __syncthreads();
    if (wave == 0) {
      float v = y1;
#pragma unroll
      for (int k = 0; k < NW - 1; ++k) v += red[k * 64 + lane];
      const int64_t row = (int64_t)r * kBlockRows + lane;
      if (direct) {
        out[orig_row(w.perm_row, row, w.N)] = v;
      } else {
        out[(int64_t)sp * w.N + row] = v;
      }
    }
  } else {
    const int plane = M * kBlockRows;
    if (wave > 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = 16 * mt + 4 * (lane >> 4) + i;
            if (m < M) red[(wave - 1) * plane + m * kBlockRows + 16 * rt + (lane & 15)] = yacc[mt][rt][i];
          }
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = 16 * mt + 4 * (lane >> 4) + i;
            if (m >= M) continue;
            const int n = 16 * rt + (lane & 15);
            float v = yacc[mt][rt][i];
#pragma unroll
            for (int k = 0; k < NW - 1; ++k) v += red[k * plane + m * kBlockRows + n];
            const int64_t row = (int64_t)r * kBlockRows + n;
            if (direct) {
              out[(int64_t)m * w.N + orig_row(w.perm_row, row, w.N)] = v;
            } else {
              out[((int64_t)sp * M + m) * w.N + row] = v;
            }
          }
    }
  }
}

// ---- M = 1 decode ------------------------------------------------------------------------
//
// Same work split as k_gemv, with the workgroup's dependency chain shortened:
// the bit map, the block offsets (one per lane / column) and the permutation
// indices of the activation gather are all read in one round trip; then each
// wavefront issues the loads of its first batch of blocks *before* gathering
// x, so the code fetch overlaps the gather instead of waiting behind it.
// Run bases come from the offsets already in registers (v_readlane).

// Finish the activation gather for item q (8 columns) whose permutation
// indices p0, p1 are already loaded: LDS x slice, and for each block column
// the 32-column k-step sums, their total and the bias-correction table.
__device__ __forceinline__ void gather_finish_m1(const uint16_t* __restrict__ x, int kk, int q,
                                                 int items, int4 p0, int4 p1, uint16_t* xs,
                                                 float* xsum, float* corr) {
  const int lane = threadIdx.x & 63;
  float part = 0.f;
  if (q < items) {
    const uint16_t u0 = x[clampi(p0.x, kk)], u1 = x[clampi(p0.y, kk)];
    const uint16_t u2 = x[clampi(p0.z, kk)], u3 = x[clampi(p0.w, kk)];
    const uint16_t u4 = x[clampi(p1.x, kk)], u5 = x[clampi(p1.y, kk)];
    const uint16_t u6 = x[clampi(p1.z, kk)], u7 = x[clampi(p1.w, kk)];
    uint4 v;
    v.x = (uint32_t)u0 | ((uint32_t)u1 << 16);
    v.y = (uint32_t)u2 | ((uint32_t)u3 << 16);
    v.z = (uint32_t)u4 | ((uint32_t)u5 << 16);
    v.w = (uint32_t)u6 | ((uint32_t)u7 << 16);
    *reinterpret_cast<uint4*>(xs + 8 * q) = v;
    part = ((bf16f(u0) + bf16f(u1)) + (bf16f(u2) + bf16f(u3))) +
           ((bf16f(u4) + bf16f(u5)) + (bf16f(u6) + bf16f(u7)));
  }
  part += __shfl_xor(part, 1, 64);
  part += __shfl_xor(part, 2, 64);
  const int g0 = lane & ~15;
  const float s0 = __shfl(part, g0, 64), s1 = __shfl(part, g0 + 4, 64);
  const float s2 = __shfl(part, g0 + 8, 64), s3 = __shfl(part, g0 + 12, 64);
  if (q < items) {
    const int j = q & 15, k = j >> 2, rt = j & 3;
    const int b = k + 1;  // bitwidths 1, 2, 3, 4
    corr[(q >> 4) * 16 + j] = exp_bias(b, 4 * rt) * s0 + exp_bias(b, 4 * rt + 1) * s1 +
                              exp_bias(b, 4 * rt + 2) * s2 + exp_bias(b, 4 * rt + 3) * s3;
    if (j == 0) xsum[q >> 4] = (s0 + s1) + (s2 + s3);
  }
}

struct GatherM1 {
  const uint16_t* x;
  const int32_t* perm_col;  // already offset to the range's first column
  int kk, items, nthreads;
  uint16_t* xs;
  float* xsum;
  float* corr;
};

// Complete the gather: the first pass with the preloaded indices, further
// passes (ranges wider than one item per thread) load their own.
__device__ __forceinline__ void gather_all_m1(const GatherM1& g, int4 p0, int4 p1) {
  gather_finish_m1(g.x, g.kk, (int)threadIdx.x, g.items, p0, p1, g.xs, g.xsum, g.corr);
  for (int q = g.nthreads + (int)threadIdx.x; q - (int)threadIdx.x < g.items; q += g.nthreads) {
    int4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
    if (q < g.items) {
      const int4* pc = reinterpret_cast<const int4*>(g.perm_col + 8 * q);
      a = pc[0];
      b = pc[1];
    }
    gather_finish_m1(g.x, g.kk, q, g.items, a, b, g.xs, g.xsum, g.corr);
  }
}

// A run of n >= 1 blocks of bitwidth B (M == 1), two blocks in flight: while
// block i is consumed the loads of block i+1 are outstanding.  The two
// register sets keep fixed roles (no swaps), issues are unconditional (a
// missing block repeats the run's last one) and the loop only exits right
// after a consume, so every path into the loop header has the same loads
// outstanding in the same order and the waits stay exact.  Code size is two
// consume bodies per bitwidth.
template <int B>
__device__ __forceinline__ void run_m1(const Ctx& cx, const uint8_t* base, uint64_t cols, int n,
                                    float& y1) {
  constexpr int64_t kStride = 1024 * B;
  f32x4 unused[1][4];
  BlockRegs<B> ra, rb;
  int ca = __builtin_amdgcn_readfirstlane(__builtin_ctzll(cols));
  cols &= cols - 1;
  int cb = ca;
  if (n > 1) {
    cb = __builtin_amdgcn_readfirstlane(__builtin_ctzll(cols));
    cols &= cols - 1;
  }
  issue_block<B>(cx, base, ca, ra);
  issue_block<B>(cx, base + (n > 1 ? kStride : 0), cb, rb);
  // compiler-only barrier: keep the loads issued here, ahead of the consume
  // below (the compiler would otherwise sink them toward their first use)
  asm volatile("" ::: "memory");
  for (int i = 0;; i += 2) {
    consume_block<B, 1, true>(cx, ca, ra, y1, unused);
    if (i + 1 >= n) break;
    // block i+2 (or a repeat of the last block) into the set just consumed
    const int ia = i + 2 < n ? i + 2 : n - 1;
    if (i + 2 < n) {
      ca = __builtin_amdgcn_readfirstlane(__builtin_ctzll(cols));
      cols &= cols - 1;
    }
    issue_block<B>(cx, base + (int64_t)ia * kStride, ca, ra);
    asm volatile("" ::: "memory");
    consume_block<B, 1, true>(cx, cb, rb, y1, unused);
    if (i + 2 >= n) break;
    const int ib = i + 3 < n ? i + 3 : n - 1;
    if (i + 3 < n) {
      cb = __builtin_amdgcn_readfirstlane(__builtin_ctzll(cols));
      cols &= cols - 1;
    }
    issue_block<B>(cx, base + (int64_t)ib * kStride, cb, rb);
    asm volatile("" ::: "memory");
  }
}

template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4))) void k_gemv_m1(
    const uint16_t* __restrict__ x, WeightView w, int split, int kmax, int xs_stride,
    float* __restrict__ out, int direct) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = blockIdx.x / split, sp = blockIdx.x - (blockIdx.x / split) * split;
  const int c0 = sp * kmax;
  const int ncl = min(w.NBc, c0 + kmax) - c0;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  float* xsum = reinterpret_cast<float*>(smem + (size_t)xs_stride * 2);
  float* corr = xsum + kmax;
  const uint32_t zero_off = (uint32_t)(((size_t)xs_stride * 2 + (size_t)kmax * 4 * 17 + 15) & ~(size_t)15);
  const int64_t rowbase = (int64_t)r * w.NBc + c0;

  // one round trip: bit map and offsets (lane = column), first gather indices
  const int bl = lane < ncl ? (int)w.bits[rowbase + lane] : 0;
  const uint32_t ol = lane < ncl ? w.block_offset[rowbase + lane] : 0u;
  const int items = ncl * 16;
  const int32_t* pcol = w.perm_col + (int64_t)c0 * kBlockCols;
  int4 p0 = {0, 0, 0, 0}, p1 = {0, 0, 0, 0};
  if ((int)threadIdx.x < items) {
    const int4* pc = reinterpret_cast<const int4*>(pcol + 8 * threadIdx.x);
    p0 = pc[0];
    p1 = pc[1];
  }
  if (threadIdx.x < 64) reinterpret_cast<uint32_t*>(smem + zero_off)[threadIdx.x] = 0u;

  uint64_t mask[5];
  int cnt[5], start[5];
  int tot = 0;
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    mask[k] = __ballot(bl == kSegBits[k]);
    cnt[k] = __popcll(mask[k]);
    start[k] = tot;
    tot += cnt[k] * kSegBits[k];
  }
  const int lo = (wave * tot + NW - 1) / NW, hi = ((wave + 1) * tot + NW - 1) / NW;
  // this wavefront's part of each run: columns and first offset
  uint64_t cols[5];
  int n[5];
  uint32_t off[5];
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    const int b = kSegBits[k];
    const int a0 = lo - start[k], a1 = hi - start[k];
    int j0 = a0 <= 0 ? 0 : (a0 + b - 1) / b;
    int j1 = a1 <= 0 ? 0 : (a1 + b - 1) / b;
    j0 = min(j0, cnt[k]);
    j1 = min(j1, cnt[k]);
    uint64_t c = mask[k];
    for (int j = 0; j < j0; ++j) c &= c - 1;
    cols[k] = c;
    n[k] = j1 - j0;
    off[k] = 0;
    if (n[k] > 0) off[k] = __builtin_amdgcn_readlane(ol, __builtin_ctzll(c));
  }

  Ctx cx{w.codes, w.block_offset, w.scale, w.zero, rowbase, xs, xsum, xs_stride, kmax, 1, corr, smem,
         0u, 0u};
  const bool live = (lane & 15) == 0;
  cx.a_lane = live ? (uint32_t)(16 * (lane >> 4)) : zero_off;
  cx.a_step = live ? (uint32_t)(kBlockCols * 2) : 0u;
  const GatherM1 g{x, pcol, (int)w.K - 1, items, NW * 64, xs, xsum, corr};
  gather_all_m1(g, p0, p1);
  __syncthreads();
  float y1 = 0.f;
  if (n[0] > 0) run_m1<1>(cx, run_base(cx, off[0]), cols[0], n[0], y1);
  if (n[1] > 0) run_m1<2>(cx, run_base(cx, off[1]), cols[1], n[1], y1);
  if (n[2] > 0) run_m1<3>(cx, run_base(cx, off[2]), cols[2], n[2], y1);
  if (n[3] > 0) run_m1<4>(cx, run_base(cx, off[3]), cols[3], n[3], y1);
  if (n[4] > 0) run_m1<8>(cx, run_base(cx, off[4]), cols[4], n[4], y1);

  // reduce the wavefronts in a fixed order and write out
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
  if (wave > 0) red[(wave - 1) * 64 + lane] = y1;
  __syncthreads();
  if (wave == 0) {
    float v = y1;
#pragma unroll
    for (int k = 0; k < NW - 1; ++k) v += red[k * 64 + lane];
    const int64_t row = (int64_t)r * kBlockRows + lane;
    if (direct) {
      out[orig_row(w.perm_row, row, w.N)] = v;
    } else {
      out[(int64_t)sp * w.N + row] = v;
    }
  }
}

// y[m][perm_row[n]] = sum over splits (in order) of partial[sp][m][n].
__global__ __launch_bounds__(256) void k_gemv_reduce(const float* __restrict__ part, int split,
                                                     int M, int64_t N,
                                                     const int32_t* __restrict__ perm_row,
                                                     float* __restrict__ y) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)M * N) return;
  const int64_t m = idx / N, n = idx - (idx / N) * N;
  const int64_t plane = (int64_t)M * N;
  const float* p = part + m * N + n;
  // issue eight partial loads at a time, then add them in split order
  float v = 0.f;
  int sp = 0;
  for (; sp + 8 <= split; sp += 8) {
    float t[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) t[k] = p[(sp + k) * plane];
#pragma unroll
    for (int k = 0; k < 8; ++k) v += t[k];
  }
  for (; sp < split; ++sp) v += p[sp * plane];
  y[m * N + orig_row(perm_row, n, N)] = v;
}

template <int NW>
hipError_t launch_m1(const uint16_t* x, const WeightView& w, float* dst, const GemvPlan& p,
                     int direct, hipStream_t stream) {
  const unsigned grid = (unsigned)(w.NBr * p.split);
  hipLaunchKernelGGL((k_gemv_m1<NW>), dim3(grid), dim3(NW * 64), p.lds_bytes, stream, x, w,
                     p.split, p.kr, p.xs_stride, dst, direct);
  return hipGetLastError();
}

template <int NW, int MT, bool M1>
hipError_t launch_cfg(const uint16_t* x, int M, const WeightView& w, float* dst,
                      const GemvPlan& p, int direct, hipStream_t stream) {
  const unsigned grid = (unsigned)(w.NBr * p.split);
  hipLaunchKernelGGL((k_gemv<NW, MT, M1>), dim3(grid), dim3(NW * 64), p.lds_bytes, stream, x, M,
                     w, p.split, p.kr, p.xs_stride, dst, direct);
  return hipGetLastError();
}

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  return (v && *v) ? std::atoi(v) : dflt;
}

}  // namespace

// Launch shape.  The block columns of a block row are split into `split`
// ranges of at most 64 columns so that the grid has about 512 workgroups of
// NW = 8 wavefronts (two per CU), using as few splits as possible because
// each split adds an fp32 partial and a reduce.  MSQ_GEMV_SPLIT overrides the
// split count (tuning only).
GemvPlan plan_gemv(int64_t M, int64_t N, int64_t K) {
  GemvPlan p{};
  const int NBr = (int)(N / kBlockRows), NBc = (int)(K / kBlockCols);
  p.mt = (int)((M + 15) / 16);
  p.nw = M > 16 ? 4 : 8;
  if (M == 1) {
    const int nw = env_int("MSQ_GEMV_WAVES", 8);  // tuning only
    p.nw = (nw == 4 || nw == 16) ? nw : 8;
  }
  // LDS per block column: x slice (2 bytes x 128 per row) + one group sum per row
  const size_t per_col = (size_t)M * (kBlockCols * 2 + 4);
  int kr_max = (int)((kLdsBudget - 16 * (size_t)M) / per_col);
  if (kr_max > kMaxCols) kr_max = kMaxCols;
  if (kr_max < 1) kr_max = 1;
  int split = env_int("MSQ_GEMV_SPLIT", 0);
  if (split <= 0) split = (512 + NBr - 1) / NBr;
  if (split > NBc) split = NBc;
  if (split < 1) split = 1;
  int kr = (NBc + split - 1) / split;
  if (kr > kr_max) kr = kr_max;
  split = (NBc + kr - 1) / kr;
  p.split = split;
  p.kr = kr;
  p.xs_stride = kr * kBlockCols + 8;  // +16 bytes per row against LDS bank conflicts
  size_t x_bytes = (size_t)M * p.xs_stride * 2 + (size_t)M * kr * 4;
  if (M == 1) x_bytes += (size_t)kr * 64 + 256 + 16;  // correction table + aligned zero area
  const size_t red_bytes = (size_t)(p.nw - 1) * (size_t)M * kBlockRows * 4;
  p.lds_bytes = x_bytes > red_bytes ? x_bytes : red_bytes;
  p.workspace = split > 1 ? (size_t)split * M * N * 4 : 0;
  return p;
}

hipError_t launch_gemv(const uint16_t* x, int64_t M, const WeightView& w, float* y,
                       void* workspace, const GemvPlan& p, hipStream_t stream) {
  const int direct = p.split == 1;
  float* dst = direct ? y : reinterpret_cast<float*>(workspace);
  hipError_t e;
  if (M == 1) {
    if (p.nw == 4) e = launch_m1<4>(x, w, dst, p, direct, stream);
    else if (p.nw == 16) e = launch_m1<16>(x, w, dst, p, direct, stream);
    else e = launch_m1<8>(x, w, dst, p, direct, stream);
  } else if (p.nw == 8) {
    e = launch_cfg<8, 1, false>(x, (int)M, w, dst, p, direct, stream);
  } else {
    switch (p.mt) {
      case 2: e = launch_cfg<4, 2, false>(x, (int)M, w, dst, p, direct, stream); break;
      case 3: e = launch_cfg<4, 3, false>(x, (int)M, w, dst, p, direct, stream); break;
      default: e = launch_cfg<4, 4, false>(x, (int)M, w, dst, p, direct, stream); break;
    }
  }
  if (e != hipSuccess || direct) return e;
  const int64_t total = M * w.N;
  hipLaunchKernelGGL(k_gemv_reduce, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                     reinterpret_cast<const float*>(workspace), p.split, (int)M, w.N, w.perm_row, y);
  return hipGetLastError();
}

}  // namespace msq

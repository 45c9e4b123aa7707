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
//  2. The activations, reordered through perm_col once per call by the
//     gather kernel (the activation reordering of the "SFMP" abstract), are
//     staged in LDS slice by slice together with their per-group sums, used
//     to fold the zero point.
//  3. Each wavefront walks its runs.  Inside a run the bitwidth is a
//     compile-time constant, so the loads of the next blocks (codes, scales,
//     zero points) are issued while the current block is unpacked and
//     multiplied, with static wait counts.  Each 16x32 fragment is unpacked
//     into exact bf16 operands and fed to v_mfma_f32_16x16x32_bf16 (M padded
//     to 16), then scale and zero point are folded per row:
//         y[row] += s * (sum_k (bias + q_k) x_k - (bias + z) * sum_k x_k).
//  4. The wavefronts reduce through LDS in a fixed order.  One K split writes
//     y directly (scattered to original rows through perm_row); several
//     splits write fp32 partials that are summed in split order (M == 1: by
//     the last workgroup of the block row to finish; M > 1: by
//     k_gemv_reduce), so results are bitwise reproducible.
//
// M == 1 has its own kernels (k_gemv_m1, after k_prep_m1 only when K is
// split into several ranges): the reordered x comes with per-column k-step
// sums for the bias corrections, the unpack avoids most shifts, the scales
// and zero points are staged in LDS, and each wavefront keeps 2 to 4 KiB of
// codes in flight.
//
// Per-block precision and block layout: "ScaleBITS" summary page, section
// Approach; RTN-g128 dequantization s * (q - z): section Limitations.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cstdlib>
#include <utility>

#include "msq_dequant.h"
#include "msq_internal.h"

namespace msq {
namespace {

// Dynamic LDS of every kernel in this file.  Device code indexes it with
// 32-bit offsets: 64-bit pointer arithmetic on it can pick up the upper half
// of a register pair that an outstanding load still owns, which costs a wait.
extern __shared__ __align__(16) unsigned char smem[];

constexpr int kMaxCols = 64;  // block columns per workgroup: one wave ballot
constexpr size_t kLdsBudget = 64 * 1024;

__device__ __forceinline__ float bf16f(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

__device__ __forceinline__ int64_t orig_row(const int32_t* perm_row, int64_t i, int64_t N) {
  const int64_t v = perm_row[i];
  return v < 0 ? 0 : (v >= N ? N - 1 : v);
}

__device__ __forceinline__ int clampi(int v, int hi) { return v < 0 ? 0 : (v > hi ? hi : v); }

__constant__ int kSegBits[5] = {1, 2, 3, 4, 8};

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
  uint32_t sums_off;     // M == 1: LDS byte offset of the k-step sums [kmax][4] f32
  uint32_t a_lane;       // M == 1: LDS byte offset of this lane's A operand in column 0
  uint32_t zero_off;     // M == 1: LDS byte offset of the zero area (A operand of dead lanes)
  uint32_t s_off;        // M == 1: LDS byte offset of the range's scales [ncl][64] f32
  uint32_t z_off;        // M == 1: LDS byte offset of the range's zero points [ncl][64] u8
};

// This lane's pointer into the first chunk of a run whose first block is at off_kib.
__device__ __forceinline__ const uint8_t* run_base(const Ctx& cx, uint32_t off_kib) {
  return cx.codes + (int64_t)off_kib * 1024 + 16 * (threadIdx.x & 63);
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
// The block index passes through an empty asm so that the compiler cannot
// tell two issues of the same block apart (the register rings repeat a
// run's last block past its end): merging such loads would tie the ring's
// register sets together and add waits.
// With kScaleZero false (M == 1) only the codes are loaded: the workgroup
// stages the scales and zero points of its range in LDS at start-up.
template <int B, bool kScaleZero = true>
__device__ __forceinline__ void issue_block(const Ctx& cx, const uint8_t* base, int cl,
                                            BlockRegs<B>& br) {
  const int lane = threadIdx.x & 63;
  cl = __builtin_amdgcn_readfirstlane(cl);
  asm("" : "+s"(cl));
  const int64_t blk = cx.rowbase + cl;
#pragma unroll
  for (int t = 0; t < B; ++t) br.ch[t] = *reinterpret_cast<const uint4*>(base + 1024 * t);
  if constexpr (kScaleZero) {
    br.s = cx.scale[blk * kBlockRows + lane];
    br.z = cx.zero[blk * kBlockRows + lane];
  }
}

// The wavefront's share of the range's blocks: per bitwidth k, the columns
// (lowest n[k] set bits of cols[k]) of its part of the run.
struct WaveRuns {
  uint64_t cols[5];
  int n[5];
};

// Cut the range's packed order (runs of bitwidths 1, 2, 3, 4, 8) into NW
// pieces of equal weight, block k of bitwidth kSegBits[k] weighing wt[k];
// bl = bitwidth of column `lane` (0 beyond the range).  A block belongs to the
// piece that holds its first unit of weight.
template <int NW>
__device__ __forceinline__ WaveRuns wave_runs(int bl, int wave, const int (&wt)[5]) {
  uint64_t mask[5];
  int cnt[5], start[5];
  int tot = 0;
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    mask[k] = __ballot(bl == kSegBits[k]);
    cnt[k] = __popcll(mask[k]);
    start[k] = tot;
    tot += cnt[k] * wt[k];
  }
  const int lo = (wave * tot + NW - 1) / NW, hi = ((wave + 1) * tot + NW - 1) / NW;
  WaveRuns wr;
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    const int b = wt[k];
    const int a0 = lo - start[k], a1 = hi - start[k];
    int j0 = a0 <= 0 ? 0 : (a0 + b - 1) / b;
    int j1 = a1 <= 0 ? 0 : (a1 + b - 1) / b;
    j0 = min(j0, cnt[k]);
    j1 = min(j1, cnt[k]);
    uint64_t c = mask[k];
    for (int j = 0; j < j0; ++j) c &= c - 1;
    wr.cols[k] = c;
    wr.n[k] = j1 - j0;
  }
  return wr;
}

// Piece weights: packed size (KiB per block) for the general path; for
// M == 1, where a block's unpack and matrix instructions take about as long
// as its loads, the measured per-block cost of a wavefront in units of
// about 0.1 us (1- and 2-bit blocks alike, 3- and 4-bit alike, 8-bit twice
// those) so that the wavefronts of a workgroup finish together.
constexpr int kWeightBytes[5] = {1, 2, 3, 4, 8};
constexpr int kWeightCostM1[5] = {4, 4, 9, 9, 17};

// ======================================================================================
// General M (2 .. 64)
// ======================================================================================

// One block: unpack + matrix-core product into acc[mt][rt].
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

// A operands of block column cl: x rows 16*mt + (l & 15), columns 32*kt + 8*(l >> 4) .. +7.
template <int MT>
__device__ __forceinline__ void load_a(const Ctx& cx, int cl, bf16x8 (&A)[MT][4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = 16 * mt + (lane & 15);
    const bool live = m < cx.M;
    const uint16_t* row = cx.xs + (size_t)m * cx.xs_stride + cl * kBlockCols + 8 * (lane >> 4);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      uint4 v = {0u, 0u, 0u, 0u};
      if (live) v = *reinterpret_cast<const uint4*>(row + 32 * kt);
      A[mt][kt] = as_bf16x8(v);
    }
  }
}

template <int B, int MT>
__device__ __forceinline__ void consume_block(const Ctx& cx, int cl, const BlockRegs<B>& br,
                                              f32x4 (&yacc)[MT][4]) {
  const int lane = threadIdx.x & 63;
  bf16x8 A[MT][4];
  load_a<MT>(cx, cl, A);
  f32x4 acc[MT][4];
  block_product<B, MT>(br.ch, A, acc);
  constexpr float bias = (float)unpack_bias(B);
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

// Blocks per register ring of a B-bit run: (depth - 1) * B KiB of codes stay
// in flight while one block is consumed.  Thousands of wavefronts share
// HBM, so shallow rings already keep more in flight than it needs; deeper
// ones only lengthen the queues that every workgroup's start-up waits in
// (M == 1 on a 70B layer: 4/2/2/2/2 blocks for 1/2/3/4/8 bits measured ~6%
// faster than 8/4/3/3/2).  More rows of M keep more accumulators live, so
// their rings are shallower still.
template <int B, int MT = 1>
constexpr int ring_depth() {
  if constexpr (MT == 1) return B == 1 ? 4 : 2;
  else if constexpr (MT == 2) return B <= 4 ? 2 : 1;
  else return B <= 2 ? 2 : 1;
}

// A run of n >= 1 blocks of bitwidth B whose columns are the lowest n set
// bits of `cols`, starting at `base` (this lane's 16 bytes of the run's first
// chunk; block i of the run starts B * i KiB later).  A ring of D register
// sets with fixed roles: set j holds blocks j, j + D, j + 2D, ...; after
// block i is consumed, the loads of block i + D go into its set.  Issues are
// unconditional and the loop runs whole passes over the ring with its only
// exit at the end of a pass, so every consume sees the same loads
// outstanding in the same order and the wait counts stay static: D - 1
// blocks in flight during each consume.  Past the end of the run an issue
// is a stand-in that is never consumed: the same loads with every lane's
// address masked to the start of the codes (one cache line per load
// instead of a KiB; no branch, so the loads keep their form).  (An exit from the middle of the
// unrolled body leaves structurized control-flow paths on which the
// compiler cannot bound the outstanding loads, and it then waits for all.)
// kScaleZero: the ring also loads each block's scales and zero points (two
// more loads per block).  consume(column, registers) uses a block;
// after_issue(integral_constant<loads issued>) runs once after the first D
// blocks are issued.
template <int B, int D, bool kScaleZero, typename Consume, typename AfterIssue>
__device__ __forceinline__ void ring_run(const Ctx& cx, const uint8_t* base, uint64_t cols, int n,
                                         Consume&& consume, AfterIssue&& after_issue) {
  constexpr int64_t kStride = 1024 * B;
  BlockRegs<B> rs[D];
  int cs[D];
  const int64_t lane_off = base - cx.codes;  // this lane's offset of the run's first block
  // block bi of the run, or (live false) the stand-in address
  auto slot = [&](bool live, int bi) __attribute__((always_inline)) {
    return cx.codes + ((lane_off + (int64_t)bi * kStride) & -(int64_t)live);
  };
  // compiler-only barriers after the issues keep the loads where they are
  // written (the compiler would otherwise sink them toward their first use)
#pragma unroll
  for (int j = 0; j < D; ++j) {
    if (j == 0 || j < n) {
      cs[j] = __builtin_amdgcn_readfirstlane(__builtin_ctzll(cols));
      cols &= cols - 1;
    } else {
      cs[j] = cs[j - 1];
    }
    int bi = __builtin_amdgcn_readfirstlane(j);
    asm("" : "+s"(bi));
    issue_block<B, kScaleZero>(cx, slot(j < n, bi), cs[j], rs[j]);
    asm volatile("" ::: "memory");
  }
  // the first run: the workgroup's start-up, while these loads fly
  after_issue(std::integral_constant<int, D * (B + (kScaleZero ? 2 : 0))>{});
  int i0 = 0;  // run index of the block in set 0
  do {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      if (i0 + j < n) consume(cs[j], rs[j]);
      const int nx = i0 + j + D;
      if (nx < n) {
        cs[j] = __builtin_amdgcn_readfirstlane(__builtin_ctzll(cols));
        cols &= cols - 1;
      }
      int bi = __builtin_amdgcn_readfirstlane(nx);
      asm("" : "+s"(bi));
      issue_block<B, kScaleZero>(cx, slot(nx < n, bi), cs[j], rs[j]);
      asm volatile("" ::: "memory");
    }
    i0 += D;
  } while (i0 < n);
}

// A run of n blocks of bitwidth B whose columns are the lowest n set bits of
// `cols`.  Blocks of one bitwidth in one block row are consecutive in packed
// order, so block i of the run starts b * i KiB after the first, at `base`
// (this lane's 16 bytes of the run's first chunk).
template <int B, int MT>
__device__ __forceinline__ void run_blocks(const Ctx& cx, const uint8_t* base, uint64_t cols, int n,
                                           f32x4 (&yacc)[MT][4]) {
  ring_run<B, ring_depth<B, MT>(), true>(
      cx, base, cols, n,
      [&](int cl, const BlockRegs<B>& br) __attribute__((always_inline)) {
        consume_block<B, MT>(cx, cl, br, yacc);
      },
      [](auto) __attribute__((always_inline)) {});
}

// The workgroup's activation slice: rows 0 .. M-1 of the reordered x_r
// (written once per call by the gather kernel) for block columns c0 ..
// c0 + ncl - 1, copied into LDS with 16-byte loads, and the group sums
// rebuilt from their three bf16 terms (S0 + S1 + S2 is exact in fp32).
// The loads of kBatch items are issued before any store, and every thread
// stores at its clamped item (threads past the end rewrite the last item
// with the value they loaded from it), so no store is conditional.
__device__ __forceinline__ void stage_x(const uint16_t* __restrict__ xr,
                                        const uint16_t* __restrict__ sxs, int M, int64_t K,
                                        int64_t Gp, int c0, int ncl, uint16_t* xs, int xs_stride,
                                        float* xsum, int kmax, int nthreads) {
  constexpr int kBatch = 4;
  const int chunks = ncl * 16;
  const int items = M * chunks;
  for (int base = threadIdx.x; base < items; base += kBatch * nthreads) {
    uint4 v[kBatch];
    int dst[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int it = min(base + u * nthreads, items - 1);
      const int m = it / chunks, q = it - (it / chunks) * chunks;
      v[u] = reinterpret_cast<const uint4*>(xr + (int64_t)m * K + (int64_t)c0 * kBlockCols)[q];
      dst[u] = m * xs_stride + 8 * q;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) *reinterpret_cast<uint4*>(xs + dst[u]) = v[u];
  }
  const int64_t plane = (int64_t)M * Gp;
  for (int it = threadIdx.x; it < M * ncl; it += nthreads) {
    const int m = it / ncl, c = it - (it / ncl) * ncl;
    const uint16_t* s = sxs + (int64_t)m * Gp + c0 + c;
    xsum[m * kmax + c] = (bf16f(s[0]) + bf16f(s[plane])) + bf16f(s[2 * plane]);
  }
}

template <int NW, int MT>
__global__ __launch_bounds__(NW * 64) void k_gemv(const uint16_t* __restrict__ xr,
                                                  const uint16_t* __restrict__ sxs, int M,
                                                  WeightView w, int split, int kmax, int xs_stride,
                                                  float* __restrict__ out, int direct) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = blockIdx.x / split, sp = blockIdx.x - (blockIdx.x / split) * split;
  const int c0 = sp * kmax;
  const int ncl = min(w.NBc, c0 + kmax) - c0;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  float* xsum = reinterpret_cast<float*>(smem + (size_t)M * xs_stride * 2);

  // 1. this wavefront's share of the range's blocks, in packed order
  const int64_t rowbase = (int64_t)r * w.NBc + c0;
  const int bl = lane < ncl ? (int)w.bits[rowbase + lane] : 0;
  const uint32_t ol = lane < ncl ? w.block_offset[rowbase + lane] : 0u;
  const WaveRuns wr = wave_runs<NW>(bl, wave, kWeightBytes);

  // 2. activation slice
  Ctx cx{w.codes, w.block_offset, w.scale, w.zero, rowbase, xs, xsum, xs_stride, kmax, M, 0u, 0u,
         0u, 0u};
  stage_x(xr, sxs, M, w.K, padded_groups(w.NBc), c0, ncl, xs, xs_stride, xsum, kmax, NW * 64);
  __syncthreads();

  f32x4 yacc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) yacc[mt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // 3. runs
  uint32_t off[5];
#pragma unroll
  for (int k = 0; k < 5; ++k)
    off[k] = wr.n[k] > 0 ? __builtin_amdgcn_readlane(ol, __builtin_ctzll(wr.cols[k])) : 0u;
  if (wr.n[0] > 0) run_blocks<1, MT>(cx, run_base(cx, off[0]), wr.cols[0], wr.n[0], yacc);
  if (wr.n[1] > 0) run_blocks<2, MT>(cx, run_base(cx, off[1]), wr.cols[1], wr.n[1], yacc);
  if (wr.n[2] > 0) run_blocks<3, MT>(cx, run_base(cx, off[2]), wr.cols[2], wr.n[2], yacc);
  if (wr.n[3] > 0) run_blocks<4, MT>(cx, run_base(cx, off[3]), wr.cols[3], wr.n[3], yacc);
  if (wr.n[4] > 0) run_blocks<8, MT>(cx, run_base(cx, off[4]), wr.cols[4], wr.n[4], yacc);

  // 4. reduce the wavefronts in a fixed order and write out
  __syncthreads();  // LDS is reused below
  float* red = reinterpret_cast<float*>(smem);
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

// ======================================================================================
// M == 1
// ======================================================================================
//
// k_prep_m1 reorders x once per call into the workspace: xg[j] = x[perm_col[j]]
// and, per block column c, the k-step sums S_c[kt] (kt = 0..3, each over 32
// reordered columns); with one K range k_gemv_m1 forms both itself.
// k_gemv_m1 copies its range of both into LDS with 16-byte loads; per block
// it forms the group sum and the bias correction
//     corr = sum_kt exp_bias(b, 4*rt + kt) * S_c[kt]
// (rt = the lane's row tile) from them.
//
// M == 1 uses one row of the 16-row A operand: lanes with (l & 15) == 0 read
// x, the others read a zero area, and the 64 row results of a block come out
// in lanes 0..15 of the four row-tile accumulators (rows_to_lanes moves row
// 16*rt + n to lane 16*rt + n).


// One wavefront per block column; lane l handles columns 2l, 2l + 1.
// Workgroup `blk` of the prep of one matrix.
__device__ __forceinline__ void prep_m1(const uint16_t* __restrict__ x, int64_t K,
                                        const int32_t* __restrict__ perm_col,
                                        uint16_t* __restrict__ xg, float4* __restrict__ sums,
                                        uint32_t* __restrict__ counters, int ncounters, int blk) {
  const int lane = threadIdx.x & 63;
  const int64_t gid = (int64_t)blk * 256 + threadIdx.x;
  if (gid < ncounters) counters[gid] = 0u;
  const int64_t c = (int64_t)blk * 4 + (threadIdx.x >> 6);
  if (c >= K / kBlockCols) return;
  const int64_t j = c * kBlockCols + 2 * lane;
  const int2 p = *reinterpret_cast<const int2*>(perm_col + j);
  const int kk = (int)K - 1;
  const uint16_t u0 = x[clampi(p.x, kk)], u1 = x[clampi(p.y, kk)];
  *reinterpret_cast<uint32_t*>(xg + j) = (uint32_t)u0 | ((uint32_t)u1 << 16);
  // k-step kt = lane >> 4: sum over its 16 lanes
  float s = bf16f(u0) + bf16f(u1);
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) s += __shfl_xor(s, d, 64);
  const float s0 = __shfl(s, 0, 64), s1 = __shfl(s, 16, 64);
  const float s2 = __shfl(s, 32, 64), s3 = __shfl(s, 48, 64);
  if (lane == 0) sums[c] = float4{s0, s1, s2, s3};
}

__global__ __launch_bounds__(256) void k_prep_m1(const uint16_t* __restrict__ x, int64_t K,
                                                 const int32_t* __restrict__ perm_col,
                                                 uint16_t* __restrict__ xg,
                                                 float4* __restrict__ sums,
                                                 uint32_t* __restrict__ counters, int ncounters) {
  prep_m1(x, K, perm_col, xg, sums, counters, ncounters, blockIdx.x);
}

// Route element 0 of v0..v3, lanes 0..15 (rows 16*rt + l of row tile rt;
// lanes 16..63 of element 0 are exact zeros, the dead rows of the padded
// product) to lane 16*rt + l: two 16-lane-row swaps and one half swap.
__device__ __forceinline__ float rows_to_lanes(float v0, float v1, float v2, float v3) {
  auto p01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v0), __float_as_uint(v1), false, false);
  auto p23 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v2), __float_as_uint(v3), false, false);
  auto q = __builtin_amdgcn_permlane32_swap(p01[0], p23[0], false, false);
  return __uint_as_float(q[0]);
}

// Unpack and multiply one B-bit block (M == 1), kt outer and rt inner so that
// consecutive matrix instructions feed different accumulators.  3-bit and
// 8-bit fragments are two planes, i.e. two matrix instructions.
template <int B>
__device__ __forceinline__ void block_product_m1(const uint4 (&ch)[B], const bf16x8 (&A)[4],
                                                 f32x4 (&acc)[4]) {
  auto step = [&](auto Ic) {
    constexpr int I = decltype(Ic)::value;
    constexpr int kt = I / 4, rt = I % 4, F = 4 * rt + kt;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const uint4& c = ch[chunk_of<B, F>()];
    f32x4 a = mfma_bf16(A[kt], exp_lo<B, F>(c), kt == 0 ? zero : acc[rt]);
    if constexpr (B == 3) a = mfma_bf16(A[kt], exp_hi<3, F>(ch[2]), a);
    if constexpr (B == 8) a = mfma_bf16(A[kt], exp_hi<8, F>(c), a);
    acc[rt] = a;
  };
  [&]<int... Is>(std::integer_sequence<int, Is...>) {
    (step(std::integral_constant<int, Is>{}), ...);
  }(std::make_integer_sequence<int, 16>{});
}

// Unpack, multiply and fold one block (column cl) into y1 (row `lane`):
//     y1 += s * ((sum_k (bias_k + q_k) x_k - corr) - z * sum_k x_k),
// corr = sum_kt bias[kt] * S[kt] with this lane's biases `bias` (row tile
// lane >> 4, bitwidth B) and the column's k-step sums S.
template <int B>
__device__ __forceinline__ void consume_m1(const Ctx& cx, int cl, const BlockRegs<B>& br,
                                           float& y1, const float4& bias) {
  const int lane = threadIdx.x & 63;
  // A operands: lanes 0, 16, 32, 48 read x; the others read the zero area
  bf16x8 A[4];
  // a shift and a select: a 32-bit multiply here becomes a 64-bit
  // multiply-add whose unused upper addend can alias an in-flight load
  const uint32_t a = (lane & 15) == 0 ? cx.a_lane + ((uint32_t)cl << 8) : cx.zero_off;
  static_assert(kBlockCols * 2 == 256, "bytes of x per block column");
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
    A[kt] = as_bf16x8(*reinterpret_cast<const uint4*>(smem + a + 64 * kt));
  f32x4 acc[4];
  block_product_m1<B>(br.ch, A, acc);
  const float v = rows_to_lanes(acc[0][0], acc[1][0], acc[2][0], acc[3][0]);
  const float4 S = *reinterpret_cast<const float4*>(smem + cx.sums_off + ((uint32_t)cl << 4));
  const float corr = bias.x * S.x + bias.y * S.y + bias.z * S.z + bias.w * S.w;
  const float xsum = (S.x + S.y) + (S.z + S.w);
  const float sc = *reinterpret_cast<const float*>(smem + cx.s_off + ((uint32_t)cl << 8) + 4 * lane);
  const uint32_t z = smem[cx.z_off + ((uint32_t)cl << 6) + lane];
  y1 += sc * ((v - corr) - (float)z * xsum);
}

// M == 1 run: the ring of ring_depth<B>() blocks, codes only.
template <int B, typename AfterIssue>
__device__ __forceinline__ void run_ring(const Ctx& cx, const uint8_t* base, uint64_t cols, int n,
                                         float& y1, AfterIssue&& after_issue) {
  // this lane's unpack biases of k-steps 0..3 (row tile lane >> 4)
  const int rt = (threadIdx.x & 63) >> 4;
  auto pick = [rt](auto KTc) __attribute__((always_inline)) {
    constexpr int kt = decltype(KTc)::value;
    return rt == 0 ? exp_bias(B, kt)
                   : (rt == 1 ? exp_bias(B, 4 + kt) : (rt == 2 ? exp_bias(B, 8 + kt) : exp_bias(B, 12 + kt)));
  };
  const float4 bias{pick(std::integral_constant<int, 0>{}), pick(std::integral_constant<int, 1>{}),
                    pick(std::integral_constant<int, 2>{}), pick(std::integral_constant<int, 3>{})};
  ring_run<B, ring_depth<B>(), false>(
      cx, base, cols, n,
      [&](int cl, const BlockRegs<B>& br) __attribute__((always_inline)) {
        consume_m1<B>(cx, cl, br, y1, bias);
      },
      after_issue);
}

// Direct global-to-LDS copies of 16 (4) bytes per lane: lane i writes at
// LDS byte `off` (wavefront-uniform, from the dynamic LDS base) + 16 i (4 i).
// Written as inline assembly because the compiler's builtin for them makes
// it wait for each copy to land before the next instruction that reuses the
// copy's address register, which serialises a run of copies; these have no
// register results, and the kernel waits for them itself (vmcnt) before the
// workgroup barrier that publishes the LDS data.  M0 carries the LDS address.
__device__ __forceinline__ uint32_t lds_addr(uint32_t off) {
  return (uint32_t)(uintptr_t)(lds_void*)(smem + off);
}
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16(const void* g, uint32_t off) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds_addr(off));
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m) : "memory", "m0");
}
__device__ __forceinline__ void lds_copy4(const void* g, uint32_t off) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds_addr(off));
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(m) : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS layout of k_gemv_m1 for ranges of ncl <= kmax block columns (38 KB at
// kmax = 64: four 8-wavefront workgroups fit a CU):
//   [0, 256 kmax)             x slice, bf16
//   [256 kmax, 272 kmax)      k-step sums [kmax][4], f32
//   zero area of 256 bytes
//   scales [ncl][64] f32, then zero points [ncl][64] u8, of the range's blocks
//   gathering workgroups only: the x row in original order, bf16 [128 kmax]
__host__ __device__ constexpr size_t m1_sums_offset(int kmax) { return (size_t)kmax * 256; }
__host__ __device__ constexpr size_t m1_zero_offset(int kmax) { return (size_t)kmax * 272; }
__host__ __device__ constexpr size_t m1_scale_offset(int kmax) { return m1_zero_offset(kmax) + 256; }
__host__ __device__ constexpr size_t m1_lds_bytes(int kmax) {
  return m1_scale_offset(kmax) + (size_t)kmax * (256 + 64);
}
__host__ __device__ constexpr size_t m1_xrow_offset(int kmax) { return m1_lds_bytes(kmax); }
__host__ __device__ constexpr size_t m1_lds_bytes_gather(int kmax) {
  return m1_xrow_offset(kmax) + (size_t)kmax * 256;
}

// Workgroup `blk` (block row blk / split, K range blk % split) of the M == 1
// decode of one matrix.  Two sources of the reordered x and its k-step sums:
// the prep kernel's output (xg, sums_g), or, with `gather` set (one K range,
// split == 1, so the workgroup needs all of x), x itself: the workgroup
// copies the x row into LDS and reorders it there through perm_col while
// its first code loads are in flight, so that no prep launch is needed.
// Both give the same bits: the reordered values are copies, and the k-step
// sums are formed by the same pairwise addition tree.
template <int NW, bool kGather>
__device__ __forceinline__ void gemv_m1(const uint16_t* __restrict__ xg,
                                        const float4* __restrict__ sums_g,
                                        const uint16_t* __restrict__ x,
                                        const WeightView& w, int split, int kmax,
                                        float* __restrict__ part, float* __restrict__ y,
                                        uint32_t* __restrict__ counters, int blk) {
  constexpr int kThreads = NW * 64;
  constexpr int kUnits = (kMaxCols * 16 + kThreads - 1) / kThreads;  // x slice loads per thread
  constexpr int kSumsUnits = (kMaxCols + kThreads - 1) / kThreads;    // k-step sum float4s
  constexpr int kSUnits = (kMaxCols * 16 + kThreads - 1) / kThreads;  // scale uint4s per thread
  constexpr int kZUnits = (kMaxCols * 4 + kThreads - 1) / kThreads;   // zero-point uint4s
  // gathering: perm_col uint4s per thread (4 reordered columns each)
  // (gathering needs at least 8 wavefronts: fewer would hold too many registers)
  constexpr int kPermUnits = (kMaxCols * 32 + kThreads - 1) / kThreads;
  static_assert(!kGather || kPermUnits <= 4, "gathering workgroups have at least 8 wavefronts");
  const int lane = threadIdx.x & 63;
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = blk / split, sp = blk - (blk / split) * split;
  const int c0 = sp * kmax;
  const int ncl = min(w.NBc, c0 + kmax) - c0;
  const int64_t rowbase = (int64_t)r * w.NBc + c0;
  const size_t sums_off = m1_sums_offset(kmax);
  const uint32_t zero_off = (uint32_t)m1_zero_offset(kmax);

  // Gathering: the x row, straight into LDS, ahead of the first round trip
  // (so the waits for the bit map below cover it too).
  const int nperm = ncl * 32;  // uint4s of perm_col in the range (c0 == 0)
  const size_t xrow_off = m1_xrow_offset(kmax);
  if constexpr (kGather) {
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      const int idx = t + u * kThreads;
      if (idx < ncl * 16)
        lds_copy16(reinterpret_cast<const uint4*>(x) + idx, (uint32_t)xrow_off + 16 * (idx - lane));
    }
    asm volatile("" ::: "memory");
  }
  // First round trip: bit map and offsets (lane = column).
  const int lc = min(lane, ncl - 1);
  const int blr = w.bits[rowbase + lc];
  const uint32_t ol = w.block_offset[rowbase + lc];
  // Gathering: with them, this thread's perm_col entries (4 per unit; the
  // loads are unconditional, past the end they repeat the last uint4, so
  // every wavefront issues the same count).
  uint4 pc[kGather ? kPermUnits : 1];
  if constexpr (kGather) {
    asm volatile("" ::: "memory");
#pragma unroll
    for (int u = 0; u < kPermUnits; ++u)
      pc[u] = reinterpret_cast<const uint4*>(w.perm_col)[min(t + u * kThreads, nperm - 1)];
  }

  const WaveRuns wr = wave_runs<NW>(lane < ncl ? blr : 0, wave, kWeightCostM1);
  uint32_t off[5];
#pragma unroll
  for (int k = 0; k < 5; ++k)
    off[k] = wr.n[k] > 0 ? __builtin_amdgcn_readlane(ol, __builtin_ctzll(wr.cols[k])) : 0u;

  // Then, copied straight into LDS (no registers; the start-up barrier waits
  // for them), the range's slices of the reordered x, corrections, group
  // sums, scales (16 uint4 per column) and zero points (4 per column),
  // issued just before the first run's code loads so that they travel with
  // them.
  const size_t s_off = m1_scale_offset(kmax);
  const size_t z_off = s_off + 256 * (size_t)ncl;  // the zero points follow the range's scales
  // the bit map and offsets have landed (the plan above used them): an
  // explicit wait here tells the compiler so, and it then has no reason
  // to wait for the copies below when it reuses those registers (gathering:
  // all but the perm_col loads and the x row copies issued after them)
  // Gathering: the perm_col entries, clamped into [0, K) and packed to 16
  // bits (K <= 128 kMaxCols <= 65536), are parked in the x slice area, in
  // the 8 bytes that the same thread later fills with the four reordered
  // values, so that they hold no registers while the ring's loads are in
  // flight.  This waits for their loads, issued with the bit map's (an
  // explicit vmcnt(0), for the reason above: every load so far has landed).
  if constexpr (kGather) {
    __builtin_amdgcn_s_waitcnt(0x0F70);
    const int kk = (int)w.K - 1;
    static_assert(kBlockCols * kMaxCols <= 65536, "16-bit column indices");
#pragma unroll
    for (int u = 0; u < kPermUnits; ++u) {
      const int i = t + u * kThreads;
      const uint2 pk{(uint32_t)clampi((int)pc[u].x, kk) | ((uint32_t)clampi((int)pc[u].y, kk) << 16),
                     (uint32_t)clampi((int)pc[u].z, kk) | ((uint32_t)clampi((int)pc[u].w, kk) << 16)};
      if (i < nperm) *reinterpret_cast<uint2*>(smem + 8 * (size_t)i) = pk;
    }
  } else {
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }
  auto stage16 = [&](const void* g, size_t lds_off, int n, auto Units) __attribute__((always_inline)) {
    constexpr int kU = decltype(Units)::value;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int idx = t + u * kThreads;
      if (idx < n)  // lane i of the wavefront lands 16 i bytes past the wavefront's base
        lds_copy16(reinterpret_cast<const uint4*>(g) + idx, (uint32_t)lds_off + 16 * (idx - lane));
    }
  };
  if constexpr (!kGather) {
    stage16(xg + (int64_t)c0 * kBlockCols, 0, ncl * 16, std::integral_constant<int, kUnits>{});
    stage16(sums_g + c0, sums_off, ncl, std::integral_constant<int, kSumsUnits>{});
  }
  stage16(w.scale + rowbase * kBlockRows, s_off, ncl * 16, std::integral_constant<int, kSUnits>{});
  stage16(w.zero + rowbase * kBlockRows, z_off, ncl * 4, std::integral_constant<int, kZUnits>{});
  asm volatile("" ::: "memory");

  Ctx cx{w.codes, w.block_offset, w.scale, w.zero, rowbase, nullptr, nullptr, 0, kmax, 1,
         (uint32_t)sums_off, 0u, 0u};
  cx.a_lane = (uint32_t)(16 * (lane >> 4));
  cx.zero_off = zero_off;
  cx.s_off = (uint32_t)s_off;
  cx.z_off = (uint32_t)z_off;

  // Start-up: the workgroup barrier runs after the wavefront has issued the
  // loads of its first run's first blocks, so their latency overlaps it.  It
  // waits for this wavefront's copies into LDS (every load but the last
  // `issued`, which are that run's) and for its LDS stores.
  if (t < 64) reinterpret_cast<uint32_t*>(smem + zero_off)[t] = 0u;
  asm volatile("" ::: "memory");
  auto startup = [&](auto Issued) __attribute__((always_inline)) {
    constexpr int n = decltype(Issued)::value;
    static_assert(n < 64, "vmcnt range");
    // s_waitcnt vmcnt(n) expcnt(7) lgkmcnt(0); vmcnt is bits [3:0] and [15:14]
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if constexpr (kGather) {
      // x row in LDS: reorder it into the x slice (xg[j] = x[perm_col[j]])
      // and form the k-step sums.  Thread unit u holds reordered columns
      // 4i .. 4i + 3 (i = t + u kThreads); eight consecutive units make a
      // k-step of 32.  Pairwise tree: (x0 + x1) + (x2 + x3) per unit, then
      // across the eight units by xor distance 1, 2, 4 (the prep kernel's
      // tree over the same pairs).
#pragma unroll
      for (int u = 0; u < kPermUnits; ++u) {
        const int i = t + u * kThreads;
        const uint16_t* xrow = reinterpret_cast<const uint16_t*>(smem + xrow_off);
        const uint2 pk = *reinterpret_cast<const uint2*>(smem + 8 * (size_t)min(i, nperm - 1));
        const uint16_t u0 = xrow[pk.x & 0xFFFFu], u1 = xrow[pk.x >> 16];
        const uint16_t u2 = xrow[pk.y & 0xFFFFu], u3 = xrow[pk.y >> 16];
        float s = (bf16f(u0) + bf16f(u1)) + (bf16f(u2) + bf16f(u3));
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        s += __shfl_xor(s, 4, 64);
        if (i < nperm) {
          *reinterpret_cast<uint2*>(smem + 8 * (size_t)i) =
              uint2{(uint32_t)u0 | ((uint32_t)u1 << 16), (uint32_t)u2 | ((uint32_t)u3 << 16)};
          if ((t & 7) == 0) reinterpret_cast<float*>(smem + sums_off)[i >> 3] = s;
        }
      }
      __syncthreads();
    }
  };
  auto none = [](auto) __attribute__((always_inline)) {};

  // runs of bitwidths 1, 2, 3, 4, 8 in order; the first non-empty one hosts the start-up
  float y1 = 0.f;
  const int kfirst = wr.n[0] > 0 ? 0 : wr.n[1] > 0 ? 1 : wr.n[2] > 0 ? 2 : wr.n[3] > 0 ? 3 : wr.n[4] > 0 ? 4 : 5;
  switch (kfirst) {
    case 0: run_ring<1>(cx, run_base(cx, off[0]), wr.cols[0], wr.n[0], y1, startup); break;
    case 1: run_ring<2>(cx, run_base(cx, off[1]), wr.cols[1], wr.n[1], y1, startup); break;
    case 2: run_ring<3>(cx, run_base(cx, off[2]), wr.cols[2], wr.n[2], y1, startup); break;
    case 3: run_ring<4>(cx, run_base(cx, off[3]), wr.cols[3], wr.n[3], y1, startup); break;
    case 4: run_ring<8>(cx, run_base(cx, off[4]), wr.cols[4], wr.n[4], y1, startup); break;
    default: startup(std::integral_constant<int, 0>{}); break;
  }
  if (kfirst < 1 && wr.n[1] > 0) run_ring<2>(cx, run_base(cx, off[1]), wr.cols[1], wr.n[1], y1, none);
  if (kfirst < 2 && wr.n[2] > 0) run_ring<3>(cx, run_base(cx, off[2]), wr.cols[2], wr.n[2], y1, none);
  if (kfirst < 3 && wr.n[3] > 0) run_ring<4>(cx, run_base(cx, off[3]), wr.cols[3], wr.n[3], y1, none);
  if (kfirst < 4 && wr.n[4] > 0) run_ring<8>(cx, run_base(cx, off[4]), wr.cols[4], wr.n[4], y1, none);

  // reduce the wavefronts in a fixed order and write out
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
  if (wave > 0) red[(wave - 1) * 64 + lane] = y1;
  __syncthreads();
  if (wave != 0) return;
  float v = y1;
#pragma unroll
  for (int k = 0; k < NW - 1; ++k) v += red[k * 64 + lane];
  const int64_t row = (int64_t)r * kBlockRows + lane;
  if (split == 1) {
    y[orig_row(w.perm_row, row, w.N)] = v;
    return;
  }
  // Several splits: the partials are stored and read back with device-scope
  // (relaxed atomic) accesses, which go to the level shared by all XCDs, and
  // the stores are complete before the row's counter (cleared by k_prep_m1)
  // is incremented; the last workgroup of the row to arrive adds the
  // partials in split order, so y is reproducible.  No cache-wide write-back
  // or invalidation is needed.
  __hip_atomic_store(&part[(int64_t)sp * w.N + row], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  unsigned prev = 0;
  if (lane == 0)
    prev = __hip_atomic_fetch_add(&counters[r], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  prev = __shfl(prev, 0, 64);
  if (prev != (unsigned)(split - 1)) return;
  float tot = 0.f;
  for (int k = 0; k < split; ++k)
    tot += __hip_atomic_load(&part[(int64_t)k * w.N + row], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  y[orig_row(w.perm_row, row, w.N)] = tot;
}

template <int NW, bool kGather>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4))) void k_gemv_m1(
    const uint16_t* __restrict__ xg, const float4* __restrict__ sums_g,
    const uint16_t* __restrict__ x, WeightView w, int split, int kmax, float* __restrict__ part,
    float* __restrict__ y, uint32_t* __restrict__ counters) {
  gemv_m1<NW, kGather>(xg, sums_g, x, w, split, kmax, part, y, counters, blockIdx.x);
}

// ---- grouped M == 1 calls: up to kGroupMax matrices per launch ---------------------------
// One decode launch covers all matrices of the group (for example the q, k,
// v projections of a layer, which read the same x), plus one prep launch for
// the jobs with several K ranges; the workgroups of the matrices run side by
// side, so small matrices no longer leave the GPU idle for a launch of their
// own.  Job j owns the workgroups [prep_begin, prep_begin of j + 1) of the
// prep launch (none when it reorders x itself) and [wg_begin, wg_begin of
// j + 1) of the decode launch.
constexpr int kGroupMax = 8;

struct M1Job {
  WeightView w;
  const uint16_t* x;
  uint16_t* xg;
  float4* sums;
  float* part;
  float* y;
  uint32_t* counters;
  int split, kr, ncounters;
  int gather;  // the decode workgroups reorder x themselves (no prep workgroups)
  int prep_begin, wg_begin;
};

struct M1Group {
  M1Job job[kGroupMax];
  int count;
};

// The job owning workgroup `b` (first index of the range), selected with
// static indices only so that the kernel arguments are never copied.
__device__ __forceinline__ int group_job(const M1Group& g, int b, bool prep) {
  int j = 0;
#pragma unroll
  for (int k = 1; k < kGroupMax; ++k)
    if (k < g.count && b >= (prep ? g.job[k].prep_begin : g.job[k].wg_begin)) j = k;
  return j;
}

// Copy of job j (wavefront-uniform) selected field by field with static indices.
__device__ __forceinline__ M1Job pick_job(const M1Group& g, int j) {
  M1Job q = g.job[0];
#pragma unroll
  for (int k = 1; k < kGroupMax; ++k)
    if (k == j) q = g.job[k];
  return q;
}

__global__ __launch_bounds__(256) void k_prep_m1_group(M1Group g) {
  const M1Job q = pick_job(g, group_job(g, blockIdx.x, true));
  prep_m1(q.x, q.w.K, q.w.perm_col, q.xg, q.sums, q.counters, q.ncounters,
          blockIdx.x - q.prep_begin);
}

template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4))) void k_gemv_m1_group(
    M1Group g) {
  const M1Job q = pick_job(g, group_job(g, blockIdx.x, false));
  // the branch is uniform over the workgroup
  if constexpr (NW >= 8) {
    if (q.gather) {
      gemv_m1<NW, true>(nullptr, nullptr, q.x, q.w, q.split, q.kr, q.part, q.y, q.counters,
                        blockIdx.x - q.wg_begin);
      return;
    }
  }
  gemv_m1<NW, false>(q.xg, q.sums, nullptr, q.w, q.split, q.kr, q.part, q.y, q.counters,
                     blockIdx.x - q.wg_begin);
}

// ======================================================================================
// K-split reduction
// ======================================================================================

// Row blockIdx.x of the same sum, one workgroup per row.  kLds: the row is
// permuted through LDS (4 N bytes of dynamic LDS) and written back with
// coalesced stores; otherwise each sum is stored at its original column.
constexpr int kReduceRowThreads = 1024;
constexpr int64_t kReduceRowMaxLdsN = 32768;
template <bool kLds>
__global__ __launch_bounds__(kReduceRowThreads) void k_gemv_reduce_rows(
    const float* __restrict__ part, int split, int M, int64_t N, const int32_t* __restrict__ perm_row,
    float* __restrict__ y) {
  const int64_t m = blockIdx.x;
  const int64_t plane = (int64_t)M * N;
  float* lrow = reinterpret_cast<float*>(smem);
  for (int64_t n = threadIdx.x; n < N; n += kReduceRowThreads) {
    const float* p = part + m * N + n;
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
    if constexpr (kLds)
      lrow[orig_row(perm_row, n, N)] = v;
    else
      y[m * N + orig_row(perm_row, n, N)] = v;
  }
  if constexpr (kLds) {
    __syncthreads();
    for (int64_t n = threadIdx.x; n < N; n += kReduceRowThreads) y[m * N + n] = lrow[n];
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

// Workspace layout of one call: [partials | xg | sums | counters] (M == 1)
// or [partials | gather buffers] (M > 1), each part 256-byte aligned; the
// partials only with several splits.
struct GemvWorkspace {
  float* part;
  void* gather;  // M > 1: the gather kernel's x_r and split group sums
  uint16_t* xg;
  float4* sums;
  uint32_t* counters;
};

constexpr size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

size_t part_bytes(const GemvPlan& p, int64_t M, int64_t N) {
  return p.split > 1 ? align256((size_t)p.split * M * N * 4) : 0;
}

size_t m1_prep_bytes(int64_t N, int64_t K) {
  const size_t nbc = (size_t)(K / kBlockCols), nbr = (size_t)(N / kBlockRows);
  return align256((size_t)K * 2) + align256(nbc * 16) + align256(nbr * 4);
}

GemvWorkspace carve(void* ws, const GemvPlan& p, int64_t M, int64_t N, int64_t K) {
  uint8_t* b = reinterpret_cast<uint8_t*>(ws);
  GemvWorkspace g{};
  g.part = reinterpret_cast<float*>(b);
  b += part_bytes(p, M, N);
  if (M > 1) g.gather = b;
  if (M == 1) {
    const size_t nbc = (size_t)(K / kBlockCols);
    g.xg = reinterpret_cast<uint16_t*>(b);
    b += align256((size_t)K * 2);
    g.sums = reinterpret_cast<float4*>(b);
    b += align256(nbc * 16);
    g.counters = reinterpret_cast<uint32_t*>(b);
  }
  return g;
}

// M == 1 calls without a K split reorder x inside the decode workgroups
// (no prep launch) when the wavefront count allows it; the boundary has
// checked that x and perm_col are 16-byte aligned, as the gathering
// workgroups read them.  MSQ_M1_GATHER=0 turns it off (tuning).
bool m1_gathers(const GemvPlan& p) {
  const char* v = std::getenv("MSQ_M1_GATHER");
  const bool enabled = !(v && *v && std::atoi(v) == 0);
  return enabled && p.split == 1 && p.nw >= 8;
}

size_t m1_launch_lds(const GemvPlan& p, bool gather) {
  return gather ? m1_lds_bytes_gather(p.kr) : p.lds_bytes;
}

template <int NW>
hipError_t launch_m1(const GemvWorkspace& g, const uint16_t* x, bool gather, const WeightView& w,
                     float* y, const GemvPlan& p, hipStream_t stream) {
  const unsigned grid = (unsigned)(w.NBr * p.split);
  if constexpr (NW >= 8) {
    if (gather) {
      hipLaunchKernelGGL((k_gemv_m1<NW, true>), dim3(grid), dim3(NW * 64), m1_launch_lds(p, true),
                         stream, nullptr, nullptr, x, w, p.split, p.kr, g.part, y, g.counters);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((k_gemv_m1<NW, false>), dim3(grid), dim3(NW * 64), m1_launch_lds(p, false),
                     stream, g.xg, g.sums, nullptr, w, p.split, p.kr, g.part, y, g.counters);
  return hipGetLastError();
}

template <int NW, int MT>
hipError_t launch_cfg(const uint16_t* xr, const uint16_t* sxs, int M, const WeightView& w,
                      float* dst, const GemvPlan& p, int direct, hipStream_t stream) {
  const unsigned grid = (unsigned)(w.NBr * p.split);
  hipLaunchKernelGGL((k_gemv<NW, MT>), dim3(grid), dim3(NW * 64), p.lds_bytes, stream, xr, sxs, M,
                     w, p.split, p.kr, p.xs_stride, dst, direct);
  return hipGetLastError();
}

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  return (v && *v) ? std::atoi(v) : dflt;
}

}  // namespace

// Launch shape.  The block columns of a block row are split into `split`
// ranges of at most 64 columns.  M == 1: at most 512 workgroups of 8
// wavefronts (two per CU) and at most 8 splits.  M > 1: about 512
// workgroups.  MSQ_GEMV_SPLIT and MSQ_GEMV_WAVES override the split count
// and, for M == 1, the wavefronts per workgroup (tuning only).
const uint16_t* gemv_reordered_x(void* workspace, const GemvPlan& p, int64_t M, int64_t N) {
  if (M <= 1) return nullptr;
  return reinterpret_cast<const uint16_t*>(reinterpret_cast<uint8_t*>(workspace) +
                                           part_bytes(p, M, N));
}

GemvPlan plan_gemv(int64_t M, int64_t N, int64_t K, int64_t group_rows) {
  GemvPlan p{};
  const int NBr = (int)(N / kBlockRows), NBc = (int)(K / kBlockCols);
  // the split heuristic counts the block rows of every matrix in the launch
  const int rows = group_rows > 0 ? (int)(group_rows / kBlockRows) : NBr;
  p.mt = (int)((M + 15) / 16);
  p.nw = M > 16 ? 4 : 8;
  if (M == 1) {
    const int nw = env_int("MSQ_GEMV_WAVES", 8);
    p.nw = (nw == 4 || nw == 16) ? nw : 8;
  }
  int kr_max = kMaxCols;
  if (M > 1) {
    // LDS per block column: x slice (2 bytes x 128 per row) + one group sum per row
    const size_t per_col = (size_t)M * (kBlockCols * 2 + 4);
    kr_max = (int)((kLdsBudget - 16 * (size_t)M) / per_col);
    if (kr_max > kMaxCols) kr_max = kMaxCols;
    if (kr_max < 1) kr_max = 1;
  }
  int split = env_int("MSQ_GEMV_SPLIT", 0);
  if (split <= 0) {
    if (M == 1) {
      // about one workgroup of 8 wavefronts per CU: more K splits add start-ups
      // and partials faster than they add memory parallelism
      split = 256 / rows;
      if (split > 8) split = 8;
    } else {
      split = (512 + NBr - 1) / NBr;
      // with enough block rows, small M prefers fewer splits (less staging
      // per workgroup and fewer partials): about one split per 4 rows of M
      if (NBr >= 128) split = std::min<int>(split, std::max<int>(1, (int)((M + 3) / 4)));
    }
  }
  if (split > NBc) split = NBc;
  if (split < 1) split = 1;
  int kr = (NBc + split - 1) / split;
  if (kr > kr_max) kr = kr_max;
  split = (NBc + kr - 1) / kr;
  p.split = split;
  p.kr = kr;
  size_t x_bytes;
  if (M == 1) {
    p.xs_stride = kr * kBlockCols;
    x_bytes = m1_lds_bytes(kr);
  } else {
    p.xs_stride = kr * kBlockCols + 8;  // +16 bytes per row against LDS bank conflicts
    x_bytes = (size_t)M * p.xs_stride * 2 + (size_t)M * kr * 4;
  }
  const size_t red_bytes = (size_t)(p.nw - 1) * (size_t)M * kBlockRows * 4;
  p.lds_bytes = x_bytes > red_bytes ? x_bytes : red_bytes;
  p.workspace = part_bytes(p, M, N) + (M == 1 ? m1_prep_bytes(N, K) : gather_workspace_bytes(M, K));
  return p;
}

// Rows of all matrices of a group: the launch the split heuristic fills.
int64_t group_rows(const WeightView* w, int count) {
  int64_t rows = 0;
  for (int i = 0; i < count; ++i) rows += w[i].N;
  return rows;
}

size_t gemv_group_workspace_m1(const WeightView* w, int count) {
  size_t total = 0;
  const int64_t rows = group_rows(w, count);
  for (int i = 0; i < count; ++i) total += align256(plan_gemv(1, w[i].N, w[i].K, rows).workspace);
  return total;
}

hipError_t launch_gemv_group_m1(const uint16_t* const* x, const WeightView* w, float* const* y,
                                int count, void* workspace, hipStream_t stream) {
  if (count < 1 || count > kGroupMax) return hipErrorInvalidValue;
  M1Group g{};
  g.count = count;
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  int prep_total = 0, wg_total = 0, nw = 0;
  size_t lds = 0;
  const int64_t rows = group_rows(w, count);
  for (int i = 0; i < count; ++i) {
    const GemvPlan p = plan_gemv(1, w[i].N, w[i].K, rows);
    if (nw == 0) nw = p.nw;
    if (p.nw != nw) return hipErrorInvalidValue;
    const GemvWorkspace gw = carve(ws, p, 1, w[i].N, w[i].K);
    ws += align256(p.workspace);
    M1Job& q = g.job[i];
    q.w = w[i];
    q.x = x[i];
    q.xg = gw.xg;
    q.sums = gw.sums;
    q.part = gw.part;
    q.y = y[i];
    q.counters = gw.counters;
    q.split = p.split;
    q.kr = p.kr;
    q.ncounters = p.split > 1 ? (int)w[i].NBr : 0;
    q.gather = m1_gathers(p) ? 1 : 0;
    q.prep_begin = prep_total;
    q.wg_begin = wg_total;
    const int64_t nbc = w[i].K / kBlockCols;
    if (!q.gather) prep_total += (int)std::max<int64_t>((nbc + 3) / 4, (q.ncounters + 255) / 256);
    wg_total += (int)(w[i].NBr * p.split);
    lds = std::max(lds, m1_launch_lds(p, q.gather != 0));
  }
  // prep workgroups only for the jobs that do not gather (a job with an
  // empty range shares its begin with the next job, which group_job picks)
  if (prep_total > 0) {
    hipLaunchKernelGGL(k_prep_m1_group, dim3((unsigned)prep_total), dim3(256), 0, stream, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (nw == 4)
    hipLaunchKernelGGL((k_gemv_m1_group<4>), dim3((unsigned)wg_total), dim3(256), lds, stream, g);
  else if (nw == 16)
    hipLaunchKernelGGL((k_gemv_m1_group<16>), dim3((unsigned)wg_total), dim3(1024), lds, stream, g);
  else
    hipLaunchKernelGGL((k_gemv_m1_group<8>), dim3((unsigned)wg_total), dim3(512), lds, stream, g);
  return hipGetLastError();
}

hipError_t launch_gemv(const uint16_t* x, int64_t M, const WeightView& w, float* y,
                       void* workspace, const GemvPlan& p, hipStream_t stream) {
  const int direct = p.split == 1;
  const GemvWorkspace g = carve(workspace, p, M, w.N, w.K);
  float* dst = direct ? y : g.part;
  hipError_t e;
  if (M == 1) {
    const bool gather = m1_gathers(p);
    if (!gather) {
      // x reordered once for all workgroups; the split counters are cleared
      // here, only needed with several splits
      const int64_t nbc = w.K / kBlockCols;
      const int ncounters = p.split > 1 ? (int)w.NBr : 0;
      const int64_t grid = std::max<int64_t>((nbc + 3) / 4, (ncounters + 255) / 256);
      hipLaunchKernelGGL(k_prep_m1, dim3((unsigned)grid), dim3(256), 0, stream, x, w.K, w.perm_col,
                         g.xg, g.sums, g.counters, ncounters);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (p.nw == 4) return launch_m1<4>(g, x, gather, w, y, p, stream);
    if (p.nw == 16) return launch_m1<16>(g, x, gather, w, y, p, stream);
    return launch_m1<8>(g, x, gather, w, y, p, stream);
  } else {
    // x reordered once per call, then staged slice by slice
    e = launch_gather_x(x, M, w, g.gather, stream);
    if (e != hipSuccess) return e;
    const uint16_t* xr = reinterpret_cast<const uint16_t*>(g.gather);
    const uint16_t* sxs = reinterpret_cast<const uint16_t*>(
        reinterpret_cast<const uint8_t*>(g.gather) + align256((size_t)M * w.K * 2));
    if (p.nw == 8) {
      e = launch_cfg<8, 1>(xr, sxs, (int)M, w, dst, p, direct, stream);
    } else {
      switch (p.mt) {
        case 2: e = launch_cfg<4, 2>(xr, sxs, (int)M, w, dst, p, direct, stream); break;
        case 3: e = launch_cfg<4, 3>(xr, sxs, (int)M, w, dst, p, direct, stream); break;
        default: e = launch_cfg<4, 4>(xr, sxs, (int)M, w, dst, p, direct, stream); break;
      }
    }
  }
  if (e != hipSuccess || direct) return e;
  return launch_split_reduce(g.part, p.split, M, w.N, w.perm_row, y, stream);
}

hipError_t launch_split_reduce(const float* part, int split, int64_t M, int64_t N,
                               const int32_t* perm_row, float* y, hipStream_t stream) {
  if (M >= 256) {
    // one workgroup per row (enough rows to fill the GPU): every 64-byte line
    // of the row is completed by one workgroup while it sits in L2
    // (workgroups sharing a row would each leave it partly written, and
    // partial lines reach HBM many times over)
    if (N <= kReduceRowMaxLdsN)
      hipLaunchKernelGGL(k_gemv_reduce_rows<true>, dim3((unsigned)M), dim3(kReduceRowThreads),
                         (size_t)N * 4, stream, part, split, (int)M, N, perm_row, y);
    else
      hipLaunchKernelGGL(k_gemv_reduce_rows<false>, dim3((unsigned)M), dim3(kReduceRowThreads), 0,
                         stream, part, split, (int)M, N, perm_row, y);
    return hipGetLastError();
  }
  const int64_t total = M * N;
  hipLaunchKernelGGL(k_gemv_reduce, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                     part, split, (int)M, N, perm_row, y);
  return hipGetLastError();
}

}  // namespace msq

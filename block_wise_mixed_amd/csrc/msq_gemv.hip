// Decode GEMV for gfx950: y = x . W^T for M <= 64, W dequantized block by
// block from packed format v2 (include/msq.h) in registers.  Memory-bound:
// every byte of the packed codes is read once, with one 16-byte load per
// lane per 1 KiB chunk.
//
// Work split.  A workgroup of NW wavefronts owns one block row r (64 output
// rows) and a range of at most 64 block columns [c0, c0 + ncl) (a K split).
//  1. Every wavefront reads the range's bit map with one lane per column and
//     forms, per bitwidth, a 64-bit mask of the columns holding it (wave
//     ballots).  Walking bitwidths 1, 2, 3, 4, 8 and columns in order gives
//     the blocks in packed order; the wavefronts cut that list into NW pieces
//     of equal cost, so each wavefront gets at most a few runs of
//     same-bitwidth blocks.
//  2. The activations reordered through perm_col (the activation reordering
//     of the "SFMP" abstract) and their per-group sums, used to fold the zero
//     point, come from the gather kernel (k_gemv16: read straight from L2
//     with each block) or, at M == 1, from the workgroup's own reordering of
//     x in LDS (or the prep kernel).
//  3. Each wavefront walks its runs.  Inside a run the bitwidth is a
//     compile-time constant, so the loads of the next blocks are issued while
//     the current block is unpacked and multiplied, with static wait counts
//     (register rings).  Each 16x32 fragment is unpacked into exact bf16
//     operands and fed to v_mfma_f32_16x16x32_bf16 (M padded to a multiple
//     of 16, one product per 16-row m tile), then
//     scale and zero point are folded per row:
//         y[row] += s * (sum_k (bias + q_k) x_k - (bias + z) * sum_k x_k).
//  4. The wavefronts reduce through LDS in a fixed order.  One K split writes
//     y directly (scattered to original rows through perm_row); several
//     splits write fp32 partials that the last workgroup of the block row to
//     finish sums in split order, so results are bitwise reproducible.
//
// Kernels: k_gemv_m1 (M == 1: per-column k-step sums for the bias
// corrections, an unpack that avoids most shifts, scales and zero points
// staged in LDS, 2 to 4 KiB of codes in flight per wavefront; half block
// rows of 32 rows for small launches instead of a K split), k_gemv16
// (2 <= M <= 64, one to four m tiles), their group variants, and the split
// reductions of the prefill GEMM's K ranges (k_gemv_reduce, k_gemv_reduce_rows).
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

// Per-block operands that live in registers while the block is in flight
// (M == 1: the codes; the workgroup stages the scales and zero points of its
// range in LDS at start-up).
template <int B>
struct BlockRegs {
  uint4 ch[B];
};

// Issue the loads of one block: its b chunks at `base` (this lane's 16 bytes
// of the block's first chunk).  The block index passes through an empty asm
// so that the compiler cannot tell two issues of the same block apart (the
// register rings repeat a run's last block past its end): merging such loads
// would tie the ring's register sets together and add waits.
template <int B>
__device__ __forceinline__ void issue_block(const uint8_t* base, int cl, BlockRegs<B>& br) {
  cl = __builtin_amdgcn_readfirstlane(cl);
  asm("" : "+s"(cl));
#pragma unroll
  for (int t = 0; t < B; ++t) br.ch[t] = *reinterpret_cast<const uint4*>(base + 1024 * t);
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

// Piece weights: the relative cost of a block in a wavefront's walk, so
// that the wavefronts of a workgroup finish together.  Each block is one
// dependent round trip of its loads plus its unpack and products, so the
// weights grow more slowly than the bytes: 1- and 2-bit blocks alike, 3-
// and 4-bit 1.5 times those, 8-bit 2.75 times (measured 2-4% faster per
// call than weights proportional to the unpack work, 4 / 4 / 9 / 9 / 17).
constexpr int kWeightCostM1[5] = {4, 4, 6, 6, 11};

// One block: unpack + matrix-core product into acc[mt][rt] (M > 1).
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

// Blocks per register ring of a B-bit run at M == 1: (depth - 1) * B KiB of
// codes stay in flight while one block is consumed.  Thousands of
// wavefronts share HBM, so shallow rings already keep more in flight than it
// needs; deeper ones only lengthen the queues that every workgroup's
// start-up waits in (M == 1 on a 70B layer: 4/2/2/2/2 blocks for 1/2/3/4/8
// bits measured ~6% faster than 8/4/3/3/2).
template <int B>
constexpr int ring_depth() { return B == 1 ? 4 : 2; }

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
// consume(column, registers) uses a block;
// after_issue(integral_constant<loads issued>) runs once after the first D
// blocks are issued.
// Regs: the register set of one block; issue(address, column, regs) issues
// its loads (the address of this lane's 16 bytes of the block's first chunk);
// kIssued: loads per issue.
template <int B, int D, int kIssued, typename Regs, typename Issue, typename Consume,
          typename AfterIssue>
__device__ __forceinline__ void ring_run_t(const uint8_t* codes, const uint8_t* base, uint64_t cols,
                                           int n, Issue&& issue, Consume&& consume,
                                           AfterIssue&& after_issue) {
  constexpr int64_t kStride = 1024 * B;
  Regs rs[D];
  int cs[D];
  const int64_t lane_off = base - codes;  // this lane's offset of the run's first block
  // block bi of the run, or (live false) the stand-in address
  auto slot = [&](bool live, int bi) __attribute__((always_inline)) {
    return codes + ((lane_off + (int64_t)bi * kStride) & -(int64_t)live);
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
    issue(slot(j < n, bi), cs[j], rs[j]);
    asm volatile("" ::: "memory");
  }
  // the first run: the workgroup's start-up, while these loads fly
  after_issue(std::integral_constant<int, D * kIssued>{});
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
      issue(slot(nx < n, bi), cs[j], rs[j]);
      asm volatile("" ::: "memory");
    }
    i0 += D;
  } while (i0 < n);
}

template <int B, int D, typename Consume, typename AfterIssue>
__device__ __forceinline__ void ring_run(const Ctx& cx, const uint8_t* base, uint64_t cols, int n,
                                         Consume&& consume, AfterIssue&& after_issue) {
  ring_run_t<B, D, B, BlockRegs<B>>(
      cx.codes, base, cols, n,
      [&](const uint8_t* addr, int cl, BlockRegs<B>& br) __attribute__((always_inline)) {
        issue_block<B>(addr, cl, br);
      },
      consume, after_issue);
}

// ======================================================================================
// 2 <= M <= 64: A operands straight from the reordered x
// ======================================================================================
//
// The activation gather leaves x_r [M][K] (reordered through perm_col) and
// the fp32 group sums [group][16 MT] in the workspace (MT = M / 16 rounded
// up: the 16-row m tiles), a few hundred KB that stay in L2.  Each block's
// register set holds, besides its b code chunks, the block column's four A
// fragments per m tile (x_r rows 16 mt + (lane & 15), columns
// 32 kt + 8 (lane >> 4) .. +7; rows past M repeat row M - 1 and their
// outputs are never stored), the group sums of rows 16 mt + 4 (lane >> 4)
// .. +3 and the scale and zero point of row `lane`, all issued together one
// ring stage ahead.  Each B fragment is unpacked once for all m tiles.  No
// slice of x is staged in LDS, so a workgroup takes a whole block row (or a
// range of 64 block columns) like the M == 1 kernel and there is no start-up
// barrier; LDS only holds the final sum over the wavefronts, one m tile at a
// time.

template <int B, int MT>
struct RegsX {
  uint4 ch[B];
  uint4 a[MT][4];
  float4 sx[MT];
  float s;
  uint32_t z;
};

template <int MT>
struct CtxX {
  const uint8_t* codes;
  const float* scale;
  const uint8_t* zero;
  int64_t rowbase;         // block index of the range's first column
  const uint16_t* xa[MT];  // this lane's A row of each m tile at the range's first column
  const float* sxa;        // this lane's four group sums (m tile 0) at the range's first column
};

template <int B, int MT>
__device__ __forceinline__ void issue_x(const CtxX<MT>& cx, const uint8_t* base, int cl,
                                        RegsX<B, MT>& br) {
  const int lane = threadIdx.x & 63;
  cl = __builtin_amdgcn_readfirstlane(cl);
  asm("" : "+s"(cl));
  const int64_t blk = cx.rowbase + cl;
#pragma unroll
  for (int t = 0; t < B; ++t) br.ch[t] = *reinterpret_cast<const uint4*>(base + 1024 * t);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const uint16_t* xa = cx.xa[mt] + (int64_t)cl * kBlockCols;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) br.a[mt][kt] = *reinterpret_cast<const uint4*>(xa + 32 * kt);
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    br.sx[mt] = *reinterpret_cast<const float4*>(cx.sxa + (int64_t)cl * 16 * MT + 16 * mt);
  br.s = cx.scale[blk * kBlockRows + lane];
  br.z = cx.zero[blk * kBlockRows + lane];
}

// One block into yacc[mt][rt] (rows 16 mt + 4 (lane >> 4) + i, output
// 16 rt + (lane & 15)):
//   yacc += s * (sum_k (bias + q_k) x_k - (bias + z) * sum_k x_k).
template <int B, int MT>
__device__ __forceinline__ void consume_x(const RegsX<B, MT>& br, f32x4 (&yacc)[MT][4]) {
  const int lane = threadIdx.x & 63;
  bf16x8 A[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) A[mt][kt] = as_bf16x8(br.a[mt][kt]);
  f32x4 acc[MT][4];
  block_product<B, MT>(br.ch, A, acc);
  constexpr float bias = (float)unpack_bias(B);
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int src = 16 * rt + (lane & 15);
    const float s = __shfl(br.s, src, 64);
    const float zz = bias + (float)__shfl((int)br.z, src, 64);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const float sx[4] = {br.sx[mt].x, br.sx[mt].y, br.sx[mt].z, br.sx[mt].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) yacc[mt][rt][i] += s * (acc[mt][rt][i] - zz * sx[i]);
    }
  }
}

// Ring depth of this kernel: two blocks, one for 8-bit blocks (the A
// fragments ride along, so the register sets are larger than at M == 1; two
// workgroups of 8 wavefronts per CU need them within 128 registers).  ONE:
// one block for every bitwidth, for ranges of 64 block columns (eight or more
// blocks per wavefront), where fewer loads in flight measured faster
// (Llama-3-70B linears at M = 16: 4-6%); with four blocks per wavefront two
// measured faster.  Deeper rings were slower at every shape tried.  Several
// m tiles (M > 16): one block (their A fragments and accumulators fill the
// registers).
template <int B, bool ONE, int MT>
constexpr int ring_depth_x() { return (ONE || MT > 1) ? 1 : (B >= 8 ? 1 : 2); }

template <int B, bool ONE, int MT>
__device__ __forceinline__ void run_x(const CtxX<MT>& cx, const uint8_t* base, uint64_t cols,
                                      int n, f32x4 (&yacc)[MT][4]) {
  ring_run_t<B, ring_depth_x<B, ONE, MT>(), B + 5 * MT + 2, RegsX<B, MT>>(
      cx.codes, base, cols, n,
      [&](const uint8_t* addr, int cl, RegsX<B, MT>& br) __attribute__((always_inline)) {
        issue_x<B, MT>(cx, addr, cl, br);
      },
      [&](int, const RegsX<B, MT>& br) __attribute__((always_inline)) {
        consume_x<B, MT>(br, yacc);
      },
      [](auto) __attribute__((always_inline)) {});
}

// Workgroup `blk` (block row blk / split, K range blk % split) of one matrix,
// M in 16 (MT - 1) + 1 .. 16 MT.  One K range: y is written directly.
// Several: the range's partial goes to part[sp][m][n] and the last workgroup
// of the block row to arrive (counters[r], cleared by the gather before this
// launch) adds the partials in split order into y.
template <int NW, bool ONE, int MT>
__device__ __forceinline__ void gemv16(const uint16_t* __restrict__ xr,
                                       const float* __restrict__ sf, int M, const WeightView& w,
                                       int split, int kmax, float* __restrict__ part,
                                       float* __restrict__ y, uint32_t* __restrict__ counters,
                                       int blk) {
  const bool direct = split == 1;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = blk / split, sp = blk - (blk / split) * split;
  const int c0 = sp * kmax;
  const int ncl = min(w.NBc, c0 + kmax) - c0;
  const int64_t rowbase = (int64_t)r * w.NBc + c0;
  // this wavefront's share of the range's blocks, in packed order
  const int lc = min(lane, ncl - 1);
  const int bl = w.bits[rowbase + lc];
  const uint32_t ol = w.block_offset[rowbase + lc];
  const WaveRuns wr = wave_runs<NW>(lane < ncl ? bl : 0, wave, kWeightCostM1);
  CtxX<MT> cx;
  cx.codes = w.codes;
  cx.scale = w.scale;
  cx.zero = w.zero;
  cx.rowbase = rowbase;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int ma = min(16 * mt + (lane & 15), M - 1);
    cx.xa[mt] = xr + (int64_t)ma * w.K + (int64_t)c0 * kBlockCols + 8 * (lane >> 4);
  }
  cx.sxa = sf + (int64_t)c0 * 16 * MT + 4 * (lane >> 4);
  f32x4 yacc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) yacc[mt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint32_t off[5];
#pragma unroll
  for (int k = 0; k < 5; ++k)
    off[k] = wr.n[k] > 0 ? __builtin_amdgcn_readlane(ol, __builtin_ctzll(wr.cols[k])) : 0u;
  auto base = [&](uint32_t o) __attribute__((always_inline)) {
    return w.codes + (int64_t)o * 1024 + 16 * lane;
  };
  if (wr.n[0] > 0) run_x<1, ONE, MT>(cx, base(off[0]), wr.cols[0], wr.n[0], yacc);
  if (wr.n[1] > 0) run_x<2, ONE, MT>(cx, base(off[1]), wr.cols[1], wr.n[1], yacc);
  if (wr.n[2] > 0) run_x<3, ONE, MT>(cx, base(off[2]), wr.cols[2], wr.n[2], yacc);
  if (wr.n[3] > 0) run_x<4, ONE, MT>(cx, base(off[3]), wr.cols[3], wr.n[3], yacc);
  if (wr.n[4] > 0) run_x<8, ONE, MT>(cx, base(off[4]), wr.cols[4], wr.n[4], yacc);

  // sum over the wavefronts in a fixed order and write out, one m tile at a
  // time through the same LDS (NW - 1 planes of min(M, 16) x 64 floats)
  float* red = reinterpret_cast<float*>(smem);
  const int plane = min(M, 16) * kBlockRows;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt > 0) __syncthreads();  // the previous tile's sums are read
    if (wave > 0) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int mr = 4 * (lane >> 4) + i;
          if (16 * mt + mr < M)
            red[(wave - 1) * plane + mr * kBlockRows + 16 * rt + (lane & 15)] = yacc[mt][rt][i];
        }
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int mr = 4 * (lane >> 4) + i;
          const int m = 16 * mt + mr;
          if (m >= M) continue;
          const int n = 16 * rt + (lane & 15);
          float v = yacc[mt][rt][i];
#pragma unroll
          for (int k = 0; k < NW - 1; ++k) v += red[k * plane + mr * kBlockRows + n];
          const int64_t row = (int64_t)r * kBlockRows + n;
          if (direct)
            y[(int64_t)m * w.N + orig_row(w.perm_row, row, w.N)] = v;
          else
            __hip_atomic_store(&part[((int64_t)sp * M + m) * w.N + row], v, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
  }
  if (direct) return;
  // Several K ranges: the partials are stored and read back with device-scope
  // (relaxed atomic) accesses, which go to the level shared by all XCDs, and
  // wavefront 0's stores (the only ones) are complete before it increments
  // the row's counter; the last workgroup of the row adds the partials in
  // split order (the order of the separate reduction kernel), so y is
  // reproducible.  Wavefront 0 has read the LDS sums above, so it may reuse
  // their first word for the verdict.
  int* verdict = reinterpret_cast<int*>(smem);
  if (wave == 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    unsigned prev = 0;
    if (lane == 0)
      prev = __hip_atomic_fetch_add(&counters[r], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __shfl(prev, 0, 64);
    if (lane == 0) *verdict = prev == (unsigned)(split - 1);
  }
  __syncthreads();
  if (*verdict == 0) return;
  const int64_t pstride = (int64_t)M * w.N;  // one split's partials
  for (int e = threadIdx.x; e < M * kBlockRows; e += NW * 64) {
    const int m = e / kBlockRows, n = e - (e / kBlockRows) * kBlockRows;
    const int64_t row = (int64_t)r * kBlockRows + n;
    const float* p = part + (int64_t)m * w.N + row;
    float v = 0.f;
    int k = 0;
    for (; k + 8 <= split; k += 8) {
      float t[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        t[j] = __hip_atomic_load(p + (k + j) * pstride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int j = 0; j < 8; ++j) v += t[j];
    }
    for (; k < split; ++k)
      v += __hip_atomic_load(p + k * pstride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    y[(int64_t)m * w.N + orig_row(w.perm_row, row, w.N)] = v;
  }
}

template <int NW, bool ONE, int MT>
__global__ __launch_bounds__(NW * 64) void k_gemv16(const uint16_t* __restrict__ xr,
                                                    const float* __restrict__ sf, int M,
                                                    WeightView w, int split, int kmax,
                                                    float* __restrict__ part, float* __restrict__ y,
                                                    uint32_t* __restrict__ counters) {
  gemv16<NW, ONE, MT>(xr, sf, M, w, split, kmax, part, y, counters, blockIdx.x);
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
  ring_run<B, ring_depth<B>()>(
      cx, base, cols, n,
      [&](int cl, const BlockRegs<B>& br) __attribute__((always_inline)) {
        consume_m1<B>(cx, cl, br, y1, bias);
      },
      after_issue);
}

// ---- half block rows (M == 1) -------------------------------------------------------------
// For launches with fewer block rows than CUs and one K range, two workgroups
// share a block row, each taking 32 of its 64 rows (row tiles 2h, 2h + 1 of
// half h) over all of K, instead of a K split: no prep launch, no split
// partials or counters.  A half loads only the chunks its row tiles use
// (b = 2: chunk h; b = 4: chunks 2h, 2h + 1; b = 8: chunks 4h .. 4h + 3; the
// 3-bit low plane: chunk h; b = 1 and the 3-bit high plane: their one chunk,
// whose slots 8h .. 8h + 7 are shifted down to 0 .. 7), so that fragment
// F' = 4 rt' + kt (rt' = rt - 2h) sits where half 0's fragment F' sits.
// For b in {2, 4, 8} and the 3-bit low plane the operands are exactly those
// of the whole-row kernel, and so are the sums; for 1-bit blocks and the
// 3-bit high plane, half 1 unpacks with half 0's exponents (a different but
// equally exact bias), so its fp32 sums may round differently.
template <int B>
constexpr int half_chunks() { return B == 1 ? 1 : (B == 2 ? 1 : (B == 8 ? 4 : 2)); }

template <int B>
struct HalfRegs {
  uint4 ch[half_chunks<B>()];
};

// Chunk of the block that register J of half h holds.
template <int B, int J>
__device__ __forceinline__ int half_chunk(int h) {
  if constexpr (B == 1) return 0;
  else if constexpr (B == 2) return h;
  else if constexpr (B == 3) return J == 0 ? h : 2;
  else if constexpr (B == 4) return 2 * h + J;
  else return 4 * h + J;
}

// One block of half h: 8 fragments, kt outer and rt' inner, each row tile's
// k-steps accumulated in the whole-row kernel's order.
template <int B>
__device__ __forceinline__ void block_product_half(const uint4 (&ch)[half_chunks<B>()],
                                                   const bf16x8 (&A)[4], f32x4 (&acc)[2]) {
  auto step = [&](auto Ic) {
    constexpr int I = decltype(Ic)::value;
    constexpr int kt = I / 2, rt = I % 2, F = 4 * rt + kt;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const uint4& c = ch[B == 4 ? F / 4 : (B == 8 ? F / 2 : 0)];
    f32x4 a = mfma_bf16(A[kt], exp_lo<B, F>(c), kt == 0 ? zero : acc[rt]);
    if constexpr (B == 3) a = mfma_bf16(A[kt], exp_hi<3, F>(ch[1]), a);
    if constexpr (B == 8) a = mfma_bf16(A[kt], exp_hi<8, F>(c), a);
    acc[rt] = a;
  };
  [&]<int... Is>(std::integer_sequence<int, Is...>) {
    (step(std::integral_constant<int, Is>{}), ...);
  }(std::make_integer_sequence<int, 8>{});
}

// consume_m1 for half h (hsh = 8 h): rows 32 h + lane for lanes 0 .. 31;
// the scales and zero points of the range are staged as [column][32].
template <int B>
__device__ __forceinline__ void consume_half(const Ctx& cx, int cl, const HalfRegs<B>& br,
                                             uint32_t hsh, float& y1, const float4& bias) {
  const int lane = threadIdx.x & 63;
  uint4 ch[half_chunks<B>()];
#pragma unroll
  for (int j = 0; j < half_chunks<B>(); ++j) ch[j] = br.ch[j];
  if constexpr (B == 1 || B == 3) {
    constexpr int k = B == 1 ? 0 : 1;
    ch[k] = uint4{ch[k].x >> hsh, ch[k].y >> hsh, ch[k].z >> hsh, ch[k].w >> hsh};
  }
  bf16x8 A[4];
  const uint32_t a = (lane & 15) == 0 ? cx.a_lane + ((uint32_t)cl << 8) : cx.zero_off;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
    A[kt] = as_bf16x8(*reinterpret_cast<const uint4*>(smem + a + 64 * kt));
  f32x4 acc[2];
  block_product_half<B>(ch, A, acc);
  const float v = rows_to_lanes(acc[0][0], acc[1][0], 0.f, 0.f);
  const float4 S = *reinterpret_cast<const float4*>(smem + cx.sums_off + ((uint32_t)cl << 4));
  const float corr = bias.x * S.x + bias.y * S.y + bias.z * S.z + bias.w * S.w;
  const float xsum = (S.x + S.y) + (S.z + S.w);
  const uint32_t l32 = (uint32_t)lane & 31u;
  const float sc = *reinterpret_cast<const float*>(smem + cx.s_off + ((uint32_t)cl << 7) + 4 * l32);
  const uint32_t z = smem[cx.z_off + ((uint32_t)cl << 5) + l32];
  y1 += sc * ((v - corr) - (float)z * xsum);
}

// M == 1 run of half h: the same register ring over the half's chunks.
template <int B, typename AfterIssue>
__device__ __forceinline__ void run_ring_half(const Ctx& cx, const uint8_t* base, uint64_t cols,
                                              int n, int h, float& y1, AfterIssue&& after_issue) {
  const int rt = (threadIdx.x & 63) >> 4;  // rt' for lanes 0 .. 31
  auto pick = [rt](auto KTc) __attribute__((always_inline)) {
    constexpr int kt = decltype(KTc)::value;
    return rt == 0 ? exp_bias(B, kt)
                   : (rt == 1 ? exp_bias(B, 4 + kt) : (rt == 2 ? exp_bias(B, 8 + kt) : exp_bias(B, 12 + kt)));
  };
  const float4 bias{pick(std::integral_constant<int, 0>{}), pick(std::integral_constant<int, 1>{}),
                    pick(std::integral_constant<int, 2>{}), pick(std::integral_constant<int, 3>{})};
  const uint32_t hsh = 8u * (uint32_t)h;
  ring_run_t<B, ring_depth<B>(), half_chunks<B>(), HalfRegs<B>>(
      cx.codes, base, cols, n,
      [&](const uint8_t* addr, int, HalfRegs<B>& br) __attribute__((always_inline)) {
        [&]<int... Js>(std::integer_sequence<int, Js...>) {
          ((br.ch[Js] = *reinterpret_cast<const uint4*>(addr + 1024 * half_chunk<B, Js>(h))), ...);
        }(std::make_integer_sequence<int, half_chunks<B>()>{});
      },
      [&](int cl, const HalfRegs<B>& br) __attribute__((always_inline)) {
        consume_half<B>(cx, cl, br, hsh, y1, bias);
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
template <int NW, bool kGather, bool kHalf = false>
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
  static_assert(!kHalf || kGather, "half block rows reorder x themselves (one K range)");
  const int lane = threadIdx.x & 63;
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // kHalf: workgroup blk takes rows 32 h .. 32 h + 31 of block row r (split == 1)
  const int r = kHalf ? blk >> 1 : blk / split, sp = kHalf ? 0 : blk - (blk / split) * split;
  const int h = kHalf ? blk & 1 : 0;
  const int c0 = sp * kmax;
  const int ncl = min(w.NBc, c0 + kmax) - c0;
  const int64_t rowbase = (int64_t)r * w.NBc + c0;
  const size_t sums_off = m1_sums_offset(kmax);
  const uint32_t zero_off = (uint32_t)m1_zero_offset(kmax);

  // Every copy into LDS goes out first, ahead of the bit map: the x row
  // (gathering) or the reordered x slice and its k-step sums (prep), then
  // the range's scales (16 uint4 per column) and zero points (4 per
  // column).  Copies need no registers; loads complete in issue order, so
  // the wait for the bit map below covers them, and the first run's code
  // loads issued after it have no staging queued ahead of them (the
  // start-up barrier then waits for nothing that is still in flight).
  const int nperm = ncl * 32;  // uint4s of perm_col in the range (c0 == 0)
  const size_t xrow_off = m1_xrow_offset(kmax);
  const size_t s_off = m1_scale_offset(kmax);
  // the zero points follow the range's scales ([ncl][64], halves [ncl][32])
  const size_t z_off = s_off + (kHalf ? 128 : 256) * (size_t)ncl;
  auto stage16 = [&](const void* g, size_t lds_off, int n, auto Units) __attribute__((always_inline)) {
    constexpr int kU = decltype(Units)::value;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int idx = t + u * kThreads;
      if (idx < n)  // lane i of the wavefront lands 16 i bytes past the wavefront's base
        lds_copy16(reinterpret_cast<const uint4*>(g) + idx, (uint32_t)lds_off + 16 * (idx - lane));
    }
  };
  if constexpr (kGather) {
    stage16(x, xrow_off, ncl * 16, std::integral_constant<int, kUnits>{});
  } else {
    stage16(xg + (int64_t)c0 * kBlockCols, 0, ncl * 16, std::integral_constant<int, kUnits>{});
    stage16(sums_g + c0, sums_off, ncl, std::integral_constant<int, kSumsUnits>{});
  }
  if constexpr (kHalf) {
    // the half's 32 scales (8 uint4) and zero points (2 uint4) of each column
    auto stage_half = [&](const void* g, size_t lds_off, int per_col, int n, auto Units)
                          __attribute__((always_inline)) {
      constexpr int kU = decltype(Units)::value;
      const uint4* g4 = reinterpret_cast<const uint4*>(g);
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int idx = t + u * kThreads;
        const int c = idx / per_col, part = idx - c * per_col;
        if (idx < n)
          lds_copy16(g4 + (int64_t)c * (2 * per_col) + h * per_col + part,
                     (uint32_t)lds_off + 16 * (idx - lane));
      }
    };
    stage_half(w.scale + rowbase * kBlockRows, s_off, 8, ncl * 8, std::integral_constant<int, kSUnits>{});
    stage_half(w.zero + rowbase * kBlockRows, z_off, 2, ncl * 2, std::integral_constant<int, kZUnits>{});
  } else {
    stage16(w.scale + rowbase * kBlockRows, s_off, ncl * 16, std::integral_constant<int, kSUnits>{});
    stage16(w.zero + rowbase * kBlockRows, z_off, ncl * 4, std::integral_constant<int, kZUnits>{});
  }
  asm volatile("" ::: "memory");
  // Then the bit map and offsets (lane = column).
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

  // Every load so far has landed (an explicit vmcnt(0): the compiler does
  // not see the copies, and with this wait it has no reason to wait for
  // anything when it reuses their registers).
  // Gathering: the perm_col entries, clamped into [0, K) and packed to 16
  // bits (K <= 128 kMaxCols <= 65536), are parked in the x slice area, in
  // the 8 bytes that the same thread later fills with the four reordered
  // values, so that they hold no registers while the ring's loads are in
  // flight.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  if constexpr (kGather) {
    const int kk = (int)w.K - 1;
    static_assert(kBlockCols * kMaxCols <= 65536, "16-bit column indices");
#pragma unroll
    for (int u = 0; u < kPermUnits; ++u) {
      const int i = t + u * kThreads;
      const uint2 pk{(uint32_t)clampi((int)pc[u].x, kk) | ((uint32_t)clampi((int)pc[u].y, kk) << 16),
                     (uint32_t)clampi((int)pc[u].z, kk) | ((uint32_t)clampi((int)pc[u].w, kk) << 16)};
      if (i < nperm) *reinterpret_cast<uint2*>(smem + 8 * (size_t)i) = pk;
    }
  }

  Ctx cx{w.codes, w.block_offset, w.scale, w.zero, rowbase, (uint32_t)sums_off, 0u, 0u};
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
  // run k (bitwidth kSegBits[k]) of this wavefront, whole rows or the half's
  auto run = [&](auto Bc, int k, auto&& after) __attribute__((always_inline)) {
    constexpr int B = decltype(Bc)::value;
    if constexpr (kHalf)
      run_ring_half<B>(cx, run_base(cx, off[k]), wr.cols[k], wr.n[k], h, y1, after);
    else
      run_ring<B>(cx, run_base(cx, off[k]), wr.cols[k], wr.n[k], y1, after);
  };
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  using I8 = std::integral_constant<int, 8>;
  switch (kfirst) {
    case 0: run(I1{}, 0, startup); break;
    case 1: run(I2{}, 1, startup); break;
    case 2: run(I3{}, 2, startup); break;
    case 3: run(I4{}, 3, startup); break;
    case 4: run(I8{}, 4, startup); break;
    default: startup(std::integral_constant<int, 0>{}); break;
  }
  if (kfirst < 1 && wr.n[1] > 0) run(I2{}, 1, none);
  if (kfirst < 2 && wr.n[2] > 0) run(I3{}, 2, none);
  if (kfirst < 3 && wr.n[3] > 0) run(I4{}, 3, none);
  if (kfirst < 4 && wr.n[4] > 0) run(I8{}, 4, none);

  // reduce the wavefronts in a fixed order and write out
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
  if (wave > 0) red[(wave - 1) * 64 + lane] = y1;
  __syncthreads();
  if (wave != 0) return;
  float v = y1;
#pragma unroll
  for (int k = 0; k < NW - 1; ++k) v += red[k * 64 + lane];
  if constexpr (kHalf) {
    if (lane < 32) y[orig_row(w.perm_row, (int64_t)r * kBlockRows + 32 * h + lane, w.N)] = v;
    return;
  }
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

template <int NW, bool kGather, bool kHalf = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4))) void k_gemv_m1(
    const uint16_t* __restrict__ xg, const float4* __restrict__ sums_g,
    const uint16_t* __restrict__ x, WeightView w, int split, int kmax, float* __restrict__ part,
    float* __restrict__ y, uint32_t* __restrict__ counters) {
  gemv_m1<NW, kGather, kHalf>(xg, sums_g, x, w, split, kmax, part, y, counters, blockIdx.x);
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
  int halves;  // two workgroups per block row, 32 rows each (gather, one K range)
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
  if constexpr (NW == 8) {
    if (q.halves) {
      gemv_m1<NW, true, true>(nullptr, nullptr, q.x, q.w, 1, q.kr, q.part, q.y, q.counters,
                              blockIdx.x - q.wg_begin);
      return;
    }
  }
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
  // kU columns per thread and pass, all their partial loads issued before any
  // is added (a pass is one memory round trip however few rows there are)
  constexpr int kU = 4;
  const int64_t m = blockIdx.x;
  const int64_t plane = (int64_t)M * N;
  float* lrow = reinterpret_cast<float*>(smem);
  const float* prow = part + m * N;
  for (int64_t n0 = threadIdx.x; n0 < N; n0 += kU * kReduceRowThreads) {
    float v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = 0.f;
    int sp = 0;
    for (; sp + 4 <= split; sp += 4) {
      float t[kU][4];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t n = min(n0 + u * kReduceRowThreads, N - 1);
#pragma unroll
        for (int k = 0; k < 4; ++k) t[u][k] = prow[(sp + k) * plane + n];
      }
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int k = 0; k < 4; ++k) v[u] += t[u][k];
    }
    for (; sp < split; ++sp) {
      float t[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) t[u] = prow[sp * plane + min(n0 + u * kReduceRowThreads, N - 1)];
#pragma unroll
      for (int u = 0; u < kU; ++u) v[u] += t[u];
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t n = n0 + u * kReduceRowThreads;
      if (n >= N) break;
      if constexpr (kLds)
        lrow[orig_row(perm_row, n, N)] = v[u];
      else
        y[m * N + orig_row(perm_row, n, N)] = v[u];
    }
  }
  if constexpr (kLds) {
    __syncthreads();
    for (int64_t n = threadIdx.x; n < N; n += kReduceRowThreads) y[m * N + n] = lrow[n];
  }
}

// y[m][perm_row[n]] = sum over splits (in order) of partial[sp][m][n], for
// element idx = m N + n.
__device__ __forceinline__ void reduce_elem(const float* __restrict__ part, int split, int M,
                                            int64_t N, const int32_t* __restrict__ perm_row,
                                            float* __restrict__ y, int64_t idx) {
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

// Workgroups of the element-wise reduction: 256 columns each, workgroup b
// taking row m = 8 (j / chunks) + b mod 8 (j = b / 8, chunks = workgroups per
// row).  Consecutive workgroup ids go to the XCDs in turn, so every
// workgroup of a row runs on one XCD and the row's scattered stores meet in
// one L2 (8B gate_proj at M = 64: 41.4 -> 39.2 us per call).
__host__ __device__ inline int64_t reduce_workgroups(int64_t M, int64_t N) {
  return 8 * ((M + 7) / 8) * ((N + 255) / 256);
}
__device__ __forceinline__ void reduce_wg(const float* __restrict__ part, int split, int M,
                                          int64_t N, const int32_t* __restrict__ perm_row,
                                          float* __restrict__ y, int64_t b) {
  const int64_t chunks = (N + 255) / 256;
  const int64_t j = b >> 3;
  const int64_t m = 8 * (j / chunks) + (b & 7);
  const int64_t n = (j - (j / chunks) * chunks) * 256 + threadIdx.x;
  if (m >= M || n >= N) return;
  reduce_elem(part, split, M, N, perm_row, y, m * N + n);
}

__global__ __launch_bounds__(256) void k_gemv_reduce(const float* __restrict__ part, int split,
                                                     int M, int64_t N,
                                                     const int32_t* __restrict__ perm_row,
                                                     float* __restrict__ y) {
  reduce_wg(part, split, M, N, perm_row, y, blockIdx.x);
}

// ---- grouped calls at 2 <= M <= 32 ---------------------------------------------------
// One gather launch (every matrix's x reordered, with fp32 group sums; the
// split counters cleared) and one decode launch whose workgroups run all
// matrices side by side (matrices with several K ranges reduce them in the
// decode's last arriving workgroups).  Job j owns the workgroups [wg_begin,
// wg_begin of j + 1) of the decode launch.
struct SmallJob {
  WeightView w;
  const uint16_t* xr;  // reordered x [M][K] in the job's workspace
  const float* sf;     // its fp32 group sums
  float* part;         // fp32 partials [split][M][N] (split > 1)
  float* y;
  uint32_t* counters;  // split counters, one per block row (split > 1)
  int split, kr, one;  // one: ranges of 64 block columns (one-block rings)
  int wg_begin;
};

struct SmallGroup {
  SmallJob job[kGroupMax];
  int count;
  int M;
};

// Copy of the job owning workgroup b of the decode launch.
__device__ __forceinline__ SmallJob pick_small_job(const SmallGroup& g, int b) {
  SmallJob q = g.job[0];
#pragma unroll
  for (int k = 1; k < kGroupMax; ++k)
    if (k < g.count && b >= g.job[k].wg_begin) q = g.job[k];
  return q;
}

template <int MT>
__global__ __launch_bounds__(512) void k_gemv16_group(SmallGroup g) {
  const SmallJob q = pick_small_job(g, blockIdx.x);
  const int b = blockIdx.x - q.wg_begin;
  if constexpr (MT == 1) {
    // the branch is uniform over the workgroup
    if (q.one)
      gemv16<8, true, 1>(q.xr, q.sf, g.M, q.w, q.split, q.kr, q.part, q.y, q.counters, b);
    else
      gemv16<8, false, 1>(q.xr, q.sf, g.M, q.w, q.split, q.kr, q.part, q.y, q.counters, b);
  } else {
    gemv16<8, true, MT>(q.xr, q.sf, g.M, q.w, q.split, q.kr, q.part, q.y, q.counters, b);
  }
}

// Workspace layout of one call: [partials | xg | sums | counters] (M == 1)
// or [partials | gather buffers | counters] (M > 1), each part 256-byte
// aligned; the partials (and, at M > 1, the counters) only with several
// splits.
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
  if (M > 1) {
    g.gather = b;
    b += align256(gather_workspace_bytes(M, K));
    if (p.split > 1) g.counters = reinterpret_cast<uint32_t*>(b);
  }
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

size_t m1_launch_lds(const GemvPlan& p, bool gather) {
  return gather ? m1_lds_bytes_gather(p.kr) : p.lds_bytes;
}

template <int NW>
hipError_t launch_m1(const GemvWorkspace& g, const uint16_t* x, bool gather, const WeightView& w,
                     float* y, const GemvPlan& p, hipStream_t stream) {
  const unsigned grid = (unsigned)(w.NBr * p.split);
  if constexpr (NW == 8) {
    if (p.halves) {
      hipLaunchKernelGGL((k_gemv_m1<8, true, true>), dim3(2 * (unsigned)w.NBr), dim3(512),
                         m1_launch_lds(p, true), stream, nullptr, nullptr, x, w, 1, p.kr, g.part, y,
                         g.counters);
      return hipGetLastError();
    }
  }
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

}  // namespace

// Launch shape.  The block columns of a block row are split into `split`
// ranges of at most 64 columns.  M == 1: at most 512 workgroups of 8
// wavefronts (two per CU) and at most 8 splits.  M > 1: about 512
// workgroups.  opt.gemv_split and opt.gemv_waves override the split count
// and, for M == 1, the wavefronts per workgroup.
const uint16_t* gemv_reordered_x(void* workspace, const GemvPlan& p, int64_t M, int64_t N) {
  if (M <= 1) return nullptr;
  return reinterpret_cast<const uint16_t*>(reinterpret_cast<uint8_t*>(workspace) +
                                           part_bytes(p, M, N));
}

GemvPlan plan_gemv(int64_t M, int64_t N, int64_t K, const Options& opt, int64_t group_rows) {
  GemvPlan p{};
  const int NBr = (int)(N / kBlockRows), NBc = (int)(K / kBlockCols);
  // the split heuristic counts the block rows of every matrix in the launch
  const int rows = group_rows > 0 ? (int)(group_rows / kBlockRows) : NBr;
  p.nw = 8;
  if (M == 1 && (opt.gemv_waves == 4 || opt.gemv_waves == 16)) p.nw = opt.gemv_waves;
  int split = opt.gemv_split;
  if (split <= 0) {
    // about one workgroup of 8 wavefronts per CU: more K splits add start-ups
    // and partials faster than they add memory parallelism
    split = 256 / rows;
    if (split > 8) split = 8;
  }
  // M == 1, all launch choices automatic, at most 64 block columns, and a K
  // split wanted (at most 128 block rows in the launch): two workgroups per
  // block row (32 rows each, all of K) instead, so that no prep launch runs.
  // (With 129 .. 255 block rows whole rows in one K range measured faster:
  // halves double the x staging per row for little more parallelism.)
  p.halves = M == 1 && opt.gemv_split <= 0 && opt.gemv_waves == 0 && !opt.m1_prep && split > 1 &&
                     NBc <= kMaxCols
                 ? 1
                 : 0;
  if (p.halves) split = 1;
  if (split > NBc) split = NBc;
  if (split < 1) split = 1;
  int kr = (NBc + split - 1) / split;
  if (kr > kMaxCols) kr = kMaxCols;
  split = (NBc + kr - 1) / kr;
  // ranges of equal width (224 block columns in 4 ranges: 56 each, not
  // 64, 64, 64, 32, whose short range leaves its workgroups idle early)
  kr = (NBc + split - 1) / split;
  p.split = split;
  p.kr = kr;
  // M == 1 with one K range reorders x inside the decode workgroups (no prep
  // launch) when the wavefront count allows it; the boundary has checked
  // that x and perm_col are 16-byte aligned, as those workgroups read them.
  p.gather = M == 1 && split == 1 && p.nw >= 8 && !opt.m1_prep ? 1 : 0;
  // M == 1: the range's staging; the sum over the wavefronts (k_gemv16: one
  // m tile of at most 16 rows at a time)
  const size_t x_bytes = M == 1 ? m1_lds_bytes(kr) : 0;
  const size_t red_bytes = (size_t)(p.nw - 1) * (size_t)std::min<int64_t>(M, 16) * kBlockRows * 4;
  p.lds_bytes = x_bytes > red_bytes ? x_bytes : red_bytes;
  p.workspace = part_bytes(p, M, N) +
                (M == 1 ? m1_prep_bytes(N, K)
                        : align256(gather_workspace_bytes(M, K)) +
                              (split > 1 ? align256((size_t)(N / kBlockRows) * 4) : 0));
  return p;
}

// Rows of all matrices of a group: the launch the split heuristic fills.
int64_t group_rows(const WeightView* w, int count) {
  int64_t rows = 0;
  for (int i = 0; i < count; ++i) rows += w[i].N;
  return rows;
}

size_t gemv_group_workspace_m1(const WeightView* w, int count, const Options& opt) {
  size_t total = 0;
  const int64_t rows = group_rows(w, count);
  for (int i = 0; i < count; ++i) total += align256(plan_gemv(1, w[i].N, w[i].K, opt, rows).workspace);
  return total;
}

hipError_t launch_gemv_group_m1(const uint16_t* const* x, const WeightView* w, float* const* y,
                                int count, void* workspace, const Options& opt,
                                hipStream_t stream) {
  if (count < 1 || count > kGroupMax) return hipErrorInvalidValue;
  M1Group g{};
  g.count = count;
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  int prep_total = 0, wg_total = 0, nw = 0;
  size_t lds = 0;
  const int64_t rows = group_rows(w, count);
  for (int i = 0; i < count; ++i) {
    const GemvPlan p = plan_gemv(1, w[i].N, w[i].K, opt, rows);
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
    q.gather = p.gather;
    q.halves = p.halves;
    q.prep_begin = prep_total;
    q.wg_begin = wg_total;
    const int64_t nbc = w[i].K / kBlockCols;
    if (!q.gather) prep_total += (int)std::max<int64_t>((nbc + 3) / 4, (q.ncounters + 255) / 256);
    wg_total += (int)(w[i].NBr * (p.halves ? 2 : p.split));
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

size_t gemv_group_workspace_small(int64_t M, const WeightView* w, int count, const Options& opt) {
  size_t total = 0;
  const int64_t rows = group_rows(w, count);
  for (int i = 0; i < count; ++i) total += align256(plan_gemv(M, w[i].N, w[i].K, opt, rows).workspace);
  return total;
}

hipError_t launch_gemv_group_small(const uint16_t* const* x, int64_t M, const WeightView* w,
                                   float* const* y, int count, void* workspace, const Options& opt,
                                   hipStream_t stream) {
  if (count < 1 || count > kGroupMax || M < 2 || M > kGemvGroupMaxSmallM) return hipErrorInvalidValue;
  SmallGroup g{};
  g.count = count;
  g.M = (int)M;
  void* gather_ws[kGroupMax];
  uint32_t* counters[kGroupMax];
  int ncounters[kGroupMax];
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  int wg_total = 0;
  size_t lds = 0;
  const int64_t rows = group_rows(w, count);
  for (int i = 0; i < count; ++i) {
    const GemvPlan p = plan_gemv(M, w[i].N, w[i].K, opt, rows);
    const GemvWorkspace gw = carve(ws, p, M, w[i].N, w[i].K);
    ws += align256(p.workspace);
    gather_ws[i] = gw.gather;
    counters[i] = gw.counters;
    ncounters[i] = p.split > 1 ? (int)w[i].NBr : 0;
    SmallJob& q = g.job[i];
    q.w = w[i];
    q.xr = reinterpret_cast<const uint16_t*>(gw.gather);
    q.sf = gather_sums_f32(gw.gather, M, w[i].K);
    q.part = gw.part;
    q.y = y[i];
    q.counters = gw.counters;
    q.split = p.split;
    q.kr = p.kr;
    q.one = p.kr >= kMaxCols ? 1 : 0;
    q.wg_begin = wg_total;
    wg_total += (int)(w[i].NBr * p.split);
    lds = std::max(lds, p.lds_bytes);
  }
  hipError_t e = launch_gather_x_group(x, M, w, gather_ws, counters, ncounters, count, stream);
  if (e != hipSuccess) return e;
  if (M <= 16)
    hipLaunchKernelGGL(k_gemv16_group<1>, dim3((unsigned)wg_total), dim3(512), lds, stream, g);
  else
    hipLaunchKernelGGL(k_gemv16_group<2>, dim3((unsigned)wg_total), dim3(512), lds, stream, g);
  e = hipGetLastError();
  // the decode kernel leaves 16-bit blocks to one more pass per matrix, as
  // in the single call
  for (int i = 0; i < count && e == hipSuccess; ++i)
    if (w[i].has16) e = launch_tile16(x[i], g.job[i].xr, M, w[i], y[i], stream);
  return e;
}

hipError_t launch_gemv(const uint16_t* x, int64_t M, const WeightView& w, float* y,
                       void* workspace, const GemvPlan& p, hipStream_t stream) {
  const int direct = p.split == 1;
  const GemvWorkspace g = carve(workspace, p, M, w.N, w.K);
  hipError_t e;
  if (M == 1) {
    const bool gather = p.gather != 0;
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
  }
  // x reordered once per call with fp32 group sums (and the split counters
  // cleared); k_gemv16 reads its A operands from it directly and, with
  // several K ranges, reduces them in its last arriving workgroups
  e = launch_gather_x(x, M, w, g.gather, stream, true, g.counters, direct ? 0 : (int)w.NBr);
  if (e != hipSuccess) return e;
  const uint16_t* xr = reinterpret_cast<const uint16_t*>(g.gather);
  const float* sf = gather_sums_f32(g.gather, M, w.K);
  const dim3 grid((unsigned)(w.NBr * p.split));
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(512), p.lds_bytes, stream, xr, sf, (int)M, w, p.split,
                       p.kr, g.part, y, g.counters);
  };
  if (M > 48) go(k_gemv16<8, true, 4>);
  else if (M > 32) go(k_gemv16<8, true, 3>);
  else if (M > 16) go(k_gemv16<8, true, 2>);
  else if (p.kr >= kMaxCols) go(k_gemv16<8, true, 1>);
  else go(k_gemv16<8, false, 1>);
  return hipGetLastError();
}

hipError_t launch_split_reduce(const float* part, int split, int64_t M, int64_t N,
                               const int32_t* perm_row, float* y, hipStream_t stream) {
  if (M >= 128) {
    // one workgroup per row: every 64-byte line of the row is completed by
    // one workgroup while it sits in L2 (workgroups sharing a row would each
    // leave it partly written, and partial lines reach HBM many times over);
    // below 128 rows too few workgroups for the GPU (measured slower at
    // M = 17 .. 64, faster at 128 and 200)
    if (N <= kReduceRowMaxLdsN)
      hipLaunchKernelGGL(k_gemv_reduce_rows<true>, dim3((unsigned)M), dim3(kReduceRowThreads),
                         (size_t)N * 4, stream, part, split, (int)M, N, perm_row, y);
    else
      hipLaunchKernelGGL(k_gemv_reduce_rows<false>, dim3((unsigned)M), dim3(kReduceRowThreads), 0,
                         stream, part, split, (int)M, N, perm_row, y);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_gemv_reduce, dim3((unsigned)reduce_workgroups(M, N)), dim3(256), 0, stream,
                     part, split, (int)M, N, perm_row, y);
  return hipGetLastError();
}

}  // namespace msq

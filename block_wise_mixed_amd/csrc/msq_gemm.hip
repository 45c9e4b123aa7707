// Prefill GEMM for gfx950: y = x . W^T for any M (the automatic choice above
// M = 16), W dequantized on the fly from packed format v2 (include/msq.h) and
// multiplied on the bf16 matrix cores.
//
// Two kernels:
//   k_gather_x : x_r[m][j] = x[m][perm_col[j]] (bf16) and the per-group sums
//                sum_j x_r[m][j] over each 128-column group (fp32), written to
//                the workspace once per call (the activation reordering of the
//                "SFMP" abstract).
//   k_gemm     : workgroup tile 128 (M) x 128 (N = two block rows), four
//                wavefronts of 64 x 64, the next K group's copies in flight
//                while the current one is multiplied; details above the kernel.
//
// Keeping the matrix-core operands exact integers and applying the fp32 scale
// per (row, group) keeps y within fp32 accumulation error of the exact
// product; rounding s * (q - z) to bf16 first would not.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cstdlib>
#include <utility>

#include "msq_dequant.h"
#include "msq_internal.h"

namespace msq {
namespace {

// Dynamic LDS of k_gather_x.
extern __shared__ __align__(16) unsigned char smem[];

__device__ __forceinline__ float bf16f(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

// ---- activation gather -----------------------------------------------------------------
//
// One workgroup per row m of x: the row is staged in LDS with coalesced
// 16-byte loads (when it fits), then every thread gathers chunks of 8
// reordered columns x_r[m][8q .. 8q+7] = x[m][perm_col[8q ..]] from LDS and
// stores them contiguously; 16 consecutive chunks are one 128-column group,
// summed with shuffles.  Each group sum S is stored as three bf16 terms
// S = t0 + t1 + t2 (t0 = bf16(S), t1 = bf16(S - t0), t2 = bf16(S - t0 - t1),
// exact to fp32 precision) in planes sxs[p][m][0 .. Gp), Gp = G rounded up
// to a multiple of 32, zero past G: the A operand of the correction product
// at the end of k_gemm.
constexpr int kGatherThreads = 256;
constexpr size_t kGatherMaxLds = 64 * 1024;

__device__ __forceinline__ uint16_t bf16_rn(float v) {
  f32x2v f = {v, 0.f};
  bf16x2v h = __builtin_convertvector(f, bf16x2v);
  return (uint16_t)__builtin_bit_cast(uint32_t, h);
}


// Chunks qs .. qe - 1 (whole groups) of row m of one matrix's gather.  The
// x row is copied into LDS with direct-to-LDS loads (when staged), and the
// perm_col loads of kBatch passes are issued before any of them is used.
// sf (optional): the group sums again as fp32, [group][Mpad] (the decode
// kernel's layout: one 16-byte load gives a lane its four rows).
__device__ __forceinline__ void gather_row(const uint16_t* __restrict__ x, int64_t K, int64_t M,
                                           const int32_t* __restrict__ perm_col,
                                           uint16_t* __restrict__ xr, uint16_t* __restrict__ sxs,
                                           float* __restrict__ sf, int64_t Mpad, int staged,
                                           int64_t m, int64_t qs, int64_t qe) {
  constexpr int kBatch = 4;
  const int lane = threadIdx.x & 63;
  const int64_t chunks = K / 8;
  const int64_t Gp = padded_groups(K / kBlockCols);
  const uint16_t* xrow = x + m * K;
  uint16_t* srow = reinterpret_cast<uint16_t*>(smem);
  // perm_col entries of kBatch passes (clamped into the row's chunks)
  int4 pa[kBatch], pb[kBatch];
  auto load_perm = [&](int64_t q0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t q = min(q0 + u * kGatherThreads + threadIdx.x, chunks - 1);
      const int4* pc = reinterpret_cast<const int4*>(perm_col + 8 * q);
      pa[u] = pc[0];
      pb[u] = pc[1];
    }
  };
  // the first passes' perm_col loads fly together with the row's copies
  load_perm(qs);
  if (staged) {
    const uint4* src = reinterpret_cast<const uint4*>(xrow);
    for (int64_t i = threadIdx.x; i < chunks; i += kGatherThreads)  // lane l lands at base + 16 l
      __builtin_amdgcn_global_load_lds(src + i, (lds_void*)(smem + 16 * (i - lane)), 16, 0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  const uint16_t* from = staged ? srow : xrow;
  const int kk = (int)K - 1;
  const int64_t plane = M * Gp;
  for (int64_t q0 = qs; q0 < qe; q0 += kBatch * kGatherThreads) {
    if (q0 != qs) load_perm(q0);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t q = q0 + u * kGatherThreads + threadIdx.x;
      if (q0 + u * kGatherThreads >= qe) break;  // uniform
      float part = 0.f;
      if (q < chunks) {
        const int4 p0 = pa[u], p1 = pb[u];
        const uint16_t u0 = from[min(max(p0.x, 0), kk)], u1 = from[min(max(p0.y, 0), kk)];
        const uint16_t u2 = from[min(max(p0.z, 0), kk)], u3 = from[min(max(p0.w, 0), kk)];
        const uint16_t u4 = from[min(max(p1.x, 0), kk)], u5 = from[min(max(p1.y, 0), kk)];
        const uint16_t u6 = from[min(max(p1.z, 0), kk)], u7 = from[min(max(p1.w, 0), kk)];
        uint4 v;
        v.x = (uint32_t)u0 | ((uint32_t)u1 << 16);
        v.y = (uint32_t)u2 | ((uint32_t)u3 << 16);
        v.z = (uint32_t)u4 | ((uint32_t)u5 << 16);
        v.w = (uint32_t)u6 | ((uint32_t)u7 << 16);
        reinterpret_cast<uint4*>(xr + m * K)[q] = v;
        part = ((bf16f(u0) + bf16f(u1)) + (bf16f(u2) + bf16f(u3))) +
               ((bf16f(u4) + bf16f(u5)) + (bf16f(u6) + bf16f(u7)));
      }
      // a group is 16 consecutive chunks, i.e. 16 consecutive threads
#pragma unroll
      for (int d = 1; d < 16; d <<= 1) part += __shfl_xor(part, d, 64);
      if (q < qe && (q & 15) == 0) {
        const uint16_t t0 = bf16_rn(part);
        const float r1 = part - bf16f(t0);
        const uint16_t t1 = bf16_rn(r1);
        const uint16_t t2 = bf16_rn(r1 - bf16f(t1));
        uint16_t* dst = sxs + m * Gp + q / 16;
        dst[0] = t0;
        dst[plane] = t1;
        dst[2 * plane] = t2;
        if (sf) sf[(q / 16) * Mpad + m] = part;
      }
    }
  }
}

// The decode's K-split counters of the call (ncounters of them, zero when
// the decode kernel has one K range) cleared by the workgroups of the gather
// that runs before it, b-th of nb workgroups.
__device__ __forceinline__ void clear_counters(uint32_t* __restrict__ counters, int ncounters,
                                               int64_t b, int64_t nb) {
  for (int64_t i = b * kGatherThreads + threadIdx.x; i < ncounters; i += nb * kGatherThreads)
    counters[i] = 0u;
}

// Row blockIdx.x, chunk slice blockIdx.y of gridDim.y (whole groups).
__global__ __launch_bounds__(kGatherThreads) void k_gather_x(const uint16_t* __restrict__ x,
                                                             int64_t K, int64_t M,
                                                             const int32_t* __restrict__ perm_col,
                                                             uint16_t* __restrict__ xr,
                                                             uint16_t* __restrict__ sxs,
                                                             float* __restrict__ sf, int64_t Mpad,
                                                             int staged,
                                                             uint32_t* __restrict__ counters,
                                                             int ncounters) {
  clear_counters(counters, ncounters, (int64_t)blockIdx.y * gridDim.x + blockIdx.x,
                 (int64_t)gridDim.x * gridDim.y);
  const int64_t Gp = padded_groups(K / kBlockCols);
  const int64_t per = (Gp + gridDim.y - 1) / gridDim.y * 16;
  const int64_t qs = (int64_t)blockIdx.y * per;
  gather_row(x, K, M, perm_col, xr, sxs, sf, Mpad, staged, blockIdx.x, qs, min(qs + per, Gp * 16));
}

// ---- GEMM ------------------------------------------------------------------------------
//
// Workgroup tile: kBM = 128 rows of x_r x kBR = 2 block rows (64 outputs
// each); four wavefronts (wm, wn) = (wave & 1, wave >> 1), each 64 rows x one
// block row.  LDS holds ONE x_r tile and two code buffers (69 KiB), so two
// workgroups share a CU and one's barrier waits and fragment-read bursts
// overlap the other's products.  Per 128-wide K group c:
//   - every wavefront reads its 16 A fragments (4 k-steps x 4 m tiles) of
//     group c from the x_r tile into registers; workgroup barrier;
//   - the next group's x_r tile (kBM x 128 bf16) goes into that same buffer
//     and the workgroup's kBR blocks of codes into the other code buffer, by
//     the direct-to-LDS loads (global_load_lds_dwordx4), and each wavefront
//     loads its block's next scales;
//   - row tile by row tile, the wavefront reads the code chunks that tile
//     needs, unpacks its 4 B fragments to exact bf16 (128 + q; 3-bit: both
//     planes merged into one operand; 8-bit: q itself, converted through
//     fp32), issues 16 v_mfma_f32_16x16x32_bf16 into a group accumulator
//     and folds it, acc += s_n * acc_g, while the next row tile's products
//     run;
//   - wait for its own copies, one barrier.
// acc_g carries the unpack bias and the zero point: acc_g = sum_k (bias +
// q_k) x_k = sum_k (q_k - z) x_k + (bias + z) S_c with S_c the group's sum
// of x_r.  The term sum_c s_c (bias + z_c) S_c of every output is removed at
// the end by one more matrix product over the groups (see below), so the
// fold is a single FMA per output and group.
// The two code buffers are distinct LDS objects and the loop is unrolled by
// two, so the compiler sees that the copies in flight never alias what the
// products read and adds no wait for them before those reads.  The x_r tile
// is stored without padding, 16-byte chunk p of row r holding column chunk
// p ^ (r & 15) (the direct-to-LDS copies write each 1 KiB contiguously; the
// swizzle keeps the fragment reads free of bank conflicts).  0-bit blocks
// skip the copies and the products.  y is scattered to original rows
// through perm_row.
constexpr int kBM = 128;
constexpr int kBR = 2;                 // block rows per workgroup
constexpr int kWaves = 2 * kBR;
constexpr int kThreads = kWaves * 64;
constexpr int kTabG = 512;  // groups whose bit map and offsets are staged in LDS

// Bias of the unpacked operands: 128 + q for b <= 4 (3 bits: both planes in
// one operand), q itself for b = 8.
__host__ __device__ constexpr float gemm_bias(int b) { return b == 8 ? 0.f : 128.f; }

// One stage of the pipeline in LDS.
struct Stage {
  uint4* a;      // x_r tile [kBM][16 chunks], swizzled
  uint4* codes;  // [kBR][CH chunks][64 lanes]; CH = 8, or 16 when 16-bit blocks occur
};

// Chunk of a B-bit block holding (the low plane of) fragment F.
template <int B, int F>
__host__ __device__ constexpr int lo_chunk() {
  return B == 1 ? 0 : (B == 2 || B == 3 ? F / 8 : (B == 4 ? F / 4 : F / 2));
}

// Unpacked B operand of fragment F from its chunk c (3 bits: low plane chunk
// c and high plane chunk c2, one operand; 8 bits: the codes themselves,
// converted exactly through fp32, since every q <= 255 is a bf16 integer: one
// matrix instruction per fragment).
template <int B, int F>
__device__ __forceinline__ bf16x8 b_lo(const uint4& c, const uint4& c2) {
  if constexpr (B == 1) return unpack_magic<1, F>(c);
  else if constexpr (B == 2) return unpack_magic<2, 2 * (F % 8)>(c);
  else if constexpr (B == 3) return unpack3_magic<F>(c, c2);
  else if constexpr (B == 4) return unpack_magic<4, 4 * (F % 4)>(c);
  else return unpack_u8<F % 2>(c);
}

// One group of this wavefront's B-bit block (block row q of the workgroup,
// scales sc of rows 16 rt + (lane & 15)), row tile by row tile: the 16 A
// fragments (4 k-steps x 4 m tiles) are read from LDS once; per row tile rt
// the code chunks it needs are read, its 4 B fragments unpacked, 16 (8 bits:
// two planes, 32) matrix instructions accumulate acc_g, and the fold
// acc += s_n * acc_g is issued while the next row tile's products run (one
// basic block, so the scheduler interleaves them).  apk[kt] = this lane's
// byte offset of its A fragment (m tile 0) for k-step kt; m tile mt is 4096
// bytes further.
__device__ __forceinline__ void read_a(const Stage& st, const uint32_t (&apk)[4],
                                       bf16x8 (&A)[4][4]) {
  const unsigned char* abase = reinterpret_cast<const unsigned char*>(st.a);
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      A[kt][mt] = as_bf16x8(*reinterpret_cast<const uint4*>(abase + apk[kt] + 4096 * mt));
}

// 16-bit block: chunk F is the B operand of fragment F as it is (bf16
// weights, no unpack, no scale), so the products go straight into acc.
// Row tiles RT0 .. RT0 + NRT - 1 of the block (acc[mt][rt - RT0]).
template <int CH, int RT0, int NRT>
__device__ __forceinline__ void group_mfma16(const Stage& st, int q, const bf16x8 (&A)[4][4],
                                             f32x4 (&acc)[4][NRT]) {
  static_assert(CH == 16, "16-bit blocks need 16 chunks per block in LDS");
  const uint4* cb = st.codes + q * CH * 64 + (threadIdx.x & 63);
#pragma unroll
  for (int j = 0; j < NRT; ++j)
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const bf16x8 bop = as_bf16x8(cb[64 * (4 * (RT0 + j) + kt)]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt][j] = mfma_bf16(A[kt][mt], bop, acc[mt][j]);
    }
}

template <int B, int CH, int RT0, int NRT>
__device__ __forceinline__ void group_mfma(const Stage& st, int q, const bf16x8 (&A)[4][4],
                                           const float (&sc)[NRT], f32x4 (&acc)[4][NRT]) {
  const int lane = threadIdx.x & 63;
  const uint4* cb = st.codes + q * CH * 64 + lane;
  auto rstep = [&](auto RTc) __attribute__((always_inline)) {
    constexpr int rt = decltype(RTc)::value;
    constexpr int k0 = lo_chunk<B, 4 * rt>(), k1 = lo_chunk<B, 4 * rt + 3>();
    const uint4 c0 = cb[64 * k0];
    const uint4 c1 = k1 == k0 ? c0 : cb[64 * k1];
    uint4 c2 = c0;
    if constexpr (B == 3) c2 = cb[64 * 2];
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 g[4];
    auto kstep = [&](auto KTc) __attribute__((always_inline)) {
      constexpr int kt = decltype(KTc)::value;
      constexpr int F = 4 * rt + kt;
      const uint4& c = lo_chunk<B, F>() == k0 ? c0 : c1;
      const bf16x8 bop = b_lo<B, F>(c, c2);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) g[mt] = mfma_bf16(A[kt][mt], bop, kt == 0 ? zero : g[mt]);
    };
    kstep(std::integral_constant<int, 0>{});
    kstep(std::integral_constant<int, 1>{});
    kstep(std::integral_constant<int, 2>{});
    kstep(std::integral_constant<int, 3>{});
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[mt][rt - RT0][i] = fmaf(sc[rt - RT0], g[mt][i], acc[mt][rt - RT0][i]);
  };
  [&]<int... Js>(std::integer_sequence<int, Js...>) {
    (rstep(std::integral_constant<int, RT0 + Js>{}), ...);
  }(std::make_integer_sequence<int, NRT>{});
}

// Scales of rows 16 (rt0 + j) + (lane & 15) of block (r, c).
template <int NRT>
__device__ __forceinline__ void load_scales(const WeightView& w, int r, int c, int rt0,
                                            float (&s)[NRT]) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = r < w.NBr ? (int64_t)r * w.NBc + c : 0;  // in range for absent rows
#pragma unroll
  for (int j = 0; j < NRT; ++j) s[j] = w.scale[blk * kBlockRows + 16 * (rt0 + j) + (lane & 15)];
}

// Correction product.  With T[n][c] = -s[n][c] (bias_c + z[n][c]) (0 for
// 0-bit blocks) the outputs need acc[m][n] += sum_c S[m][c] T[n][c], a
// product over the Gp (padded) groups.  Both operands are split into three
// bf16 terms (S = S0 + S1 + S2 from the gather kernel, T = T0 + T1 + T2
// here) and the six products Si Tj with i + j <= 2 are accumulated by the
// matrix instructions, 32 groups per instruction: the dropped terms are
// below 2^-24 of |S T| each, i.e. the correction is as accurate as an fp32
// sum.  Per batch of 32 groups the workgroup writes T for its kBR block
// rows into LDS in B-operand order, [q][term][row tile][lane][8 groups] as
// bf16 (12 KiB per block row), then every wavefront multiplies.  The
// scales, zero points and S terms of the next batch are loaded while the
// current one is built and multiplied.
constexpr int kTermBytes = 4 * 64 * 16;  // one term of one block row: 4 row tiles x 1 KiB
constexpr int kTUnits = 4;  // units of 4 rows per thread: kBR * 32 * 16 / (4 kThreads)

// Workgroup barrier that waits for the wavefront's LDS operations only (loads
// from global memory stay in flight); the empty asm statements keep the
// compiler from moving memory operations across it.
// Bitwidth as the products see it.  CH == 8 (weights without 16-bit
// blocks, or kernels that leave them to k_tile16): 16-bit blocks count as
// pruned (their scale is 0, so the correction skips them too).
template <int CH>
__device__ __forceinline__ int tile_bits(int b) { return CH == 16 || b != 16 ? b : 0; }

__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Tile (mtile, ntile) of one matrix over groups g0 .. g1 - 1: rows kBM mtile
// .., block rows kBR ntile ...  part == nullptr: the tile holds all groups
// and y is written (scattered through perm_row); otherwise the tile's share
// of a K split goes to part[m][reordered row] (summed over the splits, in
// split order, by the split-reduce kernel).
//
// BM = kBM: wavefront (wm, wn) = (wave & 1, wave >> 1) takes rows 64 wm ..
// 64 wm + 63 of the tile and all four row tiles of block row rb + wn.  BM =
// 64 (M <= 64, where a 128-row tile would leave half its wavefronts idle):
// wavefront (wr, wn) = (wave & 1, wave >> 1) takes all 64 rows and row tiles
// 2 wr, 2 wr + 1 of block row rb + wn; the products and their order per
// output are the same.
template <int CH, int BM = kBM>
__device__ __forceinline__ void gemm_tile(const uint16_t* __restrict__ xr,
                                          const uint16_t* __restrict__ sxs, int M,
                                          const WeightView& w, float* __restrict__ y, int mtile,
                                          int ntile, int g0, int g1, float* __restrict__ part) {
  static_assert(BM == kBM || BM == 64, "tile heights");
  constexpr int kRT = BM == kBM ? 4 : 2;  // row tiles per wavefront
  static_assert(kTUnits * kThreads == kBR * 32 * 16, "T units per thread");
  __shared__ __align__(16) uint4 a0[kBM * 16];
  __shared__ __align__(16) uint4 c0s[kBR * CH * 64], c1s[kBR * CH * 64];
  __shared__ uint32_t toff[kBR][kTabG];
  __shared__ uint8_t tbits[kBR][kTabG];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // wavefront (wm, wn): rows 64 wm .. 64 wm + 63 of the tile, block row rb +
  // wn, row tiles rt0 .. rt0 + kRT - 1
  const int wm = BM == kBM ? (wave & 1) : 0, wn = wave >> 1;
  const int rt0 = BM == kBM ? 0 : 2 * (wave & 1);
  const int64_t m0 = (int64_t)mtile * BM;
  const int rb = ntile * kBR;  // first block row of the workgroup
  const int r = rb + wn;            // this wavefront's block row
  // a wavefront whose 64 rows all lie past M (the upper half of the last row
  // tile when M mod 128 is in 1 .. 64, e.g. M <= 64) skips its products and
  // its share of the correction; it still copies and meets every barrier
  const bool live = m0 + 64 * wm < M;
  const int64_t K = w.K;
  const int G = w.NBc;
  const int tabG = min(g1 - g0, kTabG);
  const Stage st0{a0, c0s}, st1{a0, c1s};

  // bitwidth and KiB offset of block (rb + q, c): LDS table (groups g0 ..
  // g0 + kTabG - 1), or global past it
  auto block_at = [&](int q, int c, uint32_t& off) __attribute__((always_inline)) -> int {
    if (rb + q >= w.NBr) {
      off = 0;
      return 0;
    }
    if (c - g0 < kTabG) {
      off = __builtin_amdgcn_readfirstlane(toff[q][c - g0]);
      return __builtin_amdgcn_readfirstlane(tbits[q][c - g0]);
    }
    const int64_t blk = (int64_t)(rb + q) * w.NBc + c;
    off = __builtin_amdgcn_readfirstlane(w.block_offset[blk]);
    return tile_bits<CH>(__builtin_amdgcn_readfirstlane(w.bits[blk]));
  };

  // Direct-to-LDS copies of group c into stage st: wavefront w copies rows
  // kRows w .. kRows w + kRows - 1 of the x_r tile (rows past M repeat row
  // M - 1; their products are never stored), and wavefronts 2q, 2q + 1
  // alternate the code chunks of block q.
  auto copy_group = [&](const Stage& st, int c) __attribute__((always_inline)) {
    constexpr int kRows = BM / kWaves;
    const int g = lane >> 4, p = lane & 15;
#pragma unroll
    for (int i = 0; i < kRows / 4; ++i) {
      const int row = kRows * wave + 4 * i + g;
      const int64_t mrow = min(m0 + row, (int64_t)M - 1);
      const uint16_t* src = xr + mrow * K + (int64_t)c * kBlockCols + 8 * (p ^ (row & 15));
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(st.a + (kRows * wave + 4 * i) * 16), 16, 0,
                                       0);
    }
    const int q = wave >> 1, half = wave & 1;
    uint32_t off;
    const int b = block_at(q, c, off);
    const uint8_t* cb = w.codes + (int64_t)off * 1024 + 16 * lane;
#pragma unroll
    for (int t = 0; t < CH; t += 2)
      if (t + half < b)
        __builtin_amdgcn_global_load_lds(cb + 1024 * (t + half),
                                         (lds_void*)(st.codes + (q * CH + t + half) * 64), 16, 0, 0);
  };

  // the workgroup's bit map and offsets for the first tabG groups of its range
  for (int i = tid; i < kBR * tabG; i += kThreads) {
    const int q = i / tabG, c = i - (i / tabG) * tabG;
    const int rr = rb + q;
    const int64_t blk = (int64_t)(rr < w.NBr ? rr : 0) * w.NBc + g0 + c;
    tbits[q][c] = rr < w.NBr ? tile_bits<CH>(w.bits[blk]) : 0;
    toff[q][c] = rr < w.NBr ? w.block_offset[blk] : 0u;
  }
  __syncthreads();

  // this lane's A fragment offsets per k-step (m tile 0), bytes
  uint32_t apk[4];
  {
    const int g = lane >> 4, n = lane & 15;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      apk[kt] = (uint32_t)((64 * wm + n) * 256 + (((4 * kt + g) ^ n) << 4));
  }

  // acc[mt][j]: rows 64 wm + 16 mt + 4 (lane >> 4) + i, output row
  // 16 (rt0 + j) + (lane & 15)
  f32x4 acc[4][kRT];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int j = 0; j < kRT; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one group from stage st (A fragments A) with the block's scales sc
  // the wavefront's row tiles of one B-bit block (BM = 64: which pair is
  // uniform over the wavefront)
  auto mma = [&](const Stage& st, const bf16x8 (&A)[4][4], const float (&sc)[kRT], auto Bc)
                 __attribute__((always_inline)) {
    constexpr int B = decltype(Bc)::value;
    if constexpr (BM == kBM) {
      if constexpr (B == 16) group_mfma16<CH, 0, 4>(st, wn, A, acc);
      else group_mfma<B, CH, 0, 4>(st, wn, A, sc, acc);
    } else if (rt0 == 0) {
      if constexpr (B == 16) group_mfma16<CH, 0, 2>(st, wn, A, acc);
      else group_mfma<B, CH, 0, 2>(st, wn, A, sc, acc);
    } else {
      if constexpr (B == 16) group_mfma16<CH, 2, 2>(st, wn, A, acc);
      else group_mfma<B, CH, 2, 2>(st, wn, A, sc, acc);
    }
  };
  auto products = [&](const Stage& st, int c, const bf16x8 (&A)[4][4], const float (&sc)[kRT])
                      __attribute__((always_inline)) {
    uint32_t unused_off;
    const int b = block_at(wn, c, unused_off);
    switch (b) {
      case 0: break;
      case 1: mma(st, A, sc, std::integral_constant<int, 1>{}); break;
      case 2: mma(st, A, sc, std::integral_constant<int, 2>{}); break;
      case 3: mma(st, A, sc, std::integral_constant<int, 3>{}); break;
      case 4: mma(st, A, sc, std::integral_constant<int, 4>{}); break;
      case 16:
        if constexpr (CH == 16) mma(st, A, sc, std::integral_constant<int, 16>{});
        break;
      default: mma(st, A, sc, std::integral_constant<int, 8>{}); break;
    }
  };
  // own copies done, then the workgroup barrier (no memory fence: the copies
  // are the only producer and their completion is what is waited for)
  auto stage_barrier = [&]() __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  float cur[kRT], nxt[kRT];
  copy_group(st0, g0);
  load_scales(w, r, g0, rt0, cur);
  stage_barrier();

  // group c: A fragments from the one x_r buffer into registers, barrier,
  // copies of group c + 1 (x_r into that buffer, codes into the other code
  // buffer), products of group c, barrier
  auto group = [&](const Stage& st, const Stage& nx, int c) __attribute__((always_inline)) {
    uint32_t unused_off;
    bf16x8 A[4][4];
    if (live && block_at(wn, c, unused_off) != 0) read_a(st, apk, A);
    lds_barrier();
    if (c + 1 < g1) {
      copy_group(nx, c + 1);
      load_scales(w, r, c + 1, rt0, nxt);
    }
    if (live) products(st, c, A, cur);
    stage_barrier();
#pragma unroll
    for (int j = 0; j < kRT; ++j) cur[j] = nxt[j];
  };
  for (int c = g0; c < g1; c += 2) {
    group(st0, st1, c);
    if (c + 1 >= g1) break;
    group(st1, st0, c + 1);
  }

  // ---- correction product (the x_r buffer is free now: T of both block rows goes there)
  const int64_t Gp = padded_groups(G);
  auto tq = [&](int q) __attribute__((always_inline)) -> unsigned char* {
    return reinterpret_cast<unsigned char*>(a0) + q * 3 * kTermBytes;
  };
  static_assert(kBR * 3 * kTermBytes <= (int)sizeof(a0), "T terms of the block rows in the x_r buffer");
  const int64_t plane = (int64_t)M * Gp;
  // unit u = (q, gl, 4 rows n4 .. n4 + 3) for u = tid + kThreads * k
  float4 ls[kTUnits];
  uint32_t lz[kTUnits];
  int lb[kTUnits];
  auto load_t = [&](int64_t j0) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kTUnits; ++k) {
      const int u = tid + kThreads * k;
      const int q = u >> 9, gl = (u >> 4) & 31, n4 = 4 * (u & 15);
      const int64_t c = j0 + gl;
      const int rr = rb + q;
      const bool live = rr < w.NBr && c >= g0 && c < g1;
      const int64_t blk = live ? (int64_t)rr * w.NBc + c : 0;
      lb[k] = !live ? 0 : (c - g0 < kTabG ? (int)tbits[q][c - g0] : tile_bits<CH>(w.bits[blk]));
      ls[k] = *reinterpret_cast<const float4*>(w.scale + blk * kBlockRows + n4);
      lz[k] = *reinterpret_cast<const uint32_t*>(w.zero + blk * kBlockRows + n4);
    }
  };
  bf16x8 Sa[3][4];
  auto load_s = [&](int64_t j0) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int64_t mrow = min(m0 + 64 * wm + 16 * mt + (lane & 15), (int64_t)M - 1);
      const uint16_t* src = sxs + mrow * Gp + j0 + 8 * (lane >> 4);
#pragma unroll
      for (int t = 0; t < 3; ++t)
        Sa[t][mt] = as_bf16x8(*reinterpret_cast<const uint4*>(src + t * plane));
    }
  };
  // batches of 32 groups covering g0 .. g1 - 1 (T is zero outside the range)
  const int64_t jb = g0 & ~31;
  load_t(jb);
  for (int64_t j0 = jb; j0 < g1; j0 += 32) {
    load_s(j0);
    lds_barrier();  // previous readers of the stage buffers are done
#pragma unroll
    for (int k = 0; k < kTUnits; ++k) {
      const int u = tid + kThreads * k;
      const int q = u >> 9, gl = (u >> 4) & 31, n4 = 4 * (u & 15);
      const float bias = gemm_bias(lb[k]);
      const float sv[4] = {ls[k].x, ls[k].y, ls[k].z, ls[k].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = n4 + e;
        const float T = lb[k] == 0 ? 0.f : -sv[e] * (bias + (float)((lz[k] >> (8 * e)) & 0xFFu));
        const uint16_t t0 = bf16_rn(T);
        const float r1 = T - bf16f(t0);
        const uint16_t t1 = bf16_rn(r1);
        const uint16_t t2 = bf16_rn(r1 - bf16f(t1));
        // B operand order: row tile n >> 4, lane 16 (gl >> 3) + (n & 15), element gl & 7
        const int at = ((n >> 4) * 64 + (gl >> 3) * 16 + (n & 15)) * 16 + (gl & 7) * 2;
        *reinterpret_cast<uint16_t*>(tq(q) + at) = t0;
        *reinterpret_cast<uint16_t*>(tq(q) + kTermBytes + at) = t1;
        *reinterpret_cast<uint16_t*>(tq(q) + 2 * kTermBytes + at) = t2;
      }
    }
    if (j0 + 32 < g1) load_t(j0 + 32);
    lds_barrier();
    if (!live) continue;  // the barriers above are the loop's only ones
    bf16x8 Tb[3][kRT];
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
      for (int j = 0; j < kRT; ++j)
        Tb[t][j] = as_bf16x8(*reinterpret_cast<const uint4*>(
            tq(wn) + t * kTermBytes + ((rt0 + j) * 64 + lane) * 16));
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int j = 0; j < kRT; ++j) {
        f32x4 v = acc[mt][j];
        v = mfma_bf16(Sa[2][mt], Tb[0][j], v);
        v = mfma_bf16(Sa[1][mt], Tb[1][j], v);
        v = mfma_bf16(Sa[0][mt], Tb[2][j], v);
        v = mfma_bf16(Sa[1][mt], Tb[0][j], v);
        v = mfma_bf16(Sa[0][mt], Tb[1][j], v);
        acc[mt][j] = mfma_bf16(Sa[0][mt], Tb[0][j], v);
      }
  }

  // epilogue: y[m][perm_row[n]], or the split's partial part[m][n]
  if (r >= w.NBr) return;
#pragma unroll
  for (int j = 0; j < kRT; ++j) {
    const int64_t row = (int64_t)r * kBlockRows + 16 * (rt0 + j) + (lane & 15);
    int col = part ? (int)row : w.perm_row[row];
    col = min(max(col, 0), (int)w.N - 1);
    float* out = part ? part : y;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + 64 * wm + 16 * mt + 4 * (lane >> 4) + i;
        if (m < M) out[m * w.N + col] = acc[mt][j][i];
      }
  }
}

template <int CH, int BM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm(
    const uint16_t* __restrict__ xr, const uint16_t* __restrict__ sxs, int M, WeightView w,
    float* __restrict__ y, float* __restrict__ part, int gper) {
  // K split blockIdx.z: groups gper z .. ; partials plane z of part
  const int g0 = blockIdx.z * gper, g1 = min(w.NBc, g0 + gper);
  gemm_tile<CH, BM>(xr, sxs, M, w, y, blockIdx.x, blockIdx.y, g0, g1,
                    part ? part + (int64_t)blockIdx.z * M * w.N : nullptr);
}

// ---- grouped calls: up to kGroupMax matrices at the same M -------------------------------
// One gather launch and one GEMM launch cover all matrices of the group (for
// example q, k, v of a layer); the tiles of job j follow those of job j - 1,
// so the tiles of small matrices fill the CUs that a large one leaves idle in
// its last round.
constexpr int kGroupMax = 8;

struct GemmJob {
  WeightView w;
  const uint16_t* x;
  uint16_t* xr;
  uint16_t* sxs;
  float* y;
  float* yr;       // non-null: the tiles write y in reordered order here (= y), un-permuted after
  int staged;      // gather: x row staged in LDS
  int mtiles;      // tiles along M
  int tile_begin;  // first tile of the job in the GEMM launch
};

struct GemmGroup {
  GemmJob job[kGroupMax];
  int count;
  int M;
};

// Copy of the job owning tile (or gather row) b, selected with static indices.
__device__ __forceinline__ GemmJob pick_gemm_job(const GemmGroup& g, int b, bool gather) {
  GemmJob q = g.job[0];
#pragma unroll
  for (int k = 1; k < kGroupMax; ++k)
    if (k < g.count && b >= (gather ? k * g.M : g.job[k].tile_begin)) q = g.job[k];
  return q;
}

__global__ __launch_bounds__(kGatherThreads) void k_gather_x_group(GemmGroup g) {
  const GemmJob q = pick_gemm_job(g, blockIdx.x, true);
  gather_row(q.x, q.w.K, g.M, q.w.perm_col, q.xr, q.sxs, nullptr, 0, q.staged, blockIdx.x % g.M,
             0, padded_groups(q.w.K / kBlockCols) * 16);
}

// Grouped gather of the decode kernel at small M (fp32 sums too): job j owns
// the workgroups [begin_j, begin of j + 1), M rows x `slices` slices of
// whole groups, cut as launch_gather_x cuts one matrix's.
struct GatherJob {
  const uint16_t* x;
  const int32_t* perm_col;
  int64_t K;
  uint16_t* xr;
  uint16_t* sxs;
  float* sf;
  uint32_t* counters;  // the decode's K-split counters, cleared here
  int ncounters;
  int staged, slices, begin;
};

struct GatherGroup {
  GatherJob job[kGroupMax];
  int count;
  int M;
};

__global__ __launch_bounds__(kGatherThreads) void k_gather_x_jobs(GatherGroup g) {
  GatherJob q = g.job[0];
#pragma unroll
  for (int k = 1; k < kGroupMax; ++k)
    if (k < g.count && (int)blockIdx.x >= g.job[k].begin) q = g.job[k];
  const int b = blockIdx.x - q.begin;
  clear_counters(q.counters, q.ncounters, b, (int64_t)g.M * q.slices);
  const int m = b / q.slices, sl = b - m * q.slices;
  const int64_t Gp = padded_groups(q.K / kBlockCols);
  const int64_t per = (Gp + q.slices - 1) / q.slices * 16;
  const int64_t qs = (int64_t)sl * per;
  gather_row(q.x, q.K, g.M, q.perm_col, q.xr, q.sxs, q.sf, gather_mpad(g.M), q.staged, m, qs,
             min(qs + per, Gp * 16));
}

template <int CH>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm_group(
    GemmGroup g) {
  const GemmJob q = pick_gemm_job(g, blockIdx.x, false);
  const int t = blockIdx.x - q.tile_begin;
  gemm_tile<CH>(q.xr, q.sxs, g.M, q.w, q.y, t % q.mtiles, t / q.mtiles, 0, q.w.NBc, q.yr);
}

// ---- row un-permutation ------------------------------------------------------------
// The GEMM tiles cover consecutive reordered rows n, whose original columns
// perm_row[n] of y are scattered: writing y[m][perm_row[n]] from the tiles
// leaves every 64-byte line of y partly written by many workgroups, and the
// partial lines reach HBM many times over (about 9x the bytes of y).  So the
// tiles write y in reordered order into y itself, and one workgroup per row
// then permutes the row through LDS: coalesced reads of the row (and of
// perm_row, which stays in L2 across rows), the scatter as LDS stores, and
// coalesced writes of the permuted row back in place.
constexpr int kUnpermuteThreads = 1024;
constexpr int kUnpermuteBatch = 8;  // loads in flight per thread
constexpr int64_t kUnpermuteMaxN = 32768;  // the row in LDS: 128 KiB

struct UnpermuteJob {
  float* y;
  const int32_t* perm_row;
  int64_t N;
};
struct UnpermuteGroup {
  UnpermuteJob job[kGroupMax];
  int count;
};

// Row blockIdx.x of job blockIdx.y (N <= kUnpermuteMaxN, dynamic LDS of at
// least 4 N bytes): y[perm_row[n]] = y[n].
__global__ __launch_bounds__(kUnpermuteThreads) void k_unpermute_rows(UnpermuteGroup g) {
  UnpermuteJob q = g.job[0];
#pragma unroll
  for (int k = 1; k < kGroupMax; ++k)
    if (k == (int)blockIdx.y) q = g.job[k];
  float* row = q.y + (int64_t)blockIdx.x * q.N;
  float* lrow = reinterpret_cast<float*>(smem);
  const int N = (int)q.N;
  const int t = threadIdx.x;
  for (int base = t; base < N; base += kUnpermuteBatch * kUnpermuteThreads) {
    float v[kUnpermuteBatch];
    int dst[kUnpermuteBatch];
#pragma unroll
    for (int i = 0; i < kUnpermuteBatch; ++i) {
      const int n = min(base + i * kUnpermuteThreads, N - 1);
      v[i] = row[n];
      dst[i] = min(max(q.perm_row[n], 0), N - 1);
    }
#pragma unroll
    for (int i = 0; i < kUnpermuteBatch; ++i)
      if (base + i * kUnpermuteThreads < N) lrow[dst[i]] = v[i];
  }
  __syncthreads();  // the whole row is read (and scattered) before any of it is overwritten
  for (int n = t; n < N; n += kUnpermuteThreads) row[n] = lrow[n];
}

// The same with 16-byte accesses (every job's y and perm_row 16-byte aligned;
// N is a multiple of 64): each thread reads four float4 of the row and the
// four int4 of perm_row that go with them before scattering the sixteen
// values into LDS, and writes the permuted row back as float4.
constexpr int kUnpermuteVec = 4;  // float4 loads in flight per thread
__global__ __launch_bounds__(kUnpermuteThreads) void k_unpermute_rows4(UnpermuteGroup g) {
  UnpermuteJob q = g.job[0];
#pragma unroll
  for (int k = 1; k < kGroupMax; ++k)
    if (k == (int)blockIdx.y) q = g.job[k];
  float* row = q.y + (int64_t)blockIdx.x * q.N;
  float* lrow = reinterpret_cast<float*>(smem);
  const int N = (int)q.N, N4 = N / 4, hi = N - 1;
  const int t = threadIdx.x;
  const float4* row4 = reinterpret_cast<const float4*>(row);
  const int4* perm4 = reinterpret_cast<const int4*>(q.perm_row);
  for (int base = t; base < N4; base += kUnpermuteVec * kUnpermuteThreads) {
    float4 v[kUnpermuteVec];
    int4 p[kUnpermuteVec];
#pragma unroll
    for (int i = 0; i < kUnpermuteVec; ++i) {
      const int n4 = min(base + i * kUnpermuteThreads, N4 - 1);
      v[i] = row4[n4];
      p[i] = perm4[n4];
    }
#pragma unroll
    for (int i = 0; i < kUnpermuteVec; ++i)
      if (base + i * kUnpermuteThreads < N4) {
        lrow[min(max(p[i].x, 0), hi)] = v[i].x;
        lrow[min(max(p[i].y, 0), hi)] = v[i].y;
        lrow[min(max(p[i].z, 0), hi)] = v[i].z;
        lrow[min(max(p[i].w, 0), hi)] = v[i].w;
      }
  }
  __syncthreads();  // the whole row is read (and scattered) before any of it is overwritten
  float4* out4 = reinterpret_cast<float4*>(row);
  const float4* l4 = reinterpret_cast<const float4*>(lrow);
  for (int n4 = t; n4 < N4; n4 += kUnpermuteThreads) out4[n4] = l4[n4];
}

// Launch the un-permutation of the group's jobs (rows 0 .. M-1 of each).
hipError_t launch_unpermute(const UnpermuteGroup& u, int64_t M, int64_t maxn, hipStream_t stream) {
  bool vec = true;
  for (int i = 0; i < u.count; ++i)
    vec = vec && ((reinterpret_cast<uintptr_t>(u.job[i].y) |
                   reinterpret_cast<uintptr_t>(u.job[i].perm_row)) & 15) == 0;
  if (vec)
    hipLaunchKernelGGL(k_unpermute_rows4, dim3((unsigned)M, (unsigned)u.count),
                       dim3(kUnpermuteThreads), (size_t)maxn * 4, stream, u);
  else
    hipLaunchKernelGGL(k_unpermute_rows, dim3((unsigned)M, (unsigned)u.count),
                       dim3(kUnpermuteThreads), (size_t)maxn * 4, stream, u);
  return hipGetLastError();
}

// Launch shape of one GEMM call.  Fewer tiles than kFillTiles (two per CU)
// split K into ranges of at least kMinSplitGroups groups (the correction
// product works on batches of 32 groups, so shorter ranges waste it), the
// ranges' partials summed by the split reduction.  opt.gemm_split overrides
// the split count.
constexpr int64_t kFillTiles = 512;
constexpr int64_t kMinSplitGroups = 8;
struct GemmPlan {
  int split, gper;
};
GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, const Options& opt) {
  GemmPlan p{};
  const int64_t G = K / kBlockCols;
  const int64_t tiles = ((M + kBM - 1) / kBM) * ((N / kBlockRows + kBR - 1) / kBR);
  int64_t split = opt.gemm_split > 0 ? opt.gemm_split
                                     : (tiles >= kFillTiles ? 1 : (kFillTiles + tiles - 1) / tiles);
  split = std::min<int64_t>(split, std::max<int64_t>(1, G / kMinSplitGroups));
  if (split < 1) split = 1;
  p.gper = (int)((G + split - 1) / split);
  p.split = (int)((G + p.gper - 1) / p.gper);
  return p;
}

}  // namespace

// [x_r | three bf16 terms of the group sums | fp32 group sums], each part 256-byte aligned
size_t gather_workspace_bytes(int64_t M, int64_t K) {
  const size_t xr = (size_t)M * K * 2;
  const size_t xr_al = (xr + 255) & ~(size_t)255;
  const size_t gp = (size_t)padded_groups(K / kBlockCols);
  const size_t terms = ((3 * (size_t)M * gp * 2) + 255) & ~(size_t)255;
  return xr_al + terms + gp * (size_t)gather_mpad(M) * 4;
}

float* gather_sums_f32(void* ws, int64_t M, int64_t K) {
  const size_t xr_al = (((size_t)M * K * 2) + 255) & ~(size_t)255;
  const size_t gp = (size_t)padded_groups(K / kBlockCols);
  const size_t terms = ((3 * (size_t)M * gp * 2) + 255) & ~(size_t)255;
  return reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + xr_al + terms);
}

size_t gemm_group_workspace_bytes(int64_t M, const WeightView* w, int count, const Options& opt) {
  size_t total = 0;
  for (int i = 0; i < count; ++i)
    total += (gemm_workspace_bytes(M, w[i].N, w[i].K, opt) + 255) & ~(size_t)255;
  return total;
}

hipError_t launch_gemm_group(const uint16_t* const* x, int64_t M, const WeightView* w,
                             float* const* y, int count, void* workspace, const Options& opt,
                             hipStream_t stream) {
  if (count < 1 || count > kGroupMax) return hipErrorInvalidValue;
  GemmGroup g{};
  g.count = count;
  g.M = (int)M;
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  size_t lds = 0;
  int64_t tiles = 0;
  for (int i = 0; i < count; ++i)
    tiles += (M + kBM - 1) / kBM * ((w[i].NBr + kBR - 1) / kBR);
  if (tiles < kFillTiles || tiles > 0x7FFFFFFF || M * count > 0x7FFFFFFF) {
    // too few tiles to fill the GPU (each call then splits K), or beyond one
    // launch's grid: each matrix on its own, in its own workspace
    for (int i = 0; i < count; ++i) {
      const hipError_t e = launch_gemm(x[i], M, w[i], y[i], ws, opt, stream);
      if (e != hipSuccess) return e;
      ws += (gemm_workspace_bytes(M, w[i].N, w[i].K, opt) + 255) & ~(size_t)255;
    }
    return hipSuccess;
  }
  tiles = 0;
  for (int i = 0; i < count; ++i) {
    GemmJob& q = g.job[i];
    const int64_t K = w[i].K;
    q.w = w[i];
    q.x = x[i];
    q.xr = reinterpret_cast<uint16_t*>(ws);
    const size_t xr_bytes = (((size_t)M * K * 2) + 255) & ~(size_t)255;
    q.sxs = reinterpret_cast<uint16_t*>(ws + xr_bytes);
    ws += (gemm_workspace_bytes(M, w[i].N, K, opt) + 255) & ~(size_t)255;
    q.y = y[i];
    q.yr = w[i].N <= kUnpermuteMaxN ? y[i] : nullptr;
    q.staged = (size_t)K * 2 <= kGatherMaxLds;
    if (q.staged) lds = std::max(lds, (size_t)K * 2);
    q.mtiles = (int)((M + kBM - 1) / kBM);
    q.tile_begin = (int)tiles;
    tiles += (int64_t)q.mtiles * ((w[i].NBr + kBR - 1) / kBR);
  }
  hipLaunchKernelGGL(k_gather_x_group, dim3((unsigned)(M * count)), dim3(kGatherThreads), lds,
                     stream, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  bool any16 = false;
  for (int i = 0; i < count; ++i) any16 = any16 || w[i].has16;
  if (any16)
    hipLaunchKernelGGL((k_gemm_group<16>), dim3((unsigned)tiles), dim3(kThreads), 0, stream, g);
  else
    hipLaunchKernelGGL((k_gemm_group<8>), dim3((unsigned)tiles), dim3(kThreads), 0, stream, g);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  UnpermuteGroup u{};
  int64_t maxn = 0;
  for (int i = 0; i < count; ++i)
    if (g.job[i].yr) {
      u.job[u.count++] = UnpermuteJob{y[i], w[i].perm_row, w[i].N};
      maxn = std::max(maxn, w[i].N);
    }
  if (u.count == 0) return hipSuccess;
  return launch_unpermute(u, M, maxn, stream);
}

// Slices per row of the gather: with few rows each row's groups are cut into
// slices of their own workgroups (every slice stages the whole row), so that
// small M still fills the GPU.
static int64_t gather_slices(int64_t M, int64_t K) {
  return std::max<int64_t>(
      1, std::min<int64_t>(padded_groups(K / kBlockCols) / 16, 256 / std::max<int64_t>(M, 1)));
}

hipError_t launch_gather_x_group(const uint16_t* const* x, int64_t M, const WeightView* w,
                                 void* const* ws, uint32_t* const* counters,
                                 const int* ncounters, int count, hipStream_t stream) {
  if (count < 1 || count > kGroupMax) return hipErrorInvalidValue;
  GatherGroup g{};
  g.count = count;
  g.M = (int)M;
  size_t lds = 0;
  int64_t total = 0;
  for (int i = 0; i < count; ++i) {
    GatherJob& q = g.job[i];
    const int64_t K = w[i].K;
    uint8_t* b = reinterpret_cast<uint8_t*>(ws[i]);
    q.x = x[i];
    q.perm_col = w[i].perm_col;
    q.K = K;
    q.xr = reinterpret_cast<uint16_t*>(b);
    q.sxs = reinterpret_cast<uint16_t*>(b + ((((size_t)M * K * 2) + 255) & ~(size_t)255));
    q.sf = gather_sums_f32(ws[i], M, K);
    q.staged = (size_t)K * 2 <= kGatherMaxLds;
    if (q.staged) lds = std::max(lds, (size_t)K * 2);
    q.slices = (int)gather_slices(M, K);
    q.counters = counters[i];
    q.ncounters = ncounters[i];
    q.begin = (int)total;
    total += M * q.slices;
  }
  if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_gather_x_jobs, dim3((unsigned)total), dim3(kGatherThreads), lds, stream, g);
  return hipGetLastError();
}

hipError_t launch_gather_x(const uint16_t* x, int64_t M, const WeightView& w, void* ws,
                           hipStream_t stream, bool sums_f32, uint32_t* counters,
                           int ncounters) {
  const int64_t K = w.K;
  uint16_t* xr = reinterpret_cast<uint16_t*>(ws);
  const size_t xr_bytes = (((size_t)M * K * 2) + 255) & ~(size_t)255;
  uint16_t* sxs = reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(ws) + xr_bytes);
  const size_t row_bytes = (size_t)K * 2;
  const int staged = row_bytes <= kGatherMaxLds;
  const int64_t slices = gather_slices(M, K);
  float* sf = sums_f32 ? gather_sums_f32(ws, M, K) : nullptr;
  hipLaunchKernelGGL(k_gather_x, dim3((unsigned)M, (unsigned)slices), dim3(kGatherThreads),
                     staged ? row_bytes : 0, stream, x, K, M, w.perm_col, xr, sxs, sf,
                     (int64_t)gather_mpad(M), staged, counters, ncounters);
  return hipGetLastError();
}

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, const Options& opt) {
  const GemmPlan p = plan_gemm(M, N, K, opt);
  const size_t gather = (gather_workspace_bytes(M, K) + 255) & ~(size_t)255;
  return gather + (p.split > 1 ? (size_t)p.split * M * N * 4 : 0);
}

hipError_t launch_gemm(const uint16_t* x, int64_t M, const WeightView& w, float* y,
                       void* workspace, const Options& opt, hipStream_t stream) {
  const int64_t K = w.K;
  const GemmPlan p = plan_gemm(M, w.N, K, opt);
  uint16_t* xr = reinterpret_cast<uint16_t*>(workspace);
  const size_t xr_bytes = (((size_t)M * K * 2) + 255) & ~(size_t)255;
  uint16_t* sxs = reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(workspace) + xr_bytes);
  float* part = p.split > 1
                    ? reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(workspace) +
                                               ((gather_workspace_bytes(M, K) + 255) & ~(size_t)255))
                    : nullptr;
  hipError_t e = launch_gather_x(x, M, w, workspace, stream, false, nullptr, 0);
  if (e != hipSuccess) return e;
  // M <= 64: 64-row tiles (every wavefront holds rows below M)
  const bool short_m = M <= 64;
  const int64_t bm = short_m ? 64 : kBM;
  const dim3 grid((unsigned)((M + bm - 1) / bm), (unsigned)((w.NBr + kBR - 1) / kBR),
                  (unsigned)p.split);
  // one K range: the tiles write y in reordered order (into y), un-permuted after
  const bool unpermute = p.split == 1 && w.N <= kUnpermuteMaxN;
  float* out = p.split > 1 ? part : (unpermute ? y : nullptr);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, stream, xr, sxs, (int)M, w, y, out, p.gper);
  };
  if (w.has16) {
    if (short_m) go(k_gemm<16, 64>);
    else go(k_gemm<16, kBM>);
  } else {
    if (short_m) go(k_gemm<8, 64>);
    else go(k_gemm<8, kBM>);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.split > 1) return launch_split_reduce(part, p.split, M, w.N, w.perm_row, y, stream);
  if (!unpermute) return hipSuccess;
  UnpermuteGroup u{};
  u.job[0] = UnpermuteJob{y, w.perm_row, w.N};
  u.count = 1;
  return launch_unpermute(u, M, w.N, stream);
}

}  // namespace msq

// Prefill GEMM for gfx950: y = x . W^T for any M (used for M > 64), W
// dequantized on the fly from packed format v1 and multiplied on the bf16
// matrix cores.
//
// Two kernels:
//   k_gather_x : x_r[m][j] = x[m][perm_col[j]] (bf16) and the per-group sums
//                sum_j x_r[m][j] over each 128-column group (fp32), written to
//                the workspace once per call (the activation reordering of the
//                "SFMP" abstract).
//   k_gemm     : workgroup tile 128 (M) x 256 (N = four block rows), eight
//                wavefronts of 64 x 64, one K group ahead in flight; details
//                above the kernel.
//
// Keeping the matrix-core operands exact integers and applying the fp32 scale
// per (row, group) keeps y within fp32 accumulation error of the exact
// product; rounding s * (q - z) to bf16 first would not.
#include <hip/hip_runtime.h>
#include <stdint.h>

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
// summed with shuffles.
constexpr int kGatherThreads = 256;
constexpr size_t kGatherMaxLds = 64 * 1024;

__global__ __launch_bounds__(kGatherThreads) void k_gather_x(const uint16_t* __restrict__ x,
                                                             int64_t K,
                                                             const int32_t* __restrict__ perm_col,
                                                             uint16_t* __restrict__ xr,
                                                             float* __restrict__ xsum, int staged) {
  const int64_t m = blockIdx.x;
  const int64_t chunks = K / 8;
  const int G = (int)(K / kBlockCols);
  const uint16_t* xrow = x + m * K;
  uint16_t* srow = reinterpret_cast<uint16_t*>(smem);
  if (staged) {
    const uint4* src = reinterpret_cast<const uint4*>(xrow);
    for (int64_t i = threadIdx.x; i < chunks; i += kGatherThreads)
      reinterpret_cast<uint4*>(smem)[i] = src[i];
    __syncthreads();
  }
  const uint16_t* from = staged ? srow : xrow;
  const int kk = (int)K - 1;
  for (int64_t q0 = 0; q0 < chunks; q0 += kGatherThreads) {
    const int64_t q = q0 + threadIdx.x;
    float part = 0.f;
    if (q < chunks) {
      const int4* pc = reinterpret_cast<const int4*>(perm_col + 8 * q);
      const int4 p0 = pc[0], p1 = pc[1];
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
    if (q < chunks && (q & 15) == 0) xsum[m * G + q / 16] = part;
  }
}

// ---- GEMM ------------------------------------------------------------------------------
//
// Workgroup tile: kBM rows of x_r x kBR block rows (64 outputs each); eight
// wavefronts (wm, wn) = (wave & 1, wave >> 1), each 64 rows x one block row,
// two wavefronts per SIMD (one workgroup per CU: the LDS holds two stages).
// Per 128-wide K group c:
//   - the next group's x_r tile (kBM x 128 bf16), its group sums and the
//     workgroup's kBR blocks of codes are copied global -> LDS by the
//     direct-to-LDS loads (global_load_lds_dwordx4) into the other stage,
//     and each wavefront loads its block's next scales and zero points;
//   - the wavefront reads its block's code chunks and, per k-step of 32, its
//     4 A fragments from LDS, unpacks 4 B fragments to exact bf16 (128 + q;
//     3-bit: two planes with bias 256; 8-bit: low 7 bits and top bit, bias
//     384), and issues 16 v_mfma_f32_16x16x32_bf16 into group accumulators;
//   - fold: acc += s_n * acc_g - s_n * (bias + z_n) * sum_x[m][c];
//   - wait for its own copies, one barrier.
// The two stages are distinct LDS objects and the loop is unrolled by two,
// so the compiler sees that the copies in flight never alias what the
// products read and adds no wait for them before those reads.  The x_r tile
// is stored without padding, 16-byte chunk p of row r holding column chunk
// p ^ (r & 15) (the direct-to-LDS copies write each 1 KiB contiguously; the
// swizzle keeps the fragment reads free of bank conflicts).  0-bit blocks
// skip the copies and the products.  y is scattered to original rows
// through perm_row.
constexpr int kBM = 128;
constexpr int kBR = 4;
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kTabG = 512;  // groups whose bit map and offsets are staged in LDS

typedef __attribute__((address_space(3))) void lds_void;

__host__ __device__ constexpr float gemm_bias(int b) {
  return b == 8 ? 384.f : (b == 3 ? 256.f : 128.f);
}

// Unpacked B operand of fragment F of a B-bit block (low plane for 3- and 8-bit).
template <int B, int F>
__device__ __forceinline__ bf16x8 gemm_b_lo(const uint4* ch) {
  if constexpr (B == 8) return exp_lo<8, F>(ch[F / 2]);
  else return block_operand<B, F>(ch);
}

template <int B, int F>
__device__ __forceinline__ bf16x8 gemm_b_hi(const uint4* ch) {
  if constexpr (B == 8) return exp_hi<8, F>(ch[F / 2]);
  else return hi3_operand<F>(ch);
}

// One stage of the pipeline in LDS.
struct Stage {
  uint4* a;      // x_r tile [kBM][16 chunks], swizzled
  float* sx;     // group sums [kBM]
  uint4* codes;  // [kBR][8 chunks][64 lanes]
};

// acc_g = A . B for this wavefront's B-bit block: 4 k-steps x 4 row tiles x
// 4 m tiles.  apk[kt] = this lane's byte offset of its A fragment (m tile 0)
// for k-step kt; m tile mt is 4096 bytes further.
template <int B>
__device__ __forceinline__ void group_mfma(const Stage& st, int q, const uint32_t (&apk)[4],
                                           f32x4 (&accg)[4][4]) {
  const int lane = threadIdx.x & 63;
  uint4 ch[B];
#pragma unroll
  for (int t = 0; t < B; ++t) ch[t] = st.codes[(q * 8 + t) * 64 + lane];
  const unsigned char* abase = reinterpret_cast<const unsigned char*>(st.a);
  auto kstep = [&](auto KTc) {
    constexpr int kt = decltype(KTc)::value;
    bf16x8 A[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      A[mt] = as_bf16x8(*reinterpret_cast<const uint4*>(abase + apk[kt] + 4096 * mt));
    auto rstep = [&](auto RTc) {
      constexpr int rt = decltype(RTc)::value;
      constexpr int F = 4 * rt + kt;
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      const bf16x8 bop = gemm_b_lo<B, F>(ch);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        accg[mt][rt] = mfma_bf16(A[mt], bop, kt == 0 ? zero : accg[mt][rt]);
      if constexpr (B == 3 || B == 8) {
        const bf16x8 hop = gemm_b_hi<B, F>(ch);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) accg[mt][rt] = mfma_bf16(A[mt], hop, accg[mt][rt]);
      }
    };
    rstep(std::integral_constant<int, 0>{});
    rstep(std::integral_constant<int, 1>{});
    rstep(std::integral_constant<int, 2>{});
    rstep(std::integral_constant<int, 3>{});
  };
  kstep(std::integral_constant<int, 0>{});
  kstep(std::integral_constant<int, 1>{});
  kstep(std::integral_constant<int, 2>{});
  kstep(std::integral_constant<int, 3>{});
}

// Scale and zero point of rows 16*rt + (lane & 15) of a block, as loaded (the
// conversions happen at the fold, so that issuing these loads never waits).
struct BlockMeta {
  float s[4];
  uint32_t z[4];
};

__device__ __forceinline__ void load_meta(const WeightView& w, int r, int c, BlockMeta& bm) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = r < w.NBr ? (int64_t)r * w.NBc + c : 0;  // in range for absent rows
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int n = 16 * rt + (lane & 15);
    bm.s[rt] = w.scale[blk * kBlockRows + n];
    bm.z[rt] = w.zero[blk * kBlockRows + n];
  }
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm(
    const uint16_t* __restrict__ xr, const float* __restrict__ xsum, int M, WeightView w,
    float* __restrict__ y) {
  __shared__ __align__(16) uint4 a0[kBM * 16], a1[kBM * 16];
  __shared__ __align__(16) float sx0[kBM], sx1[kBM];
  __shared__ __align__(16) uint4 c0s[kBR * 8 * 64], c1s[kBR * 8 * 64];
  __shared__ uint32_t toff[kBR][kTabG];
  __shared__ uint8_t tbits[kBR][kTabG];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t m0 = (int64_t)blockIdx.x * kBM;
  const int rb = blockIdx.y * kBR;  // first block row of the workgroup
  const int r = rb + wn;            // this wavefront's block row
  const int64_t K = w.K;
  const int G = w.NBc;
  const int tabG = min(G, kTabG);
  const Stage st0{a0, sx0, c0s}, st1{a1, sx1, c1s};

  // bitwidth and KiB offset of block (rb + q, c): LDS table, or global past it
  auto block_at = [&](int q, int c, uint32_t& off) __attribute__((always_inline)) -> int {
    if (rb + q >= w.NBr) {
      off = 0;
      return 0;
    }
    if (c < kTabG) {
      off = __builtin_amdgcn_readfirstlane(toff[q][c]);
      return __builtin_amdgcn_readfirstlane(tbits[q][c]);
    }
    const int64_t blk = (int64_t)(rb + q) * w.NBc + c;
    off = __builtin_amdgcn_readfirstlane(w.block_offset[blk]);
    return __builtin_amdgcn_readfirstlane(w.bits[blk]);
  };

  // Direct-to-LDS copies of group c into stage st: wavefront w copies rows
  // 16w .. 16w+15 of the x_r tile (rows past M repeat row M - 1; their
  // products are never stored), wavefronts 0 and 1 the group sums, and the
  // two wavefronts of block row q alternate its code chunks.
  auto copy_group = [&](const Stage& st, int c) __attribute__((always_inline)) {
    const int g = lane >> 4, p = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * wave + 4 * i + g;
      const int64_t mrow = min(m0 + row, (int64_t)M - 1);
      const uint16_t* src = xr + mrow * K + (int64_t)c * kBlockCols + 8 * (p ^ (row & 15));
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(st.a + (16 * wave + 4 * i) * 16), 16, 0, 0);
    }
    if (wave < 2) {
      const int64_t mrow = min(m0 + 64 * wave + lane, (int64_t)M - 1);
      __builtin_amdgcn_global_load_lds(xsum + mrow * G + c, (lds_void*)(st.sx + 64 * wave), 4, 0, 0);
    }
    uint32_t off;
    const int b = block_at(wn, c, off);
    const uint8_t* cb = w.codes + (int64_t)off * 1024 + 16 * lane;
#pragma unroll
    for (int t = 0; t < 8; t += 2)
      if (t + wm < b)
        __builtin_amdgcn_global_load_lds(cb + 1024 * (t + wm),
                                         (lds_void*)(st.codes + (wn * 8 + t + wm) * 64), 16, 0, 0);
  };

  // the workgroup's bit map and offsets for the first tabG groups
  for (int i = tid; i < kBR * tabG; i += kThreads) {
    const int q = i / tabG, c = i - (i / tabG) * tabG;
    const int rr = rb + q;
    const int64_t blk = (int64_t)(rr < w.NBr ? rr : 0) * w.NBc + c;
    tbits[q][c] = rr < w.NBr ? w.bits[blk] : 0;
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

  f32x4 acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[mt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one group from stage st with the block's metadata bm
  auto compute = [&](const Stage& st, int c, const BlockMeta& bm) __attribute__((always_inline)) {
    uint32_t unused_off;
    const int b = block_at(wn, c, unused_off);
    if (b == 0) return;
    f32x4 accg[4][4];
    switch (b) {
      case 1: group_mfma<1>(st, wn, apk, accg); break;
      case 2: group_mfma<2>(st, wn, apk, accg); break;
      case 3: group_mfma<3>(st, wn, apk, accg); break;
      case 4: group_mfma<4>(st, wn, apk, accg); break;
      default: group_mfma<8>(st, wn, apk, accg); break;
    }
    // group sums of rows 64 wm + 16 mt + 4 (lane >> 4) + i
    f32x4 sxm[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      sxm[mt] = *reinterpret_cast<const f32x4*>(st.sx + 64 * wm + 16 * mt + 4 * (lane >> 4));
    const float bias = gemm_bias(b);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const float sc = bm.s[rt], szz = -sc * (bias + (float)bm.z[rt]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[mt][rt][i] = fmaf(szz, sxm[mt][i], fmaf(sc, accg[mt][rt][i], acc[mt][rt][i]));
    }
  };
  // own copies done, then the workgroup barrier (no memory fence: the copies
  // are the only producer and their completion is what is waited for)
  auto stage_barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
  };

  BlockMeta cur, nxt;
  copy_group(st0, 0);
  load_meta(w, r, 0, cur);
  stage_barrier();

  for (int c = 0; c < G; c += 2) {
    // group c from stage 0, group c + 1 arriving in stage 1
    if (c + 1 < G) {
      copy_group(st1, c + 1);
      load_meta(w, r, c + 1, nxt);
    }
    compute(st0, c, cur);
    stage_barrier();
    if (c + 1 >= G) break;
    cur = nxt;
    // group c + 1 from stage 1, group c + 2 arriving in stage 0
    if (c + 2 < G) {
      copy_group(st0, c + 2);
      load_meta(w, r, c + 2, nxt);
    }
    compute(st1, c + 1, cur);
    stage_barrier();
    cur = nxt;
  }

  // epilogue: y[m][perm_row[n]]
  if (r >= w.NBr) return;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int64_t row = (int64_t)r * kBlockRows + 16 * rt + (lane & 15);
    int col = w.perm_row[row];
    col = min(max(col, 0), (int)w.N - 1);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + 64 * wm + 16 * mt + 4 * (lane >> 4) + i;
        if (m < M) y[m * w.N + col] = acc[mt][rt][i];
      }
  }
}

}  // namespace

size_t gemm_workspace_bytes(int64_t M, int64_t K) {
  const size_t xr = (size_t)M * K * 2;
  const size_t xr_al = (xr + 255) & ~(size_t)255;
  return xr_al + (size_t)M * (K / kBlockCols) * 4;
}

hipError_t launch_gemm(const uint16_t* x, int64_t M, const WeightView& w, float* y,
                       void* workspace, hipStream_t stream) {
  const int64_t K = w.K;
  uint16_t* xr = reinterpret_cast<uint16_t*>(workspace);
  const size_t xr_bytes = (((size_t)M * K * 2) + 255) & ~(size_t)255;
  float* xsum = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(workspace) + xr_bytes);
  const size_t row_bytes = (size_t)K * 2;
  const int staged = row_bytes <= kGatherMaxLds;
  hipLaunchKernelGGL(k_gather_x, dim3((unsigned)M), dim3(kGatherThreads), staged ? row_bytes : 0,
                     stream, x, K, w.perm_col, xr, xsum, staged);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((M + kBM - 1) / kBM), (unsigned)((w.NBr + kBR - 1) / kBR));
  hipLaunchKernelGGL(k_gemm, grid, dim3(kThreads), 0, stream, xr, xsum, (int)M, w, y);
  return hipGetLastError();
}

}  // namespace msq

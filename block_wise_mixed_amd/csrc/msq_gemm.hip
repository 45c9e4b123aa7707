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
// Workgroup tile: kBM rows of x_r x kBR block rows (64 outputs each), four
// wavefronts (wm, wn) = (wave & 1, wave >> 1) of 64 rows x two block rows,
// one wavefront per SIMD with the whole register file (two blocks of fp32
// accumulators plus the per-group ones).  Per 128-wide K group c:
//   - while group c is multiplied, the next group's x_r tile (kBM x 128 bf16)
//     is loaded into registers, wavefront w loads the codes of the
//     workgroup's w-th block, and every wavefront loads the scales and zero
//     points of its two blocks (software pipelining, one group ahead);
//   - group c: the x_r tile and the codes are in LDS buffer c % 2; per block
//     the wavefront copies the code chunks to registers; per k-step of 32 it
//     reads its 4 A fragments from LDS, unpacks 4 B fragments to exact bf16
//     (128 + q; 3-bit: two planes with bias 256; 8-bit: low 7 bits and top
//     bit, bias 384), and issues 16 v_mfma_f32_16x16x32_bf16 into the group
//     accumulators;
//   - fold: acc += s_n * acc_g - s_n * (bias + z_n) * sum_x[m][c];
//   - the prefetched tile and codes go to LDS buffer (c + 1) % 2; one barrier.
// 0-bit blocks skip the products.  y is scattered to original rows through
// perm_row.
constexpr int kBM = 128;
constexpr int kBR = 4;
constexpr int kWaves = 4;
constexpr int kWaveBR = kBR / 2;  // block rows per wavefront
constexpr int kThreads = kWaves * 64;
constexpr int kAStride = kBlockCols + 8;  // bf16 per LDS row of the A tile: +16 bytes against bank conflicts
constexpr int kAPieces = kBM * kBlockCols / 8 / kThreads;  // 16-byte pieces per thread per tile

// Unpacked B operand of fragment F of a B-bit block (low plane for 3- and 8-bit).
template <int B, int F>
__device__ __forceinline__ bf16x8 gemm_b_lo(const uint4 (&ch)[8]) {
  if constexpr (B == 8) return exp_lo<8, F>(ch[F / 2]);
  else return block_operand<B, F>(ch);
}

template <int B, int F>
__device__ __forceinline__ bf16x8 gemm_b_hi(const uint4 (&ch)[8]) {
  if constexpr (B == 8) return exp_hi<8, F>(ch[F / 2]);
  else return hi3_operand<F>(ch);
}

__host__ __device__ constexpr float gemm_bias(int b) {
  return b == 8 ? 384.f : (b == 3 ? 256.f : 128.f);
}

// acc_g = A . B for one B-bit block: 4 k-steps x 4 row tiles x 4 m tiles.
template <int B>
__device__ __forceinline__ void group_mfma(const uint16_t* __restrict__ As, int wm,
                                           const uint4 (&ch)[8], f32x4 (&accg)[4][4]) {
  const int lane = threadIdx.x & 63;
  auto kstep = [&](auto KTc) {
    constexpr int kt = decltype(KTc)::value;
    bf16x8 A[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int row = 64 * wm + 16 * mt + (lane & 15);
      A[mt] = as_bf16x8(*reinterpret_cast<const uint4*>(As + row * kAStride + 32 * kt +
                                                        8 * (lane >> 4)));
    }
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

// Eight chunks held in named members (not an array): the compiler keeps
// these in registers even when loads and uses sit in different branches.
struct Chunks8 {
  uint4 c0, c1, c2, c3, c4, c5, c6, c7;
};

// This lane's 16 bytes of chunks 0..7 of a block at base, chunk t read from
// chunk min(t, last): all eight registers are always written (past the
// block's b chunks they repeat its last one, which the caches serve).
__device__ __forceinline__ Chunks8 load_chunks(const uint8_t* base, int last) {
  Chunks8 k;
  k.c0 = *reinterpret_cast<const uint4*>(base);
  k.c1 = *reinterpret_cast<const uint4*>(base + 1024 * min(1, last));
  k.c2 = *reinterpret_cast<const uint4*>(base + 1024 * min(2, last));
  k.c3 = *reinterpret_cast<const uint4*>(base + 1024 * min(3, last));
  k.c4 = *reinterpret_cast<const uint4*>(base + 1024 * min(4, last));
  k.c5 = *reinterpret_cast<const uint4*>(base + 1024 * min(5, last));
  k.c6 = *reinterpret_cast<const uint4*>(base + 1024 * min(6, last));
  k.c7 = *reinterpret_cast<const uint4*>(base + 1024 * min(7, last));
  return k;
}

constexpr int kTabG = 512;  // groups whose bit map and offsets are staged in LDS

// LDS of k_gemm: two buffers of the x_r tile and its group sums, two buffers
// of the workgroup's kBR blocks' codes (8 KiB per block), and the bit map and
// block offsets of the workgroup's block rows for the first kTabG groups.
struct GemmLds {
  uint16_t a[2][kBM * kAStride];
  float sx[2][kBM];
  uint4 codes[2][kBR][8][64];
  uint32_t off[kBR][kTabG];
  uint8_t bits[kBR][kTabG];
};

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1))) void k_gemm(
    const uint16_t* __restrict__ xr, const float* __restrict__ xsum, int M, WeightView w,
    float* __restrict__ y) {
  __shared__ GemmLds L;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t m0 = (int64_t)blockIdx.x * kBM;
  const int rb = blockIdx.y * kBR;     // first block row of the workgroup
  const int r0 = rb + kWaveBR * wn;    // first block row of this wavefront
  const int rs = rb + wave;            // block row whose codes this wavefront stages
  const int64_t K = w.K;
  const int G = w.NBc;
  const int tabG = min(G, kTabG);

  // bitwidth and KiB offset of block (rb + q, c): LDS table, or global past it
  auto block_at = [&](int q, int c, uint32_t& off) __attribute__((always_inline)) -> int {
    const int r = rb + q;
    if (r >= w.NBr) {
      off = 0;
      return 0;
    }
    if (c < kTabG) {
      off = __builtin_amdgcn_readfirstlane(L.off[q][c]);
      return __builtin_amdgcn_readfirstlane(L.bits[q][c]);
    }
    const int64_t blk = (int64_t)r * w.NBc + c;
    off = __builtin_amdgcn_readfirstlane(w.block_offset[blk]);
    return __builtin_amdgcn_readfirstlane(w.bits[blk]);
  };

  // x_r tile loads of group c into registers (zeros past row M)
  auto load_tile = [&](int c, uint4 (&v)[kAPieces], float& sx) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kAPieces; ++i) {
      const int piece = tid + kThreads * i;
      const int row = piece >> 4, seg = piece & 15;
      v[i] = uint4{0u, 0u, 0u, 0u};
      if (m0 + row < M)
        v[i] = *reinterpret_cast<const uint4*>(xr + (m0 + row) * K + (int64_t)c * kBlockCols + 8 * seg);
    }
    sx = 0.f;
    if (tid < kBM && m0 + tid < M) sx = xsum[(m0 + tid) * G + c];
  };
  // codes of the staged block of group c; nothing is read for a 0-bit block
  // (its offset is the MSQ_NO_BLOCK sentinel, and an all-pruned matrix has
  // no code buffer at all)
  auto load_staged = [&](int c) __attribute__((always_inline)) -> Chunks8 {
    uint32_t off;
    const int b = block_at(wave, c, off);
    Chunks8 k = {};
    if (b != 0) k = load_chunks(w.codes + (int64_t)off * 1024 + 16 * lane, b - 1);
    return k;
  };
  auto store_stage = [&](int buf, const uint4 (&v)[kAPieces], float sx,
                         const Chunks8& k) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kAPieces; ++i) {
      const int piece = tid + kThreads * i;
      const int row = piece >> 4, seg = piece & 15;
      *reinterpret_cast<uint4*>(&L.a[buf][row * kAStride + 8 * seg]) = v[i];
    }
    if (tid < kBM) L.sx[buf][tid] = sx;
    uint4* dst = L.codes[buf][wave][0] + lane;
    dst[0] = k.c0;
    dst[64] = k.c1;
    dst[128] = k.c2;
    dst[192] = k.c3;
    dst[256] = k.c4;
    dst[320] = k.c5;
    dst[384] = k.c6;
    dst[448] = k.c7;
  };

  // the workgroup's bit map and offsets for the first tabG groups
  for (int i = tid; i < kBR * tabG; i += kThreads) {
    const int q = i / tabG, c = i - (i / tabG) * tabG;
    const int r = rb + q;
    const int64_t blk = (int64_t)(r < w.NBr ? r : 0) * w.NBc + c;
    L.bits[q][c] = r < w.NBr ? w.bits[blk] : 0;
    L.off[q][c] = r < w.NBr ? w.block_offset[blk] : 0u;
  }
  __syncthreads();

  f32x4 acc[kWaveBR][4][4];
#pragma unroll
  for (int q = 0; q < kWaveBR; ++q)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[q][mt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};

  BlockMeta cur[kWaveBR], nxt[kWaveBR];
  {
    uint4 v[kAPieces];
    float sx;
    load_tile(0, v, sx);
    const Chunks8 k = load_staged(0);
#pragma unroll
    for (int q = 0; q < kWaveBR; ++q) load_meta(w, r0 + q, 0, cur[q]);
    store_stage(0, v, sx, k);
  }
  __syncthreads();

  for (int c = 0; c < G; ++c) {
    const int buf = c & 1;
    const bool more = c + 1 < G;
    uint4 v[kAPieces];
    Chunks8 nk;
    float sx = 0.f;
    if (more) {
      load_tile(c + 1, v, sx);
      nk = load_staged(c + 1);
#pragma unroll
      for (int q = 0; q < kWaveBR; ++q) load_meta(w, r0 + q, c + 1, nxt[q]);
    }
#pragma unroll
    for (int q = 0; q < kWaveBR; ++q) {
      uint32_t unused_off;
      const int b = block_at(kWaveBR * wn + q, c, unused_off);
      if (b == 0) continue;
      // only the first b chunks are meaningful; reading all eight with
      // static indices keeps the array in registers
      uint4 ch[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) ch[t] = L.codes[buf][kWaveBR * wn + q][t][lane];
      f32x4 accg[4][4];
      switch (b) {
        case 1: group_mfma<1>(L.a[buf], wm, ch, accg); break;
        case 2: group_mfma<2>(L.a[buf], wm, ch, accg); break;
        case 3: group_mfma<3>(L.a[buf], wm, ch, accg); break;
        case 4: group_mfma<4>(L.a[buf], wm, ch, accg); break;
        default: group_mfma<8>(L.a[buf], wm, ch, accg); break;
      }
      const float bias = gemm_bias(b);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const float s = cur[q].s[rt], szz = -s * (bias + (float)cur[q].z[rt]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float sxm = L.sx[buf][64 * wm + 16 * mt + 4 * (lane >> 4) + i];
            acc[q][mt][rt][i] = fmaf(szz, sxm, fmaf(s, accg[mt][rt][i], acc[q][mt][rt][i]));
          }
      }
    }
    if (more) {
      store_stage(buf ^ 1, v, sx, nk);
#pragma unroll
      for (int q = 0; q < kWaveBR; ++q) cur[q] = nxt[q];
    }
    __syncthreads();
  }

  // epilogue: y[m][perm_row[n]]
#pragma unroll
  for (int q = 0; q < kWaveBR; ++q) {
    const int r = r0 + q;
    if (r >= w.NBr) continue;
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
          if (m < M) y[m * w.N + col] = acc[q][mt][rt][i];
        }
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

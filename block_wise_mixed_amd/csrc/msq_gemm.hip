// Prefill GEMM for gfx950: y = x . W^T for any M (used for M > 64), W
// dequantized on the fly from packed format v1 and multiplied on the bf16
// matrix cores.
//
// Two kernels:
//   k_gather_x : x_r[m][j] = x[m][perm_col[j]] (bf16) and the per-group sums
//                sum_j x_r[m][j] over each 128-column group (fp32), written to
//                the workspace once per call (the activation reordering of the
//                "SFMP" abstract).
//   k_gemm     : workgroup tile 128 (M) x 128 (N = two block rows), four
//                wavefronts of 64 x 64.  Per 128-wide K group: the x_r tile is
//                staged in LDS, each wavefront unpacks its block's codes to
//                exact bf16 operands (128 + q), runs 16 v_mfma_f32_16x16x32_bf16
//                per 16x16 output tile group into a per-group accumulator, and
//                folds scale and zero point in fp32:
//                    acc += s_n * (acc_g - (bias + z_n) * sum_x[m]).
//                0-bit blocks are skipped.  y is scattered to original rows
//                through perm_row.
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

constexpr int kBM = 128, kThreads = 256;
constexpr int kLdsStride = kBlockCols + 8;  // bf16 elements per LDS row (pad: 16 bytes)

__device__ __forceinline__ float bf16f(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

// 1-D grid of M * ceil(G / 4) workgroups; wavefront w of workgroup
// (m, quad) handles group 4*quad + w of row m.
__global__ __launch_bounds__(256) void k_gather_x(const uint16_t* __restrict__ x, int64_t K,
                                                  const int32_t* __restrict__ perm_col,
                                                  uint16_t* __restrict__ xr,
                                                  float* __restrict__ xsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t G = K / kBlockCols;
  const int64_t quads = (G + 3) / 4;
  const int64_t m = blockIdx.x / quads;
  const int64_t g = (blockIdx.x % quads) * 4 + wave;
  if (g >= G) return;
  const int64_t j = g * kBlockCols + 2 * lane;
  int p0 = perm_col[j], p1 = perm_col[j + 1];
  p0 = min(max(p0, 0), (int)K - 1);
  p1 = min(max(p1, 0), (int)K - 1);
  const uint16_t u0 = x[m * K + p0], u1 = x[m * K + p1];
  *reinterpret_cast<uint32_t*>(xr + m * K + j) = (uint32_t)u0 | ((uint32_t)u1 << 16);
  float s = bf16f(u0) + bf16f(u1);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
  if (lane == 0) xsum[m * G + g] = s;
}

template <int B>
__device__ __forceinline__ void wave_group_mac(const uint8_t* __restrict__ base,
                                               const uint16_t* __restrict__ As, int wm,
                                               f32x4 (&accg)[4][4]) {
  const int lane = threadIdx.x & 63;
  uint4 ch[B];
#pragma unroll
  for (int t = 0; t < B; ++t) ch[t] = *reinterpret_cast<const uint4*>(base + 1024 * t);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) accg[mt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto kstep = [&](auto KTc) {
    constexpr int kt = decltype(KTc)::value;
    bf16x8 A[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int row = 64 * wm + 16 * mt + (lane & 15);
      A[mt] = as_bf16x8(*reinterpret_cast<const uint4*>(As + row * kLdsStride + 32 * kt +
                                                        8 * (lane >> 4)));
    }
    auto rstep = [&](auto RTc) {
      constexpr int rt = decltype(RTc)::value;
      constexpr int F = 4 * rt + kt;
      const bf16x8 bop = block_operand<B, F>(ch);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) accg[mt][rt] = mfma_bf16(A[mt], bop, accg[mt][rt]);
      if constexpr (B == 3) {
        const bf16x8 hop = hi3_operand<F>(ch);
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

__global__ __launch_bounds__(kThreads) void k_gemm(const uint16_t* __restrict__ xr,
                                                   const float* __restrict__ xsum, int M,
                                                   WeightView w, float* __restrict__ y) {
  __shared__ __align__(16) uint16_t As[kBM * kLdsStride];
  __shared__ float Sx[kBM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t m0 = (int64_t)blockIdx.x * kBM;
  const int r = blockIdx.y * 2 + wn;  // block row of this wavefront
  const bool rvalid = r < w.NBr;      // odd N/64: the last workgroup has one block row
  const int64_t K = w.K;
  const int G = w.NBc;

  f32x4 acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[mt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int c = 0; c < G; ++c) {
    // stage x_r[m0 .. m0+127][128c .. 128c+127]: 2048 16-byte pieces, 8 per thread
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int piece = tid + kThreads * i;
      const int row = piece >> 4, seg = piece & 15;
      uint4 v = {0u, 0u, 0u, 0u};
      if (m0 + row < M)
        v = *reinterpret_cast<const uint4*>(xr + (m0 + row) * K + (int64_t)c * kBlockCols + 8 * seg);
      *reinterpret_cast<uint4*>(As + row * kLdsStride + 8 * seg) = v;
    }
    if (tid < kBM) Sx[tid] = (m0 + tid < M) ? xsum[(m0 + tid) * G + c] : 0.f;
    __syncthreads();

    const int64_t blk = (int64_t)r * G + c;
    const int b = rvalid ? __builtin_amdgcn_readfirstlane(w.bits[blk]) : 0;
    if (b != 0) {
      const uint32_t off = __builtin_amdgcn_readfirstlane(w.block_offset[blk]);
      const uint8_t* base = w.codes + (int64_t)off * 1024 + 16 * lane;
      f32x4 accg[4][4];
      switch (b) {
        case 1: wave_group_mac<1>(base, As, wm, accg); break;
        case 2: wave_group_mac<2>(base, As, wm, accg); break;
        case 3: wave_group_mac<3>(base, As, wm, accg); break;
        case 4: wave_group_mac<4>(base, As, wm, accg); break;
        default: wave_group_mac<8>(base, As, wm, accg); break;
      }
      const float bias = (float)unpack_bias(b);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int n = 16 * rt + (lane & 15);
        const float s = w.scale[blk * kBlockRows + n];
        const float zz = bias + (float)w.zero[blk * kBlockRows + n];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float sx = Sx[64 * wm + 16 * mt + 4 * (lane >> 4) + i];
            acc[mt][rt][i] += s * (accg[mt][rt][i] - zz * sx);
          }
      }
    }
    __syncthreads();
  }

  // epilogue: y[m][perm_row[n]]
  if (!rvalid) return;
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
  const int64_t K = w.K, G = K / kBlockCols;
  uint16_t* xr = reinterpret_cast<uint16_t*>(workspace);
  const size_t xr_bytes = (((size_t)M * K * 2) + 255) & ~(size_t)255;
  float* xsum = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(workspace) + xr_bytes);
  hipLaunchKernelGGL(k_gather_x, dim3((unsigned)(M * ((G + 3) / 4))), dim3(256), 0, stream, x, K,
                     w.perm_col, xr, xsum);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((M + kBM - 1) / kBM), (unsigned)((w.NBr + 1) / 2));
  hipLaunchKernelGGL(k_gemm, grid, dim3(kThreads), 0, stream, xr, xsum, (int)M, w, y);
  return hipGetLastError();
}

}  // namespace msq

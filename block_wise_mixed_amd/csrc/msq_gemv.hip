// Decode GEMV for gfx950: y = x . W^T for M <= 64, W dequantized block by
// block from packed format v1 in registers.  Memory-bound: every byte of the
// packed codes is read once, with one 16-byte load per lane per 1 KiB chunk.
//
// Work split: workgroup = 4 wavefronts on one block row r (64 output rows)
// and a range of block columns [c0, c1) (a K split).  The workgroup first
// gathers its slice of the activations through perm_col into LDS (the
// activation reordering of the "SFMP" abstract) together with the per-group
// sums of x used to fold the zero point.  Each wavefront then walks every
// fourth block column of the range: loads the block's b chunks, unpacks each
// 16x32 fragment into exact bf16 operands and runs v_mfma_f32_16x16x32_bf16
// (M padded to 16 per tile), then folds scale and zero point per row:
//     y[row] += s * (sum_k (bias + q_k) x_k - (bias + z) * sum_k x_k).
// The four wavefronts reduce through LDS in a fixed order.  One K split writes
// y directly (scattered to original rows through perm_row); several splits
// write fp32 partials that k_gemv_reduce sums in split order, so results are
// bitwise reproducible.
//
// Per-block precision and block layout: "ScaleBITS" summary page, section
// Approach; RTN-g128 dequantization s * (q - z): section Limitations.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "msq_dequant.h"
#include "msq_internal.h"

namespace msq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr size_t kLdsBudget = 64 * 1024;

// Multiply-accumulate one B-bit block into acc[mt][rt] (16 fragments F = 4*rt + kt).
template <int B, int MT>
__device__ __forceinline__ void block_mac(const uint8_t* __restrict__ base,
                                          const bf16x8 (&A)[MT][4], f32x4 (&acc)[MT][4]) {
  uint4 ch[B];
#pragma unroll
  for (int t = 0; t < B; ++t) ch[t] = *reinterpret_cast<const uint4*>(base + 1024 * t);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[mt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto step = [&](auto Fc) {
    constexpr int F = decltype(Fc)::value;
    constexpr int rt = F / 4, kt = F % 4;
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

template <int MT>
__device__ __forceinline__ void dispatch_block(int b, const uint8_t* base, const bf16x8 (&A)[MT][4],
                                               f32x4 (&acc)[MT][4]) {
  switch (b) {
    case 1: block_mac<1, MT>(base, A, acc); break;
    case 2: block_mac<2, MT>(base, A, acc); break;
    case 3: block_mac<3, MT>(base, A, acc); break;
    case 4: block_mac<4, MT>(base, A, acc); break;
    default: block_mac<8, MT>(base, A, acc); break;
  }
}

__device__ __forceinline__ float bf16f(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

// Original row of reordered row i, clamped into [0, N) so that even an
// unvalidated permutation cannot send a store out of bounds.
__device__ __forceinline__ int64_t orig_row(const int32_t* perm_row, int64_t i, int64_t N) {
  const int64_t v = perm_row[i];
  return v < 0 ? 0 : (v >= N ? N - 1 : v);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

// Gather x[m][perm_col[128*c + j]] for the workgroup's block columns into LDS
// (bf16, [M][kr*128]) and the per-group sums into xsum ([M][kr], fp32).
__device__ __forceinline__ void gather_x(const uint16_t* __restrict__ x, int M, int64_t K,
                                         const int32_t* __restrict__ perm_col, int c0, int ncl,
                                         int kr, uint16_t* xs, float* xsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ngroups = M * ncl;
  for (int gi = wave; gi < ngroups; gi += kWaves) {
    const int m = gi / ncl, cl = gi % ncl;
    const int64_t j = (int64_t)(c0 + cl) * kBlockCols + 2 * lane;
    int p0 = perm_col[j], p1 = perm_col[j + 1];
    p0 = min(max(p0, 0), (int)K - 1);
    p1 = min(max(p1, 0), (int)K - 1);
    const uint16_t u0 = x[(int64_t)m * K + p0], u1 = x[(int64_t)m * K + p1];
    *reinterpret_cast<uint32_t*>(xs + (size_t)m * kr * kBlockCols + cl * kBlockCols + 2 * lane) =
        (uint32_t)u0 | ((uint32_t)u1 << 16);
    const float s = wave_sum(bf16f(u0) + bf16f(u1));
    if (lane == 0) xsum[m * kr + cl] = s;
  }
}

// A operand of k-step kt for the 16-row tile mt: x rows 16*mt + (l & 15),
// columns 32*kt + 8*(l >> 4) .. +7 of block column cl; zero for rows >= M.
template <int MT>
__device__ __forceinline__ void load_a(const uint16_t* xs, int M, int kr, int cl, bool m1,
                                       bf16x8 (&A)[MT][4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = 16 * mt + (lane & 15);
    const bool live = m1 ? ((lane & 15) == 0) : (m < M);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      uint4 v = {0u, 0u, 0u, 0u};
      if (live)
        v = *reinterpret_cast<const uint4*>(xs + (size_t)(m1 ? 0 : m) * kr * kBlockCols +
                                            cl * kBlockCols + 32 * kt + 8 * (lane >> 4));
      A[mt][kt] = as_bf16x8(v);
    }
  }
}

// Route lane (l & 15) of acc[rt][0] (row 16*rt + l of the block, valid in
// lanes 0..15 when only x row 0 is live) to lane 16*rt + (l & 15).
__device__ __forceinline__ float rows_to_lanes(const f32x4 (&acc)[1][4]) {
  uint32_t v0 = __float_as_uint(acc[0][0][0]), v1 = __float_as_uint(acc[0][1][0]);
  uint32_t v2 = __float_as_uint(acc[0][2][0]), v3 = __float_as_uint(acc[0][3][0]);
  // odd 16-lane rows of the first operand <-> even rows of the second
  auto p01 = __builtin_amdgcn_permlane16_swap(v0, v1, false, false);
  auto p23 = __builtin_amdgcn_permlane16_swap(v2, v3, false, false);
  // upper 32 lanes of the first operand <-> lower 32 lanes of the second
  auto q = __builtin_amdgcn_permlane32_swap(p01[0], p23[0], false, false);
  return __uint_as_float(q[0]);
}

template <int MT, bool M1>
__global__ __launch_bounds__(kThreads) void k_gemv(const uint16_t* __restrict__ x, int M,
                                                   WeightView w, int split, int kr,
                                                   float* __restrict__ out, int direct) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = blockIdx.x / split, sp = blockIdx.x % split;
  const int c0 = sp * kr;
  const int c1 = min(w.NBc, c0 + kr);
  const int ncl = c1 - c0;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  float* xsum = reinterpret_cast<float*>(smem + (size_t)M * kr * kBlockCols * 2);

  gather_x(x, M, w.K, w.perm_col, c0, ncl, kr, xs, xsum);
  __syncthreads();

  f32x4 yacc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) yacc[mt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float y1 = 0.f;

  for (int cl = wave; cl < ncl; cl += kWaves) {
    const int64_t blk = (int64_t)r * w.NBc + c0 + cl;
    const int b = __builtin_amdgcn_readfirstlane(w.bits[blk]);
    if (b == 0) continue;
    const uint32_t off = __builtin_amdgcn_readfirstlane(w.block_offset[blk]);
    const uint8_t* base = w.codes + (int64_t)off * 1024 + 16 * lane;
    const float bias = (float)unpack_bias(b);

    bf16x8 A[MT][4];
    load_a<MT>(xs, M, kr, cl, M1, A);
    f32x4 acc[MT][4];
    dispatch_block<MT>(b, base, A, acc);

    if constexpr (M1) {
      const float v = rows_to_lanes(acc);
      const float s = w.scale[blk * kBlockRows + lane];
      const float zz = bias + (float)w.zero[blk * kBlockRows + lane];
      y1 += s * (v - zz * xsum[cl]);
    } else {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int n = 16 * rt + (lane & 15);
        const float s = w.scale[blk * kBlockRows + n];
        const float zz = bias + (float)w.zero[blk * kBlockRows + n];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = 16 * mt + 4 * (lane >> 4) + i;
            const float sx = m < M ? xsum[m * kr + cl] : 0.f;
            yacc[mt][rt][i] += s * (acc[mt][rt][i] - zz * sx);
          }
      }
    }
  }

  // Reduce the four wavefronts in a fixed order (wave 0 + 1 + 2 + 3).
  __syncthreads();  // LDS is reused below
  float* red = reinterpret_cast<float*>(smem);
  if constexpr (M1) {
    if (wave > 0) red[(wave - 1) * 64 + lane] = y1;
    __syncthreads();
    if (wave == 0) {
      float v = y1 + red[lane];
      v += red[64 + lane];
      v += red[128 + lane];
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
            float v = yacc[mt][rt][i] + red[m * kBlockRows + n];
            v += red[plane + m * kBlockRows + n];
            v += red[2 * plane + m * kBlockRows + n];
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

// y[m][perm_row[n]] = sum over splits (in order) of partial[sp][m][n].
__global__ __launch_bounds__(256) void k_gemv_reduce(const float* __restrict__ part, int split,
                                                     int M, int64_t N,
                                                     const int32_t* __restrict__ perm_row,
                                                     float* __restrict__ y) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)M * N) return;
  const int64_t m = idx / N, n = idx % N;
  float v = 0.f;
  for (int sp = 0; sp < split; ++sp) v += part[((int64_t)sp * M + m) * N + n];
  y[m * N + orig_row(perm_row, n, N)] = v;
}

template <int MT, bool M1>
hipError_t launch_mt(const uint16_t* x, int M, const WeightView& w, float* dst,
                     const GemvPlan& p, int direct, hipStream_t stream) {
  const unsigned grid = (unsigned)(w.NBr * p.split);
  hipLaunchKernelGGL((k_gemv<MT, M1>), dim3(grid), dim3(kThreads), p.lds_bytes, stream, x, M, w,
                     p.split, p.kr, dst, direct);
  return hipGetLastError();
}

}  // namespace

GemvPlan plan_gemv(int64_t M, int64_t N, int64_t K) {
  GemvPlan p{};
  const int NBr = (int)(N / kBlockRows), NBc = (int)(K / kBlockCols);
  p.mt = (int)((M + 15) / 16);
  const size_t per_col = (size_t)M * (kBlockCols * 2 + 4);
  int kr_max = (int)(kLdsBudget / (per_col > 0 ? per_col : 1));
  if (kr_max < 1) kr_max = 1;
  // Aim for ~1024 workgroups (16 wavefronts per CU) while keeping at least
  // two blocks per wavefront.
  int split = (1024 + NBr - 1) / NBr;
  int max_split = NBc / (2 * kWaves);
  if (max_split < 1) max_split = 1;
  if (split > max_split) split = max_split;
  if (split < 1) split = 1;
  int kr = (NBc + split - 1) / split;
  if (kr > kr_max) kr = kr_max;
  split = (NBc + kr - 1) / kr;
  p.split = split;
  p.kr = kr;
  const size_t x_bytes = (size_t)M * kr * (kBlockCols * 2 + 4);
  const size_t red_bytes = (size_t)(kWaves - 1) * (size_t)(M > 1 ? M : 1) * kBlockRows * 4;
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
    e = launch_mt<1, true>(x, 1, w, dst, p, direct, stream);
  } else {
    switch (p.mt) {
      case 1: e = launch_mt<1, false>(x, (int)M, w, dst, p, direct, stream); break;
      case 2: e = launch_mt<2, false>(x, (int)M, w, dst, p, direct, stream); break;
      case 3: e = launch_mt<3, false>(x, (int)M, w, dst, p, direct, stream); break;
      default: e = launch_mt<4, false>(x, (int)M, w, dst, p, direct, stream); break;
    }
  }
  if (e != hipSuccess || direct) return e;
  const int64_t total = M * w.N;
  hipLaunchKernelGGL(k_gemv_reduce, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                     reinterpret_cast<const float*>(workspace), p.split, (int)M, w.N, w.perm_row, y);
  return hipGetLastError();
}

}  // namespace msq

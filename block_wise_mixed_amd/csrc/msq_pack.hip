// Quantize-and-pack kernels for gfx950.
//
//   k_block_offsets : exclusive prefix sum of the block bit map over the packed
//                     order (segments b = 1,2,3,4,8; row-major inside), in KiB.
//   k_pack          : one workgroup per 64x128 block: gather the reordered
//                     block from W through perm_row / perm_col, compute one
//                     asymmetric RTN-g128 scale and zero point per row, and
//                     write the block's codes in packed format v1.
//
// Precision per 64x128 block after two-way reordering: "ScaleBITS" summary
// page, section Approach.  RTN with group size 128: same page, section
// Limitations.  Compact buffers reused by the kernel: "TileQuant" abstract.
// The quantizer and the bit layout are spelled out in include/msq.h; every
// fp32 operation below is IEEE single precision, rounded once per operation
// (no contraction, denormals preserved, correctly rounded division), so the
// results are bit-identical to any other implementation of that definition.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msq_internal.h"

#pragma clang fp contract(off)

namespace msq {
namespace {

// Position of a bitwidth in the packed segment order, or -1 for 0 bits.
__device__ __forceinline__ int segment_of(int b) {
  switch (b) {
    case 1: return 0;
    case 2: return 1;
    case 3: return 2;
    case 4: return 3;
    case 8: return 4;
    case 16: return 5;
    default: return -1;
  }
}

constexpr int kScanThreads = 1024;
constexpr int kSegs = 6;
__constant__ int kSegBits[kSegs] = {1, 2, 3, 4, 8, 16};

// One workgroup.  Thread t owns a contiguous run of the row-major block list,
// counts the blocks of each bitwidth in it, and after a workgroup-wide
// exclusive scan of those counts assigns offset = segment base + b * rank.
__global__ __launch_bounds__(kScanThreads) void k_block_offsets(const uint8_t* __restrict__ bits,
                                                                int64_t nblk,
                                                                uint32_t* __restrict__ off) {
  __shared__ uint32_t wave_tot[kSegs][kScanThreads / 64];
  __shared__ uint32_t seg_base[kSegs];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t per = (nblk + kScanThreads - 1) / kScanThreads;
  const int64_t beg = (int64_t)tid * per;
  const int64_t end = beg + per < nblk ? beg + per : nblk;

  uint32_t cnt[kSegs] = {0, 0, 0, 0, 0, 0};
  for (int64_t i = beg; i < end; ++i) {
    int k = segment_of(bits[i]);
    if (k >= 0) cnt[k]++;
  }
  // inclusive scan inside the wave, per segment
  uint32_t incl[kSegs];
#pragma unroll
  for (int k = 0; k < kSegs; ++k) {
    uint32_t v = cnt[k];
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      uint32_t u = __shfl_up(v, d, 64);
      if (lane >= d) v += u;
    }
    incl[k] = v;
    if (lane == 63) wave_tot[k][wave] = v;
  }
  __syncthreads();
  if (tid < kSegs) {
    // scan of wave totals for segment tid, kept in place as exclusive prefixes
    uint32_t run = 0;
    for (int w = 0; w < kScanThreads / 64; ++w) {
      uint32_t t = wave_tot[tid][w];
      wave_tot[tid][w] = run;
      run += t;
    }
    seg_base[tid] = run;  // total count for now
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t acc = 0;
    for (int k = 0; k < kSegs; ++k) {
      uint32_t total = seg_base[k];
      seg_base[k] = acc;
      acc += (uint32_t)kSegBits[k] * total;
    }
  }
  __syncthreads();
  uint32_t rank[kSegs];
#pragma unroll
  for (int k = 0; k < kSegs; ++k) rank[k] = wave_tot[k][wave] + incl[k] - cnt[k];
  for (int64_t i = beg; i < end; ++i) {
    const int b = bits[i];
    const int k = segment_of(b);
    if (k < 0) {
      off[i] = kNoBlock;
    } else {
      off[i] = seg_base[k] + (uint32_t)b * rank[k];
      rank[k]++;
    }
  }
}

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float((uint32_t)u << 16);
}

// Code of one weight: clamp(rint(w / s) + z, 0, qmax); 0 when s == 0.
__device__ __forceinline__ uint32_t rtn_code(float w, float s, float z, float qmax) {
  if (!(s > 0.0f)) return 0u;
  float t = __builtin_rintf(w / s) + z;
  t = fminf(fmaxf(t, 0.0f), qmax);
  return (uint32_t)t;
}

constexpr int kPackThreads = 256;

// One workgroup per block.  The block's 64 x 128 reordered weights are
// gathered into LDS (perm_row picks the row, perm_col the column), each row's
// scale and zero point are computed from that row's 128 values, then every
// thread assembles whole 32-bit words of the packed block so the global
// stores are coalesced.
__global__ __launch_bounds__(kPackThreads) void k_pack(
    const uint16_t* __restrict__ W, int64_t N, int64_t K, const uint8_t* __restrict__ bits,
    const int32_t* __restrict__ perm_row, const int32_t* __restrict__ perm_col,
    const uint32_t* __restrict__ offsets, uint8_t* __restrict__ codes, int64_t code_bytes,
    float* __restrict__ scale, uint8_t* __restrict__ zero) {
  __shared__ float tile[kBlockRows][kBlockCols + 1];
  __shared__ int cols[kBlockCols];
  __shared__ int64_t rows[kBlockRows];
  __shared__ float row_s[kBlockRows];
  __shared__ float row_z[kBlockRows];

  const int NBc = (int)(K / kBlockCols);
  const int64_t blk = blockIdx.x;
  const int r = (int)(blk / NBc), c = (int)(blk % NBc);
  int b = bits[blk];
  const int tid = threadIdx.x;
  // a bitwidth outside the format, or a block that would end past the codes
  // buffer (a descriptor msq_plan did not size), is written as pruned
  const uint32_t off = offsets[blk];
  if (segment_of(b) < 0 || off == kNoBlock || ((int64_t)off + b) * 1024 > code_bytes) b = 0;

  if (b == 0) {
    if (tid < kBlockRows) {
      scale[blk * kBlockRows + tid] = 0.0f;
      zero[blk * kBlockRows + tid] = 0;
    }
    return;
  }
  // Indices are clamped so that even an unvalidated permutation cannot read
  // outside W; validated permutations are unaffected.
  if (tid < kBlockCols) {
    int pc = perm_col[(int64_t)c * kBlockCols + tid];
    cols[tid] = pc < 0 ? 0 : (pc >= K ? (int)(K - 1) : pc);
  }
  if (tid < kBlockRows) {
    int pr = perm_row[(int64_t)r * kBlockRows + tid];
    pr = pr < 0 ? 0 : (pr >= N ? (int)(N - 1) : pr);
    rows[tid] = (int64_t)pr * K;
  }
  __syncthreads();
  for (int e = tid; e < kBlockRows * kBlockCols; e += kPackThreads) {
    const int ib = e >> 7, jb = e & 127;
    tile[ib][jb] = bf16_to_f32(W[rows[ib] + cols[jb]]);
  }
  __syncthreads();

  // 16-bit block: the bf16 bit patterns themselves (the tile holds them
  // exactly as fp32), one fragment per chunk: word w is chunk F = w >> 8,
  // lane l, dword d, halves h = 0, 1; scale and zero point 0.
  if (b == 16) {
    if (tid < kBlockRows) {
      scale[blk * kBlockRows + tid] = 0.0f;
      zero[blk * kBlockRows + tid] = 0;
    }
    uint32_t* out = reinterpret_cast<uint32_t*>(codes + (int64_t)off * 1024);
    for (int w = tid; w < 256 * 16; w += kPackThreads) {
      const int F = w >> 8, l = (w >> 2) & 63, d = w & 3;
      const int ib = 16 * (F >> 2) + (l & 15);
      const int jb = 32 * (F & 3) + 8 * (l >> 4) + 2 * d;
      out[w] = (__float_as_uint(tile[ib][jb]) >> 16) | (__float_as_uint(tile[ib][jb + 1]) & 0xFFFF0000u);
    }
    return;
  }

  // Scale and zero point: four threads per row, 32 values each, combined by shuffles.
  const float qmax = (float)((1 << b) - 1);
  {
    const int ib = tid >> 2, part = tid & 3;
    float lo = 0.0f, hi = 0.0f;  // the range always contains 0
    for (int j = part * 32; j < part * 32 + 32; ++j) {
      const float v = tile[ib][j];
      lo = fminf(lo, v);
      hi = fmaxf(hi, v);
    }
#pragma unroll
    for (int d = 1; d < 4; d <<= 1) {
      lo = fminf(lo, __shfl_xor(lo, d, 64));
      hi = fmaxf(hi, __shfl_xor(hi, d, 64));
    }
    if (part == 0) {
      const float diff = hi - lo;
      const float s = diff / qmax;
      float z = 0.0f;
      if (s > 0.0f) z = fminf(fmaxf(__builtin_rintf((-lo) / s), 0.0f), qmax);
      row_s[ib] = s;
      row_z[ib] = z;
      scale[blk * kBlockRows + ib] = s;
      zero[blk * kBlockRows + ib] = (uint8_t)z;
    }
  }
  __syncthreads();

  // Word assembly.  Word index w of the block (byte 4*w): chunk t = w >> 8,
  // lane l = (w >> 2) & 63, dword d = w & 3.  For b == 3 words 0..511 hold the
  // low 2 bits (b == 2 rule) and words 512..767 the high bit (b == 1 rule).
  uint32_t* out = reinterpret_cast<uint32_t*>(codes + (int64_t)off * 1024);
  const int nwords = 256 * b;
  for (int w = tid; w < nwords; w += kPackThreads) {
    int width = b, plane_shift = 0, t = w >> 8;
    if (b == 3) {
      if (w < 512) {
        width = 2;
      } else {
        width = 1;
        plane_shift = 2;
        t = 0;
      }
    }
    const int phi = 16 / width;
    const int l = (w >> 2) & 63, d = w & 3;
    const int n = l & 15, kg = l >> 4;
    const uint32_t fmask = (1u << width) - 1u;
    uint32_t word = 0;
    for (int h = 0; h < 2; ++h) {
      for (int s = 0; s < phi; ++s) {
        const int F = phi * t + s;
        const int ib = 16 * (F >> 2) + n;
        const int jb = 32 * (F & 3) + 8 * kg + 2 * d + h;
        const uint32_t q = rtn_code(tile[ib][jb], row_s[ib], row_z[ib], qmax);
        word |= ((q >> plane_shift) & fmask) << (16 * h + width * s);
      }
    }
    out[w] = word;
  }
}

}  // namespace

hipError_t launch_block_offsets(const uint8_t* bits, int64_t nblocks, uint32_t* offsets,
                                hipStream_t stream) {
  hipLaunchKernelGGL(k_block_offsets, dim3(1), dim3(kScanThreads), 0, stream, bits, nblocks,
                     offsets);
  return hipGetLastError();
}

hipError_t launch_pack(const uint16_t* W, int64_t N, int64_t K, const uint8_t* bits,
                       const int32_t* perm_row, const int32_t* perm_col,
                       const uint32_t* offsets, uint8_t* codes, int64_t code_bytes, float* scale,
                       uint8_t* zero, hipStream_t stream) {
  const int64_t nblk = (N / kBlockRows) * (K / kBlockCols);
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL(k_pack, dim3((unsigned)nblk), dim3(kPackThreads), 0, stream, W, N, K, bits,
                     perm_row, perm_col, offsets, codes, code_bytes, scale, zero);
  return hipGetLastError();
}

}  // namespace msq

// Quantize-and-pack kernels for gfx950.
//
//   k_block_offsets : exclusive prefix sum of the block bit map over the packed
//                     order (segments b = 1,2,3,4,8,16; row-major inside), in KiB.
//   k_pack_rows     : K <= 32768.  One workgroup per (block row, row n of a
//                     16-row tile): it streams the four original rows behind
//                     reordered rows n, n + 16, n + 32, n + 48 of the block row
//                     into LDS (coalesced, each W row read once), gathers
//                     them through perm_col there, computes each (row, block)
//                     scale and zero point and the codes, and writes the
//                     packed words those four rows fill.
//   k_pack_blocks   : any K (used above 32768, where a row no longer fits
//                     the LDS): one workgroup per 64x128 block, gathering it
//                     element by element from W.
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
constexpr int kScanPer = 16;  // consecutive blocks per thread per pass
constexpr int kSegs = 6;

// Number of zero bytes of x (exact: no borrow between bytes).
__device__ __forceinline__ uint32_t zero_bytes(uint32_t x) {
  uint32_t t = (x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu;
  t = ~(t | x | 0x7F7F7F7Fu);
  return (uint32_t)__popc(t);
}

// Bit map bytes i0 .. i0 + 15 as four little-endian words; bytes past nblk
// read as 0 (no block).
__device__ __forceinline__ void load16_bits(const uint8_t* __restrict__ bits, int64_t nblk,
                                            int64_t i0, uint32_t (&w)[4]) {
  if (i0 + kScanPer <= nblk && (reinterpret_cast<uintptr_t>(bits + i0) & 15) == 0) {
    const uint4 v = *reinterpret_cast<const uint4*>(bits + i0);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    return;
  }
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t x = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t i = i0 + 4 * d + e;
      const uint32_t byte = bits[i < nblk ? i : nblk - 1];
      x |= (i < nblk ? byte : 0u) << (8 * e);
    }
    w[d] = x;
  }
}

// One workgroup, two sweeps over the bit map in passes of kScanThreads *
// kScanPer blocks (thread t takes 16 consecutive blocks of a pass, so the
// loads and stores of a wavefront are contiguous).  Sweep 1 counts the
// blocks of every bitwidth (zero bytes of the bits XOR the bitwidth in every
// byte): segment k starts at the sum of bits over the segments before it.
// Sweep 2 scans the per-thread counts of each pass (wavefront prefix sums,
// then across wavefronts) on top of the counts of the passes before, and
// assigns offset = segment base + b * rank, branch-free.
__global__ __launch_bounds__(kScanThreads) void k_block_offsets(const uint8_t* __restrict__ bits,
                                                                int64_t nblk,
                                                                uint32_t* __restrict__ off) {
  __shared__ uint32_t wave_tot[kSegs][kScanThreads / 64];
  __shared__ uint32_t seg_base[kSegs];
  __shared__ uint32_t seg_run[kSegs];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t pass_blocks = (int64_t)kScanThreads * kScanPer;
  constexpr uint32_t kB[kSegs] = {1, 2, 3, 4, 8, 16};

  auto count16 = [&](const uint32_t (&w)[4], uint32_t (&cnt)[kSegs]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kSegs; ++k) {
      const uint32_t rep = kB[k] * 0x01010101u;
      cnt[k] = zero_bytes(w[0] ^ rep) + zero_bytes(w[1] ^ rep) + zero_bytes(w[2] ^ rep) +
               zero_bytes(w[3] ^ rep);
    }
  };
  // sweep 1: totals per segment
  uint32_t tot[kSegs] = {0, 0, 0, 0, 0, 0};
  for (int64_t p0 = 0; p0 < nblk; p0 += pass_blocks) {
    uint32_t w[4], cnt[kSegs];
    load16_bits(bits, nblk, p0 + (int64_t)tid * kScanPer, w);
    count16(w, cnt);
#pragma unroll
    for (int k = 0; k < kSegs; ++k) tot[k] += cnt[k];
  }
#pragma unroll
  for (int k = 0; k < kSegs; ++k) {
    uint32_t v = tot[k];
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) v += __shfl_xor(v, d, 64);
    if (lane == 0) wave_tot[k][wave] = v;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t acc = 0;
    for (int k = 0; k < kSegs; ++k) {
      uint32_t total = 0;
      for (int w = 0; w < kScanThreads / 64; ++w) total += wave_tot[k][w];
      seg_base[k] = acc;
      seg_run[k] = 0;
      acc += kB[k] * total;
    }
  }
  __syncthreads();
  // sweep 2: ranks and offsets
  for (int64_t p0 = 0; p0 < nblk; p0 += pass_blocks) {
    const int64_t i0 = p0 + (int64_t)tid * kScanPer;
    uint32_t w[4], cnt[kSegs], incl[kSegs];
    load16_bits(bits, nblk, i0, w);
    count16(w, cnt);
#pragma unroll
    for (int k = 0; k < kSegs; ++k) {
      uint32_t v = cnt[k];
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t u = __shfl_up(v, d, 64);
        if (lane >= d) v += u;
      }
      incl[k] = v;
      if (lane == 63) wave_tot[k][wave] = v;
    }
    __syncthreads();
    if (tid < kSegs) {  // exclusive prefixes over the wavefronts, on top of the earlier passes
      uint32_t run = seg_run[tid];
      for (int wv = 0; wv < kScanThreads / 64; ++wv) {
        const uint32_t t = wave_tot[tid][wv];
        wave_tot[tid][wv] = run;
        run += t;
      }
      seg_run[tid] = run;
    }
    __syncthreads();
    uint32_t rank[kSegs], base[kSegs];
#pragma unroll
    for (int k = 0; k < kSegs; ++k) {
      rank[k] = wave_tot[k][wave] + incl[k] - cnt[k];
      base[k] = seg_base[k];
    }
    uint32_t o[kScanPer];
#pragma unroll
    for (int e = 0; e < kScanPer; ++e) {
      const uint32_t byte = (w[e >> 2] >> (8 * (e & 3))) & 0xFFu;
      uint32_t v = kNoBlock;
#pragma unroll
      for (int k = 0; k < kSegs; ++k) {
        const bool m = byte == kB[k];
        v = m ? base[k] + kB[k] * rank[k] : v;
        rank[k] += m ? 1u : 0u;
      }
      o[e] = v;
    }
    if (i0 + kScanPer <= nblk && (reinterpret_cast<uintptr_t>(off + i0) & 15) == 0) {
#pragma unroll
      for (int d = 0; d < 4; ++d)
        reinterpret_cast<uint4*>(off + i0)[d] = uint4{o[4 * d], o[4 * d + 1], o[4 * d + 2], o[4 * d + 3]};
    } else {
#pragma unroll
      for (int e = 0; e < kScanPer; ++e)
        if (i0 + e < nblk) off[i0 + e] = o[e];
    }
    __syncthreads();  // wave_tot is rewritten by the next pass
  }
}

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float((uint32_t)u << 16);
}

// Column index clamped into [0, K - 1] (K <= 32768, so it fits 16 bits).
__device__ __forceinline__ int clampi_pack(int v, int hi) { return v < 0 ? 0 : (v > hi ? hi : v); }

// Code of one weight: clamp(rint(w / s) + z, 0, qmax); 0 when s == 0.
__device__ __forceinline__ uint32_t rtn_code(float w, float s, float z, float qmax) {
  if (!(s > 0.0f)) return 0u;
  float t = __builtin_rintf(w / s) + z;
  t = fminf(fmaxf(t, 0.0f), qmax);
  return (uint32_t)t;
}

constexpr int kPackThreads = 256;

// One workgroup per block (any K).  The block's 64 x 128 reordered weights are
// gathered into LDS (perm_row picks the row, perm_col the column), each row's
// scale and zero point are computed from that row's 128 values, then every
// thread assembles whole 32-bit words of the packed block so the global
// stores are coalesced.
__global__ __launch_bounds__(kPackThreads) void k_pack_blocks(
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

// ---- row-streaming pack (K <= 32768) ----------------------------------------------------
//
// Which rows fill which words.  In the packed format, dword d of lane
// l = n + 16 kg of every chunk of a block holds codes of rows 16 rt + n only
// (rt = 0..3, the row tiles): for b = 4, 8, 16 a word holds one row's codes,
// for b = 1, 2, 3 it mixes the four (b = 1, and the high plane of b = 3) or
// two (b = 2, the low plane of b = 3) rows 16 apart.  So the four rows
// n, n + 16, n + 32, n + 48 of a block row complete exactly the 16-byte lane
// slices n + 16 kg (kg = 0..3) of every chunk, and nothing else.
//
// Work split inside the workgroup: 8 or 16 wavefronts x 4 groups of 16 lanes;
// group g of wavefront w takes block columns c = (4 x wavefronts) j + 4 w + g
// (round j), and lane
// (kg, d) = (lane >> 2, lane & 3) of the group takes the eight columns
// jb = 32 kt + 8 kg + 2 d + h (kt = 0..3, h = 0, 1) of that block column:
// exactly the codes of its dword d of the lane slice n + 16 kg, for every
// bitwidth.  The group's min / max run over its 16 lanes (one DPP row).
//
// Codes without a division per weight: rint(fl(w / s)) + z is taken as
// rint(T), T = fl(w * rcp(s) + z) (one fused multiply-add), unless T lies
// within 2^-13 of a half-integer.  v_rcp_f32 is within 1 ulp, so the exact
// w * rcp(s) differs from w / s by at most 2^-23 relative; with |w / s| <=
// 255 (w lies in [lo, hi], s = (hi - lo) / qmax) and z <= 255 the sum's
// rounding adds at most 2^-15 (T < 512), and fl(w / s) differs from w / s
// by at most 2^-24 relative: T and fl(w / s) + z stay within 7.6e-5 <
// 2^-13 of each other, so outside that band both round to the same integer
// (z is one).  Inside the band, and when s is not a normal number at most
// 2^125, the correctly rounded division decides.  Bit-identical to rint of
// the correctly rounded quotient for every input.
constexpr int kRowMaxK = 32768;
typedef __attribute__((address_space(3))) void lds_void_t;

// DPP row (16-lane) reductions: xor 1, xor 2 (quad permutes), then the
// half-row and row mirrors pair the remaining partners.  Every source lane
// of these patterns lies in the lane's own row and a row is active as a
// whole, so no lane keeps its old value (none is supplied).
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, true));
}// min / max of finite values as a median of three with -inf / +inf (one
// instruction; fminf / fmaxf would first quiet a possible signaling NaN of
// each permuted operand).  The infinity passes through an empty asm so that
// the compiler does not turn the median back into fminf / fmaxf.
__device__ __forceinline__ float min_f(float a, float b) {
  float lo = -__builtin_inff();
  asm("" : "+s"(lo));
  return __builtin_amdgcn_fmed3f(a, b, lo);
}
__device__ __forceinline__ float max_f(float a, float b) {
  float hi = __builtin_inff();
  asm("" : "+s"(hi));
  return __builtin_amdgcn_fmed3f(a, b, hi);
}
// Both reductions step by step, so that each step's two permutes and two
// medians interleave.
template <int kCtrl>
__device__ __forceinline__ void minmax_step(float& lo, float& hi) {
  const float a = dpp_f<kCtrl>(lo), b = dpp_f<kCtrl>(hi);
  lo = min_f(lo, a);
  hi = max_f(hi, b);
}
__device__ __forceinline__ void row_minmax16(float& lo, float& hi) {
  minmax_step<0xB1>(lo, hi);   // quad_perm [1,0,3,2]
  minmax_step<0x4E>(lo, hi);   // quad_perm [2,3,0,1]
  minmax_step<0x141>(lo, hi);  // row_half_mirror
  minmax_step<0x140>(lo, hi);  // row_mirror
}

// clamp(rint(fl(x / s)) + z, 0, qmax) for s > 0 (see above); rs = rcp(s),
// fast = s is a normal number <= 2^125, z an integer in [0, 255].  T lies
// within 2^-13 of a half-integer exactly when its distance to the nearest
// integer exceeds 1/2 - 2^-13 (T - rint(T) is exact for |T| < 2^23); the
// clamp is one median of three.
__device__ __forceinline__ uint32_t code_of(float x, float s, float rs, bool fast, float z,
                                            float qmax) {
  const float t = __builtin_fmaf(x, rs, z);
  float r = __builtin_rintf(t);
  const bool near = fabsf(t - r) > 0.5f - 0x1p-13f;
  if (!fast || near) r = __builtin_rintf(x / s) + z;
  return (uint32_t)__builtin_amdgcn_fmed3f(r, 0.0f, qmax);
}

// kThreads threads (4 groups of 16 lanes per wavefront), at most kRounds
// rounds of 4 * kThreads / 64 block columns: K <= 8192 (512 threads, 2
// rounds), 16384 (512, 4), 32768 (1024, 4).  The per-round registers are
// static, so fewer rounds hold fewer of them.
template <int kThreads, int kRounds>
__global__ __launch_bounds__(kThreads) void k_pack_rows(
    const uint16_t* __restrict__ W, int64_t N, int64_t K, const uint8_t* __restrict__ bits,
    const int32_t* __restrict__ perm_row, const int32_t* __restrict__ perm_col,
    const uint32_t* __restrict__ offsets, uint8_t* __restrict__ codes, int64_t code_bytes,
    float* __restrict__ scale, uint8_t* __restrict__ zero) {
  constexpr int kCols = 4 * kThreads / 64;  // block columns per round
  extern __shared__ __align__(16) uint16_t rowbuf[];  // two rows of K bf16
  const int NBr = (int)(N / kBlockRows), NBc = (int)(K / kBlockCols);
  // The 16 workgroups of a block row run on one XCD (consecutive workgroup
  // ids go to the XCDs in turn), so the partial lines they write of each
  // chunk, scale and zero-point row meet in one L2.
  const int bid = blockIdx.x;
  const int xcd = bid & 7, j16 = bid >> 3;
  const int r = 8 * (j16 >> 4) + xcd, n = j16 & 15;
  if (r >= NBr) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, lam = lane & 15, kg = lam >> 2, d = lam & 3;
  const int kk = (int)K - 1;

  // rows 16 rt + n of block row r, clamped original indices
  int orow[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int pr = perm_row[(int64_t)r * kBlockRows + 16 * rt + n];
    orow[rt] = pr < 0 ? 0 : (pr >= N ? (int)(N - 1) : pr);
  }
  // Row rt of the tile into LDS buffer rt & 1: 16 bytes per lane, lane i of
  // the wavefront landing 16 i bytes past the wavefront's base.
  const int nchunks = (int)(K / 8);
  auto load_row = [&](int rt) __attribute__((always_inline)) {
    const uint16_t* src = W + (int64_t)orow[rt] * K;
    uint16_t* dst = rowbuf + (rt & 1) * K;
    for (int base = wave * 64; base < nchunks; base += kThreads) {
      const int idx = base + lane;
      if (idx < nchunks)
        __builtin_amdgcn_global_load_lds(src + 8 * idx, (lds_void_t*)(dst + 8 * base), 16, 0, 0);
    }
  };
  load_row(0);

  // per round: bitwidth, offset, and this lane's eight column indices
  // (pk[j][kt] = perm_col of jb = 32 kt + 2 lam and + 1, as two 16-bit halves)
  int bw[kRounds];
  uint32_t off[kRounds];
  uint32_t pk[kRounds][4];
#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    const int c = kCols * j + 4 * wave + g;
    bw[j] = -1;  // no column
    off[j] = 0;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) pk[j][kt] = 0;
    if (c < NBc) {
      const int64_t blk = (int64_t)r * NBc + c;
      int b = bits[blk];
      const uint32_t o = offsets[blk];
      // a bitwidth outside the format, or a block that would end past the
      // codes buffer (a descriptor msq_plan did not size), is written as pruned
      if (segment_of(b) < 0 || o == kNoBlock || ((int64_t)o + b) * 1024 > code_bytes) b = 0;
      bw[j] = b;
      off[j] = o;
      const int32_t* pc = perm_col + (int64_t)c * kBlockCols + 2 * lam;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const int2 p = *reinterpret_cast<const int2*>(pc + 32 * kt);
        pk[j][kt] = (uint32_t)clampi_pack(p.x, kk) | ((uint32_t)clampi_pack(p.y, kk) << 16);
      }
    }
  }

  // words of 1-, 2- and 3-bit blocks collect the four rows: [j][chunk]
  uint32_t acc[kRounds][3];
  // a row's other outputs are held and stored after the next row's barrier,
  // so that the wait there never waits for stores issued just before it:
  // scale, zero point, and the words of 4-, 8-, 16-bit blocks (row rt: 4 bits
  // chunk rt; 8 bits chunks 2 rt, 2 rt + 1; 16 bits chunks 4 rt + kt)
  float hs[kRounds];
  uint32_t hz[kRounds];
  uint32_t hw[kRounds][4];
#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    acc[j][0] = acc[j][1] = acc[j][2] = 0;
    hs[j] = 0.0f;
    hz[j] = 0;
    hw[j][0] = hw[j][1] = hw[j][2] = hw[j][3] = 0;
  }
  // this lane's byte offset inside a chunk: lane n + 16 kg, dword d
  const uint32_t lane_off = 16 * n + 256 * kg + 4 * d;

  auto flush = [&](int rt) __attribute__((always_inline)) {  // the held outputs of row rt
    const int i = 16 * rt + n;
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      const int b = bw[j];
      if (b < 0) continue;  // uniform over the group
      const int c = kCols * j + 4 * wave + g;
      const int64_t blk = (int64_t)r * NBc + c;
      if (lam == 0) {
        scale[blk * kBlockRows + i] = hs[j];
        zero[blk * kBlockRows + i] = (uint8_t)hz[j];
      }
      uint8_t* cb = codes + (int64_t)off[j] * 1024 + lane_off;
      if (b == 4) {
        *reinterpret_cast<uint32_t*>(cb + 1024 * rt) = hw[j][0];
      } else if (b == 8) {
        *reinterpret_cast<uint32_t*>(cb + 1024 * (2 * rt)) = hw[j][0];
        *reinterpret_cast<uint32_t*>(cb + 1024 * (2 * rt + 1)) = hw[j][1];
      } else if (b == 16) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) *reinterpret_cast<uint32_t*>(cb + 1024 * (4 * rt + kt)) = hw[j][kt];
      }
    }
  };

  for (int rt = 0; rt < 4; ++rt) {
    // row rt has landed (this wavefront's copies: vmcnt; everyone's: the
    // barrier), and every wavefront is done with buffer (rt + 1) & 1
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (rt + 1 < 4) load_row(rt + 1);
    if (rt > 0) flush(rt - 1);
    const uint16_t* row = rowbuf + (rt & 1) * K;
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      if (kCols * j >= NBc) break;  // uniform: no group of this round or later has a column
      const int b = bw[j];
      if (b < 0) continue;          // uniform over the group (one DPP row)
      uint16_t u[4][2];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        u[kt][0] = row[pk[j][kt] & 0xFFFFu];
        u[kt][1] = row[pk[j][kt] >> 16];
      }
      if (b == 0 || b == 16) {
        hs[j] = 0.0f;
        hz[j] = 0;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)  // 16 bits: the bf16 bit patterns
          hw[j][kt] = (uint32_t)u[kt][0] | ((uint32_t)u[kt][1] << 16);
        continue;
      }
      float x[4][2];
      float lo = 0.0f, hi = 0.0f;  // the range always contains 0
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          x[kt][h] = bf16_to_f32(u[kt][h]);
          lo = fminf(lo, x[kt][h]);
          hi = fmaxf(hi, x[kt][h]);
        }
      row_minmax16(lo, hi);
      const float qmax = (float)((1 << b) - 1);
      const float s = (hi - lo) / qmax;
      // z = clamp(rint(fl(-lo / s)), 0, qmax) by the same rule as the codes
      // (0 <= -lo / s <= qmax: hi >= 0)
      const bool fast = s >= 0x1p-126f && s <= 0x1p125f;
      const float rs = __builtin_amdgcn_rcpf(s);
      const float z = s > 0.0f ? (float)code_of(-lo, s, rs, fast, 0.0f, qmax) : 0.0f;
      hs[j] = s;
      hz[j] = (uint32_t)z;
      uint32_t p[4];
      if (s > 0.0f) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          p[kt] = code_of(x[kt][0], s, rs, fast, z, qmax) |
                  (code_of(x[kt][1], s, rs, fast, z, qmax) << 16);
      } else {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) p[kt] = 0;
      }
      if (b == 1) {  // chunk 0, slot 4 rt + kt
        acc[j][0] |= (p[0] | (p[1] << 1) | (p[2] << 2) | (p[3] << 3)) << (4 * rt);
      } else if (b <= 3) {  // (low plane) chunk rt >> 1, slot 4 (rt & 1) + kt
        const uint32_t m = b == 3 ? 0x00030003u : 0xFFFFFFFFu;
        const uint32_t v = ((p[0] & m) | ((p[1] & m) << 2) | ((p[2] & m) << 4) | ((p[3] & m) << 6))
                           << (8 * (rt & 1));
        if (rt < 2) acc[j][0] |= v;
        else acc[j][1] |= v;
        if (b == 3)  // high plane: chunk 2, slot 4 rt + kt
          acc[j][2] |= (((p[0] >> 2) & 0x00010001u) | (((p[1] >> 2) & 0x00010001u) << 1) |
                        (((p[2] >> 2) & 0x00010001u) << 2) | (((p[3] >> 2) & 0x00010001u) << 3))
                       << (4 * rt);
      } else if (b == 4) {  // chunk rt, slot kt
        hw[j][0] = p[0] | (p[1] << 4) | (p[2] << 8) | (p[3] << 12);
      } else {  // 8: chunks 2 rt and 2 rt + 1, slots kt & 1
        hw[j][0] = p[0] | (p[1] << 8);
        hw[j][1] = p[2] | (p[3] << 8);
      }
    }
  }
  flush(3);
  // the words the four rows completed together
#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    const int b = bw[j];
    if (b < 1 || b > 3) continue;
    uint8_t* cb = codes + (int64_t)off[j] * 1024 + lane_off;
    *reinterpret_cast<uint32_t*>(cb) = acc[j][0];
    if (b >= 2) *reinterpret_cast<uint32_t*>(cb + 1024) = acc[j][1];
    if (b == 3) *reinterpret_cast<uint32_t*>(cb + 2048) = acc[j][2];
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
  if (K <= kRowMaxK) {
    // 16 workgroups per block row, block rows in groups of 8 (one per XCD)
    const int64_t grid = 128 * ((N / kBlockRows + 7) / 8);
    const size_t lds = (size_t)K * 4;
    if (K <= 8192)
      hipLaunchKernelGGL((k_pack_rows<512, 2>), dim3((unsigned)grid), dim3(512), lds, stream, W, N,
                         K, bits, perm_row, perm_col, offsets, codes, code_bytes, scale, zero);
    else if (K <= 16384)
      hipLaunchKernelGGL((k_pack_rows<512, 4>), dim3((unsigned)grid), dim3(512), lds, stream, W, N,
                         K, bits, perm_row, perm_col, offsets, codes, code_bytes, scale, zero);
    else
      hipLaunchKernelGGL((k_pack_rows<1024, 4>), dim3((unsigned)grid), dim3(1024), lds, stream, W,
                         N, K, bits, perm_row, perm_col, offsets, codes, code_bytes, scale, zero);
  } else {
    hipLaunchKernelGGL(k_pack_blocks, dim3((unsigned)nblk), dim3(kPackThreads), 0, stream, W, N, K,
                       bits, perm_row, perm_col, offsets, codes, code_bytes, scale, zero);
  }
  return hipGetLastError();
}

}  // namespace msq

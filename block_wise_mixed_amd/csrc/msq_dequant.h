// Device-side helpers shared by the GEMV and GEMM kernels: operand types, the
// bf16 matrix instruction, and the in-register unpack of packed format v1.
//
// Packed format v1 (include/msq.h): a b-bit block is b chunks of 1 KiB; lane
// l of a wavefront owns 16 bytes (four 32-bit words) of every chunk.  For
// fragment F = 4*rt + kt and b in {1,2,4}, slot s = F % (16/b) of chunk
// F / (16/b) holds, in each of the four words, two codes at bits b*s and
// 16 + b*s: the codes of row 16*rt + (l & 15), columns 32*kt + 8*(l >> 4) +
// 2*d + {0,1} for word d.  Those eight codes are exactly one B operand of
// v_mfma_f32_16x16x32_bf16 (16 columns n x 32 k, n = l & 15, k = 8*(l>>4)+i).
//
// Unpack without conversion instructions: OR-ing a code q < 128 into the
// mantissa of bf16 128.0 (0x4300) gives the bf16 value 128 + q exactly, so one
// shift and one v_and_or_b32 turn two codes into two exact bf16 operands.  The
// constant 128 per element is removed afterwards with the per-group sum of
// the activations: sum_k (128 + q_k) x_k - (128 + z) sum_k x_k = sum_k (q_k - z) x_k.
// 8-bit codes (up to 255) do not fit this trick and are converted exactly
// through fp32 instead (bias 0).  3-bit codes are two planes, each turned
// into 128 + q_lo and 128 + 4 q_hi, so their bias is 256.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msq {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

// Bias added to every code by the unpack of a b-bit block (see above).
__host__ __device__ constexpr int unpack_bias(int b) { return b == 8 ? 0 : (b == 3 ? 256 : 128); }

template <int SH>
__device__ __forceinline__ uint32_t shr(uint32_t v) {
  if constexpr (SH > 0) return v >> SH;
  else if constexpr (SH < 0) return v << (-SH);
  else return v;
}

// 128 + code for the b-bit field at bits [SH, SH+b) and [16+SH, 16+SH+b) of each word.
template <int B, int SH>
__device__ __forceinline__ bf16x8 unpack_magic(const uint4& c) {
  constexpr uint32_t mask = ((1u << B) - 1u) * 0x00010001u;
  uint4 v;
  v.x = (shr<SH>(c.x) & mask) | 0x43004300u;
  v.y = (shr<SH>(c.y) & mask) | 0x43004300u;
  v.z = (shr<SH>(c.z) & mask) | 0x43004300u;
  v.w = (shr<SH>(c.w) & mask) | 0x43004300u;
  return as_bf16x8(v);
}

// 128 + 4*hi for the 1-bit high plane of a 3-bit block, hi bit at SRC of each half.
template <int SRC>
__device__ __forceinline__ bf16x8 unpack_hi3(const uint4& c) {
  constexpr uint32_t mask = 0x00040004u;
  uint4 v;
  v.x = (shr<SRC - 2>(c.x) & mask) | 0x43004300u;
  v.y = (shr<SRC - 2>(c.y) & mask) | 0x43004300u;
  v.z = (shr<SRC - 2>(c.z) & mask) | 0x43004300u;
  v.w = (shr<SRC - 2>(c.w) & mask) | 0x43004300u;
  return as_bf16x8(v);
}

__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  f32x2v f = {lo, hi};
  bf16x2v h = __builtin_convertvector(f, bf16x2v);
  return __builtin_bit_cast(uint32_t, h);
}

// Exact bf16 of the 8-bit codes in byte S (0 or 1) of each half.
template <int S>
__device__ __forceinline__ bf16x8 unpack_u8(const uint4& c) {
  uint4 v;
  v.x = pack2_bf16((float)((c.x >> (8 * S)) & 0xFFu), (float)((c.x >> (16 + 8 * S)) & 0xFFu));
  v.y = pack2_bf16((float)((c.y >> (8 * S)) & 0xFFu), (float)((c.y >> (16 + 8 * S)) & 0xFFu));
  v.z = pack2_bf16((float)((c.z >> (8 * S)) & 0xFFu), (float)((c.z >> (16 + 8 * S)) & 0xFFu));
  v.w = pack2_bf16((float)((c.w >> (8 * S)) & 0xFFu), (float)((c.w >> (16 + 8 * S)) & 0xFFu));
  return as_bf16x8(v);
}

// B operand (one 16x32 fragment F = 4*rt + kt) of a B-bit block from its chunks.
// For B == 3 this returns the low plane; hi3_operand gives the high plane.
template <int B, int F>
__device__ __forceinline__ bf16x8 block_operand(const uint4* ch) {
  if constexpr (B == 1) {
    return unpack_magic<1, F>(ch[0]);
  } else if constexpr (B == 2 || B == 3) {
    return unpack_magic<2, 2 * (F % 8)>(ch[F / 8]);
  } else if constexpr (B == 4) {
    return unpack_magic<4, 4 * (F % 4)>(ch[F / 4]);
  } else {
    return unpack_u8<F % 2>(ch[F / 2]);
  }
}

template <int F>
__device__ __forceinline__ bf16x8 hi3_operand(const uint4* ch) {
  return unpack_hi3<F>(ch[2]);
}

// Number of 1 KiB chunks of a B-bit block.
__host__ __device__ constexpr int chunks_of(int b) { return b; }

}  // namespace msq

// Device-side helpers shared by the GEMV and GEMM kernels: operand types, the
// bf16 matrix instruction, and the in-register unpack of the quantized blocks
// of packed format v2 (16-bit blocks are B operands as they are).
//
// Packed format (include/msq.h): a b-bit block is b chunks of 1 KiB; lane
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
// LDS pointer type of the direct global-to-LDS copy builtin
typedef __attribute__((address_space(3))) void lds_void;
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

// Hide a constant from the optimizer, pinned to a scalar (opq_s) or vector
// (opq_v) register.  gfx9 VOP3 encodings take no literal operands, so with
// literal masks the compiler splits (x & mask) | c into two VOP2
// instructions; with both constants in registers it selects one
// v_and_or_b32 and still tracks every hazard around the matrix
// instructions itself.
__device__ __forceinline__ uint32_t opq_s(uint32_t v) {
  asm("" : "+s"(v));
  return v;
}
__device__ __forceinline__ uint32_t opq_v(uint32_t v) {
  asm("" : "+v"(v));
  return v;
}

// One operand fragment: word i becomes (x_i & mask) | c.
__device__ __forceinline__ uint4 and_or4(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3,
                                         uint32_t mask, uint32_t c) {
  const uint32_t m = opq_s(mask), e = opq_v(c);
  return uint4{(x0 & m) | e, (x1 & m) | e, (x2 & m) | e, (x3 & m) | e};
}

// 128 + code for the b-bit field at bits [SH, SH+b) and [16+SH, 16+SH+b) of each word.
template <int B, int SH>
__device__ __forceinline__ bf16x8 unpack_magic(const uint4& c) {
  constexpr uint32_t mask = ((1u << B) - 1u) * 0x00010001u;
  return as_bf16x8(and_or4(shr<SH>(c.x), shr<SH>(c.y), shr<SH>(c.z), shr<SH>(c.w), mask,
                           0x43004300u));
}

// 128 + 4*hi for the 1-bit high plane of a 3-bit block, hi bit at SRC of each half.
template <int SRC>
__device__ __forceinline__ bf16x8 unpack_hi3(const uint4& c) {
  constexpr uint32_t mask = 0x00040004u;
  return as_bf16x8(and_or4(shr<SRC - 2>(c.x), shr<SRC - 2>(c.y), shr<SRC - 2>(c.z),
                           shr<SRC - 2>(c.w), mask, 0x43004300u));
}

// One 3-bit fragment F in a single operand: 128 + q with q = q_lo + 4 q_hi,
// q_lo the 2-bit field of slot F % 8 of the low plane chunk lo, q_hi bit F
// of the high plane chunk hi moved to bit 2 (both and-ors merge into one
// word per pair of codes; the codes stay below 8, so they fit the mantissa).
__device__ __forceinline__ uint4 and_or4v(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3,
                                          uint32_t mask, const uint4& t) {
  const uint32_t m = opq_s(mask);
  return uint4{(x0 & m) | t.x, (x1 & m) | t.y, (x2 & m) | t.z, (x3 & m) | t.w};
}

template <int F>
__device__ __forceinline__ bf16x8 unpack3_magic(const uint4& lo, const uint4& hi) {
  constexpr int SH = 2 * (F % 8);
  uint4 t = and_or4(shr<SH>(lo.x), shr<SH>(lo.y), shr<SH>(lo.z), shr<SH>(lo.w), 0x00030003u,
                    0x43004300u);
  // opaque, so that each half stays one v_and_or_b32 (not and, and, or3)
  t = uint4{opq_v(t.x), opq_v(t.y), opq_v(t.z), opq_v(t.w)};
  return as_bf16x8(and_or4v(shr<F - 2>(hi.x), shr<F - 2>(hi.y), shr<F - 2>(hi.z), shr<F - 2>(hi.w),
                            0x00040004u, t));
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

// ---- shift-minimizing unpack (used by the M = 1 decode path) --------------------------
//
// A field q < 2^w sitting at bit p (p + w <= 7) of a 16-bit half lies inside
// the bf16 mantissa.  OR-ing exponent e = 134 - p into bits 7..14 makes that
// half the exact bf16 value 2^(7-p) + q (the mantissa LSB weighs 2^(p-7) of
// 2^(e-127)), so no shift is needed to bring the field down to bit 0.  One
// shift per word serves every field that lands in bits 0..6 after it: 1-bit
// codes in groups of 7 slots, 2-bit codes in groups of 3, 4-bit codes one
// slot at a time.  For the high plane of 3-bit codes exponent 136 - p gives
// 2^(9-p) + 4*q_hi.  8-bit codes are split into their low 7 bits (exponent
// 134 at bit 0: 128 + q_lo) and their top bit moved to bit 6 (exponent 135:
// 256 + 128*q_hi), two matrix instructions per fragment like 3-bit codes.
// Each fragment therefore carries a known bias per element, removed later
// with per-32-column activation sums.

// Chunk of a B-bit block holding (the low plane of) fragment F.
template <int B, int F>
__host__ __device__ constexpr int chunk_of() {
  return B == 1 ? 0 : (B == 2 || B == 3 ? F / 8 : (B == 4 ? F / 4 : F / 2));
}

// Slot geometry of fragment F for the shift-minimizing unpack (B in 1..4).
template <int B, int F>
struct ExpSlot {
  // right shift applied to the words, bit position after the shift
  static constexpr int kw = B == 3 ? 2 : B;  // width of the low (or only) field
  static constexpr int s = B == 1 ? F : (B == 2 || B == 3 ? F % 8 : F % 4);
  static constexpr int group = B == 1 ? s / 7 : (B == 2 || B == 3 ? s / 3 : s);
  static constexpr int shift = B == 1 ? 7 * group : (B == 2 || B == 3 ? 6 * group : 4 * group);
  static constexpr int pos = B == 1 ? s - 7 * group : (B == 2 || B == 3 ? 2 * (s - 3 * group) : 0);
  // high plane of 3-bit blocks: 1-bit field at bit F of chunk 2
  static constexpr int hgroup = F / 7;
  static constexpr int hshift = 7 * hgroup;
  static constexpr int hpos = F - 7 * hgroup;
};

// Bias of every element of fragment F of a b-bit block under this unpack
// (both planes together for b = 3 and b = 8).
__host__ __device__ constexpr float exp_bias(int b, int F) {
  if (b == 8) return 384.0f;
  int s = b == 1 ? F : (b == 4 ? F % 4 : F % 8);
  int pos = b == 1 ? s % 7 : (b == 4 ? 0 : 2 * (s % 3));
  float lo = (float)(1 << (7 - pos));
  if (b != 3) return lo;
  return lo + (float)(1 << (9 - (F % 7)));
}

// Low (or only) plane of fragment F from its chunk c.
template <int B, int F>
__device__ __forceinline__ bf16x8 exp_lo(const uint4& c) {
  if constexpr (B == 8) {
    constexpr int sh = 8 * (F % 2);
    return as_bf16x8(and_or4(c.x >> sh, c.y >> sh, c.z >> sh, c.w >> sh, 0x007F007Fu,
                             134u * 0x00800080u));
  } else {
    using G = ExpSlot<B, F>;
    constexpr uint32_t mask = (((1u << G::kw) - 1u) << G::pos) * 0x00010001u;
    constexpr uint32_t e = (uint32_t)(134 - G::pos) * 0x00800080u;  // exponent in bits 7..14
    return as_bf16x8(and_or4(c.x >> G::shift, c.y >> G::shift, c.z >> G::shift, c.w >> G::shift,
                             mask, e));
  }
}

// High plane of fragment F (B == 3: from chunk 2; B == 8: from its own chunk).
template <int B, int F>
__device__ __forceinline__ bf16x8 exp_hi(const uint4& c) {
  if constexpr (B == 8) {
    constexpr int sh = 8 * (F % 2) + 1;
    return as_bf16x8(and_or4(c.x >> sh, c.y >> sh, c.z >> sh, c.w >> sh, 0x00400040u,
                             135u * 0x00800080u));
  } else {
    using G = ExpSlot<3, F>;
    constexpr uint32_t mask = (1u << G::hpos) * 0x00010001u;
    constexpr uint32_t e = (uint32_t)(136 - G::hpos) * 0x00800080u;
    return as_bf16x8(and_or4(c.x >> G::hshift, c.y >> G::hshift, c.z >> G::hshift,
                             c.w >> G::hshift, mask, e));
  }
}

// Number of 1 KiB chunks of a B-bit block.
__host__ __device__ constexpr int chunks_of(int b) { return b; }

}  // namespace msq

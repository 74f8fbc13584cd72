// nvfp4_device.hpp -- gfx950 device primitives for NVFP4 block quantization.
//
// Everything here is binary32 arithmetic with one rounding per operation; the
// translation unit is compiled with -ffp-contract=off so that no multiply-add
// is fused (the 4/6 error must be fl(y - fl(v * d)), two roundings).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef float f32x2 __attribute__((ext_vector_type(2)));

enum Rule : int { kRuleNone = 0, kRuleMse = 1, kRuleMae = 2, kRuleMaxErr = 3 };

// ---------------------------------------------------------------- inputs ---

// bf16 is the high half of a binary32 pattern: widening is a shift.
__device__ __forceinline__ void unpack_bf16x8(const uint4 v, float* y) {
  y[0] = __uint_as_float(v.x << 16);
  y[1] = __uint_as_float(v.x & 0xFFFF0000u);
  y[2] = __uint_as_float(v.y << 16);
  y[3] = __uint_as_float(v.y & 0xFFFF0000u);
  y[4] = __uint_as_float(v.z << 16);
  y[5] = __uint_as_float(v.z & 0xFFFF0000u);
  y[6] = __uint_as_float(v.w << 16);
  y[7] = __uint_as_float(v.w & 0xFFFF0000u);
}

// ------------------------------------------------------------------ E4M3 ---

// Nearest E4M3 (OCP E4M3FN: bias 7, subnormals m * 2^-9, max 448 = 0x7E),
// ties to even mantissa, saturating: r >= 448 (and +inf) -> 0x7E.  r >= 0.
// The gfx950 fp32 -> fp8 convert rounds to nearest even and equals this
// encoding for every binary32 r in [0, 448); above 448 it does not saturate,
// so r is clamped first (448 itself encodes as 0x7E).
__device__ __forceinline__ uint32_t e4m3_encode(float r) {
  // r is +0, positive, +inf or NaN: for these the unsigned minimum of the bit
  // patterns with 448's is the saturated value (and the float minimum where both are
  // numbers), so overflowing and NaN quotients encode as 448 too
  const uint32_t c = min(__float_as_uint(r), 0x43E00000u);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(c), 0.0f, (int)c, false) & 0xFFu;
}

__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  return c < 8u ? (float)c * 0.001953125f : __uint_as_float((c + (120u << 3)) << 20);
}

// ------------------------------------------------------------------ E2M1 ---

// Round-to-nearest-even to E2M1 of two values into byte SEL of `old`
// (low nibble = a).  The gfx950 convert at scale 1.0 matches nearest-even with
// saturation at 6 and a kept sign bit for every finite binary32 input.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_rne_pair(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// Stochastic rounding of a pair of values into byte SEL of `d`, keeping d's
// other bytes.  The convert's first slot rounds its value up iff
// (r >> 10) + floor(f * 2^22) >= 2^22; its second slot reads r one bit lower.
// (Written as inline assembly because the compiler builtin does not keep the
// destination's other bytes.)
template <int SEL>
__device__ __forceinline__ uint32_t cvt_sr_byte(uint32_t d, f32x2 src, uint32_t r) {
  if constexpr (SEL == 0) {
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0" : "+v"(d) : "v"(src), "v"(r));
  } else if constexpr (SEL == 1) {
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,1,0]" : "+v"(d) : "v"(src), "v"(r));
  } else if constexpr (SEL == 2) {
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,0,1]" : "+v"(d) : "v"(src), "v"(r));
  } else {
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,1,1]" : "+v"(d) : "v"(src), "v"(r));
  }
  return d;
}

// First convert of a chain that writes all four bytes of a register: the
// register's previous contents do not matter, so it is an output operand.  It
// is an early-clobber output: the convert can write its destination byte before
// it has read the second value, so a destination that shares a register with
// that value makes the second slot round a value whose low byte has already
// been replaced (seen as rare run-to-run differences in the second slot).
__device__ __forceinline__ uint32_t cvt_sr_byte0_fresh(f32x2 src, uint32_t r) {
  uint32_t d;
  asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0" : "=&v"(d) : "v"(src), "v"(r));
  return d;
}

__device__ __forceinline__ uint32_t cvt_rne_byte0_fresh(float a, float b) {
  uint32_t d;
  asm("v_cvt_scalef32_pk_fp4_f32 %0, %1, %2, 1.0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}

// The two E2M1 values in byte SEL of a packed word (exact at scale 1.0).
template <int SEL>
__device__ __forceinline__ f32x2 fp4_pair_values(uint32_t packed) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, SEL);
}

// ---------------------------------------------------------------- Philox ---

// a ^ b ^ c in one instruction (truth table 0x96); c must be wave-uniform (the Philox key).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t d;
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(d) : "v"(a), "v"(b), "s"(c));
  return d;
}

// Philox-4x32-10 (Salmon et al., SC'11): ten rounds, each two 32x32->64
// products with the published multipliers and xors with the round key.  The
// round keys are the key advanced by the published Weyl constants before each
// round after the first (wave-uniform, computed once per kernel).
struct PhiloxKey {
  uint32_t k0[10], k1[10];
};

__device__ __forceinline__ PhiloxKey philox_key(uint32_t k0, uint32_t k1) {
  PhiloxKey K;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    K.k0[r] = k0 + (uint32_t)r * 0x9E3779B9u;
    K.k1[r] = k1 + (uint32_t)r * 0xBB67AE85u;
  }
  return K;
}

// Rounds r0 .. 9 of four instances advanced together (round-major, so that no
// product waits for the one just before it).
__device__ __forceinline__ void philox_rounds4(uint32_t* x0, uint32_t* x1, uint32_t* x2, uint32_t* x3,
                                               const PhiloxKey& K, int r0) {
#pragma unroll
  for (int r = r0; r < 10; ++r) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint64_t p0 = (uint64_t)0xD2511F53u * x0[j];
      const uint64_t p1 = (uint64_t)0xCD9E8D57u * x2[j];
      const uint32_t n0 = xor3((uint32_t)(p1 >> 32), x1[j], K.k0[r]);
      const uint32_t n2 = xor3((uint32_t)(p0 >> 32), x3[j], K.k1[r]);
      x1[j] = (uint32_t)p1;
      x3[j] = (uint32_t)p0;
      x0[j] = n0;
      x2[j] = n2;
    }
  }
}

// Words for 16 consecutive elements whose first Philox counter is (lo, hi)
// with lo + 3 < 2^32 and hi wave-uniform: counters (lo + j, hi, 0, 0).  The
// first round's second product is zero and its xor of hi with the key is
// uniform, so the second round's first product and the third round's x3 term
// are uniform too and run on the scalar unit.  Same words as four full
// Philox-4x32-10 evaluations.
__device__ __forceinline__ void sr_words16_hi_uniform(uint32_t lo, uint32_t hi, const PhiloxKey& K, uint32_t* w) {
  uint32_t x0[4], x1[4], x2[4], x3[4];
  const uint32_t u0 = hi ^ K.k0[0];                       // round 1: x0, uniform
  const uint64_t pu = (uint64_t)0xD2511F53u * u0;         // round 2: first product, uniform
  const uint32_t hu = (uint32_t)(pu >> 32) ^ K.k1[1];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint64_t p = (uint64_t)0xD2511F53u * (lo + (uint32_t)j);  // round 1
    const uint32_t a2 = (uint32_t)(p >> 32) ^ K.k1[0];
    const uint32_t a3 = (uint32_t)p;
    const uint64_t q = (uint64_t)0xCD9E8D57u * a2;                   // round 2 (x1 = 0)
    x0[j] = (uint32_t)(q >> 32) ^ K.k0[1];
    x1[j] = (uint32_t)q;
    x2[j] = a3 ^ hu;
  }
  const uint32_t u3 = (uint32_t)pu ^ K.k1[2];             // round 3: x3 uniform
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * x0[j];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * x2[j];
    const uint32_t n0 = xor3((uint32_t)(p1 >> 32), x1[j], K.k0[2]);
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ u3;
    x1[j] = (uint32_t)p1;
    x3[j] = (uint32_t)p0;
    x0[j] = n0;
    x2[j] = n2;
  }
  philox_rounds4(x0, x1, x2, x3, K, 3);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    w[4 * j + 0] = x0[j];
    w[4 * j + 1] = x1[j];
    w[4 * j + 2] = x2[j];
    w[4 * j + 3] = x3[j];
  }
}

// Words for 16 consecutive elements starting at idx0 (idx0 % 4 == 0):
// element idx uses word (idx mod 4) of the block at counter (idx/4, 0, 0).
__device__ __forceinline__ void sr_words16(uint64_t idx0, const PhiloxKey& K, uint32_t* w) {
  const uint64_t q0 = idx0 >> 2;
  uint32_t x0[4], x1[4], x2[4], x3[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint64_t q = q0 + (uint64_t)j;
    x0[j] = (uint32_t)q;
    x1[j] = (uint32_t)(q >> 32);
    x2[j] = 0u;
    x3[j] = 0u;
  }
  philox_rounds4(x0, x1, x2, x3, K, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    w[4 * j + 0] = x0[j];
    w[4 * j + 1] = x1[j];
    w[4 * j + 2] = x2[j];
    w[4 * j + 3] = x3[j];
  }
}

// ---------------------------------------------------------- Hadamard 16 ---

// y = H16 * D * x / 4: sign flips from `mask`, butterflies h = 1, 2, 4, 8 in
// that order with (a, b) -> (a + b, a - b), then the exact scaling by 1/4.
__device__ __forceinline__ void rht16(float* v, uint32_t mask) {
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = __uint_as_float(__float_as_uint(v[i]) ^ (((mask >> i) & 1u) << 31));
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i & h) continue;
      const float a = v[i], b = v[i + h];
      v[i] = a + b;
      v[i + h] = a - b;
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = 0.25f * v[i];
}

// --------------------------------------------------------- cross-lane ---

// DPP lane exchanges inside a row of 16 lanes.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within each 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i within each 16

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Max over the 16 lanes of a DPP row (exact and order-free).
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  v = fmaxf(v, dpp<kDppMirror>(v));
  return v;
}

// Pairwise sum in lane order over a 16-lane row: lanes (2k, 2k+1), then pairs
// of pairs, ...; both partners add the same two operands, so every lane ends
// with the identical value.
__device__ __forceinline__ float row16_pairwise_sum(float v) {
  v = v + dpp<kDppXor1>(v);
  v = v + dpp<kDppXor2>(v);
  v = v + dpp<kDppHalfMirror>(v);
  v = v + dpp<kDppMirror>(v);
  return v;
}

// ------------------------------------------------------- block quantize ---

struct BlockCodes {
  uint32_t lo, hi;  // 16 packed codes: element 2k in bits 4k..4k+3 of the 64-bit pair
};

// Transpose of a 16x16 tile of codes held by the 16 lanes of a DPP row: lane i
// (i = lane & 15) brings row i (code c in nibble c) and gets column i (the code
// of row r in nibble r).  Each of four exchange stages swaps one bit of the row
// index with the same bit of the column index: a code whose two bits differ
// moves to lane i ^ b and nibble c ^ b (b = 8: whole words, with lane i ^ 8;
// b = 4, 2: byte selects with lanes i ^ 4 and i ^ 2; b = 1: nibbles, lane i ^ 1).
__device__ __forceinline__ uint32_t lane_xor8(uint32_t v) {  // row_ror:8 inside a 16-lane row
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t lane_xor4(uint32_t v) {  // ds_swizzle bitmask mode: and 0x1F, xor 4
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x101F);
}
__device__ __forceinline__ uint32_t lane_xor2(uint32_t v) {  // quad_perm [2,3,0,1]
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t lane_xor1(uint32_t v) {  // quad_perm [1,0,3,2]
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}

__device__ __forceinline__ BlockCodes transpose_tile16(BlockCodes x, int i) {
  uint32_t lo = x.lo, hi = x.hi;
  {  // b = 8: lanes below 8 keep their low word and take the partner's as high word
    const bool up = (i & 8) != 0;
    const uint32_t recv = lane_xor8(up ? lo : hi);
    lo = up ? recv : lo;
    hi = up ? hi : recv;
  }
  {  // b = 4: 16-bit halves; v_perm bytes 0-3 from the own word, 4-7 from the partner's
    const uint32_t sel = (i & 4) ? 0x03020706u : 0x05040100u;
    const uint32_t plo = lane_xor4(lo), phi = lane_xor4(hi);
    lo = __builtin_amdgcn_perm(plo, lo, sel);
    hi = __builtin_amdgcn_perm(phi, hi, sel);
  }
  {  // b = 2: bytes
    const uint32_t sel = (i & 2) ? 0x03070105u : 0x06020400u;
    const uint32_t plo = lane_xor2(lo), phi = lane_xor2(hi);
    lo = __builtin_amdgcn_perm(plo, lo, sel);
    hi = __builtin_amdgcn_perm(phi, hi, sel);
  }
  {  // b = 1: nibbles; the partner's word rotated by 4 bits toward the taken nibbles
    const bool odd = (i & 1) != 0;
    const uint32_t keep = odd ? 0xF0F0F0F0u : 0x0F0F0F0Fu;
    const uint32_t sh = odd ? 4u : 28u;
    const uint32_t plo = lane_xor1(lo), phi = lane_xor1(hi);
    lo = (lo & keep) | (__builtin_amdgcn_alignbit(plo, plo, sh) & ~keep);
    hi = (hi & keep) | (__builtin_amdgcn_alignbit(phi, phi, sh) & ~keep);
  }
  return BlockCodes{lo, hi};
}

// Pairwise sum of 16 values in index order.
__device__ __forceinline__ float pairwise16(const float* t) {
  float s[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) s[i] = t[2 * i] + t[2 * i + 1];
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = s[2 * i] + s[2 * i + 1];
  s[0] = s[0] + s[1];
  s[1] = s[2] + s[3];
  return s[0] + s[1];
}

// Scale and round 16 values with reciprocal e.  For stochastic rounding `w`
// holds the element words with the odd elements' words already shifted right
// by one (the convert's second slot reads its random word one bit lower): the
// even-slot converts fill one register, the odd-slot converts another, and one
// bitfield insert takes the low nibbles of the first and the high nibbles of
// the second.
template <bool SR>
__device__ __forceinline__ BlockCodes round16(const float* y, float e, const uint32_t* w) {
  BlockCodes c;
  if constexpr (!SR) {
    uint32_t lo, hi;
    lo = cvt_rne_byte0_fresh(y[0] * e, y[1] * e);
    lo = cvt_rne_pair<1>(lo, y[2] * e, y[3] * e);
    lo = cvt_rne_pair<2>(lo, y[4] * e, y[5] * e);
    lo = cvt_rne_pair<3>(lo, y[6] * e, y[7] * e);
    hi = cvt_rne_byte0_fresh(y[8] * e, y[9] * e);
    hi = cvt_rne_pair<1>(hi, y[10] * e, y[11] * e);
    hi = cvt_rne_pair<2>(hi, y[12] * e, y[13] * e);
    hi = cvt_rne_pair<3>(hi, y[14] * e, y[15] * e);
    c.lo = lo;
    c.hi = hi;
  } else {
    f32x2 z[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) z[k] = f32x2{y[2 * k] * e, y[2 * k + 1] * e};
    uint32_t ev0, od0, ev1, od1;
    ev0 = cvt_sr_byte0_fresh(z[0], w[0]);
    od0 = cvt_sr_byte0_fresh(z[0], w[1]);
    ev0 = cvt_sr_byte<1>(ev0, z[1], w[2]);
    od0 = cvt_sr_byte<1>(od0, z[1], w[3]);
    ev0 = cvt_sr_byte<2>(ev0, z[2], w[4]);
    od0 = cvt_sr_byte<2>(od0, z[2], w[5]);
    ev0 = cvt_sr_byte<3>(ev0, z[3], w[6]);
    od0 = cvt_sr_byte<3>(od0, z[3], w[7]);
    ev1 = cvt_sr_byte0_fresh(z[4], w[8]);
    od1 = cvt_sr_byte0_fresh(z[4], w[9]);
    ev1 = cvt_sr_byte<1>(ev1, z[5], w[10]);
    od1 = cvt_sr_byte<1>(od1, z[5], w[11]);
    ev1 = cvt_sr_byte<2>(ev1, z[6], w[12]);
    od1 = cvt_sr_byte<2>(od1, z[6], w[13]);
    ev1 = cvt_sr_byte<3>(ev1, z[7], w[14]);
    od1 = cvt_sr_byte<3>(od1, z[7], w[15]);
    c.lo = (ev0 & 0x0F0F0F0Fu) | (od0 & 0xF0F0F0F0u);
    c.hi = (ev1 & 0x0F0F0F0Fu) | (od1 & 0xF0F0F0F0u);
  }
  return c;
}

// Stochastic rounding of 16 values under both 4/6 candidates, one convert per
// element: the convert's first slot rounds z6 = y * e6 with bits 31..10 of the
// element's word and its second slot z4 = y * e4 with bits 30..9 (it reads the
// same word one bit lower), which is the bit split the two candidates use.
// Element k lands in byte (k & 7) >> 1 of register P[2 (k >> 3) + (k & 1)], so
// that one shift and one bitfield insert per 8 elements gather either
// candidate's nibbles in element order.
template <int SEL>
__device__ __forceinline__ uint32_t sr_pair_byte(uint32_t d, const float* y, int k, float e6, float e4,
                                                 const uint32_t* w) {
  return cvt_sr_byte<SEL>(d, f32x2{y[k] * e6, y[k] * e4}, w[k]);
}

__device__ __forceinline__ void sr_pair_regs(const float* y, float e6, float e4, const uint32_t* w, uint32_t* P) {
  // register r holds elements k0(r), k0(r) + 2, + 4, + 6 with k0(r) = 8 (r >> 1) + (r & 1);
  // the four registers' convert chains are interleaved byte by byte
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int k0 = (r >> 1) * 8 + (r & 1);
    P[r] = cvt_sr_byte0_fresh(f32x2{y[k0] * e6, y[k0] * e4}, w[k0]);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) P[r] = sr_pair_byte<1>(P[r], y, (r >> 1) * 8 + (r & 1) + 2, e6, e4, w);
#pragma unroll
  for (int r = 0; r < 4; ++r) P[r] = sr_pair_byte<2>(P[r], y, (r >> 1) * 8 + (r & 1) + 4, e6, e4, w);
#pragma unroll
  for (int r = 0; r < 4; ++r) P[r] = sr_pair_byte<3>(P[r], y, (r >> 1) * 8 + (r & 1) + 6, e6, e4, w);
}

// (a & 0x0F0F0F0F) | (b & 0xF0F0F0F0): one v_bfi_b32.
__device__ __forceinline__ uint32_t nibble_merge(uint32_t a, uint32_t b) {
  return (a & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
}

struct CodePair {
  BlockCodes c6, c4;
};

__device__ __forceinline__ CodePair round16_sr_both(const float* y, float e6, float e4, const uint32_t* w) {
  uint32_t P[4];
  sr_pair_regs(y, e6, e4, w, P);
  CodePair cp;
  cp.c6.lo = nibble_merge(P[0], P[1] << 4);
  cp.c6.hi = nibble_merge(P[2], P[3] << 4);
  cp.c4.lo = nibble_merge(P[0] >> 4, P[1]);
  cp.c4.hi = nibble_merge(P[2] >> 4, P[3]);
  return cp;
}

// Per-element error terms of one candidate: t_i = eps_i^2 (MSE) or |eps_i|
// (MAE, MAXERR) with eps_i = fl(y_i - fl(value_i * d)).
template <int RULE>
__device__ __forceinline__ void error_terms16(const float* y, BlockCodes c, float d, float* t) {
  f32x2 v[8];
  v[0] = fp4_pair_values<0>(c.lo);
  v[1] = fp4_pair_values<1>(c.lo);
  v[2] = fp4_pair_values<2>(c.lo);
  v[3] = fp4_pair_values<3>(c.lo);
  v[4] = fp4_pair_values<0>(c.hi);
  v[5] = fp4_pair_values<1>(c.hi);
  v[6] = fp4_pair_values<2>(c.hi);
  v[7] = fp4_pair_values<3>(c.hi);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float x0 = v[k].x * d, x1 = v[k].y * d;
    const float e0 = y[2 * k] - x0, e1 = y[2 * k + 1] - x1;
    if constexpr (RULE == kRuleMse) {
      t[2 * k] = e0 * e0;
      t[2 * k + 1] = e1 * e1;
    } else {
      t[2 * k] = fabsf(e0);
      t[2 * k + 1] = fabsf(e1);
    }
  }
}

template <int RULE>
__device__ __forceinline__ float reduce16(const float* t) {
  if constexpr (RULE == kRuleMaxErr) {
    float m = t[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) m = fmaxf(m, t[i]);
    return m;
  } else {
    return pairwise16(t);
  }
}

// Scale factors of one candidate (T = 6 or 4) from the block max.
struct Scale {
  uint32_t sb;  // E4M3 code
  float d;      // fl(dec(sb) * S_t)
  float e;      // fl(1 / d), 0 when d == 0 or 1/d overflows
};

// d and e depend only on the E4M3 code and S_t: each workgroup tabulates them
// once for the 127 finite codes (one correctly rounded division per entry).
__device__ __forceinline__ void fill_scale_table(f32x2* tab, float st) {
  if (threadIdx.x < 128) {
    const float d = e4m3_decode(threadIdx.x) * st;
    float e = 0.0f;
    if (d != 0.0f) {
      e = __fdiv_rn(1.0f, d);
      if (__builtin_isinf(e)) e = 0.0f;
    }
    tab[threadIdx.x] = f32x2{d, e};
  }
}

// The candidates divide the block max by a workgroup-uniform divisor den.
// With y = fl(1/den), q0 = fl(m * y) and two residual corrections
// (r = fma(-q, den, m) is exact; q' = fma(r, y, q)) give the correctly rounded
// quotient fl(m / den) (Markstein's theorem; also checked against the
// correctly rounded division over every significand of 27 binades of the
// quotient for 64 divisors).  The theorem needs normal numbers throughout, so
// it is used only when den is in [2^-100, 2^100]; quotients of 2^20 or more
// saturate the E4M3 scale either way.
struct Divisor {
  float den;   // fl(T * S_t)
  float y;     // fl(1 / den)
  bool fast;   // den within the range where the corrected product is exact
  bool est;    // den within the range where the 4/6 error estimates are bounded
};

__device__ __forceinline__ Divisor make_divisor(float den) {
  Divisor d;
  d.den = den;
  d.fast = den >= 0x1p-100f && den <= 0x1p100f;
  d.est = den >= 0x1p-48f && den <= 0x1p48f;
  d.y = d.fast ? __fdiv_rn(1.0f, den) : 0.0f;
  return d;
}

__device__ __forceinline__ float divide(float m, const Divisor& d) {
  if (d.fast) {  // uniform branch
    const float q0 = m * d.y;
    const float r0 = __builtin_fmaf(-q0, d.den, m);
    const float q1 = __builtin_fmaf(r0, d.y, q0);
    const float r1 = __builtin_fmaf(-q1, d.den, m);
    // where m / den overflows, q0 is +inf and q2 NaN; e4m3_encode saturates both
    return __builtin_fmaf(r1, d.y, q1);
  }
  return (m == 0.0f || d.den == 0.0f) ? 0.0f : __fdiv_rn(m, d.den);
}

__device__ __forceinline__ Scale block_scale(float m, const Divisor& den, const f32x2* tab) {
  Scale s;
  s.sb = e4m3_encode(divide(m, den));
  const f32x2 de = tab[s.sb];
  s.d = de.x;
  s.e = de.y;
  return s;
}

// ------------------------------------------------- 4/6 error estimates ---
//
// The 4/6 choice compares the candidates' errors E_T: a binary32 reduction
// (pairwise sum, or max) of per-element terms of eps = fl(y - fl(v * d)).
// Most blocks are decided without forming those terms.  While an element is
// rounded, its residual in the scaled domain, r = fl(z - v) with z = fl(y * e),
// is accumulated (|r|, r^2 or max |r|), and d (MSE: d^2) times the result
// estimates E_T.  To first order in u = 2^-24, for a block of n values with
// max m, both the estimate and E_T lie within
//   MAE:    3u n m + 21u E         MSE: 6u sum|y||t| + 27u E
//   MAXERR: 3u m + 4u E
// of the exact-arithmetic error (t = y - v d; sum|y||t| <= (n m^2/16 + 16 E)/2
// by the arithmetic-geometric mean), provided the tensor scale keeps every
// non-zero d within [2^-60, 2^60] (den within [2^-48, 2^48]) and d > 0.  The
// bounds applied below are at least 2.5 times these.  When the estimates
// differ by more than the sum of the two candidates' bounds, their order is
// the order of the exact errors and decides the block; otherwise (near-ties,
// zero or extreme scales, non-finite values) the exact errors are formed.
template <int RULE>
__device__ __forceinline__ float residual_first(float r) {
  if constexpr (RULE == kRuleMse) {
    return r * r;
  } else {
    return fabsf(r);
  }
}

template <int RULE>
__device__ __forceinline__ float residual_acc(float acc, float r) {
  if constexpr (RULE == kRuleMse) {
    return __builtin_fmaf(r, r, acc);
  } else if constexpr (RULE == kRuleMaxErr) {
    return fmaxf(acc, fabsf(r));
  } else {
    return acc + fabsf(r);
  }
}

template <int RULE>
__device__ __forceinline__ float residual_join(float a, float b) {
  if constexpr (RULE == kRuleMaxErr) {
    return fmaxf(a, b);
  } else {
    return a + b;
  }
}

template <int RULE>
__device__ __forceinline__ float residual_join4(const float* a) {
  return residual_join<RULE>(residual_join<RULE>(a[0], a[1]), residual_join<RULE>(a[2], a[3]));
}

// Stochastic rounding of 16 values under both candidates (as sr_pair_regs),
// with each convert's two codes decoded at once to accumulate the residual
// sums of the scale-to-6 (s6) and scale-to-4 (s4) candidates.
template <int SEL, int RULE>
__device__ __forceinline__ void sr_pair_step(const float* y, float e6, float e4, const uint32_t* w, uint32_t* P,
                                             float* a6, float* a4) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int k = (r >> 1) * 8 + (r & 1) + 2 * SEL;
    const f32x2 z = {y[k] * e6, y[k] * e4};
    if constexpr (SEL == 0) {
      P[r] = cvt_sr_byte0_fresh(z, w[k]);
    } else {
      P[r] = cvt_sr_byte<SEL>(P[r], z, w[k]);
    }
    const f32x2 v = fp4_pair_values<SEL>(P[r]);
    if constexpr (SEL == 0) {
      a6[r] = residual_first<RULE>(z.x - v.x);
      a4[r] = residual_first<RULE>(z.y - v.y);
    } else {
      a6[r] = residual_acc<RULE>(a6[r], z.x - v.x);
      a4[r] = residual_acc<RULE>(a4[r], z.y - v.y);
    }
  }
}

template <int RULE>
__device__ __forceinline__ void sr_pair_sums(const float* y, float e6, float e4, const uint32_t* w, uint32_t* P,
                                             float& s6, float& s4) {
  float a6[4], a4[4];
  sr_pair_step<0, RULE>(y, e6, e4, w, P, a6, a4);
  sr_pair_step<1, RULE>(y, e6, e4, w, P, a6, a4);
  sr_pair_step<2, RULE>(y, e6, e4, w, P, a6, a4);
  sr_pair_step<3, RULE>(y, e6, e4, w, P, a6, a4);
  s6 = residual_join4<RULE>(a6);
  s4 = residual_join4<RULE>(a4);
}

// Round-to-nearest-even of 16 values with reciprocal e (the codes of
// round16<false>) and the candidate's residual sum s.
template <int SEL, int RULE>
__device__ __forceinline__ void rne_pair_step(const float* y, float e, uint32_t& lo, uint32_t& hi, float* a) {
  const float z0 = y[2 * SEL] * e, z1 = y[2 * SEL + 1] * e;
  const float z8 = y[8 + 2 * SEL] * e, z9 = y[9 + 2 * SEL] * e;
  if constexpr (SEL == 0) {
    lo = cvt_rne_byte0_fresh(z0, z1);
    hi = cvt_rne_byte0_fresh(z8, z9);
  } else {
    lo = cvt_rne_pair<SEL>(lo, z0, z1);
    hi = cvt_rne_pair<SEL>(hi, z8, z9);
  }
  const f32x2 vl = fp4_pair_values<SEL>(lo), vh = fp4_pair_values<SEL>(hi);
  constexpr int c = 2 * (SEL & 1);  // chains 0, 1 take bytes 0 and 2; chains 2, 3 bytes 1 and 3
  if constexpr (SEL < 2) {
    a[c] = residual_first<RULE>(z0 - vl.x);
    a[c + 1] = residual_first<RULE>(z8 - vh.x);
  } else {
    a[c] = residual_acc<RULE>(a[c], z0 - vl.x);
    a[c + 1] = residual_acc<RULE>(a[c + 1], z8 - vh.x);
  }
  a[c] = residual_acc<RULE>(a[c], z1 - vl.y);
  a[c + 1] = residual_acc<RULE>(a[c + 1], z9 - vh.y);
}

template <int RULE>
__device__ __forceinline__ BlockCodes round16_sums(const float* y, float e, float& s) {
  uint32_t lo, hi;
  float a[4];
  rne_pair_step<0, RULE>(y, e, lo, hi, a);
  rne_pair_step<1, RULE>(y, e, lo, hi, a);
  rne_pair_step<2, RULE>(y, e, lo, hi, a);
  rne_pair_step<3, RULE>(y, e, lo, hi, a);
  s = residual_join4<RULE>(a);
  return BlockCodes{lo, hi};
}

template <int RULE>
__device__ __forceinline__ float error_estimate(float s, float d) {
  if constexpr (RULE == kRuleMse) {
    return d * (d * s);
  } else {
    return d * s;
  }
}

// Whether the estimates a6, a4 of a block of N values with max m decide it.
template <int RULE, int N>
__device__ __forceinline__ bool estimates_decide(float a6, float a4, float m) {
  float b;
  if constexpr (RULE == kRuleMae) {
    b = 0x1p-18f * (a6 + a4) + (0x1p-20f * N) * m;
  } else if constexpr (RULE == kRuleMaxErr) {
    b = 0x1p-19f * (a6 + a4) + 0x1p-20f * m;
  } else {
    b = 0x1p-16f * (a6 + a4) + (0x1p-23f * N) * (m * m);
  }
  return fabsf(a4 - a6) > b;
}

struct BlockResult {
  BlockCodes codes;
  uint32_t sb;
  float e;            // reciprocal of the chosen candidate (reused to re-round the same values)
  uint32_t four = 0;  // 1 when the scale-to-4 candidate was chosen
};

// Both candidates of a block (or of a 16x16 tile spread over a DPP row, TILE)
// whose max is m, and the 4/6 choice.  Without 4/6 only the scale-to-6
// candidate is formed; its stochastic rounding pairs consecutive elements in
// one convert, so the odd elements' words are shifted right by one (the
// convert's second slot reads its word one bit lower).
// EST: decide by the error estimates where they suffice (the exact errors otherwise).
template <bool SR, int RULE, bool TILE = false, bool EST = false>
__device__ __forceinline__ BlockResult choose16(const float* y, float m, const uint32_t* w, const f32x2* tab,
                                                const Divisor& den6, const Divisor& den4) {
  const Scale s6 = block_scale(m, den6, tab);
  if constexpr (RULE == kRuleNone) {
    uint32_t ws[16];
    if constexpr (SR) {
#pragma unroll
      for (int k = 0; k < 16; ++k) ws[k] = (k & 1) ? (w[k] >> 1) : w[k];
    }
    return BlockResult{round16<SR>(y, s6.e, ws), s6.sb, s6.e};
  } else {
    const Scale s4 = block_scale(m, den4, tab);
    BlockCodes c6, c4;
    bool decided = false, pick4 = false;
    if constexpr (EST) {
      float f6, f4;  // residual sums in the scaled domain
      if constexpr (SR) {
        uint32_t P[4];
        sr_pair_sums<RULE>(y, s6.e, s4.e, w, P, f6, f4);
        c6.lo = nibble_merge(P[0], P[1] << 4);
        c6.hi = nibble_merge(P[2], P[3] << 4);
        c4.lo = nibble_merge(P[0] >> 4, P[1]);
        c4.hi = nibble_merge(P[2] >> 4, P[3]);
      } else {
        c6 = round16_sums<RULE>(y, s6.e, f6);
        c4 = round16_sums<RULE>(y, s4.e, f4);
      }
      if constexpr (TILE) {
        if constexpr (RULE == kRuleMaxErr) {
          f6 = row16_max(f6);
          f4 = row16_max(f4);
        } else {
          f6 = row16_pairwise_sum(f6);
          f4 = row16_pairwise_sum(f4);
        }
      }
      const float a6 = error_estimate<RULE>(f6, s6.d), a4 = error_estimate<RULE>(f4, s4.d);
      // (evaluated in full, so that the sums are formed while the codes are)
      decided = den6.est & (s6.d > 0.0f) & estimates_decide<RULE, TILE ? 256 : 16>(a6, a4, m);
      pick4 = a4 < a6;
    } else {
      if constexpr (SR) {
        const CodePair cp = round16_sr_both(y, s6.e, s4.e, w);
        c6 = cp.c6;
        c4 = cp.c4;
      } else {
        c6 = round16<false>(y, s6.e, nullptr);
        c4 = round16<false>(y, s4.e, nullptr);
      }
    }
    if (!decided) {
      // the exact errors (in a 16x16 tile every lane of the row takes this branch together)
      float t[16];
      error_terms16<RULE>(y, c6, s6.d, t);
      float err6 = reduce16<RULE>(t);
      error_terms16<RULE>(y, c4, s4.d, t);
      float err4 = reduce16<RULE>(t);
      if constexpr (TILE) {
        if constexpr (RULE == kRuleMaxErr) {
          err6 = row16_max(err6);
          err4 = row16_max(err4);
        } else {
          err6 = row16_pairwise_sum(err6);
          err4 = row16_pairwise_sum(err4);
        }
      }
      pick4 = err4 < err6;  // a tie keeps the scale-to-6 block
    }
    return pick4 ? BlockResult{c4, s4.sb, s4.e, 1u} : BlockResult{c6, s6.sb, s6.e, 0u};
  }
}

// One 16-element block held by one lane.  den6: fl(6 * S_t), den4: fl(4 * S_t).
template <bool SR, int RULE, bool EST = false>
__device__ __forceinline__ BlockResult quant_block16(const float* y, const uint32_t* w, const f32x2* tab,
                                                     const Divisor& den6, const Divisor& den4) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(y[i]));
  return choose16<SR, RULE, false, EST>(y, m, w, tab, den6, den4);
}

// A 16x16 tile spread over the 16 lanes of a DPP row, one tile row per lane.
// The tile max and the candidates' errors are reduced across the row; the
// error tree over the 256 values in row-major order is the in-lane pairwise
// sum of each row followed by pairwise sums across lanes.
template <bool SR, int RULE, bool EST = false>
__device__ __forceinline__ BlockResult quant_tile_row16(const float* y, const uint32_t* w, const f32x2* tab,
                                                        const Divisor& den6, const Divisor& den4) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(y[i]));
  m = row16_max(m);
  return choose16<SR, RULE, true, EST>(y, m, w, tab, den6, den4);
}

// ----------------------------------------------------------------- MXFP4 ---

// MXFP4 (the 32-element, power-of-two-scale format that "Pretraining Large
// Language Models with NVFP4" section 1 contrasts with NVFP4), with the OCP
// Microscaling scale rule: the shared exponent is floor(log2 m) - 2 for the
// block max m (2 = the largest E2M1 exponent), stored as E8M0 with bias 127
// and floored at code 0 (2^-127, also for m = 0 and subnormal m).  For a
// normal m, floor(log2 m) + 127 is its biased exponent field.
__device__ __forceinline__ uint32_t mx_scale_code(float m) {
  const uint32_t be = __float_as_uint(m) >> 23;  // m >= 0
  return be > 2u ? be - 2u : 0u;
}

// 2^(127 - code), the factor that scales the block into the E2M1 range.  For
// finite inputs code <= 252, so the factor is a normal binary32 and y * factor
// is the exact quotient y / 2^e rounded once.
__device__ __forceinline__ float mx_inv_scale(uint32_t code) { return __uint_as_float((254u - code) << 23); }

__device__ __forceinline__ float absmax16(const float* y) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(y[i]));
  return m;
}

// Lane l reads lane l ^ 16 (ds_swizzle bitmask mode: and 0x1F, or 0, xor 0x10).
__device__ __forceinline__ float swizzle_xor16(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
}

// Codes of 16 elements of a 32-element block whose scale code is `code`.
template <bool SR>
__device__ __forceinline__ BlockCodes mx_round16(const float* y, uint32_t code, const uint32_t* w) {
  uint32_t ws[16];
  if constexpr (SR) {
#pragma unroll
    for (int k = 0; k < 16; ++k) ws[k] = (k & 1) ? (w[k] >> 1) : w[k];
  }
  return round16<SR>(y, mx_inv_scale(code), ws);
}

}  // namespace nvfp4

// Device helpers for the gfx950 MXFP4 kernels: group scale, e2m1 encoders,
// bf16 rounding and the shuffled-scale address.
//
// Sources: submission 608632 (_hw_mxfp4_quant_op, steps 1-3), submission
// 711914 (_mxfp4_quant_tile, _standalone_quant_kernel).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxfp4 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Scale byte of a group from the largest |x| given as bf16 magnitude bits
// (15 bits, sign cleared).  The f32 pattern of amax is those bits << 16.
// Adding 2^21 and masking the mantissa keeps the exponent unless the top two
// mantissa bits are both set, where it moves up by one; the e8m0 byte is
// that exponent minus 2, clamped to [0, 254] (submission 608632,
// _hw_mxfp4_quant_op, step 1).
__device__ __forceinline__ uint32_t scale_byte_from_amax(uint32_t amax_mag16) {
  uint32_t r = ((amax_mag16 << 16) + 0x00200000u) & 0xFF800000u;
  int e = (int)(r >> 23);
  e -= 2;
  e = e < 0 ? 0 : e;
  e = e > 254 ? 254 : e;
  return (uint32_t)e;
}

// Largest magnitude of 32 bf16 values held as 16 dwords (two per dword),
// as 15-bit magnitude bits.  Integer order of the magnitude bits equals
// value order for finite inputs.
__device__ __forceinline__ uint32_t amax_mag16(const uint32_t (&w)[16]) {
  u16x2 m = {0, 0};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint32_t a = w[i] & 0x7FFF7FFFu;
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, a));
  }
  return m.x > m.y ? m.x : m.y;
}

// Hardware encode.  The pages use v_cvt_scalef32_pk_fp4_f32 on two f32
// values (submission 608632, _hw_mxfp4_quant_op, step 3; submission 711914,
// _mxfp4_quant_tile_hw): it divides by the power of two whose exponent field
// is the scale operand's and writes the two codes (first value in the low
// nibble) into byte `sel` of the destination.  gfx950 also has the bf16-input
// form, v_cvt_scalef32_pk_fp4_bf16, which takes the packed pair as stored
// (low half = even element) and so needs no unpacking; bf16 -> f32 is exact,
// so both forms see the same values.  The scale float is built with
// exponent field s.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_pair_hw(uint32_t old, uint32_t w, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(old, __builtin_bit_cast(bf16x2, w), scale, SEL);
}

// Software encode of one element, written from the rounding rule itself:
// v = |x| / 2^(s-127) is exact in f32 (bf16 input, power-of-two divisor;
// results in the subnormal range are far below the first decision point).
// The e2m1 grid has spacing 0.5 below 2, 1 in [2, 4) and 2 from 4 up, so
// rounding v to that grid with rint (nearest, ties to even) gives the code
// directly; 6 is the largest value.
__device__ __forceinline__ uint32_t encode_sw(uint32_t xbits16, float inv_scale) {
  float v = __uint_as_float((xbits16 & 0x7FFFu) << 16) * inv_scale;
  v = fminf(v, 8.0f);
  uint32_t code;
  if (v < 2.0f) code = (uint32_t)__builtin_rintf(v * 2.0f);
  else if (v < 4.0f) code = (uint32_t)__builtin_rintf(v) + 2u;
  else code = min((uint32_t)__builtin_rintf(v * 0.5f) + 4u, 7u);
  return code | ((xbits16 >> 12) & 0x8u);
}

// 2^(127 - s) as f32 (s in [0, 254]; s = 254 gives the subnormal 2^-127).
__device__ __forceinline__ float inv_scale_f32(uint32_t s) {
  return s < 254 ? __uint_as_float((254u - s) << 23) : __uint_as_float(0x00400000u);
}

// Quantize one 32-element group (16 dwords of bf16 pairs, element 2i in the
// low half of w[i]) to 16 bytes of packed codes (q[0..3], element 2i in the
// low nibble of byte i) and return the scale byte.
template <bool SW>
__device__ __forceinline__ uint32_t quant_group32(const uint32_t (&w)[16], uint32_t (&q)[4]) {
  uint32_t s = scale_byte_from_amax(amax_mag16(w));
  if constexpr (!SW) {
    float sf = __uint_as_float(s << 23);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t d = 0;
      d = cvt_pair_hw<0>(d, w[4 * j + 0], sf);
      d = cvt_pair_hw<1>(d, w[4 * j + 1], sf);
      d = cvt_pair_hw<2>(d, w[4 * j + 2], sf);
      d = cvt_pair_hw<3>(d, w[4 * j + 3], sf);
      q[j] = d;
    }
  } else {
    float inv = inv_scale_f32(s);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t d = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        uint32_t x = w[4 * j + b];
        uint32_t lo = encode_sw(x & 0xFFFFu, inv);
        uint32_t hi = encode_sw(x >> 16, inv);
        d |= (lo | (hi << 4)) << (8 * b);
      }
      q[j] = d;
    }
  }
  return s;
}

// Two floats -> packed bf16 bits (a in the low half) by the hardware
// convert (v_cvt_pk_bf16_f32): the top 16 bits of each f32, rounded to
// nearest with ties to even on the discarded 16 (for finite inputs this is
// (u + 0x7FFF + bit 16 of u) >> 16 on the bits u, which it was checked
// against on 5.2 M values).  NaN inputs are outside the GEMM's contract.
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){a, b}, bf16x2));
}

// Byte offset of (row, group) in a shuffled scale buffer whose rows of 32
// hold gp = pad8(K/32) groups each (see mxfp4_shuffled_scale_bytes).
__device__ __forceinline__ uint32_t shuffled_scale_offset(uint32_t row, uint32_t g, uint32_t gp) {
  uint32_t in_block = ((row >> 4) & 1u) | (((g >> 2) & 1u) << 1) | ((row & 15u) << 2) | ((g & 3u) << 6);
  return in_block + ((g >> 3) << 8) + (row >> 5) * 32u * gp;
}

// Word 3 of a gfx9 buffer resource for raw (untyped) dword access.
constexpr int kRsrcWord3 = 0x00020000;

// Buffer offset that reads zeros unless `in_range`: a buffer load past the
// descriptor's size returns zeros, and every offset used with these
// descriptors is below 2^31, so setting bit 31 puts it out of range.  An OR
// with a select of two constants keeps the compiler from turning the choice
// into a branch around the load (which would force a wait for every
// outstanding load where the paths meet).
__device__ __forceinline__ int off_or_oob(bool in_range, int off) {
  return off | (in_range ? 0 : (int)0x80000000u);
}

// DPP lane patterns within groups of four lanes.
constexpr int kQuadSwap1 = 0xB1;  // quad_perm [1, 0, 3, 2]
constexpr int kQuadSwap2 = 0x4E;  // quad_perm [2, 3, 0, 1]

__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kQuadSwap1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kQuadSwap2, 0xF, 0xF, false));
  return v;
}

// Quantize 8 consecutive elements of a 32-element group (4 dwords of bf16
// pairs) whose other 24 elements sit in the three neighbouring lanes of the
// same quad: returns the lane's dword of codes and writes the scale byte.
template <bool SW>
__device__ __forceinline__ uint32_t quant_quarter_t(const u32x4 &w, uint32_t *scale) {
  u16x2 m = __builtin_bit_cast(u16x2, w.x & 0x7FFF7FFFu);
  m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w.y & 0x7FFF7FFFu));
  m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w.z & 0x7FFF7FFFu));
  m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w.w & 0x7FFF7FFFu));
  const uint32_t amax = quad_max(m.x > m.y ? m.x : m.y);
  const uint32_t s = scale_byte_from_amax(amax);
  *scale = s;
  uint32_t d = 0;
  if constexpr (!SW) {
    const float sf = __uint_as_float(s << 23);
    d = cvt_pair_hw<0>(d, w.x, sf);
    d = cvt_pair_hw<1>(d, w.y, sf);
    d = cvt_pair_hw<2>(d, w.z, sf);
    d = cvt_pair_hw<3>(d, w.w, sf);
  } else {
    const float inv = inv_scale_f32(s);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int b = 0; b < 4; ++b)
      d |= (encode_sw(ww[b] & 0xFFFFu, inv) | (encode_sw(ww[b] >> 16, inv) << 4)) << (8 * b);
  }
  return d;
}

// Runtime choice of encoder for one call site; kernels that quantize many
// quarters branch once around a loop of quant_quarter_t instead.
__device__ __forceinline__ uint32_t quant_quarter(const u32x4 &w, int sw_quant, uint32_t *scale) {
  return sw_quant ? quant_quarter_t<true>(w, scale) : quant_quarter_t<false>(w, scale);
}

}  // namespace mxfp4

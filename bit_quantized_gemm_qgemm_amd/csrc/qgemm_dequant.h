// In-register dequantization of the packed fp16-path weight formats
// (shared by the small-M and the tiled weight-only kernels).
//
// An fp16 with exponent field 25 and mantissa field m has value 1024 + m, so
// OR-ing a code into the mantissa of 0x6400 and subtracting a constant gives
// the exact small integer (W4A16 page section 2: code - 8; W8A16 page Step 1:
// the int8 weight).  Two nibbles (or bytes) become two fp16 lanes of one
// register per operation; the per-column scale is applied later to the fp32
// sum, where it is exact to factor it out.
//
// This exponent-bias conversion is the published technique of Kim et al.,
// "Who Says Elephants Can't Run: Bringing Large Scale MoE Models into Cloud
// Scale Production" (2022), with the INT4 nibble interleave of NVIDIA's
// FasterTransformer: the fp16 format fixes its constants (0x6400 = 1024,
// 1024 + 8 = 1032 to remove the bias and the zero point, 1/16 and -72 for the
// nibble that sits four bits higher), so any implementation of the method
// uses the same ones.
#pragma once

#include "qgemm_common.h"

namespace qgemm {

// A 32-bit constant materialised in a VGPR, so that AND-OR can take it as a
// register operand next to a scalar one (gfx9 VOP3 reads at most one scalar).
__device__ __forceinline__ uint32_t vgpr_const(uint32_t c) {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
  return r;
}

struct W4Masks {
  uint32_t lo, hi;  // 0x000f000f, 0x00f000f0 held in VGPRs
};

// Eight INT4 codes (nibble order k0,k2,k4,k6,k1,k3,k5,k7) -> code - 8 as fp16.
__device__ __forceinline__ half8_t dequant_w4(uint32_t q, W4Masks mk) {
  const uint32_t magic = 0x64006400u;       // fp16 1024 in both halves
  const uint32_t t0 = (q & mk.lo) | magic;  // 1024 + c       (k0, k1)
  const uint32_t t1 = (q & mk.hi) | magic;  // 1024 + 16 c    (k2, k3)
  const uint32_t q2 = q >> 8;
  const uint32_t t2 = (q2 & mk.lo) | magic;  //               (k4, k5)
  const uint32_t t3 = (q2 & mk.hi) | magic;  //               (k6, k7)
  const half2_t sub = {(_Float16)1032.0f, (_Float16)1032.0f};
  const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const half2_t off = {(_Float16)-72.0f, (_Float16)-72.0f};
  const half2_t h0 = __builtin_bit_cast(half2_t, t0) - sub;
  const half2_t h1 = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, t1), sixteenth, off);
  const half2_t h2 = __builtin_bit_cast(half2_t, t2) - sub;
  const half2_t h3 = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, t3), sixteenth, off);
  return half8_t{h0.x, h0.y, h1.x, h1.y, h2.x, h2.y, h3.x, h3.y};
}

// Same result as dequant_w4 from shifts, AND-OR and packed subtracts only
// (11 VALU ops, no packed fma): nibble j of q holds k_{2j} and nibble j + 4
// holds k_{2j+1}, so (q >> 4j) & 0x000f000f puts that pair in the two fp16
// halves.
__device__ __forceinline__ half8_t dequant_w4_shift(uint32_t q) {
  const uint32_t magic = 0x64006400u;
  const half2_t sub = {(_Float16)1032.0f, (_Float16)1032.0f};
  const half2_t h0 = __builtin_bit_cast(half2_t, (q & 0x000f000fu) | magic) - sub;
  const half2_t h1 = __builtin_bit_cast(half2_t, ((q >> 4) & 0x000f000fu) | magic) - sub;
  const half2_t h2 = __builtin_bit_cast(half2_t, ((q >> 8) & 0x000f000fu) | magic) - sub;
  const half2_t h3 = __builtin_bit_cast(half2_t, ((q >> 12) & 0x000f000fu) | magic) - sub;
  return half8_t{h0.x, h0.y, h1.x, h1.y, h2.x, h2.y, h3.x, h3.y};
}

// Grouped formats: e = {low: fp16 1024 + z (W4) or 1152 + z (W8), high:
// fp16 scale}.  (1024 + code) - (1024 + z) is exact, so each weight becomes
// (w - z) * s rounded once to fp16 (the W4A16 page's section-1 dequant).
__device__ __forceinline__ half8_t dequant_w4_group(uint32_t q, uint32_t e) {
  const half2_t me = __builtin_bit_cast(half2_t, e);
  const half2_t zc = {me.x, me.x};
  const half2_t sc = {me.y, me.y};
  const uint32_t magic = 0x64006400u;
  const half2_t h0 = (__builtin_bit_cast(half2_t, (q & 0x000f000fu) | magic) - zc) * sc;
  const half2_t h1 = (__builtin_bit_cast(half2_t, ((q >> 4) & 0x000f000fu) | magic) - zc) * sc;
  const half2_t h2 = (__builtin_bit_cast(half2_t, ((q >> 8) & 0x000f000fu) | magic) - zc) * sc;
  const half2_t h3 = (__builtin_bit_cast(half2_t, ((q >> 12) & 0x000f000fu) | magic) - zc) * sc;
  return half8_t{h0.x, h0.y, h1.x, h1.y, h2.x, h2.y, h3.x, h3.y};
}

// The same without the scale, w - z exact in fp16 (the caller applies s to
// the fp32 sum of a whole group), in dequant_w4's form: the low nibble of a
// byte gives (1024 + code) - (1024 + z), the high one 16 code + 1024 times
// 1/16 minus (64 + z); 1024 + z - 960 = 64 + z is exact.
__device__ __forceinline__ half8_t dequant_w4_group_unscaled(uint32_t q, uint32_t e,
                                                             W4Masks mk) {
  const half2_t me = __builtin_bit_cast(half2_t, e);
  const half2_t zc = {me.x, me.x};
  const half2_t d960 = {(_Float16)960.0f, (_Float16)960.0f};
  const half2_t zc16 = zc - d960;
  const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const uint32_t magic = 0x64006400u;
  const uint32_t q2 = q >> 8;
  const half2_t h0 = __builtin_bit_cast(half2_t, (q & mk.lo) | magic) - zc;
  const half2_t h1 =
      __builtin_elementwise_fma(__builtin_bit_cast(half2_t, (q & mk.hi) | magic), sixteenth, -zc16);
  const half2_t h2 = __builtin_bit_cast(half2_t, (q2 & mk.lo) | magic) - zc;
  const half2_t h3 =
      __builtin_elementwise_fma(__builtin_bit_cast(half2_t, (q2 & mk.hi) | magic), sixteenth, -zc16);
  return half8_t{h0.x, h0.y, h1.x, h1.y, h2.x, h2.y, h3.x, h3.y};
}

__device__ __forceinline__ half8_t dequant_w8_group(uint32_t lo, uint32_t hi, uint32_t e) {
  const half2_t me = __builtin_bit_cast(half2_t, e);
  const half2_t zc = {me.x, me.x};
  const half2_t sc = {me.y, me.y};
  const half2_t a = (__builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, lo, 0x04010400u)) - zc) * sc;
  const half2_t b = (__builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, lo, 0x04030402u)) - zc) * sc;
  const half2_t c = (__builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, hi, 0x04010400u)) - zc) * sc;
  const half2_t d = (__builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, hi, 0x04030402u)) - zc) * sc;
  return half8_t{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// NVFP4 weights: the 8 E2M1 codes of word q (natural order) times the e4m3
// block scale in the low byte of sc8.  The hardware FP4 -> fp16 conversion
// is exact at scale 1.0, and an E2M1 value (2 significant bits) times an
// e4m3 value (4 significant bits, 2^-9 .. 448) is exact in fp16, so each
// weight is e2m1 * scale exactly (the per-tensor scale multiplies the fp32
// sum later).
__device__ __forceinline__ half8_t dequant_nvfp4(uint32_t q, uint32_t sc8) {
  const _Float16 sh = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)sc8, 0);
  const half2_t sc = {sh, sh};
  const half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 0) * sc;
  const half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 1) * sc;
  const half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 2) * sc;
  const half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 3) * sc;
  return half8_t{h0.x, h0.y, h1.x, h1.y, h2.x, h2.y, h3.x, h3.y};
}

// Grouped INT8 without the scale: (1024 + w + 128) - (1152 + z) = w - z,
// exact in fp16 (the caller applies s to the fp32 sum of a whole group).
__device__ __forceinline__ half8_t dequant_w8_group_unscaled(uint32_t lo, uint32_t hi,
                                                             uint32_t e) {
  const half2_t me = __builtin_bit_cast(half2_t, e);
  const half2_t zc = {me.x, me.x};
  const half2_t a = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, lo, 0x04010400u)) - zc;
  const half2_t b = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, lo, 0x04030402u)) - zc;
  const half2_t c = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, hi, 0x04010400u)) - zc;
  const half2_t d = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, hi, 0x04030402u)) - zc;
  return half8_t{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// Two biased INT8 bytes (w + 128) of a word, selected by `sel`, -> w as fp16.
__device__ __forceinline__ half2_t dequant_w8_pair(uint32_t d, uint32_t sel) {
  // byte permute of {0x64646464 : d}: selector 0..3 picks bytes of d, 4 picks 0x64
  const uint32_t t = __builtin_amdgcn_perm(0x64646464u, d, sel);
  const half2_t sub = {(_Float16)1152.0f, (_Float16)1152.0f};  // 1024 + 128
  return __builtin_bit_cast(half2_t, t) - sub;
}

__device__ __forceinline__ half8_t dequant_w8(uint32_t lo, uint32_t hi) {
  const half2_t a = dequant_w8_pair(lo, 0x04010400u);  // bytes 0, 1
  const half2_t b = dequant_w8_pair(lo, 0x04030402u);  // bytes 2, 3
  const half2_t c = dequant_w8_pair(hi, 0x04010400u);
  const half2_t d = dequant_w8_pair(hi, 0x04030402u);
  return half8_t{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

}  // namespace qgemm

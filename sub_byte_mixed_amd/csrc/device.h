// Device helpers for the gfx950 kernels: bf16 unpacking, Philox4x32-10,
// E2M1 / E4M3 / E8M0 encoders and decoders, wave reductions.
//
// Formats: "FP4 All the Way" summary, Outline (E2M1 elements, E4M3 block
// scale per 16); rounding: same page (nearest forward, stochastic backward)
// and "Research on Mixed-Precision Training for LLMs", Core Techniques
// (stochastic rounding keeps the expectation).
//
// Every encoder works on the fp32 bit pattern of a non-negative magnitude.
// Round-to-nearest-even adds (half-ulp - 1 + lsb) below the kept bits and
// truncates; stochastic rounding adds the 16 random bits aligned to the top
// of the discarded field and truncates, which rounds up with probability
// floor(frac * 2^16) / 2^16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace snip {

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// 2^e as a float for e in [-126, 127]
__device__ __forceinline__ float exp2i(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// ---------------------------------------------------------------- Philox4x32-10
// Salmon et al., SC'11: ten rounds of two 32x32->64 multiplies with a Weyl
// key schedule.
struct Words4 { uint32_t w[4]; };

__device__ __forceinline__ Words4 philox10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                           uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    // three-way xors as one v_bitop3_b32 each (truth table 0x96)
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  Words4 o;
  o.w[0] = c0; o.w[1] = c1; o.w[2] = c2; o.w[3] = c3;
  return o;
}

// 16 random bits for the 8 elements idx = 8*g .. 8*g+7, element i in the
// half (i & 1) of word (i >> 1).
__device__ __forceinline__ Words4 draws8(uint64_t seed, uint32_t tensor_id, uint64_t g) {
  return philox10((uint32_t)g, (uint32_t)(g >> 32), tensor_id, 0u,
                  (uint32_t)seed, (uint32_t)(seed >> 32));
}
__device__ __forceinline__ uint32_t r16_of(const Words4& d, int i) {
  return (d.w[(i >> 1) & 3] >> ((i & 1) * 16)) & 0xFFFFu;
}

// ---------------------------------------------------------------- E2M1
// magnitude index 0..7 <-> {0, .5, 1, 1.5, 2, 3, 4, 6}
__device__ __forceinline__ uint32_t e2m1_rne(float a) {      // a >= 0
  if (a < 1.0f) return (uint32_t)__builtin_rintf(a * 2.0f); // 0, 1, 2 (ties even)
  const uint32_t b = __float_as_uint(a);
  const uint32_t rb = b + 0x1FFFFFu + ((b >> 22) & 1u);
  const uint32_t m = (rb >> 22) - 252u;
  return m > 7u ? 7u : m;
}

__device__ __forceinline__ uint32_t e2m1_sr(float a, uint32_t r16) {   // a >= 0
  if (a >= 6.0f) return 7u;
  if (a < 1.0f) {                                 // spacing 0.5: 2^17 fixed point
    const uint32_t t = (uint32_t)(a * 131072.0f);
    return (t >> 16) + (((t & 0xFFFFu) + r16) >> 16);
  }
  const uint32_t b = __float_as_uint(a);
  return (b >> 22) - 252u + ((((b >> 6) & 0xFFFFu) + r16) >> 16);
}

// E2M1 magnitude index -> fp32 value: the 3 bits read as an fp32 exponent
// (2 bits, bias 127) and mantissa bit, rescaled by 2^126 (exact).
__device__ __forceinline__ float e2m1_val(uint32_t m) {
  return __uint_as_float(m << 22) * 8.50705917302346159e+37f /* 2^126 */;
}

// ---------------------------------------------------------------- E4M3 (fn)
__device__ __forceinline__ uint32_t e4m3_rne(float a) {      // a >= 0, saturating
  if (a < 0.015625f) return (uint32_t)__builtin_rintf(a * 512.0f);   // subnormal: step 2^-9
  const uint32_t b = __float_as_uint(a);
  const uint32_t rb = b + 0x7FFFFu + ((b >> 20) & 1u);
  const uint32_t c = (rb >> 20) - 960u;
  return c > 0x7Eu ? 0x7Eu : c;
}

__device__ __forceinline__ uint32_t e4m3_sr(float a, uint32_t r16) {  // a >= 0
  if (a >= 448.0f) return 0x7Eu;
  if (a < 0.015625f) {                            // step 2^-9: 2^25 fixed point
    const uint32_t t = (uint32_t)(a * 33554432.0f);
    return (t >> 16) + (((t & 0xFFFFu) + r16) >> 16);
  }
  const uint32_t b = __float_as_uint(a);
  const uint32_t c = (b >> 20) - 960u + ((((b >> 4) & 0xFFFFu) + r16) >> 16);
  return c > 0x7Eu ? 0x7Eu : c;
}

// E4M3 magnitude code (0..126) -> fp32 (exact): bits placed as an fp32 with
// a 4-bit exponent field, rescaled by 2^120.
__device__ __forceinline__ float e4m3_val(uint32_t c) {
  return __uint_as_float(c << 20) * 1.32922799578491587e+36f /* 2^120 */;
}

// ---------------------------------------------------------------- hardware converts
// gfx950 conversion instructions with unit scale:
//   v_cvt_scalef32_pk_fp4_f32     E2M1, round to nearest even, saturating;
//   v_cvt_scalef32_sr_pk_fp4_f32  E2M1, stochastic: the 32-bit random operand,
//                                 shifted right to align with the discarded
//                                 mantissa bits, is added and the result
//                                 truncated;
//   v_cvt_scalef32_pk_fp8_f32, v_cvt_scalef32_sr_fp8_f32  E4M3 likewise, but
//                                 not saturating: inputs are clamped to +-448;
//   v_cvt_scalef32_pk_f32_fp4 / _fp8  decoders.
// With R16 in the top half of the random operand the stochastic rule is
// exactly that of e2m1_sr / e4m3_sr above. The stochastic FP4 convert shares
// its random word between its two lanes and does not keep the other bytes of
// its destination, so it is issued once per element (lane 0, byte 0) and the
// nibble is masked and placed by hand (measured: the bits above the nibble
// are not zero). The stochastic FP8 convert with a zero `old` operand leaves
// only the code byte set. Every helper below is checked against the software
// encoders over all fp32 inputs (tests/helpers/hw_convert_check.hip).
typedef float f2_t __attribute__((ext_vector_type(2)));
typedef short s2_t __attribute__((ext_vector_type(2)));

// R16 of element i of a Philox block (i in 0..7) in the top half of a word.
__device__ __forceinline__ uint32_t sr_seed(const Words4& d, int i) {
  const uint32_t w = d.w[(i >> 1) & 3];
  return (i & 1) ? (w & 0xFFFF0000u) : (w << 16);
}

// 8 scaled values -> 8 E2M1 codes in one word (element i in nibble i), RNE.
__device__ __forceinline__ uint32_t fp4x8_rne(const float* r) {
  uint32_t w = 0u;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, r[0], r[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, r[2], r[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, r[4], r[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, r[6], r[7], 1.0f, 3);
  return w;
}

// 8 scaled values -> 8 E2M1 codes, stochastic, element i drawing R16 from d.
__device__ __forceinline__ uint32_t fp4x8_sr(const float* r, const Words4& d) {
  uint32_t w = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t c = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, f2_t{r[i], 0.0f},
                                                                   sr_seed(d, i), 1.0f, 0);
    w |= (c & 0xFu) << (4 * i);
  }
  return w;
}

// Decoded (signed) E2M1 values of the 8 codes of a word.
__device__ __forceinline__ void fp4x8_dec(uint32_t w, float* q) {
  const f2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const f2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const f2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const f2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  q[0] = v0[0]; q[1] = v0[1]; q[2] = v1[0]; q[3] = v1[1];
  q[4] = v2[0]; q[5] = v2[1]; q[6] = v3[0]; q[7] = v3[1];
}

// 4 values clamped to +-448 -> 4 E4M3 codes (byte b = element b), RNE.
__device__ __forceinline__ uint32_t fp8x4_rne(const float* c) {
  s2_t w = {0, 0};
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, c[0], c[1], 1.0f, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, c[2], c[3], 1.0f, true);
  return __builtin_bit_cast(uint32_t, w);
}

// 4 values clamped to +-448 -> 4 E4M3 codes, stochastic; element b draws
// R16 of element (first + b) of the Philox block d.
__device__ __forceinline__ uint32_t fp8x4_sr(const float* c, const Words4& d, int first) {
  uint32_t w = 0u;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint32_t v = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(0u, c[b], sr_seed(d, first + b), 1.0f, 0);
    w |= v << (8 * b);             // v holds the code in its low byte only
  }
  return w;
}

// Decoded (signed) E4M3 values of the 4 codes of a word.
__device__ __forceinline__ void fp8x4_dec(uint32_t w, float* q) {
  const f2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
  const f2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true);
  q[0] = a[0]; q[1] = a[1]; q[2] = b[0]; q[3] = b[1];
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ uint32_t wave_sum_u(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t t = __shfl_xor(v, o, 64);
    v = t > v ? t : v;
  }
  return v;
}

}  // namespace snip

// Device helpers shared by the quantizer kernels (quantize.hip,
// quantize_dual.hip): job lookup, tensor exponent, workgroup reductions of
// the tensor max and of the statistics, and the per-block codecs.
//
// "FP4 All the Way" summary, Outline: 16 E2M1 values share an E4M3 scale;
// nearest rounding forward, stochastic rounding backward and in the update.
#pragma once

#include "device.h"
#include "kernels.h"

namespace snip {

// ------------------------------------------------------------ common
__device__ __forceinline__ int find_job(const int32_t* wg0, int n) {
  int j = 0;
  for (int i = 1; i < n; ++i)
    if ((int)blockIdx.x >= wg0[i]) j = i;
  return j;
}

// Tensor exponent: smallest e with A * 2^-e <= limit, limit = 6*448 (NVFP4)
// or 448 (FP8); 0 for A == 0.
__device__ __forceinline__ int tensor_exp(float A, int format) {
  if (!(A > 0.0f)) return 0;
  int e1;
  const float f = frexpf(A, &e1);   // A = f * 2^e1, f in [0.5, 1)
  if (format == SNIP_NVFP4) return e1 - 12 + (f > 0.65625f ? 1 : 0);   // 2688 = 0.65625 * 2^12
  if (format == SNIP_FP8_E4M3) return e1 - 9 + (f > 0.875f ? 1 : 0);   //  448 = 0.875 * 2^9
  return 0;
}

// Workgroup reduction of the amax partials (or the delayed-scaling value).
__device__ inline float wg_tensor_amax(const float* amax_in, const uint32_t* amax_part, int n_amax_part,
                                      uint32_t* red) {
  if (amax_in) return *amax_in;
  uint32_t m = 0;
  for (int i = threadIdx.x; i < n_amax_part; i += blockDim.x) {
    const uint32_t v = amax_part[i];
    m = v > m ? v : m;
  }
  m = wave_max_u(m);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = m;
  __syncthreads();
  m = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) m = red[w] > m ? red[w] : m;
  __syncthreads();
  return __uint_as_float(m << 16);
}

// Workgroup reduction of one thread's statistics into part[wg].
__device__ inline void wg_store_stats(StatPart* part, double e2, double x2, uint32_t nf,
                               uint32_t amax_bits, double* dred, uint32_t* ured) {
  e2 = wave_sum(e2);
  x2 = wave_sum(x2);
  nf = wave_sum_u(nf);
  amax_bits = wave_max_u(amax_bits);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    dred[2 * wave] = e2;
    dred[2 * wave + 1] = x2;
    ured[2 * wave] = nf;
    ured[2 * wave + 1] = amax_bits;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    StatPart p{0.0, 0.0, 0u, 0u};
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
      p.e2 += dred[2 * w];
      p.x2 += dred[2 * w + 1];
      p.nf += ured[2 * w];
      p.amax_bits = ured[2 * w + 1] > p.amax_bits ? ured[2 * w + 1] : p.amax_bits;
    }
    *part = p;
  }
}

// ------------------------------------------------------------ block codecs
// Element encoding and the decode for the statistics use the gfx950
// conversion instructions through the packed helpers of device.h.

__device__ __forceinline__ void fill_inv_lut(float* lut) {
  if (threadIdx.x < 128) lut[threadIdx.x] = threadIdx.x ? 1.0f / e4m3_val(threadIdx.x) : 0.0f;
  __syncthreads();
}

// NVFP4: 16 raw values x -> 16 packed nibbles (lo: elements 0..7, hi: 8..15),
// the E4M3 block scale and the block's stats in the tensor-scaled domain.
// inv_lut[c] = fp32(1 / e4m3(c)) (IEEE division, filled once per workgroup
// by fill_inv_lut), 0 for c = 0.
template <bool SR>
__device__ __forceinline__ void nvfp4_block(const float (&x)[16], int eS, const Words4& d0,
                                            const Words4& d1, const float* inv_lut, uint32_t& lo,
                                            uint32_t& hi, uint32_t& sc, float& be2, float& bx2) {
  float xs[16];
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    xs[i] = ldexpf(x[i], -eS);
    am = fmaxf(am, fabsf(xs[i]));
  }
  sc = e4m3_rne(am / 6.0f);
  const float shat = e4m3_val(sc);
  const float inv = inv_lut[sc];                  // 0 for a zero block: signed-zero codes
  float r[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) r[i] = xs[i] * inv;
  if (SR) {
    lo = fp4x8_sr(r, d0);
    hi = fp4x8_sr(r + 8, d1);
  } else {
    lo = fp4x8_rne(r);
    hi = fp4x8_rne(r + 8);
  }
  float q[16];
  fp4x8_dec(lo, q);
  fp4x8_dec(hi, q + 8);
  be2 = 0.0f;
  bx2 = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float err = fmaf(q[i], shat, -xs[i]);
    be2 = fmaf(err, err, be2);
    bx2 = fmaf(xs[i], xs[i], bx2);
  }
}

// FP8-E4M3: 16 raw values -> 16 code bytes (4 words), stats in the scaled domain.
template <bool SR>
__device__ __forceinline__ void fp8_chunk(const float (&x)[16], int eS, const Words4& d0,
                                          const Words4& d1, uint32_t (&out)[4], float& be2,
                                          float& bx2) {
  float r[16], c[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    r[i] = ldexpf(x[i], -eS);
    c[i] = __builtin_amdgcn_fmed3f(r[i], -448.0f, 448.0f);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k)
    out[k] = SR ? fp8x4_sr(c + 4 * k, k < 2 ? d0 : d1, (4 * k) & 7) : fp8x4_rne(c + 4 * k);
  be2 = 0.0f;
  bx2 = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float q[4];
    fp8x4_dec(out[k], q);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float e = q[b] - r[4 * k + b];
      be2 = fmaf(e, e, be2);
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) bx2 = fmaf(r[i], r[i], bx2);
}

// MX-FP4: 32 raw values -> 32 nibbles (4 words), E8M0 scale; stats are
// returned already scaled back (fp64) since the scale varies per block.
template <bool SR>
__device__ __forceinline__ void mx_block(const float (&x)[32], const Words4 (&d)[4],
                                         uint32_t (&out)[4], uint32_t& sc, double& e2,
                                         double& x2, float& bx2_scaled, float& am) {
  am = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(x[i]));
  int X = -127;
  if (am > 0.0f) {
    const int e = (int)(__float_as_uint(am) >> 23);      // biased exponent (0: subnormal)
    X = e - 129;                                          // floor(log2 am) - 2
    X = X < -127 ? -127 : X;
  }
  sc = (uint32_t)(X + 127);
  const float pw = am > 0.0f ? exp2i(-X) : 0.0f;          // exact power of two (0: zero block)
  float r[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) r[i] = x[i] * pw;
#pragma unroll
  for (int k = 0; k < 4; ++k) out[k] = SR ? fp4x8_sr(r + 8 * k, d[k]) : fp4x8_rne(r + 8 * k);
  float be2 = 0.0f, bx2 = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float q[8];
    fp4x8_dec(out[k], q);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float err = q[i] - r[8 * k + i];
      be2 = fmaf(err, err, be2);
      bx2 = fmaf(r[8 * k + i], r[8 * k + i], bx2);
    }
  }
  e2 = ldexp((double)be2, 2 * X);
  x2 = ldexp((double)bx2, 2 * X);
  bx2_scaled = bx2;
}

// Non-finite slow path: count the NaN / Inf inputs, and recompute the raw
// sum of squares and the max over the finite elements (the codes of such a
// block are unspecified).
template <int N>
__device__ __forceinline__ void nonfinite_stats(const float (&x)[N], uint32_t& nf, double& x2,
                                             uint32_t& amax_bits) {
  nf = 0u;
  x2 = 0.0;
  for (int i = 0; i < N; ++i) {
    if (isfinite(x[i])) {
      x2 += (double)x[i] * (double)x[i];
      const uint32_t b = __float_as_uint(fabsf(x[i]));
      amax_bits = b > amax_bits ? b : amax_bits;
    } else {
      ++nf;
    }
  }
}

// max |x| of a block whose values are all finite, as fp32 bits: the
// current tensor's max is reported from these when the tensor scale comes
// from a supplied max (a block with a non-finite value takes the finite max
// nonfinite_stats finds instead).
template <int N>
__device__ __forceinline__ uint32_t block_absmax_bits(const float (&x)[N]) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < N; ++i) m = fmaxf(m, fabsf(x[i]));
  return __float_as_uint(m);
}

__device__ __forceinline__ void unpack16(const uint4& v0, const uint4& v1, float (&x)[16]) {
  const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[2 * i] = bf16_lo(w[i]);
    x[2 * i + 1] = bf16_hi(w[i]);
  }
}


}  // namespace snip

// Exhaustive check of the packed hardware-conversion helpers the kernels use
// (sub_byte_mixed_amd/csrc/device.h) against the library's software
// encoders in the same header, which the parity tests pin bit-exactly to the
// CPU oracle.
//
// For every 32-bit pattern u, element k of a word gets the input
// x_k = bits(u ^ (k << 20)), so each element position sees every fp32 value
// (NaN inputs are skipped: outside the contract).
//   fp4_rne  fp4x8_rne (v_cvt_scalef32_pk_fp4_f32)                vs e2m1_rne
//   fp4_sr   fp4x8_sr  (v_cvt_scalef32_sr_pk_fp4_f32), 8 random-word patterns
//                                                                 vs e2m1_sr
//   fp8_rne  fp8x4_rne of the input clamped to +-448               vs e4m3_rne
//   fp8_sr   fp8x4_sr  of the clamped input, both halves of a Philox block
//                                                                 vs e4m3_sr
//   fp4_dec  fp4x8_dec on every word                    vs the E2M1 value table
//   fp8_dec  fp8x4_dec on every word without NaN codes  vs the E4M3 value table
//   fp4_f16  the NVFP4 GEMM decode (v_cvt_scalef32_pk_f16_fp4 x fp16 mantissa)
//            for all 16 codes x 127 E4M3 scales        vs code x scale
// Prints one JSON object; exit status 0 iff no check has a mismatch.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <vector>

#include "../../sub_byte_mixed_amd/csrc/device.h"

using namespace snip;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int NCHECK = 7;
enum { FP4_RNE, FP4_SR, FP8_RNE, FP8_SR, FP4_DEC, FP8_DEC, FP4_F16 };
const char* kNames[NCHECK] = {"fp4_rne", "fp4_sr", "fp8_rne", "fp8_sr", "fp4_dec", "fp8_dec", "fp4_f16"};

__device__ __forceinline__ uint32_t mix(uint32_t x) {       // integer hash for test draws
  x ^= x >> 16; x *= 0x7FEB352Du; x ^= x >> 15; x *= 0x846CA68Bu; x ^= x >> 16;
  return x;
}

__device__ __forceinline__ float clamp448(float x) { return __builtin_amdgcn_fmed3f(x, -448.0f, 448.0f); }

__global__ __launch_bounds__(256) void sweep(unsigned long long* counts, uint32_t* first) {
  __shared__ unsigned long long sc[NCHECK][256];
  __shared__ uint32_t sf[NCHECK][256];
  unsigned long long c[NCHECK] = {0, 0, 0, 0, 0, 0, 0};
  uint32_t f[NCHECK];
  for (int k = 0; k < NCHECK; ++k) f[k] = 0xFFFFFFFFu;
  auto miss = [&](int k, uint32_t u) { ++c[k]; f[k] = min(f[k], u); };
  const uint64_t nthr = (uint64_t)gridDim.x * 256;
  for (uint64_t u64 = (uint64_t)blockIdx.x * 256 + threadIdx.x; u64 < (1ull << 32); u64 += nthr) {
    const uint32_t u = (uint32_t)u64;
    float x[8];
    bool ok[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float v = __uint_as_float(u ^ ((uint32_t)k << 20));
      ok[k] = v == v;
      x[k] = ok[k] ? v : 0.0f;
    }
    // ---- E2M1, round to nearest
    {
      const uint32_t w = fp4x8_rne(x);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t want = e2m1_rne(fabsf(x[k])) | ((__float_as_uint(x[k]) >> 28) & 8u);
        if (ok[k] && ((w >> (4 * k)) & 0xFu) != want) miss(FP4_RNE, u);
      }
    }
    // ---- E2M1 and E4M3 stochastic, 8 random-word patterns
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      Words4 d;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        d.w[j] = t == 0 ? 0u : t == 1 ? 0xFFFFFFFFu : t == 2 ? 0x80008000u : t == 3 ? 0x7FFF7FFFu
                                                         : mix(u * 32u + (uint32_t)(4 * t + j));
      const uint32_t w = fp4x8_sr(x, d);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t want = e2m1_sr(fabsf(x[k]), r16_of(d, k)) | ((__float_as_uint(x[k]) >> 28) & 8u);
        if (ok[k] && ((w >> (4 * k)) & 0xFu) != want) miss(FP4_SR, u);
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float cl[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) cl[b] = clamp448(x[4 * half + b]);
        const uint32_t w8 = fp8x4_sr(cl, d, 4 * half);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const float v = x[4 * half + b];
          const uint32_t want = e4m3_sr(fabsf(v), r16_of(d, 4 * half + b)) | ((__float_as_uint(v) >> 24) & 0x80u);
          if (ok[4 * half + b] && ((w8 >> (8 * b)) & 0xFFu) != want) miss(FP8_SR, u);
        }
      }
    }
    // ---- E4M3, round to nearest
    {
      float cl[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) cl[b] = clamp448(x[b]);
      const uint32_t w8 = fp8x4_rne(cl);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t want = e4m3_rne(fabsf(x[b])) | ((__float_as_uint(x[b]) >> 24) & 0x80u);
        if (ok[b] && ((w8 >> (8 * b)) & 0xFFu) != want) miss(FP8_RNE, u);
      }
    }
    // ---- decoders on the word u
    {
      float q[8];
      fp4x8_dec(u, q);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t n = (u >> (4 * k)) & 0xFu;
        const float want = ((n & 8u) ? -1.0f : 1.0f) * e2m1_val(n & 7u);
        if (__float_as_uint(q[k]) != __float_as_uint(want)) miss(FP4_DEC, u);
      }
      bool nan8 = false;
#pragma unroll
      for (int b = 0; b < 4; ++b) nan8 = nan8 || ((u >> (8 * b)) & 0x7Fu) == 0x7Fu;
      if (!nan8) {
        float e[4];
        fp8x4_dec(u, e);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const uint32_t cb = (u >> (8 * b)) & 0xFFu;
          const float want = ((cb & 0x80u) ? -1.0f : 1.0f) * e4m3_val(cb & 0x7Fu);
          if (__float_as_uint(e[b]) != __float_as_uint(want)) miss(FP8_DEC, u);
        }
      }
    }
    // ---- NVFP4 GEMM decode: E2M1 code (u % 16) x E4M3 scale code (u / 16)
    if (u < 16u * 127u) {
      const uint32_t code = u & 15u, s = u >> 4;
      float p2;
      _Float16 m;
      if (s >= 8u) { p2 = exp2i((int)(s >> 3) - 7); m = (_Float16)(1.0f + 0.125f * (float)(s & 7u)); }
      else { p2 = exp2i(-9); m = (_Float16)(float)s; }
      const half2_t mm = {m, m};
      const half2_t h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(code, p2, 0) * mm;
      const float want = ((code & 8u) ? -1.0f : 1.0f) * e2m1_val(code & 7u) * e4m3_val(s);
      if ((float)h[0] != want) miss(FP4_F16, u);
    }
  }
  for (int k = 0; k < NCHECK; ++k) { sc[k][threadIdx.x] = c[k]; sf[k][threadIdx.x] = f[k]; }
  __syncthreads();
  if (threadIdx.x < NCHECK) {
    const int k = threadIdx.x;
    unsigned long long s = 0;
    uint32_t m = 0xFFFFFFFFu;
    for (int i = 0; i < 256; ++i) { s += sc[k][i]; m = min(m, sf[k][i]); }
    counts[blockIdx.x * NCHECK + k] = s;
    first[blockIdx.x * NCHECK + k] = m;
  }
}

int main() {
  const int grid = 8192;
  unsigned long long* dc;
  uint32_t* df;
  if (hipMalloc(&dc, sizeof(unsigned long long) * grid * NCHECK) != hipSuccess ||
      hipMalloc(&df, sizeof(uint32_t) * grid * NCHECK) != hipSuccess) {
    std::printf("{\"error\": \"hipMalloc failed\"}\n");
    return 2;
  }
  hipLaunchKernelGGL(sweep, dim3(grid), dim3(256), 0, 0, dc, df);
  if (hipDeviceSynchronize() != hipSuccess) {
    std::printf("{\"error\": \"kernel failed\"}\n");
    return 2;
  }
  std::vector<unsigned long long> hc((size_t)grid * NCHECK);
  std::vector<uint32_t> hf((size_t)grid * NCHECK);
  if (hipMemcpy(hc.data(), dc, hc.size() * sizeof(hc[0]), hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(hf.data(), df, hf.size() * sizeof(hf[0]), hipMemcpyDeviceToHost) != hipSuccess) {
    std::printf("{\"error\": \"copy failed\"}\n");
    return 2;
  }
  bool all = true;
  std::printf("{");
  for (int k = 0; k < NCHECK; ++k) {
    unsigned long long s = 0;
    uint32_t m = 0xFFFFFFFFu;
    for (int b = 0; b < grid; ++b) {
      s += hc[(size_t)b * NCHECK + k];
      m = m < hf[(size_t)b * NCHECK + k] ? m : hf[(size_t)b * NCHECK + k];
    }
    all = all && s == 0;
    std::printf("%s\"%s\": {\"mismatches\": %llu, \"first\": \"0x%08x\"}", k ? ", " : "", kNames[k], s, m);
  }
  std::printf("}\n");
  (void)hipFree(dc);
  (void)hipFree(df);
  return all ? 0 : 1;
}

// Accuracy of gfx950's 8-bit matrix instructions on E4M3 x E4M3 products,
// against the exact result, for the choice of the FP8 GEMM path.
//
// Each trial is one 16 x 16 x 128 tile (one wave): A[16][128] and B[16][128]
// E4M3 codes, C = A . B^T computed three ways with fp32 accumulation:
//   scale_f8f6f4  one v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 operands, unit
//                 E8M0 block scales)
//   fp8_fp8       four v_mfma_f32_16x16x32_fp8_fp8
//   f16_decode    the codes converted exactly to fp16
//                 (v_cvt_scalef32_pk_f16_fp8), four v_mfma_f32_16x16x32_f16:
//                 the path the FP8 GEMM kernels take
// Every lane loads the same K positions of its A row and B column, so each
// variant sums the same 128 products (in some order). The host computes the
// exact products in fp64 and reports, per variant, the worst and mean
// |C - C_exact| / sum_k |a_k b_k| (the parity bound is 1e-5).
//
// Two data sets of 4096 tiles each:
//   full    uniformly random finite E4M3 codes (magnitudes 2^-9 .. 448)
//   gauss   E4M3 round-to-nearest of N(0, 1) data scaled to a tensor max of
//           448 (the values a quantized activation tile holds)
// Prints one JSON object. Exit status 0 iff f16_decode stays within 1e-6.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <vector>

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));

constexpr int K = 128;
constexpr int NV = 3;

__device__ __forceinline__ half8 dec8(uint32_t w0, uint32_t w1) {
  const half2 h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
  const half2 h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
  const half2 h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
  const half2 h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
  return half8{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// one wave per trial; A, B: [trials][16][K] codes; D: [trials][NV][16][16]
__global__ __launch_bounds__(64) void probe(const uint8_t* A, const uint8_t* B, float* D) {
  const int t = blockIdx.x, lane = threadIdx.x, r = lane & 15, g = lane >> 4;
  const uint8_t* a = A + (size_t)t * 16 * K + r * K;
  const uint8_t* b = B + (size_t)t * 16 * K + r * K;
  const floatx4 z = {0.f, 0.f, 0.f, 0.f};
  // scaled MFMA: lane (r, g) holds K positions 32 g .. 32 g + 31
  intx8 av, bv;
  for (int i = 0; i < 8; ++i) {
    av[i] = *reinterpret_cast<const int*>(a + 32 * g + 4 * i);
    bv[i] = *reinterpret_cast<const int*>(b + 32 * g + 4 * i);
  }
  const floatx4 d0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, z, 0, 0, 0, 127, 0, 127);
  // 16x16x32 MFMAs: lane (r, g) holds K positions 32 q + 8 g .. + 7 of step q
  floatx4 d1 = z, d2 = z;
  for (int q = 0; q < 4; ++q) {
    const long a8 = *reinterpret_cast<const long*>(a + 32 * q + 8 * g);
    const long b8 = *reinterpret_cast<const long*>(b + 32 * q + 8 * g);
    d1 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a8, b8, d1, 0, 0, 0);
    const half8 ah = dec8((uint32_t)a8, (uint32_t)(a8 >> 32));
    const half8 bh = dec8((uint32_t)b8, (uint32_t)(b8 >> 32));
    d2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh, d2, 0, 0, 0);
  }
  // lane (r, g) holds C[4 g + v][r]
  float* out = D + (size_t)t * NV * 256;
  for (int v = 0; v < 4; ++v) {
    out[0 * 256 + (4 * g + v) * 16 + r] = d0[v];
    out[1 * 256 + (4 * g + v) * 16 + r] = d1[v];
    out[2 * 256 + (4 * g + v) * 16 + r] = d2[v];
  }
}

// ---------------------------------------------------------------- host
static double e4m3_value(uint8_t c) {          // OCP E4M3 ("fn"), c != 0x7F, 0xFF
  const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  const double mag = e == 0 ? std::ldexp(m / 8.0, -6) : std::ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

static uint8_t e4m3_nearest(double x) {        // round to nearest, ties to even code
  uint8_t best = 0;
  double bd = 1e300;
  for (int c = 0; c < 127; ++c) {
    const double d = std::fabs(std::fabs(x) - e4m3_value((uint8_t)c));
    if (d < bd || (d == bd && (c & 1) == 0)) {
      bd = d;
      best = (uint8_t)c;
    }
  }
  return (uint8_t)(best | (x < 0 ? 0x80 : 0));
}

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64() {                   // splitmix64
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static double next_unit() { return (next_u64() >> 11) * (1.0 / 9007199254740992.0); }

int main() {
  const int T = 4096;
  const char* kinds[2] = {"full", "gauss"};
  const char* names[NV] = {"scale_f8f6f4", "fp8_fp8", "f16_decode"};
  uint8_t *dA, *dB;
  float* dD;
  const size_t nab = (size_t)T * 16 * K;
  if (hipMalloc(&dA, nab) != hipSuccess || hipMalloc(&dB, nab) != hipSuccess ||
      hipMalloc(&dD, (size_t)T * NV * 256 * sizeof(float)) != hipSuccess) {
    std::fprintf(stderr, "hipMalloc failed\n");
    return 2;
  }
  std::vector<uint8_t> hA(nab), hB(nab);
  std::vector<float> hD((size_t)T * NV * 256);
  bool ok = true;
  std::printf("{");
  for (int kind = 0; kind < 2; ++kind) {
    for (size_t i = 0; i < nab; ++i) {
      for (std::vector<uint8_t>* v : {&hA, &hB}) {
        uint8_t c;
        if (kind == 0) {
          do {
            c = (uint8_t)(next_u64() & 0xFF);
          } while ((c & 0x7F) == 0x7F);
        } else {
          // Box-Muller normal, scaled so that 4 sigma reaches 448
          const double u1 = next_unit() + 1e-300, u2 = next_unit();
          const double n = std::sqrt(-2.0 * std::log(u1)) * std::cos(6.283185307179586 * u2);
          c = e4m3_nearest(std::fmax(-448.0, std::fmin(448.0, n * 112.0)));
        }
        (*v)[i] = c;
      }
    }
    if (hipMemcpy(dA, hA.data(), nab, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(dB, hB.data(), nab, hipMemcpyHostToDevice) != hipSuccess) return 2;
    hipLaunchKernelGGL(probe, dim3(T), dim3(64), 0, 0, dA, dB, dD);
    if (hipGetLastError() != hipSuccess || hipDeviceSynchronize() != hipSuccess) return 2;
    if (hipMemcpy(hD.data(), dD, hD.size() * sizeof(float), hipMemcpyDeviceToHost) != hipSuccess) return 2;
    double worst[NV] = {0, 0, 0}, mean[NV] = {0, 0, 0};
    for (int t = 0; t < T; ++t) {
      const uint8_t* a = &hA[(size_t)t * 16 * K];
      const uint8_t* b = &hB[(size_t)t * 16 * K];
      for (int row = 0; row < 16; ++row)
        for (int col = 0; col < 16; ++col) {
          double ref = 0.0, bound = 0.0;
          for (int k = 0; k < K; ++k) {
            const double p = e4m3_value(a[row * K + k]) * e4m3_value(b[col * K + k]);
            ref += p;                                      // exact: every product and partial sum
            bound += std::fabs(p);                         // fits fp64's 53 bits
          }
          for (int v = 0; v < NV; ++v) {
            const double got = hD[(size_t)t * NV * 256 + v * 256 + row * 16 + col];
            const double r = bound > 0 ? std::fabs(got - ref) / bound : 0.0;
            worst[v] = std::fmax(worst[v], r);
            mean[v] += r / (T * 256.0);
          }
        }
    }
    if (worst[2] > 1e-6) ok = false;
    std::printf("%s\"%s\": {", kind ? ", " : "", kinds[kind]);
    for (int v = 0; v < NV; ++v)
      std::printf("%s\"%s\": {\"worst\": %.3e, \"mean\": %.3e}", v ? ", " : "", names[v], worst[v], mean[v]);
    std::printf("}");
  }
  std::printf(", \"tiles\": %d, \"k\": %d, \"bound\": 1e-5}\n", T, K);
  (void)hipFree(dA);
  (void)hipFree(dB);
  (void)hipFree(dD);
  return ok ? 0 : 1;
}

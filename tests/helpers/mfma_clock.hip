// Shader clock of gfx950 under sustained dense-MFMA load, and the MFMA rate
// reached, to read the GEMM kernels' fraction of the published peak (which
// assumes the 2.4 GHz peak engine clock) against the clock the chip holds.
//
// Two kernels, each on 4 x 256 workgroups of 256 threads (4 waves per CU per
// round, 16 waves per CU resident):
//   mfma   every wave issues chains of 8 independent
//          v_mfma_f32_16x16x32_f16 (accumulators kept live, results summed
//          into one output per lane so nothing is optimised away)
//   light  every wave spins on s_sleep (few instructions, little power)
// The first lane of every workgroup reads the shader-cycle counter
// (clock64, s_memtime) and the constant-rate wall clock (wall_clock64,
// s_memrealtime) at its start and end; shader cycles over wall time give
// the clock that workgroup ran at. The MFMA rate is the kernel's flops over
// its HIP-event time. Prints one JSON object.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <vector>

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int WG = 1024, NT = 256;

__global__ __launch_bounds__(NT) void mfma_load(int iters, float* out, unsigned long long* clk) {
  unsigned long long c0 = 0, r0 = 0;
  if (threadIdx.x == 0) {
    c0 = clock64();
    r0 = wall_clock64();
  }
  half8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(0.001f * (threadIdx.x + i));
    b[i] = (_Float16)(0.002f * (blockIdx.x % 7 + i));
  }
  floatx4 acc[8];
  for (int j = 0; j < 8; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  out[blockIdx.x * NT + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clk[4 * blockIdx.x + 0] = c0;
    clk[4 * blockIdx.x + 1] = clock64();
    clk[4 * blockIdx.x + 2] = r0;
    clk[4 * blockIdx.x + 3] = wall_clock64();
  }
}

__global__ __launch_bounds__(NT) void light_load(int iters, unsigned long long* clk) {
  unsigned long long c0 = 0, r0 = 0;
  if (threadIdx.x == 0) {
    c0 = clock64();
    r0 = wall_clock64();
  }
  for (int it = 0; it < iters; ++it) __builtin_amdgcn_s_sleep(8);
  if (threadIdx.x == 0) {
    clk[4 * blockIdx.x + 0] = c0;
    clk[4 * blockIdx.x + 1] = clock64();
    clk[4 * blockIdx.x + 2] = r0;
    clk[4 * blockIdx.x + 3] = wall_clock64();
  }
}

static double median_mhz(const std::vector<unsigned long long>& c, double wall_khz) {
  std::vector<double> f;
  for (int w = 0; w < WG; ++w) {
    const double cyc = (double)(c[4 * w + 1] - c[4 * w]);
    const double sec = (double)(c[4 * w + 3] - c[4 * w + 2]) / (wall_khz * 1e3);
    if (sec > 0) f.push_back(cyc / sec / 1e6);
  }
  std::sort(f.begin(), f.end());
  return f.empty() ? 0.0 : f[f.size() / 2];
}

int main() {
  int dev = 0, wall_khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || wall_khz <= 0)
    return 2;
  float* out;
  unsigned long long* clk;
  if (hipMalloc(&out, (size_t)WG * NT * sizeof(float)) != hipSuccess ||
      hipMalloc(&clk, (size_t)WG * 4 * sizeof(unsigned long long)) != hipSuccess)
    return 2;
  std::vector<unsigned long long> h(4 * WG);
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 2;
  const int iters = 20000;
  // warm-up, then the measured launch
  for (int rep = 0; rep < 2; ++rep) {
    if (hipEventRecord(e0, 0) != hipSuccess) return 2;
    hipLaunchKernelGGL(mfma_load, dim3(WG), dim3(NT), 0, 0, iters, out, clk);
    if (hipEventRecord(e1, 0) != hipSuccess || hipDeviceSynchronize() != hipSuccess) return 2;
  }
  float ms = 0.f;
  if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) return 2;
  if (hipMemcpy(h.data(), clk, h.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost) != hipSuccess)
    return 2;
  const double flops = (double)WG * (NT / 64) * iters * 8 * (16.0 * 16 * 32 * 2);
  const double mfma_mhz = median_mhz(h, wall_khz);
  hipLaunchKernelGGL(light_load, dim3(WG), dim3(NT), 0, 0, 20000, clk);
  if (hipDeviceSynchronize() != hipSuccess) return 2;
  if (hipMemcpy(h.data(), clk, h.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost) != hipSuccess)
    return 2;
  const double light_mhz = median_mhz(h, wall_khz);
  const double tf = flops / (ms * 1e-3) / 1e12;
  std::printf("{\"mfma_f16_tflops\": %.1f, \"mfma_ms\": %.3f, \"clock_mhz_under_mfma\": %.0f, "
              "\"clock_mhz_light\": %.0f, \"wall_clock_khz\": %d, \"peak_at_2400mhz_tflops\": 2516.6, "
              "\"peak_at_measured_clock_tflops\": %.1f}\n",
              tf, ms, mfma_mhz, light_mhz, wall_khz, 2516.6 * mfma_mhz / 2400.0);
  (void)hipFree(out);
  (void)hipFree(clk);
  return 0;
}

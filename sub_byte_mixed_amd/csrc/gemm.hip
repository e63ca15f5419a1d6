// Block-scaled GEMMs on gfx950 MFMA: C[M][N] = A[M][K] . B[N][K]^T,
// fp32 accumulation, tensor scales 2^(ea + eb) applied in the epilogue.
//
// "SNIP", Fig. 5: the forward and both backward GEMMs of a linear layer run
// on quantized operands. Operand formats ("FP4 All the Way" summary,
// Outline): NVFP4 = 16 E2M1 values per E4M3 scale.
//
// Per format:
//   NVFP4  code x E4M3 scale is decoded exactly into fp16 (a product of a
//          2-significant-bit E2M1 value and a 4-bit E4M3 scale spans at most
//          6 significant bits within [2^-10, 2688]) and multiplied on
//          v_mfma_f32_16x16x32_f16. Decoding: v_cvt_scalef32_pk_f16_fp4 with
//          the power-of-two part of the scale, then v_pk_mul_f16 by the
//          mantissa part. The gfx950 FP4 MFMA takes only power-of-two scales
//          per 32 elements, which cannot represent E4M3 scales per 16.
//   FP8    E4M3 codes are decoded exactly into fp16 (v_cvt_scalef32_pk_f16_fp8)
//          and multiplied on v_mfma_f32_16x16x32_f16. The gfx950 8-bit MFMA
//          (v_mfma_*_f8f6f4) sums its 128 products with only ~12 bits below
//          the largest product, measured at up to 1e-4 of sum|a||b|: outside
//          the 1e-5 bound, so it is not used for E4M3 x E4M3.
//   MXFP4  E2M1 codes and E8M0 scales straight into the same scaled MFMA
//          (FP4 operands, one scale per row and 32-element K block).
//   BF16   v_mfma_f32_16x16x32_bf16.
//
// Tiling: 128x128 output tile per workgroup of 256 threads (2x2 waves of
// 64x64, i.e. 4x4 MFMA tiles of 16x16 per wave), K stage of 128 elements
// staged through LDS; the next stage's global loads are issued before the
// current stage's MFMAs. Within a stage lane group g = lane/16 owns the K
// slice [32g, 32g+32) of its row; A and B use the same K assignment, so the
// dot products are exact permutations of the K sum.
#include "device.h"
#include "kernels.h"

namespace snip {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef int intx8_t __attribute__((ext_vector_type(8)));

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int NT = 256;

template <int FMT> struct Fmt;
template <> struct Fmt<SNIP_NVFP4>    { static constexpr int CB = 64,  SB = 8; };  // bytes per row per stage
template <> struct Fmt<SNIP_MXFP4>    { static constexpr int CB = 64,  SB = 4; };
template <> struct Fmt<SNIP_FP8_E4M3> { static constexpr int CB = 128, SB = 0; };
template <> struct Fmt<SNIP_BF16>     { static constexpr int CB = 256, SB = 0; };

// E4M3 scale code -> (power-of-two part as fp32, mantissa part as fp16x2) so
// that code value = p2 * m exactly. Subnormal codes (c < 8) are c * 2^-9.
__device__ __forceinline__ void split_e4m3(uint32_t c, float& p2, half2_t& m) {
  _Float16 mm;
  if (c >= 8u) {
    p2 = exp2i((int)(c >> 3) - 7);
    mm = (_Float16)(1.0f + 0.125f * (float)(c & 7u));
  } else {
    p2 = exp2i(-9);
    mm = (_Float16)(float)c;
  }
  m = half2_t{mm, mm};
}

// 8 E2M1 nibbles (one 32-bit word) -> 8 fp16 values code * p2 * m.
__device__ __forceinline__ half8_t decode8(uint32_t w, float p2, half2_t m) {
  const half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, p2, 0) * m;
  const half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, p2, 1) * m;
  const half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, p2, 2) * m;
  const half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, p2, 3) * m;
  return half8_t{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// 8 E4M3 codes (two 32-bit words) -> 8 fp16 values (exact).
__device__ __forceinline__ half8_t fp8x8_to_half8(uint32_t w0, uint32_t w1) {
  const half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
  const half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
  const half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
  const half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
  return half8_t{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

template <int FMT>
__global__ __launch_bounds__(NT) void gemm_kernel(GemmArgs g) {
  constexpr int CB = Fmt<FMT>::CB, SB = Fmt<FMT>::SB;
  constexpr int PITCH = CB + 16;                          // LDS row pitch (codes)
  constexpr int CCH = BM * CB / 16;                       // 16-byte chunks per operand tile
  constexpr int CPT = CCH / NT;                           // chunks per thread
  static_assert(CCH % NT == 0, "tile/thread mismatch");
  __shared__ __align__(16) uint8_t la[BM * PITCH];
  __shared__ __align__(16) uint8_t lb[BN * PITCH];
  __shared__ __align__(16) uint8_t las[SB ? BM * SB : 16];
  __shared__ __align__(16) uint8_t lbs[SB ? BN * SB : 16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r16 = lane & 15, grp = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  const int64_t K = g.K;
  const int64_t rowbytes = (FMT == SNIP_NVFP4 || FMT == SNIP_MXFP4) ? K / 2
                         : (FMT == SNIP_FP8_E4M3 ? K : 2 * K);
  const int nk = (int)(K / BK);

  uint4 ra[CPT], rb[CPT];
  uint2 ras = make_uint2(0, 0), rbs = make_uint2(0, 0);

  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      const int row = c / (CB / 16), cc = c % (CB / 16);
      const int64_t koff = (int64_t)kt * CB + cc * 16;
      ra[i] = (m0 + row < g.M) ? *reinterpret_cast<const uint4*>(g.a + (m0 + row) * rowbytes + koff)
                               : make_uint4(0, 0, 0, 0);
      rb[i] = (n0 + row < g.N) ? *reinterpret_cast<const uint4*>(g.b + (n0 + row) * rowbytes + koff)
                               : make_uint4(0, 0, 0, 0);
    }
    if constexpr (SB == 8) {          // NVFP4: 8 scale bytes per row per stage
      if (tid < BM) {
        const int64_t srow = K / 16;
        ras = (m0 + tid < g.M) ? *reinterpret_cast<const uint2*>(g.as + (m0 + tid) * srow + kt * 8) : make_uint2(0, 0);
        rbs = (n0 + tid < g.N) ? *reinterpret_cast<const uint2*>(g.bs + (n0 + tid) * srow + kt * 8) : make_uint2(0, 0);
      }
    } else if constexpr (SB == 4) {   // MX: 4 scale bytes per row per stage
      if (tid < BM) {
        const int64_t srow = K / 32;
        ras.x = (m0 + tid < g.M) ? *reinterpret_cast<const uint32_t*>(g.as + (m0 + tid) * srow + kt * 4) : 0u;
        rbs.x = (n0 + tid < g.N) ? *reinterpret_cast<const uint32_t*>(g.bs + (n0 + tid) * srow + kt * 4) : 0u;
      }
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      const int row = c / (CB / 16), cc = c % (CB / 16);
      *reinterpret_cast<uint4*>(la + row * PITCH + cc * 16) = ra[i];
      *reinterpret_cast<uint4*>(lb + row * PITCH + cc * 16) = rb[i];
    }
    if constexpr (SB == 8) {
      if (tid < BM) {
        *reinterpret_cast<uint2*>(las + tid * 8) = ras;
        *reinterpret_cast<uint2*>(lbs + tid * 8) = rbs;
      }
    } else if constexpr (SB == 4) {
      if (tid < BM) {
        *reinterpret_cast<uint32_t*>(las + tid * 4) = ras.x;
        *reinterpret_cast<uint32_t*>(lbs + tid * 4) = rbs.x;
      }
    }
  };

  floatx4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  gload(0);
  sstore();
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) gload(kt + 1);

    if constexpr (FMT == SNIP_NVFP4) {
      half8_t af[4][4], bf[4][4];     // [tile][substep]
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int arow = wm * 64 + i * 16 + r16;
        const uint4 ca = *reinterpret_cast<const uint4*>(la + arow * PITCH + grp * 16);
        const uint32_t sa = *reinterpret_cast<const uint16_t*>(las + arow * 8 + grp * 2);
        float p0, p1;
        half2_t q0, q1;
        split_e4m3(sa & 0xFFu, p0, q0);
        split_e4m3(sa >> 8, p1, q1);
        af[i][0] = decode8(ca.x, p0, q0);
        af[i][1] = decode8(ca.y, p0, q0);
        af[i][2] = decode8(ca.z, p1, q1);
        af[i][3] = decode8(ca.w, p1, q1);
        const int brow = wn * 64 + i * 16 + r16;
        const uint4 cb = *reinterpret_cast<const uint4*>(lb + brow * PITCH + grp * 16);
        const uint32_t sb = *reinterpret_cast<const uint16_t*>(lbs + brow * 8 + grp * 2);
        split_e4m3(sb & 0xFFu, p0, q0);
        split_e4m3(sb >> 8, p1, q1);
        bf[i][0] = decode8(cb.x, p0, q0);
        bf[i][1] = decode8(cb.y, p0, q0);
        bf[i][2] = decode8(cb.z, p1, q1);
        bf[i][3] = decode8(cb.w, p1, q1);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i][s], bf[j][s], acc[i][j], 0, 0, 0);
    } else if constexpr (FMT == SNIP_FP8_E4M3) {
      // E4M3 -> fp16 is exact; lane group g owns K slice [32g, 32g+32): 32 code
      // bytes, 8 per 16x16x32 substep.
      half8_t af[4][4], bf[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint8_t* pa = la + (wm * 64 + i * 16 + r16) * PITCH + grp * 32;
        const uint4 a0 = *reinterpret_cast<const uint4*>(pa), a1 = *reinterpret_cast<const uint4*>(pa + 16);
        af[i][0] = fp8x8_to_half8(a0.x, a0.y);
        af[i][1] = fp8x8_to_half8(a0.z, a0.w);
        af[i][2] = fp8x8_to_half8(a1.x, a1.y);
        af[i][3] = fp8x8_to_half8(a1.z, a1.w);
        const uint8_t* pb = lb + (wn * 64 + i * 16 + r16) * PITCH + grp * 32;
        const uint4 b0 = *reinterpret_cast<const uint4*>(pb), b1 = *reinterpret_cast<const uint4*>(pb + 16);
        bf[i][0] = fp8x8_to_half8(b0.x, b0.y);
        bf[i][1] = fp8x8_to_half8(b0.z, b0.w);
        bf[i][2] = fp8x8_to_half8(b1.x, b1.y);
        bf[i][3] = fp8x8_to_half8(b1.z, b1.w);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i][s], bf[j][s], acc[i][j], 0, 0, 0);
    } else if constexpr (FMT == SNIP_MXFP4) {
      intx8_t af[4], bf[4];
      int sa[4], sb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int arow = wm * 64 + i * 16 + r16;
        const uint4 a0 = *reinterpret_cast<const uint4*>(la + arow * PITCH + grp * 16);
        af[i] = intx8_t{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, 0, 0, 0, 0};
        sa[i] = las[arow * 4 + grp];
        const int brow = wn * 64 + i * 16 + r16;
        const uint4 b0 = *reinterpret_cast<const uint4*>(lb + brow * PITCH + grp * 16);
        bf[i] = intx8_t{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, 0, 0, 0, 0};
        sb[i] = lbs[brow * 4 + grp];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bf[j], acc[i][j], 4, 4,
                                                                       0, sa[i], 0, sb[j]);
    } else {  // BF16
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8_t af[4], bf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          af[i] = *reinterpret_cast<const bf16x8_t*>(la + (wm * 64 + i * 16 + r16) * PITCH + grp * 64 + s * 16);
          bf[i] = *reinterpret_cast<const bf16x8_t*>(lb + (wn * 64 + i * 16 + r16) * PITCH + grp * 64 + s * 16);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
    }

    __syncthreads();
    if (kt + 1 < nk) {
      sstore();
      __syncthreads();
    }
  }

  // epilogue: lane holds rows 4*grp + v, column r16 of each 16x16 tile
  const int e = (g.ea ? *g.ea : 0) + (g.eb ? *g.eb : 0);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + wn * 64 + j * 16 + r16;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = m0 + wm * 64 + i * 16 + 4 * grp + v;
        if (row < g.M && col < g.N) g.c[row * g.ldc + col] = ldexpf(acc[i][j][v], e);
      }
    }
}

hipError_t launch_gemm(int format, const GemmArgs& g, hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(g.N, BN), (unsigned)ceil_div(g.M, BM));
  switch (format) {
    case SNIP_NVFP4: hipLaunchKernelGGL(gemm_kernel<SNIP_NVFP4>, grid, dim3(NT), 0, s, g); break;
    case SNIP_FP8_E4M3: hipLaunchKernelGGL(gemm_kernel<SNIP_FP8_E4M3>, grid, dim3(NT), 0, s, g); break;
    case SNIP_MXFP4: hipLaunchKernelGGL(gemm_kernel<SNIP_MXFP4>, grid, dim3(NT), 0, s, g); break;
    case SNIP_BF16: hipLaunchKernelGGL(gemm_kernel<SNIP_BF16>, grid, dim3(NT), 0, s, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace snip

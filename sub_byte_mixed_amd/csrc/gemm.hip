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
//   MXFP4  E2M1 codes and E8M0 scales go straight into
//          v_mfma_scale_f32_16x16x128_f8f6f4 (FP4 operands, one scale per row
//          and 32-element K block).
//   BF16   v_mfma_f32_16x16x32_bf16.
//
// Tiling: a workgroup of 256 threads (2x2 waves) owns a BM x BN output tile
// (256x256 for large problems, 128x128 otherwise) and walks K in stages of
// BK elements (64; 128 for MX). Stages are double-buffered in LDS: the global
// loads of stage s+1 are issued into registers before the MFMAs of stage s,
// and written to the other LDS buffer afterwards, so one barrier per stage
// suffices. NVFP4 block scales are split into (2^e as fp32, mantissa as
// fp16x2) once, when they are staged in LDS. Within a stage, lane group
// g = lane/16 owns the K slice [g*BK/4, (g+1)*BK/4) of its row; A and B use
// the same K assignment, so every dot product is a permutation of the K sum.
//
// Tile order: the hardware hands workgroups to the 8 XCDs round-robin; tile
// ids are remapped so each XCD works on a contiguous range, and tiles are
// ordered in groups of 8 tile-rows so that concurrently running tiles share
// A and B panels in that XCD's L2. Skinny problems split K across
// workgroups into fp32 partials that a second kernel sums in a fixed order.
#include "device.h"
#include "kernels.h"

namespace snip {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef int intx8_t __attribute__((ext_vector_type(8)));

constexpr int NT = 256;

// Code bytes per row for BK elements of K, and scale bytes per row.
template <int FMT, int BK> struct KStage;
template <int BK> struct KStage<SNIP_NVFP4, BK>    { static constexpr int CB = BK / 2, NS = BK / 16; };
template <int BK> struct KStage<SNIP_FP8_E4M3, BK> { static constexpr int CB = BK,     NS = 0; };
template <int BK> struct KStage<SNIP_BF16, BK>     { static constexpr int CB = BK * 2, NS = 0; };
template <int BK> struct KStage<SNIP_MXFP4, BK>    { static constexpr int CB = BK / 2, NS = BK / 32; };

// Per-format kernel configuration, chosen from measured sweeps on MI355X:
//   NVFP4  256x256 tiles (one workgroup per CU) halve the in-register decode
//          per MFMA; 128x128 for problems with fewer than 192 big tiles.
//   FP8    decode is half as costly, so 128x128 tiles with two workgroups per
//          CU (better latency hiding) win at every size.
//   MX     no decode: 128x128 tiles, two per CU, K stage of 256.
//   BF16   as NVFP4 (256x256 when the problem is large).

// K per LDS stage: 64, except MX-FP4 (one MFMA covers K = 128), which takes
// 256 when K allows it and 128 otherwise. The API guarantees K % 128 == 0.
static int stage_k(int format, int64_t K) {
  if (format == SNIP_MXFP4) return (K % 256 == 0) ? 256 : 128;
  return 64;
}
static bool big_tiles_allowed(int format) { return format == SNIP_NVFP4 || format == SNIP_BF16; }


// E4M3 scale code -> {fp32 bits of its power-of-two part, fp16x2 bits of its
// mantissa part} with value = p2 * m exactly; subnormal codes are c * 2^-9.
__device__ __forceinline__ uint2 split_e4m3(uint32_t c) {
  uint32_t p2, m;
  if (c >= 8u) {
    p2 = ((c >> 3) + 120u) << 23;                 // 2^((c>>3) - 7)
    m = 0x3C00u | ((c & 7u) << 7);                 // fp16 1 + (c&7)/8
  } else {
    p2 = 118u << 23;                               // 2^-9
    m = __builtin_bit_cast(uint16_t, (_Float16)(float)c);
  }
  return make_uint2(p2, m | (m << 16));
}

// 8 E2M1 nibbles (one 32-bit word) -> 8 fp16 values code * p2 * m.
__device__ __forceinline__ half8_t decode8(uint32_t w, uint2 s) {
  const float p2 = __uint_as_float(s.x);
  const half2_t m = __builtin_bit_cast(half2_t, s.y);
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

// Tile id -> (tile row, tile column).
__device__ __forceinline__ void tile_coords(int id, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  if ((total & 7) == 0) id = (id & 7) * (total >> 3) + (id >> 3);
  constexpr int GM = 8;
  const int group = id / (GM * tiles_n);
  const int first = group * GM;
  const int gm = (tiles_m - first) < GM ? (tiles_m - first) : GM;
  const int r = id - group * GM * tiles_n;
  tm = first + r % gm;
  tn = r / gm;
}

template <int FMT, int BM, int BN, int BK>
__global__ __launch_bounds__(NT, BM == 256 ? 1 : 2) void gemm_kernel(GemmArgs g) {
  constexpr int CB = KStage<FMT, BK>::CB, NS = KStage<FMT, BK>::NS;
  constexpr int KG = BK / 4;                                    // K per lane group per stage
  constexpr int NSUB = (FMT == SNIP_MXFP4) ? KG / 32 : KG / 8;  // MFMAs along K per stage
  constexpr int WM = BM / 2, WN = BN / 2;            // wave tile
  constexpr int TM = WM / 16, TN = WN / 16;          // 16x16 MFMA tiles per wave
  constexpr int PITCH = CB + 16;                     // LDS bytes per row (codes)
  constexpr int CPA = BM * CB / 16 / NT;             // 16-byte chunks per thread (A)
  constexpr int CPB = BN * CB / 16 / NT;
  static_assert(CPA >= 1 && CPB >= 1, "tile too small");
  // NVFP4 scales are staged decoded (8 bytes each), MX scales raw (1 byte)
  constexpr int SBYTES = (FMT == SNIP_NVFP4) ? 8 : 1;
  constexpr int LA = BM * PITCH, LB = BN * PITCH;
  constexpr int LSA = NS ? BM * NS * SBYTES : 0, LSB = NS ? BN * NS * SBYTES : 0;
  constexpr int STAGE = LA + LB + LSA + LSB;
  __shared__ __align__(16) uint8_t smem[2 * STAGE];
  // E4M3 code -> (2^e, mantissa) table for NVFP4 scales, built once
  __shared__ uint2 lut[FMT == SNIP_NVFP4 ? 256 : 1];
  if constexpr (FMT == SNIP_NVFP4) {
    lut[threadIdx.x] = split_e4m3(threadIdx.x);
    __syncthreads();
  }

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r16 = lane & 15, grp = lane >> 4;
  int tm, tn;
  tile_coords(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t rowbytes = (int64_t)g.K * CB / BK;
  const int kt0 = blockIdx.y * g.kchunk / BK;
  const int kt1 = min((int)(g.K / BK), (int)((blockIdx.y + 1) * g.kchunk / BK));
  const int nk = kt1 - kt0;

  uint4 ra[CPA], rb[CPB];
  uint2 sa = make_uint2(0u, 0u), sb = make_uint2(0u, 0u);

  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < CPA; ++i) {
      const int c = tid + i * NT, row = c / (CB / 16), cc = c % (CB / 16);
      ra[i] = (m0 + row < g.M)
                  ? *reinterpret_cast<const uint4*>(g.a + (m0 + row) * rowbytes + (int64_t)kt * CB + cc * 16)
                  : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < CPB; ++i) {
      const int c = tid + i * NT, row = c / (CB / 16), cc = c % (CB / 16);
      rb[i] = (n0 + row < g.N)
                  ? *reinterpret_cast<const uint4*>(g.b + (n0 + row) * rowbytes + (int64_t)kt * CB + cc * 16)
                  : make_uint4(0u, 0u, 0u, 0u);
    }
    if constexpr (NS == 4) {          // 4 scale bytes per row per stage
      const int64_t srow = g.K / (FMT == SNIP_NVFP4 ? 16 : 32);
      if (tid < BM) sa.x = (m0 + tid < g.M) ? *reinterpret_cast<const uint32_t*>(g.as + (m0 + tid) * srow + kt * 4) : 0u;
      if (tid < BN) sb.x = (n0 + tid < g.N) ? *reinterpret_cast<const uint32_t*>(g.bs + (n0 + tid) * srow + kt * 4) : 0u;
    } else if constexpr (NS == 8) {   // 8 scale bytes per row per stage
      const int64_t srow = g.K / (FMT == SNIP_NVFP4 ? 16 : 32);
      if (tid < BM) sa = (m0 + tid < g.M) ? *reinterpret_cast<const uint2*>(g.as + (m0 + tid) * srow + kt * 8) : make_uint2(0u, 0u);
      if (tid < BN) sb = (n0 + tid < g.N) ? *reinterpret_cast<const uint2*>(g.bs + (n0 + tid) * srow + kt * 8) : make_uint2(0u, 0u);
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* la = smem + buf * STAGE;
    uint8_t* lb = la + LA;
#pragma unroll
    for (int i = 0; i < CPA; ++i) {
      const int c = tid + i * NT, row = c / (CB / 16), cc = c % (CB / 16);
      *reinterpret_cast<uint4*>(la + row * PITCH + cc * 16) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < CPB; ++i) {
      const int c = tid + i * NT, row = c / (CB / 16), cc = c % (CB / 16);
      *reinterpret_cast<uint4*>(lb + row * PITCH + cc * 16) = rb[i];
    }
    if constexpr (FMT == SNIP_NVFP4) {
      uint2* lsa = reinterpret_cast<uint2*>(lb + LB);
      uint2* lsb = reinterpret_cast<uint2*>(lb + LB + LSA);
      if (tid < BM) {
#pragma unroll
        for (int q = 0; q < NS; ++q) lsa[tid * NS + q] = lut[((q < 4 ? sa.x : sa.y) >> (8 * (q & 3))) & 0xFFu];
      }
      if (tid < BN) {
#pragma unroll
        for (int q = 0; q < NS; ++q) lsb[tid * NS + q] = lut[((q < 4 ? sb.x : sb.y) >> (8 * (q & 3))) & 0xFFu];
      }
    } else if constexpr (FMT == SNIP_MXFP4) {
      if (tid < BM) {
        if constexpr (NS == 4) *reinterpret_cast<uint32_t*>(lb + LB + tid * 4) = sa.x;
        else *reinterpret_cast<uint2*>(lb + LB + tid * 8) = sa;
      }
      if (tid < BN) {
        if constexpr (NS == 4) *reinterpret_cast<uint32_t*>(lb + LB + LSA + tid * 4) = sb.x;
        else *reinterpret_cast<uint2*>(lb + LB + LSA + tid * 8) = sb;
      }
    }
  };

  floatx4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  if (nk > 0) {
    gload(kt0);
    sstore(0);
  }
  __syncthreads();

  for (int it = 0; it < nk; ++it) {
    const int buf = it & 1;
    if (it + 1 < nk) gload(kt0 + it + 1);
    const uint8_t* la = smem + buf * STAGE;
    const uint8_t* lb = la + LA;

    if constexpr (FMT == SNIP_NVFP4) {
      // lane group g: K slice [g*KG, (g+1)*KG): KG/2 code bytes, KG/16 blocks
      constexpr int W = KG / 8;                        // code words per lane per tile
      const uint2* lsa = reinterpret_cast<const uint2*>(lb + LB);
      const uint2* lsb = reinterpret_cast<const uint2*>(lb + LB + LSA);
      uint32_t ca[TM][W], cbv[TN][W];
      uint2 sca[TM][W / 2], scb[TN][W / 2];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * WM + i * 16 + r16;
        const uint32_t* p = reinterpret_cast<const uint32_t*>(la + row * PITCH + grp * (KG / 2));
#pragma unroll
        for (int w = 0; w < W; ++w) ca[i][w] = p[w];
#pragma unroll
        for (int q = 0; q < W / 2; ++q) sca[i][q] = lsa[row * NS + grp * (W / 2) + q];
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row = wn * WN + j * 16 + r16;
        const uint32_t* p = reinterpret_cast<const uint32_t*>(lb + row * PITCH + grp * (KG / 2));
#pragma unroll
        for (int w = 0; w < W; ++w) cbv[j][w] = p[w];
#pragma unroll
        for (int q = 0; q < W / 2; ++q) scb[j][q] = lsb[row * NS + grp * (W / 2) + q];
      }
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        half8_t af[TM], bf[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) af[i] = decode8(ca[i][s], sca[i][s / 2]);
#pragma unroll
        for (int j = 0; j < TN; ++j) bf[j] = decode8(cbv[j][s], scb[j][s / 2]);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
    } else if constexpr (FMT == SNIP_FP8_E4M3) {
      // lane group g: K slice [g*KG, (g+1)*KG): KG code bytes
      constexpr int W = KG / 4;
      uint32_t ca[TM][W], cbv[TN][W];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(la + (wm * WM + i * 16 + r16) * PITCH + grp * KG);
#pragma unroll
        for (int w = 0; w < W; ++w) ca[i][w] = p[w];
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(lb + (wn * WN + j * 16 + r16) * PITCH + grp * KG);
#pragma unroll
        for (int w = 0; w < W; ++w) cbv[j][w] = p[w];
      }
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        half8_t af[TM], bf[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) af[i] = fp8x8_to_half8(ca[i][2 * s], ca[i][2 * s + 1]);
#pragma unroll
        for (int j = 0; j < TN; ++j) bf[j] = fp8x8_to_half8(cbv[j][2 * s], cbv[j][2 * s + 1]);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
    } else if constexpr (FMT == SNIP_BF16) {
      // lane group g: K slice [g*KG, (g+1)*KG): 2*KG bytes
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        bf16x8_t af[TM], bf[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
          af[i] = *reinterpret_cast<const bf16x8_t*>(la + (wm * WM + i * 16 + r16) * PITCH + grp * 2 * KG + s * 16);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          bf[j] = *reinterpret_cast<const bf16x8_t*>(lb + (wn * WN + j * 16 + r16) * PITCH + grp * 2 * KG + s * 16);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
    } else {  // MXFP4: lane group g owns NSUB 32-blocks; one scaled MFMA covers K = 128
      const uint8_t* lsa = lb + LB;
      const uint8_t* lsb = lb + LB + LSA;
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        intx8_t af[TM], bf[TN];
        int sva[TM], svb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int row = wm * WM + i * 16 + r16;
          const uint4 v = *reinterpret_cast<const uint4*>(la + row * PITCH + s * 64 + grp * 16);
          af[i] = intx8_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
          sva[i] = lsa[row * NS + s * 4 + grp];
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int row = wn * WN + j * 16 + r16;
          const uint4 v = *reinterpret_cast<const uint4*>(lb + row * PITCH + s * 64 + grp * 16);
          bf[j] = intx8_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
          svb[j] = lsb[row * NS + s * 4 + grp];
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bf[j], acc[i][j], 4, 4,
                                                                         0, sva[i], 0, svb[j]);
      }
    }

    if (it + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds rows 4*grp + v, column r16 of each 16x16 tile
  if (g.kchunk >= g.K) {
    const int e = (g.ea ? *g.ea : 0) + (g.eb ? *g.eb : 0);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t col = n0 + wn * WN + j * 16 + r16;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t row = m0 + wm * WM + i * 16 + 4 * grp + v;
          if (row < g.M && col < g.N) g.c[row * g.ldc + col] = ldexpf(acc[i][j][v], e);
        }
      }
  } else {
    float* part = g.partial + (int64_t)blockIdx.y * g.M * g.N;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t col = n0 + wn * WN + j * 16 + r16;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t row = m0 + wm * WM + i * 16 + 4 * grp + v;
          if (row < g.M && col < g.N) part[row * g.N + col] = acc[i][j][v];
        }
      }
  }
}

// Split-K reduction: C = 2^(ea+eb) * sum over splits, in split order.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs g, int nsplit) {
  const int e = (g.ea ? *g.ea : 0) + (g.eb ? *g.eb : 0);
  const int64_t total = g.M * g.N;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    float s = 0.0f;
    for (int k = 0; k < nsplit; ++k) s += g.partial[k * total + i];
    const int64_t row = i / g.N, col = i - row * g.N;
    g.c[row * g.ldc + col] = ldexpf(s, e);
  }
}

// Host-side plan: tile shape and K split for a problem.
GemmPlan plan_gemm(int format, int64_t M, int64_t N, int64_t K) {
  GemmPlan p;
  const int bk = stage_k(format, K);
  p.bk = bk;
  const int64_t t256 = ceil_div(M, 256) * ceil_div(N, 256);
  if (big_tiles_allowed(format) && t256 >= 192) {
    p.bm = 256;
    p.tiles = t256;
    p.ksplit = 1;
    p.kchunk = K;
    return p;
  }
  p.bm = 128;
  p.tiles = ceil_div(M, 128) * ceil_div(N, 128);
  int64_t split = p.tiles >= 192 ? 1 : 256 / p.tiles;
  const int64_t max_split = K / (4 * bk);                 // keep >= 4 stages per split
  if (split > max_split) split = max_split;
  if (split < 1) split = 1;
  const int64_t chunk = ceil_div(ceil_div(K, split), bk) * bk;
  p.kchunk = chunk;
  p.ksplit = (int)ceil_div(K, chunk);
  return p;
}

size_t gemm_partial_bytes(int format, int64_t M, int64_t N, int64_t K) {
  const GemmPlan p = plan_gemm(format, M, N, K);
  return p.ksplit > 1 ? (size_t)p.ksplit * (size_t)(M * N) * sizeof(float) : 0;
}

template <int FMT>
static void launch_fmt(const GemmPlan& p, const GemmArgs& g, hipStream_t s) {
  const dim3 grid((unsigned)p.tiles, (unsigned)p.ksplit);
  if constexpr (FMT == SNIP_MXFP4) {
    if (p.bk == 256) hipLaunchKernelGGL((gemm_kernel<FMT, 128, 128, 256>), grid, dim3(NT), 0, s, g);
    else hipLaunchKernelGGL((gemm_kernel<FMT, 128, 128, 128>), grid, dim3(NT), 0, s, g);
    return;
  } else {
    if constexpr (FMT == SNIP_NVFP4 || FMT == SNIP_BF16) {
      if (p.bm == 256) {
        hipLaunchKernelGGL((gemm_kernel<FMT, 256, 256, 64>), grid, dim3(NT), 0, s, g);
        return;
      }
    }
    hipLaunchKernelGGL((gemm_kernel<FMT, 128, 128, 64>), grid, dim3(NT), 0, s, g);
  }
}

hipError_t launch_gemm(int format, const GemmArgs& g_in, hipStream_t s) {
  GemmPlan p = plan_gemm(format, g_in.M, g_in.N, g_in.K);
  GemmArgs g = g_in;
  if (p.ksplit > 1 && g.partial == nullptr) {      // no scratch: run unsplit
    p.ksplit = 1;
    p.kchunk = g.K;
  }
  g.tiles_m = (int)ceil_div(g.M, p.bm);
  g.tiles_n = (int)ceil_div(g.N, p.bm);
  g.kchunk = p.kchunk;
  if (format < SNIP_BF16 || format > SNIP_MXFP4) return hipErrorInvalidValue;
  int slot = timing_begin(LaunchTag{SNIP_LAUNCH_GEMM, format, -1, -1, 2.0 * g.M * g.N * g.K}, s);
  switch (format) {
    case SNIP_NVFP4: launch_fmt<SNIP_NVFP4>(p, g, s); break;
    case SNIP_FP8_E4M3: launch_fmt<SNIP_FP8_E4M3>(p, g, s); break;
    case SNIP_MXFP4: launch_fmt<SNIP_MXFP4>(p, g, s); break;
    default: launch_fmt<SNIP_BF16>(p, g, s); break;
  }
  hipError_t e = hipGetLastError();
  timing_end(slot, s);
  if (e != hipSuccess || p.ksplit == 1) return e;
  int64_t wg = ceil_div(g.M * g.N, 256);
  if (wg > 4096) wg = 4096;
  slot = timing_begin(LaunchTag{SNIP_LAUNCH_SPLITK, format, -1, -1, (double)(g.M * g.N)}, s);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)wg), dim3(256), 0, s, g, p.ksplit);
  e = hipGetLastError();
  timing_end(slot, s);
  return e;
}

}  // namespace snip

// Register-staged block-scaled GEMM for 128x128 tiles of MX-FP4 and BF16:
// C[M][N] = A[M][K] . B[N][K]^T (fp32 accumulation).
//
// "SNIP", Fig. 5 (the layer's three GEMMs); MX-FP4 = E2M1 codes with one
// E8M0 scale per 32 K elements on v_mfma_scale_f32_16x16x128_f8f6f4, BF16 on
// v_mfma_f32_16x16x32_bf16 (same operand conventions as gemm.hip).
//
// Why a second kernel family: these two formats carry no decode work, so a
// 128x128 tile performs only 16 MFMAs per wave and 128-element K step; with
// two workgroups per CU the short stages are better served by staging each
// stage through registers (global loads of stage k+1 issued before the MFMAs
// of stage k, written to the other of two LDS buffers after them: one
// barrier per stage) than by the LDS-DMA ring, measured on MI355X (MX-FP4
// 1.7 vs 1.3 PFLOP/s, BF16 0.75 vs 0.54 PFLOP/s on 4096x2048x2048).
//
// LDS rows are padded by 16 bytes; lane group g = lane / 16 owns the K slice
// [g * BK/4, (g+1) * BK/4) of a stage in both A and B, so every dot product
// is a permutation of the K sum.
#include "gemm_common.h"

namespace snip {

namespace {

constexpr int NT = 256;
constexpr int BMS = 128;     // tile edge

// Code bytes per row per stage (CB) and MX scale bytes per row per stage (NS).
template <int FMT, int BK> struct SStage;
template <int BK> struct SStage<SNIP_BF16, BK>  { static constexpr int CB = BK * 2, NS = 0; };
template <int BK> struct SStage<SNIP_MXFP4, BK> { static constexpr int CB = BK / 2, NS = BK / 32; };

template <int FMT, int BK>
__global__ __launch_bounds__(NT, 2) void staged_gemm_kernel(GemmArgs g) {
  constexpr int CB = SStage<FMT, BK>::CB, NS = SStage<FMT, BK>::NS;
  constexpr int KG = BK / 4;                                     // K per lane group per stage
  constexpr int NSUB = (FMT == SNIP_MXFP4) ? KG / 32 : KG / 8;   // MFMAs along K per stage
  constexpr int WM = BMS / 2, WN = BMS / 2;                      // wave tile
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int PITCH = CB + 16;                                 // LDS bytes per row
  constexpr int CPT = BMS * CB / 16 / NT;                        // 16-byte chunks per thread
  static_assert(CPT >= 1, "tile too small");
  constexpr int LA = BMS * PITCH;
  constexpr int LS = NS ? BMS * NS : 0;
  constexpr int STAGE = 2 * LA + 2 * LS;
  __shared__ __align__(16) uint8_t smem[2 * STAGE];
  if (finalize_workgroup(g)) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r16 = lane & 15, grp = lane >> 4;
  int tm, tn;
  tile_coords(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BMS, n0 = (int64_t)tn * BMS;
  const int64_t rowbytes = (int64_t)g.K * CB / BK;
  const int kt0 = (int)(blockIdx.y * g.kchunk / BK);
  const int kt1 = min((int)(g.K / BK), (int)((blockIdx.y + 1) * g.kchunk / BK));
  const int nk = kt1 - kt0;

  uint4 ra[CPT], rb[CPT];
  uint2 sa = make_uint2(0u, 0u), sb = make_uint2(0u, 0u);
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT, row = c / (CB / 16), cc = c % (CB / 16);
      const int64_t off = (int64_t)kt * CB + cc * 16;
      ra[i] = (m0 + row < g.M) ? *reinterpret_cast<const uint4*>(g.a + (m0 + row) * rowbytes + off)
                               : make_uint4(0u, 0u, 0u, 0u);
      rb[i] = (n0 + row < g.N) ? *reinterpret_cast<const uint4*>(g.b + (n0 + row) * rowbytes + off)
                               : make_uint4(0u, 0u, 0u, 0u);
    }
    if constexpr (NS == 4 || NS == 8) {      // MX scales: NS bytes per row per stage
      const int64_t srow = g.K / 32;
      if (tid < BMS) {
        const uint8_t* pa = g.as + (m0 + tid) * srow + (int64_t)kt * NS;
        const uint8_t* pb = g.bs + (n0 + tid) * srow + (int64_t)kt * NS;
        if constexpr (NS == 4) {
          sa.x = (m0 + tid < g.M) ? *reinterpret_cast<const uint32_t*>(pa) : 0u;
          sb.x = (n0 + tid < g.N) ? *reinterpret_cast<const uint32_t*>(pb) : 0u;
        } else {
          sa = (m0 + tid < g.M) ? *reinterpret_cast<const uint2*>(pa) : make_uint2(0u, 0u);
          sb = (n0 + tid < g.N) ? *reinterpret_cast<const uint2*>(pb) : make_uint2(0u, 0u);
        }
      }
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* la = smem + buf * STAGE;
    uint8_t* lb = la + LA;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT, row = c / (CB / 16), cc = c % (CB / 16);
      *reinterpret_cast<uint4*>(la + row * PITCH + cc * 16) = ra[i];
      *reinterpret_cast<uint4*>(lb + row * PITCH + cc * 16) = rb[i];
    }
    if constexpr (NS == 4 || NS == 8) {
      if (tid < BMS) {
        uint8_t* ls = lb + LA;
        if constexpr (NS == 4) {
          *reinterpret_cast<uint32_t*>(ls + tid * 4) = sa.x;
          *reinterpret_cast<uint32_t*>(ls + LS + tid * 4) = sb.x;
        } else {
          *reinterpret_cast<uint2*>(ls + tid * 8) = sa;
          *reinterpret_cast<uint2*>(ls + LS + tid * 8) = sb;
        }
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
    if constexpr (FMT == SNIP_BF16) {
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
    } else {  // MX-FP4: lane group g owns one 32-block of each 128-element step
      const uint8_t* lsa = lb + LA;
      const uint8_t* lsb = lsa + LS;
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
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bf[j], acc[i][j], 4, 4, 0, sva[i],
                                                                         0, svb[j]);
      }
    }
    if (it + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  store_tile<TM, TN>(g, acc, m0 + wm * WM, n0 + wn * WN, r16, grp);
}

}  // namespace

// K per stage: MX-FP4 256 when K allows it (128 otherwise), BF16 64. The
// API guarantees K % 128 == 0.
int staged_stage_k(int format, int64_t K) {
  if (format == SNIP_MXFP4) return K % 256 == 0 ? 256 : 128;
  return 64;
}

void launch_staged(int format, int bk, const GemmArgs& g, dim3 grid, hipStream_t s) {
  if (format == SNIP_MXFP4) {
    if (bk == 256) hipLaunchKernelGGL((staged_gemm_kernel<SNIP_MXFP4, 256>), grid, dim3(NT), 0, s, g);
    else hipLaunchKernelGGL((staged_gemm_kernel<SNIP_MXFP4, 128>), grid, dim3(NT), 0, s, g);
  } else {
    hipLaunchKernelGGL((staged_gemm_kernel<SNIP_BF16, 64>), grid, dim3(NT), 0, s, g);
  }
}

}  // namespace snip

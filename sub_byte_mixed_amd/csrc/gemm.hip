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
//          v_mfma_f32_16x16x32_f16. Decoding: v_cvt_scalef32_pk_f16_fp4 of
//          the codes and v_cvt_scalef32_pk_f16_fp8 of the two scale bytes a
//          lane needs, then v_pk_mul_f16. The gfx950 FP4 MFMA takes only
//          power-of-two scales per 32 elements, which cannot represent E4M3
//          scales per 16.
//   FP8    E4M3 codes are decoded exactly into fp16 (v_cvt_scalef32_pk_f16_fp8)
//          and multiplied on v_mfma_f32_16x16x32_f16. The gfx950 8-bit MFMAs
//          (v_mfma_scale_f32_16x16x128_f8f6f4 and v_mfma_f32_16x16x32_fp8_fp8)
//          lose low bits of the products' sum: measured (the probe
//          tests/helpers/fp8_mfma_accuracy.hip) up to 1.9e-4 of sum|a||b| on
//          full-range E4M3 data and 2.2e-5 on Gaussian data, against 3.1e-7
//          for the decode path; the bound is 1e-5, so they are not used for
//          E4M3 x E4M3.
//   MXFP4  E2M1 codes and E8M0 scales go straight into
//          v_mfma_scale_f32_16x16x128_f8f6f4 (FP4 operands, one scale per row
//          and 32-element K block).
//   BF16   v_mfma_f32_16x16x32_bf16.
//
// Data movement. Operands are staged in LDS by direct global-to-LDS loads
// (global_load_lds_dwordx4: each lane's 16 bytes land at M0 + 16 * lane),
// so staging takes no VGPRs and no LDS write instructions. The unit of
// staging is 16 rows x 64 bytes of one operand (1 KiB), row-major in LDS:
// lane l fetches the 16 bytes at offset 16 * (l % 4) of row l / 4, so each
// quad of lanes reads 64 contiguous bytes of one row. The MFMA-side read of
// lane (r16 = l % 16, grp = l / 16) is one ds_read_b128 at 64 * r16 +
// 16 * grp: the K slice grp of row r16 that the 16x16 MFMA operand layout
// asks for. Measured on MI355X: this is 5-12 % faster for FP8 (1-7 % for
// NVFP4) than fetching row l % 16 per lane, whose LDS reads at 16 * lane
// were free of bank conflicts but whose quads touched four rows each. A and
// B use the same K slices, so every dot product is a permutation of the
// K sum. A unit covers K = 32 (BF16), 64 (FP8) or 128 (FP4) elements, and
// one K stage is one unit per 16-row block; block scales travel with it
// (8 E4M3 bytes or 4 E8M0 bytes per row and unit, dword DMA).
//
// Pipeline: S stages in a ring. The loads of stage k + S - 1 are issued
// right after the barrier that opens stage k, so S - 1 stages are in flight
// while one is multiplied. Before the barrier each wave waits (vmcnt) only
// for its own loads of stage k; the barrier then makes every wave's loads
// visible and guarantees that the ring slot about to be refilled is no
// longer read.
//
// Tiling: a workgroup of 256 threads (2x2 waves) owns a BM x BN output tile:
// 256x256 (one workgroup per CU; for NVFP4 and MX-FP4 the one-wave-per-SIMD
// kernels gemm_nvfp4_w1_kernel, gemm_mxfp4_w1_kernel and
// gemm_mxfp4_w1p_kernel below, the first and last persistent), 256x128
// (FP8 and NVFP4, two per CU), 128x128 (two per CU) or, for skinny FP8 /
// NVFP4 problems, 64x64, as plan_gemm decides from the problem's tile
// rounds. Tile order: the hardware hands workgroups to the 8 XCDs
// round-robin; tile ids are remapped so each XCD works on a contiguous range,
// and tiles are ordered in groups of 4 tile-rows so that concurrently running
// tiles share A and B panels in that XCD's L2. Skinny problems split K across
// workgroups into fp32 partials that a second kernel sums in a fixed order.
#include "gemm_common.h"

#include <utility>

namespace snip {

constexpr int NT = 256;

// Staging unit per format: K elements per 64-byte row segment (UE), MFMAs
// per fragment pair and unit (NQ), block-scale bytes per row and unit (SB).
template <int FMT> struct Unit;
template <> struct Unit<SNIP_BF16>     { static constexpr int UE = 32,  NQ = 1, SB = 0; };
template <> struct Unit<SNIP_FP8_E4M3> { static constexpr int UE = 64,  NQ = 2, SB = 0; };
template <> struct Unit<SNIP_NVFP4>    { static constexpr int UE = 128, NQ = 4, SB = 8; };
template <> struct Unit<SNIP_MXFP4>    { static constexpr int UE = 128, NQ = 1, SB = 4; };

static int unit_k(int format) {
  return format == SNIP_BF16 ? 32 : format == SNIP_FP8_E4M3 ? 64 : 128;
}

// Direct global -> LDS loads: lane l's 16 (4) bytes land at LDS byte
// address lds + 16 * l (4 * l); `lds` is wave-uniform (it goes to M0).
// Issued as asm so that the compiler, which cannot tell the ring slots
// apart, does not drain every load in flight before each LDS read; the
// waits for these loads are the explicit vmcnt waits of the main loop. One
// wait state separates the M0 write from the load that reads it.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds)
               : "memory", "m0");
}

// The same with a wave-uniform base address (scalar registers) and a 32-bit
// per-lane offset: no per-lane address arithmetic.
__device__ __forceinline__ void dma16s(const uint8_t* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4s(const uint8_t* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}

// Wait until at most N of this wave's vector-memory loads are outstanding
// and all its LDS reads have returned, then barrier. One asm statement with
// a memory clobber, so that no LDS access moves across it and no implicit
// full drain of the loads in flight is added.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// 8 E2M1 nibbles (one word) times an fp16 scale pair {s, s}: 8 exact fp16.
__device__ __forceinline__ half8_t decode_fp4(uint32_t w, half2_t s) {
  const half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
  const half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
  const half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
  const half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
  return half8_t{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// 8 E4M3 codes (two words) -> 8 fp16 values (exact).
__device__ __forceinline__ half8_t fp8x8_to_half8(uint32_t w0, uint32_t w1) {
  const half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
  const half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
  const half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
  const half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
  return half8_t{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// f(std::integral_constant<int, 0>{}), ..., f(std::integral_constant<int, N - 1>{}):
// a loop unrolled whatever the size of its body.
template <class F, int... I>
__device__ __forceinline__ void static_unroll_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_unroll(F&& f) {
  static_unroll_seq(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int q) {
  return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
}

// Workgroups per CU that the register budget is sized for. NVFP4 128x128
// tiles on a 2-stage ring of single units (36 KiB of LDS) fit three per CU
// in 144 registers without spills; measured on MI355X against the former
// two per CU (a 72 KiB ring of two units, or four single-unit stages):
// the tinyllama1b step's NVFP4 GEMMs 0.457 -> 0.441 ms.
template <int FMT, int BM, int BN, int S, int UK>
constexpr int gemm_min_wgs() {
  return BM * BN > 256 * 128 ? 1 : (FMT == SNIP_NVFP4 && BM == 128 && BN == 128 && S == 2 && UK == 1) ? 3 : 2;
}

// QO: the epilogue also quantizes C row-wise (store_tile_q; unsplit only).
template <int FMT, int BM, int BN, int S, int UK, bool QO = false>
__global__ __launch_bounds__(NT, (gemm_min_wgs<FMT, BM, BN, S, UK>())) void gemm_kernel(GemmArgs g_in) {
  using U = Unit<FMT>;
  constexpr int UE = U::UE, NQ = U::NQ, SB = U::SB;
  constexpr int RBA = BM / 16, RBB = BN / 16;              // 16-row blocks per tile
  constexpr int NUA = RBA * UK, NUB = RBB * UK;            // code units per stage
  constexpr int LA = NUA * 1024, LB = NUB * 1024;          // code bytes per stage
  constexpr int LSA = NUA * 16 * SB, LSB = NUB * 16 * SB;  // scale bytes per stage
  constexpr int STAGE = LA + LB + LSA + LSB;
  // DMA instructions per stage and wave: code units of A and of B, then
  // scale instructions (a dword per lane covers 256 bytes of scales)
  constexpr int NSA = LSA / 256, NSB = LSB / 256;
  constexpr int IA = NUA / 4, IB = NUB / 4, IS = (NSA + NSB) / 4;
  constexpr int NIW = IA + IB + IS;
  static_assert(NUA % 4 == 0 && NUB % 4 == 0 && (NSA + NSB) % 4 == 0, "DMA split over 4 waves");
  static_assert(LSA % 256 == 0 && LSB % 256 == 0, "scale staging granularity");
  static_assert(S >= 2 && NIW * (S > 2 ? S - 2 : 0) <= 63, "ring depth");
  constexpr int WM = BM / 2, WN = BN / 2;                  // wave tile
  constexpr int TM = WM / 16, TN = WN / 16;                // 16x16 MFMA tiles per wave
  constexpr int KS = UE * UK;                              // K elements per stage
  __shared__ __align__(1024) uint8_t smem[S * STAGE];
  if (finalize_workgroup(g_in)) return;

  // Grouped launch: workgroups past the first problem's tiles take the
  // second problem (unsplit), with tile ids counted from its first tile.
  GemmArgs g = g_in;
  int tile = blockIdx.x;
  if (g_in.nsec && tile >= g_in.tiles_m * g_in.tiles_n) {
    tile -= g_in.tiles_m * g_in.tiles_n;
    g.a = g_in.sec.a;
    g.b = g_in.sec.b;
    g.as = g_in.sec.as;
    g.bs = g_in.sec.bs;
    g.ea = g_in.sec.ea;
    g.eb = g_in.sec.eb;
    g.c = g_in.sec.c;
    g.M = g_in.sec.M;
    g.N = g_in.sec.N;
    g.K = g_in.sec.K;
    g.ldc = g_in.sec.ldc;
    g.kchunk = g_in.sec.K;
    g.tiles_m = g_in.sec.tiles_m;
    g.tiles_n = g_in.sec.tiles_n;
  }

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int wm = wave >> 1, wn = wave & 1;
  const int r16 = lane & 15, grp = lane >> 4;
  int tm, tn;
  tile_coords(tile, g.tiles_m, g.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t rowbytes = g.K / UE * 64;                  // code bytes per row
  const int64_t srow = SB ? g.K / UE * SB : 0;             // scale bytes per row
  const int kt0 = (int)(blockIdx.y * g.kchunk / KS);
  const int kt1 = min((int)(g.K / KS), (int)((blockIdx.y + 1) * g.kchunk / KS));
  const int nk = kt1 - kt0;

  // Per-lane DMA sources of this wave's instructions: wave w loads the code
  // units w, w + 4, ... of A and of B (unit index = row block * UK + unit
  // of the stage), and scale instructions w, w + 4, ... of the list
  // [A scales, B scales]. Offsets are 32-bit (the host keeps every operand
  // below 4 GiB). Rows past M or N load row M-1 / N-1 instead (in bounds);
  // their products are never stored.
  uint32_t offa[IA], offb[IB], offs[IS > 0 ? IS : 1];
#pragma unroll
  for (int t = 0; t < IA; ++t) {
    const int idx = wave + 4 * t;
    offa[t] = (uint32_t)(min(m0 + (idx / UK) * 16 + (lane >> 2), g.M - 1) * rowbytes) + (idx % UK) * 64 + (lane & 3) * 16;
  }
#pragma unroll
  for (int t = 0; t < IB; ++t) {
    const int idx = wave + 4 * t;
    offb[t] = (uint32_t)(min(n0 + (idx / UK) * 16 + (lane >> 2), g.N - 1) * rowbytes) + (idx % UK) * 64 + (lane & 3) * 16;
  }
#pragma unroll
  for (int t = 0; t < IS; ++t) {
    const int pp = wave + 4 * t;
    const bool isa = pp < NSA;
    const int p = isa ? pp : pp - NSA;
    // scale blocks [16 rows][SB bytes], one per code unit: NVFP4 2 blocks
    // per instruction, MX 4
    const int blk = SB == 8 ? 2 * p + (lane >> 5) : 4 * p + (lane >> 4);
    const int r = SB == 8 ? (lane & 31) >> 1 : lane & 15;
    const int part = SB == 8 ? (lane & 1) * 4 : 0;
    const int64_t row = isa ? min(m0 + (blk / UK) * 16 + r, g.M - 1) : min(n0 + (blk / UK) * 16 + r, g.N - 1);
    offs[t] = (uint32_t)(row * srow) + (blk % UK) * SB + part;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  auto issue = [&](int kt, int slot) {
    const uint32_t base = lds0 + slot * STAGE;
#pragma unroll
    for (int t = 0; t < IA; ++t) dma16(g.a + (int64_t)kt * UK * 64 + offa[t], base + (wave + 4 * t) * 1024);
#pragma unroll
    for (int t = 0; t < IB; ++t)
      dma16(g.b + (int64_t)kt * UK * 64 + offb[t], base + LA + (wave + 4 * t) * 1024);
#pragma unroll
    for (int t = 0; t < IS; ++t) {
      const int pp = wave + 4 * t;                       // wave-uniform
      if (pp < NSA) dma4(g.as + (int64_t)kt * UK * SB + offs[t], base + LA + LB + pp * 256);
      else dma4(g.bs + (int64_t)kt * UK * SB + offs[t], base + LA + LB + LSA + (pp - NSA) * 256);
    }
  };

  // Fragments of one unit in registers: A and B code slices (16 bytes per
  // lane) and the lane's block scales (NVFP4: two per fragment as fp16).
  struct Frags {
    uint4 a[TM], b[TN];
    half2_t sa[SB == 8 ? TM : 1], sb[SB == 8 ? TN : 1];
    int xa[SB == 4 ? TM : 1], xb[SB == 4 ? TN : 1];
  };
  auto load = [&](Frags& f, int slot, int u) {        // B first: decoded first
    const uint8_t* base = smem + slot * STAGE;
    const uint8_t* la = base + ((wm * TM) * UK + u) * 1024 + r16 * 64 + grp * 16;
    const uint8_t* lb = base + LA + ((wn * TN) * UK + u) * 1024 + r16 * 64 + grp * 16;
#pragma unroll
    for (int j = 0; j < TN; ++j) f.b[j] = *reinterpret_cast<const uint4*>(lb + j * UK * 1024);
    if constexpr (SB == 8) {        // lane (r16, grp): blocks 2grp, 2grp+1 of its row
      const uint8_t* sb = base + LA + LB + LSA + (((wn * TN) * UK + u) * 16 + r16) * 8 + grp * 2;
#pragma unroll
      for (int j = 0; j < TN; ++j)
        f.sb[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(
            (uint32_t)*reinterpret_cast<const uint16_t*>(sb + j * UK * 128), 1.0f, false);
    } else if constexpr (SB == 4) { // lane (r16, grp): block grp of its row
      const uint8_t* sb = base + LA + LB + LSA + (((wn * TN) * UK + u) * 16 + r16) * 4 + grp;
#pragma unroll
      for (int j = 0; j < TN; ++j) f.xb[j] = sb[j * UK * 64];
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) f.a[i] = *reinterpret_cast<const uint4*>(la + i * UK * 1024);
    if constexpr (SB == 8) {
      const uint8_t* sa = base + LA + LB + (((wm * TM) * UK + u) * 16 + r16) * 8 + grp * 2;
#pragma unroll
      for (int i = 0; i < TM; ++i)
        f.sa[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(
            (uint32_t)*reinterpret_cast<const uint16_t*>(sa + i * UK * 128), 1.0f, false);
    } else if constexpr (SB == 4) {
      const uint8_t* sa = base + LA + LB + (((wm * TM) * UK + u) * 16 + r16) * 4 + grp;
#pragma unroll
      for (int i = 0; i < TM; ++i) f.xa[i] = sa[i * UK * 64];
    }
  };

  floatx4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  // Decoded fp16 fragments (NVFP4, FP8): A_i or B_j for K slice q.
  auto dec_a = [&](const Frags& f, int q, int i) -> half8_t {
    if constexpr (FMT == SNIP_NVFP4) {
      const _Float16 s = q < 2 ? f.sa[i][0] : f.sa[i][1];
      return decode_fp4(word_of(f.a[i], q), half2_t{s, s});
    } else {
      return fp8x8_to_half8(word_of(f.a[i], 2 * q), word_of(f.a[i], 2 * q + 1));
    }
  };
  auto dec_b = [&](const Frags& f, int q, int j) -> half8_t {
    if constexpr (FMT == SNIP_NVFP4) {
      const _Float16 s = q < 2 ? f.sb[j][0] : f.sb[j][1];
      return decode_fp4(word_of(f.b[j], q), half2_t{s, s});
    } else {
      return fp8x8_to_half8(word_of(f.b[j], 2 * q), word_of(f.b[j], 2 * q + 1));
    }
  };

  // One stage's MFMAs, in rows (q, i): fragment A_i against every B_j for
  // K slice q; the B fragments of a slice are decoded once, at its first row.
  auto run_stage = [&](const Frags& f) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      half8_t bd[TN];
      if constexpr (FMT == SNIP_NVFP4 || FMT == SNIP_FP8_E4M3) {
#pragma unroll
        for (int j = 0; j < TN; ++j) bd[j] = dec_b(f, q, j);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if constexpr (FMT == SNIP_NVFP4 || FMT == SNIP_FP8_E4M3) {
          const half8_t ad = dec_a(f, q, i);
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ad, bd[j], acc[i][j], 0, 0, 0);
        } else if constexpr (FMT == SNIP_BF16) {
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, f.a[i]),
                                                                __builtin_bit_cast(bf16x8_t, f.b[j]),
                                                                acc[i][j], 0, 0, 0);
        } else {  // MXFP4: one scaled MFMA (K = 128) per fragment pair
          const intx8_t av = {(int)f.a[i].x, (int)f.a[i].y, (int)f.a[i].z, (int)f.a[i].w, 0, 0, 0, 0};
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const intx8_t bv = {(int)f.b[j].x, (int)f.b[j].y, (int)f.b[j].z, (int)f.b[j].w, 0, 0, 0, 0};
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[i][j], 4, 4, 0,
                                                                         f.xa[i], 0, f.xb[j]);
          }
        }
      }
    }
  };

  // Stage `it`: wait for this wave's loads of `it` (later stages may still
  // be in flight: stages up to it+S-2 have been issued), barrier (every
  // wave's loads of `it` are in LDS, and every wave has finished reading
  // stage it-1), refill stage it-1's slot with stage it+S-1 and read the
  // fragments (in either order: they touch different slots), multiply.
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nk) issue(kt0 + s, s);
  // NVFP4 keeps the slots of stages it and it+S-1 in counters advanced each
  // iteration, and picks its wait by iteration count; FP8 derives both from
  // `it`. The two forms compute the same slots and waits; their code
  // schedules differ, and each format keeps the one that measured faster
  // on MI355X (NVFP4 with counters 1-1.5 % faster on the tinyllama1b and
  // llama7b steps; FP8 with counters 2 % slower).
  constexpr bool kSlotCounters = FMT == SNIP_NVFP4;
  int srd = 0, swr = S - 1;
  for (int it = 0; it < nk; ++it) {
    if constexpr (kSlotCounters) {
      // S-2 stages are in flight behind stage it for it < nk-(S-2)
      if (S > 2 && it < nk - (S - 2)) wait_vm_barrier<NIW * (S > 2 ? S - 2 : 0)>();
      else if (S > 3 && it == nk - 2) wait_vm_barrier<NIW>();
      else wait_vm_barrier<0>();
    } else {
      const int ahead = min(S - 2, nk - 1 - it);       // stages issued after it
      if (S > 2 && ahead >= S - 2) wait_vm_barrier<NIW * (S > 2 ? S - 2 : 0)>();
      else if (S > 3 && ahead == 1) wait_vm_barrier<NIW>();
      else wait_vm_barrier<0>();
    }
    const int rd = kSlotCounters ? srd : it % S;        // slot of stage it
    const int wr = kSlotCounters ? swr : (it + S - 1) % S;  // slot of stage it+S-1
    // FP8 issues the refill after its fragment reads, so the DMA address
    // and issue instructions run in the shadow of the LDS read latency:
    // measured on MI355X, the tinyllama1b step's FP8 GEMMs 0.609 -> 0.594
    // ms; NVFP4 measured 1-2 % slower that way and keeps the refill first.
    constexpr bool kRefillLate = FMT == SNIP_FP8_E4M3;
    if (!kRefillLate && it + S - 1 < nk) issue(kt0 + it + S - 1, wr);
    Frags f[UK];
#pragma unroll
    for (int u = 0; u < UK; ++u) load(f[u], rd, u);
    if (kRefillLate && it + S - 1 < nk) issue(kt0 + it + S - 1, wr);
    if constexpr (kSlotCounters) {
      srd = srd == S - 1 ? 0 : srd + 1;
      swr = swr == S - 1 ? 0 : swr + 1;
    }
    // FP8: the wave runs its stage's MFMAs at raised issue priority, so that
    // with two or three waves per SIMD the one multiplying keeps the matrix
    // pipe while the others read and decode. Measured on MI355X: 3-15 %
    // faster for back-to-back GEMMs of 2048-16384 rows (most on the largest),
    // neutral inside the layer step; neutral to slightly slower for NVFP4,
    // so not used there.
    if constexpr (FMT == SNIP_FP8_E4M3) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int u = 0; u < UK; ++u) run_stage(f[u]);
    if constexpr (FMT == SNIP_FP8_E4M3) __builtin_amdgcn_s_setprio(0);
  }

  if constexpr (QO) {
    static_assert(4 * 16 * (TN * 16 + 4) * 4 <= S * STAGE, "output staging fits in the operand ring");
    store_tile_q<TM, TN>(g, acc, m0 + wm * WM, n0 + wn * WN, r16, grp, smem);
  }
  else store_tile<TM, TN>(g, acc, m0 + wm * WM, n0 + wn * WN, r16, grp);
}

// acc += a . b on v_mfma_f32_16x16x32_f16 with the accumulator kept in place
// in AGPRs: 256 accumulator registers fill the AGPR file, and the compiler's
// own MFMA selection, which may write a result to other registers than its
// input, then moves accumulators through VGPRs and spills.
// The compiler does not model an asm MFMA's hazards: a VALU result it reads
// needs 2+ independent instructions in between, and reading its result back
// needs the MFMA's latency. mfma_guard() (32 wait states, fenced against
// code motion) separates the prologue's decode from the first asm MFMA and
// the last asm MFMA from the epilogue's accumulator reads; inside the loop
// every operand is decoded at least four MFMAs before its use.
__device__ __forceinline__ void mfma_acc_agpr(floatx4_t& acc, const half8_t& a, const half8_t& b) {
  asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_guard() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Epilogue of a wave's 128x128 sub-tile whose MFMAs took B as the first
// operand: lane (r16, grp) holds C[r0 + 16 i + r16][c0 + 16 j + 4 grp + v],
// v = 0..3, so each 16x16 block is one 16-byte write per lane, scaled by
// 2^e. A sub-tile wholly inside C with 16-byte aligned rows is stored as
// TM * TN such writes per lane, all lanes active; otherwise element by
// element with bounds checks. Returns true for the first form.
template <int TM, int TN>
__device__ __forceinline__ bool store_tile_rows(const GemmArgs& g, const floatx4_t (&acc)[TM][TN], int64_t r0,
                                                int64_t c0, int r16, int grp, int e) {
  if (r0 + 16 * TM <= g.M && c0 + 16 * TN <= g.N && (g.ldc & 3) == 0 && ((uintptr_t)g.c & 15) == 0) {
    // one lane offset, stepped by 16 rows per row block (kept opaque, so
    // that no per-block addresses are precomputed into registers). The
    // offset, not the pointer, goes through the asm: a pointer would lose
    // its address space, and flat stores also count in lgkmcnt, which every
    // barrier of the K loop waits to zero.
    int64_t off = ((r0 + r16) * g.ldc + c0 + 4 * grp) * 4;
    int64_t step = 16 * g.ldc * 4;
    asm volatile("" : "+s"(step));
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      float* const rowp = reinterpret_cast<float*>(reinterpret_cast<char*>(g.c) + off);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        *reinterpret_cast<floatx4_t*>(rowp + j * 16) =
            floatx4_t{ldexpf(acc[i][j][0], e), ldexpf(acc[i][j][1], e), ldexpf(acc[i][j][2], e),
                      ldexpf(acc[i][j][3], e)};
      off += step;
      asm volatile("" : "+v"(off));
      __builtin_amdgcn_sched_barrier(0);
    }
    return true;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = r0 + i * 16 + r16, col = c0 + j * 16 + 4 * grp + v;
        if (row < g.M && col < g.N) g.c[row * g.ldc + col] = ldexpf(acc[i][j][v], e);
        __builtin_amdgcn_sched_barrier(0);
      }
  return false;
}

// Multiprocessors (CUs) of the current device, cached per device.
static int device_cus() {
  static int cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    cus[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  }
  return cus[dev];
}

// NVFP4 on 256x256 tiles, one wave per SIMD, each wave a 128x128 sub-tile.
//
// The NVFP4 decode costs one VALU instruction per element (half a
// v_cvt_scalef32_pk_f16_fp4, half a v_pk_mul_f16: the convert applies only
// the exponent of its scale operand, so the E4M3 scale's mantissa needs the
// multiply). A wave's sub-tile of WM x WN decodes (WM + WN) * 32 elements per
// K slice of 32 for WM * WN / 256 MFMAs: 3 VALU per MFMA on 128x64, 2 on
// 128x128. Measured on MI355X: while one wave streams
// v_mfma_f32_16x16x32_f16 (16 cycles each), another wave on the same SIMD
// issues a VALU instruction every 8-9.5 cycles, so about 2 fit under each
// MFMA; at 3 per MFMA the 128x64 sub-tiles are bound by VALU issue.
//
// Schedule: within K slice q, the MFMAs of A row block i run beside the
// decode of A row block i+1 and of B block i for slice q+1 (16 VALU per 8
// MFMAs). The stage's raw codes and scales are in registers, read from the
// LDS ring before its last slice: a barrier there (stage it+1 has landed,
// every wave has read stage it) lets the wave refill stage it's slot with
// stage it+4 and read stage it+1, whose first slice it decodes during the
// last slice of stage it. The refill's loads and the 32 reads go one
// after each MFMA (rows 6-7 of slice 2, rows 0-1 of slice 3): issued in a
// burst they left the lone wave's MFMA pipe idle (measured on MI355X:
// without the refill loads a timing copy ran 20 % faster; spread, the
// Llama-70B block step went from 17.99 to 17.69 ms). Ring: 4 stages of
// K = 128 codes (32 KiB each).
//
// Scales. A row holds 8 E4M3 bytes per stage, rows K/16 bytes apart. Each
// load instruction costs the MFMA stream about the same whatever it moves
// (measured on MI355X: a timing copy without the scale refills, a third of
// the loads and 1/9 of the bytes, ran 4-5 % faster), so a row's scales of
// two stages (16 contiguous bytes) come in one 16-byte load per lane: a
// group of 256 A and 256 B rows is 8 KiB, two loads per wave, issued with
// the even stage's refill into a 3-slot ring of groups (the slot's previous
// group was last read before the stage before). K % 256 == 0, so the
// stages of a workgroup's stream alternate even and odd from tile to tile.
//
// Persistent (without QO): the launch has one workgroup per CU, P in all,
// and workgroup b runs tiles b, b + P, b + 2P, ... Every tile takes the same
// time, so with one tile per workgroup each round of 256 tiles ends with all
// of them writing their 256 KiB at once, and the next round's tiles start
// only then (measured on MI355X: the kernel without its C store was 13 %
// faster at K = 4096 and 6 % at K = 8192). Here a tile's end loads the next
// tile's first four stages, then issues the tile's store, which drains
// while the next tile multiplies. The MFMAs take B as the first operand,
// so a lane's four results of a 16x16 block lie in one row of C and the
// store is 64 16-byte writes per lane. Loads issued after it share their
// counter (vmcnt counts loads and stores, in order): in the first three
// stages after a store, the wait for the next stage allows 63 operations in
// flight, which the 64 writes issued after that stage's loads guarantee;
// the fourth stage's wait covers the store. QO runs one tile per
// workgroup: its epilogue stages C in the ring.
template <bool QO>
__global__ __launch_bounds__(NT, 1) void gemm_nvfp4_w1_kernel(GemmArgs g) {
  constexpr int S = 4, NU = 16;                            // stages; 16-row units per operand
  constexpr int LA = NU * 1024, LB = NU * 1024;            // code bytes per stage
  constexpr int STAGE = LA + LB;
  constexpr int SG = 2 * NU * 16 * 16, NG = 3;             // scale group (two stages of A and B rows); ring slots
  constexpr int IA = NU / 4, IB = NU / 4, IS = 2;          // per wave: code loads of a stage, scale loads of a group
  constexpr int NE = IA + IB + IS, NO = IA + IB;           // loads per wave of an even and of an odd stage
  constexpr int TM = 8, TN = 8;                            // 16x16 MFMA tiles per wave
  static_assert(NE + NO + NE <= 63, "vmcnt range");
  static_assert(TM * TN >= 63, "a tile's 16-byte writes alone fill the vmcnt window");
  static_assert(NE <= 2 * TN, "a stage's loads go out in two rows of MFMAs");
  static_assert(SG == 4 * IS * 1024, "a group is the waves' 16-byte loads of 64 rows each");
  static_assert(S * STAGE + NG * SG <= 160 * 1024, "LDS");
  __shared__ __align__(1024) uint8_t smem[S * STAGE + NG * SG];

  const int P = (int)gridDim.x - g.fin.n;                  // tile workgroups
  if ((int)blockIdx.x >= P) {
    if (blockIdx.y == 0) finalize_one(g.fin.j[blockIdx.x - P]);
    return;
  }
  const int tiles = g.tiles_m * g.tiles_n;
  const int nk = (int)(g.K / 128);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int r16 = lane & 15, grp = lane >> 4;
  const int64_t rowbytes = g.K / 128 * 64, srow = g.K / 16;

  // DMA sources of the tile at (m0, n0), as in gemm_kernel with one unit per
  // stage: wave w loads code units w, w+4, ... of A and of B, and of a scale
  // group A rows 64 w .. 64 w + 63 and B rows the same, lane l row 64 w + l;
  // rows past M or N read the last row. Per lane a 32-bit offset from the
  // operand's start.
  uint32_t offa[IA], offb[IB], offs[IS];
  auto sources = [&](int64_t m0, int64_t n0) {
#pragma unroll
    for (int t = 0; t < IA; ++t)
      offa[t] = (uint32_t)(min(m0 + (wave + 4 * t) * 16 + (lane >> 2), g.M - 1) * rowbytes) + (lane & 3) * 16;
#pragma unroll
    for (int t = 0; t < IB; ++t)
      offb[t] = (uint32_t)(min(n0 + (wave + 4 * t) * 16 + (lane >> 2), g.N - 1) * rowbytes) + (lane & 3) * 16;
    offs[0] = (uint32_t)(min(m0 + wave * 64 + lane, g.M - 1) * srow);
    offs[1] = (uint32_t)(min(n0 + wave * 64 + lane, g.N - 1) * srow);
  };
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  const uint32_t sg0 = S * STAGE;                          // scale ring, bytes into smem
  // stage kt of the tile whose rows lie dm (A) and dn (B) rows past the
  // tile the offsets were worked out for, and with an even kt the scale
  // group of stages kt and kt+1 into group slot gsl; the bases are scalar,
  // and the wave's LDS base is made opaque per call so that the compiler
  // does not keep each instruction's LDS address in a register of its own
  auto issue = [&](int kt, int slot, int dm, int dn, int gsl) {
    uint32_t lw = lds0 + slot * STAGE + wave * 1024, ls = lds0 + sg0 + gsl * SG + wave * 1024;
    asm volatile("" : "+s"(lw), "+s"(ls));
    const uint8_t* pa = g.a + (int64_t)dm * rowbytes + (int64_t)kt * 64;
    const uint8_t* pb = g.b + (int64_t)dn * rowbytes + (int64_t)kt * 64;
#pragma unroll
    for (int t = 0; t < IA; ++t) dma16s(pa, offa[t], lw + t * 4096);
#pragma unroll
    for (int t = 0; t < IB; ++t) dma16s(pb, offb[t], lw + LA + t * 4096);
    if ((kt & 1) == 0) {
      dma16s(g.as + (int64_t)dm * srow + (int64_t)kt * 8, offs[0], ls);
      dma16s(g.bs + (int64_t)dn * srow + (int64_t)kt * 8, offs[1], ls + SG / 2);
    }
  };

  // load d of a refill whose global bases (codes of A and B, scales of A
  // and B) and LDS bases (code slot, group slot) are given; each LDS base
  // is copied through an empty asm so that no per-instruction LDS address
  // is kept in a register of its own
  auto refill1 = [&](const uint8_t* pa, const uint8_t* pb, const uint8_t* psa, const uint8_t* psb, uint32_t lw0,
                     uint32_t ls0, int d) {
    if (d < IA + IB) {
      uint32_t lw = lw0;
      asm volatile("" : "+s"(lw));
      if (d < IA) dma16s(pa, offa[d], lw + d * 4096);
      else dma16s(pb, offb[d - IA], lw + LA + (d - IA) * 4096);
    } else {
      uint32_t ls = ls0;
      asm volatile("" : "+s"(ls));
      if (d == IA + IB) dma16s(psa, offs[0], ls);
      else dma16s(psb, offs[1], ls + SG / 2);
    }
  };

  // A stage's raw operands in registers: code slices (16 bytes per lane)
  // and the lane's two E4M3 block-scale bytes per fragment. The scales are
  // converted to fp16 pairs where first needed, not where read: one wave per
  // SIMD has no other wave to run while it waits for an LDS read.
  struct RawA {
    uint4 a[TM];
    uint32_t s[TM];
  };
  struct RawB {
    uint4 b[TN];
    uint32_t s[TN];
  };
  // A stage's codes are in ring slot `slot`, its scales at byte sg of smem
  // (its group's slot, plus 8 for an odd stage): A row r's at sg + 16 r, B
  // row r's SG / 2 further
  auto read_a = [&](RawA& r, int slot, int sg) {
    const uint8_t* la = smem + slot * STAGE + (wm * TM) * 1024 + r16 * 64 + grp * 16;
    const uint8_t* sa = smem + sg + ((wm * TM) * 16 + r16) * 16 + grp * 2;
#pragma unroll
    for (int i = 0; i < TM; ++i) r.a[i] = *reinterpret_cast<const uint4*>(la + i * 1024);
#pragma unroll
    for (int i = 0; i < TM; ++i) r.s[i] = *reinterpret_cast<const uint16_t*>(sa + i * 256);
  };
  // The next stage's reads from lane addresses worked out once per stage
  // (codes at k KiB on, scales at 256 k bytes on: immediate offsets), each
  // passed through an empty asm so that the compiler keeps it rather than
  // rebuilding every read's address (two VALU additions a read).
  typedef const __attribute__((address_space(3))) uint8_t lds_u8;
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  typedef const __attribute__((address_space(3))) u32x4_t lds_u4;
  typedef const __attribute__((address_space(3))) uint16_t lds_u16;
  lds_u8* const lbase = (lds_u8*)smem;
  auto code_base = [&](int slot, int blk) {               // lane's first code read of 16-row block blk
    lds_u8* p = lbase + slot * STAGE + blk * 1024 + r16 * 64 + grp * 16;
    asm volatile("" : "+v"(p));
    return p;
  };
  auto scale_base = [&](int sg, int blk) {                // lane's first scale read of block blk
    lds_u8* p = lbase + sg + (blk * 16 + r16) * 16 + grp * 2;
    asm volatile("" : "+v"(p));
    return p;
  };
  auto read_b = [&](RawB& r, int slot, int sg) {
    const uint8_t* lb = smem + slot * STAGE + LA + (wn * TN) * 1024 + r16 * 64 + grp * 16;
    const uint8_t* sb = smem + sg + SG / 2 + ((wn * TN) * 16 + r16) * 16 + grp * 2;
#pragma unroll
    for (int j = 0; j < TN; ++j) r.b[j] = *reinterpret_cast<const uint4*>(lb + j * 1024);
#pragma unroll
    for (int j = 0; j < TN; ++j) r.s[j] = *reinterpret_cast<const uint16_t*>(sb + j * 256);
  };
  auto scale2 = [](uint32_t raw) -> half2_t { return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw, 1.0f, false); };
  // Pair p (of 4) of a fragment's decode for K slice q (elements 2p, 2p+1):
  // the E2M1 convert, then the multiply by the block scale.
  auto cvt = [](const uint4& w, int q, int p) -> half2_t {
    const uint32_t x = word_of(w, q);
    return p == 0 ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 0)
         : p == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 1)
         : p == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 2)
                  : __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 3);
  };
  auto mul = [](half2_t h, half2_t s2, int q) -> half2_t {
    const _Float16 s = q < 2 ? s2[0] : s2[1];
    return h * half2_t{s, s};
  };
  auto piece = [&](const uint4& w, half2_t s2, int q, int p) -> half2_t { return mul(cvt(w, q, p), s2, q); };
  auto join = [](std::initializer_list<half2_t> l) -> half8_t {
    const half2_t* h = l.begin();
    return half8_t{h[0][0], h[0][1], h[1][0], h[1][1], h[2][0], h[2][1], h[3][0], h[3][1]};
  };

  floatx4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  const int e = (g.ea ? *g.ea : 0) + (g.eb ? *g.eb : 0);
  auto interior = [&](int64_t r0, int64_t c0) { return r0 + 256 <= g.M && c0 + 256 <= g.N; };
  // Whether tile `tile` at (m0, n0) loads the first stages of the
  // workgroup's next tile during its own last stages, through its own
  // offsets shifted by (dm, dn) rows: both tiles wholly inside A and B, so
  // that neither has clamped rows.
  bool ahead = false;
  int dm = 0, dn = 0;
  auto plan_ahead = [&](int tile, int64_t m0, int64_t n0) {
    ahead = false;
    if (nk >= S && tile + P < tiles && interior(m0, n0)) {
      int tm2, tn2;
      tile_coords(tile + P, g.tiles_m, g.tiles_n, tm2, tn2);
      if (interior((int64_t)tm2 * 256, (int64_t)tn2 * 256)) {
        ahead = true;
        dm = (int)((int64_t)tm2 * 256 - m0);
        dn = (int)((int64_t)tn2 * 256 - n0);
      }
    }
  };
  int tile = blockIdx.x;
  int tm, tn;
  tile_coords(tile, g.tiles_m, g.tiles_n, tm, tn);
  int64_t m0 = (int64_t)tm * 256, n0 = (int64_t)tn * 256;
  sources(m0, n0);
  int slot = 0;                                          // slot of the stage to multiply next
  int gq = 0;                                            // its scale group's slot
#pragma unroll
  for (int s = 0; s < S; ++s)
    if (s < nk) issue(s, s, 0, 0, s >> 1);
  if constexpr (!QO) plan_ahead(tile, m0, n0);
  bool stored = false;                                   // a store was issued after this tile's first loads
  for (;;) {
    // stage 0's loads are followed by those of stages 1-3 (odd, even, odd)
    if (stored) wait_vm_barrier<63>();                   // the store's 64 writes follow the loads
    else if (nk >= 4) wait_vm_barrier<NO + NE + NO>();
    else wait_vm_barrier<NO>();
    RawA RA;
    RawB RB;
    read_a(RA, slot, sg0 + gq * SG);
    read_b(RB, slot, sg0 + gq * SG);
    half2_t sa[TM], sb[TN];                              // scales of the stage's fragments
#pragma unroll
    for (int i = 0; i < TM; ++i) sa[i] = scale2(RA.s[i]);
#pragma unroll
    for (int j = 0; j < TN; ++j) sb[j] = scale2(RB.s[j]);
    half8_t bd[TN], ad;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      bd[j] = join({piece(RB.b[j], sb[j], 0, 0), piece(RB.b[j], sb[j], 0, 1), piece(RB.b[j], sb[j], 0, 2),
                    piece(RB.b[j], sb[j], 0, 3)});
    }
    ad = join({piece(RA.a[0], sa[0], 0, 0), piece(RA.a[0], sa[0], 0, 1), piece(RA.a[0], sa[0], 0, 2),
               piece(RA.a[0], sa[0], 0, 3)});
    mfma_guard();

    // Stage it. While a stage it+1 follows, its B operands are read after
    // the barrier at row 6 of slice 2 and decoded for its first slice during
    // slice 3; its A operands are read at slice 3 (the first A block decoded
    // at slice 3's last row). Each MFMA is followed by one decode pair (a
    // convert and a multiply), pinned in that order; a fragment's scale pair
    // is converted in the group of its first decode (A blocks 1-7 of a stage
    // in slice 0). All stages run the same code, so the accumulators keep
    // their registers: a stage with its own copy of the loop body lets the
    // register allocator move them, and a compiler-inserted AGPR move right
    // before an asm MFMA that reads it is a hazard the compiler does not
    // see. The last stage reads (and decodes, unused) the next slot as it
    // stands: no load targets it any more.
    for (int it = 0; it < nk; ++it) {                    // stage it, in slot `slot`
      const bool more = it + 1 < nk;
      const int next = slot == S - 1 ? 0 : slot + 1;
      const bool odd = it & 1;
      const int gn = odd ? (gq == NG - 1 ? 0 : gq + 1) : gq;   // group slot of stage it+1,
      const int nsg = sg0 + gn * SG + (odd ? 0 : 8);           // its scales
      const int rgs = gq == 0 ? NG - 1 : gq - 1;               // of stage it+4 (even it)
      RawA NA;
      RawB NB;
      half2_t nsb[TN], nsa0;
      bool rf = false;                                   // this stage refills its slot: stage rkt of
      int rkt = 0, rdm = 0, rdn = 0;                     // the tile rdm / rdn rows on, from these bases
      const uint8_t *rpa = g.a, *rpb = g.b, *rpsa = g.as, *rpsb = g.bs;
      uint32_t rlw = 0, rls = 0;                         // and into these LDS bases
      lds_u8 *rcb = lbase, *rsb = lbase, *rca = lbase, *rsa = lbase;   // the next stage's read bases
      // slices and row blocks unrolled by templates: the unroller's size
      // limit would otherwise leave the slice loop rolled, its register
      // arrays indexed at run time (in scratch)
      static_unroll<4>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        half8_t bn[TN];
        static_unroll<TM>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          if constexpr (q == 2 && i == 6) {
            // the stream's stage it+1 has landed (and, as below, every wave
            // has read stage it). With `ahead` the stream runs on into the
            // next tile, two stages always following
            // (the loads of stages it+2 and it+3 follow stage it+1's, the
            // scales of an odd stage it+1 came with stage it's; near the
            // end only stage it+2, odd as nk is even, follows)
            if (more || ahead) {
              if (stored && it < S - 1) wait_vm_barrier<63>();
              else if (ahead || it + 3 < nk) wait_vm_barrier<NE + NO>();
              else if (it + 2 < nk) wait_vm_barrier<NO>();
              else wait_vm_barrier<0>();
            }
            // every wave has read stage it: its slot takes stage it+4, or
            // the next tile's stage it+4-nk (loads issued one per MFMA in
            // rows 6-7, beside the reads of stage it+1's B operands; its A
            // operands are read in rows 0-1 of the last slice)
            const bool own = it + S < nk;
            rf = own || ahead;
            rkt = own ? it + S : it + S - nk;
            rdm = own ? 0 : dm;
            rdn = own ? 0 : dn;
            // the refill's bases, worked out once for its loads
            rpa = g.a + (int64_t)rdm * rowbytes + (int64_t)rkt * 64;
            rpb = g.b + (int64_t)rdn * rowbytes + (int64_t)rkt * 64;
            rpsa = g.as + (int64_t)rdm * srow + (int64_t)rkt * 8;
            rpsb = g.bs + (int64_t)rdn * srow + (int64_t)rkt * 8;
            rlw = lds0 + slot * STAGE + wave * 1024;
            rls = lds0 + sg0 + rgs * SG + wave * 1024;
            rcb = code_base(next, NU + wn * TN);          // B codes: units after the 16 of A
          }
          if constexpr (q == 2 && i == 7) rsb = scale_base(nsg + SG / 2, wn * TN);
          if constexpr (q == 3 && i == 0) rca = code_base(next, wm * TM);
          if constexpr (q == 3 && i == 1) rsa = scale_base(nsg, wm * TM);
          // pieces 0-3: A block i+1 (or the next slice's block 0), pieces
          // 4-7: B block i for the next slice; group j converts piece j and
          // multiplies piece j-1, so no multiply waits on the convert just
          // issued (the last piece's multiply closes group 7)
          if constexpr (i < TM - 1) {
            if constexpr (q == 0) sa[i + 1] = scale2(RA.s[i + 1]);
          } else if constexpr (q == 3) {
            nsa0 = scale2(NA.s[0]);
          }
          if constexpr (q == 3) nsb[i] = scale2(NB.s[i]);
          auto cvt_j = [&](int j) -> half2_t {
            if (j < 4) return i < TM - 1 ? cvt(RA.a[i + 1], q, j) : q < 3 ? cvt(RA.a[0], q + 1, j) : cvt(NA.a[0], 0, j);
            return q < 3 ? cvt(RB.b[i], q + 1, j - 4) : cvt(NB.b[i], 0, j - 4);
          };
          auto mul_j = [&](int j, half2_t t) -> half2_t {
            if (j < 4) return i < TM - 1 ? mul(t, sa[i + 1], q) : q < 3 ? mul(t, sa[0], q + 1) : mul(t, nsa0, 0);
            return q < 3 ? mul(t, sb[i], q + 1) : mul(t, nsb[i], 0);
          };
          half2_t t[8], h[8];
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            if constexpr (QO) mfma_acc_agpr(acc[i][j], ad, bd[j]);
            else mfma_acc_agpr(acc[i][j], bd[j], ad);  // C transposed: a lane's results lie in one row
            if constexpr (q == 2 && i == 6) {
              if (rf) refill1(rpa, rpb, rpsa, rpsb, rlw, rls, j);
              NB.b[j] = __builtin_bit_cast(uint4, *(lds_u4*)(rcb + j * 1024));
            }
            if constexpr (q == 2 && i == 7) {
              if (j < IS && rf && !odd) refill1(rpa, rpb, rpsa, rpsb, rlw, rls, TN + j);
              NB.s[j] = *(lds_u16*)(rsb + j * 256);
            }
            if constexpr (q == 3 && i == 0) NA.a[j] = __builtin_bit_cast(uint4, *(lds_u4*)(rca + j * 1024));
            if constexpr (q == 3 && i == 1) NA.s[j] = *(lds_u16*)(rsa + j * 256);
            t[j] = cvt_j(j);
            asm volatile("" : "+v"(t[j]));             // computed here, not sunk to its use
            if (j > 0) {
              h[j - 1] = mul_j(j - 1, t[j - 1]);
              asm volatile("" : "+v"(h[j - 1]));
            }
            if (j == TN - 1) {
              h[j] = mul_j(j, t[j]);
              asm volatile("" : "+v"(h[j]));
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          ad = join({h[0], h[1], h[2], h[3]});
          bn[i] = join({h[4], h[5], h[6], h[7]});
        });
#pragma unroll
        for (int j = 0; j < TN; ++j) bd[j] = bn[j];
      });
      RA = NA;
      RB = NB;
      sa[0] = nsa0;
#pragma unroll
      for (int j = 0; j < TN; ++j) sb[j] = nsb[j];
      slot = next;
      gq = gn;
      // before any accumulator read: at the end of every stage (under 1 %
      // of its time) rather than after the loop, so that what the compiler
      // places on the loop's exit edge comes after it
      mfma_guard();
    }
    if constexpr (QO) break;
    // the tile is complete: unless its last stages loaded them, the next
    // tile's first stages go into the ring once every wave is done with
    // it; then this tile's store is issued
    const int64_t cm0 = m0, cn0 = n0;
    tile += P;
    const bool last = tile >= tiles;
    if (!last) {
      tile_coords(tile, g.tiles_m, g.tiles_n, tm, tn);
      m0 = (int64_t)tm * 256;
      n0 = (int64_t)tn * 256;
      sources(m0, n0);
      if (!ahead) {
        wait_vm_barrier<63>();
#pragma unroll
        for (int s = 0; s < S; ++s)
          if (s < nk) issue(s, (slot + s) & (S - 1), 0, 0, s < 2 ? gq : gq == NG - 1 ? 0 : gq + 1);
      }
      plan_ahead(tile, m0, n0);
    }
    stored = store_tile_rows<TM, TN>(g, acc, cm0 + wm * 128, cn0 + wn * 128, r16, grp, e);
    if (!stored) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the checked form may write less
    if (last) break;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    mfma_guard();                                        // the cleared accumulators before the next MFMA
  }

  if constexpr (QO) {                                    // the workgroup's one tile
    static_assert(4 * 16 * (TN * 16 + 4) * 4 <= S * STAGE, "output staging fits in the operand ring");
    store_tile_q<TM, TN>(g, acc, m0 + wm * 128, n0 + wn * 128, r16, grp, smem);
  }
}

// acc += A . B on the scaled 4-bit MFMA (MX-FP4: E2M1 codes, one E8M0
// scale per row and 32-element K block, passed in the instruction) with
// the accumulator kept in place in AGPRs, as mfma_acc_agpr.
// The instruction reads byte 0 of each scale register (op_sel 0); the
// other bytes are ignored.
__device__ __forceinline__ void mfma_mx_acc_agpr(floatx4_t& acc, const uint4& a, const uint4& b, uint32_t sa,
                                                 uint32_t sb) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:4 blgp:4"
               : "+a"(acc)
               : "v"(__builtin_bit_cast(u32x4, a)), "v"(__builtin_bit_cast(u32x4, b)), "v"(sa), "v"(sb));
}

// MX-FP4 on 256x256 tiles, one wave per SIMD, each wave a 128x128 sub-tile,
// one tile per workgroup (K % 512 != 0; gemm_mxfp4_w1p_kernel below takes
// the rest): the structure of gemm_nvfp4_w1_kernel without a decode (the MFMA takes
// the codes and block scales as they are). A stage (K = 128) is 64 MFMAs
// per wave, 16 cycles each at the FP4 rate, against 16 LDS reads of codes,
// 16 of scale words and 10 DMA instructions, so the code ring runs 4
// stages deep (32 KiB each) and the next stage's operands are read during
// the current one: after row 3 of the 8 MFMA rows a barrier (stage it+1
// has landed, every wave has read stage it) opens the refill of stage it's
// slot with stage it+4, and the reads of stage it+1 go one per MFMA into
// rows 4-7. Stages past the end reload the last one (never read as
// operands), so every stage issues the same loads and waits the same.
//
// Scales. A row holds 4 E8M0 bytes per stage, and rows lie K/32 bytes
// apart, so loading one stage's scales costs one L2 request per row: as
// many requests as the stage's 64-byte code segments (measured: without the
// scale loads the kernel ran 26-34 % faster). They are loaded 4 stages at a
// time instead, the 16 contiguous bytes of a row by a quad of lanes (one
// request), into a 3-slot ring of 8 KiB groups (512 rows x 16 bytes). A
// group's 32 instructions (16 rows each) are spread over the 4 stages that
// run 8 to 5 stages before its first stage, 2 per wave and stage, so every
// stage still issues 10 loads and group g is in LDS by the barrier that
// precedes its first read (which waits for everything issued 3 or more
// stages earlier).
__global__ __launch_bounds__(NT, 1) void gemm_mxfp4_w1_kernel(GemmArgs g_in) {
  constexpr int S = 4, NU = 16;                            // code stages; 16-row units per operand
  constexpr int LA = NU * 1024, LB = NU * 1024;            // code bytes per stage
  constexpr int STAGE = LA + LB;
  constexpr int SG = 512 * 16, NG = 3;                     // scale group bytes (4 stages), ring slots
  constexpr int IA = NU / 4, IB = NU / 4, IS = 2;          // per wave and stage: 32 instructions per group
  constexpr int NIW = IA + IB + IS;                        // DMA instructions per wave and stage
  constexpr int TM = 8, TN = 8;
  static_assert((S - 1) * NIW <= 63, "vmcnt range");
  static_assert(NIW <= 4 * TN, "the refill fits in rows 4-7");
  static_assert(4 * 4 * IS == 32, "a group is 32 instructions over 4 stages and 4 waves");
  static_assert(S * STAGE + NG * SG <= 160 * 1024, "LDS");
  __shared__ __align__(1024) uint8_t smem[S * STAGE + NG * SG];
  if (finalize_workgroup(g_in)) return;

  const GemmArgs& g = g_in;                                // grouped launches never take this kernel
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int r16 = lane & 15, grp = lane >> 4;
  int tm, tn;
  tile_coords(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * 256, n0 = (int64_t)tn * 256;
  const int64_t rowbytes = g.K / 128 * 64, srow = g.K / 32;
  const int kt0 = (int)(blockIdx.y * g.kchunk / 128);
  const int kt1 = min((int)(g.K / 128), (int)((blockIdx.y + 1) * g.kchunk / 128));
  const int nk = kt1 - kt0;

  // code DMA sources: wave w loads units w, w+4, ... of A and of B. In LDS
  // row r's 16-byte chunk c sits at position c ^ swz(r), as in
  // gemm_mxfp4_w1p_kernel, so the reads meet no bank twice in a cycle.
  auto swz = [](int r) { return ((r >> 1) ^ (r >> 2)) & 3; };
  const int chunk = ((lane & 3) ^ swz(lane >> 2)) * 16;
  const int cpos = r16 * 64 + (grp ^ swz(r16)) * 16;
  uint32_t offa[IA], offb[IB];
#pragma unroll
  for (int t = 0; t < IA; ++t)
    offa[t] = (uint32_t)(min(m0 + (wave + 4 * t) * 16 + (lane >> 2), g.M - 1) * rowbytes) + chunk;
#pragma unroll
  for (int t = 0; t < IB; ++t)
    offb[t] = (uint32_t)(min(n0 + (wave + 4 * t) * 16 + (lane >> 2), g.N - 1) * rowbytes) + chunk;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  const uint32_t sl0 = lds0 + S * STAGE;                   // scale ring
  auto code1 = [&](int kt, int slot, int d) {
    const uint32_t base = lds0 + slot * STAGE;
    if (d < IA) dma16(g.a + (int64_t)kt * 64 + offa[d], base + (wave + 4 * d) * 1024);
    else dma16(g.b + (int64_t)kt * 64 + offb[d - IA], base + LA + (wave + 4 * (d - IA)) * 1024);
  };
  // scale instruction k (of 32) of group gi: 16 rows (A rows for k < 16,
  // then B rows), lane l the word l % 4 (stage 4 gi + l % 4) of row l / 4;
  // words past the last stage repeat the last stage's (kept in the row)
  auto scale1 = [&](int gi, int k) {
    const bool isa = k < 16;
    const int64_t row = isa ? min(m0 + (k & 15) * 16 + (lane >> 2), g.M - 1)
                            : min(n0 + (k & 15) * 16 + (lane >> 2), g.N - 1);
    const int word = min(kt0 + 4 * gi + (lane & 3), kt1 - 1);
    dma4((isa ? g.as : g.bs) + row * srow + word * 4, sl0 + (gi % NG) * SG + k * 256);
  };
  // the loads stage it issues (d of NIW): codes of stage it+4, then phase
  // it % 4 of scale group it/4 + 2
  auto issue1 = [&](int it, int slot, int d) {
    if (d < IA + IB) code1(min(kt0 + it + S, kt1 - 1), slot, d);
    else scale1(it / 4 + 2, (it & 3) * 8 + wave * 2 + (d - IA - IB));
  };

  // A stage's operands in registers: code slices (lane (r16, grp) holds K
  // elements 32 grp .. 32 grp + 31 of row r16) and, per fragment, row
  // r16's 4 block scales of the stage (one LDS word), shifted so that byte
  // 0 holds the lane's block grp
  struct Frags {
    uint4 a[TM], b[TN];
    uint32_t sa[TM], sb[TN];
  };
  // read k of 32 of stage it (code slot `slot`): A codes, B codes, A scales,
  // B scales (8 each)
  auto read1 = [&](Frags& f, int it, int slot, int k) {
    const uint8_t* base = smem + slot * STAGE;
    const uint8_t* sg = smem + S * STAGE + ((it / 4) % NG) * SG + (it & 3) * 4;
    if (k < 8) f.a[k] = *reinterpret_cast<const uint4*>(base + (wm * TM + k) * 1024 + cpos);
    else if (k < 16) f.b[k - 8] = *reinterpret_cast<const uint4*>(base + LA + (wn * TN + k - 8) * 1024 + cpos);
    else if (k < 24) f.sa[k - 16] = *reinterpret_cast<const uint32_t*>(sg + ((wm * TM + k - 16) * 16 + r16) * 16);
    else f.sb[k - 24] = *reinterpret_cast<const uint32_t*>(sg + 4096 + ((wn * TN + k - 24) * 16 + r16) * 16);
  };

  floatx4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  // prologue: scale group 0, then code stages 0-3 each with a quarter of
  // scale group 1, so that every stage's loads number NIW
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int t = 0; t < IS; ++t) scale1(0, p * 8 + wave * 2 + t);
#pragma unroll
  for (int s = 0; s < S; ++s) {
#pragma unroll
    for (int d = 0; d < IA + IB; ++d) code1(min(kt0 + s, kt1 - 1), s, d);
#pragma unroll
    for (int t = 0; t < IS; ++t) scale1(1, s * 8 + wave * 2 + t);
  }
  wait_vm_barrier<(S - 1) * NIW>();                      // scale group 0 and code stage 0 have landed
  Frags F;
#pragma unroll
  for (int k = 0; k < 32; ++k) read1(F, 0, 0, k);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    F.sa[i] >>= 8 * grp;
    F.sb[i] >>= 8 * grp;
  }
  mfma_guard();

  // Stage it with its operands in `cur`, reading stage it+1's into `nxt`.
  // Two stages per loop iteration with the fragment sets swapped, so no
  // registers are copied between stages (the loop holds a barrier, which
  // keeps the compiler from unrolling it); an odd last stage follows.
  int slot = 0;                                          // code slot of stage it
  auto stage = [&](int it, const Frags& cur, Frags& nxt) {
    const int next = slot == S - 1 ? 0 : slot + 1;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      // stage it+1 has landed (stages it+2, it+3 may still be in flight),
      // every wave has read stage it
      if (i == 4) wait_vm_barrier<(S - 2) * NIW>();
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        mfma_mx_acc_agpr(acc[i][j], cur.a[i], cur.b[j], cur.sa[i], cur.sb[j]);
        // the refill: NIW loads, one per MFMA from row 4 on
        if (i >= 4 && (i - 4) * TN + j < NIW) issue1(it, slot, (i - 4) * TN + j);
        // next stage's reads, the earliest needed first: B codes and scales
        // (row 0), A scales, A codes (A block i is first used in row i)
        if (i >= 4) read1(nxt, it + 1, next, i == 4 ? 8 + j : i == 5 ? 24 + j : i == 6 ? 16 + j : j);
        // in the last row, the next stage's scale words (read in rows 5-6)
        // get the lane's byte (K block grp) shifted to byte 0, long before
        // an MFMA reads them
        if (i == TM - 1) {
          nxt.sa[j] >>= 8 * grp;
          nxt.sb[j] >>= 8 * grp;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    slot = next;
  };
  // nk >= 1: K is a positive multiple of 128
  Frags N;
  int it = 0;
  for (; it + 1 < nk; it += 2) {
    stage(it, F, N);
    stage(it + 1, N, F);
  }
  if (it < nk) stage(it, F, N);
  mfma_guard();                                          // before any accumulator read
  wait_vm_barrier<0>();                                  // the reloads have landed before the workgroup ends
  store_tile<TM, TN>(g, acc, m0 + wm * 128, n0 + wn * 128, r16, grp);
}

// MX-FP4 on 256x256 tiles where K is a multiple of 512, persistent: the
// structure of gemm_mxfp4_w1_kernel (above) with two changes.
//
// Scales of whole groups. A row's 4 stages of scales are 16 bytes, which a
// lane loads in one 16-byte load: 8 instructions of 64 rows per group, A
// rows by each wave in the group's first stage and B rows in its third
// (each load instruction costs the MFMA stream about the same whatever it
// moves), so an even stage issues 9 loads and an odd one 8, and two
// successive stages always 17, which the waits rely on.
//
// Persistent: one workgroup per CU, workgroup b running tiles b, b + P,
// ... The fp32 C of a 256x256 tile is 256 KiB against 32 KiB of operands
// per stage, and with one tile per workgroup every round of tiles ended
// with all of them storing at once (measured on MI355X: without its C
// store the one-tile kernel ran 12-31 % faster at K = 4096-11008). Here a
// tile's store drains while the next tile multiplies. The MFMAs take B as
// the first operand, so a lane's four results of a 16x16 block lie in one
// row of C and the store is 64 16-byte writes per lane. With at least two
// groups per tile and both tiles wholly inside A and B, a tile's last 4
// stages load the next tile's stages 0-3 and its last 8 the next tile's
// scale groups 0-1 (the stream runs on through the rings: K % 512 == 0
// brings the code ring back to slot 0, the group ring moves on by K/512);
// otherwise stages and groups past the end reload the last one, and after
// its last stage the tile waits for every load and fills the rings afresh.
// Loads after a store share its counter (vmcnt counts loads and stores, in
// order): in the first three stages after a store the wait for the next
// stage allows 63 operations in flight, which the 64 writes issued after
// that stage's loads guarantee; the fourth stage's wait covers the store.
__global__ __launch_bounds__(NT, 1) void gemm_mxfp4_w1p_kernel(GemmArgs g) {
  constexpr int S = 4, NU = 16;                            // code stages; 16-row units per operand
  constexpr int LA = NU * 1024, LB = NU * 1024;            // code bytes per stage
  constexpr int STAGE = LA + LB;
  constexpr int SG = 512 * 16, NG = 3;                     // scale group bytes (4 stages), ring slots
  constexpr int IA = NU / 4, IB = NU / 4;                  // code loads per wave and stage
  constexpr int NIW = IA + IB + 1;                         // DMA instructions of an even stage
  constexpr int NIW2 = 2 * (IA + IB) + 1;                  // of two successive stages
  constexpr int TM = 8, TN = 8;
  static_assert(NIW + NIW2 <= 63, "vmcnt range");
  static_assert(TM * TN >= 63, "a tile's 16-byte writes alone fill the vmcnt window");
  static_assert(NIW <= 4 * TN, "the refill fits in rows 4-7");
  static_assert(2 * 4 * 64 == 512, "a group's rows: one 16-byte load of 64 rows per wave and operand");
  static_assert(S * STAGE + NG * SG <= 160 * 1024, "LDS");
  __shared__ __align__(1024) uint8_t smem[S * STAGE + NG * SG];

  const int P = (int)gridDim.x - g.fin.n;                  // tile workgroups
  if ((int)blockIdx.x >= P) {
    if (blockIdx.y == 0) finalize_one(g.fin.j[blockIdx.x - P]);
    return;
  }
  const int tiles = g.tiles_m * g.tiles_n;
  const int nk = (int)(g.K / 128);                         // stages of a tile
  const int ng = nk / 4;                                   // scale groups of a tile
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int r16 = lane & 15, grp = lane >> 4;
  const int64_t rowbytes = g.K / 2, srow = g.K / 32;

  // DMA sources of the tile at (m0, n0), per lane a 32-bit offset from the
  // operand's start: wave w loads code units w, w+4, ... of A and of B and
  // scale rows 64 w + lane of A and of B; rows past M or N read the last
  // row. In LDS a 16-row unit is 16 rows x 64 bytes with row r's 16-byte
  // chunk c at position c ^ swz(r): the MFMA-side reads (lane (r16, grp)
  // takes chunk grp of row r16, 16 bytes) then meet no bank twice in a
  // cycle, with 32 or 64 banks (with chunks in order, rows 64 bytes apart
  // did); the load's lane l brings the chunk that its slot (row l / 4,
  // position l % 4) holds.
  auto swz = [](int r) { return ((r >> 1) ^ (r >> 2)) & 3; };
  const int chunk = ((lane & 3) ^ swz(lane >> 2)) * 16;
  int64_t m0, n0;
  uint32_t offa[IA], offb[IB], offs[2];
  auto sources = [&]() {
#pragma unroll
    for (int t = 0; t < IA; ++t)
      offa[t] = (uint32_t)(min(m0 + (wave + 4 * t) * 16 + (lane >> 2), g.M - 1) * rowbytes) + chunk;
#pragma unroll
    for (int t = 0; t < IB; ++t)
      offb[t] = (uint32_t)(min(n0 + (wave + 4 * t) * 16 + (lane >> 2), g.N - 1) * rowbytes) + chunk;
    offs[0] = (uint32_t)(min(m0 + wave * 64 + lane, g.M - 1) * srow);
    offs[1] = (uint32_t)(min(n0 + wave * 64 + lane, g.N - 1) * srow);
  };
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  const uint32_t sl0 = lds0 + S * STAGE;                   // scale ring
  // load d of a stage's codes: stage kt of the tile dm (A) and dn (B) rows
  // past the one the offsets were worked out for, into code slot `slot`
  auto code1 = [&](int kt, int slot, int d, int dm, int dn) {
    uint32_t lw = lds0 + slot * STAGE + wave * 1024;
    asm volatile("" : "+s"(lw));
    if (d < IA) dma16s(g.a + (int64_t)dm * rowbytes + (int64_t)kt * 64, offa[d], lw + d * 4096);
    else dma16s(g.b + (int64_t)dn * rowbytes + (int64_t)kt * 64, offb[d - IA], lw + LA + (d - IA) * 4096);
  };
  // Scale instruction k (of 8) of group gi (of the tile dm / dn rows on)
  // into group slot gs: 64 rows (A rows for k < 4, then B rows), lane l row
  // 64 (k % 4) + l, its 16 bytes at 16 gi
  auto scale1 = [&](int gi, int k, int gs, int dm, int dn) {
    uint32_t lw = sl0 + gs * SG + k * 1024;
    asm volatile("" : "+s"(lw));
    if (k < 4) dma16s(g.as + (int64_t)dm * srow + (int64_t)gi * 16, offs[0], lw);
    else dma16s(g.bs + (int64_t)dn * srow + (int64_t)gi * 16, offs[1], lw);
  };
  // A tile's prologue (ring slots from 0): scale group 0, then code stages
  // 0-3 each with its part of scale group 1, as the stages 4 later issue
  // theirs; stages and groups past the end reload the last one
  auto prologue = [&]() {
    const int g1 = min(1, ng - 1);
    scale1(0, wave, 0, 0, 0);
    scale1(0, 4 + wave, 0, 0, 0);
#pragma unroll
    for (int s = 0; s < S; ++s) {
#pragma unroll
      for (int d = 0; d < IA + IB; ++d) code1(min(s, nk - 1), s, d, 0, 0);
      if ((s & 1) == 0) scale1(g1, (s & 2) * 2 + wave, 1, 0, 0);
    }
  };

  // A stage's operands in registers: code slices (lane (r16, grp) holds K
  // elements 32 grp .. 32 grp + 31 of row r16) and, per fragment, row
  // r16's 4 block scales of the stage (one LDS word), shifted so that byte
  // 0 holds the lane's block grp
  struct Frags {
    uint4 a[TM], b[TN];
    uint32_t sa[TM], sb[TN];
  };
  // read k of 32 of a stage in code slot `slot` whose scales are word w of
  // group slot gs: A codes, B codes, A scales, B scales (8 each)
  const int cpos = r16 * 64 + (grp ^ swz(r16)) * 16;     // the lane's chunk in a 16-row unit
  auto read1 = [&](Frags& f, int slot, int gs, int w, int k) {
    const uint8_t* base = smem + slot * STAGE;
    const uint8_t* sg = smem + S * STAGE + gs * SG + w * 4;
    if (k < 8) f.a[k] = *reinterpret_cast<const uint4*>(base + (wm * TM + k) * 1024 + cpos);
    else if (k < 16) f.b[k - 8] = *reinterpret_cast<const uint4*>(base + LA + (wn * TN + k - 8) * 1024 + cpos);
    else if (k < 24) f.sa[k - 16] = *reinterpret_cast<const uint32_t*>(sg + ((wm * TM + k - 16) * 16 + r16) * 16);
    else f.sb[k - 24] = *reinterpret_cast<const uint32_t*>(sg + 4096 + ((wn * TN + k - 24) * 16 + r16) * 16);
  };

  floatx4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  const int e = (g.ea ? *g.ea : 0) + (g.eb ? *g.eb : 0);
  auto interior = [&](int64_t r0, int64_t c0) { return r0 + 256 <= g.M && c0 + 256 <= g.N; };
  // Whether the tile at (m0, n0) streams on into the workgroup's next tile,
  // through its own offsets shifted by (dm, dn) rows: at least two groups (the next tile's group 0 is loaded 8 to 5 stages before
  // this tile ends, by its own refills), and both tiles wholly inside A and
  // B, so that neither has clamped rows.
  bool ahead = false;
  int dm = 0, dn = 0;
  int tile = blockIdx.x;
  auto plan_ahead = [&]() {
    ahead = false;
    if (ng >= 2 && tile + P < tiles && interior(m0, n0)) {
      int tm2, tn2;
      tile_coords(tile + P, g.tiles_m, g.tiles_n, tm2, tn2);
      if (interior((int64_t)tm2 * 256, (int64_t)tn2 * 256)) {
        ahead = true;
        dm = (int)((int64_t)tm2 * 256 - m0);
        dn = (int)((int64_t)tn2 * 256 - n0);
      }
    }
  };
  {
    int tm, tn;
    tile_coords(tile, g.tiles_m, g.tiles_n, tm, tn);
    m0 = (int64_t)tm * 256;
    n0 = (int64_t)tn * 256;
  }
  sources();
  prologue();
  plan_ahead();

  int slot = 0;                                          // code slot of the stage to multiply next
  int gb = 0;                                            // group slot of the tile's group 0
  bool stored = false;                                   // a store was issued after this tile's first loads
  bool have0 = false;                                    // F holds the tile's stage 0
  Frags F, N;
  // Stage it with its operands in `cur`, reading stage it+1's (with
  // `ahead`, after the last stage, the next tile's stage 0) into `nxt`.
  auto stage = [&](int it, const Frags& cur, Frags& nxt) {
    const int next = slot == S - 1 ? 0 : slot + 1;
    const int gr = (gb + (it + 1) / 4) % NG;             // group slot of stage it+1
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      // stage it+1 has landed (stages it+2, it+3 may still be in flight; in
      // the first three stages after a store, the store's writes too),
      // every wave has read stage it
      if (i == 4) {
        if (stored && it < S - 1) wait_vm_barrier<63>();
        else wait_vm_barrier<NIW2>();
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        // C transposed: a lane's results lie in one row
        mfma_mx_acc_agpr(acc[i][j], cur.b[j], cur.a[i], cur.sb[j], cur.sa[i]);
        // the refill, one load per MFMA from row 4 on: codes of stage it+4
        // (of the next tile with `ahead`, else the last stage again past the
        // end), then, in even stages, the stage's part of scale group it/4 + 2
        const int d = (i - 4) * TN + j;
        if (i >= 4 && d < NIW && (d < IA + IB || (it & 1) == 0)) {
          const int st = it + S;
          const bool own = st < nk;
          if (d < IA + IB) {
            code1(own ? st : ahead ? st - nk : nk - 1, slot, d, own || !ahead ? 0 : dm, own || !ahead ? 0 : dn);
          } else {
            const int gi = it / 4 + 2;
            const int gs = (gb + gi) % NG;
            const bool gown = gi < ng;
            // (past the end, the next tile's groups 0-1, never past its last)
            scale1(gown ? gi : ahead ? min(gi - ng, ng - 1) : ng - 1, (it & 2) * 2 + wave, gs,
                   gown || !ahead ? 0 : dm, gown || !ahead ? 0 : dn);
          }
        }
        // next stage's reads, the earliest needed first: B codes and scales
        // (row 0), A scales, A codes (A block i is first used in row i)
        if (i >= 4) read1(nxt, next, gr, (it + 1) & 3, i == 4 ? 8 + j : i == 5 ? 24 + j : i == 6 ? 16 + j : j);
        // in the last row, the next stage's scale words (read in rows 5-6)
        // get the lane's byte (K block grp) shifted to byte 0, long before
        // an MFMA reads them (pinned: left to itself the compiler sinks the
        // shift into the next stage, right before that MFMA)
        if (i == TM - 1) {
          nxt.sa[j] >>= 8 * grp;
          nxt.sb[j] >>= 8 * grp;
          asm volatile("" : "+v"(nxt.sa[j]), "+v"(nxt.sb[j]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    slot = next;
  };

  for (;;) {
    if (!have0) {
      // stage 0 and scale group 0 have landed: after a store its 64 writes
      // follow the prologue's loads, else the loads of stages 1-3 do
      if (stored) wait_vm_barrier<63>();
      else wait_vm_barrier<NIW2 + IA + IB>();
#pragma unroll
      for (int k = 0; k < 32; ++k) read1(F, slot, gb, 0, k);
      // shifted here, not sunk next to the MFMA that reads them
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        F.sa[i] >>= 8 * grp;
        F.sb[i] >>= 8 * grp;
        asm volatile("" : "+v"(F.sa[i]), "+v"(F.sb[i]));
      }
    }
    mfma_guard();
    // two stages per loop iteration with the fragment sets swapped, so no
    // registers are copied between stages (the loop holds a barrier, which
    // keeps the compiler from unrolling it); nk is a multiple of 4, so the
    // next tile's stage 0 ends up in F. The odd last stage that follows
    // never runs, but without it the register allocator moves accumulators
    // between the loop and the tile's end (AGPR moves next to the asm
    // MFMAs, a hazard the compiler does not see).
    int it = 0;
    for (; it + 1 < nk; it += 2) {
      stage(it, F, N);
      stage(it + 1, N, F);
    }
    if (it < nk) stage(it, F, N);
    mfma_guard();                                        // before any accumulator read

    // the tile is complete: with `ahead` the next tile's first stages are
    // in the rings and its stage 0 in F; otherwise the rings are filled
    // afresh once every load has landed and every wave is done with them.
    // Then this tile's store is issued.
    const int64_t cm0 = m0, cn0 = n0;
    const bool streamed = ahead;
    tile += P;
    const bool last = tile >= tiles;
    if (!last) {
      int tm, tn;
      tile_coords(tile, g.tiles_m, g.tiles_n, tm, tn);
      m0 = (int64_t)tm * 256;
      n0 = (int64_t)tn * 256;
      sources();
      if (streamed) {
        gb = (gb + ng) % NG;
      } else {
        wait_vm_barrier<0>();
        slot = 0;
        gb = 0;
        prologue();
      }
      have0 = streamed;
      plan_ahead();
    } else {
      wait_vm_barrier<0>();                              // the reloads have landed before the workgroup ends
    }
    stored = store_tile_rows<TM, TN>(g, acc, cm0 + wm * 128, cn0 + wn * 128, r16, grp, e);
    if (!stored) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the checked form may write less
    if (last) break;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
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

// Split-K reduction that also quantizes C row-wise (QOut): a thread sums
// and quantizes one 16-element row block at a time (N % 16 == 0), with the
// row-wise quantizer's block codecs; one statistics partial per workgroup.
template <int OF, bool SR>
__global__ __launch_bounds__(256) void splitk_reduce_q_kernel(GemmArgs g, int nsplit) {
  __shared__ double dred[8];
  __shared__ uint32_t ured[8];
  __shared__ float inv_lut[OF == SNIP_NVFP4 ? 128 : 1];
  if constexpr (OF == SNIP_NVFP4) fill_inv_lut(inv_lut);
  const QOut& q = g.q;
  const int e = (g.ea ? *g.ea : 0) + (g.eb ? *g.eb : 0);
  const int eS = tensor_exp(*q.amax_in, OF);
  if (blockIdx.x == 0 && threadIdx.x == 0) *q.texp = eS;
  const int64_t total = g.M * g.N;
  const int64_t nblk = total / 16;
  double e2s = 0.0, x2s = 0.0, x2r = 0.0;
  uint32_t nf = 0u, amax_bits = 0u;
  for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < nblk; b += (int64_t)gridDim.x * 256) {
    const int64_t i0 = b * 16;
    const int64_t row = i0 / g.N, col = i0 - row * g.N;
    float x[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float s = 0.0f;
      for (int k = 0; k < nsplit; ++k) s += g.partial[k * total + i0 + t];
      x[t] = ldexpf(s, e);
      g.c[row * g.ldc + col + t] = x[t];
    }
    Words4 d0, d1;
    if (SR) {
      d0 = draws8(q.seed, q.tensor_id, (uint64_t)i0 >> 3);
      d1 = draws8(q.seed, q.tensor_id, ((uint64_t)i0 >> 3) + 1);
    }
    float be2, bx2;
    if constexpr (OF == SNIP_NVFP4) {
      uint32_t lo, hi, sc;
      nvfp4_block<SR>(x, eS, d0, d1, inv_lut, lo, hi, sc, be2, bx2);
      *reinterpret_cast<uint2*>(q.codes + i0 / 2) = make_uint2(lo, hi);
      q.scales[i0 / 16] = (uint8_t)sc;
    } else {
      uint32_t out[4];
      fp8_chunk<SR>(x, eS, d0, d1, out, be2, bx2);
      *reinterpret_cast<uint4*>(q.codes + i0) = make_uint4(out[0], out[1], out[2], out[3]);
    }
    const bool bad = !(bx2 <= 3.0e38f);
    uint32_t bnf = 0u, bam = 0u;
    double rx2 = 0.0;
    if (bad) nonfinite_stats<16>(x, bnf, rx2, bam);
    else bam = block_absmax_bits<16>(x);
    amax_bits = max(amax_bits, bam);
    nf += bnf;
    x2r += rx2;
    e2s += bad ? 0.0 : (double)be2;
    x2s += bad ? 0.0 : (double)bx2;
  }
  wg_store_stats(q.part + blockIdx.x, ldexp(e2s, 2 * eS), ldexp(x2s, 2 * eS) + x2r, nf, amax_bits, dred, ured);
}

// Host-side plan: kernel, tile shape and K split for a problem.
//
// A CU holds one 256x256 workgroup or two smaller ones (128x128, or 256x128
// for FP8 and NVFP4), so a launch runs in rounds of 256 big or 512 smaller
// tiles. Per
// unit of tile area the bigger tiles run faster by measured factors (less
// decode and operand traffic per MFMA; for MX-FP4 and BF16 the 128x128
// tiles run on the register-staged kernel, gemm_staged.hip, which nearly
// matches). A last, partial round of two-per-CU tiles costs a full round
// when more than 256 tiles remain and about 0.6 of one otherwise (one per
// CU, running faster alone). The plan takes the cheapest shape, in units of
// one round of 128x128 tiles; problems with fewer than 192 small tiles split
// K so that about 256 workgroups run.
// NVFP4 256x256 tiles (gemm_nvfp4_w1_kernel, one per CU) run their K loop
// about 10 % faster than the 256x128 tiles but pay more per tile at its
// ends (pipeline fill and the store of a 256 KiB tile). Measured on MI355X
// with one tile per workgroup: faster by 3-9 % for K >= 8192
// (4096x8192x28672 1.486 -> 1.359 ms), mixed at K = 4096 and slower below
// (4096x8192x1024 0.069 -> 0.087 ms). Persistent, with each tile's store
// overlapping the next tile: also 1-3 % faster than 256x128 tiles at
// K = 4096 (28672x8192x4096 1.546 -> 1.527 ms; the Llama-70B block step
// 18.73 -> 18.51 ms), so planned for K >= 4096 at first. With the later
// refinements of its loop it also wins at K = 2048-3072 (measured on
// MI355X, outputs bit-identical: 8192x4096x2048 0.117 -> 0.114 ms,
// 8192x4096x3072 0.169 -> 0.158 ms) but not at K = 1024 (4096x8192x1024
// 0.070 -> 0.075 ms): planned for K >= 2048, in pairs of 128-element
// stages (the kernel loads each row's scales of two stages at once).
// MX-FP4 256x256 tiles with K % 512 == 0 run persistent
// (gemm_mxfp4_w1p_kernel): priced at 1.25 instead of 1.03, they take
// shapes the register-staged 128x128 kernel had (measured on MI355X:
// 4096x11008x16384 0.562 -> 0.387 ms, 4096x11008x4096 0.154 -> 0.127 ms,
// 11008x4096x8192 0.277 -> 0.212 ms; no shape slower). At 1.6 some shapes
// gained and others lost (4096x5632x2048 0.049 -> 0.053 ms).
static double big_tile_gain(int format, int64_t K) {
  switch (format) {
    case SNIP_FP8_E4M3: return 1.15;
    case SNIP_MXFP4: return K % 512 == 0 ? 1.25 : 1.03;
    case SNIP_NVFP4: return K >= 2048 && K % 256 == 0 ? 1.18 : 0.0;
    default: return 1.02;
  }
}
// 256x128 over 128x128: FP8 (3-stage ring, 72 KiB) and NVFP4 (2-stage
// ring, 54 KiB; a wave's 128x64 sub-tile needs 3 decode instructions per
// MFMA instead of 4), both two workgroups per CU
static double rect_gain(int format) {
  return format == SNIP_FP8_E4M3 ? 1.17 : format == SNIP_NVFP4 ? 1.12 : 0.0;
}

static double rounds2(int64_t tiles) {    // two tiles per CU
  const int64_t rem = tiles % 512;
  return (double)(tiles / 512) + (rem == 0 ? 0.0 : rem <= 256 ? 0.6 : 1.0);
}

// Estimated time of an unsplit problem on each tile shape, in rounds of
// 128x128 tiles (two per CU) of the same K.
struct TileTimes {
  int64_t t128, t256, trect;
  double time128, time256, timerect;
};
static TileTimes tile_times(int format, int64_t M, int64_t N, int64_t K) {
  TileTimes t;
  t.t256 = ceil_div(M, 256) * ceil_div(N, 256);
  t.t128 = ceil_div(M, 128) * ceil_div(N, 128);
  t.trect = ceil_div(M, 256) * ceil_div(N, 128);
  t.time128 = rounds2(t.t128);
  const double g256 = big_tile_gain(format, K);
  t.time256 = g256 > 0.0 ? (double)ceil_div(t.t256, 256) * 2.0 / g256 : 1e30;
  t.timerect = rect_gain(format) > 0.0 ? rounds2(t.trect) * 2.0 / rect_gain(format) : 1e30;
  // FP8 256x128 tiles whose last round is less than half full leave CUs idle
  // that the 128x128 tiles, three per CU, fill. Measured on MI355X for
  // 4096x5632x2048 (704 such tiles, a last round of 192): the tinyllama1b
  // step's FP8 GEMMs 0.604 -> 0.595 ms on 128x128 tiles; the llama7b FP8
  // shapes (whole rounds of 256x128 tiles) keep them.
  if (format == SNIP_FP8_E4M3 && t.trect % 512 != 0 && t.trect % 512 < 256) t.timerect = 1e30;
  return t;
}

GemmPlan plan_gemm(int format, int64_t M, int64_t N, int64_t K) {
  GemmPlan p;
  const TileTimes tt = tile_times(format, M, N, K);
  const int64_t t256 = tt.t256, t128 = tt.t128, trect = tt.trect;
  const double time128 = tt.time128, time256 = tt.time256, timerect = tt.timerect;
  p.staged = 0;
  p.ksplit = 1;
  p.kchunk = K;
  p.bk = unit_k(format);
  if (t128 >= 192 && (time256 < time128 || timerect < time128)) {
    p.bm = 256;
    p.bn = time256 <= timerect ? 256 : 128;
    p.tiles = p.bn == 256 ? t256 : trect;
    return p;
  }
  p.bm = p.bn = 128;
  p.tiles = t128;
  p.staged = (format == SNIP_MXFP4 || format == SNIP_BF16) ? 1 : 0;
  int64_t split = p.tiles >= 192 ? 1 : 256 / p.tiles;
  if (t128 < 192 && (format == SNIP_FP8_E4M3 || format == SNIP_NVFP4)) {
    // skinny problems: 64x64 tiles, unsplit when they fill the chip, else
    // split K over about 512 workgroups (measured on the K/V projections:
    // 4096x256x2048 22 -> 14 us, 256x2048x4096 16 -> 13 us)
    p.bm = p.bn = 64;
    p.tiles = ceil_div(M, 64) * ceil_div(N, 64);
    split = p.tiles >= 192 ? 1 : ceil_div(512, p.tiles);
  }
  // split in whole stages (the staged MX kernel then runs 128-element
  // stages), at least 4 per split
  const int64_t gran = p.staged ? (format == SNIP_MXFP4 ? 128 : 64) : unit_k(format);
  const int64_t max_split = K / (4 * gran);
  if (split > max_split) split = max_split;
  if (split < 1) split = 1;
  const int64_t chunk = ceil_div(ceil_div(K, split), gran) * gran;
  p.kchunk = chunk;
  p.ksplit = (int)ceil_div(K, chunk);
  p.bk = p.ksplit > 1 ? (int)gran : p.staged ? staged_stage_k(format, K) : unit_k(format);
  return p;
}

size_t gemm_partial_bytes(int format, int64_t M, int64_t N, int64_t K) {
  const GemmPlan p = plan_gemm(format, M, N, K);
  return p.ksplit > 1 ? (size_t)p.ksplit * (size_t)(M * N) * sizeof(float) : 0;
}

// Returns false when the plan names a kernel this format has no instance of.
template <int FMT, bool QO = false>
static bool launch_fmt(const GemmPlan& p, const GemmArgs& g, hipStream_t s) {
  const dim3 grid((unsigned)(p.tiles + g.fin.n), (unsigned)p.ksplit);
  if constexpr (FMT == SNIP_FP8_E4M3) {
    if (p.bm == 256 && p.bn == 128) {     // 3-stage ring: 72 KiB, two per CU
      hipLaunchKernelGGL((gemm_kernel<FMT, 256, 128, 3, 1, QO>), grid, dim3(NT), 0, s, g);
      return true;
    }
  }
  if constexpr (FMT == SNIP_NVFP4) {
    if (p.bm == 256 && p.bn == 128) {     // 2-stage ring: 54 KiB, two per CU
      hipLaunchKernelGGL((gemm_kernel<FMT, 256, 128, 2, 1, QO>), grid, dim3(NT), 0, s, g);
      return true;
    }
  }
  if constexpr (FMT == SNIP_FP8_E4M3 || FMT == SNIP_NVFP4) {
    if (p.bm == 64) {
      // skinny problems: a 4-stage ring of two units per stage where K and
      // the K split are whole such stages (4096x256x2048 FP8 13.6 -> 11.4 us,
      // NVFP4 12.7 -> 11.7 us), else of single units
      constexpr int K2 = 2 * Unit<FMT>::UE;
      if (g.K % K2 == 0 && g.kchunk % K2 == 0)
        hipLaunchKernelGGL((gemm_kernel<FMT, 64, 64, 4, 2, QO>), grid, dim3(NT), 0, s, g);
      else
        hipLaunchKernelGGL((gemm_kernel<FMT, 64, 64, 4, 1, QO>), grid, dim3(NT), 0, s, g);
      return true;
    }
  }
  if (p.bm == 256) {
    if constexpr (FMT == SNIP_NVFP4) {
      // one workgroup per CU, each running its tiles in turn; with QO one
      // per tile (its epilogue uses the operand ring)
      if (p.ksplit != 1 || g.nsec || g.K % 256) return false;
      const int64_t wgs = QO ? p.tiles : std::min<int64_t>(p.tiles, device_cus());
      hipLaunchKernelGGL((gemm_nvfp4_w1_kernel<QO>), dim3((unsigned)(wgs + g.fin.n)), dim3(NT), 0, s, g);
    } else if constexpr (FMT == SNIP_MXFP4 && !QO) {
      // K % 512 == 0: one workgroup per CU, each running its tiles in turn
      if (g.K % 512 == 0 && p.ksplit == 1 && !g.nsec) {
        const dim3 pgrid((unsigned)(std::min<int64_t>(p.tiles, device_cus()) + g.fin.n));
        hipLaunchKernelGGL(gemm_mxfp4_w1p_kernel, pgrid, dim3(NT), 0, s, g);
      } else {
        hipLaunchKernelGGL(gemm_mxfp4_w1_kernel, grid, dim3(NT), 0, s, g);
      }
    }
    else hipLaunchKernelGGL((gemm_kernel<FMT, 256, 256, 4, 1, QO>), grid, dim3(NT), 0, s, g);
  } else if (p.staged) {
    if constexpr (QO) return false;
    else launch_staged(FMT, p.bk, g, grid, s);
  }
  else if constexpr (FMT == SNIP_FP8_E4M3) {
    // FP8 128x128: a 3-stage ring (48 KiB) lets a third workgroup share the
    // CU where registers allow (measured up to 7 % faster). With at most one
    // tile per CU (no third workgroup to gain) two 64-element units per
    // stage halve the barriers per K: 2048x2048x4096 45.0 -> 41.6 us.
    if (p.ksplit == 1 && p.tiles <= 256 && g.K % (2 * Unit<FMT>::UE) == 0)
      hipLaunchKernelGGL((gemm_kernel<FMT, 128, 128, 2, 2, QO>), grid, dim3(NT), 0, s, g);
    else
      hipLaunchKernelGGL((gemm_kernel<FMT, 128, 128, 3, 1, QO>), grid, dim3(NT), 0, s, g);
  } else if constexpr (FMT == SNIP_NVFP4) {
    // NVFP4 128x128: a 2-stage ring of single units (36 KiB), three
    // workgroups per CU
    hipLaunchKernelGGL((gemm_kernel<FMT, 128, 128, 2, 1, QO>), grid, dim3(NT), 0, s, g);
  } else {
    hipLaunchKernelGGL((gemm_kernel<FMT, 128, 128, 4, 1, QO>), grid, dim3(NT), 0, s, g);
  }
  return true;
}

// Whether two GEMMs of one format share a launch: both FP8 or NVFP4, both
// unsplit on tiles of 128 rows or more in their own plans, and the grouped
// launch on 128x128 tiles (both problems' tiles balanced over two
// workgroups per CU) estimated cheaper than the two planned launches, each
// problem's time weighted by its K. Measured: the TinyLlama-1B pairs group
// (1.716 -> 1.628 ms per step); the Llama-7B Gate/Down pairs, whose own plans
// take 256x128 tiles in full rounds, do not (grouped 1326 vs 1265 us).
static bool pair_grouped(int format, const GemmArgs& g1, const GemmArgs& g2) {
  if (format != SNIP_FP8_E4M3 && format != SNIP_NVFP4) return false;
  const GemmPlan p1 = plan_gemm(format, g1.M, g1.N, g1.K), p2 = plan_gemm(format, g2.M, g2.N, g2.K);
  if (!(p1.ksplit == 1 && p2.ksplit == 1 && p1.bm >= 128 && p2.bm >= 128)) return false;
  const TileTimes a = tile_times(format, g1.M, g1.N, g1.K), b = tile_times(format, g2.M, g2.N, g2.K);
  auto planned = [](const TileTimes& t) { return std::min(t.time128, std::min(t.time256, t.timerect)); };
  const double separate = planned(a) * (double)g1.K + planned(b) * (double)g2.K;
  const double grouped = ((double)a.t128 * (double)g1.K + (double)b.t128 * (double)g2.K) / 512.0;
  return grouped < separate;
}

hipError_t launch_gemm_pair(int format, const GemmArgs& g1_in, const GemmArgs& g2_in, hipStream_t s) {
  // every kernel runs whole K units (the ABI requires K % 128 == 0)
  if (g1_in.K % unit_k(format) || g2_in.K % unit_k(format)) return hipErrorInvalidValue;
  if (!pair_grouped(format, g1_in, g2_in)) {
    hipError_t e = launch_gemm(format, g1_in, s);
    return e != hipSuccess ? e : launch_gemm(format, g2_in, s);
  }
  // the problem with the longer K (longer tiles) is dispatched first
  const bool swap = g2_in.K > g1_in.K;
  GemmArgs g = swap ? g2_in : g1_in;
  const GemmArgs& h = swap ? g1_in : g2_in;
  g.fin = g2_in.fin;
  g.tiles_m = (int)ceil_div(g.M, 128);
  g.tiles_n = (int)ceil_div(g.N, 128);
  g.kchunk = g.K;
  g.nsec = 1;
  g.sec = GemmArgs::Second{h.a, h.b, h.as, h.bs, h.ea, h.eb, h.c, h.M, h.N, h.K, h.ldc,
                           (int32_t)ceil_div(h.M, 128), (int32_t)ceil_div(h.N, 128)};
  const int64_t tiles = (int64_t)g.tiles_m * g.tiles_n + (int64_t)g.sec.tiles_m * g.sec.tiles_n;
  const dim3 grid((unsigned)(tiles + g.fin.n), 1);
  const double flops = 2.0 * g.M * g.N * g.K + 2.0 * h.M * h.N * h.K;
  const int slot = timing_begin(LaunchTag{SNIP_LAUNCH_GEMM, format, -1, -1, flops}, s);
  if (format == SNIP_FP8_E4M3) {
    hipLaunchKernelGGL((gemm_kernel<SNIP_FP8_E4M3, 128, 128, 3, 1>), grid, dim3(NT), 0, s, g);
  } else {
    hipLaunchKernelGGL((gemm_kernel<SNIP_NVFP4, 128, 128, 2, 1>), grid, dim3(NT), 0, s, g);
  }
  const hipError_t e = hipGetLastError();
  timing_end(slot, s);
  return e;
}

hipError_t launch_gemm(int format, const GemmArgs& g_in, hipStream_t s) {
  if (format < SNIP_BF16 || format > SNIP_MXFP4) return hipErrorInvalidValue;
  if (g_in.K % unit_k(format)) return hipErrorInvalidValue;   // whole K units only
  GemmPlan p = plan_gemm(format, g_in.M, g_in.N, g_in.K);
  GemmArgs g = g_in;
  if (p.ksplit > 1 && g.partial == nullptr) {      // no scratch: run unsplit
    p.ksplit = 1;
    p.kchunk = g.K;
    if (p.staged) p.bk = staged_stage_k(format, g.K);
  }
  g.tiles_m = (int)ceil_div(g.M, p.bm);
  g.tiles_n = (int)ceil_div(g.N, p.bn);
  g.kchunk = p.kchunk;
  // output quantization: in the GEMM's epilogue when unsplit, else in the
  // split-K reduction (FP8 and NVFP4 operands; NVFP4 or FP8 output)
  const bool qo = g.q.codes != nullptr;
  if (qo && ((format != SNIP_NVFP4 && format != SNIP_FP8_E4M3) ||
             (g.q.fmt != SNIP_NVFP4 && g.q.fmt != SNIP_FP8_E4M3) || g.N % 16))
    return hipErrorInvalidValue;
  int slot = timing_begin(LaunchTag{SNIP_LAUNCH_GEMM, format, -1, -1, 2.0 * g.M * g.N * g.K}, s);
  bool launched;
  const bool qo_here = qo && p.ksplit == 1;
  switch (format) {
    case SNIP_NVFP4:
      launched = qo_here ? launch_fmt<SNIP_NVFP4, true>(p, g, s) : launch_fmt<SNIP_NVFP4>(p, g, s);
      break;
    case SNIP_FP8_E4M3:
      launched = qo_here ? launch_fmt<SNIP_FP8_E4M3, true>(p, g, s) : launch_fmt<SNIP_FP8_E4M3>(p, g, s);
      break;
    case SNIP_MXFP4: launched = launch_fmt<SNIP_MXFP4>(p, g, s); break;
    default: launched = launch_fmt<SNIP_BF16>(p, g, s); break;
  }
  hipError_t e = launched ? hipGetLastError() : hipErrorInvalidValue;
  timing_end(slot, s);
  if (e != hipSuccess || p.ksplit == 1) return e;
  slot = timing_begin(LaunchTag{SNIP_LAUNCH_SPLITK, format, -1, -1, (double)(g.M * g.N)}, s);
  if (qo) {
    const dim3 grid((unsigned)gemm_qout_parts(format, g.M, g.N, g.K));
    if (g.q.fmt == SNIP_NVFP4) {
      if (g.q.sr) hipLaunchKernelGGL((splitk_reduce_q_kernel<SNIP_NVFP4, true>), grid, dim3(256), 0, s, g, p.ksplit);
      else hipLaunchKernelGGL((splitk_reduce_q_kernel<SNIP_NVFP4, false>), grid, dim3(256), 0, s, g, p.ksplit);
    } else {
      if (g.q.sr) hipLaunchKernelGGL((splitk_reduce_q_kernel<SNIP_FP8_E4M3, true>), grid, dim3(256), 0, s, g, p.ksplit);
      else hipLaunchKernelGGL((splitk_reduce_q_kernel<SNIP_FP8_E4M3, false>), grid, dim3(256), 0, s, g, p.ksplit);
    }
  } else {
    int64_t wg = ceil_div(g.M * g.N, 256);
    if (wg > 4096) wg = 4096;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)wg), dim3(256), 0, s, g, p.ksplit);
  }
  e = hipGetLastError();
  timing_end(slot, s);
  return e;
}

int64_t gemm_qout_parts(int format, int64_t M, int64_t N, int64_t K) {
  const GemmPlan p = plan_gemm(format, M, N, K);
  if (p.ksplit == 1) return p.tiles;
  const int64_t wg = ceil_div(M * N / 16, 256);
  return wg < 1 ? 1 : wg > kQuantWG ? kQuantWG : wg;
}

}  // namespace snip

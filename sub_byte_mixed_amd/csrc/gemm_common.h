// Pieces shared by the two GEMM kernel families (gemm.hip: LDS-DMA staged
// kernel; gemm_staged.hip: register-staged kernel): vector types, the tile
// order and the epilogue.
#pragma once

#include "device.h"
#include "kernels.h"
#include "quant_common.h"
#include "stats_common.h"

namespace snip {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef int intx8_t __attribute__((ext_vector_type(8)));

// Tile id -> (tile row, tile column). The hardware hands workgroups to the 8
// XCDs round-robin; ids are remapped so each XCD works on a contiguous range,
// and tiles are ordered in groups of 4 tile-rows so that concurrently
// running tiles share A and B panels in that XCD's L2. Group heights
// measured on MI355X (paired runs): 4 beats 8 by 0.3 % on the tinyllama1b
// step and 0.8 % on llama7b; 1, 2 and 16 are slower than 4.
__device__ __forceinline__ void tile_coords(int id, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  if ((total & 7) == 0) id = (id & 7) * (total >> 3) + (id >> 3);
  constexpr int GM = 4;
  const int group = id / (GM * tiles_n);
  const int first = group * GM;
  const int gm = (tiles_m - first) < GM ? (tiles_m - first) : GM;
  const int r = id - group * GM * tiles_n;
  tm = first + r % gm;
  tn = r / gm;
}

// Workgroups past the last tile finalise the statistics jobs the launch
// carries (one job each, on the first K split); the kernel boundary orders
// them after the quantize launches that wrote the partials. Returns true
// for such a workgroup, which then does nothing else.
__device__ __forceinline__ bool finalize_workgroup(const GemmArgs& g) {
  const int tiles = g.tiles_m * g.tiles_n + (g.nsec ? g.sec.tiles_m * g.sec.tiles_n : 0);
  if ((int)blockIdx.x < tiles) return false;
  if (blockIdx.y == 0) finalize_one(g.fin.j[blockIdx.x - tiles]);
  return true;
}

// Epilogue of a 2x2-wave tile: the wave's accumulators (lane holds rows
// 4*grp + v, column r16 of each 16x16 block) go to C scaled by 2^(ea+eb),
// or, under split-K, unscaled to this split's fp32 partial.
template <int TM, int TN>
__device__ __forceinline__ void store_tile(const GemmArgs& g, const floatx4_t (&acc)[TM][TN], int64_t r0,
                                           int64_t c0, int r16, int grp) {
  const bool whole = g.kchunk >= g.K;
  float* const base = whole ? g.c : g.partial + (int64_t)blockIdx.y * g.M * g.N;
  const int64_t ld = whole ? g.ldc : g.N;
  // A wave's sub-tile lying wholly inside C (every tile but the ragged last
  // row and column of tiles) is stored without per-element checks: r0 and c0
  // are wave-uniform, so each of the TM*16 rows starts at a scalar address
  // and a lane adds one 32-bit byte offset (its row within the 4-row group
  // and its column), with the 16-column blocks j as immediate offsets. The
  // 128x128 wave tiles keep the checked form: with their 256 accumulators
  // the extra code path adds register spills.
  if (TM * TN <= 32 && r0 + 16 * TM <= g.M && c0 + 16 * TN <= g.N && ld <= (int64_t(1) << 26)) {
    const uint32_t loff = (uint32_t)((4 * grp * ld + r16) * 4);
    if (whole) {
      const int e = (g.ea ? *g.ea : 0) + (g.eb ? *g.eb : 0);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          char* const rowp = reinterpret_cast<char*>(base + (r0 + i * 16 + v) * ld + c0) + loff;
#pragma unroll
          for (int j = 0; j < TN; ++j) *reinterpret_cast<float*>(rowp + j * 64) = ldexpf(acc[i][j][v], e);
        }
    } else {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          char* const rowp = reinterpret_cast<char*>(base + (r0 + i * 16 + v) * ld + c0) + loff;
#pragma unroll
          for (int j = 0; j < TN; ++j) *reinterpret_cast<float*>(rowp + j * 64) = acc[i][j][v];
        }
    }
    return;
  }
  if (whole) {
    const int e = (g.ea ? *g.ea : 0) + (g.eb ? *g.eb : 0);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t col = c0 + j * 16 + r16;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t row = r0 + i * 16 + 4 * grp + v;
          if (row < g.M && col < g.N) base[row * ld + col] = ldexpf(acc[i][j][v], e);
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t col = c0 + j * 16 + r16;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t row = r0 + i * 16 + 4 * grp + v;
          if (row < g.M && col < g.N) base[row * ld + col] = acc[i][j][v];
        }
      }
  }
}

// ---------------------------------------------------------------- output quantization
// Epilogue that also quantizes C row-wise (blocks of 16 along N; N % 16 ==
// 0, so a block lies wholly inside or outside C). The operand ring in LDS
// is idle once the K loop ends: each wave moves one 16-row slice of its
// accumulators at a time into its own part of it (as C's values
// y = acc * 2^(ea+eb)), and every lane then takes whole 16-element row
// blocks of the slice: it writes the block to C (64 contiguous bytes) and
// quantizes it with the row-wise quantizer's block codec (nvfp4_block /
// fp8_chunk: the same arithmetic, element index row * N + col for the
// stochastic draws). Statistics go to one partial per workgroup.
template <int TM, int TN>
__device__ __forceinline__ void store_tile_q(const GemmArgs& g, const floatx4_t (&acc)[TM][TN], int64_t r0,
                                             int64_t c0, int r16, int grp, uint8_t* lds) {
  __shared__ double dred[8];
  __shared__ uint32_t ured[8];
  __shared__ float inv_lut[128];
  constexpr int PITCH = TN * 16 + 4;                         // floats per staged row
  const QOut& q = g.q;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = (g.ea ? *g.ea : 0) + (g.eb ? *g.eb : 0);
  const int eS = tensor_exp(*q.amax_in, q.fmt);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *q.texp = eS;
  __syncthreads();                                           // every wave is done with the ring
  fill_inv_lut(inv_lut);                                     // (ends with a barrier)
  float* const st = reinterpret_cast<float*>(lds) + wave * 16 * PITCH;
  double e2s = 0.0, x2s = 0.0, x2r = 0.0;
  uint32_t nf = 0u, amax_bits = 0u;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) st[(4 * grp + v) * PITCH + j * 16 + r16] = ldexpf(acc[i][j][v], e);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int b = lane; b < 16 * TN; b += 64) {
      const int rr = b / TN, jb = b % TN;
      const int64_t row = r0 + i * 16 + rr, col = c0 + jb * 16;
      if (row >= g.M || col >= g.N) continue;
      float x[16];
      const float4* src = reinterpret_cast<const float4*>(st + rr * PITCH + jb * 16);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float4 f = src[t];
        x[4 * t] = f.x;
        x[4 * t + 1] = f.y;
        x[4 * t + 2] = f.z;
        x[4 * t + 3] = f.w;
      }
      float4* dst = reinterpret_cast<float4*>(g.c + row * g.ldc + col);
#pragma unroll
      for (int t = 0; t < 4; ++t) dst[t] = make_float4(x[4 * t], x[4 * t + 1], x[4 * t + 2], x[4 * t + 3]);
      const uint64_t i0 = (uint64_t)(row * g.N + col);
      Words4 d0, d1;
      if (q.sr) {
        d0 = draws8(q.seed, q.tensor_id, i0 >> 3);
        d1 = draws8(q.seed, q.tensor_id, (i0 >> 3) + 1);
      }
      float be2, bx2;
      if (q.fmt == SNIP_NVFP4) {
        uint32_t lo, hi, sc;
        if (q.sr) nvfp4_block<true>(x, eS, d0, d1, inv_lut, lo, hi, sc, be2, bx2);
        else nvfp4_block<false>(x, eS, d0, d1, inv_lut, lo, hi, sc, be2, bx2);
        *reinterpret_cast<uint2*>(q.codes + i0 / 2) = make_uint2(lo, hi);
        q.scales[i0 / 16] = (uint8_t)sc;
      } else {
        uint32_t out[4];
        if (q.sr) fp8_chunk<true>(x, eS, d0, d1, out, be2, bx2);
        else fp8_chunk<false>(x, eS, d0, d1, out, be2, bx2);
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
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  wg_store_stats(q.part + blockIdx.x, ldexp(e2s, 2 * eS), ldexp(x2s, 2 * eS) + x2r, nf, amax_bits, dred, ured);
}

// Register-staged 128x128 kernel (MX-FP4 and BF16): K per stage and launch.
int staged_stage_k(int format, int64_t K);
void launch_staged(int format, int bk, const GemmArgs& g, dim3 grid, hipStream_t s);

}  // namespace snip

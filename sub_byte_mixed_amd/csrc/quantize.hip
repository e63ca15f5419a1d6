// Quantizer kernels for gfx950: amax pre-pass, row-wise and column-wise
// NVFP4 / FP8-E4M3 / MX-FP4 quantization with round-to-nearest-even or
// Philox stochastic rounding, fused per-tensor statistics, bf16 copy /
// transpose for the unquantized baseline, and statistics finalisation.
//
// "FP4 All the Way" summary, Outline: 16 E2M1 values share an E4M3 scale;
// nearest rounding forward, stochastic rounding backward and in the update.
// "SNIP", Abstract: activation and gradient statistics feed the precision
// decision -- every quantize pass accumulates sum (Q(x)-x)^2, sum x^2 and
// counts non-finite inputs, next to the tensor max.
//
// Work layout. Row-wise: one thread per 16-element block (32 for MX, 16
// elements per thread for FP8); consecutive threads own consecutive blocks,
// so the packed code stores of a wave are contiguous. Column-wise: a
// workgroup owns a 256-row x 128-column source tile; each lane reads two
// adjacent columns with dword loads (a wave covers 256 contiguous bytes of a
// source row), quantizes 16-row (32 for MX) blocks down the columns, stages
// the codes in LDS and writes each output row segment (128 bytes of codes)
// with 8-byte stores. All kernels are HBM-bound scans.
#include "quant_common.h"
#include "stats_common.h"

namespace snip {

// Largest finite |x| of a packed pair of bf16 (as magnitude bits).
__device__ __forceinline__ uint32_t pair_max(uint32_t w, uint32_t m) {
  uint32_t lo = w & 0x7FFFu, hi = (w >> 16) & 0x7FFFu;
  lo = lo >= 0x7F80u ? 0u : lo;
  hi = hi >= 0x7F80u ? 0u : hi;
  m = lo > m ? lo : m;
  return hi > m ? hi : m;
}

// ------------------------------------------------------------ amax pass
// The tensor is streamed once and not needed again soon in the cache (the
// quantize pass that follows reads it after the whole pre-pass has run), so
// the loads are non-temporal. Measured on MI355X on the llama70b block's
// tensors: 3.6 -> 5.8 TB/s (0.83 -> 0.52 ms per step).
__global__ __launch_bounds__(kAmaxThreads) void amax_kernel(AJobs jobs) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  int32_t wg0[kMaxJobs];
  for (int i = 0; i < kMaxJobs; ++i) wg0[i] = jobs.j[i].wg0;
  const int jn = find_job(wg0, jobs.n);
  const AJob J = jobs.j[jn];
  const int wg = blockIdx.x - J.wg0;
  const int64_t cpr = J.cols >> 3;                    // 8-element chunks per row
  const int64_t nchunk = J.rows * cpr;
  const bool flat = J.ld == J.cols;
  uint32_t m = 0;
  // kAmaxUnroll independent 16-byte loads per thread in flight
  for (int64_t c0 = (int64_t)wg * kAmaxThreads * kAmaxUnroll + threadIdx.x; c0 < nchunk;
       c0 += (int64_t)J.nwg * kAmaxThreads * kAmaxUnroll) {
    uint4 v[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      const int64_t c = c0 + u * kAmaxThreads;
      const int64_t off = flat ? c * 8 : (c / cpr) * J.ld + (c % cpr) * 8;
      const u32x4 t = c < nchunk ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(J.x + off))
                                 : u32x4{0u, 0u, 0u, 0u};
      v[u] = make_uint4(t.x, t.y, t.z, t.w);
    }
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      m = pair_max(v[u].x, m);
      m = pair_max(v[u].y, m);
      m = pair_max(v[u].z, m);
      m = pair_max(v[u].w, m);
    }
  }
  m = wave_max_u(m);
  constexpr int NW = kAmaxThreads / 64;
  __shared__ uint32_t red[NW];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
    for (int w = 1; w < NW; ++w) r = red[w] > r ? red[w] : r;
    J.part[wg] = r;
  }
}

// ------------------------------------------------------------ row-wise
// One thread item = one 16-element NVFP4 block, 16 FP8 elements, or one
// 32-element MX block; item `it` covers output elements it*EPT .. +EPT. Each
// thread handles two items per iteration (both loads issued first).
template <int FMT, bool SR>
struct RowAcc {
  double e2s = 0.0, x2s = 0.0;      // tensor-scaled domain (NVFP4, FP8)
  double e2r = 0.0, x2r = 0.0;      // raw domain (MX, non-finite blocks)
  uint32_t nf = 0u, amax_bits = 0u;
  uint32_t tmax = 0u;               // max |x| seen (reported under a supplied max)
};

template <int FMT, bool SR>
__device__ __forceinline__ void row_item(const QJob& J, int eS, const float* inv_lut, int64_t it,
                                         const uint4 (&v)[FMT == SNIP_MXFP4 ? 4 : 2],
                                         RowAcc<FMT, SR>& acc) {
  constexpr int EPT = (FMT == SNIP_MXFP4) ? 32 : 16;
  const uint64_t g0 = (uint64_t)it * (EPT / 8);           // first Philox counter of the item
  if constexpr (FMT == SNIP_MXFP4) {
    float x[32], h0[16], h1[16];
    unpack16(v[0], v[1], h0);
    unpack16(v[2], v[3], h1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      x[i] = h0[i];
      x[16 + i] = h1[i];
    }
    Words4 d[4];
    if (SR) {
#pragma unroll
      for (int q = 0; q < 4; ++q) d[q] = draws8(J.seed, J.tensor_id, g0 + q);
    }
    uint32_t out[4], sc;
    double be2, bx2;
    float bx2f, am;
    mx_block<SR>(x, d, out, sc, be2, bx2, bx2f, am);
    const bool bad = !(bx2f <= 3.0e38f);
    uint32_t bnf = 0u, bam = __float_as_uint(am);
    double rx2 = bx2;
    if (bad) {
      bam = 0u;
      nonfinite_stats<32>(x, bnf, rx2, bam);
    }
    acc.nf += bnf;
    acc.x2r += rx2;
    acc.e2r += bad ? 0.0 : be2;
    acc.amax_bits = max(acc.amax_bits, bam);
    *reinterpret_cast<uint4*>(J.codes + it * 16) = make_uint4(out[0], out[1], out[2], out[3]);
    J.scales[it] = (uint8_t)sc;
  } else {
    float x[16];
    unpack16(v[0], v[1], x);
    Words4 d0, d1;
    if (SR) {
      d0 = draws8(J.seed, J.tensor_id, g0);
      d1 = draws8(J.seed, J.tensor_id, g0 + 1);
    }
    float be2, bx2;
    if constexpr (FMT == SNIP_NVFP4) {
      uint32_t lo, hi, sc;
      nvfp4_block<SR>(x, eS, d0, d1, inv_lut, lo, hi, sc, be2, bx2);
      *reinterpret_cast<uint2*>(J.codes + it * 8) = make_uint2(lo, hi);
      J.scales[it] = (uint8_t)sc;
    } else {
      uint32_t out[4];
      fp8_chunk<SR>(x, eS, d0, d1, out, be2, bx2);
      *reinterpret_cast<uint4*>(J.codes + it * 16) = make_uint4(out[0], out[1], out[2], out[3]);
    }
    const bool bad = !(bx2 <= 3.0e38f);
    uint32_t bnf = 0u, dummy = 0u;
    double rx2 = 0.0;
    if (bad) nonfinite_stats<16>(x, bnf, rx2, dummy);
    if (J.amax_in) acc.tmax = max(acc.tmax, bad ? dummy : block_absmax_bits<16>(x));
    acc.nf += bnf;
    acc.x2r += rx2;
    acc.e2s += bad ? 0.0 : (double)be2;
    acc.x2s += bad ? 0.0 : (double)bx2;
  }
}

template <int FMT, bool SR>
__global__ __launch_bounds__(256) void quant_row_kernel(QJobs jobs) {
  int32_t wg0[kMaxJobs];
  for (int i = 0; i < kMaxJobs; ++i) wg0[i] = jobs.j[i].wg0;
  const QJob J = jobs.j[find_job(wg0, jobs.n)];
  const int wg = blockIdx.x - J.wg0;
  __shared__ uint32_t ured[8];
  __shared__ double dred[8];

  constexpr int EPT = (FMT == SNIP_MXFP4) ? 32 : 16;
  constexpr int NV = EPT / 8;                             // 16-byte loads per item
  const int64_t tpr = J.cols / EPT;
  const int64_t nitems = J.rows * tpr;
  const bool flat = J.ld == J.cols;
  const int64_t stride = (int64_t)J.nwg * 512;
  int64_t it = (int64_t)wg * 512 + threadIdx.x;

  // first loads before the tensor-max reduction, to overlap its latency
  uint4 v[2][NV];
  auto load = [&](int64_t item, uint4 (&dst)[NV]) {
    if (item < nitems) {
      const int64_t off = flat ? item * EPT : (item / tpr) * J.ld + (item % tpr) * EPT;
      const uint4* src = reinterpret_cast<const uint4*>(J.x + off);
#pragma unroll
      for (int q = 0; q < NV; ++q) dst[q] = src[q];
    }
  };
  load(it, v[0]);
  load(it + 256, v[1]);

  const float A = (FMT == SNIP_MXFP4) ? 0.0f : wg_tensor_amax(J.amax_in, J.amax_part, J.n_amax_part, ured);
  const int eS = tensor_exp(A, FMT);
  if (wg == 0 && threadIdx.x == 0 && J.texp) *J.texp = eS;
  __shared__ float inv_lut[FMT == SNIP_NVFP4 ? 128 : 1];
  if constexpr (FMT == SNIP_NVFP4) fill_inv_lut(inv_lut);

  RowAcc<FMT, SR> acc;
  for (; it < nitems; it += stride) {
    uint4 cur[2][NV];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int q = 0; q < NV; ++q) cur[u][q] = v[u][q];
    load(it + stride, v[0]);                                // prefetch the next iteration
    load(it + stride + 256, v[1]);
    row_item<FMT, SR>(J, eS, inv_lut, it, cur[0], acc);
    if (it + 256 < nitems) row_item<FMT, SR>(J, eS, inv_lut, it + 256, cur[1], acc);
  }
  if (FMT != SNIP_MXFP4) acc.amax_bits = J.amax_in ? acc.tmax : __float_as_uint(A);
  const double e2 = ldexp(acc.e2s, 2 * eS) + acc.e2r;
  const double x2 = ldexp(acc.x2s, 2 * eS) + acc.x2r;
  wg_store_stats(J.part + wg, e2, x2, acc.nf, acc.amax_bits, dred, ured);
}

// ------------------------------------------------------------ column-wise
// Source x[R][C] -> output [C][R] with blocks running down the source
// columns. Tile: kColTileRows x kColTileCols; lane l owns columns c0+2l and
// c0+2l+1, wave w owns the block rows w, w+4, ... All loads of a tile are
// issued before its blocks are encoded; codes are staged in LDS and written
// as contiguous output row segments.
template <int FMT, bool SR>
__global__ __launch_bounds__(256) void quant_col_kernel(QJobs jobs) {
  int32_t wg0[kMaxJobs];
  for (int i = 0; i < kMaxJobs; ++i) wg0[i] = jobs.j[i].wg0;
  const QJob J = jobs.j[find_job(wg0, jobs.n)];
  const int wg = blockIdx.x - J.wg0;
  __shared__ uint32_t ured[8];
  __shared__ double dred[8];

  constexpr int BLK = (FMT == SNIP_MXFP4) ? 32 : 16;
  constexpr int TR = kColTileRows, TC = kColTileCols;
  constexpr int NB = TR / BLK;                                  // blocks per column per tile
  constexpr int NBT = NB / 4;                                   // block rows per wave
  constexpr int CB = (FMT == SNIP_NVFP4) ? 8 : 16;              // code bytes per block
  constexpr int PITCH = NB * CB + 8;                            // LDS bytes per column
  __shared__ __align__(16) uint8_t lcodes[TC * PITCH];
  __shared__ uint8_t lsc[TC * NB];

  const float A = (FMT == SNIP_MXFP4) ? 0.0f : wg_tensor_amax(J.amax_in, J.amax_part, J.n_amax_part, ured);
  const int eS = tensor_exp(A, FMT);
  if (wg == 0 && threadIdx.x == 0 && J.texp) *J.texp = eS;
  __shared__ float inv_lut[FMT == SNIP_NVFP4 ? 128 : 1];
  if constexpr (FMT == SNIP_NVFP4) fill_inv_lut(inv_lut);

  const int64_t R = J.rows, C = J.cols;
  const int64_t rowbytes = R / BLK * CB;                        // output row length (codes)
  const int64_t tiles_c = ceil_div(C, TC);
  const int64_t ntiles = ceil_div(R, TR) * tiles_c;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double e2s = 0.0, x2s = 0.0, e2r = 0.0, x2r = 0.0;
  uint32_t nf = 0u, amax_bits = 0u;
  uint32_t tmax = 0u;                                          // max |x| seen (supplied-max runs)

  for (int64_t tile = wg; tile < ntiles; tile += J.nwg) {
    const int64_t r0 = (tile / tiles_c) * TR;
    const int64_t c0 = (tile % tiles_c) * TC;
    const int nbt = (int)((R - r0) / BLK < NB ? (R - r0) / BLK : NB);
    const int64_t col = c0 + 2 * lane;
    if (col < C) {
      uint32_t w[NBT][BLK];
#pragma unroll
      for (int t = 0; t < NBT; ++t) {
        const int rb = wave + 4 * t;
        if (rb < nbt) {
          const uint16_t* src = J.x + (r0 + (int64_t)rb * BLK) * J.ld + col;
#pragma unroll
          for (int i = 0; i < BLK; ++i) w[t][i] = *reinterpret_cast<const uint32_t*>(src + (int64_t)i * J.ld);
        }
      }
#pragma unroll
      for (int t = 0; t < NBT; ++t) {
        const int rb = wave + 4 * t;
        if (rb >= nbt) continue;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float x[BLK];
#pragma unroll
          for (int i = 0; i < BLK; ++i) x[i] = h ? bf16_hi(w[t][i]) : bf16_lo(w[t][i]);
          const int cl = 2 * lane + h;
          const uint64_t g0 = ((uint64_t)(col + h) * (uint64_t)R + (uint64_t)(r0 + rb * BLK)) >> 3;
          uint8_t* dst = lcodes + cl * PITCH + rb * CB;
          if constexpr (FMT == SNIP_MXFP4) {
            Words4 d[4];
            if (SR) {
#pragma unroll
              for (int q = 0; q < 4; ++q) d[q] = draws8(J.seed, J.tensor_id, g0 + q);
            }
            uint32_t out[4], sc;
            double be2, bx2;
            float bx2f, am;
            mx_block<SR>(x, d, out, sc, be2, bx2, bx2f, am);
            const bool bad = !(bx2f <= 3.0e38f);
            uint32_t bnf = 0u, bam = __float_as_uint(am);
            double rx2 = bx2;
            if (bad) {
              bam = 0u;
              nonfinite_stats<32>(x, bnf, rx2, bam);
            }
            nf += bnf;
            x2r += rx2;
            e2r += bad ? 0.0 : be2;
            amax_bits = max(amax_bits, bam);
            *reinterpret_cast<uint2*>(dst) = make_uint2(out[0], out[1]);
            *reinterpret_cast<uint2*>(dst + 8) = make_uint2(out[2], out[3]);
            lsc[cl * NB + rb] = (uint8_t)sc;
          } else {
            Words4 d0, d1;
            if (SR) {
              d0 = draws8(J.seed, J.tensor_id, g0);
              d1 = draws8(J.seed, J.tensor_id, g0 + 1);
            }
            float be2, bx2;
            if constexpr (FMT == SNIP_NVFP4) {
              uint32_t lo, hi, sc;
              nvfp4_block<SR>(x, eS, d0, d1, inv_lut, lo, hi, sc, be2, bx2);
              *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
              lsc[cl * NB + rb] = (uint8_t)sc;
            } else {
              uint32_t out[4];
              fp8_chunk<SR>(x, eS, d0, d1, out, be2, bx2);
              *reinterpret_cast<uint2*>(dst) = make_uint2(out[0], out[1]);
              *reinterpret_cast<uint2*>(dst + 8) = make_uint2(out[2], out[3]);
            }
            const bool bad = !(bx2 <= 3.0e38f);
            uint32_t bnf = 0u, dummy = 0u;
            double rx2 = 0.0;
            if (bad) nonfinite_stats<16>(x, bnf, rx2, dummy);
            if (J.amax_in) tmax = max(tmax, bad ? dummy : block_absmax_bits<16>(x));
            nf += bnf;
            x2r += rx2;
            e2s += bad ? 0.0 : (double)be2;
            x2s += bad ? 0.0 : (double)bx2;
          }
        }
      }
    }
    __syncthreads();
    // write the tile's output row segments: nbt*CB bytes of codes per column
    constexpr int CH = NB * CB / 8;                              // 8-byte chunks per column
    const int valid_ch = nbt * CB / 8;
    for (int q = threadIdx.x; q < TC * CH; q += 256) {
      const int cl = q / CH, ch = q % CH;
      if (ch < valid_ch && c0 + cl < C) {
        *reinterpret_cast<uint2*>(J.codes + (c0 + cl) * rowbytes + r0 / BLK * CB + ch * 8) =
            *reinterpret_cast<const uint2*>(lcodes + cl * PITCH + ch * 8);
      }
    }
    if constexpr (FMT != SNIP_FP8_E4M3) {
      for (int q = threadIdx.x; q < TC * NB; q += 256) {
        const int cl = q / NB, b = q % NB;
        if (b < nbt && c0 + cl < C) J.scales[(c0 + cl) * (R / BLK) + r0 / BLK + b] = lsc[cl * NB + b];
      }
    }
    __syncthreads();
  }
  if (FMT != SNIP_MXFP4) amax_bits = J.amax_in ? tmax : __float_as_uint(A);
  const double e2 = ldexp(e2s, 2 * eS) + e2r;
  const double x2 = ldexp(x2s, 2 * eS) + x2r;
  wg_store_stats(J.part + wg, e2, x2, nf, amax_bits, dred, ured);
}

// ------------------------------------------------------------ bf16 (unquantized)
// Row-wise: copy x[rows][cols] (leading dim ld) to a contiguous buffer, or
// only gather the statistics when no destination is given.
__global__ __launch_bounds__(256) void bf16_copy_kernel(QJobs jobs) {
  int32_t wg0[kMaxJobs];
  for (int i = 0; i < kMaxJobs; ++i) wg0[i] = jobs.j[i].wg0;
  const QJob J = jobs.j[find_job(wg0, jobs.n)];
  const int wg = blockIdx.x - J.wg0;
  __shared__ uint32_t ured[8];
  __shared__ double dred[8];
  const int64_t cpr = J.cols >> 3;
  const int64_t nchunk = J.rows * cpr;
  const bool flat = J.ld == J.cols;
  double x2 = 0.0;
  uint32_t nf = 0u, amax_bits = 0u;
  for (int64_t c = (int64_t)wg * 256 + threadIdx.x; c < nchunk; c += (int64_t)J.nwg * 256) {
    const int64_t off = flat ? c * 8 : (c / cpr) * J.ld + (c % cpr) * 8;
    const uint4 v = *reinterpret_cast<const uint4*>(J.x + off);
    if (J.codes) *reinterpret_cast<uint4*>(J.codes + c * 16) = v;   // null: statistics only
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = bf16_lo(w[i]), b = bf16_hi(w[i]);
      if (isfinite(a)) { s = fmaf(a, a, s); amax_bits = max(amax_bits, __float_as_uint(fabsf(a))); } else ++nf;
      if (isfinite(b)) { s = fmaf(b, b, s); amax_bits = max(amax_bits, __float_as_uint(fabsf(b))); } else ++nf;
    }
    x2 += (double)s;
  }
  wg_store_stats(J.part + wg, 0.0, x2, nf, amax_bits, dred, ured);
}

// Column-wise: out[cols][rows] = x^T through 64x64 LDS tiles.
__global__ __launch_bounds__(256) void bf16_transpose_kernel(QJobs jobs) {
  int32_t wg0[kMaxJobs];
  for (int i = 0; i < kMaxJobs; ++i) wg0[i] = jobs.j[i].wg0;
  const QJob J = jobs.j[find_job(wg0, jobs.n)];
  const int wg = blockIdx.x - J.wg0;
  __shared__ uint32_t ured[8];
  __shared__ double dred[8];
  __shared__ uint16_t tileb[64][66];
  const int64_t R = J.rows, C = J.cols;
  const int64_t tiles_c = ceil_div(C, 64);
  const int64_t ntiles = ceil_div(R, 64) * tiles_c;
  const int tr = threadIdx.x >> 2, tq = (threadIdx.x & 3) * 16;
  double x2 = 0.0;
  uint32_t nf = 0u, amax_bits = 0u;
  for (int64_t tile = wg; tile < ntiles; tile += J.nwg) {
    const int64_t r0 = (tile / tiles_c) * 64, c0 = (tile % tiles_c) * 64;
    // load: thread reads 16 consecutive elements of source row r0+tr
    if (r0 + tr < R && c0 + tq < C) {
      const uint4* s = reinterpret_cast<const uint4*>(J.x + (r0 + tr) * J.ld + c0 + tq);
      const uint4 v0 = s[0], v1 = s[1];
      const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      float s2 = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        tileb[tr][tq + 2 * i] = (uint16_t)(w[i] & 0xFFFFu);
        tileb[tr][tq + 2 * i + 1] = (uint16_t)(w[i] >> 16);
        const float a = bf16_lo(w[i]), b = bf16_hi(w[i]);
        if (isfinite(a)) { s2 = fmaf(a, a, s2); amax_bits = max(amax_bits, __float_as_uint(fabsf(a))); } else ++nf;
        if (isfinite(b)) { s2 = fmaf(b, b, s2); amax_bits = max(amax_bits, __float_as_uint(fabsf(b))); } else ++nf;
      }
      x2 += (double)s2;
    }
    __syncthreads();
    // store: thread writes 16 consecutive elements of output row c0+tr
    if (c0 + tr < C && r0 + tq < R) {
      uint32_t w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        w[i] = (uint32_t)tileb[tq + 2 * i][tr] | ((uint32_t)tileb[tq + 2 * i + 1][tr] << 16);
      uint4* d = reinterpret_cast<uint4*>(J.codes + ((c0 + tr) * R + r0 + tq) * 2);
      d[0] = make_uint4(w[0], w[1], w[2], w[3]);
      d[1] = make_uint4(w[4], w[5], w[6], w[7]);
    }
    __syncthreads();
  }
  wg_store_stats(J.part + wg, 0.0, x2, nf, amax_bits, dred, ured);
}

// ------------------------------------------------------------ finalisation
// One workgroup per tensor: fixed-order sum of the partials.
__global__ __launch_bounds__(256) void finalize_kernel(FJobs jobs) { finalize_one(jobs.j[blockIdx.x]); }

// ------------------------------------------------------------ launchers
hipError_t launch_amax(const AJobs& jobs, int total_wg, hipStream_t s) {
  hipLaunchKernelGGL(amax_kernel, dim3(total_wg), dim3(kAmaxThreads), 0, s, jobs);
  return hipGetLastError();
}

template <int FMT>
static hipError_t quant_row_fmt(bool sr, const QJobs& jobs, int total_wg, hipStream_t s) {
  if (sr) hipLaunchKernelGGL((quant_row_kernel<FMT, true>), dim3(total_wg), dim3(256), 0, s, jobs);
  else hipLaunchKernelGGL((quant_row_kernel<FMT, false>), dim3(total_wg), dim3(256), 0, s, jobs);
  return hipGetLastError();
}

template <int FMT>
static hipError_t quant_col_fmt(bool sr, const QJobs& jobs, int total_wg, hipStream_t s) {
  if (sr) hipLaunchKernelGGL((quant_col_kernel<FMT, true>), dim3(total_wg), dim3(256), 0, s, jobs);
  else hipLaunchKernelGGL((quant_col_kernel<FMT, false>), dim3(total_wg), dim3(256), 0, s, jobs);
  return hipGetLastError();
}

hipError_t launch_quant_row(int format, bool sr, const QJobs& jobs, int total_wg, hipStream_t s) {
  switch (format) {
    case SNIP_NVFP4: return quant_row_fmt<SNIP_NVFP4>(sr, jobs, total_wg, s);
    case SNIP_FP8_E4M3: return quant_row_fmt<SNIP_FP8_E4M3>(sr, jobs, total_wg, s);
    case SNIP_MXFP4: return quant_row_fmt<SNIP_MXFP4>(sr, jobs, total_wg, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_quant_col(int format, bool sr, const QJobs& jobs, int total_wg, hipStream_t s) {
  switch (format) {
    case SNIP_NVFP4: return quant_col_fmt<SNIP_NVFP4>(sr, jobs, total_wg, s);
    case SNIP_FP8_E4M3: return quant_col_fmt<SNIP_FP8_E4M3>(sr, jobs, total_wg, s);
    case SNIP_MXFP4: return quant_col_fmt<SNIP_MXFP4>(sr, jobs, total_wg, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bf16_copy(const QJobs& jobs, int total_wg, hipStream_t s) {
  hipLaunchKernelGGL(bf16_copy_kernel, dim3(total_wg), dim3(256), 0, s, jobs);
  return hipGetLastError();
}

hipError_t launch_bf16_transpose(const QJobs& jobs, int total_wg, hipStream_t s) {
  hipLaunchKernelGGL(bf16_transpose_kernel, dim3(total_wg), dim3(256), 0, s, jobs);
  return hipGetLastError();
}

hipError_t launch_finalize(const FJobs& jobs, hipStream_t s) {
  if (jobs.n == 0) return hipSuccess;
  hipLaunchKernelGGL(finalize_kernel, dim3(jobs.n), dim3(256), 0, s, jobs);
  return hipGetLastError();
}

}  // namespace snip

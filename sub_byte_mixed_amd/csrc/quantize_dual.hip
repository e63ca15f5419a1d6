// Dual quantizer for gfx950: one read of a bf16 tensor x[R][C] yields both
// its row-wise codes (blocks along C, output [R][C]) and its column-wise
// codes (blocks down the columns, output [C][R]) in one format (NVFP4,
// FP8-E4M3 or MX-FP4), each with its own rounding, Philox stream (tensor
// id) and statistics, and the one tensor exponent both share.
//
// "FP4 All the Way" summary, Outline: nearest rounding for the forward
// operands, stochastic rounding for the backward and update operands; a
// linear layer's input and weight feed the forward GEMM row-wise and the
// update / input-gradient GEMMs column-wise, and its output gradient feeds
// both backward GEMMs ("SNIP", Fig. 5). Every code, scale and exponent is
// the one the separate row-wise and column-wise passes produce: the same
// per-element arithmetic with the same Philox counters (element index in
// the output layout, divided by 8).
//
// Work layout. A tile of 64 source rows (128 for MX) x 128 columns: wave w
// owns block row w (16 rows, 32 for MX) and lane l loads columns 2l, 2l+1
// of its rows with dword loads, as in the column-wise pass (whose 256-row
// tiles would leave a 4096 x 2048 tensor with one workgroup per CU); the
// column blocks are encoded from these registers. The same registers are written
// to a wave-private LDS block (BLK rows x 256 bytes) and read back as 16
// bytes per lane, so lane l holds 8 consecutive elements of row
// 4j + l / 16 (columns 8 (l % 16) ... + 7) in read j: exactly one Philox
// draw of the row-wise layout. An NVFP4 block (16 elements) then spans the
// lane pair (2k, 2k + 1), an MX block (32) four lanes; the block max and
// the non-finite flag are exchanged with DPP lane permutations.
#include <type_traits>

#include "quant_common.h"

namespace snip {

namespace {

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. N-1, so
// that register arrays indexed by i stay in registers.
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// Value of lane ^ 1 (quad_perm 1,0,3,2) and lane ^ 2 (quad_perm 2,3,0,1);
// both lanes of a pair are always active together.
__device__ __forceinline__ int xor1i(int v) { return __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ int xor2i(int v) { return __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false); }
__device__ __forceinline__ float xor1f(float v) { return __int_as_float(xor1i(__float_as_int(v))); }
__device__ __forceinline__ float xor2f(float v) { return __int_as_float(xor2i(__float_as_int(v))); }

// Row-wise statistics of one lane: only the quantization error. Sum x^2,
// the non-finite count and max|x| are properties of the tensor, the same in
// both layouts; the column-wise half (which sees every element once) gives
// them to both statistics records.
struct RowStats {
  double e2s = 0.0;                 // tensor-scaled domain (NVFP4, FP8)
  double e2r = 0.0;                 // raw domain (MX)
};

// Eight consecutive row elements of one lane: codes, scale (NVFP4, MX) and
// error statistics, with the block-wide quantities shared over the lanes of
// the block. A block holding a non-finite value (its error sum is then NaN
// or infinite) adds no error. `store` is false for a group past the last
// column (its partner lanes are past it too).
template <int FMT, bool SR>
__device__ __forceinline__ void row_group(const float (&x)[8], int eS, const float* inv_lut,
                                          const Words4& d, int64_t row, int64_t col, int64_t C,
                                          const DOut& o, bool store, RowStats& st) {
  if constexpr (FMT == SNIP_NVFP4) {
    float xs[8], am = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      xs[i] = ldexpf(x[i], -eS);
      am = fmaxf(am, fabsf(xs[i]));
    }
    am = fmaxf(am, xor1f(am));                        // max over the 16-element block
    const uint32_t sc = e4m3_rne(am / 6.0f);
    const float shat = e4m3_val(sc);
    const float inv = inv_lut[sc];
    float r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = xs[i] * inv;
    const uint32_t code = SR ? fp4x8_sr(r, d) : fp4x8_rne(r);
    float q[8], be2 = 0.0f;
    fp4x8_dec(code, q);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float err = fmaf(q[i], shat, -xs[i]);
      be2 = fmaf(err, err, be2);
    }
    const int bad = (int)!(be2 <= 3.0e38f) | xor1i((int)!(be2 <= 3.0e38f));
    if (store) {
      *reinterpret_cast<uint32_t*>(o.codes + row * (C / 2) + col / 2) = code;
      if ((col & 15) == 0) o.scales[row * (C / 16) + col / 16] = (uint8_t)sc;
      st.e2s += bad ? 0.0 : (double)be2;
    }
  } else if constexpr (FMT == SNIP_FP8_E4M3) {
    float r[8], c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      r[i] = ldexpf(x[i], -eS);
      c[i] = __builtin_amdgcn_fmed3f(r[i], -448.0f, 448.0f);
    }
    const uint32_t w0 = SR ? fp8x4_sr(c, d, 0) : fp8x4_rne(c);
    const uint32_t w1 = SR ? fp8x4_sr(c + 4, d, 4) : fp8x4_rne(c + 4);
    float q[8], be2 = 0.0f;
    fp8x4_dec(w0, q);
    fp8x4_dec(w1, q + 4);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float e = q[i] - r[i];
      be2 = fmaf(e, e, be2);
    }
    // non-finite flag over the 16-element chunk of the row-wise pass
    const int bad = (int)!(be2 <= 3.0e38f) | xor1i((int)!(be2 <= 3.0e38f));
    if (store) {
      *reinterpret_cast<uint2*>(o.codes + row * C + col) = make_uint2(w0, w1);
      st.e2s += bad ? 0.0 : (double)be2;
    }
  } else {  // MX-FP4: 32-element block over four lanes
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(x[i]));
    am = fmaxf(am, xor1f(am));
    am = fmaxf(am, xor2f(am));
    int X = -127;
    if (am > 0.0f) {
      const int e = (int)(__float_as_uint(am) >> 23);
      X = e - 129;
      X = X < -127 ? -127 : X;
    }
    const uint32_t sc = (uint32_t)(X + 127);
    const float pw = am > 0.0f ? exp2i(-X) : 0.0f;
    float r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = x[i] * pw;
    const uint32_t code = SR ? fp4x8_sr(r, d) : fp4x8_rne(r);
    float q[8], be2 = 0.0f;
    fp4x8_dec(code, q);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float err = q[i] - r[i];
      be2 = fmaf(err, err, be2);
    }
    int bad = (int)!(be2 <= 3.0e38f);
    bad |= xor1i(bad);
    bad |= xor2i(bad);
    if (store) {
      *reinterpret_cast<uint32_t*>(o.codes + row * (C / 2) + col / 2) = code;
      if ((col & 31) == 0) o.scales[row * (C / 32) + col / 32] = (uint8_t)sc;
      st.e2r += bad ? 0.0 : ldexp((double)be2, 2 * X);
    }
  }
}

template <int FMT, bool SR_ROW, bool SR_COL>
__global__ __launch_bounds__(256) void quant_dual_kernel(DJobs jobs) {
  int32_t wg0[kMaxJobs];
  for (int i = 0; i < kMaxJobs; ++i) wg0[i] = jobs.j[i].wg0;
  const DJob J = jobs.j[find_job(wg0, jobs.n)];
  const int wg = blockIdx.x - J.wg0;
  __shared__ uint32_t ured[8];
  __shared__ double dred[8];

  constexpr int BLK = (FMT == SNIP_MXFP4) ? 32 : 16;
  constexpr int TR = dual_tile_rows(FMT), TC = kColTileCols;
  constexpr int NB = TR / BLK;                                  // blocks per column per tile
  constexpr int NBT = NB / 4;                                   // block rows per wave
  static_assert(NBT >= 1, "one block row per wave at least");
  constexpr int CB = (FMT == SNIP_NVFP4) ? 8 : 16;              // code bytes per column block
  constexpr int PITCH = NB * CB + 8;                            // LDS bytes per column
  __shared__ __align__(16) uint8_t lcodes[TC * PITCH];
  __shared__ uint8_t lsc[TC * NB];
  __shared__ __align__(16) uint32_t lrow[4][BLK * 64];         // wave-private row staging

  const int64_t R = J.rows, C = J.cols;
  const int64_t rowbytes = R / BLK * CB;                        // column-wise output row (codes)
  const int64_t tiles_c = ceil_div(C, TC);
  const int64_t ntiles = ceil_div(R, TR) * tiles_c;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // a tile's block rows of this wave: lane l holds columns 2l, 2l+1 (dword loads)
  uint32_t w[NBT][BLK];
  auto load_tile = [&](int64_t tile) {
    const int64_t r0 = (tile / tiles_c) * TR;
    const int64_t c0 = (tile % tiles_c) * TC;
    const int nbt = (int)((R - r0) / BLK < NB ? (R - r0) / BLK : NB);
    const int64_t col = c0 + 2 * lane;
    const bool lane_ok = col < C;
    // Lanes past the last column read column 0 of the same rows (in bounds)
    // and drop it, so all loads issue without branches. ld is a multiple of
    // 8, so a row is a whole number of dwords.
    const int64_t pitch = J.ld >> 1;
    const uint32_t* base = reinterpret_cast<const uint32_t*>(J.x + r0 * J.ld + (lane_ok ? col : 0));
#pragma unroll
    for (int t = 0; t < NBT; ++t) {
      const int rb = wave + 4 * t;
      if (rb < nbt) {
        const uint32_t* src = base + (int64_t)rb * BLK * pitch;
        uint32_t v[BLK];
#pragma unroll
        for (int i = 0; i < BLK; ++i) v[i] = src[i * pitch];
#pragma unroll
        for (int i = 0; i < BLK; ++i) w[t][i] = lane_ok ? v[i] : 0u;
      }
    }
  };
  // The first tile's loads need no tensor scale: issue them before the
  // tensor max is reduced from the amax partials, so the two reads overlap.
  if (wg < ntiles) load_tile(wg);

  const float A = (FMT == SNIP_MXFP4) ? 0.0f : wg_tensor_amax(J.amax_in, J.amax_part, J.n_amax_part, ured);
  const int eS = tensor_exp(A, FMT);
  if (wg == 0 && threadIdx.x == 0) {
    if (J.row.texp) *J.row.texp = eS;
    if (J.col.texp) *J.col.texp = eS;
  }
  __shared__ float inv_lut[FMT == SNIP_NVFP4 ? 128 : 1];
  if constexpr (FMT == SNIP_NVFP4) fill_inv_lut(inv_lut);

  double e2s = 0.0, x2s = 0.0, e2r = 0.0, x2r = 0.0;           // column-wise statistics
  uint32_t nf = 0u, amax_bits = 0u;
  uint32_t tmax = 0u;                                          // max |x| seen (supplied-max runs)
  RowStats rs;
  uint32_t* stg = lrow[wave];

  for (int64_t tile = wg; tile < ntiles; tile += J.nwg) {
    const int64_t r0 = (tile / tiles_c) * TR;
    const int64_t c0 = (tile % tiles_c) * TC;
    const int nbt = (int)((R - r0) / BLK < NB ? (R - r0) / BLK : NB);
    const int64_t col = c0 + 2 * lane;
    const bool lane_ok = col < C;
    if (tile != wg) load_tile(tile);
    static_for<NBT>([&](auto tc) {
      constexpr int t = decltype(tc)::value;
      const int rb = wave + 4 * t;                              // wave-uniform
      if (rb >= nbt) return;
      // ---- column blocks, from registers
      if (lane_ok) {
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
            if (SR_COL) {
#pragma unroll
              for (int q = 0; q < 4; ++q) d[q] = draws8(J.seed, J.col.tensor_id, g0 + q);
            }
            uint32_t out[4], sc;
            double be2, bx2;
            float bx2f, am;
            mx_block<SR_COL>(x, d, out, sc, be2, bx2, bx2f, am);
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
            if (SR_COL) {
              d0 = draws8(J.seed, J.col.tensor_id, g0);
              d1 = draws8(J.seed, J.col.tensor_id, g0 + 1);
            }
            float be2, bx2;
            if constexpr (FMT == SNIP_NVFP4) {
              uint32_t lo, hi, sc;
              nvfp4_block<SR_COL>(x, eS, d0, d1, inv_lut, lo, hi, sc, be2, bx2);
              *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
              lsc[cl * NB + rb] = (uint8_t)sc;
            } else {
              uint32_t out[4];
              fp8_chunk<SR_COL>(x, eS, d0, d1, out, be2, bx2);
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
      // ---- row blocks, through the wave's LDS block: row i of the block
      // row at stg[64 i ...], as the wave loaded it (4 bytes per lane)
#pragma unroll
      for (int i = 0; i < BLK; ++i) stg[i * 64 + lane] = w[t][i];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int j = 0; j < BLK / 4; ++j) {
        const uint4 v = *reinterpret_cast<const uint4*>(stg + j * 256 + lane * 4);
        const int64_t row = r0 + (int64_t)rb * BLK + 4 * j + (lane >> 4);
        const int64_t colg = c0 + (lane & 15) * 8;
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[2 * i] = bf16_lo(wv[i]);
          x[2 * i + 1] = bf16_hi(wv[i]);
        }
        Words4 d;
        if (SR_ROW) d = draws8(J.seed, J.row.tensor_id, ((uint64_t)row * (uint64_t)C + (uint64_t)colg) >> 3);
        row_group<FMT, SR_ROW>(x, eS, inv_lut, d, row, colg, C, J.row, colg < C, rs);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    });
    __syncthreads();
    // column-wise output row segments: nbt*CB bytes of codes per column
    constexpr int CH = NB * CB / 8;                              // 8-byte chunks per column
    const int valid_ch = nbt * CB / 8;
    for (int q = threadIdx.x; q < TC * CH; q += 256) {
      const int cl = q / CH, ch = q % CH;
      if (ch < valid_ch && c0 + cl < C) {
        *reinterpret_cast<uint2*>(J.col.codes + (c0 + cl) * rowbytes + r0 / BLK * CB + ch * 8) =
            *reinterpret_cast<const uint2*>(lcodes + cl * PITCH + ch * 8);
      }
    }
    if constexpr (FMT != SNIP_FP8_E4M3) {
      for (int q = threadIdx.x; q < TC * NB; q += 256) {
        const int cl = q / NB, b = q % NB;
        if (b < nbt && c0 + cl < C) J.col.scales[(c0 + cl) * (R / BLK) + r0 / BLK + b] = lsc[cl * NB + b];
      }
    }
    __syncthreads();
  }
  // the tensor max used for scaling, or under a supplied max the current
  // tensor's own (the column blocks cover every element once)
  if (FMT != SNIP_MXFP4) amax_bits = J.amax_in ? tmax : __float_as_uint(A);
  // Sum x^2, the non-finite count and the max from the column blocks serve
  // both records; only the errors differ
  const double x2 = ldexp(x2s, 2 * eS) + x2r;
  wg_store_stats(J.col.part + wg, ldexp(e2s, 2 * eS) + e2r, x2, nf, amax_bits, dred, ured);
  __syncthreads();
  wg_store_stats(J.row.part + wg, ldexp(rs.e2s, 2 * eS) + rs.e2r, x2, nf, amax_bits, dred, ured);
}

template <int FMT>
hipError_t dual_fmt(bool sr_row, bool sr_col, const DJobs& jobs, int total_wg, hipStream_t s) {
  const dim3 grid(total_wg), block(256);
  if (sr_row && sr_col) hipLaunchKernelGGL((quant_dual_kernel<FMT, true, true>), grid, block, 0, s, jobs);
  else if (sr_row) hipLaunchKernelGGL((quant_dual_kernel<FMT, true, false>), grid, block, 0, s, jobs);
  else if (sr_col) hipLaunchKernelGGL((quant_dual_kernel<FMT, false, true>), grid, block, 0, s, jobs);
  else hipLaunchKernelGGL((quant_dual_kernel<FMT, false, false>), grid, block, 0, s, jobs);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_dual(int format, bool sr_row, bool sr_col, const DJobs& jobs, int total_wg,
                             hipStream_t s) {
  switch (format) {
    case SNIP_NVFP4: return dual_fmt<SNIP_NVFP4>(sr_row, sr_col, jobs, total_wg, s);
    case SNIP_FP8_E4M3: return dual_fmt<SNIP_FP8_E4M3>(sr_row, sr_col, jobs, total_wg, s);
    case SNIP_MXFP4: return dual_fmt<SNIP_MXFP4>(sr_row, sr_col, jobs, total_wg, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace snip

// FP4 design-space variants for gfx950: E2M1 codes with a block of 16 or 32
// elements and an E4M3 (with the power-of-two tensor scale), E8M0 or BF16
// block scale, row-wise or column-wise, nearest or stochastic rounding,
// with the same statistics as every quantize pass.
//
// "FP4 All the Way" summary, Outline: the study explored block size,
// scaling format and rounding before settling on NVFP4 (16 E2M1 values per
// E4M3 scale). These kernels quantize with the other points of that space
// so that their error statistics and sqrt(3) diagnostic can be compared on
// the same tensors; the GEMMs take NVFP4 and MX-FP4 only.
//
// Rules (per block of BLK elements along K):
//   E4M3  as NVFP4: x' = ldexp(x, -eS), s = E4M3_RNE(max|x'| / 6),
//         r = x' * fp32(1 / s);
//   E8M0  as MX: X = floor(log2 max|x|) - 2, r = x * 2^-X;
//   BF16  s = bf16_RNE(fp32(max|x| / 6)), r = x * fp32(1 / s);
// then E2M1 rounding of r; a zero scale gives signed-zero codes.
//
// Work layout: one thread per block. Row-wise, consecutive threads take
// consecutive blocks of a row (16- or 32-element loads). Column-wise,
// consecutive threads take consecutive source columns of one block row, so
// each of the BLK 2-byte loads of a wave covers 128 contiguous bytes.
#include "quant_common.h"

namespace snip {

namespace {

constexpr int kE4M3 = 0, kE8M0 = 1, kBF16 = 2;

template <int F> struct Variant;
template <> struct Variant<SNIP_FP4_E4M3_B32> { static constexpr int BLK = 32, KIND = kE4M3; };
template <> struct Variant<SNIP_FP4_E8M0_B16> { static constexpr int BLK = 16, KIND = kE8M0; };
template <> struct Variant<SNIP_FP4_BF16_B16> { static constexpr int BLK = 16, KIND = kBF16; };
template <> struct Variant<SNIP_FP4_BF16_B32> { static constexpr int BLK = 32, KIND = kBF16; };

// Round a non-negative finite fp32 to bfloat16, nearest, ties to even.
__device__ __forceinline__ uint32_t bf16_rne_bits(float t) {
  const uint32_t b = __float_as_uint(t);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

struct VAcc {
  double e2 = 0.0, x2 = 0.0;
  uint32_t nf = 0u, amax_bits = 0u;
  uint32_t tmax = 0u;                           // E4M3 scales: max |x| seen
};

// One block: codes (BLK/8 words), scale code, statistics.
template <int BLK, int KIND, bool SR>
__device__ __forceinline__ void fp4v_block(const float (&x)[BLK], int eS, uint64_t seed, uint32_t tid_,
                                           uint64_t g0, const float* inv_lut, uint32_t (&out)[BLK / 8],
                                           uint32_t& sc, VAcc& acc) {
  constexpr int NW = BLK / 8;
  float r[BLK], ref[BLK];
  float shat;                                   // decoded scale (E4M3: scaled domain)
  int X = 0;                                    // E8M0 exponent
  float am = 0.0f;
  float amr = 0.0f;                             // E4M3: max |x| before scaling
  if constexpr (KIND == kE4M3) {
#pragma unroll
    for (int i = 0; i < BLK; ++i) {
      ref[i] = ldexpf(x[i], -eS);
      am = fmaxf(am, fabsf(ref[i]));
      amr = fmaxf(amr, fabsf(x[i]));
    }
    sc = e4m3_rne(am / 6.0f);
    shat = e4m3_val(sc);
    const float inv = inv_lut[sc];
#pragma unroll
    for (int i = 0; i < BLK; ++i) r[i] = ref[i] * inv;
  } else if constexpr (KIND == kE8M0) {
#pragma unroll
    for (int i = 0; i < BLK; ++i) am = fmaxf(am, fabsf(x[i]));
    X = -127;
    if (am > 0.0f) {
      X = (int)(__float_as_uint(am) >> 23) - 129;
      X = X < -127 ? -127 : X;
    }
    sc = (uint32_t)(X + 127);
    const float pw = am > 0.0f ? exp2i(-X) : 0.0f;
#pragma unroll
    for (int i = 0; i < BLK; ++i) {
      r[i] = x[i] * pw;
      ref[i] = r[i];
    }
    shat = 1.0f;
  } else {
#pragma unroll
    for (int i = 0; i < BLK; ++i) {
      ref[i] = x[i];
      am = fmaxf(am, fabsf(x[i]));
    }
    sc = bf16_rne_bits(am / 6.0f);
    shat = __uint_as_float(sc << 16);
    const float inv = shat > 0.0f ? 1.0f / shat : 0.0f;
#pragma unroll
    for (int i = 0; i < BLK; ++i) r[i] = x[i] * inv;
  }
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (SR) {
      const Words4 d = draws8(seed, tid_, g0 + w);
      out[w] = fp4x8_sr(r + 8 * w, d);
    } else {
      out[w] = fp4x8_rne(r + 8 * w);
    }
  }
  float be2 = 0.0f, bx2 = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    float q[8];
    fp4x8_dec(out[w], q);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float err = fmaf(q[i], shat, -ref[8 * w + i]);
      be2 = fmaf(err, err, be2);
      bx2 = fmaf(ref[8 * w + i], ref[8 * w + i], bx2);
    }
  }
  const int sh = KIND == kE4M3 ? 2 * eS : KIND == kE8M0 ? 2 * X : 0;
  if (!(bx2 <= 3.0e38f)) {                      // non-finite input: count, sum the finite part
    uint32_t bnf = 0u, bam = 0u;
    double rx2 = 0.0;
    nonfinite_stats<BLK>(x, bnf, rx2, bam);
    acc.nf += bnf;
    acc.x2 += rx2;
    if (KIND != kE4M3) acc.amax_bits = max(acc.amax_bits, bam);
    else acc.tmax = max(acc.tmax, bam);
  } else {
    acc.e2 += ldexp((double)be2, sh);
    acc.x2 += ldexp((double)bx2, sh);
    if (KIND != kE4M3) acc.amax_bits = max(acc.amax_bits, __float_as_uint(am));
    else acc.tmax = max(acc.tmax, __float_as_uint(amr));
  }
}

template <int BLK>
__device__ __forceinline__ void store_codes(uint8_t* p, const uint32_t (&w)[BLK / 8]) {
  if constexpr (BLK == 16) *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
  else *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}

template <int KIND>
__device__ __forceinline__ void store_scale(uint8_t* scales, int64_t i, uint32_t sc) {
  if constexpr (KIND == kBF16) reinterpret_cast<uint16_t*>(scales)[i] = (uint16_t)sc;
  else scales[i] = (uint8_t)sc;
}

template <int FMT, bool SR, bool COL>
__global__ __launch_bounds__(256) void quant_fp4v_kernel(QJobs jobs) {
  constexpr int BLK = Variant<FMT>::BLK, KIND = Variant<FMT>::KIND;
  int32_t wg0[kMaxJobs];
  for (int i = 0; i < kMaxJobs; ++i) wg0[i] = jobs.j[i].wg0;
  const QJob J = jobs.j[find_job(wg0, jobs.n)];
  const int wg = blockIdx.x - J.wg0;
  __shared__ uint32_t ured[8];
  __shared__ double dred[8];
  const float A = KIND == kE4M3 ? wg_tensor_amax(J.amax_in, J.amax_part, J.n_amax_part, ured) : 0.0f;
  const int eS = KIND == kE4M3 ? tensor_exp(A, SNIP_NVFP4) : 0;
  if (wg == 0 && threadIdx.x == 0 && J.texp) *J.texp = eS;
  __shared__ float inv_lut[KIND == kE4M3 ? 128 : 1];
  if constexpr (KIND == kE4M3) fill_inv_lut(inv_lut);

  const int64_t R = J.rows, C = J.cols;
  // row-wise: item = (row, block along C); column-wise: item = (block along R, column)
  const int64_t nitems = COL ? (R / BLK) * C : R * (C / BLK);
  VAcc acc;
  for (int64_t it = (int64_t)wg * 256 + threadIdx.x; it < nitems; it += (int64_t)J.nwg * 256) {
    float x[BLK];
    int64_t first;                              // output index of the block's first element
    if constexpr (COL) {
      const int64_t b = it / C, c = it - b * C;
      const uint16_t* src = J.x + b * BLK * J.ld + c;
#pragma unroll
      for (int i = 0; i < BLK; ++i) x[i] = __uint_as_float((uint32_t)src[(int64_t)i * J.ld] << 16);
      first = c * R + b * BLK;
    } else {
      const int64_t tpr = C / BLK, row = it / tpr, kb = it - row * tpr;
      const uint4* src = reinterpret_cast<const uint4*>(J.x + row * J.ld + kb * BLK);
#pragma unroll
      for (int h = 0; h < BLK / 16; ++h) {
        float xx[16];
        unpack16(src[2 * h], src[2 * h + 1], xx);
#pragma unroll
        for (int i = 0; i < 16; ++i) x[16 * h + i] = xx[i];
      }
      first = it * BLK;
    }
    uint32_t out[BLK / 8], sc;
    fp4v_block<BLK, KIND, SR>(x, eS, J.seed, J.tensor_id, (uint64_t)first >> 3, inv_lut, out, sc, acc);
    store_codes<BLK>(J.codes + first / 2, out);
    store_scale<KIND>(J.scales, first / BLK, sc);
  }
  // E4M3 scales: the tensor max used for scaling, or under a supplied max
  // the current tensor's own
  if (KIND == kE4M3) acc.amax_bits = J.amax_in ? acc.tmax : __float_as_uint(A);
  wg_store_stats(J.part + wg, acc.e2, acc.x2, acc.nf, acc.amax_bits, dred, ured);
}

template <int FMT>
hipError_t fp4v_fmt(bool sr, bool col, const QJobs& jobs, int total_wg, hipStream_t s) {
  const dim3 g(total_wg), b(256);
  if (col) {
    if (sr) hipLaunchKernelGGL((quant_fp4v_kernel<FMT, true, true>), g, b, 0, s, jobs);
    else hipLaunchKernelGGL((quant_fp4v_kernel<FMT, false, true>), g, b, 0, s, jobs);
  } else {
    if (sr) hipLaunchKernelGGL((quant_fp4v_kernel<FMT, true, false>), g, b, 0, s, jobs);
    else hipLaunchKernelGGL((quant_fp4v_kernel<FMT, false, false>), g, b, 0, s, jobs);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_fp4v(int format, int layout, bool sr, const QJobs& jobs, int total_wg, hipStream_t s) {
  const bool col = layout == SNIP_COLWISE;
  switch (format) {
    case SNIP_FP4_E4M3_B32: return fp4v_fmt<SNIP_FP4_E4M3_B32>(sr, col, jobs, total_wg, s);
    case SNIP_FP4_E8M0_B16: return fp4v_fmt<SNIP_FP4_E8M0_B16>(sr, col, jobs, total_wg, s);
    case SNIP_FP4_BF16_B16: return fp4v_fmt<SNIP_FP4_BF16_B16>(sr, col, jobs, total_wg, s);
    case SNIP_FP4_BF16_B32: return fp4v_fmt<SNIP_FP4_BF16_B32>(sr, col, jobs, total_wg, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace snip

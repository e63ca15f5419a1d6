// Internal launch interface between the host API (api.hip) and the kernels
// (quantize.hip, gemm.hip). Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/snip.h"

namespace snip {

constexpr int kMaxJobs = 4;       // tensors per multi-tensor launch
constexpr int kAmaxWG = 512;      // max workgroups of one amax pass (per tensor)
constexpr int kAmaxUnroll = 8;    // 16-byte loads in flight per amax thread
constexpr int kAmaxThreads = 256;  // threads per amax workgroup
constexpr int kQuantWG = 2048;    // max workgroups of one quantize pass (per tensor)

// One workgroup's partial statistics (already in the unscaled domain).
struct StatPart {
  double e2;           // sum of (Q(x) - x)^2 over finite elements
  double x2;           // sum of x^2 over finite elements
  uint32_t nf;         // non-finite count
  uint32_t amax_bits;  // fp32 bits of max|x| (the tensor max, or this
                       // workgroup's max for the unquantized copy)
};

// amax pre-pass over one bf16 tensor: per-workgroup max of the finite
// |x| as bf16 magnitude bits.
struct AJob {
  const uint16_t* x;
  int64_t rows, cols, ld;
  uint32_t* part;      // [nwg]
  int32_t wg0, nwg;
};
struct AJobs {
  AJob j[kMaxJobs];
  int32_t n;
};

// One quantize pass (row-wise or column-wise) of one tensor.
struct QJob {
  const uint16_t* x;
  int64_t rows, cols, ld;        // source bf16 [rows][cols], leading dim ld
  uint8_t* codes;
  uint8_t* scales;
  int32_t* texp;                 // tensor exponent out (NVFP4/FP8) or null
  const float* amax_in;          // delayed-scaling max or null
  const uint32_t* amax_part;     // amax pre-pass partials (bf16 magnitude bits)
  int32_t n_amax_part;
  StatPart* part;                // [nwg]
  uint64_t seed;
  uint32_t tensor_id;
  int32_t wg0, nwg;
};
struct QJobs {
  QJob j[kMaxJobs];
  int32_t n;
};

// Dual quantize pass of one tensor: one read of x[rows][cols] gives its
// row-wise codes ([rows][cols], blocks along cols) and its column-wise codes
// ([cols][rows], blocks down the columns), in one format.
struct DOut {
  uint8_t* codes;
  uint8_t* scales;
  int32_t* texp;                 // tensor exponent out (NVFP4/FP8) or null
  StatPart* part;                // [nwg]
  uint32_t tensor_id;
};
struct DJob {
  const uint16_t* x;
  int64_t rows, cols, ld;
  const float* amax_in;
  const uint32_t* amax_part;
  int32_t n_amax_part;
  uint64_t seed;
  DOut row, col;
  int32_t wg0, nwg;
};
struct DJobs {
  DJob j[kMaxJobs];
  int32_t n;
};

// Statistics finalisation of one tensor.
struct FJob {
  const StatPart* part;
  int32_t nwg;
  snip_stats* out;
};
struct FJobs {
  FJob j[kMaxJobs * 2];
  int32_t n;
};

// Row-wise quantization of a GEMM's fp32 output C[M][N] in the launch that
// computes it (blocks along N): codes, scales and tensor exponent in
// `fmt` (NVFP4 or FP8), tensor scale from the supplied max, one statistics
// partial per workgroup.
struct QOut {
  uint8_t* codes;          // [M][N/2] (NVFP4) or [M][N] (FP8); null: no quantization
  uint8_t* scales;         // [M][N/16] E4M3 (NVFP4)
  int32_t* texp;           // tensor exponent out
  const float* amax_in;    // supplied max|C| (delayed scaling)
  StatPart* part;          // [workgroups]
  uint64_t seed;
  uint32_t tensor_id;
  int32_t fmt;
  int32_t sr;
};

// GEMM problem: C[M][N] = A[M][K] . B[N][K]^T * 2^(ea + eb).
struct GemmArgs {
  const uint8_t* a;        // codes (bf16 for BF16)
  const uint8_t* b;
  const uint8_t* as;       // block scales or null
  const uint8_t* bs;
  const int32_t* ea;       // tensor exponents or null
  const int32_t* eb;
  float* c;
  int64_t M, N, K, ldc;
  float* partial;          // split-K scratch [ksplit][M][N] or null (no split)
  int32_t tiles_m, tiles_n;
  int64_t kchunk;          // K elements per split (set by launch_gemm)
  FJobs fin;               // statistics finalisations run as extra workgroups
                           // of the launch (fin.n == 0: none)
  // A second, independent problem of the same format run by the same launch
  // (launch_gemm_pair): its tiles follow the first problem's, unsplit.
  struct Second {
    const uint8_t *a, *b, *as, *bs;
    const int32_t *ea, *eb;
    float* c;
    int64_t M, N, K, ldc;
    int32_t tiles_m, tiles_n;
  } sec;
  int32_t nsec;            // 0: one problem; 1: `sec` follows
  QOut q;                  // output quantization (q.codes null: none)
};

// Tile shape and K split chosen on the host for one GEMM.
struct GemmPlan {
  int bm, bn;              // tile: 256x256, 256x128 (FP8) or 128x128
  int bk;                  // K per LDS stage
  int64_t tiles;
  int ksplit;
  int64_t kchunk;
  int staged;              // 1: register-staged kernel (128x128 MX-FP4, BF16)
};
GemmPlan plan_gemm(int format, int64_t M, int64_t N, int64_t K);
size_t gemm_partial_bytes(int format, int64_t M, int64_t N, int64_t K);
// Statistics partials (workgroups) of a GEMM launch that quantizes its output.
int64_t gemm_qout_parts(int format, int64_t M, int64_t N, int64_t K);

// Launchers (all asynchronous on `s`); they return the hipError_t of the launch.
hipError_t launch_amax(const AJobs& jobs, int total_wg, hipStream_t s);
hipError_t launch_quant_row(int format, bool sr, const QJobs& jobs, int total_wg, hipStream_t s);
hipError_t launch_quant_col(int format, bool sr, const QJobs& jobs, int total_wg, hipStream_t s);
hipError_t launch_quant_dual(int format, bool sr_row, bool sr_col, const DJobs& jobs, int total_wg,
                             hipStream_t s);
hipError_t launch_quant_fp4v(int format, int layout, bool sr, const QJobs& jobs, int total_wg, hipStream_t s);
hipError_t launch_bf16_copy(const QJobs& jobs, int total_wg, hipStream_t s);
hipError_t launch_bf16_transpose(const QJobs& jobs, int total_wg, hipStream_t s);
hipError_t launch_finalize(const FJobs& jobs, hipStream_t s);
hipError_t launch_gemm(int format, const GemmArgs& g, hipStream_t s);
// Two independent GEMMs of one format (a layer's dgrad and wgrad). Where both
// run unsplit on 128x128 tiles they share one launch (g2's tiles after
// g1's) so that each fills the other's idle workgroup slots and tail;
// otherwise two launches. g2 carries the statistics finalisations; g1.fin
// must be empty. Both need the same split-K scratch rules as launch_gemm.
hipError_t launch_gemm_pair(int format, const GemmArgs& g1, const GemmArgs& g2, hipStream_t s);

// Launch timing (snip_timing_*): when enabled, each launch is bracketed by
// a pair of HIP events. timing_begin returns the slot to close with
// timing_end (-1: not timed).
struct LaunchTag {
  int kind, format, layout, rounding;
  double work;
};
int timing_begin(const LaunchTag& t, hipStream_t s);
void timing_end(int slot, hipStream_t s);

// Work decomposition helpers shared by host and kernels.
constexpr int kColTileRows = 256;   // column-wise quantizer: source rows per tile
constexpr int kColTileCols = 128;   // source columns per tile (2 per lane)
// dual quantizer: source rows per tile, one block row (16, MX 32) per wave
__host__ __device__ constexpr int dual_tile_rows(int format) { return format == SNIP_MXFP4 ? 128 : 64; }
__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace snip

// Host side of libsnip's C ABI: argument validation (before any HIP call),
// workspace carving and kernel enqueueing. See include/snip.h for the
// contract of each entry point.
//
// The quantized linear layer follows "SNIP", Fig. 5 (forward GEMM and the
// two backward GEMMs of a linear layer, each in the layer's plan format) and
// "FP4 All the Way" summary, Outline (round-to-nearest forward operands,
// stochastic rounding for back-propagation and update operands).
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"

using namespace snip;

// ================================================================ launch timing
// Process-global recorder behind snip_timing_*: event pairs created up front,
// handed out in launch order while enabled.
namespace {
struct TimingState {
  bool on = false;
  std::vector<hipEvent_t> ev;          // 2 per slot: start, stop
  std::vector<LaunchTag> tag;
  int used = 0;
  int64_t untimed = 0;
};
TimingState g_timing;
}  // namespace

namespace snip {
int timing_begin(const LaunchTag& t, hipStream_t s) {
  if (!g_timing.on) return -1;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return -1;
  if (g_timing.used >= (int)g_timing.tag.size()) {
    ++g_timing.untimed;
    return -1;
  }
  const int slot = g_timing.used++;
  g_timing.tag[slot] = t;
  if (hipEventRecord(g_timing.ev[2 * slot], s) != hipSuccess) {
    g_timing.tag[slot].kind = -1;       // dropped on read
  }
  return slot;
}
void timing_end(int slot, hipStream_t s) {
  if (slot < 0) return;
  if (hipEventRecord(g_timing.ev[2 * slot + 1], s) != hipSuccess) g_timing.tag[slot].kind = -1;
}
}  // namespace snip

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return SNIP_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
constexpr size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Formats a qtensor may hold (the FP4 design-space variants included) and
// the formats the GEMM and layer calls take.
bool valid_format(int f) { return f >= SNIP_BF16 && f <= SNIP_FP4_BF16_B32; }
bool gemm_format(int f) { return f >= SNIP_BF16 && f <= SNIP_MXFP4; }
bool fp4_variant(int f) { return f >= SNIP_FP4_E4M3_B32 && f <= SNIP_FP4_BF16_B32; }
int block_of(int f) {
  return (f == SNIP_MXFP4 || f == SNIP_FP4_E4M3_B32 || f == SNIP_FP4_BF16_B32) ? 32 : 16;
}
bool has_scales(int f) { return f == SNIP_NVFP4 || f == SNIP_MXFP4 || fp4_variant(f); }
bool has_texp(int f) { return f == SNIP_NVFP4 || f == SNIP_FP8_E4M3 || f == SNIP_FP4_E4M3_B32; }
bool needs_amax(int f) { return has_texp(f); }

int64_t code_bytes(int f, int64_t rows, int64_t k) {
  if (f == SNIP_NVFP4 || f == SNIP_MXFP4 || fp4_variant(f)) return rows * k / 2;
  if (f == SNIP_FP8_E4M3) return rows * k;
  if (f == SNIP_BF16) return rows * k * 2;
  return -1;
}
int64_t scale_bytes(int f, int64_t rows, int64_t k) {
  if (!has_scales(f)) return 0;
  const int per = (f == SNIP_FP4_BF16_B16 || f == SNIP_FP4_BF16_B32) ? 2 : 1;
  return rows * (k / block_of(f)) * per;
}

// The LDS-DMA GEMM kernels address an operand's rows with 32-bit byte
// offsets, so the codes of every GEMM operand (A[M][K] and B[N][K]; their
// block scales are smaller) must stay below 4 GiB. Checked before any HIP
// call; a larger problem is split by the caller.
constexpr double kMaxOperandBytes = 4294967296.0 - 1024.0;
int gemm_operands_fit(int f, int64_t M, int64_t N, int64_t K, const char* who) {
  const double per = f == SNIP_FP8_E4M3 ? 1.0 : f == SNIP_BF16 ? 2.0 : 0.5;
  const int64_t rows[2] = {M, N};
  for (int64_t r : rows)
    if ((double)r * (double)K * per > kMaxOperandBytes)
      return fail(SNIP_E_SHAPE, "%s: a %lld x %lld GEMM operand exceeds 4 GiB of codes", who, (long long)r,
                  (long long)K);
  return 0;
}

constexpr size_t kAlign = 256;
constexpr size_t kAmaxBytes = align_up(kAmaxWG * sizeof(uint32_t), kAlign);
constexpr size_t kPartBytes = align_up(kQuantWG * sizeof(StatPart), kAlign);
// scratch of one quantize pass: amax partials + statistics partials
constexpr size_t kQuantWS = kAmaxBytes + kPartBytes;

size_t qtensor_ws_bytes(int f, int64_t rows, int64_t k) {
  return align_up((size_t)code_bytes(f, rows, k), kAlign) +
         align_up((size_t)scale_bytes(f, rows, k), kAlign) + kAlign;
}

// Bump allocator over the caller's workspace.
struct Carver {
  uint8_t* base;
  size_t used = 0;
  explicit Carver(void* p) : base(static_cast<uint8_t*>(p)) {}
  uint8_t* take(size_t n) {
    uint8_t* p = base + used;
    used += align_up(n, kAlign);
    return p;
  }
};

// Grid sizes.
int amax_wg(int64_t rows, int64_t cols) {
  const int64_t chunks = rows * cols / 8;
  int64_t wg = ceil_div(chunks, kAmaxThreads * kAmaxUnroll);
  if (wg < 1) wg = 1;
  return (int)(wg > kAmaxWG ? kAmaxWG : wg);
}
int quant_wg(int layout, int f, int64_t rows, int64_t cols) {
  int64_t wg;
  if (f == SNIP_BF16) {
    wg = layout == SNIP_ROWWISE ? ceil_div(rows * cols / 8, 256 * 2) : ceil_div(rows, 64) * ceil_div(cols, 64);
  } else if (fp4_variant(f)) {
    wg = ceil_div(rows * cols / block_of(f), 256);                  // one thread per block
  } else if (layout == SNIP_ROWWISE) {
    wg = ceil_div(rows * cols / (f == SNIP_MXFP4 ? 32 : 16), 512);     // two items per thread
  } else {
    wg = ceil_div(rows, kColTileRows) * ceil_div(cols, kColTileCols);
  }
  if (wg < 1) wg = 1;
  return (int)(wg > kQuantWG ? kQuantWG : wg);
}

hipError_t g_last_hip = hipSuccess;

int hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    g_last_hip = e;
    return fail(SNIP_E_HIP, "%s: %s", what, hipGetErrorString(e));
  }
  return SNIP_OK;
}

// One planned quantize pass (used by snip_quantize and the linear layer).
struct QPlan {
  const uint16_t* x;
  int64_t rows, cols, ld;
  int layout, format;
  bool sr;
  uint64_t seed;
  uint32_t tensor_id;
  const float* amax_in;
  const uint32_t* amax_part;   // partials of the amax pass (if any)
  int n_amax_part;
  uint8_t* codes;
  uint8_t* scales;
  int32_t* texp;
  StatPart* part;
  int nwg;
  snip_stats* stats;
};

QJob make_qjob(const QPlan& p, int wg0) {
  QJob j;
  j.x = p.x;
  j.rows = p.rows;
  j.cols = p.cols;
  j.ld = p.ld;
  j.codes = p.codes;
  j.scales = p.scales;
  j.texp = p.texp;
  j.amax_in = p.amax_in;
  j.amax_part = p.amax_part;
  j.n_amax_part = p.n_amax_part;
  j.part = p.part;
  j.seed = p.seed;
  j.tensor_id = p.tensor_id;
  j.wg0 = wg0;
  j.nwg = p.nwg;
  return j;
}

// Enqueue a group of quantize passes sharing (layout, format, rounding).
int run_quant_group(const QPlan* const* ps, int n, hipStream_t s) {
  if (n == 0) return SNIP_OK;
  QJobs jobs;
  std::memset(&jobs, 0, sizeof(jobs));
  int wg = 0;
  for (int i = 0; i < n; ++i) {
    jobs.j[i] = make_qjob(*ps[i], wg);
    wg += ps[i]->nwg;
  }
  for (int i = n; i < kMaxJobs; ++i) jobs.j[i].wg0 = 1 << 30;
  jobs.n = n;
  const QPlan& p = *ps[0];
  double elems = 0.0;
  for (int i = 0; i < n; ++i) elems += (double)ps[i]->rows * (double)ps[i]->cols;
  const int slot = timing_begin(LaunchTag{SNIP_LAUNCH_QUANTIZE, p.format, p.layout, p.sr ? SNIP_SR : SNIP_RNE,
                                          elems}, s);
  hipError_t e;
  if (p.format == SNIP_BF16) {
    e = p.layout == SNIP_ROWWISE ? launch_bf16_copy(jobs, wg, s) : launch_bf16_transpose(jobs, wg, s);
  } else if (fp4_variant(p.format)) {
    e = launch_quant_fp4v(p.format, p.layout, p.sr, jobs, wg, s);
  } else if (p.layout == SNIP_ROWWISE) {
    e = launch_quant_row(p.format, p.sr, jobs, wg, s);
  } else {
    e = launch_quant_col(p.format, p.sr, jobs, wg, s);
  }
  timing_end(slot, s);
  return hip_check(e, "quantize launch");
}

// Amax passes for up to kMaxJobs tensors in one launch.
struct APlan {
  const uint16_t* x;
  int64_t rows, cols, ld;
  uint32_t* part;
  int nwg;
};

int run_amax(const APlan* ps, int n, hipStream_t s) {
  if (n == 0) return SNIP_OK;
  AJobs jobs;
  std::memset(&jobs, 0, sizeof(jobs));
  int wg = 0;
  for (int i = 0; i < n; ++i) {
    jobs.j[i] = AJob{ps[i].x, ps[i].rows, ps[i].cols, ps[i].ld, ps[i].part, wg, ps[i].nwg};
    wg += ps[i].nwg;
  }
  for (int i = n; i < kMaxJobs; ++i) jobs.j[i].wg0 = 1 << 30;
  jobs.n = n;
  double elems = 0.0;
  for (int i = 0; i < n; ++i) elems += (double)ps[i].rows * (double)ps[i].cols;
  const int slot = timing_begin(LaunchTag{SNIP_LAUNCH_AMAX, -1, -1, -1, elems}, s);
  const hipError_t e = launch_amax(jobs, wg, s);
  timing_end(slot, s);
  return hip_check(e, "amax launch");
}

// Finalisation jobs of the passes that requested statistics.
FJobs fjobs_of(const QPlan* const* ps, int n) {
  FJobs f;
  std::memset(&f, 0, sizeof(f));
  for (int i = 0; i < n; ++i) {
    if (!ps[i] || !ps[i]->stats) continue;
    f.j[f.n++] = FJob{ps[i]->part, ps[i]->nwg, ps[i]->stats};
  }
  return f;
}

int run_finalize(const QPlan* const* ps, int n, hipStream_t s) {
  const FJobs f = fjobs_of(ps, n);
  const int slot = f.n ? timing_begin(LaunchTag{SNIP_LAUNCH_FINALIZE, -1, -1, -1, (double)f.n}, s) : -1;
  const hipError_t e = launch_finalize(f, s);
  timing_end(slot, s);
  return hip_check(e, "finalize launch");
}

// Group passes by (layout, format, rounding) and launch each group once.
int run_quant_all(QPlan* const* ps, int n, hipStream_t s) {
  bool done[8] = {false};
  for (int i = 0; i < n; ++i) {
    if (done[i]) continue;
    const QPlan* grp[kMaxJobs];
    int g = 0;
    for (int j = i; j < n && g < kMaxJobs; ++j) {
      if (done[j]) continue;
      if (ps[j]->layout == ps[i]->layout && ps[j]->format == ps[i]->format && ps[j]->sr == ps[i]->sr) {
        grp[g++] = ps[j];
        done[j] = true;
      }
    }
    const int rc = run_quant_group(grp, g, s);
    if (rc) return rc;
  }
  return SNIP_OK;
}

// One planned dual pass (row-wise and column-wise outputs of one tensor).
struct DPlan {
  const uint16_t* x;
  int64_t rows, cols, ld;
  int format;
  bool sr_row, sr_col;
  uint64_t seed;
  const float* amax_in;
  const uint32_t* amax_part;
  int n_amax_part;
  DOut row, col;
  snip_stats* stats_row;
  snip_stats* stats_col;
  int nwg;
};

// Enqueue dual passes sharing (format, sr_row, sr_col) in one launch.
int run_dual_group(const DPlan* const* ps, int n, hipStream_t s) {
  if (n == 0) return SNIP_OK;
  DJobs jobs;
  std::memset(&jobs, 0, sizeof(jobs));
  int wg = 0;
  double elems = 0.0;
  for (int i = 0; i < n; ++i) {
    const DPlan& p = *ps[i];
    jobs.j[i] = DJob{p.x, p.rows, p.cols, p.ld, p.amax_in, p.amax_part, p.n_amax_part, p.seed,
                     p.row, p.col, wg, p.nwg};
    wg += p.nwg;
    elems += (double)p.rows * (double)p.cols;
  }
  for (int i = n; i < kMaxJobs; ++i) jobs.j[i].wg0 = 1 << 30;
  jobs.n = n;
  const DPlan& p = *ps[0];
  // launch record: rounding = rounding_row + 2 * rounding_col
  const int rnd = (p.sr_row ? SNIP_SR : SNIP_RNE) + 2 * (p.sr_col ? SNIP_SR : SNIP_RNE);
  const int slot = timing_begin(LaunchTag{SNIP_LAUNCH_QUANTIZE, p.format, SNIP_BOTHWISE, rnd, elems}, s);
  const hipError_t e = launch_quant_dual(p.format, p.sr_row, p.sr_col, jobs, wg, s);
  timing_end(slot, s);
  return hip_check(e, "dual quantize launch");
}

// Statistics finalisation of the dual passes' requested outputs.
FJobs fjobs_of_dual(const DPlan* const* ps, int n) {
  FJobs f;
  std::memset(&f, 0, sizeof(f));
  for (int i = 0; i < n; ++i) {
    if (ps[i]->stats_row) f.j[f.n++] = FJob{ps[i]->row.part, ps[i]->nwg, ps[i]->stats_row};
    if (ps[i]->stats_col) f.j[f.n++] = FJob{ps[i]->col.part, ps[i]->nwg, ps[i]->stats_col};
  }
  return f;
}

int run_finalize_dual(const DPlan* const* ps, int n, hipStream_t s) {
  const FJobs f = fjobs_of_dual(ps, n);
  const int slot = f.n ? timing_begin(LaunchTag{SNIP_LAUNCH_FINALIZE, -1, -1, -1, (double)f.n}, s) : -1;
  const hipError_t e = launch_finalize(f, s);
  timing_end(slot, s);
  return hip_check(e, "finalize launch");
}

DOut dout_of(const snip_qtensor& q, StatPart* part, uint32_t tensor_id) {
  return DOut{static_cast<uint8_t*>(q.codes), static_cast<uint8_t*>(q.scales),
              has_texp(q.format) ? q.tensor_exp : nullptr, part, tensor_id};
}

bool dual_format(int f) { return f == SNIP_FP8_E4M3 || f == SNIP_NVFP4 || f == SNIP_MXFP4; }

int dual_wg(int f, int64_t rows, int64_t cols) {
  const int64_t wg = ceil_div(rows, dual_tile_rows(f)) * ceil_div(cols, kColTileCols);
  return (int)(wg < 1 ? 1 : wg > kQuantWG ? kQuantWG : wg);
}

int validate_qtensor(const snip_qtensor* q, const char* name, bool need_codes = true) {
  if (!q) return fail(SNIP_E_NULL, "%s: descriptor is NULL", name);
  if (!valid_format(q->format)) return fail(SNIP_E_FORMAT, "%s: unknown format %d", name, q->format);
  if (q->rows <= 0 || q->k <= 0) return fail(SNIP_E_SHAPE, "%s: rows=%lld k=%lld must be > 0", name,
                                           (long long)q->rows, (long long)q->k);
  if (q->k % block_of(q->format)) return fail(SNIP_E_SHAPE, "%s: k=%lld not a multiple of %d", name,
                                             (long long)q->k, block_of(q->format));
  if (need_codes && !q->codes) return fail(SNIP_E_NULL, "%s: codes is NULL", name);
  if (has_scales(q->format) && !q->scales) return fail(SNIP_E_NULL, "%s: scales is NULL", name);
  if (has_texp(q->format) && !q->tensor_exp) return fail(SNIP_E_NULL, "%s: tensor_exp is NULL", name);
  if (!aligned(q->codes, 16) || !aligned(q->scales, 16) || !aligned(q->tensor_exp, 4))
    return fail(SNIP_E_ALIGN, "%s: device pointers must be 16-byte aligned", name);
  return SNIP_OK;
}

}  // namespace

// ====================================================================== API
extern "C" {

const char* snip_last_error(void) { return g_err.c_str(); }

int snip_version(void) { return 100; }

namespace {
void timing_release() {
  for (hipEvent_t e : g_timing.ev) (void)hipEventDestroy(e);
  g_timing.ev.clear();
  g_timing.tag.clear();
  g_timing.used = 0;
  g_timing.on = false;
}
}  // namespace

int snip_timing_start(int capacity) {
  if (capacity < 1 || capacity > (1 << 20))
    return fail(SNIP_E_SHAPE, "snip_timing_start: capacity %d outside 1 .. 2^20", capacity);
  timing_release();
  g_timing.ev.reserve(2 * (size_t)capacity);
  for (int i = 0; i < 2 * capacity; ++i) {
    hipEvent_t e;
    const hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      timing_release();
      return hip_check(r, "snip_timing_start: hipEventCreate");
    }
    g_timing.ev.push_back(e);
  }
  g_timing.tag.assign((size_t)capacity, LaunchTag{-1, -1, -1, -1, 0.0});
  g_timing.untimed = 0;
  g_timing.on = true;
  return ok();
}

int snip_timing_read(snip_launch_record* out, int max, int64_t* n_untimed) {
  if (g_timing.ev.empty()) return fail(SNIP_E_FORMAT, "snip_timing_read: timing was not started");
  if (max > 0 && !out) return fail(SNIP_E_NULL, "snip_timing_read: out is NULL");
  g_timing.on = false;
  int n = 0;
  int rc = SNIP_OK;
  for (int i = 0; i < g_timing.used; ++i) {
    const LaunchTag& t = g_timing.tag[i];
    if (t.kind < 0) continue;
    hipError_t r = hipEventSynchronize(g_timing.ev[2 * i + 1]);
    float ms = 0.0f;
    if (r == hipSuccess) r = hipEventElapsedTime(&ms, g_timing.ev[2 * i], g_timing.ev[2 * i + 1]);
    if (r != hipSuccess) {
      rc = hip_check(r, "snip_timing_read: event");
      break;
    }
    if (n < max) out[n++] = snip_launch_record{t.kind, t.format, t.layout, t.rounding, t.work, (double)ms};
  }
  if (n_untimed) *n_untimed = g_timing.untimed;
  timing_release();
  return rc ? rc : (ok(), n);
}

int64_t snip_qtensor_bytes(int format, int64_t rows, int64_t k, int part) {
  if (!valid_format(format) || rows <= 0 || k <= 0 || (part != 0 && part != 1)) return -1;
  if (k % block_of(format)) return -1;
  return part == 0 ? code_bytes(format, rows, k) : scale_bytes(format, rows, k);
}

size_t snip_quantize_workspace(int64_t rows, int64_t cols, int layout, int format) {
  if (rows <= 0 || cols <= 0 || !valid_format(format) || (layout != SNIP_ROWWISE && layout != SNIP_COLWISE))
    return 0;
  return kQuantWS;
}

size_t snip_qgemm_workspace(int64_t M, int64_t N, int64_t K, int format) {
  if (M <= 0 || N <= 0 || K <= 0 || !gemm_format(format)) return 0;
  return gemm_partial_bytes(format, M, N, K);
}

size_t snip_linear_fwd_workspace(int64_t T, int64_t in, int64_t out, int format) {
  if (T <= 0 || in <= 0 || out <= 0 || !gemm_format(format)) return 0;
  return 2 * kQuantWS + qtensor_ws_bytes(format, T, in) + qtensor_ws_bytes(format, out, in) +
         align_up(gemm_partial_bytes(format, T, out, in), kAlign);
}

size_t snip_linear_bwd_workspace(int64_t T, int64_t in, int64_t out, int fmt_dgrad, int fmt_wgrad) {
  if (T <= 0 || in <= 0 || out <= 0 || !gemm_format(fmt_dgrad) || !gemm_format(fmt_wgrad)) return 0;
  const size_t split = std::max(gemm_partial_bytes(fmt_dgrad, T, in, out),
                                gemm_partial_bytes(fmt_wgrad, out, in, T));
  return 3 * kAmaxBytes + 4 * kPartBytes + qtensor_ws_bytes(fmt_dgrad, T, out) +
         qtensor_ws_bytes(fmt_dgrad, in, out) + qtensor_ws_bytes(fmt_wgrad, out, T) +
         qtensor_ws_bytes(fmt_wgrad, in, T) + align_up(split, kAlign);
}

size_t snip_quantize_dual_workspace(int64_t rows, int64_t cols, int format) {
  if (rows <= 0 || cols <= 0 || !dual_format(format)) return 0;
  return kAmaxBytes + 2 * kPartBytes;
}

size_t snip_linear_fwd_save_workspace(int64_t T, int64_t in, int64_t out, int format) {
  if (T <= 0 || in <= 0 || out <= 0 || !dual_format(format)) return 0;
  return 2 * kAmaxBytes + 4 * kPartBytes + qtensor_ws_bytes(format, T, in) + qtensor_ws_bytes(format, out, in) +
         align_up(gemm_partial_bytes(format, T, out, in), kAlign);
}

size_t snip_linear_bwd_saved_workspace(int64_t T, int64_t in, int64_t out, int format) {
  if (T <= 0 || in <= 0 || out <= 0 || !dual_format(format)) return 0;
  const size_t split = std::max(gemm_partial_bytes(format, T, in, out), gemm_partial_bytes(format, out, in, T));
  return kAmaxBytes + 2 * kPartBytes + qtensor_ws_bytes(format, T, out) + qtensor_ws_bytes(format, out, T) +
         align_up(split, kAlign);
}

size_t snip_workspace_size(int op, int64_t M, int64_t N, int64_t K, int format) {
  switch (op) {
    case SNIP_OP_QUANTIZE: return snip_quantize_workspace(M, N, SNIP_ROWWISE, format);
    case SNIP_OP_QGEMM: return snip_qgemm_workspace(M, N, K, format);
    case SNIP_OP_LINEAR_FWD: return snip_linear_fwd_workspace(M, K, N, format);
    case SNIP_OP_LINEAR_BWD: return snip_linear_bwd_workspace(M, K, N, format, format);
    case SNIP_OP_QUANTIZE_DUAL: return snip_quantize_dual_workspace(M, N, format);
    case SNIP_OP_LINEAR_FWD_SAVE: return snip_linear_fwd_save_workspace(M, K, N, format);
    case SNIP_OP_LINEAR_BWD_SAVED: return snip_linear_bwd_saved_workspace(M, K, N, format);
    case SNIP_OP_QGEMM_QOUT: return snip_qgemm_qout_workspace(M, N, K, format);
    default: return 0;
  }
}

size_t snip_qgemm_qout_workspace(int64_t M, int64_t N, int64_t K, int format) {
  if (M <= 0 || N <= 0 || K <= 0 || (format != SNIP_FP8_E4M3 && format != SNIP_NVFP4)) return 0;
  return align_up((size_t)gemm_qout_parts(format, M, N, K) * sizeof(StatPart), kAlign) +
         align_up(gemm_partial_bytes(format, M, N, K), kAlign);
}

int snip_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld, int layout, int format,
                  int rounding, uint64_t seed, uint32_t tensor_id, const float* amax_in,
                  const snip_qtensor* out, snip_stats* stats, void* ws, size_t ws_bytes,
                  void* stream) {
  if (!x) return fail(SNIP_E_NULL, "snip_quantize: x is NULL");
  if (!valid_format(format)) return fail(SNIP_E_FORMAT, "snip_quantize: unknown format %d", format);
  if (rounding != SNIP_RNE && rounding != SNIP_SR)
    return fail(SNIP_E_FORMAT, "snip_quantize: unknown rounding %d", rounding);
  if (layout != SNIP_ROWWISE && layout != SNIP_COLWISE)
    return fail(SNIP_E_FORMAT, "snip_quantize: unknown layout %d", layout);
  if (rows <= 0 || cols <= 0) return fail(SNIP_E_SHAPE, "snip_quantize: rows=%lld cols=%lld must be > 0",
                                          (long long)rows, (long long)cols);
  if (cols % 16) return fail(SNIP_E_SHAPE, "snip_quantize: cols=%lld not a multiple of 16", (long long)cols);
  if (ld < cols || ld % 8) return fail(SNIP_E_SHAPE, "snip_quantize: ld=%lld must be >= cols and a multiple of 8",
                                       (long long)ld);
  const int blk = block_of(format);
  const int64_t K = layout == SNIP_ROWWISE ? cols : rows;
  const int64_t R = layout == SNIP_ROWWISE ? rows : cols;
  if (K % blk) return fail(SNIP_E_SHAPE, "snip_quantize: K=%lld not a multiple of %d", (long long)K, blk);
  const int rc = validate_qtensor(out, "snip_quantize: out");
  if (rc) return rc;
  if (out->format != format) return fail(SNIP_E_FORMAT, "snip_quantize: out->format %d != format %d",
                                         out->format, format);
  if (out->rows != R || out->k != K)
    return fail(SNIP_E_SHAPE, "snip_quantize: out is [%lld][%lld], expected [%lld][%lld]",
                (long long)out->rows, (long long)out->k, (long long)R, (long long)K);
  if (!aligned(x, 16) || !aligned(amax_in, 4) || !aligned(stats, 8) || !aligned(ws, 16))
    return fail(SNIP_E_ALIGN, "snip_quantize: misaligned pointer");
  if (!ws || ws_bytes < kQuantWS)
    return fail(SNIP_E_WORKSPACE, "snip_quantize: workspace of %zu bytes needed", (size_t)kQuantWS);

  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver cv(ws);
  uint32_t* apart = reinterpret_cast<uint32_t*>(cv.take(kAmaxBytes));
  StatPart* part = reinterpret_cast<StatPart*>(cv.take(kPartBytes));

  QPlan p{};
  p.x = static_cast<const uint16_t*>(x);
  p.rows = rows;
  p.cols = cols;
  p.ld = ld;
  p.layout = layout;
  p.format = format;
  p.sr = rounding == SNIP_SR;
  p.seed = seed;
  p.tensor_id = tensor_id;
  p.amax_in = amax_in;
  p.codes = static_cast<uint8_t*>(out->codes);
  p.scales = static_cast<uint8_t*>(out->scales);
  p.texp = has_texp(format) ? out->tensor_exp : nullptr;
  p.part = part;
  p.nwg = quant_wg(layout, format, rows, cols);
  p.stats = stats;
  if (needs_amax(format) && !amax_in) {
    APlan a{p.x, rows, cols, ld, apart, amax_wg(rows, cols)};
    int r = run_amax(&a, 1, s);
    if (r) return r;
    p.amax_part = apart;
    p.n_amax_part = a.nwg;
  }
  const QPlan* grp[1] = {&p};
  int r = run_quant_group(grp, 1, s);
  if (r) return r;
  if (stats) {
    r = run_finalize(grp, 1, s);
    if (r) return r;
  }
  return ok();
}

int snip_qgemm(const snip_qtensor* a, const snip_qtensor* b, float* c, int64_t ldc, void* ws,
               size_t ws_bytes, void* stream) {
  int rc = validate_qtensor(a, "snip_qgemm: a");
  if (rc) return rc;
  rc = validate_qtensor(b, "snip_qgemm: b");
  if (rc) return rc;
  if (!c) return fail(SNIP_E_NULL, "snip_qgemm: c is NULL");
  if (a->format != b->format)
    return fail(SNIP_E_FORMAT, "snip_qgemm: operand formats differ (%d, %d)", a->format, b->format);
  if (!gemm_format(a->format))
    return fail(SNIP_E_FORMAT, "snip_qgemm: format %d is a quantizer-only FP4 variant", a->format);
  if (a->k != b->k) return fail(SNIP_E_SHAPE, "snip_qgemm: K differs (%lld, %lld)", (long long)a->k,
                                (long long)b->k);
  if (a->k % 128) return fail(SNIP_E_SHAPE, "snip_qgemm: K=%lld not a multiple of 128", (long long)a->k);
  if (ldc < b->rows) return fail(SNIP_E_SHAPE, "snip_qgemm: ldc=%lld < N=%lld", (long long)ldc,
                                 (long long)b->rows);
  if (!aligned(c, 16)) return fail(SNIP_E_ALIGN, "snip_qgemm: c must be 16-byte aligned");
  rc = gemm_operands_fit(a->format, a->rows, b->rows, a->k, "snip_qgemm");
  if (rc) return rc;
  GemmArgs g;
  std::memset(&g, 0, sizeof(g));
  g.a = static_cast<const uint8_t*>(a->codes);
  g.b = static_cast<const uint8_t*>(b->codes);
  g.as = static_cast<const uint8_t*>(a->scales);
  g.bs = static_cast<const uint8_t*>(b->scales);
  g.ea = has_texp(a->format) ? a->tensor_exp : nullptr;
  g.eb = has_texp(b->format) ? b->tensor_exp : nullptr;
  g.c = c;
  g.M = a->rows;
  g.N = b->rows;
  g.K = a->k;
  g.ldc = ldc;
  if (ws && !aligned(ws, 16)) return fail(SNIP_E_ALIGN, "snip_qgemm: workspace must be 16-byte aligned");
  const size_t need = gemm_partial_bytes(a->format, g.M, g.N, g.K);
  // a split-K plan needs its scratch; without it the GEMM runs unsplit
  g.partial = (need > 0 && ws && ws_bytes >= need) ? static_cast<float*>(ws) : nullptr;
  rc = hip_check(launch_gemm(a->format, g, static_cast<hipStream_t>(stream)), "gemm launch");
  if (rc) return rc;
  return ok();
}

int snip_qgemm_qout(const snip_qtensor* a, const snip_qtensor* b, float* c, int64_t ldc, int rounding,
                    uint64_t seed, uint32_t tensor_id, const float* amax_in, const snip_qtensor* out,
                    snip_stats* stats, void* ws, size_t ws_bytes, void* stream) {
  const char* who = "snip_qgemm_qout";
  int rc = validate_qtensor(a, "snip_qgemm_qout: a");
  if (rc) return rc;
  rc = validate_qtensor(b, "snip_qgemm_qout: b");
  if (rc) return rc;
  rc = validate_qtensor(out, "snip_qgemm_qout: out");
  if (rc) return rc;
  if (!c || !amax_in) return fail(SNIP_E_NULL, "%s: c and amax_in must be non-NULL", who);
  if (a->format != b->format || (a->format != SNIP_FP8_E4M3 && a->format != SNIP_NVFP4))
    return fail(SNIP_E_FORMAT, "%s: operands must both be FP8_E4M3 or NVFP4 (got %d, %d)", who, a->format,
                b->format);
  if (out->format != SNIP_FP8_E4M3 && out->format != SNIP_NVFP4)
    return fail(SNIP_E_FORMAT, "%s: output format %d is not FP8_E4M3 or NVFP4", who, out->format);
  if (rounding != SNIP_RNE && rounding != SNIP_SR) return fail(SNIP_E_FORMAT, "%s: unknown rounding %d", who, rounding);
  if (a->k != b->k) return fail(SNIP_E_SHAPE, "%s: K differs (%lld, %lld)", who, (long long)a->k, (long long)b->k);
  if (a->k % 128) return fail(SNIP_E_SHAPE, "%s: K=%lld not a multiple of 128", who, (long long)a->k);
  if (b->rows % 16) return fail(SNIP_E_SHAPE, "%s: N=%lld not a multiple of 16", who, (long long)b->rows);
  if (out->rows != a->rows || out->k != b->rows)
    return fail(SNIP_E_SHAPE, "%s: out is [%lld][%lld], expected [%lld][%lld]", who, (long long)out->rows,
                (long long)out->k, (long long)a->rows, (long long)b->rows);
  if (ldc < b->rows || ldc % 4)
    return fail(SNIP_E_SHAPE, "%s: ldc=%lld must be >= N=%lld and a multiple of 4", who, (long long)ldc,
                (long long)b->rows);
  if (!aligned(c, 16) || !aligned(amax_in, 4) || !aligned(stats, 8) || !aligned(ws, 16))
    return fail(SNIP_E_ALIGN, "%s: misaligned pointer", who);
  rc = gemm_operands_fit(a->format, a->rows, b->rows, a->k, who);
  if (rc) return rc;
  const int64_t M = a->rows, N = b->rows, K = a->k;
  const size_t need = snip_qgemm_qout_workspace(M, N, K, a->format);
  if (!ws || ws_bytes < need) return fail(SNIP_E_WORKSPACE, "%s: workspace of %zu bytes needed", who, need);

  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver cv(ws);
  const int64_t nparts = gemm_qout_parts(a->format, M, N, K);
  StatPart* part = reinterpret_cast<StatPart*>(cv.take((size_t)nparts * sizeof(StatPart)));
  const size_t split_bytes = gemm_partial_bytes(a->format, M, N, K);
  float* split = split_bytes ? reinterpret_cast<float*>(cv.take(split_bytes)) : nullptr;
  GemmArgs g;
  std::memset(&g, 0, sizeof(g));
  g.a = static_cast<const uint8_t*>(a->codes);
  g.b = static_cast<const uint8_t*>(b->codes);
  g.as = static_cast<const uint8_t*>(a->scales);
  g.bs = static_cast<const uint8_t*>(b->scales);
  g.ea = a->tensor_exp;
  g.eb = b->tensor_exp;
  g.c = c;
  g.M = M;
  g.N = N;
  g.K = K;
  g.ldc = ldc;
  g.partial = split;
  g.q = QOut{static_cast<uint8_t*>(out->codes), static_cast<uint8_t*>(out->scales), out->tensor_exp, amax_in,
             part, seed, tensor_id, out->format, rounding == SNIP_SR ? 1 : 0};
  rc = hip_check(launch_gemm(a->format, g, s), "gemm launch");
  if (rc) return rc;
  if (stats) {
    FJobs f;
    std::memset(&f, 0, sizeof(f));
    f.j[0] = FJob{part, (int32_t)nparts, stats};
    f.n = 1;
    const int slot = timing_begin(LaunchTag{SNIP_LAUNCH_FINALIZE, -1, -1, -1, 1.0}, s);
    const hipError_t e = launch_finalize(f, s);
    timing_end(slot, s);
    rc = hip_check(e, "finalize launch");
    if (rc) return rc;
  }
  return ok();
}

}  // extern "C"

namespace {

// A quantized operand carved from the workspace.
struct QBuf {
  snip_qtensor t;
};

QBuf carve_q(Carver& cv, int f, int64_t rows, int64_t k) {
  QBuf q;
  q.t.format = f;
  q.t.reserved = 0;
  q.t.rows = rows;
  q.t.k = k;
  q.t.codes = cv.take((size_t)code_bytes(f, rows, k));
  q.t.scales = has_scales(f) ? cv.take((size_t)scale_bytes(f, rows, k)) : nullptr;
  q.t.tensor_exp = reinterpret_cast<int32_t*>(cv.take(4));
  return q;
}

// One GEMM; `fin` (may be null) lists statistics finalisations that the
// launch runs as extra workgroups after the quantize launches before it.
GemmArgs gemm_args(const snip_qtensor& a, const snip_qtensor& b, float* c, int64_t ldc, float* partial,
                   const FJobs* fin) {
  GemmArgs g;
  std::memset(&g, 0, sizeof(g));
  if (fin) g.fin = *fin;
  g.a = static_cast<const uint8_t*>(a.codes);
  g.b = static_cast<const uint8_t*>(b.codes);
  g.as = static_cast<const uint8_t*>(a.scales);
  g.bs = static_cast<const uint8_t*>(b.scales);
  g.ea = has_texp(a.format) ? a.tensor_exp : nullptr;
  g.eb = has_texp(b.format) ? b.tensor_exp : nullptr;
  g.c = c;
  g.M = a.rows;
  g.N = b.rows;
  g.K = a.k;
  g.ldc = ldc;
  g.partial = partial;
  return g;
}

int gemm_q(const snip_qtensor& a, const snip_qtensor& b, float* c, int64_t ldc, float* partial,
           hipStream_t s, const FJobs* fin = nullptr) {
  return hip_check(launch_gemm(a.format, gemm_args(a, b, c, ldc, partial, fin), s), "gemm launch");
}

// A layer's dgrad and wgrad GEMMs (same format, independent): one launch
// where both run unsplit on 128x128 tiles, else two in order. `fin` rides
// with the second.
int gemm_q_pair(const snip_qtensor& a1, const snip_qtensor& b1, float* c1, int64_t ldc1,
                const snip_qtensor& a2, const snip_qtensor& b2, float* c2, int64_t ldc2, float* partial,
                hipStream_t s, const FJobs* fin) {
  return hip_check(launch_gemm_pair(a1.format, gemm_args(a1, b1, c1, ldc1, partial, nullptr),
                                    gemm_args(a2, b2, c2, ldc2, partial, fin), s),
                   "gemm launch");
}

}  // namespace

extern "C" {

int snip_linear_fwd(const void* x, const void* w, int64_t T, int64_t in, int64_t out, int format,
                    uint64_t seed, uint32_t layer_id, float* y, snip_stats* stats2, void* ws,
                    size_t ws_bytes, void* stream) {
  if (!x || !w || !y) return fail(SNIP_E_NULL, "snip_linear_fwd: x, w and y must be non-NULL");
  if (!gemm_format(format)) return fail(SNIP_E_FORMAT, "snip_linear_fwd: format %d is not a GEMM format", format);
  if (T <= 0 || in <= 0 || out <= 0) return fail(SNIP_E_SHAPE, "snip_linear_fwd: dimensions must be > 0");
  if (in % 128) return fail(SNIP_E_SHAPE, "snip_linear_fwd: in=%lld not a multiple of 128", (long long)in);
  if (int rc = gemm_operands_fit(format, T, out, in, "snip_linear_fwd")) return rc;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16) || !aligned(stats2, 8) || !aligned(ws, 16))
    return fail(SNIP_E_ALIGN, "snip_linear_fwd: misaligned pointer");
  const size_t need = snip_linear_fwd_workspace(T, in, out, format);
  if (!ws || ws_bytes < need) return fail(SNIP_E_WORKSPACE, "snip_linear_fwd: workspace of %zu bytes needed", need);

  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver cv(ws);
  const uint16_t* xs = static_cast<const uint16_t*>(x);
  const uint16_t* wsrc = static_cast<const uint16_t*>(w);
  QPlan px{}, pw{};
  uint32_t* apx = reinterpret_cast<uint32_t*>(cv.take(kAmaxBytes));
  px.part = reinterpret_cast<StatPart*>(cv.take(kPartBytes));
  uint32_t* apw = reinterpret_cast<uint32_t*>(cv.take(kAmaxBytes));
  pw.part = reinterpret_cast<StatPart*>(cv.take(kPartBytes));
  QBuf qx, qw;
  const bool bf = format == SNIP_BF16;
  if (!bf) {
    qx = carve_q(cv, format, T, in);
    qw = carve_q(cv, format, out, in);
  }
  const size_t split_bytes = gemm_partial_bytes(format, T, out, in);
  float* split = split_bytes ? reinterpret_cast<float*>(cv.take(split_bytes)) : nullptr;
  auto fill = [&](QPlan& p, const uint16_t* src, int64_t rows, QBuf& q, uint32_t role) {
    p.x = src;
    p.rows = rows;
    p.cols = in;
    p.ld = in;
    p.layout = SNIP_ROWWISE;
    p.format = format;
    p.sr = false;
    p.seed = seed;
    p.tensor_id = 8u * layer_id + role;
    p.codes = bf ? nullptr : static_cast<uint8_t*>(q.t.codes);
    p.scales = bf ? nullptr : static_cast<uint8_t*>(q.t.scales);
    p.texp = bf ? nullptr : q.t.tensor_exp;
    p.nwg = quant_wg(SNIP_ROWWISE, format, rows, in);
  };
  fill(px, xs, T, qx, 0);
  fill(pw, wsrc, out, qw, 1);
  px.stats = stats2 ? stats2 + 0 : nullptr;
  pw.stats = stats2 ? stats2 + 1 : nullptr;
  int r;
  if (needs_amax(format)) {
    APlan a[2] = {{xs, T, in, in, apx, amax_wg(T, in)}, {wsrc, out, in, in, apw, amax_wg(out, in)}};
    r = run_amax(a, 2, s);
    if (r) return r;
    px.amax_part = apx;
    px.n_amax_part = a[0].nwg;
    pw.amax_part = apw;
    pw.n_amax_part = a[1].nwg;
  }
  if (!bf || stats2) {           // bf16: statistics-only pass, the GEMM reads x and w
    const QPlan* grp[2] = {&px, &pw};
    r = run_quant_group(grp, 2, s);
    if (r) return r;
  }
  const QPlan* fin_grp[2] = {&px, &pw};
  const FJobs fin = fjobs_of(fin_grp, stats2 ? 2 : 0);
  if (bf) {
    snip_qtensor ax{SNIP_BF16, 0, T, in, const_cast<void*>(x), nullptr, nullptr};
    snip_qtensor aw{SNIP_BF16, 0, out, in, const_cast<void*>(w), nullptr, nullptr};
    r = gemm_q(ax, aw, y, out, split, s, &fin);
  } else {
    r = gemm_q(qx.t, qw.t, y, out, split, s, &fin);
  }
  if (r) return r;
  return ok();
}

int snip_linear_bwd(const void* dy, const void* x, const void* w, int64_t T, int64_t in, int64_t out,
                    int fmt_dgrad, int fmt_wgrad, uint64_t seed, uint32_t layer_id,
                    const snip_stats* fwd_stats2, float* dx, float* dw, snip_stats* stats4, void* ws,
                    size_t ws_bytes, void* stream) {
  if (!dy || !x || !w) return fail(SNIP_E_NULL, "snip_linear_bwd: dy, x and w must be non-NULL");
  if (!gemm_format(fmt_dgrad) || !gemm_format(fmt_wgrad))
    return fail(SNIP_E_FORMAT, "snip_linear_bwd: formats (%d, %d) must be GEMM formats", fmt_dgrad, fmt_wgrad);
  if (T <= 0 || in <= 0 || out <= 0) return fail(SNIP_E_SHAPE, "snip_linear_bwd: dimensions must be > 0");
  if (dx) {
    if (out % 128) return fail(SNIP_E_SHAPE, "snip_linear_bwd: out=%lld not a multiple of 128 (dgrad K)", (long long)out);
    if (in % 16) return fail(SNIP_E_SHAPE, "snip_linear_bwd: in=%lld not a multiple of 16", (long long)in);
  }
  if (dw) {
    if (T % 128) return fail(SNIP_E_SHAPE, "snip_linear_bwd: T=%lld not a multiple of 128 (wgrad K)", (long long)T);
    if (in % 16 || out % 16) return fail(SNIP_E_SHAPE, "snip_linear_bwd: in and out must be multiples of 16");
  }
  if (dx) {
    if (int rc = gemm_operands_fit(fmt_dgrad, T, in, out, "snip_linear_bwd (dgrad)")) return rc;
  }
  if (dw) {
    if (int rc = gemm_operands_fit(fmt_wgrad, out, in, T, "snip_linear_bwd (wgrad)")) return rc;
  }
  if (!aligned(dy, 16) || !aligned(x, 16) || !aligned(w, 16) || !aligned(dx, 16) || !aligned(dw, 16) ||
      !aligned(stats4, 8) || !aligned(fwd_stats2, 8) || !aligned(ws, 16))
    return fail(SNIP_E_ALIGN, "snip_linear_bwd: misaligned pointer");
  const size_t need = snip_linear_bwd_workspace(T, in, out, fmt_dgrad, fmt_wgrad);
  if (!ws || ws_bytes < need) return fail(SNIP_E_WORKSPACE, "snip_linear_bwd: workspace of %zu bytes needed", need);
  if (!dx && !dw) return ok();

  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver cv(ws);
  const uint16_t* dys = static_cast<const uint16_t*>(dy);
  const uint16_t* xs = static_cast<const uint16_t*>(x);
  const uint16_t* wsrc = static_cast<const uint16_t*>(w);
  uint32_t* ap_dy = reinterpret_cast<uint32_t*>(cv.take(kAmaxBytes));
  uint32_t* ap_w = reinterpret_cast<uint32_t*>(cv.take(kAmaxBytes));
  uint32_t* ap_x = reinterpret_cast<uint32_t*>(cv.take(kAmaxBytes));
  QPlan p[4] = {};
  for (int i = 0; i < 4; ++i) p[i].part = reinterpret_cast<StatPart*>(cv.take(kPartBytes));
  // p[0]: dY row-wise [T][out]      (dgrad A)
  // p[1]: W column-wise -> [in][out] (dgrad B)
  // p[2]: dY column-wise -> [out][T] (wgrad A)
  // p[3]: X column-wise -> [in][T]   (wgrad B)
  const uint16_t* src[4] = {dys, wsrc, dys, xs};
  const int64_t rows[4] = {T, out, T, T};
  const int64_t cols[4] = {out, in, out, in};
  const int lay[4] = {SNIP_ROWWISE, SNIP_COLWISE, SNIP_COLWISE, SNIP_COLWISE};
  const int fmt[4] = {fmt_dgrad, fmt_dgrad, fmt_wgrad, fmt_wgrad};
  const bool use[4] = {dx != nullptr, dx != nullptr, dw != nullptr, dw != nullptr};
  QBuf q[4];
  for (int i = 0; i < 4; ++i) {
    const int64_t R = lay[i] == SNIP_ROWWISE ? rows[i] : cols[i];
    const int64_t K = lay[i] == SNIP_ROWWISE ? cols[i] : rows[i];
    // a bf16 row-wise operand is read in place; everything else is materialised
    const bool in_place = fmt[i] == SNIP_BF16 && lay[i] == SNIP_ROWWISE;
    if (use[i] && !in_place) {
      q[i] = carve_q(cv, fmt[i], R, K);
    } else {
      q[i].t = snip_qtensor{fmt[i], 0, R, K, const_cast<uint16_t*>(src[i]), nullptr, nullptr};
    }
    p[i].x = src[i];
    p[i].rows = rows[i];
    p[i].cols = cols[i];
    p[i].ld = cols[i];
    p[i].layout = lay[i];
    p[i].format = fmt[i];
    p[i].sr = true;
    p[i].seed = seed;
    p[i].tensor_id = 8u * layer_id + 2u + (uint32_t)i;
    p[i].codes = in_place ? nullptr : static_cast<uint8_t*>(q[i].t.codes);
    p[i].scales = static_cast<uint8_t*>(q[i].t.scales);
    p[i].texp = has_texp(fmt[i]) ? q[i].t.tensor_exp : nullptr;
    p[i].nwg = quant_wg(lay[i], fmt[i], rows[i], cols[i]);
    p[i].stats = stats4 ? stats4 + i : nullptr;
  }
  // amax passes: dY (shared by both of its quantizations), W, X -- the
  // forward pass's statistics, when given, already hold max|w| and max|x|
  if (fwd_stats2) {
    p[1].amax_in = &fwd_stats2[1].amax;
    p[3].amax_in = &fwd_stats2[0].amax;
  }
  APlan a[3];
  int na = 0;
  const bool need_dy = (use[0] && needs_amax(fmt[0])) || (use[2] && needs_amax(fmt[2]));
  const bool need_w = use[1] && needs_amax(fmt[1]) && !fwd_stats2;
  const bool need_x = use[3] && needs_amax(fmt[3]) && !fwd_stats2;
  if (need_dy) a[na++] = APlan{dys, T, out, out, ap_dy, amax_wg(T, out)};
  if (need_w) a[na++] = APlan{wsrc, out, in, in, ap_w, amax_wg(out, in)};
  if (need_x) a[na++] = APlan{xs, T, in, in, ap_x, amax_wg(T, in)};
  int r = run_amax(a, na, s);
  if (r) return r;
  const int n_dy = need_dy ? amax_wg(T, out) : 0;
  p[0].amax_part = ap_dy; p[0].n_amax_part = n_dy;
  p[2].amax_part = ap_dy; p[2].n_amax_part = n_dy;
  p[1].amax_part = ap_w; p[1].n_amax_part = need_w ? amax_wg(out, in) : 0;
  p[3].amax_part = ap_x; p[3].n_amax_part = need_x ? amax_wg(T, in) : 0;

  QPlan* todo[4];
  int nt = 0;
  for (int i = 0; i < 4; ++i) {
    if (!use[i]) continue;
    const bool in_place = fmt[i] == SNIP_BF16 && lay[i] == SNIP_ROWWISE;
    if (in_place && !stats4) continue;
    todo[nt++] = &p[i];
  }
  r = run_quant_all(todo, nt, s);
  if (r) return r;
  const size_t split_bytes = std::max(gemm_partial_bytes(fmt_dgrad, T, in, out),
                                      gemm_partial_bytes(fmt_wgrad, out, in, T));
  float* split = split_bytes ? reinterpret_cast<float*>(cv.take(split_bytes)) : nullptr;
  // statistics are finalised by the last GEMM launch
  const QPlan* fin_grp[4];
  int nfin = 0;
  for (int i = 0; i < 4 && stats4; ++i)
    if (use[i]) fin_grp[nfin++] = &p[i];
  const FJobs fin = fjobs_of(fin_grp, nfin);
  // dX = [T][out] . ([in][out])^T, dW = [out][T] . ([in][T])^T
  if (dx && dw && fmt_dgrad == fmt_wgrad) {
    r = gemm_q_pair(q[0].t, q[1].t, dx, in, q[2].t, q[3].t, dw, in, split, s, &fin);
    if (r) return r;
    return ok();
  }
  if (dx) {
    r = gemm_q(q[0].t, q[1].t, dx, in, split, s, dw ? nullptr : &fin);
    if (r) return r;
  }
  if (dw) {
    r = gemm_q(q[2].t, q[3].t, dw, in, split, s, &fin);
    if (r) return r;
  }
  return ok();
}

int snip_quantize_dual(const void* x, int64_t rows, int64_t cols, int64_t ld, int format,
                       int rounding_row, int rounding_col, uint64_t seed, uint32_t tensor_id_row,
                       uint32_t tensor_id_col, const float* amax_in, const snip_qtensor* out_row,
                       const snip_qtensor* out_col, snip_stats* stats2, void* ws, size_t ws_bytes,
                       void* stream) {
  if (!x) return fail(SNIP_E_NULL, "snip_quantize_dual: x is NULL");
  if (!dual_format(format))
    return fail(SNIP_E_FORMAT, "snip_quantize_dual: format %d is not NVFP4, FP8_E4M3 or MXFP4", format);
  if ((rounding_row != SNIP_RNE && rounding_row != SNIP_SR) || (rounding_col != SNIP_RNE && rounding_col != SNIP_SR))
    return fail(SNIP_E_FORMAT, "snip_quantize_dual: unknown rounding (%d, %d)", rounding_row, rounding_col);
  const int blk = block_of(format);
  if (rows <= 0 || cols <= 0 || rows % blk || cols % blk)
    return fail(SNIP_E_SHAPE, "snip_quantize_dual: rows=%lld cols=%lld must be positive multiples of %d",
                (long long)rows, (long long)cols, blk);
  if (ld < cols || ld % 8)
    return fail(SNIP_E_SHAPE, "snip_quantize_dual: ld=%lld must be >= cols and a multiple of 8", (long long)ld);
  int rc = validate_qtensor(out_row, "snip_quantize_dual: out_row");
  if (rc) return rc;
  rc = validate_qtensor(out_col, "snip_quantize_dual: out_col");
  if (rc) return rc;
  if (out_row->format != format || out_col->format != format)
    return fail(SNIP_E_FORMAT, "snip_quantize_dual: output formats (%d, %d) != format %d", out_row->format,
                out_col->format, format);
  if (out_row->rows != rows || out_row->k != cols || out_col->rows != cols || out_col->k != rows)
    return fail(SNIP_E_SHAPE, "snip_quantize_dual: out_row must be [%lld][%lld] and out_col [%lld][%lld]",
                (long long)rows, (long long)cols, (long long)cols, (long long)rows);
  if (!aligned(x, 16) || !aligned(amax_in, 4) || !aligned(stats2, 8) || !aligned(ws, 16))
    return fail(SNIP_E_ALIGN, "snip_quantize_dual: misaligned pointer");
  const size_t need = snip_quantize_dual_workspace(rows, cols, format);
  if (!ws || ws_bytes < need) return fail(SNIP_E_WORKSPACE, "snip_quantize_dual: workspace of %zu bytes needed", need);

  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver cv(ws);
  uint32_t* apart = reinterpret_cast<uint32_t*>(cv.take(kAmaxBytes));
  StatPart* prow = reinterpret_cast<StatPart*>(cv.take(kPartBytes));
  StatPart* pcol = reinterpret_cast<StatPart*>(cv.take(kPartBytes));
  DPlan p{};
  p.x = static_cast<const uint16_t*>(x);
  p.rows = rows;
  p.cols = cols;
  p.ld = ld;
  p.format = format;
  p.sr_row = rounding_row == SNIP_SR;
  p.sr_col = rounding_col == SNIP_SR;
  p.seed = seed;
  p.amax_in = amax_in;
  p.row = dout_of(*out_row, prow, tensor_id_row);
  p.col = dout_of(*out_col, pcol, tensor_id_col);
  p.stats_row = stats2 ? stats2 + 0 : nullptr;
  p.stats_col = stats2 ? stats2 + 1 : nullptr;
  p.nwg = dual_wg(format, rows, cols);
  if (needs_amax(format) && !amax_in) {
    APlan a{p.x, rows, cols, ld, apart, amax_wg(rows, cols)};
    rc = run_amax(&a, 1, s);
    if (rc) return rc;
    p.amax_part = apart;
    p.n_amax_part = a.nwg;
  }
  const DPlan* grp[1] = {&p};
  rc = run_dual_group(grp, 1, s);
  if (rc) return rc;
  if (stats2) {
    rc = run_finalize_dual(grp, 1, s);
    if (rc) return rc;
  }
  return ok();
}

}  // extern "C"

namespace {

// snip_linear_fwd_save and its allocation-free variant. `who` names the entry
// point in error messages; check_only: validate every argument (all on the
// host: no HIP call) and return; noalloc: the workspace is the library's
// static scratch array (its size is the one that must fit).
int linear_fwd_save_impl(const char* who, const void* x, const void* w, int64_t T, int64_t in, int64_t out,
                         int format, uint64_t seed, uint32_t layer_id, const float* amax_x, const float* amax_w,
                         float* y, const snip_qtensor* wt, const snip_qtensor* xt, snip_stats* stats4, void* ws,
                         size_t ws_bytes, void* stream, bool check_only, bool noalloc) {
  if (!x || !w || !y) return fail(SNIP_E_NULL, "%s: x, w and y must be non-NULL", who);
  if (!dual_format(format))
    return fail(SNIP_E_FORMAT, "%s: format %d is not NVFP4, FP8_E4M3 or MXFP4", who, format);
  if (T <= 0 || in <= 0 || out <= 0 || T % 128 || in % 128 || out % 128)
    return fail(SNIP_E_SHAPE, "%s: T=%lld in=%lld out=%lld must be positive multiples of 128", who,
                (long long)T, (long long)in, (long long)out);
  int rc = gemm_operands_fit(format, T, out, in, who);
  if (!rc) rc = gemm_operands_fit(format, T, in, out, who);
  if (!rc) rc = gemm_operands_fit(format, out, in, T, who);
  if (rc) return rc;
  char what[160];
  std::snprintf(what, sizeof(what), "%s: wt", who);
  rc = validate_qtensor(wt, what);
  if (rc) return rc;
  std::snprintf(what, sizeof(what), "%s: xt", who);
  rc = validate_qtensor(xt, what);
  if (rc) return rc;
  if (wt->format != format || xt->format != format)
    return fail(SNIP_E_FORMAT, "%s: wt/xt formats (%d, %d) != format %d", who, wt->format, xt->format, format);
  if (wt->rows != in || wt->k != out || xt->rows != in || xt->k != T)
    return fail(SNIP_E_SHAPE, "%s: wt must be [%lld][%lld] and xt [%lld][%lld]", who, (long long)in,
                (long long)out, (long long)in, (long long)T);
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16) || !aligned(stats4, 8) || !aligned(ws, 16) ||
      !aligned(amax_x, 4) || !aligned(amax_w, 4))
    return fail(SNIP_E_ALIGN, "%s: misaligned pointer", who);
  const size_t need = snip_linear_fwd_save_workspace(T, in, out, format);
  if (noalloc && need > ws_bytes)
    return fail(SNIP_E_WORKSPACE, "%s: this layer needs %zu bytes of scratch, more than the %zu bytes of the "
                "library's static scratch array; use snip_linear_fwd_save with a caller workspace", who, need,
                ws_bytes);
  if (!ws || ws_bytes < need) return fail(SNIP_E_WORKSPACE, "%s: workspace of %zu bytes needed", who, need);
  if (check_only) return SNIP_OK;

  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver cv(ws);
  uint32_t* apx = reinterpret_cast<uint32_t*>(cv.take(kAmaxBytes));
  uint32_t* apw = reinterpret_cast<uint32_t*>(cv.take(kAmaxBytes));
  StatPart* part[4];
  for (int i = 0; i < 4; ++i) part[i] = reinterpret_cast<StatPart*>(cv.take(kPartBytes));
  QBuf qx = carve_q(cv, format, T, in);
  QBuf qw = carve_q(cv, format, out, in);
  const size_t split_bytes = gemm_partial_bytes(format, T, out, in);
  float* split = split_bytes ? reinterpret_cast<float*>(cv.take(split_bytes)) : nullptr;

  const uint16_t* xs = static_cast<const uint16_t*>(x);
  const uint16_t* wsrc = static_cast<const uint16_t*>(w);
  // X: row-wise RNE (forward A, id 8L+0) + column-wise SR (wgrad B, id 8L+5)
  // W: row-wise RNE (forward B, id 8L+1) + column-wise SR (dgrad B, id 8L+3)
  DPlan px{}, pw{};
  px.x = xs;
  px.rows = T;
  px.cols = in;
  px.ld = in;
  px.row = dout_of(qx.t, part[0], 8u * layer_id + 0u);
  px.col = dout_of(*xt, part[3], 8u * layer_id + 5u);
  px.stats_row = stats4 ? stats4 + 0 : nullptr;
  px.stats_col = stats4 ? stats4 + 3 : nullptr;
  pw.x = wsrc;
  pw.rows = out;
  pw.cols = in;
  pw.ld = in;
  pw.row = dout_of(qw.t, part[1], 8u * layer_id + 1u);
  pw.col = dout_of(*wt, part[2], 8u * layer_id + 3u);
  pw.stats_row = stats4 ? stats4 + 1 : nullptr;
  pw.stats_col = stats4 ? stats4 + 2 : nullptr;
  px.amax_in = amax_x;
  pw.amax_in = amax_w;
  for (DPlan* p : {&px, &pw}) {
    p->format = format;
    p->sr_row = false;
    p->sr_col = true;
    p->seed = seed;
    p->nwg = dual_wg(format, p->rows, p->cols);
  }
  if (needs_amax(format)) {
    // the tensor-max pre-pass of every tensor without a supplied max
    APlan a[2];
    DPlan* of[2];
    uint32_t* dst[2] = {apx, apw};
    int na = 0;
    for (DPlan* p : {&px, &pw}) {
      if (p->amax_in) continue;
      a[na] = APlan{p->x, p->rows, p->cols, p->ld, dst[na], amax_wg(p->rows, p->cols)};
      of[na++] = p;
    }
    if (na) {
      rc = run_amax(a, na, s);
      if (rc) return rc;
      for (int i = 0; i < na; ++i) {
        of[i]->amax_part = a[i].part;
        of[i]->n_amax_part = a[i].nwg;
      }
    }
  }
  const DPlan* grp[2] = {&px, &pw};
  rc = run_dual_group(grp, 2, s);
  if (rc) return rc;
  const FJobs fin = fjobs_of_dual(grp, 2);      // empty when stats4 is NULL
  rc = gemm_q(qx.t, qw.t, y, out, split, s, &fin);
  if (rc) return rc;
  return ok();
}

// ---------------------------------------------------------------- static scratch
// Scratch of the allocation-free entry point: device memory the library
// holds on every GPU it runs on until the process ends. In host code
// `scratch` names a host-side stand-in, not a device address: its device
// address on each GPU comes from hipGetSymbolAddress, taken once per device
// with that device current, and only that address is passed to kernels.
constexpr size_t kScratchBytes = SNIP_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch granularity");
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the device that runs `stream` (the
// current device for the null stream).
int scratch_for(hipStream_t stream, void** out) {
  int dev = 0;
  int rc = stream ? hip_check(hipStreamGetDevice(stream, &dev), "hipStreamGetDevice")
                  : hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (rc) return rc;
  if (dev < 0 || dev >= kMaxDevices) return fail(SNIP_E_HIP, "device %d outside 0..%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    int cur = 0;
    if ((rc = hip_check(hipGetDevice(&cur), "hipGetDevice"))) return rc;
    if (cur != dev && (rc = hip_check(hipSetDevice(dev), "hipSetDevice"))) return rc;
    void* p = nullptr;
    rc = hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (cur != dev) {
      const int rc2 = hip_check(hipSetDevice(cur), "hipSetDevice");
      if (!rc) rc = rc2;
    }
    if (rc) return rc;
    if (!p || !aligned(p, 256)) return fail(SNIP_E_HIP, "scratch array at a bad device address %p", p);
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return SNIP_OK;
}

}  // namespace

extern "C" {

int snip_linear_fwd_save(const void* x, const void* w, int64_t T, int64_t in, int64_t out, int format,
                         uint64_t seed, uint32_t layer_id, const float* amax_x, const float* amax_w, float* y,
                         const snip_qtensor* wt, const snip_qtensor* xt, snip_stats* stats4, void* ws,
                         size_t ws_bytes, void* stream) {
  return linear_fwd_save_impl("snip_linear_fwd_save", x, w, T, in, out, format, seed, layer_id, amax_x, amax_w,
                              y, wt, xt, stats4, ws, ws_bytes, stream, false, false);
}

int snip_linear_fwd_save_noalloc(const void* x, const void* w, int64_t T, int64_t in, int64_t out, int format,
                                 uint64_t seed, uint32_t layer_id, const float* amax_x, const float* amax_w,
                                 float* y, const snip_qtensor* wt, const snip_qtensor* xt, snip_stats* stats4,
                                 void* stream) {
  const char* who = "snip_linear_fwd_save_noalloc";
  // every argument, the scratch size included, is checked before any HIP
  // call (a 256-aligned stand-in marks the workspace as present)
  void* const present = reinterpret_cast<void*>(uintptr_t(256));
  int rc = linear_fwd_save_impl(who, x, w, T, in, out, format, seed, layer_id, amax_x, amax_w, y, wt, xt, stats4,
                                present, kScratchBytes, stream, true, true);
  if (rc) return rc;
  void* p = nullptr;
  rc = scratch_for(static_cast<hipStream_t>(stream), &p);
  if (rc) return rc;
  return linear_fwd_save_impl(who, x, w, T, in, out, format, seed, layer_id, amax_x, amax_w, y, wt, xt, stats4, p,
                              kScratchBytes, stream, false, true);
}

int snip_linear_bwd_saved(const void* dy, const snip_qtensor* wt, const snip_qtensor* xt, int64_t T,
                          int64_t in, int64_t out, uint64_t seed, uint32_t layer_id, const float* amax_dy,
                          float* dx, float* dw, snip_stats* stats2, void* ws, size_t ws_bytes, void* stream) {
  if (!dy) return fail(SNIP_E_NULL, "snip_linear_bwd_saved: dy is NULL");
  int rc = validate_qtensor(wt, "snip_linear_bwd_saved: wt");
  if (rc) return rc;
  rc = validate_qtensor(xt, "snip_linear_bwd_saved: xt");
  if (rc) return rc;
  const int format = wt->format;
  if (!dual_format(format) || xt->format != format)
    return fail(SNIP_E_FORMAT, "snip_linear_bwd_saved: wt/xt formats (%d, %d) must match and be quantized",
                wt->format, xt->format);
  if (T <= 0 || in <= 0 || out <= 0 || T % 128 || in % 128 || out % 128)
    return fail(SNIP_E_SHAPE, "snip_linear_bwd_saved: T=%lld in=%lld out=%lld must be positive multiples of 128",
                (long long)T, (long long)in, (long long)out);
  if (wt->rows != in || wt->k != out || xt->rows != in || xt->k != T)
    return fail(SNIP_E_SHAPE, "snip_linear_bwd_saved: wt must be [%lld][%lld] and xt [%lld][%lld]", (long long)in,
                (long long)out, (long long)in, (long long)T);
  rc = gemm_operands_fit(format, T, in, out, "snip_linear_bwd_saved (dgrad)");
  if (!rc) rc = gemm_operands_fit(format, out, in, T, "snip_linear_bwd_saved (wgrad)");
  if (rc) return rc;
  if (!aligned(dy, 16) || !aligned(dx, 16) || !aligned(dw, 16) || !aligned(stats2, 8) || !aligned(ws, 16) ||
      !aligned(amax_dy, 4))
    return fail(SNIP_E_ALIGN, "snip_linear_bwd_saved: misaligned pointer");
  const size_t need = snip_linear_bwd_saved_workspace(T, in, out, format);
  if (!ws || ws_bytes < need)
    return fail(SNIP_E_WORKSPACE, "snip_linear_bwd_saved: workspace of %zu bytes needed", need);
  if (!dx && !dw) return ok();

  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver cv(ws);
  uint32_t* ap = reinterpret_cast<uint32_t*>(cv.take(kAmaxBytes));
  StatPart* prow = reinterpret_cast<StatPart*>(cv.take(kPartBytes));
  StatPart* pcol = reinterpret_cast<StatPart*>(cv.take(kPartBytes));
  QBuf qr = carve_q(cv, format, T, out);      // dY row-wise  [T][out]  (dgrad A)
  QBuf qc = carve_q(cv, format, out, T);      // dY column-wise [out][T] (wgrad A)
  const size_t split_bytes = std::max(gemm_partial_bytes(format, T, in, out), gemm_partial_bytes(format, out, in, T));
  float* split = split_bytes ? reinterpret_cast<float*>(cv.take(split_bytes)) : nullptr;
  const uint16_t* dys = static_cast<const uint16_t*>(dy);
  int n_ap = 0;
  if (needs_amax(format) && !amax_dy) {
    APlan a{dys, T, out, out, ap, amax_wg(T, out)};
    rc = run_amax(&a, 1, s);
    if (rc) return rc;
    n_ap = a.nwg;
  }
  if (dx && dw) {       // both layouts from one read of dY
    DPlan p{};
    p.x = dys;
    p.rows = T;
    p.cols = out;
    p.ld = out;
    p.format = format;
    p.sr_row = true;
    p.sr_col = true;
    p.seed = seed;
    p.amax_in = amax_dy;
    p.amax_part = n_ap ? ap : nullptr;
    p.n_amax_part = n_ap;
    p.row = dout_of(qr.t, prow, 8u * layer_id + 2u);
    p.col = dout_of(qc.t, pcol, 8u * layer_id + 4u);
    p.stats_row = stats2 ? stats2 + 0 : nullptr;
    p.stats_col = stats2 ? stats2 + 1 : nullptr;
    p.nwg = dual_wg(format, T, out);
    const DPlan* grp[1] = {&p};
    rc = run_dual_group(grp, 1, s);
    if (rc) return rc;
    const FJobs fin = fjobs_of_dual(grp, 1);
    rc = gemm_q_pair(qr.t, *wt, dx, in, qc.t, *xt, dw, in, split, s, &fin);
    if (rc) return rc;
    return ok();
  }
  // one GEMM only: the one layout it needs
  const bool row = dx != nullptr;
  QPlan p{};
  p.x = dys;
  p.rows = T;
  p.cols = out;
  p.ld = out;
  p.layout = row ? SNIP_ROWWISE : SNIP_COLWISE;
  p.format = format;
  p.sr = true;
  p.seed = seed;
  p.tensor_id = 8u * layer_id + (row ? 2u : 4u);
  p.amax_in = amax_dy;
  p.amax_part = n_ap ? ap : nullptr;
  p.n_amax_part = n_ap;
  const snip_qtensor& q = row ? qr.t : qc.t;
  p.codes = static_cast<uint8_t*>(q.codes);
  p.scales = static_cast<uint8_t*>(q.scales);
  p.texp = has_texp(format) ? q.tensor_exp : nullptr;
  p.part = row ? prow : pcol;
  p.nwg = quant_wg(p.layout, format, T, out);
  p.stats = stats2 ? stats2 + (row ? 0 : 1) : nullptr;
  const QPlan* grp[1] = {&p};
  rc = run_quant_group(grp, 1, s);
  if (rc) return rc;
  const FJobs fin = fjobs_of(grp, 1);
  rc = row ? gemm_q(qr.t, *wt, dx, in, split, s, &fin) : gemm_q(qc.t, *xt, dw, in, split, s, &fin);
  if (rc) return rc;
  return ok();
}

int snip_layer_stats(const snip_stats* dev_stats, int n, snip_tensor_report* host_out, void* stream) {
  if (!dev_stats || !host_out) return fail(SNIP_E_NULL, "snip_layer_stats: NULL pointer");
  if (n <= 0 || n > 4096) return fail(SNIP_E_SHAPE, "snip_layer_stats: n=%d out of range", n);
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::vector<snip_stats> tmp((size_t)n);
  int r = hip_check(hipMemcpyAsync(tmp.data(), dev_stats, sizeof(snip_stats) * n, hipMemcpyDeviceToHost, s),
                    "stats copy");
  if (r) return r;
  r = hip_check(hipStreamSynchronize(s), "stream sync");
  if (r) return r;
  bool nonfinite = false;
  for (int i = 0; i < n; ++i) {
    const snip_stats& st = tmp[i];
    snip_tensor_report& o = host_out[i];
    o.sum_err2 = st.sum_err2;
    o.sum_x2 = st.sum_x2;
    o.rel_mse = st.sum_x2 > 0 ? st.sum_err2 / st.sum_x2 : (st.sum_err2 == 0 ? 0.0 : INFINITY);
    o.norm_ratio = st.sum_err2 > 0 ? std::sqrt(st.sum_x2) / std::sqrt(st.sum_err2) : INFINITY;
    o.amax = st.amax;
    o.n_nonfinite = st.n_nonfinite;
    o.below_sqrt3 = st.sum_x2 < 3.0 * st.sum_err2 ? 1 : 0;
    o.reserved = 0;
    nonfinite = nonfinite || st.n_nonfinite > 0;
  }
  if (nonfinite) return fail(SNIP_E_NONFINITE, "snip_layer_stats: non-finite inputs counted");
  return ok();
}

}  // extern "C"

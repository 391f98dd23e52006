// C ABI of the library: argument validation, workspace layout and the
// sequence of kernel launches behind each entry point declared in qat.h.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/qat.h"
#include "common.h"
#include "launch.h"

#define QAT_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return QAT_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(QAT_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool pow2_dc(int64_t d_c) { return d_c == 32 || d_c == 64 || d_c == 128 || d_c == 256; }

// ---------------------------------------------------------------- ESA
struct EsaLayout {
  int nsplit_q = 1, nkeysplit = 1, nqsplit = 1, nscan = 1, ndec = 1;
  int64_t n_mid = 0, mid0 = 0, rows = 0;
  double* qpart = nullptr;
  float* qc = nullptr;
  qat::bf16* qhi = nullptr;
  qat::bf16* qlo = nullptr;
  float* rowmax_part = nullptr;
  float* rowsum_part = nullptr;
  float* rowmax = nullptr;
  float* upart = nullptr;
  float* sraw = nullptr;
  float* smax = nullptr;
  float* ssum = nullptr;
  int32_t* tk_hist = nullptr;
  int2* tk_cnt = nullptr;
  uint32_t* keys = nullptr;
  float* po = nullptr;
  float* pm = nullptr;
  float* pl = nullptr;
  int32_t* keylist = nullptr;
  size_t bytes = 0;
};

int esa_check(const qat_esa_params* p) {
  if (!p) return fail(QAT_EINVAL, "params is NULL");
  if (p->batch < 1 || p->n_heads < 1) return fail(QAT_EINVAL, "batch and n_heads must be >= 1");
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(QAT_EUNSUPPORTED, "head_dim %lld not supported (64 or 128)", (long long)p->head_dim);
  if (p->per_head != 0 && p->per_head != 1) return fail(QAT_EINVAL, "per_head must be 0 or 1");
  if (!p->per_head && !pow2_dc(p->d_c))
    return fail(QAT_EUNSUPPORTED, "d_c %lld not supported (32, 64, 128, 256)", (long long)p->d_c);
  if (p->ctx_len < 1 || p->ctx_len >= (1ll << 31)) return fail(QAT_EINVAL, "ctx_len out of range");
  if (p->chunk_start < 0 || p->chunk_len < 1 || p->chunk_start + p->chunk_len > p->ctx_len)
    return fail(QAT_EINVAL, "chunk [%lld, %lld) outside the cache of %lld rows", (long long)p->chunk_start,
                (long long)(p->chunk_start + p->chunk_len), (long long)p->ctx_len);
  if (p->n_init < 0 || p->window < 0 || p->radius < 0) return fail(QAT_EINVAL, "n_init, window, radius must be >= 0");
  if (p->radius > qat::esa_topk_max_radius())
    return fail(QAT_EUNSUPPORTED, "radius %d above the supported %d", p->radius, qat::esa_topk_max_radius());
  if (p->topk < 1) return fail(QAT_EINVAL, "topk must be >= 1");
  if (p->correction != QAT_CORR_CLAMP && p->correction != QAT_CORR_VOTES)
    return fail(QAT_EINVAL, "unknown correction %d", p->correction);
  if (p->correction == QAT_CORR_CLAMP && !(p->clip > 0.f)) return fail(QAT_EINVAL, "clip must be > 0 (or +inf)");
  if (p->correction == QAT_CORR_VOTES && !std::isfinite(p->vote_tau))
    return fail(QAT_EINVAL, "vote_tau must be finite");
  if (!std::isfinite(p->scale) || !(p->scale > 0.f)) return fail(QAT_EINVAL, "scale must be finite and > 0");
  if (p->dtype != QAT_F32 && p->dtype != QAT_BF16) return fail(QAT_EINVAL, "unknown dtype %d", p->dtype);
  if (p->batch * p->chunk_len * p->n_heads >= (1ll << 31)) return fail(QAT_EUNSUPPORTED, "too many query rows");
  if (p->per_head && p->dtype != QAT_BF16) return fail(QAT_EUNSUPPORTED, "per-head selection takes bfloat16 inputs");
  if (p->per_head && p->ctx_len * p->n_heads * p->head_dim >= (1ll << 31))
    return fail(QAT_EUNSUPPORTED, "per-head selection: one sequence's cache must hold fewer than 2^31 elements");
  return QAT_OK;
}

EsaLayout esa_layout(const qat_esa_params* p, void* ws) {
  EsaLayout L;
  // B: selections (one per sequence, or one per (sequence, head))
  const int64_t B = p->per_head ? p->batch * p->n_heads : p->batch, m = p->chunk_len, c0 = p->chunk_start;
  L.rows = B * m;
  L.mid0 = p->n_init;
  L.n_mid = c0 > p->n_init ? std::max<int64_t>(p->n_init, c0 - p->window) - p->n_init : 0;
  const int64_t D = p->n_heads * p->head_dim;
  L.nsplit_q = p->per_head ? 0 : qat::compress_splits(L.rows, D, p->d_c);
  const int64_t dcq = p->per_head ? 0 : p->d_c;   // per head: no compressed queries
  L.nkeysplit = qat::esa_key_splits(L.n_mid > 0 ? L.n_mid : 1, m);
  L.nqsplit = qat::esa_prefill_qsplits_eff(L.n_mid > 0 ? L.n_mid : 1, m);
  L.nscan = qat::esa_scan_wgs(L.n_mid > 0 ? L.n_mid : 1);
  L.ndec = qat::esa_decode_splits(p->batch, p->n_init, p->topk, p->window);
  qat::Carver c(ws);
  L.qpart = c.take<double>((size_t)L.nsplit_q * L.rows * dcq);
  L.qc = c.take<float>((size_t)L.rows * dcq);
  L.qhi = c.take<qat::bf16>((size_t)L.rows * dcq);
  L.qlo = c.take<qat::bf16>((size_t)L.rows * dcq);
  const size_t nm = (size_t)(L.n_mid > 0 ? L.n_mid : 1);
  if (m > 1) {
    L.rowmax_part = c.take<float>((size_t)L.rows * L.nkeysplit);
    L.rowsum_part = c.take<float>((size_t)L.rows * L.nkeysplit);
    L.rowmax = c.take<float>((size_t)L.rows);
    L.upart = c.take<float>((size_t)B * L.nqsplit * nm);
  } else {
    L.sraw = c.take<float>((size_t)B * nm);
    L.smax = c.take<float>((size_t)B * L.nscan);
    L.ssum = c.take<float>((size_t)B * L.nscan);
  }
  L.tk_hist = c.take<int32_t>((size_t)B * 3 * 2048);
  L.tk_cnt = c.take<int2>((size_t)B * qat::esa_topk_slices((int64_t)nm));
  L.keys = c.take<uint32_t>((size_t)B * nm);
  L.keylist = c.take<int32_t>((size_t)B * qat::esa_keylist_len(p->n_init, p->topk, p->window, m));
  if (m == 1) {
    L.po = c.take<float>((size_t)p->batch * L.ndec * D);
    L.pm = c.take<float>((size_t)p->batch * L.ndec * p->n_heads);
    L.pl = c.take<float>((size_t)p->batch * L.ndec * p->n_heads);
  }
  L.bytes = c.bytes();
  return L;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return QAT_OK;
  if (!ws) return fail(QAT_EWORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (((uintptr_t)ws) & 255) return fail(QAT_EWORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < need) return fail(QAT_EWORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  return QAT_OK;
}

// ---------------------------------------------------------------- MoBA
struct MobaLayout {
  int64_t nbc = 0, nrows = 0, nbuckets = 0, max_tiles = 0;
  double* mp_part = nullptr;
  float* kbar = nullptr;
  qat::bf16* kplanes = nullptr;
  int32_t* counts = nullptr;
  int32_t* offsets = nullptr;
  int32_t* cursor = nullptr;
  int2* entries = nullptr;
  int4* tiles = nullptr;
  int32_t* ntiles = nullptr;
  void* part_o = nullptr;
  float* part_lse = nullptr;
  bool decode = false;        // few rows, no window: split-key kernels
  int dec_pieces = 0;
  float* dec_po = nullptr;    // [rows, dec_pieces, d] piece outputs
  float* dec_plse = nullptr;  // [rows, dec_pieces] piece log-sum-exps
  float* delta = nullptr;     // [rows] D = sum_j p_j dp_j of the gradient pass
  float* dq_part = nullptr;   // gradient pass: float32 dq partials per (row, gated slot)
  int32_t* run_off = nullptr; // gradient pass: runs of dispatch tiles per bucket
  int32_t* wg_counts = nullptr;   // gradient pass: stable dispatch, per-workgroup bucket counts
  int32_t* wg_base = nullptr;     // gradient pass: stable dispatch, per-workgroup bucket offsets
  int32_t* wg_loc = nullptr;      // forward: per-workgroup bucket counts of the atomic placement
  float* kv_part = nullptr;   // gradient pass: dK, dV sums per (run, key chunk)
  size_t bytes = 0;
};

// Few query rows per (sequence, head) and no extra window: the split-key
// kernels (one wave per row and piece of up to 256 keys) replace the tiled
// ones, whose tiles would hold one or two rows.
constexpr int64_t kMobaDecodeMaxQ = 8;
constexpr int kMobaDecodeMaxPieces = 64;

int moba_check(const qat_moba_params* p) {
  if (!p) return fail(QAT_EINVAL, "params is NULL");
  if (p->batch < 1 || p->seq_len < 1 || p->n_q_heads < 1 || p->n_kv_heads < 1)
    return fail(QAT_EINVAL, "batch, seq_len and head counts must be >= 1");
  if (p->n_q_heads % p->n_kv_heads) return fail(QAT_EINVAL, "n_kv_heads must divide n_q_heads");
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(QAT_EUNSUPPORTED, "head_dim %lld not supported (64 or 128)", (long long)p->head_dim);
  if (p->seq_len >= (1ll << 31)) return fail(QAT_EUNSUPPORTED, "seq_len too large");
  if (p->q_start < 0 || p->q_len < 1 || p->q_start + p->q_len > p->seq_len)
    return fail(QAT_EINVAL, "query rows [%lld, %lld) outside the sequence of %lld", (long long)p->q_start,
                (long long)(p->q_start + p->q_len), (long long)p->seq_len);
  if (p->block < 1) return fail(QAT_EINVAL, "block must be >= 1");
  if (p->topk < 1 || p->topk > 16) return fail(QAT_EINVAL, "topk must be in 1..16");
  if (p->window < 0) return fail(QAT_EINVAL, "window must be >= 0");
  if (!std::isfinite(p->scale) || !(p->scale > 0.f)) return fail(QAT_EINVAL, "scale must be finite and > 0");
  if (p->dtype != QAT_F32 && p->dtype != QAT_BF16) return fail(QAT_EINVAL, "unknown dtype %d", p->dtype);
  if (p->batch * p->q_len * p->n_q_heads >= (1ll << 27)) return fail(QAT_EUNSUPPORTED, "too many query rows");
  if (p->batch * p->seq_len * p->n_q_heads >= (1ll << 31)) return fail(QAT_EUNSUPPORTED, "q holds too many rows");
  // one block's K (or V) rows are addressed with 32-bit byte offsets
  if ((int64_t)p->block * p->n_kv_heads * p->head_dim * 4 >= (1ll << 31))
    return fail(QAT_EUNSUPPORTED, "block * n_kv_heads * head_dim too large");
  return QAT_OK;
}

MobaLayout moba_layout(const qat_moba_params* p, void* ws, bool bwd = false) {
  MobaLayout L;
  L.nbc = p->seq_len / p->block;
  L.nrows = p->batch * p->q_len * p->n_q_heads;
  L.nbuckets = p->batch * p->n_kv_heads * L.nbc;
  L.max_tiles = qat::moba_max_tiles(L.nrows, p->topk, L.nbuckets);
  const int64_t cols = p->n_kv_heads * p->head_dim;
  const size_t esz = p->dtype == QAT_BF16 ? 2 : 4;
  qat::Carver c(ws);
  L.mp_part = c.take<double>((size_t)p->batch * L.nbc * qat::meanpool_splits(p->block) * cols);
  L.kbar = c.take<float>((size_t)p->batch * L.nbc * cols);
  L.kplanes = c.take<qat::bf16>((size_t)3 * p->batch * L.nbc * cols);
  L.counts = c.take<int32_t>((size_t)L.nbuckets + 1);
  L.offsets = c.take<int32_t>((size_t)L.nbuckets + 1);
  L.cursor = c.take<int32_t>((size_t)L.nbuckets + 1);
  L.entries = c.take<int2>((size_t)L.nrows * (p->topk - 1) + 1);
  L.tiles = c.take<int4>((size_t)L.max_tiles + 1);
  L.ntiles = c.take<int32_t>(1);
  L.part_o = (void*)c.take<char>((size_t)L.nrows * (p->topk - 1) * p->head_dim * esz + 1);
  L.part_lse = c.take<float>((size_t)L.nrows * (p->topk - 1) + 1);
  L.dec_pieces = qat::moba_decode_pieces(p->block, p->topk);
  L.decode = p->window == 0 && p->q_len <= kMobaDecodeMaxQ && L.dec_pieces <= kMobaDecodeMaxPieces;
  if (L.decode) {
    L.dec_po = c.take<float>((size_t)L.nrows * L.dec_pieces * p->head_dim);
    L.dec_plse = c.take<float>((size_t)L.nrows * L.dec_pieces);
  }
  L.delta = c.take<float>((size_t)L.nrows);
  if (!bwd) {
    const int64_t wi = qat::moba_dispatch_wg_ints(L.nrows, L.nbuckets);
    L.wg_loc = wi > 0 ? c.take<int32_t>((size_t)wi) : nullptr;
  }
  if (bwd) {
    L.dq_part = c.take<float>((size_t)qat::moba_bwd_part_floats(L.nrows, p->topk, p->head_dim) + 1);
    L.run_off = c.take<int32_t>((size_t)L.nbuckets + 1);
    const int64_t sti = qat::moba_dispatch_stable_ints(L.nrows, L.nbuckets, p->topk);
    L.wg_counts = sti > 0 ? c.take<int32_t>((size_t)sti) : nullptr;
    L.wg_base = sti > 0 ? c.take<int32_t>((size_t)sti) : nullptr;
    L.kv_part = c.take<float>((size_t)qat::moba_bwd_kv_part_floats(L.max_tiles, L.nbuckets, p->block, p->head_dim));
  }
  L.bytes = c.bytes();
  return L;
}

// ---------------------------------------------------------------- timing
struct TimerRec {
  std::string name;
  hipEvent_t a, b;
};
std::mutex g_tmu;
bool g_timing = false;
std::string g_timing_only;   // empty: every stage
std::vector<TimerRec> g_recs;
std::vector<hipEvent_t> g_pool;
std::map<std::string, hipEvent_t> g_open;

hipEvent_t pool_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  // timing-only events: no system-scope fence (cache write-back and
  // invalidation) when they complete, so recording them does not slow the
  // kernels they bracket; they are read only after a full synchronisation
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

namespace qat {
bool ktimer_kernel_events(const char* name, hipEvent_t* a, hipEvent_t* b) {
  if (!g_timing) return false;
  std::lock_guard<std::mutex> lk(g_tmu);
  if (g_timing_only != name) return false;
  *a = pool_event();
  *b = pool_event();
  return *a && *b;
}
void ktimer_kernel_record(const char* name, hipEvent_t a, hipEvent_t b) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_recs.push_back({name, a, b});
}
void ktimer_start(const char* name, hipStream_t s) {
  if (!g_timing) return;
  std::lock_guard<std::mutex> lk(g_tmu);
  if (!g_timing_only.empty()) return;   // one stage selected: its kernel is timed by its dispatch
  hipEvent_t e = pool_event();
  if (!e) return;
  (void)hipEventRecord(e, s);
  g_open[name] = e;
}
void ktimer_stop(const char* name, hipStream_t s) {
  if (!g_timing) return;
  std::lock_guard<std::mutex> lk(g_tmu);
  auto it = g_open.find(name);
  if (it == g_open.end()) return;
  hipEvent_t e = pool_event();
  if (!e) return;
  (void)hipEventRecord(e, s);
  g_recs.push_back({name, it->second, e});
  g_open.erase(it);
}
}  // namespace qat

// ======================================================================
QAT_EXPORT const char* qat_last_error(void) { return g_last_error.c_str(); }
QAT_EXPORT int qat_abi_version(void) { return QAT_ABI_VERSION; }

QAT_EXPORT int qat_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_timing = on != 0;
  return ok();
}

QAT_EXPORT int qat_timing_select(const char* name) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_timing_only = name ? name : "";
  return ok();
}

QAT_EXPORT int qat_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_tmu);
  for (auto& r : g_recs) {
    (void)hipEventSynchronize(r.b);
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
  return ok();
}

QAT_EXPORT int qat_timing_query(const char* name, double* total_ms, int* count) {
  if (!name || !total_ms || !count) return fail(QAT_EINVAL, "name, total_ms and count must be non-NULL");
  std::lock_guard<std::mutex> lk(g_tmu);
  double tot = 0.0;
  int n = 0;
  for (auto& r : g_recs) {
    if (r.name != name) continue;
    hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) return hip_status(e, "qat_timing_query");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) return hip_status(e, "qat_timing_query");
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *count = n;
  return ok();
}

// ---------------------------------------------------------------- ESA
QAT_EXPORT int esa_workspace_size(const qat_esa_params* p, size_t* bytes) {
  int rc = esa_check(p);
  if (rc) return rc;
  if (!bytes) return fail(QAT_EINVAL, "bytes is NULL");
  *bytes = esa_layout(p, nullptr).bytes;
  return ok();
}

QAT_EXPORT int esa_compress_workspace_size(int64_t n, int64_t d_model, int64_t d_c, size_t* bytes) {
  if (!bytes) return fail(QAT_EINVAL, "bytes is NULL");
  if (n < 1 || d_model < 32 || d_model % 32 || !pow2_dc(d_c))
    return fail(QAT_EINVAL, "bad compression shape n=%lld d_model=%lld d_c=%lld", (long long)n,
                (long long)d_model, (long long)d_c);
  qat::Carver c(nullptr);
  c.take<double>((size_t)qat::compress_splits(n, d_model, d_c) * n * d_c);
  *bytes = c.bytes();
  return ok();
}

QAT_EXPORT int esa_compress(const void* x, int64_t n, int64_t x_stride, int64_t d_model, int32_t in_dtype,
                            const void* W, const float* bias, int64_t d_c, void* out, int64_t out_stride,
                            int32_t out_dtype, void* ws, size_t ws_bytes, void* stream) {
  if (!x || !W || !out) return fail(QAT_EINVAL, "x, W and out must be non-NULL");
  if (n < 1 || d_model < 32 || d_model % 32) return fail(QAT_EINVAL, "n >= 1 and d_model a multiple of 32 required");
  if (!pow2_dc(d_c)) return fail(QAT_EUNSUPPORTED, "d_c %lld not supported", (long long)d_c);
  if (x_stride < d_model || out_stride < d_c) return fail(QAT_EINVAL, "row strides shorter than the rows");
  if (x_stride % 8 || ((uintptr_t)x | (uintptr_t)W) % 16)
    return fail(QAT_EINVAL, "x and W must be 16-byte aligned and x_stride a multiple of 8 elements");
  if ((in_dtype != QAT_F32 && in_dtype != QAT_BF16) || (out_dtype != QAT_F32 && out_dtype != QAT_BF16))
    return fail(QAT_EINVAL, "unknown dtype");
  size_t need = 0;
  esa_compress_workspace_size(n, d_model, d_c, &need);
  int rc = check_ws(ws, ws_bytes, need);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  const int ns = qat::compress_splits(n, d_model, d_c);
  const bool bf = in_dtype == QAT_BF16;
  qat::KTimer tm("esa_compress", s);
  hipError_t e = qat::launch_compress_partial(x, n, x_stride, d_model, bf, W, bf, d_c, ns, (double*)ws, s);
  if (e == hipSuccess)
    e = qat::launch_compress_finalize((const double*)ws, ns, n, d_c, bias, out, out_stride,
                                      out_dtype == QAT_BF16 ? 1 : 0, nullptr, nullptr, s);
  return hip_status(e, "esa_compress");
}

// Scoring, correction, importance, neighbour step and top-k of nsel
// selections whose operands ScGeom g places (shared by the merged and the
// per-head selection). q_hi / q_lo: bf16 query rows for the prefill passes
// (q_lo NULL: one exact term); q_dec: the decode query rows (float32, or
// bfloat16 when dec_bf16).
static int esa_score_and_select(const qat_esa_params* p, const EsaLayout& L, const qat::bf16* q_hi,
                                const qat::bf16* q_lo, const void* q_dec, bool dec_bf16, const qat::bf16* kc,
                                const qat::ScGeom& g, int64_t nsel, int64_t dc, float tau, int32_t* sel,
                                int32_t* n_sel, float* scores, hipStream_t s) {
  // votes: temperature in log2 units (exp(tau x) = exp2(tau log2(e) x))
  const bool votes = p->correction == QAT_CORR_VOTES;
  const float tau2 = votes ? tau * 1.4426950408889634f : 0.f;
  hipError_t e;
  int mode;
  // the scoring kernels also clear the top-k histograms (n_mid > 0: they run)
  const int64_t nhist = nsel * 3 * 2048;
  if (p->chunk_len > 1) {
    mode = 0;
    qat::KTimer tm("esa_scores", s);
    e = qat::launch_esa_prefill_scores(q_hi, q_lo, kc, g, nsel, p->chunk_len, L.mid0, L.n_mid, dc, p->clip, tau2,
                                       L.rowmax_part, L.rowsum_part, L.rowmax, L.upart, L.tk_hist, nhist, s);
  } else {
    mode = votes ? 2 : 1;
    qat::KTimer tm("esa_decode_scan", s);
    e = qat::launch_esa_decode_scan(q_dec, dec_bf16, kc, g, nsel, L.mid0, L.n_mid, dc, tau2, L.sraw, L.smax, L.ssum,
                                    L.tk_hist, nhist, s);
  }
  if (e != hipSuccess) return hip_status(e, "esa selection: scoring");
  qat::KTimer tm("esa_topk", s);
  e = qat::launch_esa_topk(mode, L.upart, L.nqsplit, L.sraw, L.smax, L.ssum, L.nscan, p->clip, tau2, nsel, L.n_mid,
                           p->radius, p->topk, L.mid0, L.tk_hist, L.tk_cnt, L.keys, scores, sel, n_sel, true, s);
  return hip_status(e, "esa selection: top-k");
}

QAT_EXPORT int esa_select(const qat_esa_params* p, const void* q, const void* Wq, const float* bq,
                          const void* kc_cache, int32_t* sel, int32_t* n_sel, float* scores, void* ws,
                          size_t ws_bytes, void* stream) {
  int rc = esa_check(p);
  if (rc) return rc;
  if (p->per_head) return fail(QAT_EINVAL, "esa_select merges the heads: per_head must be 0 (esa_select_heads)");
  if (!q || !Wq || !kc_cache || !sel || !n_sel) return fail(QAT_EINVAL, "q, Wq, kc_cache, sel, n_sel must be non-NULL");
  if (((uintptr_t)q | (uintptr_t)Wq | (uintptr_t)kc_cache) % 16)
    return fail(QAT_EINVAL, "q, Wq and kc_cache must be 16-byte aligned");
  EsaLayout L = esa_layout(p, nullptr);
  if ((rc = check_ws(ws, ws_bytes, L.bytes))) return rc;
  L = esa_layout(p, ws);
  hipStream_t s = (hipStream_t)stream;
  const bool bf = p->dtype == QAT_BF16;
  const int64_t D = p->n_heads * p->head_dim;
  // q~ = Wq concat_h(q) + bq -> float32 + hi/lo bf16: a chunk's rows on the
  // bf16 matrix cores (float32 accumulation), decode rows in float64
  hipError_t e;
  {
    qat::KTimer tm("esa_qcompress", s);
    if (bf && qat::compress_bf16_rows_ok(L.rows, D, p->d_c)) {
      e = qat::launch_compress_bf16_rows(q, L.rows, D, D, Wq, p->d_c, bq, L.qc, L.qhi, L.qlo, s);
    } else {
      e = qat::launch_compress_partial(q, L.rows, D, D, bf, Wq, bf, p->d_c, L.nsplit_q, L.qpart, s);
      if (e == hipSuccess)
        e = qat::launch_compress_finalize(L.qpart, L.nsplit_q, L.rows, p->d_c, bq, L.qc, p->d_c, 2, L.qhi, L.qlo,
                                          s);
    }
  }
  if (e != hipSuccess) return hip_status(e, "esa_select: query compression");
  const qat::bf16* kc = (const qat::bf16*)kc_cache;
  // q~ rows [B, m, d_c], compressed cache [B, T, d_c]
  const qat::ScGeom g{p->chunk_len * p->d_c, 0, p->d_c, p->ctx_len * p->d_c, 0, p->d_c, 1};
  return esa_score_and_select(p, L, L.qhi, L.qlo, L.qc, false, kc, g, p->batch, p->d_c, p->vote_tau > 0.f
                              ? p->vote_tau : 1.f / std::sqrt((float)p->d_c), sel, n_sel, scores, s);
}

QAT_EXPORT int esa_select_heads(const qat_esa_params* p, const void* q, const void* k_cache, int32_t* sel,
                                int32_t* n_sel, float* scores, void* ws, size_t ws_bytes, void* stream) {
  int rc = esa_check(p);
  if (rc) return rc;
  if (!p->per_head) return fail(QAT_EINVAL, "esa_select_heads selects per head: per_head must be 1");
  if (!q || !k_cache || !sel || !n_sel) return fail(QAT_EINVAL, "q, k_cache, sel, n_sel must be non-NULL");
  if (((uintptr_t)q | (uintptr_t)k_cache) % 16) return fail(QAT_EINVAL, "q and k_cache must be 16-byte aligned");
  EsaLayout L = esa_layout(p, nullptr);
  if ((rc = check_ws(ws, ws_bytes, L.bytes))) return rc;
  L = esa_layout(p, ws);
  const int64_t H = p->n_heads, d = p->head_dim;
  // selection v = b H + h: q rows of head h in [B, m, H, d], K rows in [B, T, H, d]
  const qat::ScGeom g{p->chunk_len * H * d, d, H * d, p->ctx_len * H * d, d, H * d, H};
  const qat::bf16* qb = (const qat::bf16*)q;
  return esa_score_and_select(p, L, qb, nullptr, q, true, (const qat::bf16*)k_cache, g, p->batch * H, d,
                              p->vote_tau > 0.f ? p->vote_tau : 1.f / std::sqrt((float)d), sel, n_sel, scores,
                              (hipStream_t)stream);
}

QAT_EXPORT int esa_sparse_attn(const qat_esa_params* p, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* sel, const int32_t* n_sel, void* out, float* lse, void* ws,
                               size_t ws_bytes, void* stream) {
  int rc = esa_check(p);
  if (rc) return rc;
  if (!q || !k_cache || !v_cache || !sel || !n_sel || !out)
    return fail(QAT_EINVAL, "q, k_cache, v_cache, sel, n_sel, out must be non-NULL");
  EsaLayout L = esa_layout(p, nullptr);
  if ((rc = check_ws(ws, ws_bytes, L.bytes))) return rc;
  L = esa_layout(p, ws);
  hipStream_t s = (hipStream_t)stream;
  const bool bf = p->dtype == QAT_BF16;
  hipError_t e;
  const bool ph = p->per_head != 0;
  if (bf && p->chunk_len == 1 && qat::esa_decode_supported(p->n_heads, p->head_dim, ph)) {
    qat::KTimer tm("esa_decode_attn", s);
    e = qat::launch_esa_decode_attn(q, k_cache, v_cache, sel, n_sel, L.po, L.pm, L.pl, out, lse, p->batch,
                                    p->n_heads, p->head_dim, p->ctx_len, p->chunk_start, p->n_init, p->window,
                                    p->topk, p->scale, ph, s);
  } else if (bf && p->ctx_len * p->n_heads * p->head_dim < (1ll << 31)) {
    // the matrix-core kernel addresses K/V rows of one sequence with 32-bit offsets
    qat::KTimer tm("esa_prefill_attn", s);
    e = qat::launch_esa_prefill_attn(q, k_cache, v_cache, sel, n_sel, L.keylist, out, lse, p->batch, p->n_heads,
                                     p->head_dim,
                                     p->ctx_len, p->chunk_start, p->chunk_len, p->n_init, p->window, p->topk,
                                     p->scale, ph, s);
  } else if (ph) {
    return fail(QAT_EUNSUPPORTED, "per-head selection: no attention path for this shape");
  } else {
    qat::KTimer tm("esa_generic_attn", s);
    e = qat::launch_esa_generic(q, k_cache, v_cache, sel, n_sel, out, lse, bf, p->batch, p->n_heads,
                                p->head_dim, p->ctx_len, p->chunk_start, p->chunk_len, p->n_init, p->window,
                                p->topk, p->scale, s);
  }
  return hip_status(e, "esa_sparse_attn");
}

QAT_EXPORT int esa_bwd_workspace_size(const qat_esa_params* p, size_t* bytes) {
  int rc = esa_check(p);
  if (rc) return rc;
  if (!bytes) return fail(QAT_EINVAL, "bytes is NULL");
  qat::Carver c(nullptr);
  const int64_t nsel = p->per_head ? p->batch * p->n_heads : p->batch;
  c.take<int32_t>((size_t)nsel * qat::esa_keylist_len(p->n_init, p->topk, p->window, p->chunk_len));
  c.take<float>((size_t)p->batch * p->chunk_len * p->n_heads);
  *bytes = c.bytes();
  return ok();
}

QAT_EXPORT int esa_sparse_attn_bwd(const qat_esa_params* p, const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* sel, const int32_t* n_sel, const void* dout, const float* lse,
                                   float* dq, float* dk, float* dv, void* ws, size_t ws_bytes, void* stream) {
  int rc = esa_check(p);
  if (rc) return rc;
  if (!q || !k_cache || !v_cache || !sel || !n_sel || !dout || !lse || !dq || !dk || !dv)
    return fail(QAT_EINVAL, "q, k_cache, v_cache, sel, n_sel, dout, lse, dq, dk, dv must be non-NULL");
  if (p->dtype != QAT_BF16) return fail(QAT_EUNSUPPORTED, "ESA gradients take bfloat16 inputs");
  if (p->ctx_len * p->n_heads * p->head_dim >= (1ll << 31))
    return fail(QAT_EUNSUPPORTED, "one sequence's cache must hold fewer than 2^31 elements");
  size_t need = 0;
  if ((rc = esa_bwd_workspace_size(p, &need))) return rc;
  if ((rc = check_ws(ws, ws_bytes, need))) return rc;
  qat::Carver c(ws);
  const int64_t nsel = p->per_head ? p->batch * p->n_heads : p->batch;
  int32_t* keylist = c.take<int32_t>((size_t)nsel * qat::esa_keylist_len(p->n_init, p->topk, p->window,
                                                                         p->chunk_len));
  float* delta = c.take<float>((size_t)p->batch * p->chunk_len * p->n_heads);
  hipError_t e = qat::launch_esa_bwd(q, k_cache, v_cache, sel, n_sel, dout, lse, keylist, dq, delta, dk, dv, p->batch,
                                     p->n_heads, p->head_dim, p->ctx_len, p->chunk_start, p->chunk_len, p->n_init,
                                     p->window, p->topk, p->scale, p->per_head != 0, (hipStream_t)stream);
  return hip_status(e, "esa_sparse_attn_bwd");
}

// ---------------------------------------------------------------- MoBA
QAT_EXPORT int moba_workspace_size(const qat_moba_params* p, size_t* bytes) {
  int rc = moba_check(p);
  if (rc) return rc;
  if (!bytes) return fail(QAT_EINVAL, "bytes is NULL");
  *bytes = moba_layout(p, nullptr).bytes;
  return ok();
}

QAT_EXPORT int moba_block_select(const qat_moba_params* p, const void* q, const void* k, int32_t* blk, void* ws,
                                 size_t ws_bytes, void* stream) {
  int rc = moba_check(p);
  if (rc) return rc;
  if (!q || !k || !blk) return fail(QAT_EINVAL, "q, k, blk must be non-NULL");
  MobaLayout L = moba_layout(p, nullptr);
  if ((rc = check_ws(ws, ws_bytes, L.bytes))) return rc;
  L = moba_layout(p, ws);
  hipStream_t s = (hipStream_t)stream;
  const bool bf = p->dtype == QAT_BF16;
  // only blocks that can be candidates of the processed rows are pooled
  const int64_t nbc_need = std::min<int64_t>(L.nbc, (p->q_start + p->q_len - 1) / p->block);
  hipError_t e = hipSuccess;
  if (p->topk > 1 && nbc_need > 0) {
    qat::KTimer tm("moba_meanpool", s);
    e = qat::launch_moba_meanpool(k, bf, p->batch, p->seq_len, p->n_kv_heads, p->head_dim, p->block, nbc_need,
                                  L.mp_part, L.kbar, bf ? L.kplanes : nullptr, s);
    if (e != hipSuccess) return hip_status(e, "moba_block_select: mean pool");
  }
  qat::KTimer tm("moba_select", s);
  e = qat::launch_moba_select(q, bf, L.kbar, L.kplanes, blk, p->batch, p->seq_len, p->n_q_heads, p->n_kv_heads, p->head_dim,
                              nbc_need, p->q_start, p->q_len, p->block, p->topk, s);
  return hip_status(e, "moba_block_select: scoring");
}

// Attention for the rows of p with q holding q_seq positions per sequence
// from position q_off on.
int moba_attn_rows(const qat_moba_params* p, const void* q, int64_t q_seq, int64_t q_off, const void* k,
                   const void* v, const int32_t* blk, void* out, float* lse, const MobaLayout& L, hipStream_t s,
                   const char* who) {
  const bool bf = p->dtype == QAT_BF16;
  hipError_t e;
  if (L.decode) {
    e = qat::launch_moba_decode(q, k, v, blk, L.dec_po, L.dec_plse, out, lse, bf, p->batch, p->seq_len, q_seq,
                                q_off, p->n_q_heads, p->n_kv_heads, p->head_dim, p->q_start, p->q_len, p->block,
                                p->topk, p->scale, s);
  } else if (bf && p->window == 0 && q_seq == p->seq_len) {
    if (p->topk > 1 && L.nbuckets > 0) {
      qat::KTimer tm("moba_dispatch", s);
      e = qat::launch_moba_dispatch(blk, p->batch, p->seq_len, p->n_q_heads, p->n_kv_heads, p->head_dim,
                                    p->q_start, p->q_len, p->block, p->topk, L.nbc, L.counts, L.offsets, L.cursor,
                                    L.entries, L.tiles, L.ntiles, s, nullptr, nullptr, L.wg_loc, L.part_lse);
      if (e != hipSuccess) return hip_status(e, who);
    }
    e = qat::launch_moba_attn_mfma(q, k, v, blk, L.tiles, L.ntiles, L.entries, L.part_o, L.part_lse, out, lse,
                                   p->batch, p->seq_len, p->n_q_heads, p->n_kv_heads, p->head_dim, L.nbc,
                                   p->q_start, p->q_len, p->block, p->topk, p->scale,
                                   L.nbuckets > 0 ? L.max_tiles : 0, s);
  } else {
    qat::KTimer tm("moba_generic_attn", s);
    e = qat::launch_moba_generic(q, k, v, blk, out, lse, bf, p->batch, p->seq_len, q_seq, q_off, p->n_q_heads,
                                 p->n_kv_heads, p->head_dim, p->q_start, p->q_len, p->block, p->topk, p->window,
                                 p->scale, s);
  }
  return hip_status(e, who);
}

QAT_EXPORT int moba_sparse_attn(const qat_moba_params* p, const void* q, const void* k, const void* v,
                                const int32_t* blk, void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  int rc = moba_check(p);
  if (rc) return rc;
  if (!q || !k || !v || !blk || !out) return fail(QAT_EINVAL, "q, k, v, blk, out must be non-NULL");
  MobaLayout L = moba_layout(p, nullptr);
  if ((rc = check_ws(ws, ws_bytes, L.bytes))) return rc;
  L = moba_layout(p, ws);
  return moba_attn_rows(p, q, p->seq_len, 0, k, v, blk, out, lse, L, (hipStream_t)stream, "moba_sparse_attn");
}

QAT_EXPORT int moba_block_means(const qat_moba_params* p, const void* k, int64_t first_block, int64_t n_blocks,
                                float* kbar, void* ws, size_t ws_bytes, void* stream) {
  int rc = moba_check(p);
  if (rc) return rc;
  if (!k || !kbar) return fail(QAT_EINVAL, "k, kbar must be non-NULL");
  const int64_t nbc = p->seq_len / p->block;
  if (first_block < 0 || n_blocks < 0 || first_block + n_blocks > nbc)
    return fail(QAT_EINVAL, "blocks [%lld, %lld) are not complete blocks of a %lld-token sequence",
                (long long)first_block, (long long)(first_block + n_blocks), (long long)p->seq_len);
  MobaLayout L = moba_layout(p, nullptr);
  if ((rc = check_ws(ws, ws_bytes, L.bytes))) return rc;
  L = moba_layout(p, ws);
  hipStream_t s = (hipStream_t)stream;
  qat::KTimer tm("moba_meanpool", s);
  hipError_t e = qat::launch_moba_meanpool(k, p->dtype == QAT_BF16, p->batch, p->seq_len, p->n_kv_heads,
                                           p->head_dim, p->block, nbc, L.mp_part, kbar, nullptr, s, first_block,
                                           n_blocks);
  return hip_status(e, "moba_block_means");
}

QAT_EXPORT int moba_decode_select(const qat_moba_params* p, const void* q, const float* kbar, int32_t* blk,
                                  void* stream) {
  int rc = moba_check(p);
  if (rc) return rc;
  if (!q || !blk) return fail(QAT_EINVAL, "q, blk must be non-NULL");
  // the means are read only when some row has an earlier complete block
  const bool need_means = p->topk > 1 && (p->q_start + p->q_len - 1) / p->block > 0;
  if (need_means && !kbar) return fail(QAT_EINVAL, "kbar must be non-NULL");
  hipStream_t s = (hipStream_t)stream;
  qat::KTimer tm("moba_decode_select", s);
  hipError_t e = qat::launch_moba_select_means(q, p->dtype == QAT_BF16, kbar, blk, p->batch, p->seq_len, p->q_len,
                                               p->q_start, p->n_q_heads, p->n_kv_heads, p->head_dim,
                                               p->seq_len / p->block, p->q_start, p->q_len, p->block, p->topk, s);
  return hip_status(e, "moba_decode_select");
}

QAT_EXPORT int moba_decode_attn(const qat_moba_params* p, const void* q, const void* k, const void* v,
                                const int32_t* blk, void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  int rc = moba_check(p);
  if (rc) return rc;
  if (!q || !k || !v || !blk || !out) return fail(QAT_EINVAL, "q, k, v, blk, out must be non-NULL");
  MobaLayout L = moba_layout(p, nullptr);
  if ((rc = check_ws(ws, ws_bytes, L.bytes))) return rc;
  L = moba_layout(p, ws);
  return moba_attn_rows(p, q, p->q_len, p->q_start, k, v, blk, out, lse, L, (hipStream_t)stream,
                        "moba_decode_attn");
}

// ---------------------------------------------------------------- no allocation
// Fixed device scratch of moba_decode_attn_noalloc: the split-key pieces'
// float32 partial outputs and log-sum-exps. Every GPU holds its own copy for
// the life of the process. Host code never names the array (its name on the
// host is not a device address): the address of the current device's copy
// is fetched once per device and kept.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "moba_decode_attn_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(QAT_EUNSUPPORTED, "device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "moba_decode_attn_noalloc: hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return QAT_OK;
}
}  // namespace

QAT_EXPORT int moba_decode_attn_noalloc(const qat_moba_params* p, const void* q, const void* k, const void* v,
                                        const int32_t* blk, void* out, float* lse, void* stream) {
  int rc = moba_check(p);
  if (rc) return rc;
  if (!q || !k || !v || !blk || !out) return fail(QAT_EINVAL, "q, k, v, blk, out must be non-NULL");
  const MobaLayout L = moba_layout(p, nullptr);
  if (!L.decode)
    return fail(QAT_EUNSUPPORTED,
                "moba_decode_attn_noalloc takes the split-key case only (q_len <= %lld, window 0, at most %d "
                "pieces of 256 keys per row)",
                (long long)kMobaDecodeMaxQ, kMobaDecodeMaxPieces);
  const size_t po_bytes = ((size_t)L.nrows * L.dec_pieces * p->head_dim * sizeof(float) + 255) & ~size_t(255);
  const size_t need = po_bytes + (size_t)L.nrows * L.dec_pieces * sizeof(float);
  if (need > kNoAllocScratchBytes)
    return fail(QAT_EUNSUPPORTED, "moba_decode_attn_noalloc needs %zu bytes of scratch; its fixed buffer holds %zu",
                need, kNoAllocScratchBytes);
  void* base = nullptr;
  if ((rc = noalloc_scratch(&base))) return rc;
  float* po = static_cast<float*>(base);
  float* plse = reinterpret_cast<float*>(static_cast<char*>(base) + po_bytes);
  const hipError_t e = qat::launch_moba_decode(q, k, v, blk, po, plse, out, lse, p->dtype == QAT_BF16, p->batch,
                                               p->seq_len, p->q_len, p->q_start, p->n_q_heads, p->n_kv_heads,
                                               p->head_dim, p->q_start, p->q_len, p->block, p->topk, p->scale,
                                               (hipStream_t)stream);
  return hip_status(e, "moba_decode_attn_noalloc");
}

QAT_EXPORT int moba_bwd_workspace_size(const qat_moba_params* p, size_t* bytes) {
  int rc = moba_check(p);
  if (rc) return rc;
  if (!bytes) return fail(QAT_EINVAL, "bytes is NULL");
  *bytes = moba_layout(p, nullptr, true).bytes;
  return ok();
}

QAT_EXPORT int moba_sparse_attn_bwd(const qat_moba_params* p, const void* q, const void* k, const void* v,
                                    const int32_t* blk, const void* dout, const float* lse, float* dq, float* dk,
                                    float* dv, void* ws, size_t ws_bytes, void* stream) {
  int rc = moba_check(p);
  if (rc) return rc;
  if (!q || !k || !v || !blk || !dout || !lse || !dq || !dk || !dv)
    return fail(QAT_EINVAL, "q, k, v, blk, dout, lse, dq, dk, dv must be non-NULL");
  if (p->window != 0) return fail(QAT_EUNSUPPORTED, "gradients with an extra local window are not implemented");
  MobaLayout L = moba_layout(p, nullptr, true);
  if ((rc = check_ws(ws, ws_bytes, L.bytes))) return rc;
  L = moba_layout(p, ws, true);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  const bool gated = p->topk > 1 && L.nbuckets > 0;
  if (gated) {
    qat::KTimer tm("moba_dispatch", s);
    // stable placement: the gated-key pass sums a bucket's rows in entry order
    e = qat::launch_moba_dispatch(blk, p->batch, p->seq_len, p->n_q_heads, p->n_kv_heads, p->head_dim, p->q_start,
                                  p->q_len, p->block, p->topk, L.nbc, L.counts, L.offsets, L.cursor, L.entries,
                                  L.tiles, L.ntiles, s, L.wg_counts, L.wg_base);
    if (e != hipSuccess) return hip_status(e, "moba_sparse_attn_bwd: dispatch");
  }
  e = qat::launch_moba_bwd(q, k, v, blk, dout, lse, L.tiles, L.ntiles, L.entries, gated ? L.max_tiles : 0,
                           L.counts, L.nbuckets, L.run_off, L.kv_part, L.dq_part, dq, L.delta, dk, dv, p->dtype == QAT_BF16, p->batch, p->seq_len, p->n_q_heads,
                           p->n_kv_heads, p->head_dim, p->q_start, p->q_len, p->block, p->topk, p->scale, s);
  return hip_status(e, "moba_sparse_attn_bwd");
}

// ---------------------------------------------------------------- CCA
int cca_check(const qat_cca_params* p) {
  if (!p) return fail(QAT_EINVAL, "params is NULL");
  if (p->batch < 1 || p->seq_len < 1 || p->n_q_heads < 1 || p->n_kv_heads < 1)
    return fail(QAT_EINVAL, "batch, seq_len and head counts must be >= 1");
  if (p->n_q_heads % p->n_kv_heads) return fail(QAT_EINVAL, "n_kv_heads must divide n_q_heads");
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(QAT_EUNSUPPORTED, "head_dim %lld not supported (64 or 128)", (long long)p->head_dim);
  if (p->dtype != QAT_BF16) return fail(QAT_EUNSUPPORTED, "CCA attention takes bfloat16 inputs");
  if (p->q_start < 0 || p->q_len < 1 || p->q_start + p->q_len > p->seq_len)
    return fail(QAT_EINVAL, "query rows [%lld, %lld) outside the sequence of %lld", (long long)p->q_start,
                (long long)(p->q_start + p->q_len), (long long)p->seq_len);
  if (p->group < 1) return fail(QAT_EINVAL, "group must be >= 1");
  if (p->window < 0) return fail(QAT_EINVAL, "window must be >= 0");
  if (!std::isfinite(p->scale) || !(p->scale > 0.f)) return fail(QAT_EINVAL, "scale must be finite and > 0");
  if (p->seq_len * p->n_q_heads * p->head_dim >= (1ll << 31))
    return fail(QAT_EUNSUPPORTED, "one sequence's q must hold fewer than 2^31 elements");
  return QAT_OK;
}

QAT_EXPORT int cca_pool(const qat_cca_params* p, const void* q, const void* k, const void* v, void* kc, void* vc,
                        void* stream) {
  int rc = cca_check(p);
  if (rc) return rc;
  if (!q || !k || !v || !kc || !vc) return fail(QAT_EINVAL, "q, k, v, kc, vc must be non-NULL");
  const int64_t ngroups = p->seq_len / p->group;
  const int64_t need = qat::cca_groups_needed(p->seq_len, p->q_start, p->q_len, p->group, p->window);
  hipStream_t s = (hipStream_t)stream;
  qat::KTimer tm("cca_pool", s);
  hipError_t e = qat::launch_cca_pool(q, k, v, kc, vc, p->batch, p->seq_len, p->n_q_heads, p->n_kv_heads,
                                      p->head_dim, ngroups, need, p->group, p->scale, s);
  return hip_status(e, "cca_pool");
}

QAT_EXPORT int cca_attn(const qat_cca_params* p, const void* q, const void* k, const void* v, const void* kc,
                        const void* vc, void* out, float* lse, void* stream) {
  int rc = cca_check(p);
  if (rc) return rc;
  if (!q || !k || !v || !out) return fail(QAT_EINVAL, "q, k, v, out must be non-NULL");
  const int64_t need = qat::cca_groups_needed(p->seq_len, p->q_start, p->q_len, p->group, p->window);
  if (need > 0 && (!kc || !vc)) return fail(QAT_EINVAL, "kc, vc must be non-NULL");
  hipStream_t s = (hipStream_t)stream;
  qat::KTimer tm("cca_attn", s);
  hipError_t e = qat::launch_cca_attn(q, k, v, kc, vc, out, lse, p->batch, p->seq_len, p->n_q_heads, p->n_kv_heads,
                                      p->head_dim, p->q_start, p->q_len, p->seq_len / p->group, p->group,
                                      p->window, p->scale, s);
  return hip_status(e, "cca_attn");
}

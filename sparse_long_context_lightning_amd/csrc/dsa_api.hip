// C ABI of the DSA hot path: host-side validation, workspace carving and launch order.
// The contract of every entry point is documented in include/dsa.h.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "../../include/dsa.h"
#include "kernels.h"

namespace {

thread_local char g_last_error[512] = "";

// DSA_LOG=1 in the environment: every entry point logs its call (name and sizes) and every
// rejected call its reason, one line each on stderr.  Read once.
bool log_enabled() {
  static const bool on = [] {
    const char* v = getenv("DSA_LOG");
    return v && v[0] && strcmp(v, "0") != 0;
  }();
  return on;
}


int vfail(int status, const char* fmt, va_list ap) {
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  if (log_enabled()) fprintf(stderr, "[dsa] -> status %d: %s\n", status, g_last_error);
  return status;
}

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  const int st = vfail(status, fmt, ap);
  va_end(ap);
  return st;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return DSA_OK;
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Launch timing (dsa_timing_enable): while on, every launch of the library is bracketed by two
// HIP events on its stream, and the pairs are summed per launch name when the record is read.
// A diagnostic: one host thread, no graph capture while it is on.
struct TimedLaunch {
  int slot;
  hipEvent_t a, b;
};
struct TimingRecord {
  bool on = false;
  std::vector<const char*> names;  // static strings
  std::vector<double> ms;
  std::vector<long long> launches;
  std::vector<TimedLaunch> pending;
  std::vector<hipEvent_t> pool;  // events whose pair has been read, for reuse
};
TimingRecord g_timing;

int timing_slot(const char* name) {
  for (size_t i = 0; i < g_timing.names.size(); ++i)
    if (strcmp(g_timing.names[i], name) == 0) return (int)i;
  g_timing.names.push_back(name);
  g_timing.ms.push_back(0.0);
  g_timing.launches.push_back(0);
  return (int)g_timing.names.size() - 1;
}

hipEvent_t timing_event() {
  if (!g_timing.pool.empty()) {
    hipEvent_t e = g_timing.pool.back();
    g_timing.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  return hipEventCreate(&e) == hipSuccess ? e : nullptr;
}

// Waits for the recorded launches and adds their times to the record.
hipError_t timing_resolve() {
  hipError_t err = hipSuccess;
  for (const TimedLaunch& t : g_timing.pending) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(t.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.a, t.b);
    if (e == hipSuccess) {
      g_timing.ms[t.slot] += ms;
      g_timing.launches[t.slot] += 1;
    } else if (err == hipSuccess) {
      err = e;
    }
    g_timing.pool.push_back(t.a);
    g_timing.pool.push_back(t.b);
  }
  g_timing.pending.clear();
  return err;
}

// One library launch: logged with DSA_LOG, timed while launch timing is on.
class LaunchScope {
 public:
  LaunchScope(const char* name, hipStream_t s) : name_(name), s_(s) {
    if (log_enabled()) fprintf(stderr, "[dsa]   launch %s\n", name);
    if (!g_timing.on) return;
    a_ = timing_event();
    b_ = timing_event();
    if (a_ && b_ && hipEventRecord(a_, s) != hipSuccess) a_ = nullptr;
  }
  ~LaunchScope() {
    if (a_ && b_ && hipEventRecord(b_, s_) == hipSuccess) g_timing.pending.push_back({timing_slot(name_), a_, b_});
  }
  LaunchScope(const LaunchScope&) = delete;
  LaunchScope& operator=(const LaunchScope&) = delete;

 private:
  const char* name_;
  hipStream_t s_;
  hipEvent_t a_ = nullptr, b_ = nullptr;
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

long long round_up(long long x, long long m) { return (x + m - 1) / m * m; }

// Supported indexer shapes (one kernel instantiation each).
bool indexer_shape_ok(int h_idx, int d_idx) {
  return (d_idx == 128 && (h_idx == 16 || h_idx == 32 || h_idx == 64)) || (h_idx == 4 && d_idx == 64);
}

int check_attn_shape(int hq, int hkv, int head_dim) {
  if (hq <= 0 || hkv <= 0 || head_dim <= 0) return fail(DSA_ERR_INVALID_ARG, "head counts and head_dim must be positive");
  if (hq % hkv != 0) return fail(DSA_ERR_INVALID_ARG, "hq (%d) must be a multiple of hkv (%d)", hq, hkv);
  if (head_dim != 128) return fail(DSA_ERR_UNSUPPORTED, "head_dim %d is not supported (only 128)", head_dim);
  if (hq / hkv > 16) return fail(DSA_ERR_UNSUPPORTED, "group size hq/hkv = %d exceeds 16", hq / hkv);
  return DSA_OK;
}

int check_topk(int k) {
  if (k < 1 || k > DSA_MAX_TOP_K) return fail(DSA_ERR_UNSUPPORTED, "top_k %d outside [1, %d]", k, DSA_MAX_TOP_K);
  return DSA_OK;
}

int check_indexer_shape(int h_idx, int d_idx) {
  if (h_idx <= 0 || d_idx <= 0) return fail(DSA_ERR_INVALID_ARG, "h_idx and d_idx must be positive");
  if (!indexer_shape_ok(h_idx, d_idx))
    return fail(DSA_ERR_UNSUPPORTED, "indexer shape (h_idx=%d, d_idx=%d) is not supported", h_idx, d_idx);
  return DSA_OK;
}

// The indexer backward is built for the 64-head, 128-dim indexer only.
int check_indexer_bwd_shape(int h_idx, int d_idx) {
  if (h_idx <= 0 || d_idx <= 0) return fail(DSA_ERR_INVALID_ARG, "h_idx and d_idx must be positive");
  if (h_idx != 64 || d_idx != 128)
    return fail(DSA_ERR_UNSUPPORTED, "indexer backward supports h_idx = 64, d_idx = 128 only (got %d, %d)", h_idx,
                d_idx);
  return DSA_OK;
}

// Validates host cu_seqlens and returns the longest sequence in *max_len.
int check_cu_host(const int32_t* cu, int batch, int total_tokens, int* max_len) {
  if (!cu) return fail(DSA_ERR_INVALID_ARG, "cu_seqlens_host is null");
  if (batch <= 0) return fail(DSA_ERR_INVALID_ARG, "batch must be positive");
  if (cu[0] != 0) return fail(DSA_ERR_INVALID_ARG, "cu_seqlens_host[0] must be 0");
  int ml = 0;
  for (int b = 0; b < batch; ++b) {
    if (cu[b + 1] < cu[b]) return fail(DSA_ERR_INVALID_ARG, "cu_seqlens_host must be non-decreasing");
    ml = std::max(ml, cu[b + 1] - cu[b]);
  }
  if (cu[batch] != total_tokens)
    return fail(DSA_ERR_INVALID_ARG, "cu_seqlens_host[batch] = %d != total_tokens = %d", cu[batch], total_tokens);
  *max_len = ml;
  return DSA_OK;
}

#define DSA_TRY(expr)              \
  do {                             \
    const int st_ = (expr);        \
    if (st_ != DSA_OK) return st_; \
  } while (0)

// A library launch (expr returns hipError_t) under a LaunchScope named `name`.
#define DSA_LAUNCH(name, stream, expr)     \
  do {                                     \
    hipError_t e_;                         \
    {                                      \
      LaunchScope ls_(name, stream);       \
      e_ = (expr);                         \
    }                                      \
    DSA_TRY(hip_status(e_, name " launch")); \
  } while (0)

// The same for a launch whose status is the caller's return value.
#define DSA_LAUNCH_RETURN(name, stream, expr) \
  do {                                        \
    hipError_t e_;                            \
    {                                         \
      LaunchScope ls_(name, stream);          \
      e_ = (expr);                            \
    }                                         \
    return hip_status(e_, name " launch");    \
  } while (0)

#define DSA_NONNULL(p) \
  if (!(p)) return fail(DSA_ERR_INVALID_ARG, "%s is null", #p)

#define DSA_ALIGNED(p) \
  if (!aligned16(p)) return fail(DSA_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p)

constexpr int kKeySplit = 4096;        // keys per prefill-indexer workgroup (at most)

// Keys per prefill-indexer workgroup for rows whose longest prefix is t_max + 1: up to
// kKeySplit, but short prefixes are cut into about 16 splits of at least 1024 keys (multiples
// of the 64-key tile), so a launch over short rows still has many workgroups of similar length
// instead of a few rounds of long ones.  Every score is computed by exactly one workgroup, so the
// split never changes a result.
int key_split_for(int t_max) {
  const int want = (t_max + 1 + 15) / 16;
  const int ks = (want + 63) / 64 * 64;
  return std::min(kKeySplit, std::max(1024, ks));
}
constexpr int kMinChunkRows = 64;
constexpr int kDefaultChunkRows = 2048;

size_t topk_scratch(int rows, long long ld) {
  return ld <= dsa::kTopkWaveMaxLd ? round_up((long long)dsa::topk_wave_workspace_bytes(rows), 256) : 0;
}

// Workspace of one prefill chunk: its fp32 score rows, then the top-k scratch.
size_t prefill_chunk_bytes(int rows, long long ld) {
  return (size_t)round_up((long long)rows * ld * 4, 256) + topk_scratch(rows, ld);
}

// Blocks of kUnionBlockRows rows; a block is attended from its merged set when that set has at
// most kUnionRatio x (rows x k_sel) entries.  Measured on MI355X at 128K / k = 2048 / GQA 32:4,
// blocks of 8 rows beat blocks of 16 (the merged-set work grows with rows x |merged set| while
// the gathered bytes change little), and with 8-row blocks the merged-set kernel beat the
// per-row one at every merged-set size (ratios 0.8 / 0.9 / 1.0: 160.9 / 157.4 / 152.4 ms for the
// whole prefill), so only blocks that repeat a position go per row.
constexpr int kUnionBlockRows = 8;
constexpr float kUnionRatio = 1.0f;

// Workspace of the dedup attention: per-block counts and path flags, merged KV rows and masks.
struct UnionLayout {
  int n_blocks = 0, cap = 0;
  size_t counts = 0, flags = 0, rows = 0, masks = 0, bytes = 0;
};
UnionLayout union_layout(int total_tokens, int k_sel, int block_rows = kUnionBlockRows, int mask_bytes = 2) {
  UnionLayout u;
  u.n_blocks = (total_tokens + block_rows - 1) / block_rows;
  u.cap = (int)round_up((long long)block_rows * k_sel, dsa::kUnionChunk);
  long long off = 0;
  u.counts = (size_t)off;
  off += round_up((long long)u.n_blocks * 4, 256);
  u.flags = (size_t)off;
  off += round_up((long long)u.n_blocks * 4, 256);
  u.rows = (size_t)off;
  off += round_up((long long)u.n_blocks * u.cap * 4, 256);
  u.masks = (size_t)off;
  off += round_up((long long)u.n_blocks * u.cap * mask_bytes, 256);
  u.bytes = (size_t)off;
  return u;
}

// Workspace of the merged-set attention backward: the same lists with 32-bit masks, for blocks of
// union_bwd_block_rows(hq / hkv) rows.
UnionLayout union_bwd_layout(int total_tokens, int k_sel, int hq, int hkv) {
  return union_layout(total_tokens, k_sel, dsa::union_bwd_block_rows(hq / hkv), 4);
}

// Sparse attention of the prefill rows described by `a` with adjacent-query dedup: merged sets
// of every kUnionBlockRows-row block, the merged-set kernel on the blocks flagged for it, the per-row kernel
// on the others.  `ws` holds union_layout(a.rows, a.k_sel).bytes bytes.
hipError_t launch_attn_dedup(dsa::SparseAttnArgs a, void* ws, hipStream_t s) {
  const UnionLayout u = union_layout(a.rows, a.k_sel);
  char* base = static_cast<char*>(ws);
  int* counts = reinterpret_cast<int*>(base + u.counts);
  int* flags = reinterpret_cast<int*>(base + u.flags);
  int* kv_rows = reinterpret_cast<int*>(base + u.rows);
  uint16_t* masks = reinterpret_cast<uint16_t*>(base + u.masks);
  dsa::QueryUnionArgs q = {};
  q.idx = a.idx;
  q.k_sel = a.k_sel;
  q.cu_seqlens = a.cu_seqlens;
  q.batch = a.batch;
  q.rows = a.rows;
  q.block_rows = kUnionBlockRows;
  q.block_begin = 0;
  q.block_end = u.n_blocks;
  q.cap = u.cap;
  q.counts = counts;
  q.kv_rows = kv_rows;
  q.masks = masks;
  q.use_union = flags;
  q.ratio = kUnionRatio;
  hipError_t e;
  {
    LaunchScope ls("query_union", s);
    e = dsa::launch_query_union(q, s);
  }
  if (e != hipSuccess) return e;
  dsa::UnionAttnArgs m = {};
  m.q = a.q;
  m.k = a.k;
  m.v = a.v;
  m.counts = counts;
  m.kv_rows = kv_rows;
  m.masks = masks;
  m.cap = u.cap;
  m.block_rows = kUnionBlockRows;
  m.rows = a.rows;
  m.hq = a.hq;
  m.hkv = a.hkv;
  m.softmax_scale = a.softmax_scale;
  m.out = a.out;
  m.lse = a.lse;
  m.use_union = flags;
  {
    LaunchScope ls("sparse_attn_union", s);
    e = dsa::launch_sparse_attn_union(m, s);
  }
  if (e != hipSuccess) return e;
  a.skip_block = flags;
  a.skip_block_rows = kUnionBlockRows;
  LaunchScope ls("sparse_attn", s);
  return dsa::launch_sparse_attn(a, s);
}

// Backward of the sparse attention with adjacent-query dedup: dk / dv zeroed, the merged sets
// of every block built, the merged-set backward on the blocks where no row repeats a position,
// the per-row backward on the rows of the others.  `ws` holds union_bwd_layout(..).bytes bytes.
hipError_t launch_attn_bwd_dedup(dsa::SparseAttnBwdArgs a, void* ws, hipStream_t s) {
  const int R = dsa::union_bwd_block_rows(a.hq / a.hkv);
  const UnionLayout u = union_bwd_layout(a.rows, a.k_sel, a.hq, a.hkv);
  char* base = static_cast<char*>(ws);
  int* counts = reinterpret_cast<int*>(base + u.counts);
  int* flags = reinterpret_cast<int*>(base + u.flags);
  int* kv_rows = reinterpret_cast<int*>(base + u.rows);
  uint32_t* masks = reinterpret_cast<uint32_t*>(base + u.masks);
  const long long nkv = (long long)a.rows * a.hkv * 128;
  hipError_t e = dsa::launch_zero_f32(a.dk, nkv, s);
  if (e == hipSuccess) e = dsa::launch_zero_f32(a.dv, nkv, s);
  if (e != hipSuccess) return e;
  dsa::QueryUnionArgs q = {};
  q.idx = a.idx;
  q.k_sel = a.k_sel;
  q.cu_seqlens = a.cu_seqlens;
  q.batch = a.batch;
  q.rows = a.rows;
  q.block_rows = R;
  q.block_begin = 0;
  q.block_end = u.n_blocks;
  q.cap = u.cap;
  q.counts = counts;
  q.kv_rows = kv_rows;
  q.masks32 = masks;
  q.use_union = flags;
  q.ratio = 1.0f;  // every block whose rows list no position twice
  e = dsa::launch_query_union(q, s);
  if (e != hipSuccess) return e;
  dsa::UnionBwdArgs m = {};
  m.q = a.q;
  m.k = a.k;
  m.v = a.v;
  m.out = a.out;
  m.dout = a.dout;
  m.lse = a.lse;
  m.counts = counts;
  m.kv_rows = kv_rows;
  m.masks = masks;
  m.cap = u.cap;
  m.use_union = flags;
  m.rows = a.rows;
  m.hq = a.hq;
  m.hkv = a.hkv;
  m.softmax_scale = a.softmax_scale;
  m.dq = a.dq;
  m.dk = a.dk;
  m.dv = a.dv;
  e = dsa::launch_sparse_attn_bwd_union(m, s);
  if (e != hipSuccess) return e;
  a.skip_block = flags;
  a.skip_block_rows = R;
  return dsa::launch_sparse_attn_bwd(a, s);
}

int decode_nsplit(int batch, int hkv, int top_k) {
  const int nchunk = (top_k + 31) / 32;
  const int want = (1024 + batch * hkv - 1) / (batch * hkv);
  return std::max(1, std::min(want, nchunk));
}

// Decode attention over a contiguous cache: partials of nsplit index ranges per (sequence, group),
// then their combine.  `part` holds decode_attn_part_bytes(batch, hq, nsplit) bytes.
size_t decode_attn_part_bytes(int batch, int hq, int nsplit) {
  return nsplit > 1 ? (size_t)batch * hq * nsplit * (128 + 2) * 4 : 0;
}

hipError_t launch_decode_attn(const void* q, const void* k_cache, const void* v_cache, const int32_t* idx, int k_sel,
                              const int32_t* seq_lens, int batch, int s_max, int hq, int hkv, float softmax_scale,
                              void* out, float* lse, void* part, hipStream_t s) {
  const int nsplit = decode_nsplit(batch, hkv, k_sel);
  dsa::SparseAttnArgs a = {};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_cache);
  a.v = static_cast<const uint16_t*>(v_cache);
  a.idx = idx;
  a.k_sel = k_sel;
  a.cu_seqlens = nullptr;
  a.batch = batch;
  a.seq_lens = seq_lens;
  a.s_max = s_max;
  a.rows = batch;
  a.hq = hq;
  a.hkv = hkv;
  a.softmax_scale = softmax_scale;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.nsplit = nsplit;
  a.part_o = static_cast<float*>(part);
  a.part_ml = a.part_o + (size_t)batch * hq * nsplit * 128;
  hipError_t e;
  {
    LaunchScope ls("sparse_attn_decode", s);
    e = dsa::launch_sparse_attn(a, s);
  }
  if (e != hipSuccess || nsplit == 1) return e;
  LaunchScope ls("attn_combine", s);
  return dsa::launch_attn_combine(a, s);
}

// mode 0: scores (dsa_index_scores); 1 / 2 / 3: the fused top-k's sampling, emitting and
// rescoring passes over the top-k scratch `ts` of the rows [row_begin, row_end) (one sequence's
// chunk).
int launch_index_rows(const void* q_idx, const void* k_idx, const float* w, const int32_t* cu, int batch,
                      int h_idx, int d_idx, int row_begin, int row_end, int out_row0, float* scores, long long ld,
                      hipStream_t stream, int mode = 0, const dsa::TopkScratch* ts = nullptr, int k = 0) {
  for (int b = 0; b < batch; ++b) {
    const int r0 = std::max(row_begin, cu[b]);
    const int r1 = std::min(row_end, cu[b + 1]);
    if (r0 >= r1) continue;
    dsa::IndexerPrefillArgs a;
    a.q_idx = static_cast<const uint16_t*>(q_idx);
    a.k_idx = static_cast<const uint16_t*>(k_idx);
    a.w = w;
    a.h_idx = h_idx;
    a.d_idx = d_idx;
    a.seq_off = cu[b];
    a.row_begin = r0;
    a.row_end = r1;
    a.out_row0 = out_row0;
    a.scores = scores;
    a.ld = ld;
    a.key_split = key_split_for(r1 - 1 - cu[b]);
    if (mode == 1)
      DSA_LAUNCH("indexer_sample", stream, dsa::launch_indexer_prefill_sample(a, *ts, k, stream));
    else if (mode == 2)
      DSA_LAUNCH("indexer_emit", stream, dsa::launch_indexer_prefill_emit(a, *ts, k, stream));
    else if (mode == 3)
      DSA_LAUNCH("indexer_rescore", stream, dsa::launch_indexer_prefill_rescore(a, *ts, stream));
    else
      DSA_LAUNCH("indexer", stream, dsa::launch_indexer_prefill(a, stream));
  }
  return DSA_OK;
}

}  // namespace

namespace dsa {
int api_fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  const int st = vfail(status, fmt, ap);
  va_end(ap);
  return st;
}
void api_clear_error() { g_last_error[0] = 0; }
ApiRange::ApiRange(const char* name) { roctxRangePushA(name); }
ApiRange::~ApiRange() { roctxRangePop(); }
void api_log(const char* name, const char* fmt, ...) {
  if (!log_enabled()) return;
  char buf[400];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  fprintf(stderr, "[dsa] %s(%s)\n", name, buf);
}
}  // namespace dsa

extern "C" {

int dsa_abi_version(void) { return DSA_ABI_VERSION; }

int dsa_timing_enable(int on) {
  g_last_error[0] = 0;
  const hipError_t e = timing_resolve();  // finish the launches recorded so far before clearing
  for (size_t i = 0; i < g_timing.ms.size(); ++i) {
    g_timing.ms[i] = 0.0;
    g_timing.launches[i] = 0;
  }
  g_timing.on = on != 0;
  return hip_status(e, "launch timing");
}

int dsa_timing_count(int* n) {
  g_last_error[0] = 0;
  DSA_NONNULL(n);
  const hipError_t e = timing_resolve();
  *n = (int)g_timing.names.size();
  return hip_status(e, "launch timing");
}

int dsa_timing_entry(int i, const char** name, double* total_ms, int64_t* launches) {
  g_last_error[0] = 0;
  DSA_NONNULL(name);
  DSA_NONNULL(total_ms);
  DSA_NONNULL(launches);
  if (i < 0 || i >= (int)g_timing.names.size())
    return fail(DSA_ERR_INVALID_ARG, "timing entry %d outside [0, %d)", i, (int)g_timing.names.size());
  *name = g_timing.names[i];
  *total_ms = g_timing.ms[i];
  *launches = g_timing.launches[i];
  return DSA_OK;
}

const char* dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE";
    case DSA_ERR_HIP: return "DSA_ERR_HIP";
    default: return "DSA_ERR_UNKNOWN";
  }
}

const char* dsa_last_error(void) { return g_last_error; }

int dsa_index_scores(const void* q_idx, const void* k_idx, const float* w, const int32_t* cu_seqlens_host, int batch,
                     int total_tokens, int h_idx, int d_idx, int row_begin, int row_count, float* scores, int64_t ld,
                     void* stream) {
  g_last_error[0] = 0;
  const dsa::ApiRange range_("dsa_index_scores");
  dsa::api_log("dsa_index_scores", "batch=%d total=%d h_idx=%d d_idx=%d rows=[%d,+%d) ld=%lld", batch, total_tokens, h_idx, d_idx, row_begin, row_count, (long long)ld);
  DSA_NONNULL(q_idx);
  DSA_NONNULL(k_idx);
  DSA_NONNULL(w);
  DSA_NONNULL(scores);
  DSA_ALIGNED(q_idx);
  DSA_ALIGNED(k_idx);
  DSA_ALIGNED(w);
  DSA_ALIGNED(scores);
  if (total_tokens < 0 || row_begin < 0 || row_count < 0 || row_begin + (long long)row_count > total_tokens)
    return fail(DSA_ERR_INVALID_ARG, "row range [%d, %d + %d) outside [0, %d)", row_begin, row_begin, row_count,
                total_tokens);
  DSA_TRY(check_indexer_shape(h_idx, d_idx));
  int max_len = 0;
  DSA_TRY(check_cu_host(cu_seqlens_host, batch, total_tokens, &max_len));
  if (ld % 4 != 0) return fail(DSA_ERR_INVALID_ARG, "ld (%lld) must be a multiple of 4", (long long)ld);
  for (int b = 0; b < batch; ++b) {
    const int r1 = std::min(row_begin + row_count, cu_seqlens_host[b + 1]);
    if (r1 > std::max(row_begin, cu_seqlens_host[b]) && r1 - cu_seqlens_host[b] > ld)
      return fail(DSA_ERR_INVALID_ARG, "ld (%lld) shorter than a row's prefix (%d)", (long long)ld,
                  r1 - cu_seqlens_host[b]);
  }
  if (row_count == 0) return DSA_OK;
  return launch_index_rows(q_idx, k_idx, w, cu_seqlens_host, batch, h_idx, d_idx, row_begin, row_begin + row_count,
                           row_begin, scores, ld, static_cast<hipStream_t>(stream));
}

int dsa_decode_index_scores(const void* q_idx, const float* w, const void* k_idx_cache, const int32_t* seq_lens,
                            int batch, int s_max, int max_seq_len, int h_idx, int d_idx, float* scores, int64_t ld,
                            void* stream) {
  g_last_error[0] = 0;
  const dsa::ApiRange range_("dsa_decode_index_scores");
  dsa::api_log("dsa_decode_index_scores", "batch=%d s_max=%d max_seq_len=%d h_idx=%d d_idx=%d ld=%lld", batch, s_max,
           max_seq_len, h_idx, d_idx, (long long)ld);
  DSA_NONNULL(q_idx);
  DSA_NONNULL(w);
  DSA_NONNULL(k_idx_cache);
  DSA_NONNULL(seq_lens);
  DSA_NONNULL(scores);
  DSA_ALIGNED(q_idx);
  DSA_ALIGNED(w);
  DSA_ALIGNED(k_idx_cache);
  DSA_ALIGNED(scores);
  if (batch <= 0 || s_max <= 0) return fail(DSA_ERR_INVALID_ARG, "batch and s_max must be positive");
  if (max_seq_len <= 0 || max_seq_len > s_max)
    return fail(DSA_ERR_INVALID_ARG, "max_seq_len (%d) must be in [1, s_max = %d]", max_seq_len, s_max);
  DSA_TRY(check_indexer_shape(h_idx, d_idx));
  if (ld < s_max || ld % 4 != 0)
    return fail(DSA_ERR_INVALID_ARG, "ld (%lld) must be a multiple of 4 and >= s_max (%d)", (long long)ld, s_max);
  dsa::IndexerDecodeArgs ia;
  ia.q_idx = static_cast<const uint16_t*>(q_idx);
  ia.w = w;
  ia.k_cache = static_cast<const uint16_t*>(k_idx_cache);
  ia.seq_lens = seq_lens;
  ia.batch = batch;
  ia.s_max = s_max;
  ia.max_len = max_seq_len;
  ia.h_idx = h_idx;
  ia.d_idx = d_idx;
  ia.scores = scores;
  ia.ld = ld;
  DSA_LAUNCH_RETURN("indexer_decode", static_cast<hipStream_t>(stream),
                    dsa::launch_indexer_decode(ia, static_cast<hipStream_t>(stream)));
}

int dsa_index_scores_bwd(const void* q_idx, const void* k_idx, const float* w, const int32_t* cu_seqlens_host,
                         int batch, int total_tokens, int h_idx, int d_idx, int row_begin, int row_count,
                         const float* dscores, int64_t ld, float* dq_idx, float* dw, float* dk_idx, void* stream) {
  g_last_error[0] = 0;
  const dsa::ApiRange range_("dsa_index_scores_bwd");
  dsa::api_log("dsa_index_scores_bwd", "batch=%d total=%d h_idx=%d d_idx=%d rows=[%d,+%d) ld=%lld", batch, total_tokens, h_idx, d_idx, row_begin, row_count, (long long)ld);
  DSA_NONNULL(q_idx);
  DSA_NONNULL(k_idx);
  DSA_NONNULL(w);
  DSA_NONNULL(dscores);
  DSA_NONNULL(dq_idx);
  DSA_NONNULL(dw);
  DSA_NONNULL(dk_idx);
  DSA_ALIGNED(q_idx);
  DSA_ALIGNED(k_idx);
  DSA_ALIGNED(w);
  DSA_ALIGNED(dscores);
  DSA_ALIGNED(dq_idx);
  DSA_ALIGNED(dk_idx);
  if (total_tokens < 0 || row_begin < 0 || row_count < 0 || row_begin + (long long)row_count > total_tokens)
    return fail(DSA_ERR_INVALID_ARG, "row range [%d, %d + %d) outside [0, %d)", row_begin, row_begin, row_count,
                total_tokens);
  DSA_TRY(check_indexer_bwd_shape(h_idx, d_idx));
  int max_len = 0;
  DSA_TRY(check_cu_host(cu_seqlens_host, batch, total_tokens, &max_len));
  if (ld % 4 != 0) return fail(DSA_ERR_INVALID_ARG, "ld (%lld) must be a multiple of 4", (long long)ld);
  for (int b = 0; b < batch; ++b) {
    const int r1 = std::min(row_begin + row_count, cu_seqlens_host[b + 1]);
    if (r1 > std::max(row_begin, cu_seqlens_host[b]) && r1 - cu_seqlens_host[b] > ld)
      return fail(DSA_ERR_INVALID_ARG, "ld (%lld) shorter than a row's prefix (%d)", (long long)ld,
                  r1 - cu_seqlens_host[b]);
  }
  if (row_count == 0) return DSA_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  for (int b = 0; b < batch; ++b) {
    const int r0 = std::max(row_begin, cu_seqlens_host[b]);
    const int r1 = std::min(row_begin + row_count, cu_seqlens_host[b + 1]);
    if (r0 >= r1) continue;
    dsa::IndexerBwdArgs a;
    a.q_idx = static_cast<const uint16_t*>(q_idx);
    a.k_idx = static_cast<const uint16_t*>(k_idx);
    a.w = w;
    a.g = dscores;
    a.ld = ld;
    a.seq_off = cu_seqlens_host[b];
    a.row_begin = r0;
    a.row_end = r1;
    a.grad_row0 = row_begin;
    a.dq = dq_idx;
    a.dw = dw;
    a.dk = dk_idx;
    DSA_LAUNCH("indexer_bwd", s, dsa::launch_indexer_bwd(a, s));
  }
  return DSA_OK;
}

int dsa_attn_head_mean(const void* q, const void* k, const int32_t* cu_seqlens_host, int batch, int total_tokens,
                       int hq, int hkv, int head_dim, float softmax_scale, int row_begin, int row_count, float* probs,
                       int64_t ld, float* lse, void* stream) {
  g_last_error[0] = 0;
  const dsa::ApiRange range_("dsa_attn_head_mean");
  dsa::api_log("dsa_attn_head_mean", "batch=%d total=%d hq=%d hkv=%d rows=[%d,+%d) ld=%lld", batch, total_tokens, hq, hkv, row_begin, row_count, (long long)ld);
  DSA_NONNULL(q);
  DSA_NONNULL(k);
  DSA_NONNULL(probs);
  DSA_NONNULL(lse);
  DSA_ALIGNED(q);
  DSA_ALIGNED(k);
  if (total_tokens < 0 || row_begin < 0 || row_count < 0 || row_begin + (long long)row_count > total_tokens)
    return fail(DSA_ERR_INVALID_ARG, "row range [%d, %d + %d) outside [0, %d)", row_begin, row_begin, row_count,
                total_tokens);
  DSA_TRY(check_attn_shape(hq, hkv, head_dim));
  if (hq / hkv < 4 || (hq / hkv) % 4 != 0 || (hkv != 1 && hkv != 2 && hkv != 4 && hkv != 8))
    return fail(DSA_ERR_UNSUPPORTED, "the head-mean target needs hq / hkv in {4, 8, 12, 16} and hkv in {1, 2, 4, 8}");
  int max_len = 0;
  DSA_TRY(check_cu_host(cu_seqlens_host, batch, total_tokens, &max_len));
  if (ld <= 0) return fail(DSA_ERR_INVALID_ARG, "ld must be positive");
  for (int b = 0; b < batch; ++b) {
    const int r1 = std::min(row_begin + row_count, cu_seqlens_host[b + 1]);
    if (r1 > std::max(row_begin, cu_seqlens_host[b]) && r1 - cu_seqlens_host[b] > ld)
      return fail(DSA_ERR_INVALID_ARG, "ld (%lld) shorter than a row's prefix (%d)", (long long)ld,
                  r1 - cu_seqlens_host[b]);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int b = 0; b < batch; ++b) {
    const int r0 = std::max(row_begin, cu_seqlens_host[b]);
    const int r1 = std::min(row_begin + row_count, cu_seqlens_host[b + 1]);
    if (r0 >= r1) continue;
    dsa::HeadMeanArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.hq = hq;
    a.hkv = hkv;
    a.seq_off = cu_seqlens_host[b];
    a.row_begin = r0;
    a.row_end = r1;
    a.out_row0 = row_begin;
    a.softmax_scale = softmax_scale;
    a.lse = lse;
    a.probs = probs;
    a.ld = ld;
    DSA_LAUNCH("attn_head_mean", s, dsa::launch_attn_head_mean(a, s));
  }
  return DSA_OK;
}

int dsa_indexer_kl(const float* scores, const float* target, int64_t ld, int rows, const int32_t* row_len,
                   float* row_loss, float* grad, void* stream) {
  g_last_error[0] = 0;
  const dsa::ApiRange range_("dsa_indexer_kl");
  dsa::api_log("dsa_indexer_kl", "rows=%d ld=%lld", rows, (long long)ld);
  DSA_NONNULL(scores);
  DSA_NONNULL(target);
  DSA_NONNULL(row_len);
  DSA_NONNULL(row_loss);
  DSA_NONNULL(grad);
  if (rows < 0 || ld <= 0) return fail(DSA_ERR_INVALID_ARG, "rows must be non-negative and ld positive");
  if (rows == 0) return DSA_OK;
  DSA_LAUNCH_RETURN("indexer_kl", static_cast<hipStream_t>(stream),
                    dsa::launch_indexer_kl(scores, target, ld, rows, row_len, 0, row_loss, grad,
                                           static_cast<hipStream_t>(stream)));
}

int dsa_topk_workspace_size(int rows, int64_t ld, int k, size_t* bytes) {
  g_last_error[0] = 0;
  DSA_NONNULL(bytes);
  if (rows < 0 || ld < 0) return fail(DSA_ERR_INVALID_ARG, "rows and ld must be non-negative");
  DSA_TRY(check_topk(k));
  *bytes = topk_scratch(rows, ld);
  return DSA_OK;
}

namespace {

int topk_entry(const float* scores, int64_t ld, int rows, const int32_t* row_len, int k, int32_t* idx_out,
               float* values_out, void* workspace, size_t workspace_bytes, void* stream, bool ranked) {
  g_last_error[0] = 0;
  const dsa::ApiRange range_(ranked ? "dsa_topk_sorted" : "dsa_topk");
  dsa::api_log(ranked ? "dsa_topk_sorted" : "dsa_topk", "rows=%d ld=%lld k=%d ws=%zu", rows, (long long)ld, k, workspace_bytes);
  DSA_NONNULL(scores);
  DSA_NONNULL(row_len);
  DSA_NONNULL(idx_out);
  DSA_ALIGNED(scores);
  if (rows < 0) return fail(DSA_ERR_INVALID_ARG, "rows must be non-negative");
  if (ld <= 0 || ld % 4 != 0) return fail(DSA_ERR_INVALID_ARG, "ld (%lld) must be a positive multiple of 4", (long long)ld);
  DSA_TRY(check_topk(k));
  DSA_ALIGNED(workspace);
  if (rows == 0) return DSA_OK;
  const size_t need = topk_scratch(rows, ld);
  if (workspace && workspace_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu bytes needed", workspace_bytes, need);
  dsa::TopkArgs a;
  a.scores = scores;
  a.ld = ld;
  a.rows = rows;
  a.row_len = row_len;
  a.len_base = 0;
  a.k = k;
  a.idx_out = idx_out;
  a.values_out = ranked ? nullptr : values_out;
  a.workspace = need ? workspace : nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  DSA_LAUNCH("topk", s, dsa::launch_topk(a, s));
  if (!ranked) return DSA_OK;
  a.values_out = values_out;
  DSA_LAUNCH_RETURN("topk_rank", s, dsa::launch_topk_rank(a, s));
}

}  // namespace

int dsa_topk(const float* scores, int64_t ld, int rows, const int32_t* row_len, int k, int32_t* idx_out,
             float* values_out, void* workspace, size_t workspace_bytes, void* stream) {
  return topk_entry(scores, ld, rows, row_len, k, idx_out, values_out, workspace, workspace_bytes, stream, false);
}

int dsa_topk_sorted(const float* scores, int64_t ld, int rows, const int32_t* row_len, int k, int32_t* idx_out,
                    float* values_out, void* workspace, size_t workspace_bytes, void* stream) {
  return topk_entry(scores, ld, rows, row_len, k, idx_out, values_out, workspace, workspace_bytes, stream, true);
}

int dsa_sparse_gqa_attn(const void* q, const void* k, const void* v, const int32_t* idx, int k_sel,
                        const int32_t* cu_seqlens, int batch, int total_tokens, int hq, int hkv, int head_dim,
                        float softmax_scale, void* out, float* lse, void* stream) {
  g_last_error[0] = 0;
  const dsa::ApiRange range_("dsa_sparse_gqa_attn");
  dsa::api_log("dsa_sparse_gqa_attn", "batch=%d total=%d hq=%d hkv=%d d=%d k_sel=%d", batch, total_tokens, hq, hkv, head_dim, k_sel);
  DSA_NONNULL(q);
  DSA_NONNULL(k);
  DSA_NONNULL(v);
  DSA_NONNULL(idx);
  DSA_NONNULL(cu_seqlens);
  DSA_NONNULL(out);
  DSA_ALIGNED(q);
  DSA_ALIGNED(k);
  DSA_ALIGNED(v);
  DSA_ALIGNED(out);
  if (batch <= 0 || total_tokens < 0) return fail(DSA_ERR_INVALID_ARG, "batch must be positive, total_tokens >= 0");
  if (k_sel <= 0) return fail(DSA_ERR_INVALID_ARG, "k_sel must be positive");
  DSA_TRY(check_attn_shape(hq, hkv, head_dim));
  if (total_tokens == 0) return DSA_OK;
  dsa::SparseAttnArgs a = {};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.idx = idx;
  a.k_sel = k_sel;
  a.cu_seqlens = cu_seqlens;
  a.batch = batch;
  a.seq_lens = nullptr;
  a.rows = total_tokens;
  a.hq = hq;
  a.hkv = hkv;
  a.softmax_scale = softmax_scale;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.nsplit = 1;
  DSA_LAUNCH_RETURN("sparse_attn", static_cast<hipStream_t>(stream),
                    dsa::launch_sparse_attn(a, static_cast<hipStream_t>(stream)));
}

int dsa_query_union_size(int total_tokens, int k_sel, int block_rows, int* n_blocks, int* cap) {
  g_last_error[0] = 0;
  DSA_NONNULL(n_blocks);
  DSA_NONNULL(cap);
  if (total_tokens < 0 || k_sel <= 0) return fail(DSA_ERR_INVALID_ARG, "total_tokens >= 0 and k_sel > 0 required");
  if (!dsa::union_block_rows_ok(block_rows)) return fail(DSA_ERR_UNSUPPORTED, "block_rows %d is not 8 or 16", block_rows);
  if (k_sel > (1 << 24)) return fail(DSA_ERR_UNSUPPORTED, "k_sel %d too large", k_sel);
  *n_blocks = (total_tokens + block_rows - 1) / block_rows;
  *cap = (int)round_up((long long)block_rows * k_sel, dsa::kUnionChunk);
  return DSA_OK;
}

int dsa_query_union(const int32_t* idx, int k_sel, const int32_t* cu_seqlens, int batch, int total_tokens,
                    int block_rows, int cap, int32_t* counts, int32_t* kv_rows, uint16_t* masks, void* stream) {
  g_last_error[0] = 0;
  const dsa::ApiRange range_("dsa_query_union");
  dsa::api_log("dsa_query_union", "batch=%d total=%d k_sel=%d block_rows=%d cap=%d", batch, total_tokens, k_sel, block_rows, cap);
  DSA_NONNULL(idx);
  DSA_NONNULL(cu_seqlens);
  DSA_NONNULL(counts);
  DSA_NONNULL(kv_rows);
  DSA_NONNULL(masks);
  DSA_ALIGNED(kv_rows);
  if (reinterpret_cast<uintptr_t>(masks) & 3u) return fail(DSA_ERR_INVALID_ARG, "masks must be 4-byte aligned");
  if (batch <= 0 || total_tokens < 0) return fail(DSA_ERR_INVALID_ARG, "batch must be positive, total_tokens >= 0");
  int n_blocks = 0, need = 0;
  DSA_TRY(dsa_query_union_size(total_tokens, k_sel, block_rows, &n_blocks, &need));
  if (cap < need || cap % dsa::kUnionChunk != 0)
    return fail(DSA_ERR_INVALID_ARG, "cap %d must be a multiple of %d and >= %d", cap, dsa::kUnionChunk, need);
  if (total_tokens == 0) return DSA_OK;
  dsa::QueryUnionArgs a = {};
  a.idx = idx;
  a.k_sel = k_sel;
  a.cu_seqlens = cu_seqlens;
  a.batch = batch;
  a.rows = total_tokens;
  a.block_rows = block_rows;
  a.block_begin = 0;
  a.block_end = n_blocks;
  a.cap = cap;
  a.counts = counts;
  a.kv_rows = kv_rows;
  a.masks = masks;
  DSA_LAUNCH_RETURN("query_union", static_cast<hipStream_t>(stream),
                    dsa::launch_query_union(a, static_cast<hipStream_t>(stream)));
}

int dsa_sparse_gqa_attn_union(const void* q, const void* k, const void* v, const int32_t* counts,
                              const int32_t* kv_rows, const uint16_t* masks, int block_rows, int cap,
                              int total_tokens, int hq, int hkv, int head_dim, float softmax_scale, void* out,
                              float* lse, void* stream) {
  g_last_error[0] = 0;
  const dsa::ApiRange range_("dsa_sparse_gqa_attn_union");
  dsa::api_log("dsa_sparse_gqa_attn_union", "total=%d hq=%d hkv=%d block_rows=%d cap=%d", total_tokens, hq, hkv, block_rows, cap);
  DSA_NONNULL(q);
  DSA_NONNULL(k);
  DSA_NONNULL(v);
  DSA_NONNULL(counts);
  DSA_NONNULL(kv_rows);
  DSA_NONNULL(masks);
  DSA_NONNULL(out);
  DSA_ALIGNED(q);
  DSA_ALIGNED(k);
  DSA_ALIGNED(v);
  DSA_ALIGNED(out);
  DSA_ALIGNED(kv_rows);
  if (reinterpret_cast<uintptr_t>(masks) & 3u) return fail(DSA_ERR_INVALID_ARG, "masks must be 4-byte aligned");
  if (total_tokens < 0) return fail(DSA_ERR_INVALID_ARG, "total_tokens must be >= 0");
  if (cap <= 0 || cap % dsa::kUnionChunk != 0)
    return fail(DSA_ERR_INVALID_ARG, "cap %d must be a positive multiple of %d", cap, dsa::kUnionChunk);
  if (!dsa::union_block_rows_ok(block_rows)) return fail(DSA_ERR_UNSUPPORTED, "block_rows %d is not 8 or 16", block_rows);
  DSA_TRY(check_attn_shape(hq, hkv, head_dim));
  if (!dsa::union_attn_supported(hq, hkv, total_tokens))
    return fail(DSA_ERR_UNSUPPORTED,
                "merged-set attention supports hq / hkv in {4, 8, 16} (got %d) and total_tokens * hkv < 2^24", hq / hkv);
  if (total_tokens == 0) return DSA_OK;
  dsa::UnionAttnArgs a = {};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.counts = counts;
  a.kv_rows = kv_rows;
  a.masks = masks;
  a.cap = cap;
  a.block_rows = block_rows;
  a.rows = total_tokens;
  a.hq = hq;
  a.hkv = hkv;
  a.softmax_scale = softmax_scale;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  DSA_LAUNCH_RETURN("sparse_attn_union", static_cast<hipStream_t>(stream),
                    dsa::launch_sparse_attn_union(a, static_cast<hipStream_t>(stream)));
}

int dsa_sparse_gqa_attn_dedup_workspace_size(int total_tokens, int k_sel, int hq, int hkv, size_t* bytes) {
  g_last_error[0] = 0;
  DSA_NONNULL(bytes);
  if (total_tokens < 0 || k_sel <= 0) return fail(DSA_ERR_INVALID_ARG, "total_tokens >= 0 and k_sel > 0 required");
  if (k_sel > (1 << 24)) return fail(DSA_ERR_UNSUPPORTED, "k_sel %d too large", k_sel);
  *bytes = dsa::union_attn_supported(hq, hkv, total_tokens) ? union_layout(total_tokens, k_sel).bytes : 0;
  return DSA_OK;
}

int dsa_sparse_gqa_attn_dedup(const void* q, const void* k, const void* v, const int32_t* idx, int k_sel,
                              const int32_t* cu_seqlens, int batch, int total_tokens, int hq, int hkv, int head_dim,
                              float softmax_scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                              void* stream) {
  g_last_error[0] = 0;
  const dsa::ApiRange range_("dsa_sparse_gqa_attn_dedup");
  dsa::api_log("dsa_sparse_gqa_attn_dedup", "batch=%d total=%d hq=%d hkv=%d k_sel=%d ws=%zu", batch, total_tokens, hq, hkv, k_sel, workspace_bytes);
  DSA_NONNULL(q);
  DSA_NONNULL(k);
  DSA_NONNULL(v);
  DSA_NONNULL(idx);
  DSA_NONNULL(cu_seqlens);
  DSA_NONNULL(out);
  DSA_ALIGNED(q);
  DSA_ALIGNED(k);
  DSA_ALIGNED(v);
  DSA_ALIGNED(out);
  if (batch <= 0 || total_tokens < 0) return fail(DSA_ERR_INVALID_ARG, "batch must be positive, total_tokens >= 0");
  if (k_sel <= 0) return fail(DSA_ERR_INVALID_ARG, "k_sel must be positive");
  DSA_TRY(check_attn_shape(hq, hkv, head_dim));
  size_t need = 0;
  DSA_TRY(dsa_sparse_gqa_attn_dedup_workspace_size(total_tokens, k_sel, hq, hkv, &need));
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu bytes needed", workspace_bytes, need);
  if (need > 0) DSA_ALIGNED(workspace);
  if (total_tokens == 0) return DSA_OK;
  dsa::SparseAttnArgs a = {};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.idx = idx;
  a.k_sel = k_sel;
  a.cu_seqlens = cu_seqlens;
  a.batch = batch;
  a.seq_lens = nullptr;
  a.rows = total_tokens;
  a.hq = hq;
  a.hkv = hkv;
  a.softmax_scale = softmax_scale;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.nsplit = 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (need == 0) DSA_LAUNCH_RETURN("sparse_attn", s, dsa::launch_sparse_attn(a, s));
  return hip_status(launch_attn_dedup(a, workspace, s), "dedup attention launch");
}

int dsa_sparse_gqa_attn_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
                            const void* dout, const int32_t* idx, int k_sel, const int32_t* cu_seqlens, int batch,
                            int total_tokens, int hq, int hkv, int head_dim, float softmax_scale, float* dq,
                            float* dk, float* dv, void* stream) {
  g_last_error[0] = 0;
  const dsa::ApiRange range_("dsa_sparse_gqa_attn_bwd");
  dsa::api_log("dsa_sparse_gqa_attn_bwd", "batch=%d total=%d hq=%d hkv=%d k_sel=%d", batch, total_tokens, hq, hkv, k_sel);
  DSA_NONNULL(q);
  DSA_NONNULL(k);
  DSA_NONNULL(v);
  DSA_NONNULL(out);
  DSA_NONNULL(lse);
  DSA_NONNULL(dout);
  DSA_NONNULL(idx);
  DSA_NONNULL(cu_seqlens);
  DSA_NONNULL(dq);
  DSA_NONNULL(dk);
  DSA_NONNULL(dv);
  DSA_ALIGNED(q);
  DSA_ALIGNED(k);
  DSA_ALIGNED(v);
  DSA_ALIGNED(out);
  DSA_ALIGNED(dout);
  DSA_ALIGNED(dq);
  DSA_ALIGNED(dk);
  DSA_ALIGNED(dv);
  if (batch <= 0 || total_tokens < 0) return fail(DSA_ERR_INVALID_ARG, "batch must be positive, total_tokens >= 0");
  if (k_sel <= 0) return fail(DSA_ERR_INVALID_ARG, "k_sel must be positive");
  DSA_TRY(check_attn_shape(hq, hkv, head_dim));
  if (total_tokens == 0) return DSA_OK;
  dsa::SparseAttnBwdArgs a = {};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.out = static_cast<const uint16_t*>(out);
  a.dout = static_cast<const uint16_t*>(dout);
  a.lse = lse;
  a.idx = idx;
  a.k_sel = k_sel;
  a.cu_seqlens = cu_seqlens;
  a.batch = batch;
  a.rows = total_tokens;
  a.hq = hq;
  a.hkv = hkv;
  a.softmax_scale = softmax_scale;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  DSA_LAUNCH_RETURN("sparse_attn_bwd", static_cast<hipStream_t>(stream),
                    dsa::launch_sparse_attn_bwd(a, static_cast<hipStream_t>(stream)));
}

int dsa_sparse_gqa_attn_bwd_dedup_workspace_size(int total_tokens, int k_sel, int hq, int hkv, size_t* bytes) {
  g_last_error[0] = 0;
  DSA_NONNULL(bytes);
  if (total_tokens < 0 || k_sel <= 0) return fail(DSA_ERR_INVALID_ARG, "total_tokens >= 0 and k_sel > 0 required");
  if (k_sel > (1 << 24)) return fail(DSA_ERR_UNSUPPORTED, "k_sel %d too large", k_sel);
  *bytes = dsa::union_bwd_supported(hq, hkv) ? union_bwd_layout(total_tokens, k_sel, hq, hkv).bytes : 0;
  return DSA_OK;
}

int dsa_sparse_gqa_attn_bwd_dedup(const void* q, const void* k, const void* v, const void* out, const float* lse,
                                  const void* dout, const int32_t* idx, int k_sel, const int32_t* cu_seqlens,
                                  int batch, int total_tokens, int hq, int hkv, int head_dim, float softmax_scale,
                                  float* dq, float* dk, float* dv, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  g_last_error[0] = 0;
  const dsa::ApiRange range_("dsa_sparse_gqa_attn_bwd_dedup");
  dsa::api_log("dsa_sparse_gqa_attn_bwd_dedup", "batch=%d total=%d hq=%d hkv=%d k_sel=%d ws=%zu", batch, total_tokens,
               hq, hkv, k_sel, workspace_bytes);
  DSA_NONNULL(q);
  DSA_NONNULL(k);
  DSA_NONNULL(v);
  DSA_NONNULL(out);
  DSA_NONNULL(lse);
  DSA_NONNULL(dout);
  DSA_NONNULL(idx);
  DSA_NONNULL(cu_seqlens);
  DSA_NONNULL(dq);
  DSA_NONNULL(dk);
  DSA_NONNULL(dv);
  DSA_ALIGNED(q);
  DSA_ALIGNED(k);
  DSA_ALIGNED(v);
  DSA_ALIGNED(out);
  DSA_ALIGNED(dout);
  DSA_ALIGNED(dq);
  DSA_ALIGNED(dk);
  DSA_ALIGNED(dv);
  if (batch <= 0 || total_tokens < 0) return fail(DSA_ERR_INVALID_ARG, "batch must be positive, total_tokens >= 0");
  if (k_sel <= 0) return fail(DSA_ERR_INVALID_ARG, "k_sel must be positive");
  DSA_TRY(check_attn_shape(hq, hkv, head_dim));
  size_t need = 0;
  DSA_TRY(dsa_sparse_gqa_attn_bwd_dedup_workspace_size(total_tokens, k_sel, hq, hkv, &need));
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu bytes needed", workspace_bytes, need);
  if (need > 0) DSA_ALIGNED(workspace);
  if (total_tokens == 0) return DSA_OK;
  dsa::SparseAttnBwdArgs a = {};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.out = static_cast<const uint16_t*>(out);
  a.dout = static_cast<const uint16_t*>(dout);
  a.lse = lse;
  a.idx = idx;
  a.k_sel = k_sel;
  a.cu_seqlens = cu_seqlens;
  a.batch = batch;
  a.rows = total_tokens;
  a.hq = hq;
  a.hkv = hkv;
  a.softmax_scale = softmax_scale;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (need == 0) DSA_LAUNCH_RETURN("sparse_attn_bwd", s, dsa::launch_sparse_attn_bwd(a, s));
  return hip_status(launch_attn_bwd_dedup(a, workspace, s), "dedup attention backward launch");
}

int dsa_prefill_workspace_size(int batch, int total_tokens, int max_seqlen, int hq, int hkv, int head_dim, int h_idx,
                               int d_idx, int top_k, size_t* bytes) {
  g_last_error[0] = 0;
  DSA_NONNULL(bytes);
  if (batch <= 0 || total_tokens < 0 || max_seqlen < 0)
    return fail(DSA_ERR_INVALID_ARG, "batch must be positive, sizes non-negative");
  DSA_TRY(check_attn_shape(hq, hkv, head_dim));
  DSA_TRY(check_indexer_shape(h_idx, d_idx));
  DSA_TRY(check_topk(top_k));
  const long long ld = round_up(std::max(max_seqlen, 1), 4);
  const int rows = std::max(1, std::min(total_tokens, kDefaultChunkRows));
  // The dedup attention's merged sets use the same memory once the chunk loop is over.
  const size_t dedup = dsa::union_attn_supported(hq, hkv, total_tokens) ? union_layout(total_tokens, top_k).bytes : 0;
  *bytes = std::max(prefill_chunk_bytes(rows, ld), dedup);
  return DSA_OK;
}

int dsa_prefill(const void* q, const void* k, const void* v, const void* q_idx, const void* k_idx, const float* w,
                const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int batch, int total_tokens,
                int max_seqlen, int hq, int hkv, int head_dim, int h_idx, int d_idx, int top_k, float softmax_scale,
                void* out, float* lse, int32_t* idx_out, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  const dsa::ApiRange range_("dsa_prefill");
  dsa::api_log("dsa_prefill", "batch=%d total=%d max_seqlen=%d hq=%d hkv=%d h_idx=%d d_idx=%d top_k=%d ws=%zu", batch, total_tokens, max_seqlen, hq, hkv, h_idx, d_idx, top_k, workspace_bytes);
  DSA_NONNULL(q);
  DSA_NONNULL(k);
  DSA_NONNULL(v);
  DSA_NONNULL(q_idx);
  DSA_NONNULL(k_idx);
  DSA_NONNULL(w);
  DSA_NONNULL(cu_seqlens);
  DSA_NONNULL(out);
  DSA_NONNULL(idx_out);
  DSA_ALIGNED(q);
  DSA_ALIGNED(k);
  DSA_ALIGNED(v);
  DSA_ALIGNED(q_idx);
  DSA_ALIGNED(k_idx);
  DSA_ALIGNED(w);
  DSA_ALIGNED(out);
  DSA_ALIGNED(workspace);
  if (total_tokens < 0) return fail(DSA_ERR_INVALID_ARG, "total_tokens must be non-negative");
  DSA_TRY(check_attn_shape(hq, hkv, head_dim));
  DSA_TRY(check_indexer_shape(h_idx, d_idx));
  DSA_TRY(check_topk(top_k));
  int max_len = 0;
  DSA_TRY(check_cu_host(cu_seqlens_host, batch, total_tokens, &max_len));
  if (max_seqlen < max_len)
    return fail(DSA_ERR_INVALID_ARG, "max_seqlen (%d) is below the longest sequence (%d)", max_seqlen, max_len);
  if (total_tokens == 0) return DSA_OK;
  const long long ld = round_up(std::max(max_seqlen, 1), 4);
  const int min_rows = std::min(total_tokens, kMinChunkRows);
  if (!workspace || workspace_bytes < prefill_chunk_bytes(min_rows, ld))
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu bytes of the smallest chunk (%d rows)",
                workspace_bytes, prefill_chunk_bytes(min_rows, ld), min_rows);
  // Largest chunk of at most kDefaultChunkRows rows (a multiple of 64 when above 64 and short of
  // all rows) whose scores and top-k scratch fit (larger chunks measured slower).
  long long chunk = std::min<long long>(std::min(total_tokens, kDefaultChunkRows), (long long)(workspace_bytes / (ld * 4)));
  while (chunk > min_rows && prefill_chunk_bytes((int)chunk, ld) > workspace_bytes) --chunk;
  if (chunk > 64 && chunk < total_tokens) chunk = chunk / 64 * 64;  // (one chunk for everything: as is)
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* scores = static_cast<float*>(workspace);
  void* topk_ws = topk_scratch((int)chunk, ld)
                      ? static_cast<void*>(static_cast<char*>(workspace) + round_up(chunk * ld * 4, 256))
                      : nullptr;

  for (int b = 0; b < batch; ++b) {
    const int o = cu_seqlens_host[b], e = cu_seqlens_host[b + 1];
    for (int c0 = o; c0 < e; c0 += (int)chunk) {
      const int c1 = (int)std::min<long long>(e, c0 + chunk);
      dsa::TopkArgs t;
      t.scores = scores;
      t.ld = ld;
      t.rows = c1 - c0;
      t.row_len = nullptr;
      t.len_base = c0 - o;
      t.k = top_k;
      t.idx_out = idx_out + (size_t)c0 * top_k;
      t.values_out = nullptr;
      t.workspace = topk_ws;
      // Fused top-k (64-head indexer, more than 512 rows): a sampling indexer pass, the threshold
      // from its samples, the indexer pass that appends the candidates (no scores written), the
      // select; a row whose candidates under- or overflowed is then scored into the chunk's score
      // rows and selected exactly from them (two launches that find nothing to do when no row
      // failed).  Otherwise: the indexer, then threshold / collect / select over the scores.
      if (topk_ws && dsa::indexer_emit_supported(h_idx, d_idx) && c1 - c0 > 512) {
        const dsa::TopkScratch ts = dsa::topk_wave_scratch(topk_ws, c1 - c0);
        DSA_TRY(launch_index_rows(q_idx, k_idx, w, cu_seqlens_host, batch, h_idx, d_idx, c0, c1, c0, scores, ld, s, 1,
                                  &ts, top_k));
        DSA_LAUNCH("topk_threshold", s, dsa::launch_topk_wave_threshold_from_samples(t, s));
        DSA_TRY(launch_index_rows(q_idx, k_idx, w, cu_seqlens_host, batch, h_idx, d_idx, c0, c1, c0, scores, ld, s, 2,
                                  &ts, top_k));
        DSA_LAUNCH("topk_select", s, dsa::launch_topk_wave_select(t, s));
        DSA_TRY(launch_index_rows(q_idx, k_idx, w, cu_seqlens_host, batch, h_idx, d_idx, c0, c1, c0, scores, ld, s, 3,
                                  &ts, top_k));
        DSA_LAUNCH("topk_redo", s, dsa::launch_topk_wave_redo(t, s));
      } else {
        DSA_TRY(launch_index_rows(q_idx, k_idx, w, cu_seqlens_host, batch, h_idx, d_idx, c0, c1, c0, scores, ld, s));
        DSA_LAUNCH("topk", s, dsa::launch_topk(t, s));
      }
    }
  }
  dsa::SparseAttnArgs a = {};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.idx = idx_out;
  a.k_sel = top_k;
  a.cu_seqlens = cu_seqlens;
  a.batch = batch;
  a.seq_lens = nullptr;
  a.rows = total_tokens;
  a.hq = hq;
  a.hkv = hkv;
  a.softmax_scale = softmax_scale;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.nsplit = 1;
  // With room for the merged sets (they reuse the chunk memory, no longer needed), the attention
  // runs with adjacent-query dedup; otherwise per row.
  if (dsa::union_attn_supported(hq, hkv, total_tokens) && workspace_bytes >= union_layout(total_tokens, top_k).bytes)
    return hip_status(launch_attn_dedup(a, workspace, s), "dedup attention launch");
  DSA_LAUNCH_RETURN("sparse_attn", s, dsa::launch_sparse_attn(a, s));
}

int dsa_decode_workspace_size(int batch, int s_max, int hq, int hkv, int head_dim, int h_idx, int d_idx, int top_k,
                              size_t* bytes) {
  g_last_error[0] = 0;
  DSA_NONNULL(bytes);
  if (batch <= 0 || s_max <= 0) return fail(DSA_ERR_INVALID_ARG, "batch and s_max must be positive");
  DSA_TRY(check_attn_shape(hq, hkv, head_dim));
  DSA_TRY(check_indexer_shape(h_idx, d_idx));
  DSA_TRY(check_topk(top_k));
  const long long ld = round_up(s_max, 4);
  const long long score_bytes = (long long)batch * ld * 4;
  const size_t part_bytes = decode_attn_part_bytes(batch, hq, decode_nsplit(batch, hkv, top_k));
  *bytes = (size_t)round_up(score_bytes, 256) + topk_scratch(batch, ld) + part_bytes;
  return DSA_OK;
}

int dsa_decode(const void* q, const void* q_idx, const float* w, const void* k_cache, const void* v_cache,
               const void* k_idx_cache, const int32_t* seq_lens, int batch, int s_max, int max_seq_len, int hq,
               int hkv, int head_dim, int h_idx, int d_idx, int top_k, float softmax_scale, void* out, float* lse,
               int32_t* idx_out, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  const dsa::ApiRange range_("dsa_decode");
  dsa::api_log("dsa_decode", "batch=%d s_max=%d max_seq_len=%d hq=%d hkv=%d h_idx=%d d_idx=%d top_k=%d ws=%zu", batch, s_max, max_seq_len, hq, hkv, h_idx, d_idx, top_k, workspace_bytes);
  DSA_NONNULL(q);
  DSA_NONNULL(q_idx);
  DSA_NONNULL(w);
  DSA_NONNULL(k_cache);
  DSA_NONNULL(v_cache);
  DSA_NONNULL(k_idx_cache);
  DSA_NONNULL(seq_lens);
  DSA_NONNULL(out);
  DSA_NONNULL(idx_out);
  DSA_ALIGNED(q);
  DSA_ALIGNED(q_idx);
  DSA_ALIGNED(w);
  DSA_ALIGNED(k_cache);
  DSA_ALIGNED(v_cache);
  DSA_ALIGNED(k_idx_cache);
  DSA_ALIGNED(out);
  DSA_ALIGNED(workspace);
  if (batch <= 0 || s_max <= 0) return fail(DSA_ERR_INVALID_ARG, "batch and s_max must be positive");
  if (max_seq_len <= 0 || max_seq_len > s_max)
    return fail(DSA_ERR_INVALID_ARG, "max_seq_len (%d) must be in [1, s_max = %d]", max_seq_len, s_max);
  DSA_TRY(check_attn_shape(hq, hkv, head_dim));
  DSA_TRY(check_indexer_shape(h_idx, d_idx));
  DSA_TRY(check_topk(top_k));
  size_t need = 0;
  DSA_TRY(dsa_decode_workspace_size(batch, s_max, hq, hkv, head_dim, h_idx, d_idx, top_k, &need));
  if (!workspace || workspace_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu bytes needed", workspace_bytes, need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const long long ld = round_up(s_max, 4);
  float* scores = static_cast<float*>(workspace);
  char* after_scores = static_cast<char*>(workspace) + round_up((long long)batch * ld * 4, 256);
  void* topk_ws = topk_scratch(batch, ld) ? static_cast<void*>(after_scores) : nullptr;
  void* part = after_scores + topk_scratch(batch, ld);

  dsa::IndexerDecodeArgs ia;
  ia.q_idx = static_cast<const uint16_t*>(q_idx);
  ia.w = w;
  ia.k_cache = static_cast<const uint16_t*>(k_idx_cache);
  ia.seq_lens = seq_lens;
  ia.batch = batch;
  ia.s_max = s_max;
  ia.max_len = max_seq_len;
  ia.h_idx = h_idx;
  ia.d_idx = d_idx;
  ia.scores = scores;
  ia.ld = ld;
  DSA_LAUNCH("indexer_decode", s, dsa::launch_indexer_decode(ia, s));

  dsa::TopkArgs t;
  t.scores = scores;
  t.ld = ld;
  t.rows = batch;
  t.row_len = seq_lens;
  t.len_base = 0;
  t.k = top_k;
  t.idx_out = idx_out;
  t.values_out = nullptr;
  t.workspace = topk_ws;
  DSA_LAUNCH("topk", s, dsa::launch_topk(t, s));

  return hip_status(launch_decode_attn(q, k_cache, v_cache, idx_out, top_k, seq_lens, batch, s_max, hq, hkv,
                                       softmax_scale, out, lse, part, s),
                    "decode attention launch");
}

int dsa_sparse_gqa_attn_decode_workspace_size(int batch, int hq, int hkv, int k_sel, size_t* bytes) {
  g_last_error[0] = 0;
  DSA_NONNULL(bytes);
  if (batch <= 0 || k_sel <= 0) return fail(DSA_ERR_INVALID_ARG, "batch and k_sel must be positive");
  DSA_TRY(check_attn_shape(hq, hkv, 128));
  *bytes = decode_attn_part_bytes(batch, hq, decode_nsplit(batch, hkv, k_sel));
  return DSA_OK;
}

int dsa_sparse_gqa_attn_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* idx, int k_sel,
                               const int32_t* seq_lens, int batch, int s_max, int hq, int hkv, int head_dim,
                               float softmax_scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                               void* stream) {
  g_last_error[0] = 0;
  const dsa::ApiRange range_("dsa_sparse_gqa_attn_decode");
  dsa::api_log("dsa_sparse_gqa_attn_decode", "batch=%d s_max=%d hq=%d hkv=%d k_sel=%d ws=%zu", batch, s_max, hq, hkv,
               k_sel, workspace_bytes);
  DSA_NONNULL(q);
  DSA_NONNULL(k_cache);
  DSA_NONNULL(v_cache);
  DSA_NONNULL(idx);
  DSA_NONNULL(seq_lens);
  DSA_NONNULL(out);
  DSA_ALIGNED(q);
  DSA_ALIGNED(k_cache);
  DSA_ALIGNED(v_cache);
  DSA_ALIGNED(out);
  DSA_ALIGNED(workspace);
  if (batch <= 0 || s_max <= 0) return fail(DSA_ERR_INVALID_ARG, "batch and s_max must be positive");
  if (k_sel <= 0) return fail(DSA_ERR_INVALID_ARG, "k_sel must be positive");
  DSA_TRY(check_attn_shape(hq, hkv, head_dim));
  const size_t need = decode_attn_part_bytes(batch, hq, decode_nsplit(batch, hkv, k_sel));
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu bytes needed", workspace_bytes, need);
  return hip_status(launch_decode_attn(q, k_cache, v_cache, idx, k_sel, seq_lens, batch, s_max, hq, hkv,
                                       softmax_scale, out, lse, workspace, static_cast<hipStream_t>(stream)),
                    "decode attention launch");
}

}  // extern "C"

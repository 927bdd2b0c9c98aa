// Internal launch interface between the C ABI (dsa_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// Scores of packed rows [row_begin, row_end), all in one sequence that starts at packed row
// seq_off, written to scores[(r - out_row0) * ld + s] for s <= r - seq_off.
struct IndexerPrefillArgs {
  const uint16_t* q_idx;
  const uint16_t* k_idx;
  const float* w;
  int h_idx, d_idx;
  int seq_off, row_begin, row_end, out_row0;
  float* scores;
  long long ld;
  int key_split;  // keys per workgroup, multiple of 64
};

struct IndexerDecodeArgs {
  const uint16_t* q_idx;
  const float* w;
  const uint16_t* k_cache;
  const int* seq_lens;
  int batch, s_max, max_len, h_idx, d_idx;
  float* scores;
  long long ld;
};

// Row lengths come from row_len[i] if non-null, else len_base + i + 1 (causal prefill rows).
struct TopkArgs {
  const float* scores;
  long long ld;
  int rows;
  const int* row_len;
  int len_base;
  int k;
  int* idx_out;       // [rows, k] at row stride k
  float* values_out;  // optional
  void* workspace;    // >= topk_wave_workspace_bytes(rows) selects the wave-parallel kernels; may be null
};

// Scratch of the wave-parallel top-k (per-row threshold, counter and candidate list).
size_t topk_wave_workspace_bytes(int rows);
// Its layout: tau_lo [rows] uint32, cnt [rows] uint32, fail [rows] uint32 (the fused form's
// redo flags), then (256-byte aligned) cand [rows, kTopkCandCap] (key, position) pairs.
constexpr int kTopkCandCap = 8192;
struct TopkScratch {
  uint32_t* tau_lo;
  uint32_t* cnt;
  uint32_t* fail;
  uint2* cand;
};
TopkScratch topk_wave_scratch(void* workspace, int rows);
// The prefill's fused top-k (no collect pass, no scores written): the sampling indexer pass
// leaves, per row with more than k positions, m <= 2048 sample scores as floats at the start of
// the row's candidate list and m in tau_lo; this threshold launch turns them into tau_lo (and
// clears cnt and fail), the emitting indexer pass appends the candidates itself, and the select
// launch finishes every row whose list holds k to kTopkCandCap entries and sets fail for the
// others.  The rescoring indexer pass then writes the flagged rows' scores (a.scores) and the
// redo launch selects those rows exactly from them; both find nothing to do when no row failed.
// Rows must be more than 512 (the sample size of the few-row form differs); no values_out.
hipError_t launch_topk_wave_threshold_from_samples(const TopkArgs& a, hipStream_t s);
hipError_t launch_topk_wave_select(const TopkArgs& a, hipStream_t s);
hipError_t launch_topk_wave_redo(const TopkArgs& a, hipStream_t s);
// Longest row (ld) the wave-parallel top-k handles; longer rows use the row-block kernel.
constexpr long long kTopkWaveMaxLd = 262144;
hipError_t launch_topk_wave(const TopkArgs& a, hipStream_t s);

// Row r: prefill mode (seq_lens == nullptr) finds its sequence in cu_seqlens, decode mode uses
// sequence r with kv rows starting at r * s_max and valid length seq_lens[r].
struct SparseAttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int* idx;
  int k_sel;
  const int* cu_seqlens;
  int batch;
  const int* seq_lens;
  int s_max;
  int rows, hq, hkv;
  float softmax_scale;
  uint16_t* out;
  float* lse;
  int nsplit;       // > 1: write partials to part_o / part_ml instead of out / lse
  float* part_o;    // [rows, hq, nsplit, 128]
  float* part_ml;   // [rows, hq, nsplit, 2] (running max in log2 units, sum)
  const int* skip_block;  // prefill, optional: rows of blocks b (skip_block_rows rows each) with
  int skip_block_rows;    // skip_block[b] != 0 are left alone
};

// Backward of the sparse attention (prefill layout): dq written, dk / dv zeroed then accumulated.
struct SparseAttnBwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* out;   // forward output O
  const uint16_t* dout;  // dL/dO
  const float* lse;      // forward log-sum-exp (natural log)
  const int* idx;
  int k_sel;
  const int* cu_seqlens;
  int batch;
  int rows, hq, hkv;
  float softmax_scale;
  float* dq;  // [rows, hq, 128]
  float* dk;  // [rows, hkv, 128]
  float* dv;  // [rows, hkv, 128]
  const int* skip_block;  // optional: rows of blocks b (skip_block_rows rows each) with
  int skip_block_rows;    // skip_block[b] != 0 are left alone (dk / dv are then not zeroed)
};

// Backward of the indexer scores for packed rows [row_begin, row_end) of one sequence starting at
// packed row seq_off (64 heads x 128 only).  g[(r - grad_row0) * ld + s] is the gradient of
// I[r, s]; dq / dw of the rows are written, dk of the sequence's keys accumulated.
struct IndexerBwdArgs {
  const uint16_t* q_idx;
  const uint16_t* k_idx;
  const float* w;
  const float* g;
  long long ld;
  int seq_off, row_begin, row_end, grad_row0;
  float* dq;
  float* dw;
  float* dk;
};

// Head-mean causal attention distribution of packed rows [row_begin, row_end) of one sequence
// starting at packed row seq_off: probs[(r - out_row0) * ld + s] for s <= r - seq_off, and the
// per-head log-sum-exp lse[(r - out_row0) * hq + h].  Requires hq / hkv >= 4.
struct HeadMeanArgs {
  const uint16_t* q;
  const uint16_t* k;
  int hq, hkv;
  int seq_off, row_begin, row_end, out_row0;
  float softmax_scale;
  float* lse;
  float* probs;
  long long ld;
};

// Adjacent-query dedup.  Block b = packed rows R b .. R b + R - 1 with R = block_rows, 8 or 16
// (the last block may be shorter).  Its merged list has counts[b] entries at kv_rows / masks +
// b * cap: packed KV rows in ascending order and 16-bit masks (bit j: row R b + j selected the
// KV row), padded with mask-0 entries to a multiple of kUnionChunk.  cap must be a multiple of
// kUnionChunk and at least R * k_sel rounded up to one.  With masks32 set instead of masks, the
// masks are 32-bit and R may be any of 1 .. 32 (the attention backward's blocks).
constexpr int kMaxQueryBlock = 32;
constexpr int kUnionChunk = 32;
inline bool union_block_rows_ok(int r) { return r == 8 || r == 16; }
struct QueryUnionArgs {
  const int* idx;
  int k_sel;
  const int* cu_seqlens;
  int batch;
  int rows;                     // packed rows in all (for the last, shorter block)
  int block_rows;               // R
  int block_begin, block_end;   // blocks built by this launch
  int cap;
  int* counts;
  int* kv_rows;
  uint16_t* masks;
  uint32_t* masks32;  // set (and masks NULL) for 32-bit masks
  // Optional: use_union[b] = 1 when the merged set is at most ratio x (rows x k_sel) entries,
  // i.e. when the merged-set attention is expected to beat the per-row one for the block, and
  // no row of the block lists a position twice.
  int* use_union;
  float ratio;
};
struct UnionAttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int* counts;
  const int* kv_rows;
  const uint16_t* masks;
  int cap;
  int block_rows;
  int rows, hq, hkv;
  float softmax_scale;
  uint16_t* out;
  float* lse;
  const int* use_union;  // optional: blocks with use_union[b] == 0 are left alone
};
// Backward of the sparse attention over merged sets (32-bit masks) of blocks of
// union_bwd_block_rows(hq / hkv) rows: dq of the blocks' rows written, their dk / dv
// contributions added to dk / dv (which the caller has zeroed).
struct UnionBwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* out;
  const uint16_t* dout;
  const float* lse;
  const int* counts;
  const int* kv_rows;
  const uint32_t* masks;
  int cap;
  const int* use_union;  // optional: blocks with use_union[b] == 0 are left alone
  int rows, hq, hkv;
  float softmax_scale;
  float* dq;
  float* dk;
  float* dv;
};
// hq / hkv in {4, 8, 16}; blocks of 32 rows (16 at hq / hkv = 16), so a block's (row, head)
// pairs of one KV group number 128 or 256.
bool union_bwd_supported(int hq, int hkv);
int union_bwd_block_rows(int g);
hipError_t launch_sparse_attn_bwd_union(const UnionBwdArgs& a, hipStream_t s);
hipError_t launch_zero_f32(float* p, long long n, hipStream_t s);

hipError_t launch_query_union(const QueryUnionArgs& a, hipStream_t s);
// The union attention handles G = hq / hkv in {4, 8, 16}.
bool union_attn_supported(int hq, int hkv, long long rows);
hipError_t launch_sparse_attn_union(const UnionAttnArgs& a, hipStream_t s);

hipError_t launch_indexer_prefill(const IndexerPrefillArgs& a, hipStream_t s);
// The fused top-k's indexer passes (h_idx = 64, d_idx = 128 only; rows index the top-k scratch
// as packed row - out_row0): 2048 stratified sample scores per row (sample); every (key,
// position) at or above the row's tau_lo appended to its candidate list, no scores written
// (emit); the scores of the rows whose fail flag is set, as launch_indexer_prefill writes them
// (rescore: the other 4-row blocks return at once).
bool indexer_emit_supported(int h_idx, int d_idx);
hipError_t launch_indexer_prefill_sample(const IndexerPrefillArgs& a, const TopkScratch& t, int k, hipStream_t s);
hipError_t launch_indexer_prefill_emit(const IndexerPrefillArgs& a, const TopkScratch& t, int k, hipStream_t s);
hipError_t launch_indexer_prefill_rescore(const IndexerPrefillArgs& a, const TopkScratch& t, hipStream_t s);
hipError_t launch_attn_head_mean(const HeadMeanArgs& a, hipStream_t s);
// Row loss KL(target || softmax(scores)) and grad = softmax(scores) - target (grad may alias
// scores); row lengths from row_len or len_base + row + 1.
hipError_t launch_indexer_kl(const float* scores, const float* target, long long ld, int rows, const int* row_len,
                             int len_base, float* row_loss, float* grad, hipStream_t s);
hipError_t launch_indexer_decode(const IndexerDecodeArgs& a, hipStream_t s);
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);
// Reorder each row's selected positions (idx_out, as launch_topk leaves them) by descending score,
// equal scores by ascending position; values_out (optional) gets the scores in that order.
hipError_t launch_topk_rank(const TopkArgs& a, hipStream_t s);
hipError_t launch_sparse_attn(const SparseAttnArgs& a, hipStream_t s);
hipError_t launch_attn_combine(const SparseAttnArgs& a, hipStream_t s);
hipError_t launch_sparse_attn_bwd(const SparseAttnBwdArgs& a, hipStream_t s);
hipError_t launch_indexer_bwd(const IndexerBwdArgs& a, hipStream_t s);

// Host-side status reporting shared by the entry points of every source file: records the
// message returned by dsa_last_error (and logs it under DSA_LOG), returns `status`.
int api_fail(int status, const char* fmt, ...);
void api_clear_error();
void api_log(const char* name, const char* fmt, ...);
// One library call as a roctx range (named after the entry point), so a profiler's marker trace
// shows each call around its kernels; without a profiler attached the calls do nothing.
struct ApiRange {
  explicit ApiRange(const char* name);
  ~ApiRange();
  ApiRange(const ApiRange&) = delete;
  ApiRange& operator=(const ApiRange&) = delete;
};

}  // namespace dsa

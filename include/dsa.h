/*
 * dsa.h - C ABI of the DSA (DeepSeek Sparse Attention, GQA form) hot path for AMD MI355X.
 *
 * The path, as the Keye-VL-2.0 report digest (mqxn.cn news 1966, section 一) describes it:
 * a light "Lightning Indexer" with an MQA-shared key scores every earlier position of each
 * query token, the 2048 best positions of the context are kept per token, and attention
 * runs only over those positions.  The same section (and the aihot summary of the report's
 * abstract) says the method was adapted to a GQA decoder: here every query head of every KV
 * group of a token uses the token's one index set.  The report runs it over packed
 * variable-length sequences (QbitAI re-post on news.chathome.org, training-infrastructure
 * paragraph) and needs a deterministic top-k (digest, section 八).
 *
 * The pages print no formula.  This library computes, for packed row r of sequence b
 * (offset o = cu_seqlens[b], local position t = r - o):
 *
 *   score   I[r, s] = sum_j w[r, j] * max(0, <q_idx[r, j, :], k_idx[o + s, :]>),  0 <= s <= t
 *   select  the k positions with the largest I (ties -> lower s), all of [0, t] if t+1 <= k,
 *           returned in ascending order and padded with -1
 *   attend  z_s = scale * <q[r, h, :], k[o + s, h / G, :]>,  O[r, h] = sum_s softmax(z)_s v[o + s, h / G]
 *           lse[r, h] = log(sum_s exp(z_s))   (natural log, includes the scale)
 *
 * Conventions shared by every call:
 *   - All pointers are device pointers unless the name ends in _host.  Tensors are dense,
 *     row-major, in the order of their shape.  bf16 tensors are passed as `const void*`
 *     (16-bit storage, round-to-nearest-even bf16).  `stream` is a hipStream_t (NULL = the
 *     default stream).
 *   - The caller owns every buffer, including the workspace and the KV cache.  The library
 *     allocates nothing, keeps no pointer after a call returns, and never synchronises: work
 *     is enqueued on `stream` and results are valid once the stream has passed the call.
 *     Inputs must stay unchanged until then.  Calls on different streams are independent.
 *   - Arguments are validated on the host before anything is enqueued; on any error nothing
 *     runs.  Errors: DSA_ERR_INVALID_ARG (null pointer, negative size, inconsistent
 *     cu_seqlens, misaligned pointer), DSA_ERR_UNSUPPORTED (a shape the library has no kernel
 *     for), DSA_ERR_WORKSPACE (workspace too small), DSA_ERR_HIP (a launch failed; the HIP
 *     error text is in dsa_last_error()).  Faults inside kernels are only visible at the next
 *     synchronisation of the stream.
 *   - Supported shapes: head_dim = 128; Hq % Hkv == 0 with 1 <= Hq / Hkv <= 16;
 *     (h_idx, d_idx) in {(4, 64), (16, 128), (32, 128), (64, 128)}; 1 <= top_k <= 2048.
 *     Every bf16/float pointer must be 16-byte aligned.
 *   - Positions are sequence-local.  Selected positions that lie outside the causal prefix
 *     [0, t] (or outside [0, seq_len) in decode) are ignored by the attention calls.
 *   - With DSA_LOG=1 in the environment every entry point logs its call (name and sizes) and
 *     every rejected call its reason, and every kernel launch it makes its name ("launch ..."),
 *     one line each on stderr.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 1
#define DSA_MAX_TOP_K 2048

enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1,
  DSA_ERR_UNSUPPORTED = 2,
  DSA_ERR_WORKSPACE = 3,
  DSA_ERR_HIP = 4
};

/* Version of this ABI (DSA_ABI_VERSION). */
int dsa_abi_version(void);

/* Static text for a status code. */
const char* dsa_status_string(int status);

/* Message of the last failing call made by this host thread ("" if none). */
const char* dsa_last_error(void);

/*
 * Launch timing, a diagnostic of the library's own kernel launches (for the benchmark's
 * per-kernel attribution of the fused calls; off by default).
 *
 * dsa_timing_enable(on)   waits for the launches recorded so far, clears the record and turns
 *                         timing on (on != 0) or off.  While on, each launch the library makes
 *                         is bracketed by two HIP events recorded on the launch's stream, and
 *                         its time is later added to the entry of its name ("indexer_emit",
 *                         "topk_select", "sparse_attn_union", ...; one name may cover a short
 *                         sequence of kernels, e.g. "topk").  The events cost a little time
 *                         between launches, so time throughput with timing off.
 * dsa_timing_count(n)     waits for every recorded launch (host-blocking), adds their times to
 *                         the record and returns the number of names in *n.
 * dsa_timing_entry(i, name, total_ms, launches)
 *                         entry i < n of the record as of the last dsa_timing_count: the name (a
 *                         static string owned by the library), the summed milliseconds and the
 *                         number of launches.  i out of range: DSA_ERR_INVALID_ARG.
 * Not thread-safe (one host thread drives timed calls); do not turn it on while a stream is
 * being captured into a graph.  Errors of the event calls: DSA_ERR_HIP.
 */
int dsa_timing_enable(int on);
int dsa_timing_count(int* n);
int dsa_timing_entry(int i, const char** name, double* total_ms, int64_t* launches);

/*
 * Lightning-indexer scores (digest section 一: light scout, MQA-shared key).
 *
 * q_idx   [total_tokens, h_idx, d_idx] bf16    indexer queries of every packed row
 * k_idx   [total_tokens, d_idx]        bf16    one indexer key per packed position
 * w       [total_tokens, h_idx]        float   per-row, per-head weights
 * cu_seqlens_host [batch + 1] int32 (host)     packed offsets, cu[0] = 0, cu[batch] = total_tokens
 * row_begin, row_count                         packed rows [row_begin, row_begin + row_count) to score
 * scores  [row_count, ld]              float   output: scores[i * ld + s] = I[row_begin + i, s] for
 *                                              0 <= s <= t (the row's local position); entries with
 *                                              s > t are left untouched.  ld >= t + 1 for every row,
 *                                              ld % 4 == 0.
 */
int dsa_index_scores(const void* q_idx, const void* k_idx, const float* w,
                     const int32_t* cu_seqlens_host, int batch, int total_tokens,
                     int h_idx, int d_idx, int row_begin, int row_count,
                     float* scores, int64_t ld, void* stream);

/*
 * Lightning-indexer scores of one new token per sequence against its cached keys (the decode
 * form of dsa_index_scores; digest section 一 for the indexer, section 八 for DSA-specific decode).
 *
 * q_idx   [batch, h_idx, d_idx] bf16       indexer query of each sequence's new token
 * w       [batch, h_idx]        float      its per-head weights
 * k_idx_cache [batch, s_max, d_idx] bf16   cached indexer keys; sequence b uses rows 0 .. seq_lens[b]-1
 * seq_lens [batch] int32 (device)          cache length of each sequence, including the new token;
 *                                          1 <= seq_lens[b] <= max_seq_len
 * max_seq_len (host)                       upper bound of seq_lens, 1 <= max_seq_len <= s_max (sizes the launch)
 * scores  [batch, ld]           float      output: scores[b * ld + s] = I[b, s] for 0 <= s < seq_lens[b];
 *                                          entries at s >= seq_lens[b] are left untouched.  ld >= s_max,
 *                                          ld % 4 == 0.
 * Same arithmetic as dsa_index_scores, so for the same bf16 values the scores are equal bit for bit.
 * dsa_decode runs exactly this step first, on the first batch * ld floats of its workspace.
 */
int dsa_decode_index_scores(const void* q_idx, const float* w, const void* k_idx_cache, const int32_t* seq_lens,
                            int batch, int s_max, int max_seq_len, int h_idx, int d_idx, float* scores, int64_t ld,
                            void* stream);

/*
 * Backward of dsa_index_scores (digest section 一: the dense warm-up trains the indexer, which
 * needs the gradient of its scores with respect to q_idx, k_idx and w).
 *
 * With c[r, j, s] = <q_idx[r, j], k_idx[o + s]> and g = dscores, for packed rows
 * [row_begin, row_begin + row_count) of sequences starting at o (local position t):
 *   dq_idx[r, j] = w[r, j] sum_{s<=t} g[r, s] [c > 0] k_idx[o + s]          (rows overwritten)
 *   dw[r, j]     = sum_{s<=t} g[r, s] max(0, c[r, j, s])                    (rows overwritten)
 *   dk_idx[o + s] += sum_r g[r, s] sum_j w[r, j] [c > 0] q_idx[r, j]        (accumulated)
 * dscores [row_count, ld] float, laid out as dsa_index_scores writes scores (row i = packed row
 *   row_begin + i, column s = local key position); entries with s > t are not read.
 * dq_idx [total_tokens, h_idx, d_idx], dw [total_tokens, h_idx], dk_idx [total_tokens, d_idx]
 *   float.  dk_idx is added to, so a pass over several row chunks zeroes it once first.
 * Arithmetic: c is recomputed on bf16 MFMA with fp32 accumulation ([c > 0] is the forward's
 *   ReLU decision); g [c > 0] (for dk_idx g w [c > 0]) is rounded to bf16 for the second
 *   contraction, fp32 accumulation.  dk_idx (and dq_idx / dw when a row's keys are split over
 *   workgroups) is summed with fp32 atomics, so its last bits can differ between runs.
 * Needs no workspace.  Supports h_idx = 64, d_idx = 128 (DSA_ERR_UNSUPPORTED otherwise).
 */
int dsa_index_scores_bwd(const void* q_idx, const void* k_idx, const float* w,
                         const int32_t* cu_seqlens_host, int batch, int total_tokens,
                         int h_idx, int d_idx, int row_begin, int row_count,
                         const float* dscores, int64_t ld,
                         float* dq_idx, float* dw, float* dk_idx, void* stream);

/*
 * Target of the indexer's dense warm-up (digest section 一: with the full attention unchanged,
 * the indexer is trained to follow the full attention distribution, measured by KL divergence).
 *
 * For packed rows [row_begin, row_begin + row_count) with local position t:
 *   probs[i * ld + s] = (1 / hq) sum_h softmax_s(scale <q[r, h], k[o + s, h / G]>)  for s <= t
 *   lse[i * hq + h]   = log sum_s exp(scale <q[r, h], k[o + s, h / G]>)  (the dense causal lse)
 * (i = r - row_begin).  Entries with s > t are left untouched (entries s <= t may hold scratch
 * values while the call runs).  q, k, cu_seqlens_host as for dsa_prefill / dsa_index_scores.
 * Needs hq / hkv in {4, 8, 12, 16} and hkv in {1, 2, 4, 8} (DSA_ERR_UNSUPPORTED otherwise).
 * Costs two dense passes of Q K^T over the causal prefix (statistics, then probabilities).
 */
int dsa_attn_head_mean(const void* q, const void* k, const int32_t* cu_seqlens_host, int batch,
                       int total_tokens, int hq, int hkv, int head_dim, float softmax_scale,
                       int row_begin, int row_count, float* probs, int64_t ld, float* lse,
                       void* stream);

/*
 * KL divergence from a target to the indexer's distribution, per row, with its gradient
 * (digest section 一, dense warm-up).
 *
 * scores, target [rows, ld] float: row i holds row_len[i] entries (indexer scores I and a
 *   target distribution p over the same positions).
 * row_loss [rows] float: sum_s p_s (log p_s - log r_s), r = softmax(I) over the row (terms with
 *   p_s = 0 are 0).
 * grad [rows, ld] float: d row_loss / d I_s = r_s - p_s; may alias scores.
 */
int dsa_indexer_kl(const float* scores, const float* target, int64_t ld, int rows,
                   const int32_t* row_len, float* row_loss, float* grad, void* stream);

/* Bytes of scratch the fast dsa_topk path uses for `rows` rows of stride ld (0 when ld > 262144,
 * where only the scratch-free path exists). */
int dsa_topk_workspace_size(int rows, int64_t ld, int k, size_t* bytes);

/*
 * Deterministic per-row top-k (digest section 一: k best positions per query; section 八:
 * identical sets in training and inference).
 *
 * scores  [rows, ld] float     row i holds row_len[i] valid scores in scores[i * ld + 0 .. row_len-1];
 *                              ld % 4 == 0.  Scores must not be NaN; -0.0 equals +0.0.
 * row_len [rows] int32         valid length of each row (>= 0, <= ld)
 * k                            1 <= k <= DSA_MAX_TOP_K
 * idx_out [rows, k] int32      output: the selected positions in ascending order; if row_len <= k
 *                              the row is 0 .. row_len-1; padding is -1.  Among equal scores the
 *                              lower position wins, so the set is unique.
 * values_out [rows, k] float   optional (NULL): the scores of idx_out, same order; padding -inf.
 * workspace, workspace_bytes   NULL, or at least dsa_topk_workspace_size bytes: with it, rows of
 *                              ld <= 262144 use the wave-parallel kernels (a sampled threshold, one
 *                              streaming pass, an exact select over the candidates); without it a
 *                              scratch-free row-per-workgroup kernel runs.  Both give the same result.
 *                              A non-NULL workspace below the needed size is DSA_ERR_WORKSPACE.
 */
int dsa_topk(const float* scores, int64_t ld, int rows, const int32_t* row_len, int k,
             int32_t* idx_out, float* values_out, void* workspace, size_t workspace_bytes,
             void* stream);

/*
 * Deterministic top-k in the shape of torch.topk(sorted=True) (digest section 八: a
 * deterministic top-k in place of torch.topk, so training and inference keep identical sets).
 *
 * Same arguments, workspace and set as dsa_topk; only the order differs.  idx_out[i, :] holds
 * the kept positions by descending score, equal scores by ascending position; values_out
 * (optional) the scores in that order, -0.0 returned as +0.0.  A row with row_len < k keeps all
 * its positions and is padded at the end with -1 (values -inf).
 */
int dsa_topk_sorted(const float* scores, int64_t ld, int rows, const int32_t* row_len, int k,
                    int32_t* idx_out, float* values_out, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * Sparse GQA attention over selected positions (digest section 一 and the GQA adaptation).
 *
 * q   [total_tokens, hq, head_dim]  bf16
 * k,v [total_tokens, hkv, head_dim] bf16
 * idx [total_tokens, k_sel] int32   sequence-local positions per row; entries < 0 or > t are ignored
 * cu_seqlens [batch + 1] int32      device copy of the packed offsets
 * out [total_tokens, hq, head_dim]  bf16 output.  A row with no valid position gets O = 0.
 * lse [total_tokens, hq] float      optional (NULL) output; -inf for a row with no valid position.
 */
int dsa_sparse_gqa_attn(const void* q, const void* k, const void* v,
                        const int32_t* idx, int k_sel,
                        const int32_t* cu_seqlens, int batch, int total_tokens,
                        int hq, int hkv, int head_dim, float softmax_scale,
                        void* out, float* lse, void* stream);

/*
 * Sparse GQA attention of one new token per sequence over selected positions of a contiguous KV
 * cache (the attention step of dsa_decode; digest section 八, DSA-specific decode).
 *
 * q   [batch, hq, head_dim] bf16              the new token of each sequence
 * k_cache, v_cache [batch, s_max, hkv, head_dim] bf16
 * idx [batch, k_sel] int32                   positions into cache[b, 0 : seq_lens[b]]; entries < 0 or
 *                                            >= seq_lens[b] are ignored
 * seq_lens [batch] int32 (device)            1 <= seq_lens[b] <= s_max
 * out [batch, hq, head_dim] bf16, lse [batch, hq] float or NULL   as for dsa_sparse_gqa_attn
 * workspace  at least dsa_sparse_gqa_attn_decode_workspace_size bytes (per-split partials; 0 bytes
 *            and NULL allowed when that size is 0), 16-byte aligned; contents on return unspecified.
 * The index entries of a sequence are split into ranges attended in parallel and merged by their
 * (max, sum) pairs, so the result equals dsa_sparse_gqa_attn's on the same positions up to rounding.
 */
int dsa_sparse_gqa_attn_decode_workspace_size(int batch, int hq, int hkv, int k_sel, size_t* bytes);
int dsa_sparse_gqa_attn_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* idx,
                               int k_sel, const int32_t* seq_lens, int batch, int s_max, int hq, int hkv,
                               int head_dim, float softmax_scale, void* out, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * Adjacent-query dedup, step 1 (digest section 八: neighbouring query tokens select largely the
 * same positions, so the top-k sets of 16 adjacent queries are de-duplicated and the attention
 * kernel masks inside its matrix tiles).
 *
 * Block b is packed rows R b .. R b + R - 1 with R = block_rows, 16 (the pages' count) or 8;
 * n_blocks = ceil(total_tokens / R); the last block may be shorter and a block may span two
 * sequences.  Entry p of row r (sequence offset o, local position t) counts when 0 <= p <= t and
 * names the packed KV row o + p; a position a row lists twice counts once.
 *
 * idx [total_tokens, k_sel] int32   as for dsa_sparse_gqa_attn (any order)
 * cu_seqlens [batch + 1] int32      device copy of the packed offsets
 * block_rows                        8 or 16 (DSA_ERR_UNSUPPORTED otherwise)
 * cap                               entries per block: a multiple of 32, at least R * k_sel
 *                                   rounded up to a multiple of 32 (dsa_query_union_size)
 * counts  [n_blocks] int32          out: number of distinct KV rows the block's rows selected
 * kv_rows [n_blocks, cap] int32     out: those packed KV rows in ascending order, followed by
 *                                   padding to a multiple of 32 entries (the offset of the block's
 *                                   first sequence); entries after the padding are not written
 * masks   [n_blocks, cap] uint16    out: bit j set when row R b + j selected the KV row; 0 in the
 *                                   padding
 * kv_rows must be 16-byte aligned, masks 4-byte aligned.
 */
int dsa_query_union_size(int total_tokens, int k_sel, int block_rows, int* n_blocks, int* cap);
int dsa_query_union(const int32_t* idx, int k_sel, const int32_t* cu_seqlens, int batch, int total_tokens,
                    int block_rows, int cap, int32_t* counts, int32_t* kv_rows, uint16_t* masks, void* stream);

/*
 * Adjacent-query dedup, step 2: sparse GQA attention from the merged sets dsa_query_union wrote.
 * Each KV row of a block's merged set is read once for all of the block's rows; row R b + j
 * attends over the KV rows whose mask has bit j, with the softmax of dsa_sparse_gqa_attn.  For
 * index sets that repeat no position the result is dsa_sparse_gqa_attn's (up to rounding).
 *
 * q, k, v, total_tokens, hq, hkv, head_dim, softmax_scale, out, lse   as for dsa_sparse_gqa_attn
 * counts, kv_rows, masks, block_rows, cap   as dsa_query_union wrote them (KV rows outside
 *                                   [0, total_tokens) are clamped into it, counts above cap read
 *                                   as cap, so no access leaves the buffers)
 * Supports hq / hkv in {4, 8, 16} and total_tokens * hkv < 2^24 (K and V rows are addressed
 * with 32-bit byte offsets; DSA_ERR_UNSUPPORTED otherwise).  Needs no workspace.
 */
int dsa_sparse_gqa_attn_union(const void* q, const void* k, const void* v, const int32_t* counts,
                              const int32_t* kv_rows, const uint16_t* masks, int block_rows, int cap,
                              int total_tokens, int hq, int hkv, int head_dim, float softmax_scale,
                              void* out, float* lse, void* stream);

/*
 * Sparse GQA attention with adjacent-query dedup: what dsa_sparse_gqa_attn computes (up to
 * rounding), with the same arguments plus a workspace.  The call builds the merged sets of every
 * block of 8 rows (dsa_query_union) in the workspace and attends each block from its merged set
 * (dsa_sparse_gqa_attn_union), except blocks in which a row lists a position twice, which are
 * attended per row (so that the repeat counts as dsa_sparse_gqa_attn counts it).  Where
 * dsa_sparse_gqa_attn_union does not apply (hq / hkv outside {4, 8, 16}, or total_tokens * hkv
 * >= 2^24) the workspace size is 0 and the call is dsa_sparse_gqa_attn.
 *
 * workspace  device buffer of at least dsa_sparse_gqa_attn_dedup_workspace_size bytes, 16-byte
 *            aligned (DSA_ERR_WORKSPACE if smaller); its contents on return are unspecified.
 */
int dsa_sparse_gqa_attn_dedup_workspace_size(int total_tokens, int k_sel, int hq, int hkv, size_t* bytes);
int dsa_sparse_gqa_attn_dedup(const void* q, const void* k, const void* v,
                              const int32_t* idx, int k_sel,
                              const int32_t* cu_seqlens, int batch, int total_tokens,
                              int hq, int hkv, int head_dim, float softmax_scale,
                              void* out, float* lse, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * Backward of dsa_sparse_gqa_attn (digest section 一: the sparse adaptation stage trains the
 * whole model in the sparse mode, so gradients pass through this attention).
 *
 * q, k, v, idx, k_sel, cu_seqlens, batch, total_tokens, hq, hkv, head_dim, softmax_scale
 *                                   as for the forward call
 * out  [total_tokens, hq, head_dim] bf16   the forward's output O
 * lse  [total_tokens, hq] float            the forward's log-sum-exp (required)
 * dout [total_tokens, hq, head_dim] bf16   gradient of the loss with respect to O
 * dq   [total_tokens, hq, head_dim] float  output, written
 * dk, dv [total_tokens, hkv, head_dim] float  outputs: zeroed by the call, then every
 *                                   (row, head, selected position) adds its contribution with
 *                                   float atomics, so the summation order (and the last bits)
 *                                   can vary from run to run.
 * The softmax weights are recomputed from lse; they and dZ are rounded to bf16 as MFMA
 * operands (fp32 accumulation).
 */
int dsa_sparse_gqa_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                            const float* lse, const void* dout, const int32_t* idx, int k_sel,
                            const int32_t* cu_seqlens, int batch, int total_tokens,
                            int hq, int hkv, int head_dim, float softmax_scale,
                            float* dq, float* dk, float* dv, void* stream);

/*
 * dsa_sparse_gqa_attn_bwd with adjacent-query dedup (digest section 八: adjacent queries select
 * largely the same positions).  The float-atomic adds of dk / dv bound the per-row backward, so
 * here the index sets of each block of 32 adjacent packed rows (16 when hq / hkv = 16) are merged
 * in the workspace, and every merged position's contributions are summed over the block's rows
 * and heads before they are added: one atomic per (merged position, KV head, dim) instead of one
 * per (row, selected entry, KV head, dim).  Blocks in which a row lists a position twice are done
 * per row (each entry counts once per occurrence, as in dsa_sparse_gqa_attn_bwd).
 *
 * Arguments as dsa_sparse_gqa_attn_bwd, plus:
 * workspace           device memory of at least
 *                     dsa_sparse_gqa_attn_bwd_dedup_workspace_size(total_tokens, k_sel, hq, hkv)
 *                     bytes, 16-byte aligned, owned by the caller, clobbered (per block a count, a
 *                     path flag, up to R x k_sel merged positions and 32-bit row masks: about
 *                     8 k_sel bytes per row).  When that size is 0 (hq / hkv not 4, 8 or 16) the
 *                     call is the per-row backward and the workspace may be NULL.
 * The result equals dsa_sparse_gqa_attn_bwd's up to the order of the float additions; dZ and P
 * enter the dk / dv products as bf16 in both.
 */
int dsa_sparse_gqa_attn_bwd_dedup_workspace_size(int total_tokens, int k_sel, int hq, int hkv,
                                                 size_t* bytes);
int dsa_sparse_gqa_attn_bwd_dedup(const void* q, const void* k, const void* v, const void* out,
                                  const float* lse, const void* dout, const int32_t* idx, int k_sel,
                                  const int32_t* cu_seqlens, int batch, int total_tokens,
                                  int hq, int hkv, int head_dim, float softmax_scale,
                                  float* dq, float* dk, float* dv, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * Workspace bytes for dsa_prefill: the larger of (a) a score buffer for a chunk of 2048 query
 * rows (never the whole L x L matrix) plus the top-k scratch of those rows and (b), when
 * hq / hkv is 4, 8 or 16, the merged index sets of dsa_sparse_gqa_attn_dedup, which reuse the
 * same memory after the last chunk.  A smaller workspace gives smaller chunks (down to 64 rows)
 * and, below (b), the attention without dedup.
 */
int dsa_prefill_workspace_size(int batch, int total_tokens, int max_seqlen, int hq, int hkv,
                               int head_dim, int h_idx, int d_idx, int top_k, size_t* bytes);

/*
 * Fused prefill: indexer -> top-k -> sparse GQA attention for every packed row.
 *
 * q, k, v, q_idx, k_idx, w      as above, over all total_tokens packed rows
 * cu_seqlens [batch + 1]        device copy of the packed offsets
 * cu_seqlens_host [batch + 1]   host copy of the same offsets (used to schedule chunks)
 * max_seqlen                    >= the longest sequence
 * out [total_tokens, hq, head_dim] bf16, lse [total_tokens, hq] float or NULL
 * idx_out [total_tokens, top_k] int32   the selected positions (required)
 * workspace                     the call uses the largest chunk of at most 2048 rows whose scores
 *                               and top-k scratch fit; it must hold at least a 64-row chunk (or all
 *                               rows if fewer).  When it also holds the merged index sets
 *                               (dsa_sparse_gqa_attn_dedup_workspace_size), the attention step is
 *                               dsa_sparse_gqa_attn_dedup, else dsa_sparse_gqa_attn; the two give
 *                               the same result up to rounding.  dsa_prefill_workspace_size gives
 *                               the size for both.
 */
int dsa_prefill(const void* q, const void* k, const void* v,
                const void* q_idx, const void* k_idx, const float* w,
                const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                int batch, int total_tokens, int max_seqlen,
                int hq, int hkv, int head_dim, int h_idx, int d_idx, int top_k,
                float softmax_scale, void* out, float* lse, int32_t* idx_out,
                void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes for dsa_decode (per-sequence score rows plus split partials). */
int dsa_decode_workspace_size(int batch, int s_max, int hq, int hkv, int head_dim,
                              int h_idx, int d_idx, int top_k, size_t* bytes);

/*
 * Fused decode step over a contiguous KV cache (digest section 八: DSA-specific decode).
 *
 * q [batch, hq, head_dim] bf16, q_idx [batch, h_idx, d_idx] bf16, w [batch, h_idx] float:
 *     the new token of each sequence
 * k_cache, v_cache [batch, s_max, hkv, head_dim] bf16, k_idx_cache [batch, s_max, d_idx] bf16
 * seq_lens [batch] int32 (device): valid cache length of each sequence, which already includes
 *     the new token at position seq_lens[b] - 1; 1 <= seq_lens[b] <= s_max
 * max_seq_len (host): an upper bound of seq_lens (used to size the launch)
 * out [batch, hq, head_dim] bf16, lse [batch, hq] float or NULL, idx_out [batch, top_k] int32
 */
int dsa_decode(const void* q, const void* q_idx, const float* w,
               const void* k_cache, const void* v_cache, const void* k_idx_cache,
               const int32_t* seq_lens, int batch, int s_max, int max_seq_len,
               int hq, int hkv, int head_dim, int h_idx, int d_idx, int top_k,
               float softmax_scale, void* out, float* lse, int32_t* idx_out,
               void* workspace, size_t workspace_bytes, void* stream);

/* Scratch bytes dsa_decode_noalloc holds per device (32 MiB). */
#define DSA_DECODE_NOALLOC_MAX_BYTES (32u << 20)

/*
 * dsa_decode for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments and results as
 * dsa_decode, without the workspace: the step's scratch is a static device array of
 * DSA_DECODE_NOALLOC_MAX_BYTES inside the library, one per device, held until the process ends.
 * The call allocates and frees nothing.
 *   - Uses the scratch of the current device (hipGetDevice); `stream` must belong to that device.
 *     The first call on a device looks the array's address up (no allocation).
 *   - Every call on a device shares that device's array and leaves its contents behind: calls
 *     that can overlap on one device (different streams, or different host threads) race and
 *     must be serialised by the caller.
 *   - A step whose dsa_decode_workspace_size exceeds DSA_DECODE_NOALLOC_MAX_BYTES is rejected with
 *     DSA_ERR_WORKSPACE before anything is enqueued (batch 32 x 131072 and batch 8 x 262144 caches
 *     at k = 2048 fit).
 */
int dsa_decode_noalloc(const void* q, const void* q_idx, const float* w,
                       const void* k_cache, const void* v_cache, const void* k_idx_cache,
                       const int32_t* seq_lens, int batch, int s_max, int max_seq_len,
                       int hq, int hkv, int head_dim, int h_idx, int d_idx, int top_k,
                       float softmax_scale, void* out, float* lse, int32_t* idx_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */

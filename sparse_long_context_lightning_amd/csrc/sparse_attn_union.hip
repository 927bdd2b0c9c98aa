// Sparse GQA attention over the merged index sets of adjacent query rows, for gfx950.
//
// Neighbouring query tokens select largely the same positions (Keye-VL-2.0 report digest,
// mqxn.cn news 1966, section 八: the top-k sets of adjacent queries are de-duplicated and the
// attention kernel masks inside its matrix tiles), so the sets of R consecutive packed rows
// (R = 16 as on that page, or 8) are merged, every KV row of the merged set is fetched once for
// all R rows, and a 16-bit mask per merged position keeps each row to its own positions.
//
// query_union_kernel: one workgroup per block of R rows.  Entry p of row r (sequence offset
// o, local position t) counts when 0 <= p <= t and names packed KV row o + p; bit j (row j of
// the block) is OR-ed into an R-bit-per-position bitmap in LDS (64 KiB: one window of 65536
// KV rows at R = 8, 32768 at R = 16, 16384 at R = 32), and each window is compacted in ascending order with
// ballots.  The list is padded to a multiple of 32 entries with (the block's smallest possible
// KV row, mask 0).
//
// sparse_attn_union_kernel: one workgroup of R / 4 waves per (block, KV group).  Per chunk of
// 32 merged positions the workgroup DMAs the 32 key rows and 32 value rows of the group into
// LDS (a ring of stages; a chunk's positions and masks arrive in an earlier stage, so the
// gather addresses are read from LDS), and each wave uses them for its 4 rows x G heads:
//   * S^T = K Q^T on 16x16x32 bf16 MFMA, keys on rows, (row, head) pairs on columns; with
//     G = 8 one 16-column tile is two rows' eight heads;
//   * online softmax in base 2 per column, its offset allowed to lag the largest logit by a
//     bounded margin so that the masked maximum is needed only when that margin is passed;
//   * the lane that holds P^T[key][column] keeps its bf16 weight only where the key's mask
//     carries the column's row bit (the "mask that knows the MFMA thread layout");
//   * O^T += V^T P^T with V^T read transposed from LDS (ds_read_b64_tr_b16) in the key order
//     the P^T registers carry, and the row sums on the same MFMA with a ones operand.
// The cost per block grows with R x |merged set| while the gathered bytes shrink with the
// overlap, so R trades compute against memory traffic.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kUnionThreads = 512;
// 64 KiB of LDS: 4 positions per dword at 8 rows, 2 at 16, 1 at 32.  Two workgroups fit a CU;
// with 128 KiB (one per CU, every window twice as long) the 128K prefill's builder took 1.35
// against 1.06 ms, with 32 / 16 KiB 1.08 / 1.27 ms.
constexpr int kBitmapWords = 16384;

__device__ __forceinline__ int seq_of_row(const int* cu, int batch, int r) {
  int lo = 0, hi = batch;  // largest s with cu[s] <= r
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ int lanes_below(uint64_t bal) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
}

// BPP bits per position (8 for blocks of up to 8 rows, 16 for up to 16, 32 for up to 32 with
// 32-bit masks): a window covers kBitmapWords * 32 / BPP KV rows.
template <int BPP>
__global__ __launch_bounds__(kUnionThreads) void query_union_kernel(QueryUnionArgs a) {
  constexpr int PPW = 32 / BPP;                  // positions per dword
  constexpr int kWindow = kBitmapWords * PPW;
  constexpr uint32_t kField = BPP == 8 ? 0xFFu : BPP == 16 ? 0xFFFFu : 0xFFFFFFFFu;
  typedef typename std::conditional<BPP == 32, uint32_t, uint16_t>::type MaskT;
  constexpr int kWaves = kUnionThreads / 64;
  __shared__ __attribute__((aligned(16))) uint32_t bm[kBitmapWords];
  __shared__ int row_base[kMaxQueryBlock], row_t[kMaxQueryBlock];
  __shared__ int wave_cnt[kWaves];
  __shared__ int wave_chk[kWaves][2];  // valid entries set and bits found, per wave
  const int b = a.block_begin + blockIdx.x;
  const int r0 = b * a.block_rows;
  const int nr = min(a.block_rows, a.rows - r0);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (tid < kMaxQueryBlock) {
    int base = 0, t = -1;
    if (tid < nr) {
      base = a.cu_seqlens[seq_of_row(a.cu_seqlens, a.batch, r0 + tid)];
      t = r0 + tid - base;
    }
    row_base[tid] = base;
    row_t[tid] = t;
  }
  __syncthreads();
  const int b0 = row_base[0];          // no entry of the block names a KV row below this one
  const int span = r0 + nr - b0;       // KV rows b0 .. r0 + nr - 1
  int* out_rows = a.kv_rows + (size_t)b * a.cap;
  MaskT* out_masks = reinterpret_cast<MaskT*>(BPP == 32 ? (void*)a.masks32 : (void*)a.masks) + (size_t)b * a.cap;
  int total = 0;
  // A row that lists a position twice sets one bit for two valid entries: the block repeats a
  // position exactly when the bits in its bitmaps number fewer than its valid entries, so the
  // bits are set with ORs that return nothing and counted in the compaction.
  int entries = 0, bits = 0;
  constexpr int kRowGroup = 8;                                    // rows whose entries are loaded together
  constexpr int kEpt = (kMaxTopK + kUnionThreads - 1) / kUnionThreads;  // entries per thread, row and pass
  for (int w0 = 0; w0 < span; w0 += kWindow) {
    const int lo = b0 + w0;
    const int limit = min(kWindow, span - w0);   // positions in this window
    const int words = (limit + PPW - 1) / PPW;
    for (int i = tid; i < (words + 3) / 4; i += kUnionThreads) reinterpret_cast<uint4*>(bm)[i] = uint4{0, 0, 0, 0};
    __syncthreads();
    for (int j0 = 0; j0 < nr; j0 += kRowGroup) {
      for (int c0 = 0; c0 < a.k_sel; c0 += kEpt * kUnionThreads) {
        // every load of the row group issued before any bit is set: one memory latency per group
        int pv[kRowGroup][kEpt];
#pragma unroll
        for (int jj = 0; jj < kRowGroup; ++jj)
#pragma unroll
          for (int e = 0; e < kEpt; ++e) {
            const int j = j0 + jj, i = c0 + e * kUnionThreads + tid;
            pv[jj][e] = (j < nr && i < a.k_sel) ? a.idx[(size_t)(r0 + j) * a.k_sel + i] : -1;
          }
#pragma unroll
        for (int jj = 0; jj < kRowGroup; ++jj) {
          const int j = j0 + jj;
          if (j >= nr) break;
          const int off = row_base[j] - lo, t = row_t[j];
#pragma unroll
          for (int e = 0; e < kEpt; ++e) {
            const int p = pv[jj][e];
            const int x = off + p;
            if (p >= 0 && p <= t && x >= 0 && x < limit) {
              const uint32_t bit = 1u << ((BPP == 32 ? 0 : BPP * (x % PPW)) + j);
              __hip_atomic_fetch_or(&bm[x / PPW], bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
              ++entries;
            }
          }
        }
      }
    }
    __syncthreads();
    // Compaction, one dword (PPW positions) per lane and step; wave w takes a contiguous share.
    // A lane's entry count c (at most PPW) is split into bits, one ballot each, for the prefix.
    const int per_wave = (words + kWaves - 1) / kWaves;
    const int s_begin = wave * per_wave, s_end = min(s_begin + per_wave, words);
    auto nz_count = [&](uint32_t wd) {
      int c = 0;
#pragma unroll
      for (int f = 0; f < PPW; ++f) c += ((wd >> (BPP * f)) & kField) != 0u;
      return c;
    };
    int cnt = 0;
    for (int s = s_begin; s < s_end; s += 64) {
      const int x = s + lane;
      const uint32_t wd = x < s_end ? bm[x] : 0u;
      cnt += nz_count(wd);
      bits += __popc(wd);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
    if (lane == 0) wave_cnt[wave] = cnt;
    __syncthreads();
    int pos = total;
    for (int w = 0; w < wave; ++w) pos += wave_cnt[w];
    for (int w = 0; w < kWaves; ++w) total += wave_cnt[w];
    for (int s = s_begin; s < s_end; s += 64) {
      const int x = s + lane;
      const uint32_t wd = x < s_end ? bm[x] : 0u;
      const int c = nz_count(wd);
      const uint64_t b1 = __ballot(c & 1), b2 = __ballot(c & 2), b4 = __ballot(c & 4);
      int e = pos + lanes_below(b1) + 2 * lanes_below(b2) + 4 * lanes_below(b4);
#pragma unroll
      for (int f = 0; f < PPW; ++f) {
        const uint32_t m = (wd >> (BPP * f)) & kField;
        if (m != 0u) {
          out_rows[e] = lo + x * PPW + f;
          out_masks[e] = (MaskT)m;
          ++e;
        }
      }
      pos += __popcll(b1) + 2 * __popcll(b2) + 4 * __popcll(b4);
    }
    __syncthreads();  // the next window clears the bitmap and rewrites wave_cnt
  }
  const int padded = (total + kUnionChunk - 1) / kUnionChunk * kUnionChunk;
  for (int e = total + tid; e < padded; e += kUnionThreads) {
    out_rows[e] = b0;
    out_masks[e] = 0;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    entries += __shfl_xor(entries, o);
    bits += __shfl_xor(bits, o);
  }
  if (lane == 0) {
    wave_chk[wave][0] = entries;
    wave_chk[wave][1] = bits;
  }
  __syncthreads();
  if (tid == 0) {
    int all_entries = 0, all_bits = 0;
    for (int w = 0; w < kWaves; ++w) {
      all_entries += wave_chk[w][0];
      all_bits += wave_chk[w][1];
    }
    const bool repeated = all_bits < all_entries;  // some row lists one position twice
    a.counts[b] = total;
    // A block whose rows repeat a position stays with the per-row attention, which counts each
    // listed entry.
    if (a.use_union) a.use_union[b] = (!repeated && (float)total <= a.ratio * (float)nr * (float)a.k_sel) ? 1 : 0;
  }
}

// ---------------------------------------------------------------------------------------

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLazyMax = 8.f;  // log2 units the softmax offset may lag the largest logit
constexpr int kRowBytes = 128 * 2;                    // one key or value row of a group (swz layout)
constexpr int kStageBytes = 2 * kUnionChunk * kRowBytes;  // 32 key rows, then 32 value rows
// Chunks in the K/V ring (16 KiB each) for blocks of 16 and of 8 rows: with two waves per
// workgroup (8 rows) a shallower ring leaves room for more workgroups per CU.
constexpr int kStages16 = 3;
constexpr int kUnionRun = 16;  // consecutive blocks per XCD run
constexpr int kStages8 = 2;
constexpr int kMetaBytes = 256;                       // positions (128 B) + masks (64 B) of a chunk

template <int G, int NST, int NW>
__global__ __launch_bounds__(64 * NW) void sparse_attn_union_kernel(UnionAttnArgs a, float scale_log2, int n_blocks) {
  constexpr int CT = G / 4;  // 16-column tiles per wave: 4 rows x G heads
  constexpr int R = 4 * NW;  // rows per block
  // A chunk's metadata is DMA'd NST - 1 chunks ahead of its K/V stage, which is issued NST - 1
  // chunks ahead of its use: 2 NST - 1 chunks of metadata are live at once.
  constexpr int MS = (2 * NST - 1 <= 8) ? 8 : 16;
  __shared__ __attribute__((aligned(16))) unsigned char kv_lds[NST][kStageBytes];
  __shared__ __attribute__((aligned(16))) unsigned char meta_lds[MS][kMetaBytes];
  // Workgroups are dispatched to the 8 XCDs round-robin; XCD x takes runs of RUN consecutive
  // items (runs x, x + 8, ...).  The blocks of a run start together and scan their merged sets
  // in ascending order at about the same pace, so a KV row several of them selected is fetched
  // from HBM once and then hit in the XCD's L2; every XCD still gets an even share of long and
  // short blocks.  KV group slowest (its gathered rows stay in the last-level cache); within a
  // group the latest blocks, whose merged sets are the largest, start first.
  constexpr int RUN = kUnionRun;
  const int xp = blockIdx.x >> 3;
  const int wi = ((xp / RUN) * 8 + (blockIdx.x & 7)) * RUN + (xp % RUN);
  if (wi >= n_blocks * a.hkv) return;
  const int g = wi / n_blocks;
  const int blk = n_blocks - 1 - (wi - g * n_blocks);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, lg = lane >> 4;
  if (a.use_union && a.use_union[blk] == 0) return;
  const int r0 = blk * R;
  const int hq = a.hq;
  const int n_u = min(a.counts[blk], a.cap);
  const int nchunk = (n_u + kUnionChunk - 1) / kUnionChunk;
  const int* urows = a.kv_rows + (size_t)blk * a.cap;
  const uint16_t* umask = a.masks + (size_t)blk * a.cap;
  const size_t row_stride = (size_t)a.hkv * 128;
  const uint16_t* kg = a.k + (size_t)g * 128;
  const uint16_t* vg = a.v + (size_t)g * 128;

  // B operands of S^T: column n of tile T = CT wave + c is block row (16 T + n) / G, head
  // (16 T + n) % G of group g; rows past the end give zero columns.
  u32x4 qreg[CT][4];
  int rbit[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const int col = 16 * (CT * wave + c) + n;
    rbit[c] = col / G;
    const int row = r0 + rbit[c];
    const uint16_t* qp = a.q + ((size_t)min(row, a.rows - 1) * hq + g * G + col % G) * 128 + lg * 32;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qreg[c][ks] = row < a.rows ? ldg16(qp + ks * 8) : u32x4{0, 0, 0, 0};
  }
  const uint32_t wave_rows = 0xFu << (4 * wave);

  f32x4 oacc[8][CT];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int c = 0; c < CT; ++c) oacc[dt][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Running offsets (base-2 logits) and row sums.  The sums are an MFMA accumulator: the A
  // operand "ones" has bf16 1.0 in row 0 and zeros elsewhere, so C row 0 (element 0 of the
  // lanes of group 0) collects the column sums of P^T.
  float m_run[CT];
  f32x4 lacc[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    m_run[c] = -INFINITY;
    lacc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const uint32_t one2 = n == 0 ? 0x3F803F80u : 0u;
  const u32x4 ones = {one2, one2, one2, one2};

  // Positions (dwords 0..31) and masks (dwords 32..47) of chunk ch into meta slot ch % 8.
  auto meta_dma = [&](int ch) {
    const void* src = lane < 32 ? (const void*)(urows + ch * kUnionChunk + lane)
                                : (const void*)(umask + ch * kUnionChunk + 2 * (min(lane, 47) - 32));
    lds_dma4_untracked(src, meta_lds[ch % MS]);
  };
  // The chunk's 32 key rows and 32 value rows go in 8 + 8 copies of 4 rows (1 KiB each); wave w
  // issues copies w, w + NW, ...: key and value rows 4 j + lane / 16 for those j.  Each copy
  // takes the group's K or V base in scalar registers and a 32-bit byte offset per lane (the
  // host admits this kernel only for total_tokens * hkv < 2^24).
  auto stage = [&](int ch) {
    const int* pos = reinterpret_cast<const int*>(meta_lds[ch % MS]);
    unsigned char* buf = kv_lds[ch % NST];
    int pr[8 / NW];
#pragma unroll
    for (int i = 0; i < 8 / NW; ++i)  // clamped into [0, rows): a foreign list cannot move the gather off K / V
      pr[i] = min(max(pos[4 * (wave + i * NW) + (lane >> 4)], 0), a.rows - 1);
#pragma unroll
    for (int i = 0; i < 8 / NW; ++i) {
      const int j = wave + i * NW;
      const int piece = (lane & 15) ^ swz(4 * j + (lane >> 4));
      const uint32_t off = (uint32_t)pr[i] * (uint32_t)(row_stride * 2) + (uint32_t)piece * 16u;
      lds_dma16_saddr(kg, off, __builtin_amdgcn_readfirstlane(lds_offset(buf + (4 * j) * kRowBytes)));
      lds_dma16_saddr(vg, off, __builtin_amdgcn_readfirstlane(lds_offset(buf + (32 + 4 * j) * kRowBytes)));
    }
    if (wave == 0 && ch + NST - 1 < nchunk) meta_dma(ch + NST - 1);
  };
  auto stage_ops = [&](int ch) { return 16 / NW + ((wave == 0 && ch + NST - 1 < nchunk) ? 1 : 0); };

  const int trow = 4 * lg + (n >> 2), tm = n & 3, tsw = swz(trow);
  auto compute = [&](int ch) {
    const unsigned char* kt = kv_lds[ch % NST];
    const unsigned char* vt = kt + kUnionChunk * kRowBytes;
    const unsigned char* meta = meta_lds[ch % MS];
    // Masks of keys 4 lg + i (lo) and 16 + 4 lg + i (hi), i = 0..3.
    const uint2 mlo = *reinterpret_cast<const uint2*>(meta + 128 + 8 * lg);
    const uint2 mhi = *reinterpret_cast<const uint2*>(meta + 128 + 32 + 8 * lg);
    const uint32_t any = mlo.x | mlo.y | mhi.x | mhi.y;
    if (__ballot(((any | (any >> 16)) & wave_rows) != 0u) == 0ull) return;  // none of the wave's rows
    u32x4 ak[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        ak[j][ks] = *reinterpret_cast<const u32x4*>(kt + (16 * j + n) * kRowBytes + (((4 * lg + ks) ^ swz(n)) << 4));
    // V^T operands: lane j of lane group lg addresses key 4 lg + j / 4 (and 16 + that), dims
    // 16 dt + 4 (j % 4) .. + 3, so lane n receives dim 16 dt + n of keys 4 lg + 0..3 (16 + ..).
    u32x4 av[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int piece = 2 * dt + (tm >> 1);
      const unsigned char* p = vt + trow * kRowBytes + ((piece ^ tsw) << 4) + 8 * (tm & 1);
      const uint2 lo = lds_read_tr16(p);
      const uint2 hi = lds_read_tr16(p + 16 * kRowBytes);
      av[dt] = u32x4{lo.x, lo.y, hi.x, hi.y};
    }
    f32x4 s[2][CT];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int c = 0; c < CT; ++c) s[j][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int c = 0; c < CT; ++c) s[j][c] = mfma16x16x32(ak[j][ks], qreg[c][ks], s[j][c]);
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      // Slot e of the lane carries key 16 (e / 4) + 4 lg + e % 4; its mask is 16-bit field
      // e % 2 of dword mdw[e / 2], and the column's row is bit rbit[c] of a field.
      const uint32_t mdw[4] = {mlo.x, mlo.y, mhi.x, mhi.y};
      float mx = s[0][c][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, s[e >> 2][c][e & 3]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      // The offset m_run may lag the column's largest selected logit by up to kLazyMax (the
      // weights then stay below 2^kLazyMax); it is raised, with a rescale, only when the
      // chunk's largest logit (selected or not, an upper bound) passes that margin.
      if (__ballot(mx * scale_log2 > m_run[c] + kLazyMax) != 0ull) {
        float zm = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const bool sel = (mdw[e >> 1] >> (((e & 1) << 4) + rbit[c])) & 1u;
          zm = fmaxf(zm, sel ? s[e >> 2][c][e & 3] : -INFINITY);
        }
        zm = fmaxf(zm, __shfl_xor(zm, 16));
        zm = fmaxf(zm, __shfl_xor(zm, 32));
        const float m_new = fmaxf(m_run[c], zm * scale_log2);
        const float alpha = m_new > m_run[c] ? __builtin_amdgcn_exp2f(m_run[c] - m_new) : 1.f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) oacc[dt][c] *= alpha;
        lacc[c] *= alpha;
        m_run[c] = m_new;
      }
      const float moff = (m_run[c] == -INFINITY) ? 0.f : m_run[c];
      const int sh = 15 - rbit[c];
      u32x4 pb;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        // The weights enter the P.V product as bf16.  The row bit of each half is moved to the
        // half's top bit and sign-extended over the half (v_perm selectors 8 and 9), so the
        // AND keeps the weights of selected keys and zeroes the rest (an overflowed inf too).
        const uint32_t w2 = cvt_bf16x2(__builtin_amdgcn_exp2f(fmaf(s[e2 >> 1][c][2 * (e2 & 1)], scale_log2, -moff)),
                                       __builtin_amdgcn_exp2f(fmaf(s[e2 >> 1][c][2 * (e2 & 1) + 1], scale_log2, -moff)));
        pb[e2] = w2 & __builtin_amdgcn_perm(0u, mdw[e2] << sh, 0x09090808u);
      }
      // O^T += V^T P^T, and the row sums of the same bf16 weights on the ones operand.
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) oacc[dt][c] = mfma16x16x32(av[dt], pb, oacc[dt][c]);
      lacc[c] = mfma16x16x32(ones, pb, lacc[c]);
    }
  };

  // Operations of the stages after `ch` that are already issued when stage ch must be complete.
  auto ops_after = [&](int ch, int last_issued) {
    int n_ops = 0;
    for (int c = ch + 1; c <= last_issued; ++c) n_ops += stage_ops(c);
    return n_ops;
  };
  if (nchunk > 0) {
    if (wave == 0)
      for (int c = 0; c < NST - 1 && c < nchunk; ++c) meta_dma(c);
    vm_wait<0>();
    ring_barrier();
    for (int c = 0; c < NST - 1 && c < nchunk; ++c) stage(c);
    vm_wait_at_most(ops_after(0, min(NST - 2, nchunk - 1)));
    ring_barrier();
    for (int ch = 0; ch < nchunk; ++ch) {
      if (ch + NST - 1 < nchunk) stage(ch + NST - 1);
      compute(ch);
      // Chunk ch + 1 (with the metadata its stage brought in) must have landed; the later
      // stages may stay in flight.
      if (ch + 1 < nchunk) vm_wait_at_most(ops_after(ch + 1, min(ch + NST - 1, nchunk - 1)));
      ring_barrier();
    }
  }

#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const float l_tot = __shfl(lacc[c][0], n);  // lane (group 0, column n) holds the sum
    const int row = r0 + rbit[c];
    if (row >= a.rows) continue;
    const int h = g * G + (16 * (CT * wave + c) + n) % G;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* op = a.out + ((size_t)row * hq + h) * 128 + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      uint2 st;
      st.x = pack_bf16x2(oacc[dt][c][0] * inv, oacc[dt][c][1] * inv);
      st.y = pack_bf16x2(oacc[dt][c][2] * inv, oacc[dt][c][3] * inv);
      *reinterpret_cast<uint2*>(op + 16 * dt) = st;
    }
    const float moff = (m_run[c] == -INFINITY) ? 0.f : m_run[c];
    if (a.lse && lg == 0) a.lse[(size_t)row * hq + h] = l_tot > 0.f ? (moff + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_query_union(const QueryUnionArgs& a, hipStream_t s) {
  const int nb = a.block_end - a.block_begin;
  if (nb <= 0) return hipSuccess;
  if (a.masks32) {
    if (a.block_rows < 1 || a.block_rows > 32) return hipErrorInvalidValue;
    hipLaunchKernelGGL(query_union_kernel<32>, dim3(nb), dim3(kUnionThreads), 0, s, a);
    return hipGetLastError();
  }
  if (!union_block_rows_ok(a.block_rows)) return hipErrorInvalidValue;
  if (a.block_rows <= 8)
    hipLaunchKernelGGL(query_union_kernel<8>, dim3(nb), dim3(kUnionThreads), 0, s, a);
  else
    hipLaunchKernelGGL(query_union_kernel<16>, dim3(nb), dim3(kUnionThreads), 0, s, a);
  return hipGetLastError();
}

bool union_attn_supported(int hq, int hkv, long long rows) {
  const int g = hkv > 0 ? hq / hkv : 0;
  // K / V rows are addressed with 32-bit byte offsets from the group's base.
  return hkv > 0 && hq % hkv == 0 && (g == 4 || g == 8 || g == 16) && rows * hkv * 256 < (1ll << 32);
}

template <int G>
void launch_union_g(const UnionAttnArgs& a, unsigned grid, float scale_log2, int n_blocks, hipStream_t s) {
  if (a.block_rows == 8)
    hipLaunchKernelGGL((sparse_attn_union_kernel<G, kStages8, 2>), dim3(grid), dim3(128), 0, s, a, scale_log2, n_blocks);
  else
    hipLaunchKernelGGL((sparse_attn_union_kernel<G, kStages16, 4>), dim3(grid), dim3(256), 0, s, a, scale_log2, n_blocks);
}

hipError_t launch_sparse_attn_union(const UnionAttnArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (!union_block_rows_ok(a.block_rows)) return hipErrorInvalidValue;
  const int n_blocks = (a.rows + a.block_rows - 1) / a.block_rows;
  const long long items = (long long)n_blocks * a.hkv;
  const unsigned grid = (unsigned)((items + 8 * kUnionRun - 1) / (8 * kUnionRun) * (8 * kUnionRun));  // whole runs
  const float scale_log2 = a.softmax_scale * 1.4426950408889634f;
  switch (a.hq / a.hkv) {
    case 4: launch_union_g<4>(a, grid, scale_log2, n_blocks, s); break;
    case 8: launch_union_g<8>(a, grid, scale_log2, n_blocks, s); break;
    case 16: launch_union_g<16>(a, grid, scale_log2, n_blocks, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dsa

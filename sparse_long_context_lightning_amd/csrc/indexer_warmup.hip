// The indexer's dense warm-up objective for gfx950: the target distribution (head-mean causal
// attention), the KL divergence to the indexer's softmax with its gradient, and (in
// indexer_bwd.hip) the backward of the indexer scores.
//
// In the dense warm-up of the Keye-VL-2.0 report digest (mqxn.cn news 1966, section 一) the full
// attention stays as it is and only the Lightning Indexer trains, pulled towards the full
// attention's distribution with a KL divergence.  For query row t (local position, causal
// prefix s <= t):
//     p_t[s] = (1 / Hq) sum_h softmax_s(scale <Q[t,h], K[s, h / G]>)        (fixed target)
//     r_t[s] = softmax_s(I[t, s]),   loss_t = sum_s p_t[s] (log p_t[s] - log r_t[s])
//     d loss_t / d I[t, s] = r_t[s] - p_t[s]
#include "common.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994530942f;

// Start value of a running max: below every logit the kernel meets (|scale * <q, k>| of bf16
// inputs is far smaller), yet finite, so differences against it never form inf - inf.
constexpr float kNoLogit = -1.0e30f;
// How far (log2 units) a row's softmax offset may lag its largest logit in pass 1: terms stay
// below 2^kLazyMax, so the fp32 sum of up to 2^20 of them cannot overflow.
constexpr float kLazyMax = 8.f;

// 2^x on the hardware exp2 (results below 2^-126 flush to zero, which no softmax sum here
// notices: every sum holds a term equal to 1).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Head-mean target, two passes over the causal keys.  A workgroup of NWV waves takes a block of
// consecutive query tokens and one range of key positions: wave w works on KV group w % HKV for
// token set w / HKV, whose RT * 16 (token, head) rows of that group (row r: token r / G, head
// r % G, G = Hq / Hkv a multiple of 4, so a lane's four C rows are one token's) sit on the MFMA
// row axis of RT 16x16x32 bf16 tiles, with 16 keys of the group on the column axis.  Key tiles
// of TK positions hold every group's 256-byte row of each position (one contiguous KiB per
// position at 4 KV heads); they are DMA'd global->LDS, double buffered and shared by the
// workgroup, with 16-byte piece c of position p stored at slot c ^ (p mod 16) (conflict-free B
// reads).  Each wave reads only its group's key rows, and each B operand it reads serves its RT
// row tiles: LDS reads per flop are what bound the kernel when every wave read all groups' rows
// for two tokens.
//
// PASS 1 keeps a lane-local (offset, sum) per row over the keys the lane sees and merges the 16
// lanes of each row at the end: lse per (token, head).  The offset may lag the row's largest
// logit by up to kLazyMax, so a logit costs one fma, one exp2 and one add, and the offset moves
// (with a rescale of the sum) only for a logit past that margin, in a branch the wave skips when
// no lane needs it; tiles on the causal diagonal mask their keys.  PASS 2 recomputes the logits,
// turns them into probabilities with that lse (one fma and one exp2 per logit), leaves each
// lane group's sum over its four heads in LDS, and after the tile's barrier sums a token's Hq / 4
// shares (its heads of every group) and writes p_t[s] / Hq.
//
// The key range of a workgroup is cut into splits of kHeadMeanSplitKeys positions, one
// workgroup per (token block, split) (grid y), so that a call on a few thousand rows still puts
// several waves on every SIMD.  With more than one split, pass 1 leaves each split's (max, sum)
// per (token, head) in the token's own probs row (entries (split hq + head) 2 and + 1, inside the
// causal prefix, which pass 2 overwrites), head_mean_lse_combine merges them into lse, and pass 2
// writes each split's positions.
constexpr int kHeadMeanSplitKeys = 2048;

template <int HKV>
struct HeadMeanShape {
  // 16 waves of 2 row tiles (32K target, 2048-row calls: 13.2 ms) against 8 of 4 (15.8 ms), 8 of
  // 2 (14.2 ms), 16 of 1 (15.8 ms); 16 of 4 spill at the 128 registers 1024 threads allow.
  static constexpr int NWV = 16;                  // waves per workgroup
  static constexpr int NTS = NWV / HKV;           // token sets per workgroup
  static constexpr int RT = 2;                    // 16-row MFMA tiles per wave
  static constexpr int TK = HKV <= 4 ? 32 : 16;   // positions per key tile
};
// Tokens of one wave's rows (the rows past TPW G, when G does not divide 16 RT, are idle).
__host__ __device__ constexpr int head_mean_tpw(int rt, int g) { return 16 * rt / g; }

template <int PASS, int HKV>
__global__ __launch_bounds__(64 * HeadMeanShape<HKV>::NWV) void attn_head_mean_kernel(HeadMeanArgs a,
                                                                                      float scale_log2) {
  using SH = HeadMeanShape<HKV>;
  constexpr int NWV = SH::NWV, NTS = SH::NTS, RT = SH::RT, TK = SH::TK;
  constexpr int ROWB = HKV * 256;            // bytes per key position (all KV groups)
  constexpr int TILE = TK * ROWB;
  constexpr int NJOB = TILE / 1024;          // 1 KiB DMA instructions per tile
  constexpr int NLD = (NJOB + NWV - 1) / NWV;  // of them per wave (the last may be idle)
  __shared__ __attribute__((aligned(16))) unsigned char tiles[2][TILE];
  // Pass 2: per tile, every lane group's four-head share of its token's sum (slot rt 4 + lg of its
  // wave, key column); two buffers so that a tile's shares can be written while the last are summed.
  __shared__ float part[PASS == 2 ? 2 : 1][PASS == 2 ? NWV * 4 * RT * TK : 1];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, lg = lane >> 4;
  const int hq = a.hq, G = hq / HKV;
  const int tpw = head_mean_tpw(RT, G);
  const int tpb = NTS * tpw;                 // tokens per workgroup
  const int g = wave % HKV, ts = wave / HKV;
  const int wg_r0 = a.row_begin + blockIdx.x * tpb;
  const int wg_last = min(wg_r0 + tpb, a.row_end) - 1;
  const int ntiles = (wg_last - a.seq_off) / TK + 1;
  constexpr int TPS = kHeadMeanSplitKeys / TK;  // tiles per split
  const int nsplit = (ntiles + TPS - 1) / TPS;
  const int sp = blockIdx.y;
  if (sp >= nsplit) return;  // the whole workgroup: this block of tokens has fewer splits
  const int it0 = sp * TPS, it1 = min(ntiles, it0 + TPS);
  const int w_r0 = wg_r0 + ts * tpw;                        // the wave's first token
  const int w_last = min(w_r0 + tpw, a.row_end) - 1;        // and its last (< w_r0: no tokens)
  const bool active = w_last >= w_r0;
  const int t_min = w_r0 - a.seq_off, t_max = w_last - a.seq_off;

  // A operands: row 16 rt + n of the wave is token (16 rt + n) / G, head g G + (16 rt + n) % G.
  u32x4 qa[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = 16 * rt + n;
    const int tok = min(w_r0 + r / G, a.row_end - 1);
    const uint16_t* qp = a.q + ((size_t)tok * hq + g * G + r % G) * 128 + lg * 32;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qa[rt][ks] = ldg16(qp + ks * 8);
  }
  // This lane's C rows 16 rt + 4 lg + i are token c_row[rt], heads g G + (16 rt + 4 lg + i) % G.
  int c_row[RT];
  bool c_ok[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = 16 * rt + 4 * lg;
    c_row[rt] = w_r0 + r / G;
    c_ok[rt] = active && r / G < tpw && c_row[rt] <= w_last;
  }

  float m_st[RT][4], l_st[RT][4], lse2[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m_st[rt][i] = kNoLogit;
      l_st[rt][i] = 0.f;
      lse2[rt][i] = 0.f;
      if (PASS == 2 && c_ok[rt]) {
        const int head = g * G + (16 * rt + 4 * lg + i) % G;
        lse2[rt][i] = a.lse[(size_t)(c_row[rt] - a.out_row0) * hq + head] * kLog2e;
      }
    }

  // DMA mapping: instruction p of wave w (job P = p * NWV + w) fills LDS bytes [P*1024, +1024);
  // lane l's 16 bytes land at row (position pos, group gg), slot l % 16, which holds piece
  // (l % 16) ^ swz(pos) (the plain pos % 16 would put lanes of different quarters of a wave on
  // the same LDS slots in the operand reads).
  const uint16_t* kseq = a.k + (size_t)a.seq_off * HKV * 128;
  const int kv_len = wg_last - a.seq_off + 1;  // positions the workgroup can use
  auto load_tile = [&](int tile, int buf) {
#pragma unroll
    for (int p = 0; p < NLD; ++p) {
      if (NJOB % NWV != 0 && p * NWV + wave >= NJOB) break;
      const int byte = (p * NWV + wave) * 1024 + lane * 16;
      const int pos_in = byte / ROWB;
      const int gg = (byte % ROWB) / 256;
      const int piece = (lane & 15) ^ swz(pos_in);
      const int pos = min(tile * TK + pos_in, kv_len - 1);
      lds_dma16(kseq + (size_t)pos * HKV * 128 + gg * 128 + piece * 8, &tiles[buf][(p * NWV + wave) * 1024]);
    }
  };

  load_tile(it0, it0 & 1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int it = it0; it < it1; ++it) {
    if (it + 1 < it1) load_tile(it + 1, (it + 1) & 1);
    const unsigned char* tile = tiles[it & 1];
    float* part_t = part[PASS == 2 ? (it & 1) : 0];
    if (PASS == 2 && !(active && it * TK <= t_max)) {
      // no keys of this tile for the wave's tokens: its shares are 0
      for (int i = lane; i < 4 * RT * TK; i += 64) part_t[wave * 4 * RT * TK + i] = 0.f;
    }
    if (active && it * TK <= t_max) {
      // Tiles wholly inside every row's prefix take the short update; the diagonal tiles mask.
      const bool full = it * TK + TK - 1 <= t_min;
#pragma unroll
      for (int st = 0; st < TK / 16; ++st) {
        const int pos_t = 16 * st + n;      // position within the tile
        const int key = it * TK + pos_t;
        const unsigned char* rowp = tile + (pos_t * HKV + g) * 256;
        f32x4 c[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) c[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const u32x4 kb = *reinterpret_cast<const u32x4*>(rowp + (((lg * 4 + ks) ^ swz(pos_t)) * 16));
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) c[rt] = mfma16x16x32(qa[rt][ks], kb, c[rt]);
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int c_t = c_row[rt] - a.seq_off;
          const bool kv = c_ok[rt] && key <= c_t;
          if (PASS == 1 && full) {
            // m is an offset that may lag the row's largest logit by up to kLazyMax: the new
            // term is 2^d; only a logit past that margin (rare after the first keys) moves m,
            // rescaling the sum, in a branch the whole wave skips when no lane needs it.
            float d[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) d[i] = fmaf(c[rt][i], scale_log2, -m_st[rt][i]);
            const float dm = fmaxf(fmaxf(d[0], d[1]), fmaxf(d[2], d[3]));
            if (__ballot(dm > kLazyMax) != 0ull) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                if (d[i] > kLazyMax) {
                  const float z = c[rt][i] * scale_log2;
                  l_st[rt][i] *= fast_exp2(m_st[rt][i] - z);
                  m_st[rt][i] = z;
                  d[i] = 0.f;
                }
              }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) l_st[rt][i] += fast_exp2(d[i]);
          } else if (PASS == 1) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              // diagonal tile: masked keys add 0 and never move the offset
              const float z = c[rt][i] * scale_log2;
              if (kv && z > m_st[rt][i] + kLazyMax) {
                l_st[rt][i] *= fast_exp2(m_st[rt][i] - z);
                m_st[rt][i] = z;
              }
              l_st[rt][i] += kv ? fast_exp2(z - m_st[rt][i]) : 0.f;
            }
          } else {
            float tok_sum = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) tok_sum += fast_exp2(fmaf(c[rt][i], scale_log2, -lse2[rt][i]));
            part_t[((wave * RT + rt) * 4 + lg) * TK + pos_t] = kv ? tok_sum : 0.f;
          }
        }
      }
    }
    if (it + 1 < it1) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (PASS == 2) {
      // Shares of the tile complete: token tok of token set ts is rows (tok % tpw) G .. + G - 1
      // of each of the set's HKV waves, i.e. slots (tok % tpw) G / 4 .. + G / 4 - 1 of each.
      for (int i = threadIdx.x; i < tpb * TK; i += 64 * NWV) {
        const int tok = i / TK, pos_t = i % TK;
        const int r = wg_r0 + tok, key = it * TK + pos_t;
        if (r <= wg_last && key <= r - a.seq_off) {
          const int tset = tok / tpw, s0 = (tok - tset * tpw) * (G / 4);
          float sum = 0.f;
          for (int gg = 0; gg < HKV; ++gg) {
            const float* pw = part_t + (size_t)((tset * HKV + gg) * 4 * RT) * TK;
            for (int j = 0; j < G / 4; ++j) sum += pw[(s0 + j) * TK + pos_t];
          }
          a.probs[(size_t)(r - a.out_row0) * a.ld + key] = sum / (float)hq;
        }
      }
    }
  }

  if (PASS == 1 && active) {
    // Merge the 16 lanes of each row (same lg): log-sum-exp of (m, l) pairs.
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float m = m_st[rt][i], l = l_st[rt][i];
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          const float mo = __shfl_xor(m, o), lo = __shfl_xor(l, o);
          const float mn = fmaxf(m, mo);
          l = l * fast_exp2(m - mn) + lo * fast_exp2(mo - mn);
          m = mn;
        }
        if (n == 0 && c_ok[rt]) {
          const int head = g * G + (16 * rt + 4 * lg + i) % G;
          if (nsplit == 1) {
            a.lse[(size_t)(c_row[rt] - a.out_row0) * hq + head] = (m + log2f(l)) * kLn2;
          } else {
            float* part = a.probs + (size_t)(c_row[rt] - a.out_row0) * a.ld + (size_t)(sp * hq + head) * 2;
            part[0] = m;
            part[1] = l;
          }
        }
      }
  }
}

// lse of the rows whose keys pass 1 split: merge the splits' (max, sum) pairs left in each
// row's probs entries.  One thread per (row, head); rows_per_wg and TK as in the launch of pass 1.
__global__ __launch_bounds__(256) void head_mean_lse_combine(HeadMeanArgs a, int rows_per_wg, int tk) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const int hq = a.hq;
  if (i >= (long long)(a.row_end - a.row_begin) * hq) return;
  const int r = a.row_begin + (int)(i / hq), head = (int)(i % hq);
  const int wg_last = min(a.row_begin + ((r - a.row_begin) / rows_per_wg + 1) * rows_per_wg, a.row_end) - 1;
  const int ntiles = (wg_last - a.seq_off) / tk + 1;
  const int tps = kHeadMeanSplitKeys / tk;
  const int nsplit = (ntiles + tps - 1) / tps;
  if (nsplit == 1) return;  // pass 1 wrote this row's lse
  const float* row = a.probs + (size_t)(r - a.out_row0) * a.ld;
  float m = kNoLogit;
  for (int sp = 0; sp < nsplit; ++sp) m = fmaxf(m, row[(size_t)(sp * hq + head) * 2]);
  float l = 0.f;
  for (int sp = 0; sp < nsplit; ++sp) {
    const float* part = row + (size_t)(sp * hq + head) * 2;
    l += part[1] * fast_exp2(part[0] - m);
  }
  a.lse[(size_t)(r - a.out_row0) * hq + head] = (m + log2f(l)) * kLn2;
}

// KL(target || softmax(I)) per row and its gradient r - p, one 256-thread workgroup per row.
// grad may alias scores: each element is read and rewritten by the same thread.
__device__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}
__device__ float block_max(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__global__ __launch_bounds__(256) void indexer_kl_kernel(const float* scores, const float* __restrict__ target,
                                                        long long ld, const int* __restrict__ row_len, int len_base,
                                                        float* __restrict__ row_loss, float* grad) {
  __shared__ float red[4];
  const int row = blockIdx.x;
  const int n = row_len ? row_len[row] : len_base + row + 1;
  const float* s_row = scores + (size_t)row * ld;
  const float* p_row = target + (size_t)row * ld;
  float* g_row = grad + (size_t)row * ld;
  float m = -INFINITY;
  for (int i = threadIdx.x; i < n; i += 256) m = fmaxf(m, s_row[i]);
  m = block_max(m, red);
  float l = 0.f;
  for (int i = threadIdx.x; i < n; i += 256) l += __expf(s_row[i] - m);
  l = block_sum(l, red);
  const float lse = m + __logf(l);
  float loss = 0.f;
  for (int i = threadIdx.x; i < n; i += 256) {
    const float log_r = s_row[i] - lse;
    const float p = p_row[i];
    if (p > 0.f) loss += p * (__logf(p) - log_r);
    g_row[i] = __expf(log_r) - p;
  }
  loss = block_sum(loss, red);
  if (threadIdx.x == 0) row_loss[row] = loss;
}

template <int HKV>
hipError_t launch_head_mean_t(const HeadMeanArgs& a, hipStream_t s) {
  using SH = HeadMeanShape<HKV>;
  const int G = a.hq / HKV;
  const int tpb = SH::NTS * head_mean_tpw(SH::RT, G);  // tokens per workgroup
  const int rows = a.row_end - a.row_begin;
  const unsigned grid = (unsigned)((rows + tpb - 1) / tpb);
  const int max_tiles = (a.row_end - 1 - a.seq_off) / SH::TK + 1;
  constexpr int TPS = kHeadMeanSplitKeys / SH::TK;
  const unsigned max_split = (unsigned)((max_tiles + TPS - 1) / TPS);
  const float scale_log2 = a.softmax_scale * kLog2e;
  hipLaunchKernelGGL((attn_head_mean_kernel<1, HKV>), dim3(grid, max_split), dim3(64 * SH::NWV), 0, s, a, scale_log2);
  if (max_split > 1) {
    const long long n = (long long)rows * a.hq;
    hipLaunchKernelGGL(head_mean_lse_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a, tpb, SH::TK);
  }
  hipLaunchKernelGGL((attn_head_mean_kernel<2, HKV>), dim3(grid, max_split), dim3(64 * SH::NWV), 0, s, a, scale_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_head_mean(const HeadMeanArgs& a, hipStream_t s) {
  if (a.row_end <= a.row_begin) return hipSuccess;
  switch (a.hkv) {
    case 1: return launch_head_mean_t<1>(a, s);
    case 2: return launch_head_mean_t<2>(a, s);
    case 4: return launch_head_mean_t<4>(a, s);
    case 8: return launch_head_mean_t<8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_indexer_kl(const float* scores, const float* target, long long ld, int rows, const int* row_len,
                             int len_base, float* row_loss, float* grad, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(indexer_kl_kernel, dim3((unsigned)rows), dim3(256), 0, s, scores, target, ld, row_len, len_base,
                     row_loss, grad);
  return hipGetLastError();
}

}  // namespace dsa

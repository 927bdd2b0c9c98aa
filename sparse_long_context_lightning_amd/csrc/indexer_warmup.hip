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

// 2^x on the hardware exp2 (results below 2^-126 flush to zero, which no softmax sum here
// notices: every sum holds a term equal to 1).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Head-mean target, two passes over the causal keys of a workgroup of 4 waves, each wave a
// block of 16 / G consecutive query tokens: the block's 16 (token, head) rows of one KV group
// sit on the MFMA row axis and 16 keys of that group on the column axis (16x16x32 bf16).  Key
// tiles of TK positions hold every group's 256-byte row of each position (one contiguous KiB
// per position at 4 KV heads); they are DMA'd global->LDS, double buffered and shared by the 4
// waves, with 16-byte piece c of position p stored at slot c ^ (p mod 16) (conflict-free B
// reads).  PASS 1 keeps a lane-local online (max, sum) per row over the keys the lane sees and
// merges the 16 lanes of each row at the end: lse per (token, head).  Its update takes one exp2
// per logit: with d = z - m, e = 2^-|d| is both the new term (d <= 0) and the rescale of the old
// sum (d > 0, then the new term is 1).  PASS 2 recomputes the
// logits, turns them into probabilities with that lse, sums the token's heads over all groups
// and writes p_t[s] / Hq.  Needs G = Hq / Hkv >= 4, so each lane's four C rows are one token's.
template <int PASS, int HKV, int NWV>
__global__ __launch_bounds__(64 * NWV) void attn_head_mean_kernel(HeadMeanArgs a, float scale_log2, int n_blocks) {
  constexpr int ROWB = HKV * 256;            // bytes per key position (all KV groups)
  constexpr int TK = HKV <= 4 ? 32 : 16;     // positions per tile
  constexpr int TILE = TK * ROWB;
  constexpr int NJOB = TILE / 1024;          // 1 KiB DMA instructions per tile
  constexpr int NLD = (NJOB + NWV - 1) / NWV;  // of them per wave (the last may be idle)
  __shared__ __attribute__((aligned(16))) unsigned char tiles[2][TILE];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, lg = lane >> 4;
  const int hq = a.hq, G = hq / HKV, TB = 16 / G;
  const int blk = blockIdx.x * NWV + wave;
  const int wg_r0 = a.row_begin + blockIdx.x * NWV * TB;
  const int wg_last = min(wg_r0 + NWV * TB, a.row_end) - 1;
  const int ntiles = (wg_last - a.seq_off) / TK + 1;
  const bool active = blk < n_blocks;
  const int r0 = a.row_begin + blk * TB;
  const int r_last = active ? min(r0 + TB, a.row_end) - 1 : r0;
  const int t_max = r_last - a.seq_off;
  // Row m of a group's tile: token m / G of the block, head g G + m % G.
  const int a_tok = min(min(r0 + n / G, r_last), a.row_end - 1);
  u32x4 qa[HKV][4];
#pragma unroll
  for (int g = 0; g < HKV; ++g) {
    const uint16_t* qp = a.q + ((size_t)a_tok * hq + g * G + n % G) * 128 + lg * 32;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qa[g][ks] = ldg16(qp + ks * 8);
  }
  // This lane's C rows 4 lg + i all belong to token c_row (G >= 4).
  const int c_row = r0 + (4 * lg) / G;
  const bool c_ok = active && c_row <= r_last;
  const int c_t = c_row - a.seq_off;

  float m_st[HKV][4], l_st[HKV][4], lse2[HKV][4];
#pragma unroll
  for (int g = 0; g < HKV; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m_st[g][i] = kNoLogit;
      l_st[g][i] = 0.f;
      lse2[g][i] = 0.f;
      if (PASS == 2 && c_ok) {
        const int head = g * G + (4 * lg + i) % G;
        lse2[g][i] = a.lse[(size_t)(c_row - a.out_row0) * hq + head] * kLog2e;
      }
    }

  // DMA mapping: instruction p of wave w (job P = p * NWV + w) fills LDS bytes [P*1024, +1024);
  // lane l's 16 bytes land at row (position pos, group g), slot l % 16, which holds piece
  // (l % 16) ^ (pos % 16).
  const uint16_t* kseq = a.k + (size_t)a.seq_off * HKV * 128;
  int st_pos[NLD], st_off[NLD];
#pragma unroll
  for (int p = 0; p < NLD; ++p) {
    const int byte = min(p * NWV + wave, NJOB - 1) * 1024 + lane * 16;
    const int pos = byte / ROWB;
    const int g = (byte % ROWB) / 256;
    const int piece = (lane & 15) ^ (pos & 15);
    st_pos[p] = pos;
    st_off[p] = g * 128 + piece * 8;  // elements within the position's HKV * 128
  }
  const int kv_len = wg_last - a.seq_off + 1;  // positions the workgroup can use
  auto load_tile = [&](int tile, int buf) {
#pragma unroll
    for (int p = 0; p < NLD; ++p) {
      if (NJOB % NWV != 0 && p * NWV + wave >= NJOB) break;
      const int pos = min(tile * TK + st_pos[p], kv_len - 1);
      lds_dma16(kseq + (size_t)pos * HKV * 128 + st_off[p], &tiles[buf][(p * NWV + wave) * 1024]);
    }
  };

  load_tile(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    if (it + 1 < ntiles) load_tile(it + 1, (it + 1) & 1);
    if (active && it * TK <= t_max) {
      const unsigned char* tile = tiles[it & 1];
#pragma unroll
      for (int st = 0; st < TK / 16; ++st) {
        const int pos_t = 16 * st + n;      // position within the tile
        const int key = it * TK + pos_t;
        const bool kv = c_ok && key <= c_t;
        float tok_sum = 0.f;
#pragma unroll
        for (int g = 0; g < HKV; ++g) {
          const unsigned char* rowp = tile + (pos_t * HKV + g) * 256;
          f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const u32x4 kb = *reinterpret_cast<const u32x4*>(rowp + (((lg * 4 + ks) ^ (pos_t & 15)) * 16));
            c = mfma16x16x32(qa[g][ks], kb, c);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float z = c[i] * scale_log2;
            if (PASS == 1) {
              // masked keys enter as a logit far below any real one: e = 0, no update of m
              const float d = (kv ? z : 2.f * kNoLogit) - m_st[g][i];
              const float e = fast_exp2(-fabsf(d));
              const bool up = d > 0.f;
              l_st[g][i] = up ? fmaf(l_st[g][i], e, 1.f) : l_st[g][i] + e;
              m_st[g][i] = up ? z : m_st[g][i];
            } else {
              tok_sum += kv ? fast_exp2(z - lse2[g][i]) : 0.f;
            }
          }
        }
        if (PASS == 2) {
          // Sum the token's lane groups (G / 4 of them) and store from its first one.
          if (G >= 8) tok_sum += __shfl_xor(tok_sum, 16);
          if (G >= 16) tok_sum += __shfl_xor(tok_sum, 32);
          if (kv && (4 * lg) % G == 0) a.probs[(size_t)(c_row - a.out_row0) * a.ld + key] = tok_sum / (float)hq;
        }
      }
    }
    if (it + 1 < ntiles) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  if (PASS == 1 && active) {
    // Merge the 16 lanes of each row (same lg): log-sum-exp of (m, l) pairs.
#pragma unroll
    for (int g = 0; g < HKV; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float m = m_st[g][i], l = l_st[g][i];
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          const float mo = __shfl_xor(m, o), lo = __shfl_xor(l, o);
          const float mn = fmaxf(m, mo);
          l = l * fast_exp2(m - mn) + lo * fast_exp2(mo - mn);
          m = mn;
        }
        if (n == 0 && c_ok) {
          const int head = g * G + (4 * lg + i) % G;
          a.lse[(size_t)(c_row - a.out_row0) * hq + head] = (m + log2f(l)) * kLn2;
        }
      }
  }
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

// Waves (token blocks) per head-mean workgroup, all sharing its staged key tiles.
constexpr int kHeadMeanWaves = 4;

template <int HKV>
hipError_t launch_head_mean_t(const HeadMeanArgs& a, hipStream_t s) {
  const int G = a.hq / HKV;
  const int TB = 16 / G;
  const int rows = a.row_end - a.row_begin;
  const int n_blocks = (rows + TB - 1) / TB;
  const unsigned grid = (unsigned)((n_blocks + kHeadMeanWaves - 1) / kHeadMeanWaves);
  const float scale_log2 = a.softmax_scale * kLog2e;
  hipLaunchKernelGGL((attn_head_mean_kernel<1, HKV, kHeadMeanWaves>), dim3(grid), dim3(64 * kHeadMeanWaves), 0, s, a,
                     scale_log2, n_blocks);
  hipLaunchKernelGGL((attn_head_mean_kernel<2, HKV, kHeadMeanWaves>), dim3(grid), dim3(64 * kHeadMeanWaves), 0, s, a,
                     scale_log2, n_blocks);
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

// Deterministic per-row top-k for gfx950, row-block form (one 1024-thread workgroup per row).
// Used for rows longer than the wave-parallel kernels of topk_wave.hip handle, or when the
// caller passes no scratch.
//
// The digest of the Keye-VL-2.0 report (mqxn.cn news 1966) keeps the 2048 best positions per
// query token (section 一) and requires the selection to be deterministic so training and
// inference agree (section 八).  Here the selected set is unique: larger score first, and among
// equal scores the lower position; the positions are returned in ascending order.
//
// Scores are mapped to order-preserving 32-bit keys (-0 folded into +0).  Per row:
//   1. a jittered stratified sample of up to 8192 keys (the whole row when it is that short)
//      goes to LDS, and an 8-bit radix select over it picks a threshold tau_lo that the true
//      k-th key clears with a wide margin (the whole-row case gives the exact k-th key);
//   2. ONE ordered pass over the row (loads run one round ahead of the scans) (block-wide scans keep position order) copies every
//      position with key >= tau_lo, with its key, into LDS;
//   3. an 8-bit radix select over those candidates finds the exact k-th key tau and how many
//      positions equal to tau are taken; a last ordered pass over the candidates writes the
//      selected positions, which come out ascending, lowest positions winning ties.
// If the sample misjudged the row (fewer than k candidates, or more than LDS holds, e.g. long
// runs of equal scores), the row falls back to an exact radix select over global memory and an
// ordered emit pass.  The result does not depend on the path taken or on thread timing.
#include "common.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kCap = 8192;  // candidate capacity (and sample size)
constexpr int kPer = 8;     // consecutive positions per thread in the ordered pass

struct TopkSmem {
  uint32_t cand_key[kCap];  // holds the sample first, then the candidates' keys
  int cand_pos[kCap];
  uint32_t hist[256];
  uint32_t wsum[kWaves];
  uint32_t digit, digit_above;
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// Block-wide exclusive scan of v; also returns the block total.  Contains barriers: every
// thread of the block must call it.
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const int lane = lane_id(), wave = wave_id();
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const uint32_t s = wsum[i];
    pre += (i < wave) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return pre + x - v;
}

// LDS histogram increment; when the whole active wave hits one bin, a single add is issued.
__device__ __forceinline__ void hist_add(uint32_t* h, uint32_t bin) {
  const uint32_t first = __builtin_amdgcn_readfirstlane(bin);
  const unsigned long long active = __ballot(1);
  const unsigned long long same = __ballot(bin == first);
  if (same == active) {
    if (lane_id() == __builtin_ctzll(active)) atomicAdd(&h[first], (uint32_t)__popcll(active));
  } else {
    atomicAdd(&h[bin], 1u);
  }
}

// In the 256-bin histogram (high bins = large keys) find the bin holding rank `need` counted
// from the top (1-based) and the count strictly above it.  Contains barriers.
__device__ void find_rank_bin(TopkSmem& sm, uint32_t need) {
  const int b = 255 - (int)threadIdx.x;  // thread t owns bin 255 - t (threads >= 256 own none)
  const uint32_t c = (b >= 0) ? sm.hist[b] : 0u;
  uint32_t tot;
  const uint32_t run = block_excl_scan(c, sm.wsum, tot);
  if (b >= 0 && run < need && run + c >= need) {
    sm.digit = (uint32_t)b;
    sm.digit_above = run;
  }
  __syncthreads();
}

// The need-th largest of the keys produced by key_at(i), i < count, and how many keys equal
// to it complete `need` together with all larger keys.  Contains barriers.
template <typename KeyAt>
__device__ void radix_select(TopkSmem& sm, KeyAt key_at, uint32_t count, uint32_t need, uint32_t* tau,
                             uint32_t* n_eq) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) sm.hist[tid] = 0;
    __syncthreads();
    for (uint32_t i = tid; i < count; i += kThreads) {
      const uint32_t key = key_at(i);
      if ((key & mask) == prefix) hist_add(sm.hist, (key >> shift) & 255u);
    }
    __syncthreads();
    find_rank_bin(sm, need);
    prefix |= sm.digit << shift;
    mask |= 255u << shift;
    need -= sm.digit_above;
    __syncthreads();
  }
  *tau = prefix;
  *n_eq = need;
}

// Ordered selection over count items (key_at, pos_at), position order = item order: emit
// key > tau, and key == tau while fewer than n_eq such items were emitted.  Contains barriers.
template <typename KeyAt, typename PosAt>
__device__ void emit_ordered(TopkSmem& sm, KeyAt key_at, PosAt pos_at, uint32_t count, uint32_t tau, uint32_t n_eq,
                             int* out, float* vout) {
  uint32_t written = 0, eq_seen = 0;
  for (uint32_t base = 0; base < count; base += 4 * kThreads) {
    const uint32_t i0 = base + 4 * threadIdx.x;
    uint32_t key[4];
    uint32_t ce = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      key[c] = (i0 + c < count) ? key_at(i0 + c) : 0u;
      ce += (i0 + c < count && key[c] == tau) ? 1u : 0u;
    }
    uint32_t tot_e;
    uint32_t rank = eq_seen + block_excl_scan(ce, sm.wsum, tot_e);
    bool take[4];
    uint32_t cs = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      take[c] = false;
      if (i0 + c >= count) continue;
      if (key[c] > tau) {
        take[c] = true;
      } else if (key[c] == tau) {
        take[c] = rank < n_eq;
        ++rank;
      }
      cs += take[c] ? 1u : 0u;
    }
    uint32_t tot_s;
    uint32_t os = written + block_excl_scan(cs, sm.wsum, tot_s);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (take[c]) {
        out[os] = pos_at(i0 + c);
        if (vout) vout[os] = key_float(key[c]);
        ++os;
      }
    written += tot_s;
    eq_seen += tot_e;
  }
}

__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ scores, long long ld, int rows,
                                                        const int* __restrict__ row_len, int len_base, int k,
                                                        int* __restrict__ idx_out, float* __restrict__ values_out) {
  __shared__ TopkSmem sm;
  const int row = rows - 1 - (int)blockIdx.x;  // longest rows first when lengths grow with the row
  // Defensive clamp: a row never reads past its ld entries.
  const int n = max(0, (int)min((long long)(row_len ? row_len[row] : len_base + row + 1), ld));
  const int tid = threadIdx.x;
  int* out = idx_out + (size_t)row * k;
  float* vout = values_out ? values_out + (size_t)row * k : nullptr;
  const float* src = scores + (size_t)row * ld;

  if (n <= k) {
    for (int i = tid; i < k; i += kThreads) {
      out[i] = i < n ? i : -1;
      if (vout) vout[i] = i < n ? key_float(float_key(src[i])) : -INFINITY;
    }
    return;
  }

  // 1. Threshold from a sample (jittered strata; the whole row if it fits).
  const int m = n < kCap ? n : kCap;
  const int stride = n / m;  // >= 1
  for (int i = tid; i < m; i += kThreads) {
    int p = i;
    if (m < n) {
      const uint32_t h = (uint32_t)i * 2654435761u;
      p = min((int)((long long)i * n / m) + (int)((h >> 8) % (uint32_t)stride), n - 1);
    }
    sm.cand_key[i] = float_key(src[p]);
  }
  __syncthreads();
  uint32_t r;
  if (m == n) {
    r = (uint32_t)k;
  } else {
    const float e = (float)m * (float)k / (float)n;
    r = (uint32_t)fminf((float)m, 1.5f * e + 4.f * sqrtf(e) + 16.f);
  }
  uint32_t tau_lo, unused;
  radix_select(sm, [&](uint32_t i) { return sm.cand_key[i]; }, (uint32_t)m, r, &tau_lo, &unused);

  // 2. One ordered pass: every position with key >= tau_lo, in position order.  Thread t owns
  //    kPer consecutive positions per round; the next round's loads are issued before this
  //    round's scan.
  const int n4 = (n + 3) >> 2;
  const float4* src4 = reinterpret_cast<const float4*>(src);
  auto load_round = [&](int base, float4 (&v)[kPer / 4]) {
#pragma unroll
    for (int u = 0; u < kPer / 4; ++u) {
      const int i4 = ((base + kPer * tid) >> 2) + u;
      v[u] = (i4 < n4) ? src4[i4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  uint32_t n_cand = 0;
  float4 cur[kPer / 4], nxt[kPer / 4];
  load_round(0, cur);
  for (int base = 0; base < n; base += kPer * kThreads) {
    if (base + kPer * kThreads < n) load_round(base + kPer * kThreads, nxt);
    const int p0 = base + kPer * tid;
    uint32_t key[kPer];
    uint32_t cnt = 0;
#pragma unroll
    for (int u = 0; u < kPer / 4; ++u) {
      key[4 * u + 0] = float_key(cur[u].x);
      key[4 * u + 1] = float_key(cur[u].y);
      key[4 * u + 2] = float_key(cur[u].z);
      key[4 * u + 3] = float_key(cur[u].w);
    }
#pragma unroll
    for (int c = 0; c < kPer; ++c) cnt += (p0 + c < n && key[c] >= tau_lo) ? 1u : 0u;
    uint32_t tot;
    uint32_t o = n_cand + block_excl_scan(cnt, sm.wsum, tot);
    if (cnt) {
#pragma unroll
      for (int c = 0; c < kPer; ++c) {
        if (p0 + c < n && key[c] >= tau_lo) {
          if (o < (uint32_t)kCap) {
            sm.cand_key[o] = key[c];
            sm.cand_pos[o] = p0 + c;
          }
          ++o;
        }
      }
    }
    n_cand += tot;
#pragma unroll
    for (int u = 0; u < kPer / 4; ++u) cur[u] = nxt[u];
  }
  __syncthreads();

  uint32_t tau, n_eq;
  if (n_cand >= (uint32_t)k && n_cand <= (uint32_t)kCap) {
    // 3. Exact k-th key among the candidates, then the ordered selection.
    radix_select(sm, [&](uint32_t i) { return sm.cand_key[i]; }, n_cand, (uint32_t)k, &tau, &n_eq);
    emit_ordered(sm, [&](uint32_t i) { return sm.cand_key[i]; }, [&](uint32_t i) { return sm.cand_pos[i]; }, n_cand,
                 tau, n_eq, out, vout);
    return;
  }

  // Fallback: exact radix select over global memory, then an ordered emit pass.
  radix_select(sm, [&](uint32_t i) { return float_key(src[i]); }, (uint32_t)n, (uint32_t)k, &tau, &n_eq);
  emit_ordered(sm, [&](uint32_t i) { return float_key(src[i]); }, [&](uint32_t i) { return (int)i; }, (uint32_t)n,
               tau, n_eq, out, vout);
}

// Rank order for the torch.topk-shaped form: one 256-thread workgroup per row reorders the
// row's selected positions (as the selection kernels leave them, ascending) by descending
// score, equal scores by ascending position.  Each entry becomes the 64-bit word
// (~key << 32) | position, so one ascending bitonic sort of 2048 words gives that order;
// padding (-1, and the slots past k) sorts last as all-ones.  Thread t holds words 8t .. 8t+7
// in registers: compare-exchange distances below 8 stay inside a thread, 8 .. 256 are lane
// exchanges inside the wave, and only 512 and 1024 go through LDS (3 of the 66 stages).
constexpr int kRankMax = 2048;
constexpr int kRankPer = kRankMax / 256;

__device__ __forceinline__ void rank_cas(unsigned long long& a, unsigned long long& b, bool up) {
  const bool sw = (a > b) == up;
  const unsigned long long lo = sw ? b : a, hi = sw ? a : b;
  a = lo;
  b = hi;
}

__global__ __launch_bounds__(256) void topk_rank_kernel(const float* __restrict__ scores, long long ld, int k,
                                                       int* __restrict__ idx_out, float* __restrict__ values_out) {
  __shared__ unsigned long long w[kRankMax];
  const int row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  int* out = idx_out + (size_t)row * k;
  const float* src = scores + (size_t)row * ld;
  unsigned long long e[kRankPer];
#pragma unroll
  for (int j = 0; j < kRankPer; ++j) {
    const int i = kRankPer * tid + j;
    unsigned long long c = ~0ull;
    if (i < k) {
      const int p = out[i];
      if (p >= 0) c = ((unsigned long long)(~float_key(src[p])) << 32) | (uint32_t)p;
    }
    e[j] = c;
  }
#pragma unroll
  for (int size = 2; size <= kRankMax; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride >= 64 * kRankPer) {
        // partner in another wave: through LDS
#pragma unroll
        for (int j = 0; j < kRankPer; ++j) w[kRankPer * tid + j] = e[j];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kRankPer; ++j) {
          const int i = kRankPer * tid + j;
          const unsigned long long o = w[i ^ stride];
          const bool keep_min = ((i & stride) == 0) == ((i & size) == 0);
          e[j] = keep_min ? (o < e[j] ? o : e[j]) : (o > e[j] ? o : e[j]);
        }
        __syncthreads();
      } else if (stride >= kRankPer) {
        // partner in another lane of this wave (same slot j)
        const int ls = stride / kRankPer;
        const bool lower = (lane & ls) == 0;
#pragma unroll
        for (int j = 0; j < kRankPer; ++j) {
          const int i = kRankPer * tid + j;
          const unsigned long long o = __shfl_xor(e[j], ls);
          const bool keep_min = lower == ((i & size) == 0);
          e[j] = keep_min ? (o < e[j] ? o : e[j]) : (o > e[j] ? o : e[j]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < kRankPer; ++j)
          if ((j & stride) == 0) rank_cas(e[j], e[j | stride], ((kRankPer * tid + j) & size) == 0);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kRankPer; ++j) {
    const int i = kRankPer * tid + j;
    if (i < k) {
      const unsigned long long c = e[j];
      const bool pad = c == ~0ull;
      out[i] = pad ? -1 : (int)(uint32_t)c;
      if (values_out) values_out[(size_t)row * k + i] = pad ? -INFINITY : key_float(~(uint32_t)(c >> 32));
    }
  }
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (a.workspace && a.ld <= kTopkWaveMaxLd) return launch_topk_wave(a, s);
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)a.rows), dim3(kThreads), 0, s, a.scores, a.ld, a.rows, a.row_len,
                     a.len_base, a.k, a.idx_out, a.values_out);
  return hipGetLastError();
}

hipError_t launch_topk_rank(const TopkArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (a.k > kRankMax) return hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_rank_kernel, dim3((unsigned)a.rows), dim3(256), 0, s, a.scores, a.ld, a.k, a.idx_out,
                     a.values_out);
  return hipGetLastError();
}

}  // namespace dsa

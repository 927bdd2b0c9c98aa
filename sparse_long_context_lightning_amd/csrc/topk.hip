// Deterministic per-row top-k for gfx950 (one 1024-thread workgroup per row).
//
// The digest of the Keye-VL-2.0 report (mqxn.cn news 1966) keeps the 2048 best positions per
// query token (section 一) and requires the selection to be deterministic so training and
// inference agree (section 八).  Here the selected set is unique: larger score first, and among
// equal scores the lower position; the positions are returned in ascending order.
//
// Scores are mapped to order-preserving 32-bit keys (-0 folded into +0).  Per row:
//   1. a strided sample of 4096 scores gives the key range [lo, hi] the row occupies, which
//      defines 4094 equal-width buckets plus one below and one above the range, so the LDS
//      histogram spreads over many bins (few atomic collisions) even when scores cluster;
//   2. one pass builds the bucket histogram and finds the bucket b* holding the k-th key;
//   3. one ordered pass (block-wide scans keep position order) collects every position of a
//      bucket above b* (all selected) and every candidate of b* into LDS;
//   4. an 8-bit radix select over the candidates finds the exact k-th key tau and how many
//      positions equal to tau are taken; candidates are kept in position order, so the lowest
//      such positions win;
//   5. the two ascending lists are merged into the output.
// Rows whose candidate bucket overflows LDS (long runs of equal scores) fall back to an exact
// radix select over global memory followed by an ordered emit pass.  The result does not
// depend on the path taken or on thread timing.
#include "common.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 4096;
constexpr int kCap = 8192;
constexpr int kSample = 4096;

struct TopkSmem {
  uint32_t hist[kBins];
  uint32_t cand_key[kCap];
  int cand_pos[kCap];
  uint32_t sel_key[kMaxTopK];
  int sel_pos[kMaxTopK];
  uint32_t sel2_key[kMaxTopK];
  int sel2_pos[kMaxTopK];
  uint32_t wsum[kWaves];
  uint32_t red[2][kWaves];
  uint32_t bstar, n_above, digit, digit_above;
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

// Given a histogram of nbins bins (high bins = large keys) and a rank `need` (1-based, counted
// from the top), find the bin holding that rank and the count strictly above it.  Bins are
// scanned from the top in per-thread runs.  Contains barriers.
__device__ void find_rank_bin(const uint32_t* hist, int nbins, uint32_t need, TopkSmem& sm, uint32_t* out_bin,
                              uint32_t* out_above) {
  const int per = (nbins + kThreads - 1) / kThreads;  // bins per thread
  const int tid = threadIdx.x;
  // Thread tid owns bins [nbins - per*(tid+1), nbins - per*tid), scanned high to low.
  const int hi = nbins - per * tid;
  uint32_t local = 0;
  for (int j = 0; j < per; ++j) {
    const int b = hi - 1 - j;
    if (b >= 0) local += hist[b];
  }
  uint32_t tot;
  uint32_t run = block_excl_scan(local, sm.wsum, tot);
  for (int j = 0; j < per; ++j) {
    const int b = hi - 1 - j;
    if (b < 0) break;
    const uint32_t c = hist[b];
    if (run < need && run + c >= need) {
      *out_bin = (uint32_t)b;
      *out_above = run;
    }
    run += c;
  }
  __syncthreads();
}

__device__ __forceinline__ uint32_t bucket_of(uint32_t key, uint32_t lo, uint32_t hi, uint32_t shift) {
  return key < lo ? 0u : (key > hi ? (uint32_t)(kBins - 1) : 1u + ((key - lo) >> shift));
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

  // 1. Key range from a strided sample.
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  {
    const int ns = n < kSample ? n : kSample;
    for (int i = tid; i < ns; i += kThreads) {
      const long long p = (long long)i * n / ns;
      const uint32_t key = float_key(src[p]);
      kmin = min(kmin, key);
      kmax = max(kmax, key);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
      kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
    }
    if (lane_id() == 0) {
      sm.red[0][wave_id()] = kmin;
      sm.red[1][wave_id()] = kmax;
    }
    for (int i = tid; i < kBins; i += kThreads) sm.hist[i] = 0;
    __syncthreads();
    kmin = 0xFFFFFFFFu;
    kmax = 0u;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      kmin = min(kmin, sm.red[0][i]);
      kmax = max(kmax, sm.red[1][i]);
    }
  }
  const uint32_t lo = kmin, hi = kmax;
  uint32_t shift = 0;
  while (((hi - lo) >> shift) > (uint32_t)(kBins - 3)) ++shift;

  // 2. Bucket histogram (coalesced float4 reads; order does not matter here).
  const int n4 = (n + 3) >> 2;
  const float4* src4 = reinterpret_cast<const float4*>(src);
  for (int base = 0; base < n4; base += 4 * kThreads) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = base + u * kThreads + tid;
      if (i < n4) v[u] = src4[i];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = base + u * kThreads + tid;
      if (i < n4) {
        const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (4 * i + c < n) hist_add(sm.hist, bucket_of(float_key(e[c]), lo, hi, shift));
      }
    }
  }
  __syncthreads();
  find_rank_bin(sm.hist, kBins, (uint32_t)k, sm, &sm.bstar, &sm.n_above);
  const uint32_t bstar = sm.bstar;

  // 3. Ordered collection: thread tid owns 16 consecutive positions per round.
  uint32_t n_sel = 0, n_cand = 0;
  for (int base = 0; base < n; base += 16 * kThreads) {
    const int p0 = base + 16 * tid;
    float e[16];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i4 = (p0 >> 2) + u;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i4 < n4) v = src4[i4];
      e[4 * u + 0] = v.x;
      e[4 * u + 1] = v.y;
      e[4 * u + 2] = v.z;
      e[4 * u + 3] = v.w;
    }
    uint32_t key[16];
    uint32_t ca = 0, cc = 0;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      key[c] = float_key(e[c]);
      const uint32_t b = bucket_of(key[c], lo, hi, shift);
      const bool valid = p0 + c < n;
      ca += (valid && b > bstar) ? 1u : 0u;
      cc += (valid && b == bstar) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t off = block_excl_scan(ca | (cc << 16), sm.wsum, tot);
    uint32_t oa = n_sel + (off & 0xFFFFu), oc = n_cand + (off >> 16);
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      if (p0 + c >= n) break;
      const uint32_t b = bucket_of(key[c], lo, hi, shift);
      if (b > bstar) {
        sm.sel_key[oa] = key[c];
        sm.sel_pos[oa] = p0 + c;
        ++oa;
      } else if (b == bstar) {
        if (oc < (uint32_t)kCap) {
          sm.cand_key[oc] = key[c];
          sm.cand_pos[oc] = p0 + c;
        }
        ++oc;
      }
    }
    n_sel += tot & 0xFFFFu;
    n_cand += tot >> 16;
  }
  __syncthreads();

  if (n_cand <= (uint32_t)kCap) {
    // 4. Exact k-th key among the candidates: four 8-bit radix rounds in LDS.
    uint32_t need = (uint32_t)k - n_sel;  // >= 1
    uint32_t prefix = 0, mask = 0;
    for (int shift8 = 24; shift8 >= 0; shift8 -= 8) {
      for (int i = tid; i < 256; i += kThreads) sm.hist[i] = 0;
      __syncthreads();
      for (uint32_t i = tid; i < n_cand; i += kThreads) {
        const uint32_t key = sm.cand_key[i];
        if ((key & mask) == prefix) hist_add(sm.hist, (key >> shift8) & 255u);
      }
      __syncthreads();
      find_rank_bin(sm.hist, 256, need, sm, &sm.digit, &sm.digit_above);
      prefix |= sm.digit << shift8;
      mask |= 255u << shift8;
      need -= sm.digit_above;
    }
    const uint32_t tau = prefix;
    const uint32_t n_eq = need;  // positions equal to tau that are taken (lowest first)

    // Candidates in position order: select key > tau, or key == tau within the first n_eq.
    uint32_t n_sel2 = 0, eq_seen = 0;
    for (uint32_t base = 0; base < n_cand; base += 4 * kThreads) {
      const uint32_t i0 = base + 4 * tid;
      uint32_t key[4];
      int pos[4];
      uint32_t ce = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bool valid = i0 + c < n_cand;
        key[c] = valid ? sm.cand_key[i0 + c] : 0u;
        pos[c] = valid ? sm.cand_pos[i0 + c] : -1;
        ce += (valid && key[c] == tau) ? 1u : 0u;
      }
      uint32_t tot_e;
      const uint32_t off_e = block_excl_scan(ce, sm.wsum, tot_e);
      uint32_t rank = eq_seen + off_e;
      uint32_t cs = 0;
      bool take[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        take[c] = false;
        if (pos[c] < 0) continue;
        if (key[c] > tau) take[c] = true;
        else if (key[c] == tau) {
          take[c] = rank < n_eq;
          ++rank;
        }
        cs += take[c] ? 1u : 0u;
      }
      uint32_t tot_s;
      uint32_t os = n_sel2 + block_excl_scan(cs, sm.wsum, tot_s);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (take[c]) {
          sm.sel2_key[os] = key[c];
          sm.sel2_pos[os] = pos[c];
          ++os;
        }
      n_sel2 += tot_s;
      eq_seen += tot_e;
    }
    __syncthreads();

    // 5. Merge the two ascending position lists (positions are distinct).
    for (uint32_t i = tid; i < n_sel; i += kThreads) {
      const int p = sm.sel_pos[i];
      uint32_t a = 0, b = n_sel2;
      while (a < b) {
        const uint32_t m = (a + b) >> 1;
        if (sm.sel2_pos[m] < p) a = m + 1; else b = m;
      }
      out[i + a] = p;
      if (vout) vout[i + a] = key_float(sm.sel_key[i]);
    }
    for (uint32_t j = tid; j < n_sel2; j += kThreads) {
      const int p = sm.sel2_pos[j];
      uint32_t a = 0, b = n_sel;
      while (a < b) {
        const uint32_t m = (a + b) >> 1;
        if (sm.sel_pos[m] < p) a = m + 1; else b = m;
      }
      out[j + a] = p;
      if (vout) vout[j + a] = key_float(sm.sel2_key[j]);
    }
    return;
  }

  // Fallback: exact radix select over global memory, then an ordered emit pass.
  uint32_t need = (uint32_t)k;
  uint32_t prefix = 0, mask = 0;
  for (int shift8 = 24; shift8 >= 0; shift8 -= 8) {
    for (int i = tid; i < 256; i += kThreads) sm.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kThreads) {
      const uint32_t key = float_key(src[i]);
      if ((key & mask) == prefix) hist_add(sm.hist, (key >> shift8) & 255u);
    }
    __syncthreads();
    find_rank_bin(sm.hist, 256, need, sm, &sm.digit, &sm.digit_above);
    prefix |= sm.digit << shift8;
    mask |= 255u << shift8;
    need -= sm.digit_above;
  }
  const uint32_t tau = prefix;
  const uint32_t n_eq = need;
  uint32_t written = 0, eq_seen = 0;
  for (int base = 0; base < n; base += 4 * kThreads) {
    const int p0 = base + 4 * tid;
    uint32_t key[4];
    uint32_t ce = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      key[c] = (p0 + c < n) ? float_key(src[p0 + c]) : 0u;
      ce += (p0 + c < n && key[c] == tau) ? 1u : 0u;
    }
    uint32_t tot_e;
    uint32_t rank = eq_seen + block_excl_scan(ce, sm.wsum, tot_e);
    bool take[4];
    uint32_t cs = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      take[c] = false;
      if (p0 + c >= n) continue;
      if (key[c] > tau) take[c] = true;
      else if (key[c] == tau) {
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
        out[os] = p0 + c;
        if (vout) vout[os] = key_float(key[c]);
        ++os;
      }
    written += tot_s;
    eq_seen += tot_e;
  }
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)a.rows), dim3(kThreads), 0, s, a.scores, a.ld, a.rows, a.row_len,
                     a.len_base, a.k, a.idx_out, a.values_out);
  return hipGetLastError();
}

}  // namespace dsa

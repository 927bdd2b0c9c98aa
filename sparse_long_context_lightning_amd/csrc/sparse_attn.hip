// Sparse GQA attention over selected positions, for gfx950.
//
// After the indexer and top-k, attention runs only between a query token and its selected
// positions (Keye-VL-2.0 report digest, mqxn.cn news 1966, section 一).  In the GQA form every
// query head of every KV group of the token uses the token's one index set.
//
// One wave handles one (row, KV group, split) item with head_dim 128 and G = Hq / Hkv query
// heads (G <= 16).  The work is gather-bound: per selected position it fetches one 256-byte
// key row and one 256-byte value row of the group.  Per chunk of 32 positions the wave
//   * gathers the 32 key rows straight into MFMA A-operand registers (each lane reads 64
//     contiguous bytes of one row; the reduction index is permuted so this is legal) and the
//     32 value rows likewise, one chunk ahead of use (double-buffered registers), with the
//     indices fetched two chunks ahead;
//   * computes S^T = K Q^T on 16x16x32 bf16 MFMA (keys on rows, heads on columns, heads padded
//     to 16), so each lane owns one head's logits for 8 keys;
//   * runs the online softmax in base 2 on those values (the head's running max is uniform
//     over its four lane groups, the running sum stays a per-lane partial);
//   * stages the value rows in LDS and reads them back transposed as the A operand of
//     O^T += V^T P^T, whose B operand is exactly the lane's own probabilities, so the
//     rescale by exp2(m_old - m_new) is lane-local.
// Positions outside the row's causal prefix (or cache length) and negative entries are
// masked.  With nsplit > 1 each split writes unnormalised partials that a combine kernel
// merges with their (max, sum) pairs.
#include "common.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kVPitch = 128 * 2 + 16;  // bytes per LDS value row
constexpr float kLn2 = 0.69314718055994530942f;

__global__ __launch_bounds__(256) void sparse_attn_kernel(SparseAttnArgs a, float scale_log2, int n_wg) {
  __shared__ __attribute__((aligned(16))) unsigned char vlds_all[4][32 * kVPitch];
  // Workgroups reach the 8 XCDs round-robin; XCD x takes the x-th eighth of the items.  When
  // blocks of rows are skipped (attended from their merged sets instead), XCD x takes runs of 16
  // consecutive workgroups (64 rows), runs x, x + 8, ..., so every XCD keeps an even share of
  // the remaining rows while neighbouring rows, whose selections overlap, still share an L2.
  int wg;
  if (!a.skip_block) {
    wg = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  } else {
    const int xp = blockIdx.x >> 3;
    wg = ((xp >> 4) * 8 + (blockIdx.x & 7)) * 16 + (xp & 15);
  }
  if (wg >= n_wg) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, lg = lane >> 4;
  const long long item = (long long)wg * 4 + wave;
  const long long n_items = (long long)a.rows * a.nsplit * a.hkv;
  if (item >= n_items) return;
  // Prefill: KV group slowest, so all rows of group g run before group g+1 and the gathered K/V
  // rows of one group (a quarter of the cache at 4 KV heads) stay resident in the last-level
  // cache.  Decode (each cache read by one query): KV group fastest, so the waves of a workgroup
  // gather the groups of the same positions, one contiguous KiB per position between them.
  const long long per_group = (long long)a.rows * a.nsplit;
  int g;
  long long tmp;
  if (a.seq_lens) {
    g = (int)(item % a.hkv);
    tmp = item / a.hkv;
  } else {
    g = (int)(item / per_group);
    tmp = item - (long long)g * per_group;
  }
  const int sp = (int)(tmp % a.nsplit);
  const int row = (int)(tmp / a.nsplit);
  if (a.skip_block && a.skip_block[row / a.skip_block_rows]) return;  // attended from its block's merged set
  unsigned char* vlds = vlds_all[wave];

  // Row -> key/value rows and the last valid position.
  long long kv_base;
  int t_lim;
  if (a.seq_lens) {
    kv_base = (long long)row * a.s_max;
    t_lim = min(a.seq_lens[row], a.s_max) - 1;  // defensive: never read past the cache
  } else {
    int lo = 0, hi = a.batch;  // largest b with cu[b] <= row
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.cu_seqlens[mid] <= row) lo = mid; else hi = mid;
    }
    kv_base = a.cu_seqlens[lo];
    t_lim = row - a.cu_seqlens[lo];
  }
  const int hq = a.hq, hkv = a.hkv;
  const int G = hq / hkv;
  const int nchunk = (a.k_sel + 31) >> 5;
  const int cps = (nchunk + a.nsplit - 1) / a.nsplit;
  const int c_begin = sp * cps;
  const int c_end = min(nchunk, c_begin + cps);
  const int* idx_row = a.idx + (long long)row * a.k_sel;
  const size_t row_stride = (size_t)hkv * 128;  // elements between consecutive positions
  const uint16_t* kbase = a.k + ((size_t)kv_base * hkv + g) * 128 + lg * 32;
  const uint16_t* vbase = a.v + ((size_t)kv_base * hkv + g) * 128 + lg * 32;

  // Q^T as the B operand: column n = head g*G + n (zero for padding heads).
  u32x4 qreg[4];
  {
    const uint16_t* qp = a.q + ((size_t)row * hq + g * G + (n < G ? n : 0)) * 128 + lg * 32;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qreg[ks] = (n < G) ? ldg16(qp + ks * 8) : u32x4{0, 0, 0, 0};
  }

  f32x4 oacc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  auto load_idx = [&](int c, int& i0, int& i1) {
    const int s0 = c * 32 + n, s1 = s0 + 16;
    i0 = (c < c_end && s0 < a.k_sel) ? idx_row[s0] : -1;
    i1 = (c < c_end && s1 < a.k_sel) ? idx_row[s1] : -1;
  };
  auto load_kv = [&](int i0, int i1, u32x4 (&kr)[2][4], u32x4 (&vr)[2][4]) {
    const int p0 = (i0 >= 0 && i0 <= t_lim) ? i0 : 0;
    const int p1 = (i1 >= 0 && i1 <= t_lim) ? i1 : 0;
    const uint16_t* k0 = kbase + (size_t)p0 * row_stride;
    const uint16_t* k1 = kbase + (size_t)p1 * row_stride;
    const uint16_t* v0 = vbase + (size_t)p0 * row_stride;
    const uint16_t* v1 = vbase + (size_t)p1 * row_stride;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      kr[0][q] = ldg16(k0 + q * 8);
      kr[1][q] = ldg16(k1 + q * 8);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      vr[0][q] = ldg16(v0 + q * 8);
      vr[1][q] = ldg16(v1 + q * 8);
    }
  };
  auto compute = [&](int i0, int i1, const u32x4 (&kr)[2][4], const u32x4 (&vr)[2][4]) {
    // Stage the value rows: LDS row 16*j + n, bytes [64*lg, 64*lg + 64).
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<u32x4*>(vlds + (16 * j + n) * kVPitch + lg * 64 + q * 16) = vr[j][q];
    const bool ok0 = i0 >= 0 && i0 <= t_lim;
    const bool ok1 = i1 >= 0 && i1 <= t_lim;
    const uint32_t m0 = (uint32_t)(__ballot(ok0) & 0xFFFFull);
    const uint32_t m1 = (uint32_t)(__ballot(ok1) & 0xFFFFull);
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      s0 = mfma16x16x32(kr[0][ks], qreg[ks], s0);
      s1 = mfma16x16x32(kr[1][ks], qreg[ks], s1);
    }
    float z[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = ((m0 >> (4 * lg + i)) & 1u) ? s0[i] * scale_log2 : -INFINITY;
      z[4 + i] = ((m1 >> (4 * lg + i)) & 1u) ? s1[i] * scale_log2 : -INFINITY;
    }
    float mx = z[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, z[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float p[8];
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // The weights are rounded to bf16 for the P.V product; the normaliser sums the same
      // rounded values so the applied weights sum to one.
      p[i] = round_bf16(exp2f(z[i] - m_use));
      ps += p[i];
    }
    l_run = l_run * alpha + ps;
    m_run = m_new;
    const u32x4 pb = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                      pack_bf16x2(p[6], p[7])};
    wave_lds_sync();
    const uint16_t* vl = reinterpret_cast<const uint16_t*>(vlds);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int d = 16 * dt + n;
      uint32_t w4[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        // slots 2*e2, 2*e2+1 -> keys (e<4: 4*lg+e, else 16+4*lg+e-4)
        const int e0 = 2 * e2, e1 = 2 * e2 + 1;
        const int key0 = (e0 < 4) ? 4 * lg + e0 : 12 + 4 * lg + e0;
        const int key1 = (e1 < 4) ? 4 * lg + e1 : 12 + 4 * lg + e1;
        const uint32_t lo16 = vl[(key0 * kVPitch) / 2 + d];
        const uint32_t hi16 = vl[(key1 * kVPitch) / 2 + d];
        w4[e2] = lo16 | (hi16 << 16);
      }
      oacc[dt] *= alpha;
      oacc[dt] = mfma16x16x32(u32x4{w4[0], w4[1], w4[2], w4[3]}, pb, oacc[dt]);
    }
  };

  if (c_begin < c_end) {
    int ia0, ia1, ib0, ib1, ic0, ic1;
    u32x4 kA[2][4], vA[2][4], kB[2][4], vB[2][4];
    load_idx(c_begin, ia0, ia1);
    load_idx(c_begin + 1, ib0, ib1);
    load_kv(ia0, ia1, kA, vA);
    for (int c = c_begin; c < c_end; c += 2) {
      load_idx(c + 2, ic0, ic1);
      if (c + 1 < c_end) load_kv(ib0, ib1, kB, vB);
      compute(ia0, ia1, kA, vA);
      if (c + 1 >= c_end) break;
      load_idx(c + 3, ia0, ia1);
      if (c + 2 < c_end) load_kv(ic0, ic1, kA, vA);
      compute(ib0, ib1, kB, vB);
      ib0 = ia0;
      ib1 = ia1;
      ia0 = ic0;
      ia1 = ic1;
    }
  }

  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (n >= G) return;
  const int h = g * G + n;
  if (a.nsplit == 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* op = a.out + ((size_t)row * hq + h) * 128 + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      uint2 st;
      st.x = pack_bf16x2(oacc[dt][0] * inv, oacc[dt][1] * inv);
      st.y = pack_bf16x2(oacc[dt][2] * inv, oacc[dt][3] * inv);
      *reinterpret_cast<uint2*>(op + 16 * dt) = st;
    }
    if (a.lse && lg == 0) a.lse[(size_t)row * hq + h] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    const size_t slot = ((size_t)row * hq + h) * a.nsplit + sp;
    float* po = a.part_o + slot * 128 + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4*>(po + 16 * dt) = oacc[dt];
    if (lg == 0) {
      a.part_ml[slot * 2 + 0] = m_run;
      a.part_ml[slot * 2 + 1] = l_tot;
    }
  }
}

// Merge split partials: one wave per (row, head), two output dims per lane.  The splits'
// (max, sum) pairs are fetched by the lanes together (lane s holds split s, 64 splits per
// round) and reduced across the wave, so only the value rows are read in a loop, eight in flight.
__global__ __launch_bounds__(256) void attn_combine_kernel(SparseAttnArgs a) {
  const long long item = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (item >= (long long)a.rows * a.hq) return;
  const int ns = a.nsplit;
  const size_t slot0 = (size_t)item * ns;
  const float2* ml = reinterpret_cast<const float2*>(a.part_ml) + slot0;
  float mmax = -INFINITY;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    const float2 v = (s0 + lane < ns) ? ml[s0 + lane] : make_float2(-INFINITY, 0.f);
    mmax = fmaxf(mmax, v.x);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mmax = fmaxf(mmax, __shfl_xor(mmax, o));
  const float m_use = (mmax == -INFINITY) ? 0.f : mmax;
  float l = 0.f, o0 = 0.f, o1 = 0.f;
  const float2* po = reinterpret_cast<const float2*>(a.part_o + slot0 * 128) + lane;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    const float2 v = (s0 + lane < ns) ? ml[s0 + lane] : make_float2(-INFINITY, 0.f);
    const float sc_mine = (s0 + lane < ns) ? exp2f(v.x - m_use) : 0.f;
    l += v.y * sc_mine;
    const int cnt = min(64, ns - s0);
    int s = 0;
    for (; s + 8 <= cnt; s += 8) {
      float2 pv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) pv[j] = po[(size_t)(s0 + s + j) * 64];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float sc = __shfl(sc_mine, s + j);
        o0 += pv[j].x * sc;
        o1 += pv[j].y * sc;
      }
    }
    for (; s < cnt; ++s) {
      const float2 pv = po[(size_t)(s0 + s) * 64];
      const float sc = __shfl(sc_mine, s);
      o0 += pv.x * sc;
      o1 += pv.y * sc;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  reinterpret_cast<uint32_t*>(a.out + (size_t)item * 128)[lane] = pack_bf16x2(o0 * inv, o1 * inv);
  if (a.lse && lane == 0) a.lse[item] = l > 0.f ? (mmax + log2f(l)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_sparse_attn(const SparseAttnArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  const long long items = (long long)a.rows * a.nsplit * a.hkv;
  const long long n_wg = (items + 3) / 4;
  const long long grid = a.skip_block ? (n_wg + 127) / 128 * 128 : (n_wg + 7) / 8 * 8;
  const float scale_log2 = a.softmax_scale * 1.4426950408889634f;
  hipLaunchKernelGGL(sparse_attn_kernel, dim3((unsigned)grid), dim3(256), 0, s, a, scale_log2, (int)n_wg);
  return hipGetLastError();
}

hipError_t launch_attn_combine(const SparseAttnArgs& a, hipStream_t s) {
  const long long items = (long long)a.rows * a.hq;
  if (items <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace dsa

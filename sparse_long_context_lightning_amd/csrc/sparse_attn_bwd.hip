// Backward of the sparse GQA attention for gfx950: dq, dk, dv from dO.
//
// Training the whole model in the sparse mode (the sparse adaptation stage of the Keye-VL-2.0
// report digest, mqxn.cn news 1966, section 一) sends gradients through the attention over the
// selected positions.  Per query head h of KV group g and selected key s, with p the forward's
// softmax weights (recomputed from the saved log-sum-exp):
//     dp_s = <dO_h, v_s>,  D_h = <dO_h, O_h>,  dz_s = p_s (dp_s - D_h)
//     dq_h = scale sum_s dz_s k_s,   dk_s += scale sum_h dz_s q_h,   dv_s += sum_h p_s dO_h
// One wave handles one (row, KV group) item, like the forward: per chunk of 32 selected
// positions the key and value rows are gathered straight into MFMA A registers (next chunk in
// flight), S^T = K Q^T and dP^T = V dO^T run on 16x16x32 bf16 MFMA with heads on the column
// axis, so p and dz are lane-local; dQ^T += K^T dZ^T reads the key rows back transposed from
// LDS; dz and p are written to LDS once more in key-major order so that dK^T = Q^T dZ and
// dV^T = dO^T P run on 16x16x16 bf16 MFMA (reduction over the group's heads), and each key's
// 128 + 128 fp32 contributions are added to dk / dv with hardware float atomics, staged through
// LDS so that one atomic instruction covers 64 consecutive floats of one key row (the L2 then
// sees two cache lines per instruction rather than sixteen; 4x faster in measurement).  Rows
// select keys independently, so the scatter has no structure to exploit; atomics make dk / dv
// exact sums in an order that varies from run to run.
#include "common.h"
#include "kernels.h"

namespace dsa {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// 16x16x16 bf16 MFMA: lane l supplies A[l % 16][4 (l / 16) + e] and B[4 (l / 16) + e][l % 16]
// (e = 0..3, two dwords each) and receives C[4 (l / 16) + i][l % 16].
__device__ __forceinline__ f32x4 mfma16x16x16(const uint2& a, const uint2& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0,
                                                   0, 0);
}

constexpr int kKPitch = 128 * 2 + 16;  // bytes per LDS key row
constexpr int kAccPitch = 128 + 4;     // floats per LDS row of a 16-key dk / dv tile
constexpr float kLog2e = 1.4426950408889634f;

__global__ __launch_bounds__(256) void sparse_attn_bwd_kernel(SparseAttnBwdArgs a, float scale_log2, int n_wg) {
  __shared__ __attribute__((aligned(16))) unsigned char klds_all[4][32 * kKPitch];
  __shared__ __attribute__((aligned(16))) uint16_t zt_all[4][2][32 * 16];  // [dz | p][key][head], bf16
  __shared__ __attribute__((aligned(16))) float acc_all[4][2][16 * kAccPitch];  // [dk | dv][key][d]
  const int per_xcd = gridDim.x >> 3;
  const int wg = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (wg >= n_wg) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, lg = lane >> 4;
  const long long item = (long long)wg * 4 + wave;
  if (item >= (long long)a.rows * a.hkv) return;
  // KV group slowest, as in the forward.
  const int g = (int)(item / a.rows);
  const int row = (int)(item - (long long)g * a.rows);
  if (a.skip_block && a.skip_block[row / a.skip_block_rows] != 0) return;  // done over its block's merged set
  unsigned char* klds = klds_all[wave];
  uint16_t* zt = zt_all[wave][0];
  uint16_t* pt = zt_all[wave][1];
  float* dkl = acc_all[wave][0];
  float* dvl = acc_all[wave][1];

  int lo = 0, hi = a.batch;  // largest b with cu[b] <= row
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.cu_seqlens[mid] <= row) lo = mid; else hi = mid;
  }
  const long long kv_base = a.cu_seqlens[lo];
  const int t_lim = row - a.cu_seqlens[lo];
  const int hq = a.hq, hkv = a.hkv;
  const int G = hq / hkv;
  const int nchunk = (a.k_sel + 31) >> 5;
  const int* idx_row = a.idx + (long long)row * a.k_sel;
  const size_t row_stride = (size_t)hkv * 128;
  const uint16_t* kbase = a.k + ((size_t)kv_base * hkv + g) * 128 + lg * 32;
  const uint16_t* vbase = a.v + ((size_t)kv_base * hkv + g) * 128 + lg * 32;
  const bool head_ok = n < G;
  const int h = g * G + (head_ok ? n : 0);

  // B operands Q^T and dO^T (column n = head g*G + n, zero past G); the reduction index of
  // k-step ks in lane group lg is the 8-dim piece 4 lg + ks.
  u32x4 qreg[4], doreg[4];
  float dsum = 0.f;
  {
    const size_t base = ((size_t)row * hq + h) * 128 + lg * 32;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qreg[ks] = head_ok ? ldg16(a.q + base + ks * 8) : u32x4{0, 0, 0, 0};
      doreg[ks] = head_ok ? ldg16(a.dout + base + ks * 8) : u32x4{0, 0, 0, 0};
      const u32x4 o4 = head_ok ? ldg16(a.out + base + ks * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dsum += __uint_as_float(doreg[ks][e] << 16) * __uint_as_float(o4[e] << 16);
        dsum += __uint_as_float(doreg[ks][e] & 0xFFFF0000u) * __uint_as_float(o4[e] & 0xFFFF0000u);
      }
    }
  }
  dsum += __shfl_xor(dsum, 16);
  dsum += __shfl_xor(dsum, 32);
  const float D = dsum;
  const float lse2 = head_ok ? a.lse[(size_t)row * hq + h] * kLog2e : 0.f;

  // A operands for the head reductions, d-major: QT[dt] = Q[head 4 lg + e][d = 16 dt + n].
  uint2 qt[8], dot[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    uint32_t qv[4], dv4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int hh = 4 * lg + e;
      const size_t off = ((size_t)row * hq + g * G + (hh < G ? hh : 0)) * 128 + 16 * dt + n;
      qv[e] = hh < G ? a.q[off] : 0u;
      dv4[e] = hh < G ? a.dout[off] : 0u;
    }
    qt[dt] = make_uint2(qv[0] | (qv[1] << 16), qv[2] | (qv[3] << 16));
    dot[dt] = make_uint2(dv4[0] | (dv4[1] << 16), dv4[2] | (dv4[3] << 16));
  }

  f32x4 dqacc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) dqacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float* dk_g = a.dk + (size_t)kv_base * row_stride + (size_t)g * 128;
  float* dv_g = a.dv + (size_t)kv_base * row_stride + (size_t)g * 128;
  const float scale = a.softmax_scale;

  auto load_idx = [&](int c, int& i0, int& i1) {
    const int s0 = c * 32 + n, s1 = s0 + 16;
    i0 = (c < nchunk && s0 < a.k_sel) ? idx_row[s0] : -1;
    i1 = (c < nchunk && s1 < a.k_sel) ? idx_row[s1] : -1;
  };
  auto load_kv = [&](int i0, int i1, u32x4 (&kr)[2][4], u32x4 (&vr)[2][4]) {
    const int p0 = (i0 >= 0 && i0 <= t_lim) ? i0 : 0;
    const int p1 = (i1 >= 0 && i1 <= t_lim) ? i1 : 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      kr[0][q] = ldg16(kbase + (size_t)p0 * row_stride + q * 8);
      kr[1][q] = ldg16(kbase + (size_t)p1 * row_stride + q * 8);
      vr[0][q] = ldg16(vbase + (size_t)p0 * row_stride + q * 8);
      vr[1][q] = ldg16(vbase + (size_t)p1 * row_stride + q * 8);
    }
  };
  auto compute = [&](int i0, int i1, const u32x4 (&kr)[2][4], const u32x4 (&vr)[2][4]) {
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<u32x4*>(klds + (16 * j + n) * kKPitch + lg * 64 + q * 16) = kr[j][q];
    const bool ok0 = i0 >= 0 && i0 <= t_lim;
    const bool ok1 = i1 >= 0 && i1 <= t_lim;
    const uint32_t m0 = (uint32_t)(__ballot(ok0) & 0xFFFFull);
    const uint32_t m1 = (uint32_t)(__ballot(ok1) & 0xFFFFull);
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0, dp0 = s0, dp1 = s0;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      s0 = mfma16x16x32(kr[0][ks], qreg[ks], s0);
      s1 = mfma16x16x32(kr[1][ks], qreg[ks], s1);
      dp0 = mfma16x16x32(vr[0][ks], doreg[ks], dp0);
      dp1 = mfma16x16x32(vr[1][ks], doreg[ks], dp1);
    }
    float p[8], dz[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool v0 = head_ok && ((m0 >> (4 * lg + i)) & 1u);
      const bool v1 = head_ok && ((m1 >> (4 * lg + i)) & 1u);
      p[i] = v0 ? exp2f(s0[i] * scale_log2 - lse2) : 0.f;
      p[4 + i] = v1 ? exp2f(s1[i] * scale_log2 - lse2) : 0.f;
      dz[i] = p[i] * (dp0[i] - D);
      dz[4 + i] = p[4 + i] * (dp1[i] - D);
    }
    // dQ^T += K^T dZ^T.  B slot 2 e2 (+1) carries key 4 lg + e (e < 4) or 16 + 4 lg + e - 4.
    const u32x4 zb = {pack_bf16x2(dz[0], dz[1]), pack_bf16x2(dz[2], dz[3]), pack_bf16x2(dz[4], dz[5]),
                      pack_bf16x2(dz[6], dz[7])};
    // Key-major copies of dz and p (bf16) for the reductions over heads.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      zt[(4 * lg + i) * 16 + n] = (uint16_t)(pack_bf16x2(dz[i], 0.f) & 0xFFFFu);
      zt[(16 + 4 * lg + i) * 16 + n] = (uint16_t)(pack_bf16x2(dz[4 + i], 0.f) & 0xFFFFu);
      pt[(4 * lg + i) * 16 + n] = (uint16_t)(pack_bf16x2(p[i], 0.f) & 0xFFFFu);
      pt[(16 + 4 * lg + i) * 16 + n] = (uint16_t)(pack_bf16x2(p[4 + i], 0.f) & 0xFFFFu);
    }
    wave_lds_sync();
    const uint16_t* kl = reinterpret_cast<const uint16_t*>(klds);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int d = 16 * dt + n;
      uint32_t w4[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int e0 = 2 * e2, e1 = 2 * e2 + 1;
        const int key0 = (e0 < 4) ? 4 * lg + e0 : 12 + 4 * lg + e0;
        const int key1 = (e1 < 4) ? 4 * lg + e1 : 12 + 4 * lg + e1;
        const uint32_t lo16 = kl[(key0 * kKPitch) / 2 + d];
        const uint32_t hi16 = kl[(key1 * kKPitch) / 2 + d];
        w4[e2] = lo16 | (hi16 << 16);
      }
      dqacc[dt] = mfma16x16x32(u32x4{w4[0], w4[1], w4[2], w4[3]}, zb, dqacc[dt]);
    }
    // dK^T = Q^T dZ and dV^T = dO^T P for keys 16 kt + n.  The 16-key tiles go through LDS so
    // that each atomic instruction covers 64 consecutive floats of one key row (two cache
    // lines) instead of one 16-float piece of 16 rows.
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const uint32_t mk = kt ? m1 : m0;
      const uint2 zbk = *reinterpret_cast<const uint2*>(zt + (16 * kt + n) * 16 + 4 * lg);
      const uint2 pbk = *reinterpret_cast<const uint2*>(pt + (16 * kt + n) * 16 + 4 * lg);
      if (kt) wave_lds_sync();  // the previous tile's reads are done before it is overwritten
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const f32x4 ck = mfma16x16x16(qt[dt], zbk, f32x4{0.f, 0.f, 0.f, 0.f});
        const f32x4 cv = mfma16x16x16(dot[dt], pbk, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dkl[n * kAccPitch + 16 * dt + 4 * lg + i] = scale * ck[i];
          dvl[n * kAccPitch + 16 * dt + 4 * lg + i] = cv[i];
        }
      }
      wave_lds_sync();
      // key kk of the tile: position from lane kk's index (lanes 0..15 hold keys n of the chunk)
#pragma unroll 4
      for (int j = 0; j < 32; ++j) {
        const int kk = j >> 1;
        if (!((mk >> kk) & 1u)) continue;  // uniform: masked keys add nothing
        const int pos = __shfl(kt ? i1 : i0, kk);
        const int dcol = (j & 1) * 64 + lane;
        unsafeAtomicAdd(dk_g + (size_t)pos * row_stride + dcol, dkl[kk * kAccPitch + dcol]);
        unsafeAtomicAdd(dv_g + (size_t)pos * row_stride + dcol, dvl[kk * kAccPitch + dcol]);
      }
    }
  };

  if (nchunk > 0) {
    int ia0, ia1, ib0, ib1, ic0, ic1;
    u32x4 kA[2][4], vA[2][4], kB[2][4], vB[2][4];
    load_idx(0, ia0, ia1);
    load_idx(1, ib0, ib1);
    load_kv(ia0, ia1, kA, vA);
    for (int c = 0; c < nchunk; c += 2) {
      load_idx(c + 2, ic0, ic1);
      if (c + 1 < nchunk) load_kv(ib0, ib1, kB, vB);
      compute(ia0, ia1, kA, vA);
      if (c + 1 >= nchunk) break;
      load_idx(c + 3, ia0, ia1);
      if (c + 2 < nchunk) load_kv(ic0, ic1, kA, vA);
      compute(ib0, ib1, kB, vB);
      ib0 = ia0;
      ib1 = ia1;
      ia0 = ic0;
      ia1 = ic1;
    }
  }

  if (!head_ok) return;
  float* dqp = a.dq + ((size_t)row * hq + h) * 128 + 4 * lg;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4*>(dqp + 16 * dt) = dqacc[dt] * scale;
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ p, long long n) {
  const long long stride = (long long)gridDim.x * 256;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) p[i] = 0.f;
}

}  // namespace

hipError_t launch_zero_f32(float* p, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const unsigned zgrid = (unsigned)std::min<long long>((n + 255) / 256, 16384);
  hipLaunchKernelGGL(zero_f32_kernel, dim3(zgrid), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_sparse_attn_bwd(const SparseAttnBwdArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (!a.skip_block) {
    const long long nkv = (long long)a.rows * a.hkv * 128;
    hipError_t e = launch_zero_f32(a.dk, nkv, s);
    if (e == hipSuccess) e = launch_zero_f32(a.dv, nkv, s);
    if (e != hipSuccess) return e;
  }
  const long long items = (long long)a.rows * a.hkv;
  const long long n_wg = (items + 3) / 4;
  const long long grid = (n_wg + 7) / 8 * 8;
  const float scale_log2 = a.softmax_scale * kLog2e;
  hipLaunchKernelGGL(sparse_attn_bwd_kernel, dim3((unsigned)grid), dim3(256), 0, s, a, scale_log2, (int)n_wg);
  return hipGetLastError();
}

}  // namespace dsa

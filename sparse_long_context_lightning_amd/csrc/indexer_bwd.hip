// Backward of the lightning-indexer scores for gfx950 (bf16 MFMA, fp32 accumulation).
//
// The indexer of the Keye-VL-2.0 report digest (mqxn.cn news 1966, section 一) is trained in the
// dense warm-up stage to follow the full attention distribution, so its scores
//     I[t, s] = sum_j w[t, j] * relu(c[t, j, s]),   c[t, j, s] = <q_idx[t, j], k_idx[s]>,
// need a backward.  With g[t, s] the incoming gradient of I and m = [c > 0]:
//     u[t, j]  = sum_s g[t, s] m[t, j, s] k_idx[s]
//     dq[t, j] = w[t, j] u[t, j]
//     dw[t, j] = sum_s g[t, s] relu(c[t, j, s]) = <q_idx[t, j], u[t, j]>      (m c = relu(c))
//     dk[s]    = sum_t sum_j g[t, s] m[t, j, s] (w[t, j] q_idx[t, j])
// Two kernels share the work.  The query-major one streams key tiles through LDS and keeps u of
// its (token, head) rows in registers (dq, dw); the key-major one streams query tokens through
// LDS and keeps dk of its keys in registers.  Each recomputes c on MFMA with the forward's
// operands and fp32 accumulation, so m is the forward's ReLU decision; the second contraction
// takes g m (g w m for dk) rounded to bf16.  That contraction runs over the keys (or the heads),
// so its A operand is the staged tile read transposed, with ds_read_b64_tr_b16.
//
// MFMA C layout: lane (a, n) with a = lane / 16, n = lane % 16 holds C[4a + i][n], i = 0..3.
// Both second contractions take their B operand straight from the first one's C registers:
// C rows 4a + i of two 16-row tiles (h = 0, 1) become the 8 reduction slots e = 4h + i of lane
// group a, and the transposed reads gather the same 8 tile rows 32p + 16h + 4a + i for lane
// group a, so both operands agree on which key (head) each slot carries.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kBH = 64;    // indexer heads
constexpr int kBD = 128;   // indexer dim

constexpr int kRowTileBytes = 64 * 256;

// Row tiles of both passes (64 keys, or one token's 64 heads) are staged with the swz layout and
// read both ways (row-wise and transposed).
__device__ __forceinline__ const uint16_t* swz_tile_src(const uint16_t* base, int P, int lane, int last_row) {
  const int row = 4 * P + (lane >> 4);
  const int piece = (lane & 15) ^ swz(row);
  return base + (size_t)min(row, last_row) * kBD + piece * 8;
}

// ---------------------------------------------------------------------------------------
// dq and dw: a workgroup of 2 NTOK waves takes NTOK consecutive query rows of one sequence and
// one split of their keys; wave w handles heads 32 (w & 1) .. + 31 of token w / 2.  Per 64-key
// tile (the k rows and the tokens' g values DMA'd to LDS, in a ring of NST stages):
//   X^T = K Q^T           (A: key rows from LDS, B: the wave's q rows in registers)
//   u^T += K^T (g m)^T    (A: the same key rows read transposed, B: bf16 of g m from the X^T
//                          registers)
template <int NTOK, int NST>
__global__ __launch_bounds__(128 * NTOK) void indexer_bwd_q_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx, const float* __restrict__ w,
    const float* __restrict__ g, long long ld, int seq_off, int row_begin, int row_end, int grad_row0,
    float* __restrict__ dq, float* __restrict__ dw, int key_split, int n_rowblk, int n_items, int accumulate) {
  constexpr int NWV = 2 * NTOK;
  constexpr int GBYTES = ((NTOK * 256 + 1023) / 1024) * 1024;
  constexpr int NJOB = 16 + GBYTES / 1024;
  __shared__ __attribute__((aligned(16))) unsigned char kt_lds[NST][kRowTileBytes];
  __shared__ __attribute__((aligned(16))) float g_lds[NST][GBYTES / 4];

  const int per_xcd = gridDim.x >> 3;
  const int wi = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (wi >= n_items) return;
  const int split = wi / n_rowblk;
  const int rb = wi - split * n_rowblk;
  const int r0 = row_begin + rb * NTOK;
  const int t_last = min(r0 + NTOK, row_end) - 1 - seq_off;
  const int kbeg = split * key_split;
  if (kbeg > t_last) return;
  const int kend = min(kbeg + key_split, t_last + 1);
  const int ntiles = (kend - kbeg + 63) >> 6;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, lg = lane >> 4;
  const int tok = wave >> 1, hh = wave & 1;
  const int r = r0 + tok;
  const bool row_ok = r < row_end;
  const int rr = min(r, row_end - 1);
  const int t = rr - seq_off;

  // B operands of X^T: head 32 hh + 16 ht + n, reduction piece lg * 4 + ks (as the forward).
  u32x4 qreg[2][4];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const uint16_t* qp = q_idx + ((size_t)rr * kBH + 32 * hh + 16 * ht + n) * kBD + lg * 32;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qreg[ht][ks] = ldg16(qp + ks * 8);
  }
  f32x4 u[8][2];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) u[dt][ht] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint16_t* kseq = k_idx + (size_t)seq_off * kBD;
  // DMA jobs of 1 KiB each per stage: P = wave, wave + NWV, ... < NJOB.
  const int jobs = (NJOB - wave + NWV - 1) / NWV;
  auto stage = [&](int it) {
    const int buf = it % NST;
    const int key0 = kbeg + it * 64;
    const int last = kend - 1 - key0;
    for (int P = wave; P < NJOB; P += NWV) {
      if (P < 16) {
        lds_dma16_untracked(swz_tile_src(kseq + (size_t)key0 * kBD, P, lane, last), &kt_lds[buf][P * 1024]);
      } else {
        const int m = (P - 16) * 64 + lane;  // 16-byte piece: token m / 16, keys 4 (m % 16) ..
        const int gr = min(r0 + min(m >> 4, NTOK - 1), row_end - 1);
        int a = key0 + 4 * (m & 15);
        if (a > gr - seq_off) a = 0;  // past the row's prefix: any valid address (masked below)
        lds_dma16_untracked(g + (size_t)(gr - grad_row0) * ld + a, reinterpret_cast<unsigned char*>(g_lds[buf]) + (P - 16) * 1024);
      }
    }
  };

  // Ring of NST stages: tiles it + 1 .. it + NST - 1 are in flight while tile it is used.
  for (int i = 0; i < NST - 1 && i < ntiles; ++i) stage(i);
  vm_wait_at_most(jobs * (min(NST - 1, ntiles) - 1));
  ring_barrier();

  for (int it = 0; it < ntiles; ++it) {
    const int buf = it % NST;
    if (it + NST - 1 < ntiles) stage(it + NST - 1);
    const int key0 = kbeg + it * 64;
    if (row_ok && key0 <= t) {
      const unsigned char* ktile = kt_lds[buf];
      const bool diag = key0 + 63 > t;   // the token's last tile: keys past t get g = 0
      // Transposed reads: lane j of lane group lg addresses key 32 p + 16 h + 4 lg + j / 4, dims
      // 16 dt + 4 (j % 4) .. + 3, so lane n receives dim 16 dt + n of those four keys.
      const int trow = 4 * lg + (n >> 2);
      const int tm = n & 3;
      const int tsw = swz(trow);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        // All LDS operands of the 32-key pair first, so their latency hides under the MFMAs.
        u32x4 ax[2][4], au[8];
        f32x4 gv[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const unsigned char* bp = ktile + (16 * (2 * p + h) + n) * 256;
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            ax[h][ks] = *reinterpret_cast<const u32x4*>(bp + (((lg * 4 + ks) ^ swz(n)) << 4));
          gv[h] = *reinterpret_cast<const f32x4*>(&g_lds[buf][tok * 64 + 16 * (2 * p + h) + 4 * lg]);
        }
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const int piece = 2 * dt + (tm >> 1);
          const unsigned char* b0 = ktile + (32 * p + trow) * 256 + ((piece ^ tsw) << 4) + 8 * (tm & 1);
          const uint2 lo = lds_read_tr16(b0);
          const uint2 hi = lds_read_tr16(b0 + 16 * 256);
          au[dt] = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
        f32x4 x[2][2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int ht = 0; ht < 2; ++ht) x[h][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int ht = 0; ht < 2; ++ht) x[h][ht] = mfma16x16x32(ax[h][ks], qreg[ht][ks], x[h][ht]);
        if (diag) {
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (key0 + 16 * (2 * p + h) + 4 * lg + i > t) gv[h][i] = 0.f;
        }
        u32x4 yv[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int ht = 0; ht < 2; ++ht) {
            yv[ht][2 * h] = cvt_bf16x2(x[h][ht][0] > 0.f ? gv[h][0] : 0.f, x[h][ht][1] > 0.f ? gv[h][1] : 0.f);
            yv[ht][2 * h + 1] = cvt_bf16x2(x[h][ht][2] > 0.f ? gv[h][2] : 0.f, x[h][ht][3] > 0.f ? gv[h][3] : 0.f);
          }
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
          for (int ht = 0; ht < 2; ++ht) u[dt][ht] = mfma16x16x32(au[dt], yv[ht], u[dt][ht]);
      }
    }
    // Tile it + 1 must have landed; later stages may stay in flight.
    if (it + 1 < ntiles) vm_wait_at_most(jobs * (min(it + NST - 1, ntiles - 1) - (it + 1)));
    ring_barrier();
  }

  if (!row_ok) return;
  // Lane (lg, n) holds u^T[16 dt + 4 lg + i][head 32 hh + 16 ht + n].
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const int head = 32 * hh + 16 * ht + n;
    const size_t hrow = (size_t)r * kBH + head;
    const float wv = w[hrow];
    const uint16_t* qp = q_idx + hrow * kBD + 4 * lg;
    float* dqp = dq + hrow * kBD + 4 * lg;
    float dot = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const uint2 qv = *reinterpret_cast<const uint2*>(qp + 16 * dt);
      dot = fmaf(__uint_as_float(qv.x << 16), u[dt][ht][0], dot);
      dot = fmaf(__uint_as_float(qv.x & 0xFFFF0000u), u[dt][ht][1], dot);
      dot = fmaf(__uint_as_float(qv.y << 16), u[dt][ht][2], dot);
      dot = fmaf(__uint_as_float(qv.y & 0xFFFF0000u), u[dt][ht][3], dot);
      const f32x4 v = u[dt][ht] * wv;
      if (accumulate) {
#pragma unroll
        for (int i = 0; i < 4; ++i) unsafeAtomicAdd(dqp + 16 * dt + i, v[i]);
      } else {
        *reinterpret_cast<f32x4*>(dqp + 16 * dt) = v;
      }
    }
    dot += __shfl_xor(dot, 16);
    dot += __shfl_xor(dot, 32);
    if (lg == 0) {
      if (accumulate) unsafeAtomicAdd(dw + hrow, dot);
      else dw[hrow] = dot;
    }
  }
}

// ---------------------------------------------------------------------------------------
// dk: a workgroup of NW waves takes 16 KT NW consecutive keys of one sequence and one group of
// query tokens; wave w holds keys 16 KT w .. + 16 KT - 1 of the block.  Per token (its 64 q rows, its g
// values over the block and its 64 weights DMA'd to LDS, double buffered):
//   X = Q K^T             (A: q rows from LDS, B: the wave's key rows in registers)
//   dk^T += Q^T (g w m)   (A: the same q rows read transposed, B: bf16 of g w m from the X
//                          registers)
// and the block's dk is added to the output with fp32 atomics at the end.
template <int NW, int KT, int NST>
__global__ __launch_bounds__(64 * NW) void indexer_bwd_k_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, const uint16_t* __restrict__ k_idx,
    const float* __restrict__ g, long long ld, int seq_off, int row_begin, int row_end, int grad_row0,
    float* __restrict__ dk, int tok_group, int n_keyblk, int n_items) {
  constexpr int KB = 16 * KT * NW;  // keys of the block (16 KT per wave)
  constexpr int GBYTES = ((KB * 4 + 256 + 1023) / 1024) * 1024;  // g of the block, then the 64 weights
  constexpr int NJOB = 16 + GBYTES / 1024;
  __shared__ __attribute__((aligned(16))) unsigned char q_lds[NST][kRowTileBytes];
  __shared__ __attribute__((aligned(16))) float g_lds[NST][GBYTES / 4];

  const int per_xcd = gridDim.x >> 3;
  const int wi = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (wi >= n_items) return;
  const int tg = wi / n_keyblk;
  const int kb = wi - tg * n_keyblk;
  const int kb0 = kb * KB;                                     // local key of the block start
  const int tb = row_begin - seq_off + tg * tok_group;         // local token range of the group
  const int te = min(tb + tok_group, row_end - seq_off);
  const int ts = max(tb, kb0);                                  // earlier tokens see none of the block
  if (ts >= te) return;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, lg = lane >> 4;
  const int kw0 = kb0 + 16 * KT * wave;

  // B operands of X: key kw0 + 16 kt + n, reduction piece lg * 4 + ks.
  u32x4 kreg[KT][4];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const int key = min(kw0 + 16 * kt + n, te - 1);
    const uint16_t* kp = k_idx + ((size_t)seq_off + key) * kBD + lg * 32;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kreg[kt][ks] = ldg16(kp + ks * 8);
  }
  f32x4 acc[8][KT];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) acc[dt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int jobs = (NJOB - wave + NW - 1) / NW;
  auto stage = [&](int tl) {
    const int buf = (tl - ts) % NST;
    const int r = seq_off + tl;
    for (int P = wave; P < NJOB; P += NW) {
      if (P < 16) {
        lds_dma16_untracked(swz_tile_src(q_idx + (size_t)r * kBH * kBD, P, lane, kBH - 1), &q_lds[buf][P * 1024]);
      } else {
        const int m = (P - 16) * 64 + lane;  // 16-byte piece of the g / w region
        const float* src;
        if (m < KB / 4) {
          int a = kb0 + 4 * m;
          if (a > tl) a = kb0;  // past the row's prefix: any valid address (masked below)
          src = g + (size_t)(r - grad_row0) * ld + a;
        } else {
          src = w + (size_t)r * kBH + 4 * min(m - KB / 4, kBH / 4 - 1);
        }
        lds_dma16_untracked(src, reinterpret_cast<unsigned char*>(g_lds[buf]) + (P - 16) * 1024);
      }
    }
  };

  // Ring of NST stages: tokens tl + 1 .. tl + NST - 1 are in flight while token tl is used.
  const int ntok = te - ts;
  for (int i = 0; i < NST - 1 && i < ntok; ++i) stage(ts + i);
  vm_wait_at_most(jobs * (min(NST - 1, ntok) - 1));
  ring_barrier();

  for (int tl = ts; tl < te; ++tl) {
    const int buf = (tl - ts) % NST;
    if (tl + NST - 1 < te) stage(tl + NST - 1);
    if (kw0 <= tl) {
      const unsigned char* qtile = q_lds[buf];
      const float* wl = g_lds[buf] + KB;  // the token's 64 weights
      float gk[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const int key = kw0 + 16 * kt + n;
        gk[kt] = (key <= tl) ? g_lds[buf][key - kb0] : 0.f;
      }
      // Transposed reads: lane j of lane group lg addresses head 32 p + 16 h + 4 lg + j / 4,
      // dims 16 dt + 4 (j % 4) .. + 3, so lane n receives dim 16 dt + n of those four heads.
      const int trow = 4 * lg + (n >> 2);
      const int tm = n & 3;
      const int tsw = swz(trow);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        u32x4 yv[KT];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int ht = 2 * p + h;
          f32x4 x[KT];
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) x[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
          const unsigned char* bp = qtile + (16 * ht + n) * 256;
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(bp + (((lg * 4 + ks) ^ swz(n)) << 4));
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) x[kt] = mfma16x16x32(a, kreg[kt][ks], x[kt]);
          }
          // weights of heads 16 ht + 4 lg + i (the C rows this lane holds)
          const f32x4 wv = *reinterpret_cast<const f32x4*>(wl + 16 * ht + 4 * lg);
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
            const f32x4 gw = wv * gk[kt];
            yv[kt][2 * h] = cvt_bf16x2(x[kt][0] > 0.f ? gw[0] : 0.f, x[kt][1] > 0.f ? gw[1] : 0.f);
            yv[kt][2 * h + 1] = cvt_bf16x2(x[kt][2] > 0.f ? gw[2] : 0.f, x[kt][3] > 0.f ? gw[3] : 0.f);
          }
        }
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const int piece = 2 * dt + (tm >> 1);
          const unsigned char* b0 = qtile + (32 * p + trow) * 256 + ((piece ^ tsw) << 4) + 8 * (tm & 1);
          const uint2 lo = lds_read_tr16(b0);
          const uint2 hi = lds_read_tr16(b0 + 16 * 256);
          const u32x4 a = u32x4{lo.x, lo.y, hi.x, hi.y};
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) acc[dt][kt] = mfma16x16x32(a, yv[kt], acc[dt][kt]);
        }
      }
    }
    if (tl + 1 < te) vm_wait_at_most(jobs * (min(tl + NST - 1, te - 1) - (tl + 1)));
    ring_barrier();
  }

  // Lane (lg, n) holds dk^T[16 dt + 4 lg + i][key kw0 + 16 kt + n]; keys past the group's last
  // token received nothing (and may lie past the sequence).
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const int key = kw0 + 16 * kt + n;
    if (key >= te) continue;
    float* dkp = dk + ((size_t)seq_off + key) * kBD + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) unsafeAtomicAdd(dkp + 16 * dt + i, acc[dt][kt][i]);
  }
}

__global__ void bwd_zero_kernel(float* __restrict__ p, long long n) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

constexpr int kBwdTok = 4;     // query tokens per dq workgroup (8 waves)
constexpr int kBwdKeyW = 12;   // waves per dk workgroup
constexpr int kBwdKeyT = 2;    // 16-key tiles per dk wave (384 keys per workgroup)
constexpr int kBwdTokGroup = 128;
constexpr int kBwdStages = 2;  // staging ring depth of the dk pass
constexpr int kBwdStagesQ = 2; // and of the dq pass

}  // namespace

hipError_t launch_indexer_bwd(const IndexerBwdArgs& a, hipStream_t s) {
  const int rows = a.row_end - a.row_begin;
  if (rows <= 0) return hipSuccess;
  const int t_last = a.row_end - 1 - a.seq_off;
  const int nkeys = t_last + 1;
  // dq, dw: row blocks x key splits; split the keys only while the row blocks alone leave
  // the chip under-filled.
  const int n_rowblk = (rows + kBwdTok - 1) / kBwdTok;
  const int ktiles = (nkeys + 63) / 64;
  int nsplit = n_rowblk >= 256 ? 1 : std::min(ktiles, (512 + n_rowblk - 1) / n_rowblk);
  const int key_split = ((ktiles + nsplit - 1) / nsplit) * 64;
  nsplit = (nkeys + key_split - 1) / key_split;
  const int accumulate = nsplit > 1;
  if (accumulate) {
    hipLaunchKernelGGL(bwd_zero_kernel, dim3(std::min(1024, (rows * kBH * kBD + 255) / 256)), dim3(256), 0, s,
                       a.dq + (size_t)a.row_begin * kBH * kBD, (long long)rows * kBH * kBD);
    hipLaunchKernelGGL(bwd_zero_kernel, dim3(std::min(1024, (rows * kBH + 255) / 256)), dim3(256), 0, s,
                       a.dw + (size_t)a.row_begin * kBH, (long long)rows * kBH);
  }
  const int q_items = n_rowblk * nsplit;
  hipLaunchKernelGGL((indexer_bwd_q_kernel<kBwdTok, kBwdStagesQ>), dim3((q_items + 7) / 8 * 8), dim3(128 * kBwdTok), 0, s,
                     a.q_idx, a.k_idx, a.w, a.g, a.ld, a.seq_off, a.row_begin, a.row_end, a.grad_row0, a.dq, a.dw,
                     key_split, n_rowblk, q_items, accumulate);

  // dk: key blocks x token groups.
  const int n_keyblk = (nkeys + 16 * kBwdKeyT * kBwdKeyW - 1) / (16 * kBwdKeyT * kBwdKeyW);
  const int n_tg = (rows + kBwdTokGroup - 1) / kBwdTokGroup;
  const int k_items = n_keyblk * n_tg;
  hipLaunchKernelGGL((indexer_bwd_k_kernel<kBwdKeyW, kBwdKeyT, kBwdStages>), dim3((k_items + 7) / 8 * 8), dim3(64 * kBwdKeyW), 0, s,
                     a.q_idx, a.w, a.k_idx, a.g, a.ld, a.seq_off, a.row_begin, a.row_end,
                     a.grad_row0, a.dk, kBwdTokGroup, n_keyblk, k_items);
  return hipGetLastError();
}

}  // namespace dsa

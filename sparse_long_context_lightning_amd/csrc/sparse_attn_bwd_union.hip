// Backward of the sparse GQA attention over the merged index sets of blocks of adjacent rows,
// for gfx950.
//
// The sparse adaptation stage trains the whole model in the sparse mode (Keye-VL-2.0 report
// digest, mqxn.cn news 1966, section 一), so the gradient passes through the attention over the
// selected positions:
//     p_s = exp(scale <q_h, k_s> - lse_h),  dp_s = <dO_h, v_s>,  D_h = <dO_h, O_h>,
//     dz_s = p_s (dp_s - D_h),  dq_h = scale sum_s dz_s k_s,
//     dk_s += scale sum_h dz_s q_h,  dv_s += sum_h p_s dO_h.
// Per row, dk and dv are a scatter over 2048 positions per KV group: 2 x 128 floats per
// selected (row, group), added with float atomics, whose device-wide rate (about 3.3e11 adds/s
// on MI355X, the same for any address pattern with at least 16 consecutive floats of a row per
// instruction) bounds the per-row kernel.  Adjacent rows share many positions (the observation
// behind the adjacent-query dedup of the report's section 八), so here one workgroup takes a
// block of R rows and one KV group, walks the block's merged set (ascending packed KV rows with
// a 32-bit row mask each, built by query_union_kernel<32>) in chunks of 32 positions, and sums
// each position's contributions over all the block's (row, head) columns before adding them:
// one atomic per (merged position, group, dim) instead of one per (row, selected position,
// group, dim).
//
// The block's Q and dO rows stay in LDS for the whole walk (64 KiB each at R x G = 256 columns).
// Per chunk (K and V rows gathered one chunk ahead through registers into LDS):
//   phase A, wave w on its 32 (row, head) columns: S^T = K Q^T and dP^T = V dO^T on 16x16x32
//     bf16 MFMA (keys on rows, columns lane-local), p and dz lane-local (a column's row bit in
//     the key's mask selects; the others are 0), dQ^T += K^T dZ^T with K^T read transposed from
//     LDS (ds_read_b64_tr_b16), dz stored as bf16 [key][column] in LDS;
//   phase B, wave w on its 128 / NW dims: dK = dZ^T Q with the reduction over all R x G columns
//     (Q read transposed from LDS), each 16 x 16 result tile added to dk with float atomics, four
//     key rows x 16 consecutive floats per instruction; then p replaces dz in LDS and
//     dV = P^T dO is formed and added the same way.
#include "common.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kRowBytes = 128 * 2;  // one row of 128 bf16 in LDS (swz layout)
constexpr float kLog2e = 1.4426950408889634f;

template <int G>
struct BwdShape {
  static constexpr int R = G == 16 ? 16 : 32;  // rows per block
  static constexpr int COLS = R * G;           // (row, head) columns of a block and KV group
  static constexpr int NW = COLS / 32;         // waves: 32 columns each in phase A
  static constexpr int DS = 128 / NW;          // head dims per wave in phase B
  static constexpr int NT = DS / 16;           // 16-dim result tiles per wave
  static constexpr int KS = COLS / 32;         // k-steps of phase B's column reduction
  static constexpr int PPT = 8 / NW;           // 16-byte pieces of K (and of V) per thread and chunk
};

template <int G>
__global__ __launch_bounds__(64 * BwdShape<G>::NW) void sparse_attn_bwd_union_kernel(UnionBwdArgs a, float scale_log2,
                                                                                      int n_blocks) {
  using S = BwdShape<G>;
  constexpr int R = S::R, COLS = S::COLS, NW = S::NW, DS = S::DS, NT = S::NT, KS = S::KS, PPT = S::PPT;
  constexpr int PITCH = COLS * 2;  // bytes per key row of the dZ / P store
  // Q and dO rows of the block's columns (column c = block row c / G, head c % G of the group),
  // piece p of row r at slot p ^ swz(r); zeros for rows past the end.
  __shared__ __attribute__((aligned(16))) unsigned char q_lds[COLS * kRowBytes];
  __shared__ __attribute__((aligned(16))) unsigned char do_lds[COLS * kRowBytes];
  // K rows 0..31 then V rows 0..31 of the chunk, piece p of row r at slot p ^ swz(r).
  __shared__ __attribute__((aligned(16))) unsigned char kv_lds[2 * kUnionChunk * kRowBytes];
  // dZ, then P (bf16) [key][column], 16-byte piece p of key row r at slot p ^ (r mod 16).
  __shared__ __attribute__((aligned(16))) unsigned char zp_lds[kUnionChunk * PITCH];

  // Latest blocks (largest merged sets) first; the KV groups of a block side by side.
  const int wi = blockIdx.x;
  if (wi >= n_blocks * a.hkv) return;
  const int blk = n_blocks - 1 - wi / a.hkv;
  const int g = wi - (wi / a.hkv) * a.hkv;
  if (a.use_union && a.use_union[blk] == 0) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, lg = lane >> 4;
  const int r0 = blk * R;
  const int hq = a.hq, rows = a.rows;
  const int n_u = min(a.counts[blk], a.cap);
  const int nchunk = (n_u + kUnionChunk - 1) / kUnionChunk;
  const int* urows = a.kv_rows + (size_t)blk * a.cap;
  const uint32_t* umask = a.masks + (size_t)blk * a.cap;
  const size_t kv_stride = (size_t)a.hkv * 128;  // elements (or floats) per packed KV row
  const float scale = a.softmax_scale;

  // The block's Q and dO rows into LDS.
  for (int q = tid; q < COLS * 16; q += 64 * NW) {
    const int col = q >> 4, pc = q & 15;
    const int row = r0 + col / G;
    const size_t off = ((size_t)(row < rows ? row : 0) * hq + g * G + col % G) * 128 + pc * 8;
    const int slot = (col * kRowBytes) + ((pc ^ swz(col)) << 4);
    *reinterpret_cast<u32x4*>(q_lds + slot) = row < rows ? ldg16(a.q + off) : u32x4{0, 0, 0, 0};
    *reinterpret_cast<u32x4*>(do_lds + slot) = row < rows ? ldg16(a.dout + off) : u32x4{0, 0, 0, 0};
  }

  // Per lane: columns 32 wave + 16 c + n (c = 0, 1): row bit, D = <dO, O> and lse in base 2.
  int rb[2];
  float dcol[2], lse2[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int col = 32 * wave + 16 * c + n;
    rb[c] = col / G;
    const int row = r0 + rb[c];
    const bool ok = row < rows;
    const size_t base = ((size_t)(ok ? row : 0) * hq + g * G + col % G) * 128 + lg * 32;
    float dsum = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4 d4 = ok ? ldg16(a.dout + base + ks * 8) : u32x4{0, 0, 0, 0};
      const u32x4 o4 = ok ? ldg16(a.out + base + ks * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dsum += __uint_as_float(d4[e] << 16) * __uint_as_float(o4[e] << 16);
        dsum += __uint_as_float(d4[e] & 0xFFFF0000u) * __uint_as_float(o4[e] & 0xFFFF0000u);
      }
    }
    dsum += __shfl_xor(dsum, 16);
    dsum += __shfl_xor(dsum, 32);
    dcol[c] = dsum;
    lse2[c] = ok ? a.lse[(size_t)row * hq + g * G + col % G] * kLog2e : 0.f;
  }

  f32x4 dqacc[8][2];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) dqacc[dt][0] = dqacc[dt][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Gather: piece u of this thread is q = tid + 64 NW u: key q / 16, 16-byte piece q % 16.
  // Metadata per lane: positions and masks of keys 4 lg + i (lo) and 16 + 4 lg + i (hi), the
  // keys of the lane's result rows in both phases.
  const uint16_t* kg = a.k + (size_t)g * 128;
  const uint16_t* vg = a.v + (size_t)g * 128;
  int posr[PPT];
  u32x4 kreg[PPT], vreg[PPT];
  u32x4 nplo, nphi, nmlo, nmhi;  // the next chunk's metadata
  auto load_pos = [&](int ch) {
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int key = (tid + 64 * NW * u) >> 4;
      posr[u] = min(max(urows[ch * kUnionChunk + key], 0), rows - 1);  // a foreign list cannot leave K / V
    }
  };
  auto gather = [&]() {
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int pc = (tid + 64 * NW * u) & 15;
      kreg[u] = ldg16(kg + (size_t)posr[u] * kv_stride + pc * 8);
      vreg[u] = ldg16(vg + (size_t)posr[u] * kv_stride + pc * 8);
    }
  };
  auto load_meta = [&](int ch) {
    const int b = ch * kUnionChunk + 4 * lg;
    nplo = ldg16(urows + b);
    nphi = ldg16(urows + b + 16);
    nmlo = ldg16(umask + b);
    nmhi = ldg16(umask + b + 16);
  };
  auto put = [&]() {
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int q = tid + 64 * NW * u, key = q >> 4, pc = q & 15;
      const int slot = (pc ^ swz(key)) << 4;
      *reinterpret_cast<u32x4*>(kv_lds + key * kRowBytes + slot) = kreg[u];
      *reinterpret_cast<u32x4*>(kv_lds + (kUnionChunk + key) * kRowBytes + slot) = vreg[u];
    }
  };

  // Transposed-read lane roles: row 4 lg + (n >> 2) (+ 16), dims 4 (n & 3) .. + 3 of a 16-dim tile.
  const int trow = 4 * lg + (n >> 2), tm = n & 3, tsw = swz(trow);
  const unsigned char* kt = kv_lds;
  const unsigned char* vt = kv_lds + kUnionChunk * kRowBytes;

  // Phase A.  Leaves dz and p of the lane's keys and columns as bf16 pairs (B-operand order) in
  // zb and pb.
  auto phase_a = [&](const u32x4& mlo, const u32x4& mhi, u32x4 (&zb)[2], u32x4 (&pb)[2]) {
    f32x4 s[2][2], dp[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int c = 0; c < 2; ++c) s[j][c] = dp[j][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      // B operands Q^T, dO^T: column 32 wave + 16 c + n, dims of piece 4 lg + ks.
      u32x4 bq[2], bo[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int col = 32 * wave + 16 * c + n;
        const int off = col * kRowBytes + (((4 * lg + ks) ^ swz(col)) << 4);
        bq[c] = *reinterpret_cast<const u32x4*>(q_lds + off);
        bo[c] = *reinterpret_cast<const u32x4*>(do_lds + off);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int off = (16 * j + n) * kRowBytes + (((4 * lg + ks) ^ swz(n)) << 4);
        const u32x4 ak = *reinterpret_cast<const u32x4*>(kt + off);
        const u32x4 av = *reinterpret_cast<const u32x4*>(vt + off);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          s[j][c] = mfma16x16x32(ak, bq[c], s[j][c]);
          dp[j][c] = mfma16x16x32(av, bo[c], dp[j][c]);
        }
      }
    }
    // p and dz of key 16 j + 4 lg + i, column 32 wave + 16 c + n, packed to bf16 pairs in the
    // B-operand order of dQ (slot e: key 16 (e / 4) + 4 lg + e % 4).
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float pz[8], zz[8];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t m = j ? mhi[i] : mlo[i];
          const bool sel = (m >> rb[c]) & 1u;
          const float p = sel ? exp2f(s[j][c][i] * scale_log2 - lse2[c]) : 0.f;
          pz[4 * j + i] = p;
          zz[4 * j + i] = p * (dp[j][c][i] - dcol[c]);
        }
      zb[c] = u32x4{pack_bf16x2(zz[0], zz[1]), pack_bf16x2(zz[2], zz[3]), pack_bf16x2(zz[4], zz[5]),
                    pack_bf16x2(zz[6], zz[7])};
      pb[c] = u32x4{pack_bf16x2(pz[0], pz[1]), pack_bf16x2(pz[2], pz[3]), pack_bf16x2(pz[4], pz[5]),
                    pack_bf16x2(pz[6], pz[7])};
    }
    // dQ^T += K^T dZ^T with K^T read transposed from the key rows.
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int piece = 2 * dt + (tm >> 1);
      const unsigned char* p = kt + trow * kRowBytes + ((piece ^ tsw) << 4) + 8 * (tm & 1);
      const uint2 lo = lds_read_tr16(p);
      const uint2 hi = lds_read_tr16(p + 16 * kRowBytes);
      const u32x4 akt = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
      for (int c = 0; c < 2; ++c) dqacc[dt][c] = mfma16x16x32(akt, zb[c], dqacc[dt][c]);
    }
  };
  // bf16 values (B-operand order, slot e = key 16 (e / 4) + 4 lg + e % 4) of the lane's two
  // columns into the [key][column] store.
  auto store_zp = [&](const u32x4 (&v)[2]) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int col = 32 * wave + 16 * c + n;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = 16 * (e >> 2) + 4 * lg + (e & 3);
        const int off = key * PITCH + ((((col >> 3) ^ (key & 15))) << 4) + (col & 7) * 2;
        *reinterpret_cast<uint16_t*>(zp_lds + off) = (uint16_t)(v[c][e >> 1] >> (16 * (e & 1)));
      }
    }
  };
  // Phase B on the store's contents against Q (src = q_lds) or dO (do_lds), results scaled by
  // `mul` and added to dst (dk or dv) at the lane's keys.
  auto phase_b = [&](const unsigned char* src, float* dst, float mul, const u32x4& plo, const u32x4& phi,
                     const u32x4& mlo, const u32x4& mhi) {
    f32x4 acc[2][NT];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[j][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // B operand [column 32 ks + 8 lg + e][dim wave DS + 16 nt + n]: two transposed reads of
      // columns 32 ks + 8 lg + 4 h + 0..3.
      u32x4 b[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int piece = (wave * DS + 16 * nt) / 8 + (tm >> 1);
        uint2 h2[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int r = 32 * ks + 8 * lg + 4 * h + (n >> 2);
          h2[h] = lds_read_tr16(src + r * kRowBytes + ((piece ^ swz(r)) << 4) + 8 * (tm & 1));
        }
        b[nt] = u32x4{h2[0].x, h2[0].y, h2[1].x, h2[1].y};
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int off = (16 * j + n) * PITCH + (((4 * ks + lg) ^ n) << 4);
        const u32x4 az = *reinterpret_cast<const u32x4*>(zp_lds + off);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[j][nt] = mfma16x16x32(az, b[nt], acc[j][nt]);
      }
    }
    // Result row 4 lg + i of tile j is key 16 j + 4 lg + i; column n is dim wave DS + 16 nt + n.
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if ((j ? mhi[i] : mlo[i]) == 0u) continue;  // padding: no row selected it
        const int pos = min(max((int)(j ? phi[i] : plo[i]), 0), rows - 1);
        float* p = dst + (size_t)pos * kv_stride + g * 128 + wave * DS + n;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) unsafeAtomicAdd(p + 16 * nt, mul * acc[j][nt][i]);
      }
  };

  if (nchunk > 0) {
    load_pos(0);
    gather();
    load_meta(0);
    if (nchunk > 1) load_pos(1);
    for (int ch = 0; ch < nchunk; ++ch) {
      put();
      const u32x4 plo = nplo, phi = nphi, mlo = nmlo, mhi = nmhi;
      if (ch + 1 < nchunk) {
        gather();
        load_meta(ch + 1);
        if (ch + 2 < nchunk) load_pos(ch + 2);
      }
      __syncthreads();  // the chunk's K / V rows (and, the first time, Q / dO) in LDS; last P read
      u32x4 zb[2], pb[2];
      phase_a(mlo, mhi, zb, pb);
      store_zp(zb);
      __syncthreads();  // dZ complete; every wave's K / V reads of the chunk done
      phase_b(q_lds, a.dk, scale, plo, phi, mlo, mhi);
      __syncthreads();  // dZ read
      store_zp(pb);
      __syncthreads();  // P complete
      phase_b(do_lds, a.dv, 1.f, plo, phi, mlo, mhi);
    }
  }

#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int col = 32 * wave + 16 * c + n;
    const int row = r0 + col / G;
    if (row >= rows) continue;
    float* dqp = a.dq + ((size_t)row * hq + g * G + col % G) * 128 + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4*>(dqp + 16 * dt) = dqacc[dt][c] * scale;
  }
}

}  // namespace

bool union_bwd_supported(int hq, int hkv) {
  const int g = hkv > 0 ? hq / hkv : 0;
  return hkv > 0 && hq % hkv == 0 && (g == 4 || g == 8 || g == 16);
}

int union_bwd_block_rows(int g) { return g == 16 ? BwdShape<16>::R : g == 8 ? BwdShape<8>::R : BwdShape<4>::R; }

hipError_t launch_sparse_attn_bwd_union(const UnionBwdArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (!union_bwd_supported(a.hq, a.hkv)) return hipErrorInvalidValue;
  const int G = a.hq / a.hkv;
  const int R = union_bwd_block_rows(G);
  const int n_blocks = (a.rows + R - 1) / R;
  const unsigned grid = (unsigned)((long long)n_blocks * a.hkv);
  const float scale_log2 = a.softmax_scale * kLog2e;
  switch (G) {
    case 4:
      hipLaunchKernelGGL(sparse_attn_bwd_union_kernel<4>, dim3(grid), dim3(64 * BwdShape<4>::NW), 0, s, a, scale_log2,
                         n_blocks);
      break;
    case 8:
      hipLaunchKernelGGL(sparse_attn_bwd_union_kernel<8>, dim3(grid), dim3(64 * BwdShape<8>::NW), 0, s, a, scale_log2,
                         n_blocks);
      break;
    default:
      hipLaunchKernelGGL(sparse_attn_bwd_union_kernel<16>, dim3(grid), dim3(64 * BwdShape<16>::NW), 0, s, a,
                         scale_log2, n_blocks);
      break;
  }
  return hipGetLastError();
}

}  // namespace dsa

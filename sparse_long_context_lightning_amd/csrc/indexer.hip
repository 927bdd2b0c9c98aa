// Lightning-indexer score kernels for gfx950 (bf16 MFMA, fused ReLU * weight * head sum).
//
// The indexer of the Keye-VL-2.0 report digest (mqxn.cn news 1966, section 一) scores every
// earlier position of a query token with several light heads that share one key per
// position (MQA).  The score this library computes is
//     I[t, s] = sum_j w[t, j] * max(0, <q_idx[t, j, :], k_idx[s, :]>).
//
// Both kernels run the contraction on 16x16x32 bf16 MFMA with the (token, head) rows of the
// query side on the MFMA row axis and 16 keys on the column axis, so each lane ends a tile
// holding four (head, key) results of one key column: ReLU, the weight multiply and most of
// the head sum are lane-local, and the remaining sum over the four lane groups is folded
// into a transpose-reduction that leaves lane l with the score of key l of a 64-key tile
// (one coalesced 256-byte store per token and tile).
//
// The reduction dimension is permuted: MFMA slot (lane group g, k-step s, element e) carries
// d = (g * NKS + s) * 8 + e, so each lane reads one contiguous 16*NKS-byte run of a key row.
#include "common.h"
#include "kernels.h"

namespace dsa {
namespace {

// Sum the partial scores of four 16-key subtiles over the four lane groups; on return lane l
// holds the total for subtile l / 16, column l % 16, i.e. key l of the 64-key tile.
// permlane32_swap(a, b) yields (a.lo32 | b.lo32, a.hi32 | b.hi32) and permlane16_swap does the
// same per 16-lane quarter inside each half, so the sum of the two results pairs every lane
// with its partner group in one exchange: three exchanges and three adds in all.
__device__ __forceinline__ float swap_sum32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(a), __float_as_int(b), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}
__device__ __forceinline__ float swap_sum16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(a), __float_as_int(b), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}
// Slot permutation of a key row's 16-byte pieces in an LDS tile.  ds_read_b128 serves a wave in
// lane groups that mix the four 16-lane quarters, so the plain row XOR (piece ^ r) puts lanes of
// different quarters on the same slots; 256-byte rows use swz, which keeps every group on
// distinct slots (128-byte rows keep the plain XOR).
template <int CPR>
__device__ __forceinline__ int tile_swizzle(int r) {
  if constexpr (CPR == 16) return swz(r);
  return r % CPR;
}

__device__ __forceinline__ float transpose_reduce4(float p0, float p1, float p2, float p3) {
  // lanes < 32 now hold subtiles 0 / 1 over groups {g, g^2}; lanes >= 32 subtiles 2 / 3
  const float k0 = swap_sum32(p0, p2);
  const float k1 = swap_sum32(p1, p3);
  return swap_sum16(k0, k1);
}

// ---------------------------------------------------------------------------------------
// Prefill: a workgroup of 4 waves scores 4 * (16 RT / H) consecutive query rows of one
// sequence against one split of keys; key tiles of 64 rows are staged in LDS (double buffered)
// and shared by the 4 waves.  Each wave keeps its 16 RT (token, head) query rows in registers
// (RT = 4: one token of 64 heads), so every key operand read from LDS feeds RT MFMAs.
//
// MODE 0 writes the scores (with only_rows set, only for the 4-row blocks holding a flagged row:
// the fused top-k's rescoring pass).  The prefill's fused top-k adds two modes (64 heads only,
// one token per wave):
//   MODE 1 (sample): the workgroup's keys are 2048 stratified positions of the causal prefix of
//     its first row (one jittered run of 4 in each of 512 strata; 4096 in 1024 strata past
//     131072 positions, where 2048 would leave too few samples above the k-th score to keep the
//     candidate count inside the list; or the whole prefix when it is no longer), gathered tile
//     by tile by kSampleSplits workgroups; each row with more than k positions gets their scores
//     as floats at the start of its candidate list and their number in tau_lo;
//   MODE 2 (emit): every (key, position) whose key reaches the row's tau_lo is staged in LDS and
//     appended to the row's candidate list with one atomic per stage; no score is written, so
//     neither this pass nor the top-k moves the score rows through memory.
constexpr int kSampleCount = 2048;  // sample positions per row (512 strata of 4)
constexpr int kSampleLongRow = 131072;  // longer prefixes take 2 kSampleCount positions
constexpr int kSampleSplits = 4;    // workgroups per row block in the sampling pass (512 entries each)
constexpr int kEmitStage = 512;     // staged candidates per wave

template <int H, int DI, int RT, int MODE>
__global__ __launch_bounds__(256) void indexer_prefill_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx, const float* __restrict__ w,
    int seq_off, int row_begin, int row_end, int out_row0, float* __restrict__ scores, long long ld,
    int key_split, int n_rowblk, uint32_t* __restrict__ tau_lo, uint32_t* __restrict__ cnt,
    uint2* __restrict__ cand, int topk, const uint32_t* __restrict__ only_rows) {
  static_assert(MODE == 0 || (H == 64 && RT == 4), "the fused top-k modes take one 64-head token per wave");
  // RT row tiles of 16 (token, head) rows per wave.
  constexpr int TOKW = (H >= 16) ? 16 * RT / H : 4 * RT;  // tokens per wave (H = 4: 4 per row tile)
  constexpr int TOKWG = 4 * TOKW;
  constexpr int NKS = DI / 32;
  constexpr int PITCH = DI * 2;       // bytes per LDS key row
  constexpr int CPR = DI / 8;         // 16-byte chunks per key row
  constexpr int NLD = 64 * CPR / 256; // chunks each thread stages per tile
  constexpr int NSLOT = (H >= 16) ? TOKW : RT;
  static_assert(H == 4 || H == 16 || H == 32 || H == 64, "unsupported indexer head count");
  static_assert(DI == 64 || DI == 128, "unsupported indexer dim");
  // Key tiles: 64 rows, chunk c of row r stored at slot c ^ tile_swizzle<CPR>(r) (the swizzle keeps
  // the MFMA operand reads free of bank conflicts without padding, so whole waves can fill the
  // tile with direct global-to-LDS loads).
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][64 * PITCH];

  // XCD-aware order: consecutive work items (same key split, neighbouring rows) land on the
  // same XCD, whose L2 then serves the shared key tiles.
  const int per_xcd = gridDim.x >> 3;
  const int wi = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  const int split = wi / n_rowblk;
  const int rb = wi - split * n_rowblk;
  const int r0 = row_begin + rb * TOKWG;
  if (r0 >= row_end) return;
  if (MODE == 0 && only_rows) {
    bool any = false;
#pragma unroll
    for (int i = 0; i < TOKWG; ++i) any |= r0 + i < row_end && only_rows[r0 + i - out_row0] != 0;
    if (!any) return;
  }
  const int t_last = min(r0 + TOKWG, row_end) - 1 - seq_off;
  // MODE 1: the sample of the first row's prefix (n0 positions), m <= msz entries
  const int n0 = r0 - seq_off + 1;
  const int msz = n0 > kSampleLongRow ? 2 * kSampleCount : kSampleCount;
  const bool whole = n0 <= msz;
  const uint32_t sf = whole ? 1u : (uint32_t)(n0 >> 2) / (uint32_t)(msz / 4);  // float4 slots per stratum
  const int m = whole ? n0 : msz;
  if (MODE == 1 && t_last + 1 <= topk) return;  // no row needs a threshold
  // MODE 1: split s takes sample entries [s * msz / kSampleSplits, ...) of the m
  const int kbeg = MODE == 1 ? split * (msz / kSampleSplits) : split * key_split;
  if (MODE == 1 ? kbeg >= m : kbeg > t_last) return;
  const int kend = MODE == 1 ? min(m, kbeg + msz / kSampleSplits) : min(kbeg + key_split, t_last + 1);
  const int ntiles = (kend - kbeg + 63) >> 6;

  // the wave index is uniform over the wave: kept in a scalar register, as is all that derives from it
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 15, lg = lane >> 4;

  // Query rows of this wave as MFMA A operands: lane supplies row 16*rt + n.
  u32x4 areg[RT][NKS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int m = 16 * rt + n;
    const int tok = (H >= 16) ? wave * TOKW + m / H : wave * TOKW + m / 4;
    const int head = (H >= 16) ? m % H : m % 4;
    const int r = min(r0 + tok, row_end - 1);
    const uint16_t* qp = q_idx + ((size_t)r * H + head) * DI + lg * NKS * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) areg[rt][ks] = ldg16(qp + ks * 8);
  }
  // Weights of the C rows this lane holds: row 16*rt + 4*lg + i.
  float wreg[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 16 * rt + 4 * lg + i;
      const int tok = (H >= 16) ? wave * TOKW + m / H : wave * TOKW + m / 4;
      const int head = (H >= 16) ? m % H : m % 4;
      const int r = min(r0 + tok, row_end - 1);
      wreg[rt][i] = w[(size_t)r * H + head];
    }
  // Local position of the wave's last valid token (for skipping fully-masked tiles).
  const int wave_t_last = min(r0 + wave * TOKW + TOKW, row_end) - 1 - seq_off;
  const int wave_r0 = r0 + wave * TOKW;

  // Tile staging: instruction p of wave w fills LDS bytes [p*4096 + w*1024, +1024) of the
  // tile, lane l the 16 bytes at + 16 l, i.e. row r = (p*4096 + w*1024 + 16 l) / PITCH, slot
  // l % CPR, which holds the row's chunk (l % CPR) ^ tile_swizzle(r).  Full tiles use fixed
  // per-thread byte offsets from a tile base that advances uniformly (kept in scalar registers,
  // as are the LDS destinations, so a copy costs no vector instruction); only the last, partial
  // tile clamps its rows to the key range.
  // (MODE 1 gathers by absolute position: its base is the sequence start)
  const char* ktile = reinterpret_cast<const char*>(k_idx + (size_t)(seq_off + (MODE == 1 ? 0 : kbeg)) * DI);
  int st_row[NLD];
  uint32_t st_off[NLD];      // byte offset of the lane's 16 bytes within a tile
  uint32_t lds_dst[2][NLD];  // wave-uniform LDS destinations
#pragma unroll
  for (int p = 0; p < NLD; ++p) {
    const int pos = p * 4096 + wave * 1024 + lane * 16;
    const int r = pos / PITCH;
    const int chunk = (lane % CPR) ^ tile_swizzle<CPR>(r);
    st_row[p] = r;
    st_off[p] = (uint32_t)(r * DI + chunk * 8) * 2u;
#pragma unroll
    for (int b = 0; b < 2; ++b)
      lds_dst[b][p] = __builtin_amdgcn_readfirstlane(lds_offset(&lds[b][p * 4096 + wave * 1024]));
  }
  auto load_tile = [&](int tile, int buf) {
    if (MODE == 1) {
      // gathered rows: row rr of the tile is sample entry j = 64 tile + rr (the last one repeated
      // past m), stratum j / 4 at its jittered slot
#pragma unroll
      for (int p = 0; p < NLD; ++p) {
        const uint32_t j = (uint32_t)min(kbeg + tile * 64 + st_row[p], m - 1);
        const uint32_t st = j >> 2;
        const uint32_t pos = whole ? j : 4u * (st * sf + ((st * 2654435761u) >> 8) % sf) + (j & 3u);
        const uint32_t off = pos * (uint32_t)(DI * 2) + (st_off[p] - (uint32_t)st_row[p] * (uint32_t)(DI * 2));
        lds_dma16_saddr(ktile, off, buf ? lds_dst[1][p] : lds_dst[0][p]);
      }
      return;
    }
    const char* base = ktile + (size_t)tile * 64 * DI * 2;
    const int keys_left = kend - kbeg - tile * 64;
    if (keys_left >= 64) {
#pragma unroll
      for (int p = 0; p < NLD; ++p) lds_dma16_saddr(base, st_off[p], buf ? lds_dst[1][p] : lds_dst[0][p]);
    } else {
#pragma unroll
      for (int p = 0; p < NLD; ++p) {
        const uint32_t off = st_off[p] - (uint32_t)(st_row[p] - min(st_row[p], keys_left - 1)) * (uint32_t)(DI * 2);
        lds_dma16_saddr(base, off, buf ? lds_dst[1][p] : lds_dst[0][p]);
      }
    }
  };
  auto wait_tile = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  // MODE 1: the wave's sample scores, staged in LDS until the end (so the tile waits need not
  // wait for stores) — at most 2 kSampleCount / kSampleSplits entries.
  constexpr int kSmpStage = MODE == 1 ? 2 * kSampleCount / kSampleSplits : 1;
  __shared__ float smp_stage_all[MODE == 1 ? 4 : 1][kSmpStage];
  float* smp_stage = smp_stage_all[MODE == 1 ? wave : 0];

  // MODE 2: this wave's token (one per wave), its threshold and its candidate list.
  __shared__ uint2 stage_all[MODE == 2 ? 4 : 1][MODE == 2 ? kEmitStage : 1];
  uint2* stage = stage_all[MODE == 2 ? wave : 0];
  uint32_t ns = 0;
  const int er = wave_r0 - out_row0;  // the token's row in the top-k scratch
  const bool e_ok = MODE == 2 && wave_r0 < row_end && wave_r0 - seq_off + 1 > topk;
  const uint32_t tau = e_ok ? tau_lo[er] : 0xFFFFFFFFu;
  // The same test on the float itself: the key order is the float order (non-NaN scores, -0 = +0)
  // and key_float inverts float_key, so float_key(v) >= tau exactly when v >= tau_f (the one key
  // with no float, 0x7FFFFFFF, gives -0.0, which is still the right bound; no threshold: NaN).
  const float tau_f = key_float(tau);
  auto flush = [&]() {
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(&cnt[er], ns);
    base = __shfl(base, 0);
    wave_lds_sync();
    uint2* cand_row = cand + (size_t)er * kTopkCandCap;
    for (uint32_t i = lane; i < ns; i += 64)
      if (base + i < (uint32_t)kTopkCandCap) cand_row[base + i] = stage[i];
    ns = 0;
    wave_lds_sync();
  };

  load_tile(0, 0);
  wait_tile();
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    if (it + 1 < ntiles) load_tile(it + 1, (it + 1) & 1);
    const int key0 = kbeg + it * 64;
    if (wave_r0 < row_end && (MODE == 1 || key0 <= wave_t_last)) {
      const unsigned char* tile = lds[it & 1];
      float part[4][NSLOT];
      // Software pipeline over the four 16-key subtiles: the B operand of subtile st + 1 is read
      // from LDS while subtile st's MFMAs run, and the ReLU / weight / head-sum epilogue of
      // subtile st - 1 is interleaved with those MFMAs (one MFMA, then two VALU operations), so
      // each wave keeps the matrix pipe fed through its own epilogue.
      auto read_b = [&](int st, u32x4 (&b)[NKS]) {
        const unsigned char* bp = tile + (16 * st + n) * PITCH;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          b[ks] = *reinterpret_cast<const u32x4*>(bp + (((lg * NKS + ks) ^ tile_swizzle<CPR>(n)) * 16));
      };
      auto mma = [&](const u32x4 (&b)[NKS], f32x4 (&c)[RT]) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) c[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) c[rt] = mfma16x16x32(areg[rt][ks], b[ks], c[rt]);
      };
      auto epilogue = [&](const f32x4 (&c)[RT], float (&p)[NSLOT]) {
#pragma unroll
        for (int s = 0; s < NSLOT; ++s) p[s] = 0.f;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int slot = (H >= 16) ? (16 * rt) / H : rt;
#pragma unroll
          for (int i = 0; i < 4; ++i) p[slot] = fmaf(relu(c[rt][i]), wreg[rt][i], p[slot]);
        }
      };
      // A pipeline stage's schedule: its LDS reads (nr instructions) first, then one MFMA and two
      // VALU operations (ReLU and fma of one earlier result) at a time; stages are fenced off
      // from each other.
      auto schedule = [&](auto reads) {
        if constexpr (decltype(reads)::value) __builtin_amdgcn_sched_group_barrier(0x100, NKS, 0);
#pragma unroll
        for (int i = 0; i < RT * NKS; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      };
      u32x4 b0[NKS], b1[NKS];
      f32x4 c0[RT], c1[RT];
      read_b(0, b0);
      read_b(1, b1);
      mma(b0, c0);
      __builtin_amdgcn_sched_barrier(0);
      read_b(2, b0);
      mma(b1, c1);
      epilogue(c0, part[0]);
      schedule(std::true_type{});
      read_b(3, b1);
      mma(b0, c0);
      epilogue(c1, part[1]);
      schedule(std::true_type{});
      mma(b1, c1);
      epilogue(c0, part[2]);
      schedule(std::false_type{});
      epilogue(c1, part[3]);
      if constexpr (H >= 16) {
#pragma unroll
        for (int s = 0; s < NSLOT; ++s) {
          const float v = transpose_reduce4(part[0][s], part[1][s], part[2][s], part[3][s]);
          const int r = wave_r0 + s;
          const int key = key0 + lane;
          if (MODE == 1) {
            if (key < kend) smp_stage[key - kbeg] = v;
            continue;
          }
          if (MODE == 0 && r < row_end && key <= r - seq_off) scores[(size_t)(r - out_row0) * ld + key] = v;
          if (MODE == 2) {
            const bool take = e_ok && key <= r - seq_off && v >= tau_f;
            const unsigned long long b = __ballot(take);
            if (b != 0ull) {
              if (take) stage[ns + __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u))] =
                  make_uint2(float_key(v), (uint32_t)key);
              ns += (uint32_t)__popcll(b);
              if (ns > (uint32_t)(kEmitStage - 64)) flush();
            }
          }
        }
      } else {
#pragma unroll
        for (int s = 0; s < NSLOT; ++s) {
          const int r = wave_r0 + 4 * s + lg;
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            const int key = key0 + 16 * st + n;
            if (r < row_end && key <= r - seq_off) scores[(size_t)(r - out_row0) * ld + key] = part[st][s];
          }
        }
      }
    }
    if (it + 1 < ntiles) wait_tile();
    __syncthreads();
  }
  if (MODE == 2 && ns > 0) flush();
  if (MODE == 1 && wave_r0 < row_end && wave_r0 - seq_off + 1 > topk) {
    // the token's sample scores leave in one coalesced burst
    float* dst_row = reinterpret_cast<float*>(cand + (size_t)(wave_r0 - out_row0) * kTopkCandCap);
    for (int i = lane; i < kend - kbeg; i += 64) dst_row[kbeg + i] = smp_stage[i];
  }
  if (MODE == 1 && split == 0 && lane == 0) {
#pragma unroll
    for (int s = 0; s < NSLOT; ++s) {
      const int r = wave_r0 + s;
      if (r < row_end && r - seq_off + 1 > topk) tau_lo[r - out_row0] = (uint32_t)m;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Decode: one query token per sequence against its cached keys; HBM-bound (64 flop per key
// byte at 64 heads x 128 dims).  The 4 waves of a workgroup share each 64-key tile (a
// full tile DMA'd global->LDS, every load instruction one contiguous KiB) and split the heads:
// wave w scores heads w*H/4 .. w*H/4 + H/4 - 1 (one 16-row MFMA tile, rows past H/4 zero),
// reduces them to one partial per key, and the four partials meet in LDS.  With NT > 2 tiles a
// 3-deep ring keeps two tiles in flight while one is scored; the only vector-memory operations
// inside the loop are the tile loads, so the wait for the next tile can name it exactly.  Scores
// collect in LDS and leave in one burst at the end.  A workgroup covers KPW = 64 * NT keys of
// one sequence.
template <int H, int DI, int NT>
__global__ __launch_bounds__(256) void indexer_decode_coop_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, const uint16_t* __restrict__ k_cache,
    const int* __restrict__ seq_lens, int s_max, float* __restrict__ scores, long long ld, int nsplit) {
  constexpr int NKS = DI / 32;
  constexpr int PITCH = DI * 2;
  constexpr int CPR = DI / 8;
  constexpr int NLD = 64 * CPR / 256;  // 16-byte DMA pieces per thread per tile
  constexpr int HW = H / 4;            // heads per wave
  constexpr int KPW = 64 * NT;
  constexpr int NB = NT < 3 ? NT : 3;  // tile buffers: all tiles when there are fewer than 3
  static_assert(H == 4 || H == 16 || H == 32 || H == 64, "unsupported indexer head count");
  __shared__ __attribute__((aligned(16))) unsigned char tiles[NB][64 * PITCH];
  __shared__ float part[2][4][64];
  __shared__ float sc[KPW];
  const int b = blockIdx.x / nsplit;
  const int split = blockIdx.x - b * nsplit;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, lg = lane >> 4;
  const int len = min(seq_lens[b], s_max);  // defensive: never read past the cache
  const int kbeg = split * KPW;
  if (kbeg >= len) return;                  // uniform over the workgroup
  const int kend = min(kbeg + KPW, len);
  const int ntiles = (kend - kbeg + 63) >> 6;

  // A operand: row n of the wave's tile is head wave*HW + n (zero past HW).
  u32x4 areg[NKS];
  {
    const uint16_t* qp = q_idx + ((size_t)b * H + wave * HW + (n < HW ? n : 0)) * DI + lg * NKS * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) areg[ks] = (n < HW) ? ldg16(qp + ks * 8) : u32x4{0, 0, 0, 0};
  }
  float wreg[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * lg + i;
    wreg[i] = (m < HW) ? w[(size_t)b * H + wave * HW + m] : 0.f;
  }

  // Tile staging as in the prefill kernel: instruction p of wave w fills LDS bytes
  // [p*4096 + w*1024, +1024) of the tile; the row's piece (l % CPR) ^ tile_swizzle(r) lands at slot l % CPR.
  const uint16_t* kseq = k_cache + ((size_t)b * s_max + kbeg) * DI;
  int st_row[NLD], st_off[NLD];
#pragma unroll
  for (int p = 0; p < NLD; ++p) {
    const int pos = p * 4096 + wave * 1024 + lane * 16;
    const int r = pos / PITCH;
    const int chunk = (lane % CPR) ^ tile_swizzle<CPR>(r);
    st_row[p] = r;
    st_off[p] = chunk * 8;
  }
  auto load_tile = [&](int tile, int buf) {
    const int keys_left = kend - kbeg - tile * 64;
#pragma unroll
    for (int p = 0; p < NLD; ++p) {
      const int r = min(st_row[p], keys_left - 1);
      lds_dma16(kseq + ((size_t)tile * 64 + r) * DI + st_off[p], &tiles[buf][p * 4096 + wave * 1024]);
    }
  };

  load_tile(0, 0);
  if (NB > 1 && ntiles > 1) load_tile(1, 1);
  int cur = 0;
  for (int it = 0; it < ntiles; ++it) {
    // Tile `it` must have landed for every wave: own loads, then the barrier.
    if (it + 1 < ntiles) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NLD) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    // Sum the previous tile's four partials (written before the barrier just passed).
    if (it > 0 && wave == ((it - 1) & 3)) {
      const float* pp = part[(it - 1) & 1][0];
      sc[(it - 1) * 64 + lane] = pp[lane] + pp[64 + lane] + pp[128 + lane] + pp[192 + lane];
    }
    // The buffer of tile it+2 was last read while scoring tile it-1, before that barrier.
    if (NB == 3 && it + 2 < ntiles) load_tile(it + 2, cur == 0 ? 2 : cur - 1);
    const unsigned char* tile = tiles[cur];
    float pst[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const unsigned char* bp = tile + (16 * st + n) * PITCH;
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const u32x4 bq = *reinterpret_cast<const u32x4*>(bp + (((lg * NKS + ks) ^ tile_swizzle<CPR>(n)) * 16));
        c = mfma16x16x32(areg[ks], bq, c);
      }
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = fmaf(relu(c[i]), wreg[i], acc);
      pst[st] = acc;
    }
    part[it & 1][wave][lane] = transpose_reduce4(pst[0], pst[1], pst[2], pst[3]);
    cur = (cur == NB - 1) ? 0 : cur + 1;
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  if (wave == ((ntiles - 1) & 3)) {
    const float* pp = part[(ntiles - 1) & 1][0];
    sc[(ntiles - 1) * 64 + lane] = pp[lane] + pp[64 + lane] + pp[128 + lane] + pp[192 + lane];
  }
  __syncthreads();
  float* dst = scores + (size_t)b * ld + kbeg;
  for (int i = threadIdx.x; i < kend - kbeg; i += 256) dst[i] = sc[i];
}

}  // namespace

// ---------------------------------------------------------------------------------------
// Host launchers.

template <int H, int DI, int RT, int MODE>
static hipError_t launch_prefill_t(const IndexerPrefillArgs& a, const TopkScratch* t, int k, hipStream_t s,
                                   const uint32_t* only_rows = nullptr) {
  constexpr int TOKWG = 4 * ((H >= 16) ? 16 * RT / H : 4 * RT);
  const int rows = a.row_end - a.row_begin;
  const int n_rowblk = (rows + TOKWG - 1) / TOKWG;
  const int t_max = a.row_end - 1 - a.seq_off;
  const int n_split = MODE == 1 ? kSampleSplits : (t_max + a.key_split) / a.key_split;
  long long n = (long long)n_rowblk * n_split;
  n = (n + 7) / 8 * 8;
  hipLaunchKernelGGL((indexer_prefill_kernel<H, DI, RT, MODE>), dim3((unsigned)n), dim3(256), 0, s, a.q_idx, a.k_idx,
                     a.w, a.seq_off, a.row_begin, a.row_end, a.out_row0, a.scores, a.ld, a.key_split, n_rowblk,
                     t ? t->tau_lo : nullptr, t ? t->cnt : nullptr, t ? t->cand : nullptr, k, only_rows);
  return hipGetLastError();
}

hipError_t launch_indexer_prefill(const IndexerPrefillArgs& a, hipStream_t s) {
  if (a.h_idx == 64 && a.d_idx == 128) return launch_prefill_t<64, 128, 4, 0>(a, nullptr, 0, s);
  if (a.h_idx == 32 && a.d_idx == 128) return launch_prefill_t<32, 128, 4, 0>(a, nullptr, 0, s);
  if (a.h_idx == 16 && a.d_idx == 128) return launch_prefill_t<16, 128, 4, 0>(a, nullptr, 0, s);
  if (a.h_idx == 4 && a.d_idx == 64) return launch_prefill_t<4, 64, 4, 0>(a, nullptr, 0, s);
  return hipErrorInvalidValue;
}

bool indexer_emit_supported(int h_idx, int d_idx) { return h_idx == 64 && d_idx == 128; }

hipError_t launch_indexer_prefill_sample(const IndexerPrefillArgs& a, const TopkScratch& t, int k, hipStream_t s) {
  if (!indexer_emit_supported(a.h_idx, a.d_idx)) return hipErrorInvalidValue;
  return launch_prefill_t<64, 128, 4, 1>(a, &t, k, s);
}

hipError_t launch_indexer_prefill_emit(const IndexerPrefillArgs& a, const TopkScratch& t, int k, hipStream_t s) {
  if (!indexer_emit_supported(a.h_idx, a.d_idx)) return hipErrorInvalidValue;
  return launch_prefill_t<64, 128, 4, 2>(a, &t, k, s);
}

hipError_t launch_indexer_prefill_rescore(const IndexerPrefillArgs& a, const TopkScratch& t, hipStream_t s) {
  if (!indexer_emit_supported(a.h_idx, a.d_idx)) return hipErrorInvalidValue;
  return launch_prefill_t<64, 128, 4, 0>(a, nullptr, 0, s, t.fail);
}

// Keys per decode workgroup: 2 tiles of 64, both loaded at once (short workgroups, four per CU,
// kept 6.0 TB/s streaming in measurement against 5.7 TB/s for 8 tiles through the 3-deep ring).
constexpr int kDecodeTiles = 2;

template <int H, int DI>
static hipError_t launch_decode_t(const IndexerDecodeArgs& a, hipStream_t s) {
  constexpr int kpw = 64 * kDecodeTiles;
  const int nsplit = (a.max_len + kpw - 1) / kpw;
  hipLaunchKernelGGL((indexer_decode_coop_kernel<H, DI, kDecodeTiles>), dim3((unsigned)(a.batch * nsplit)), dim3(256),
                     0, s, a.q_idx, a.w, a.k_cache, a.seq_lens, a.s_max, a.scores, a.ld, nsplit);
  return hipGetLastError();
}

hipError_t launch_indexer_decode(const IndexerDecodeArgs& a, hipStream_t s) {
  if (a.h_idx == 64 && a.d_idx == 128) return launch_decode_t<64, 128>(a, s);
  if (a.h_idx == 32 && a.d_idx == 128) return launch_decode_t<32, 128>(a, s);
  if (a.h_idx == 16 && a.d_idx == 128) return launch_decode_t<16, 128>(a, s);
  if (a.h_idx == 4 && a.d_idx == 64) return launch_decode_t<4, 64>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace dsa

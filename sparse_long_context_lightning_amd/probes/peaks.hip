// Achievable-peak probes: what the device reaches on the resources the path's kernels are priced
// against, measured with the same toolchain and launch style as those kernels.  They compute
// nothing of the method and are built into their own library (libdsa_probes.so, include/dsa_probes.h);
// the benchmark reads the path's kernels against them beside the spec peaks.
#include <stdarg.h>
#include <stdio.h>

#include "../../include/dsa_probes.h"
#include "../csrc/common.h"

namespace dsa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kChains = 8;  // independent accumulation chains per wave

// MFMA only: kChains independent 16x16x32 bf16 chains per wave (the prefill indexer's
// instruction), operands in registers.  The final compare keeps the loop live; with seed 0 the
// operands are zero and nothing is stored.
__global__ __launch_bounds__(256) void mfma_loop16_kernel(int iters, unsigned seed, float* sink) {
  const u32x4 a = {seed ^ threadIdx.x, seed, seed, seed};
  const u32x4 b = {seed, seed ^ threadIdx.x, seed, seed};
  f32x4 c[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int j = 0; j < kChains; ++j) c[j] = mfma16x16x32(a, b, c[j]);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
  if (s == 1.0e30f) sink[blockIdx.x] = s;
}

// The same with 32x32x16 bf16 (four chains: 16 accumulators each).
__global__ __launch_bounds__(256) void mfma_loop32_kernel(int iters, unsigned seed, float* sink) {
  const u32x4 a = {seed ^ threadIdx.x, seed, seed, seed};
  const u32x4 b = {seed, seed ^ threadIdx.x, seed, seed};
  f32x16 c[kChains / 2];
#pragma unroll
  for (int j = 0; j < kChains / 2; ++j) c[j] = f32x16{};
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int j = 0; j < kChains / 2; ++j)
      c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                     c[j], 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains / 2; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c[j][e];
  if (s == 1.0e30f) sink[blockIdx.x] = s;
}

// Streaming read: each thread reads 16-byte pieces, eight in flight, grid-stride over the
// buffer, and folds them into one word (stored only if it matches a value the caller never
// produces, so the loads stay live).
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, long long n16,
                                                          unsigned never, unsigned* sink) {
  const long long stride = (long long)gridDim.x * 256;
  long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = src[i + j * stride];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= v[j];
  }
  for (; i < n16; i += stride) acc ^= src[i];
  const unsigned r = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (r == never) sink[blockIdx.x] = r;
}

// Gather: the sparse attention's memory traffic with nothing else.  One wave per (row, KV
// group, split) in the attention kernels' work orders; per chunk of 32 index entries the wave
// reads the 32 key rows and 32 value rows with 16 loads of 16 bytes per lane, DEPTH chunks in
// flight, and folds the data into one word.  Load shape 0 (the per-row attention kernel's): lane
// (n, q) reads 64 contiguous bytes of entries n and 16 + n, four 16-byte pieces, so one
// instruction touches 16 rows; shape 1 (whole rows): the 16 lanes of a lane group read one
// 256-byte row, so one instruction covers four whole rows.
template <int DEPTH, int SHAPE>
__global__ __launch_bounds__(256) void gather_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                     long long n_pos, const int* __restrict__ idx, int k_sel, int rows,
                                                     int hkv, int nsplit, long long row_stride, int group_fastest,
                                                     unsigned never, unsigned* sink) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, lg = lane >> 4;
  const long long n_items = (long long)rows * hkv * nsplit;
  const long long n_wg = (n_items + 3) / 4;
  // XCD x (workgroups reach the 8 XCDs round-robin) takes the x-th eighth of the items.
  const long long wg = (long long)(blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  if (wg >= n_wg) return;
  const long long item = wg * 4 + wave;
  if (item >= n_items) return;
  int g, sp, row;
  if (group_fastest) {
    g = (int)(item % hkv);
    const long long t = item / hkv;
    sp = (int)(t % nsplit);
    row = (int)(t / nsplit);
  } else {
    const long long per_group = (long long)rows * nsplit;
    g = (int)(item / per_group);
    const long long t = item - (long long)g * per_group;
    sp = (int)(t % nsplit);
    row = (int)(t / nsplit);
  }
  const int nchunk = (k_sel + 31) >> 5;
  const int cps = (nchunk + nsplit - 1) / nsplit;
  const int c_begin = sp * cps;
  const int c_end = min(nchunk, c_begin + cps);
  const int* idx_row = idx + (long long)row * k_sel;
  const long long base = (long long)row * row_stride;
  const size_t pos_stride = (size_t)hkv * 128;
  const uint16_t* kb = k + (size_t)g * 128 + (SHAPE == 0 ? lg * 32 : n * 8);
  const uint16_t* vb = v + (size_t)g * 128 + (SHAPE == 0 ? lg * 32 : n * 8);
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int c0 = c_begin; c0 < c_end; c0 += DEPTH) {
    u32x4 buf[DEPTH][2][8];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      if (SHAPE == 0) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int s = (c0 + d) * 32 + 16 * j + n;
          int p = (c0 + d < c_end && s < k_sel) ? idx_row[s] : -1;
          long long pos = p >= 0 ? base + p : 0;
          pos = pos < n_pos ? pos : 0;
          const uint16_t* kp = kb + (size_t)pos * pos_stride;
          const uint16_t* vp = vb + (size_t)pos * pos_stride;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            buf[d][j][q] = ldg16(kp + q * 8);
            buf[d][j][4 + q] = ldg16(vp + q * 8);
          }
        }
      } else {
        // instruction j reads entries 4 j + lg whole (lane n: bytes 16 n .. 16 n + 15)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int s = (c0 + d) * 32 + 4 * j + lg;
          int p = (c0 + d < c_end && s < k_sel) ? idx_row[s] : -1;
          long long pos = p >= 0 ? base + p : 0;
          pos = pos < n_pos ? pos : 0;
          buf[d][j >> 2][j & 3] = ldg16(kb + (size_t)pos * pos_stride);
          buf[d][j >> 2][4 + (j & 3)] = ldg16(vb + (size_t)pos * pos_stride);
        }
      }
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc ^= buf[d][j][q];
  }
  const unsigned r = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (r == never) sink[blockIdx.x] = r;
}

// Float-atomic throughput: each instruction adds 1.0 at 64 addresses lying in 64 / W rows of 128
// floats with W consecutive floats in each (W = 64: one row piece, as the per-row attention
// backward scatters dk / dv; W = 16: four rows, as the merged-set backward does).  Rows are drawn
// from [0, n_rows) by a per-wave (and per row piece) LCG; every address stays in its row.
template <int W>
__global__ __launch_bounds__(256) void atomic_add_kernel(float* __restrict__ buf, long long n_rows, int iters) {
  const int lane = threadIdx.x & 63;
  const unsigned wave = blockIdx.x * 4u + (threadIdx.x >> 6);
  const int grp = lane / W, off = lane % W;
  unsigned s = (wave * 2654435761u) ^ ((unsigned)grp * 40503u) ^ 0x9E3779B9u;
  for (int i = 0; i < iters; ++i) {
    s = s * 1664525u + 1013904223u;
    const long long r = (long long)(((unsigned long long)s * (unsigned long long)n_rows) >> 32);
    unsafeAtomicAdd(buf + r * 128 + (i % (128 / W)) * W + off, 1.0f);
  }
}

thread_local char g_probe_error[256] = "";

int probe_fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_probe_error, sizeof(g_probe_error), fmt, ap);
  va_end(ap);
  return status;
}

int launched(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return DSA_PROBE_OK;
  return probe_fail(DSA_PROBE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace
}  // namespace dsa

using namespace dsa;

extern "C" {

const char* dsa_probe_last_error(void) { return g_probe_error; }

int dsa_probe_mfma_bf16(int shape, int grid, int iters, float* sink, long long* flops, void* stream) {
  g_probe_error[0] = 0;
  if (shape != 16 && shape != 32) return probe_fail(DSA_PROBE_ERR_INVALID_ARG, "shape must be 16 or 32, got %d", shape);
  if (grid < 1 || grid > (1 << 20) || iters < 1) return probe_fail(DSA_PROBE_ERR_INVALID_ARG, "grid / iters out of range");
  if (!sink) return probe_fail(DSA_PROBE_ERR_INVALID_ARG, "sink is null");
  // per wave and iteration: kChains 16x16x32 (16384 flop) or kChains / 2 32x32x16 (32768 flop)
  const long long per =
      shape == 16 ? (long long)kChains * 16 * 16 * 32 * 2 : (long long)(kChains / 2) * 32 * 32 * 16 * 2;
  if (flops) *flops = (long long)grid * 4 * iters * per;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (shape == 16)
    hipLaunchKernelGGL(mfma_loop16_kernel, dim3(grid), dim3(256), 0, s, iters, 0u, sink);
  else
    hipLaunchKernelGGL(mfma_loop32_kernel, dim3(grid), dim3(256), 0, s, iters, 0u, sink);
  return launched("MFMA probe launch");
}

int dsa_probe_stream_read(const void* src, size_t bytes, int grid, uint32_t* sink, void* stream) {
  g_probe_error[0] = 0;
  if (!src || !sink) return probe_fail(DSA_PROBE_ERR_INVALID_ARG, "pointers must not be null");
  if ((reinterpret_cast<uintptr_t>(src) & 15u) != 0 || bytes % 16 != 0 || bytes == 0)
    return probe_fail(DSA_PROBE_ERR_INVALID_ARG, "source must be 16-byte aligned with a positive multiple of 16 bytes");
  if (grid < 1 || grid > (1 << 20)) return probe_fail(DSA_PROBE_ERR_INVALID_ARG, "grid out of range");
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     reinterpret_cast<const u32x4*>(src), (long long)(bytes / 16), 0xFFFFFFFFu, sink);
  return launched("stream-read probe launch");
}

int dsa_probe_gather(const void* k, const void* v, int64_t n_pos, int hkv, const int32_t* idx, int k_sel, int rows,
                     int nsplit, int64_t row_stride, int group_fastest, int depth, int whole_rows, uint32_t* sink,
                     int64_t sink_len, void* stream) {
  g_probe_error[0] = 0;
  if (!k || !v || !idx || !sink) return probe_fail(DSA_PROBE_ERR_INVALID_ARG, "pointers must not be null");
  if (((reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v)) & 15u) != 0)
    return probe_fail(DSA_PROBE_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
  if (n_pos < 1 || hkv < 1 || k_sel < 1 || rows < 1 || nsplit < 1 || row_stride < 0)
    return probe_fail(DSA_PROBE_ERR_INVALID_ARG, "sizes must be positive (row_stride non-negative)");
  if (depth != 1 && depth != 2 && depth != 4) return probe_fail(DSA_PROBE_ERR_INVALID_ARG, "depth must be 1, 2 or 4");
  const long long items = (long long)rows * hkv * nsplit;
  const long long n_wg = (items + 3) / 4;
  const long long grid = (n_wg + 7) / 8 * 8;
  if (grid > (1LL << 31) - 1) return probe_fail(DSA_PROBE_ERR_INVALID_ARG, "too many items");
  if (sink_len < grid) return probe_fail(DSA_PROBE_ERR_INVALID_ARG, "sink holds %lld entries, %lld needed",
                                         (long long)sink_len, grid);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, s, kk, vv, (long long)n_pos, idx, k_sel, rows, hkv,
                       nsplit, (long long)row_stride, group_fastest, 0xFFFFFFFFu, sink);
  };
  if (whole_rows) {
    if (depth == 1) go(gather_kernel<1, 1>);
    else if (depth == 2) go(gather_kernel<2, 1>);
    else go(gather_kernel<4, 1>);
  } else {
    if (depth == 1) go(gather_kernel<1, 0>);
    else if (depth == 2) go(gather_kernel<2, 0>);
    else go(gather_kernel<4, 0>);
  }
  return launched("gather probe launch");
}

int dsa_probe_atomic_add(float* buf, int64_t n_rows, int floats_per_row, int grid, int iters, long long* adds,
                         void* stream) {
  g_probe_error[0] = 0;
  if (!buf) return probe_fail(DSA_PROBE_ERR_INVALID_ARG, "buf is null");
  if (n_rows < 1 || n_rows > (1LL << 32)) return probe_fail(DSA_PROBE_ERR_INVALID_ARG, "n_rows out of range");
  if (floats_per_row != 16 && floats_per_row != 64)
    return probe_fail(DSA_PROBE_ERR_INVALID_ARG, "floats_per_row must be 16 or 64, got %d", floats_per_row);
  if (grid < 1 || grid > (1 << 20) || iters < 1) return probe_fail(DSA_PROBE_ERR_INVALID_ARG, "grid / iters out of range");
  if (adds) *adds = (long long)grid * 4 * iters * 64;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (floats_per_row == 16)
    hipLaunchKernelGGL(atomic_add_kernel<16>, dim3(grid), dim3(256), 0, s, buf, (long long)n_rows, iters);
  else
    hipLaunchKernelGGL(atomic_add_kernel<64>, dim3(grid), dim3(256), 0, s, buf, (long long)n_rows, iters);
  return launched("atomic-add probe launch");
}

}  // extern "C"

// Achievable-peak probes: what the box reaches on the two resources the path is priced
// against, measured with the same toolchain and launch style as the path's kernels.  They
// compute nothing of the method; the benchmark reports the path's kernels against them beside
// the spec peaks.
#include "common.h"
#include "kernels.h"

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

}  // namespace

hipError_t launch_peak_mfma(int shape, int grid, int iters, float* sink, hipStream_t s) {
  if (shape == 16)
    hipLaunchKernelGGL(mfma_loop16_kernel, dim3(grid), dim3(256), 0, s, iters, 0u, sink);
  else
    hipLaunchKernelGGL(mfma_loop32_kernel, dim3(grid), dim3(256), 0, s, iters, 0u, sink);
  return hipGetLastError();
}

long long peak_mfma_flops(int shape, int grid, int iters) {
  // per wave and iteration: kChains 16x16x32 (16384 flop) or kChains / 2 32x32x16 (32768 flop)
  const long long per = shape == 16 ? (long long)kChains * 16 * 16 * 32 * 2 : (long long)(kChains / 2) * 32 * 32 * 16 * 2;
  return (long long)grid * 4 * iters * per;
}

hipError_t launch_peak_stream_read(const void* src, long long bytes, int grid, unsigned* sink, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, s, reinterpret_cast<const u32x4*>(src), bytes / 16,
                     0xFFFFFFFFu, sink);
  return hipGetLastError();
}

}  // namespace dsa

// Shared device helpers for the gfx950 kernels of the DSA path (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kHeadDim = 128;
constexpr int kMaxTopK = 2048;

// 16x16x32 bf16 MFMA (CDNA4).  Lane l supplies A[l % 16][8 * (l / 16) + e] and
// B[8 * (l / 16) + e][l % 16] for e = 0..7 and receives C[4 * (l / 16) + i][l % 16], i = 0..3.
// Only the pairing "element e of A in lane l meets element e of B in lane l" matters for
// the contraction, so callers are free to permute which reduction index a slot carries, as
// long as both operands use the same permutation.
__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Round-to-nearest-even fp32 -> bf16 of two values packed into one dword (lo = a, hi = b).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
  ua = (ua + 0x7FFFu + ((ua >> 16) & 1u)) >> 16;
  ub = (ub + 0x7FFFu + ((ub >> 16) & 1u)) >> 16;
  return ua | (ub << 16);
}

// fp32 rounded to the nearest bf16 value (ties to even), returned as fp32.
__device__ __forceinline__ float round_bf16(float a) {
  uint32_t u = __float_as_uint(a);
  u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
  return __uint_as_float(u);
}

// max(x, 0) as one integer max on the bit pattern: negative floats (and -0) are negative
// int32 values, non-negative floats pass through unchanged.  Avoids the NaN-quieting
// canonicalisation an IEEE-mode fmaxf carries.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Order-preserving map float -> uint32 (larger float -> larger key).  -0.0 is folded into
// +0.0 first so the two compare equal.
__device__ __forceinline__ uint32_t float_key(float x) {
  uint32_t u = __float_as_uint(x);
  u = (u == 0x80000000u) ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// Wait for this wave's outstanding LDS operations and keep the compiler from moving memory
// accesses across the point: used where lanes of one wave exchange data through LDS.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Direct global -> LDS copy of 16 bytes per lane: lane l's bytes land at lds_wave_base + 16 l
// (lds_wave_base must be the same for the whole wave).  Completion is tracked by vmcnt.
__device__ __forceinline__ void lds_dma16(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, lds_wave_base, 16, 0, 0);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Two fp32 values to one dword of bf16 (round to nearest even, lo = a): v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// 256-byte rows staged in LDS with 16-byte piece c of row r at slot c ^ swz(r), where for
// r mod 16 = 4a + b, swz = (b << 1) | (a >> 1) | ((a & 1) << 3).  It is a permutation of 0..15,
// so the 16 rows one row-wise MFMA operand read touches hit 16 distinct slots, and the
// transposed reads (rows 4a + 0..3, two neighbouring pieces, two lane groups a) do as well.
__device__ __forceinline__ int swz(int r) {
  const int a = (r >> 2) & 3, b = r & 3;
  return (b << 1) | (a >> 1) | ((a & 1) << 3);
}

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i % 4 of the 8-byte
// words that lanes i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4 address (in that order).
__device__ __forceinline__ uint2 lds_read_tr16(const unsigned char* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  return __builtin_bit_cast(uint2, v);
}

// s_waitcnt vmcnt(N) through the builtin, so the compiler's own wait-count bookkeeping sees it
// (after vmcnt(0) it knows its earlier loads have landed and adds no wait of its own for them).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  // vmcnt bits [3:0] and [15:14]; the lgkmcnt and expcnt fields at their maximum (no wait).
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
}
// Wait until at most n of this wave's vector-memory operations are outstanding (the largest
// listed immediate <= n is used, which only ever waits longer).
__device__ __forceinline__ void vm_wait_at_most(int n) {
  if (n >= 32) vm_wait<32>();
  else if (n >= 24) vm_wait<24>();
  else if (n >= 20) vm_wait<20>();
  else if (n >= 18) vm_wait<18>();
  else if (n >= 16) vm_wait<16>();
  else if (n >= 15) vm_wait<15>();
  else if (n >= 12) vm_wait<12>();
  else if (n >= 10) vm_wait<10>();
  else if (n >= 9) vm_wait<9>();
  else if (n >= 8) vm_wait<8>();
  else if (n >= 6) vm_wait<6>();
  else if (n >= 5) vm_wait<5>();
  else if (n >= 4) vm_wait<4>();
  else if (n >= 3) vm_wait<3>();
  else if (n >= 2) vm_wait<2>();
  else if (n >= 1) vm_wait<1>();
  else vm_wait<0>();
}
// Barrier of a staging ring: this wave's LDS operations done, every wave past the point.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
}

// The same copies issued from inline assembly, which the compiler does not track.  Its
// wait-count pass cannot tell which LDS bytes a tracked copy writes, so before an LDS read that
// might overlap (any transposed read, for one) it waits for every copy in flight, including the
// ring stages issued ahead of the read.  With these forms the caller alone orders the copies and
// its LDS reads, with s_waitcnt vmcnt and a barrier.  M0 carries the LDS base (wave-uniform).
// M0 is listed as clobbered (the compiler reserves it and warns; it sets M0 itself right before
// each instruction of its own that reads it).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ uint32_t lds_offset(const void* lds_ptr) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_ptr;
}
__device__ __forceinline__ void lds_dma16_untracked(const void* g, void* lds_wave_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_offset(lds_wave_base));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(base) : "memory", "m0");
}
// Scalar-base form: the wave-uniform 64-bit base in SGPRs, a 32-bit per-lane byte offset, and
// the LDS destination (wave-uniform) already in an SGPR, so no vector address arithmetic runs.
__device__ __forceinline__ void lds_dma16_saddr(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_base)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4_untracked(const void* g, void* lds_wave_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_offset(lds_wave_base));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(base) : "memory", "m0");
}
#pragma clang diagnostic pop

}  // namespace dsa

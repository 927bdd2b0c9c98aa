// dsa_decode without a caller workspace, for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The decode
// step's scratch (indexer scores, top-k candidate lists, split-attention partials) lives in one
// file-scope device array per GPU, sized once at compile time; nothing is allocated or freed.
#include <mutex>

#include "../../include/dsa.h"
#include "kernels.h"

namespace {

// Each device holds its own copy of this array until the process ends.  Host code never uses
// the name as an address (on the host it is only a stand-in): the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) unsigned char scratch[DSA_DECODE_NOALLOC_MAX_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch; looked up on the first call on that device.
int current_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return dsa::api_fail(DSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return dsa::api_fail(DSA_ERR_UNSUPPORTED, "device %d is beyond the %d devices the static scratch serves", dev,
                         kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return dsa::api_fail(DSA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

}  // namespace

extern "C" int dsa_decode_noalloc(const void* q, const void* q_idx, const float* w, const void* k_cache,
                                  const void* v_cache, const void* k_idx_cache, const int32_t* seq_lens, int batch,
                                  int s_max, int max_seq_len, int hq, int hkv, int head_dim, int h_idx, int d_idx,
                                  int top_k, float softmax_scale, void* out, float* lse, int32_t* idx_out,
                                  void* stream) {
  dsa::api_clear_error();
  const dsa::ApiRange range_("dsa_decode_noalloc");
  dsa::api_log("dsa_decode_noalloc", "batch=%d s_max=%d max_seq_len=%d hq=%d hkv=%d h_idx=%d d_idx=%d top_k=%d",
               batch, s_max, max_seq_len, hq, hkv, h_idx, d_idx, top_k);
  size_t need = 0;
  const int st = dsa_decode_workspace_size(batch, s_max, hq, hkv, head_dim, h_idx, d_idx, top_k, &need);
  if (st != DSA_OK) return st;
  if (need > (size_t)DSA_DECODE_NOALLOC_MAX_BYTES)
    return dsa::api_fail(DSA_ERR_WORKSPACE,
                         "this decode step needs %zu bytes of scratch; the static scratch holds %zu (use dsa_decode "
                         "with a caller workspace)",
                         need, (size_t)DSA_DECODE_NOALLOC_MAX_BYTES);
  void* ws = nullptr;
  const int st2 = current_scratch(&ws);
  if (st2 != DSA_OK) return st2;
  // The decode kernels clear what they count (the top-k candidate counters) themselves, so the
  // scratch left by an earlier call needs no reset.
  return dsa_decode(q, q_idx, w, k_cache, v_cache, k_idx_cache, seq_lens, batch, s_max, max_seq_len, hq, hkv,
                    head_dim, h_idx, d_idx, top_k, softmax_scale, out, lse, idx_out, ws,
                    (size_t)DSA_DECODE_NOALLOC_MAX_BYTES, stream);
}

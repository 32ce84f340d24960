// hs2_decode_step_noalloc: the decode step of hs2_decode_step with its
// workspace in a device array that the library holds, for callers that cannot
// allocate device memory themselves.
#include <mutex>

#include "hs2_internal.h"
#include "validate.h"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;  // 32 MiB per GPU

// The step's workspace.  In host code `scratch` names a host-side stand-in,
// not the device memory: kernels get the address from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's `scratch`, looked up once per device
// (with that device current) and kept.
hs2_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HS2_EHIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return HS2_EHIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return HS2_OK;
}

}  // namespace

extern "C" {

hs2_status hs2_decode_step_noalloc(const hs2_attn_desc* desc, const void* q, const void* q_sparse,
                                   const void* k, const void* v, int64_t kv_stride,
                                   const int32_t* ctx_len, int kv_capacity, float* scores,
                                   float* lse_full, int32_t* top_idx, int32_t* top_cnt, float* o,
                                   float* lse, hs2_stream_t stream) {
  // Every argument is checked before the runtime is asked for anything.
  hs2_status s = hs2::validate_step_noalloc(desc, q, q_sparse, k, v, kv_stride, ctx_len,
                                            kv_capacity, scores, lse_full, top_idx, top_cnt, o,
                                            lse, kScratchBytes);
  if (s != HS2_OK) return s;
  const size_t need = hs2_workspace_size(desc, kv_capacity);
  void* ws = nullptr;
  if ((s = scratch_address(&ws)) != HS2_OK) return s;
  return hs2_decode_step(desc, q, q_sparse, k, v, kv_stride, ctx_len, kv_capacity, scores,
                         lse_full, top_idx, top_cnt, o, lse, ws, need, stream);
}

}  // extern "C"

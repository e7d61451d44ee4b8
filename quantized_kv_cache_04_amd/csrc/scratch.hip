// kvq_decode_attention_scratch: the decode step of kvq_decode_attention
// with its split-K partial softmax states in a static device array of the
// library instead of the workspace region of the caller's cache allocation.
// For callers that cannot allocate device memory at all (code under HIP
// graph capture, serving loops that forbid allocation): the call allocates
// nothing, and neither does anything it launches.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kvq_internal.h"

namespace kvq {
namespace {

// Partial states (o, m, l) of the splits: [B][Hq][S][d + 2] float32.  Each
// GPU the library runs on holds its own copy until the process ends.
constexpr uint64_t kScratchBytes = KVQ_DECODE_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
float* g_ptr[kMaxDevices] = {};   // device address of ``scratch`` per device

// Device address of this device's copy of ``scratch``, looked up once per
// device with that device current.  (In host code the array's name is only
// a host-side handle: it must never reach a kernel.)
kvq_status scratch_ptr(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return set_error(KVQ_ERR_DEVICE, "kvq_decode_attention_scratch: no current HIP device");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(KVQ_ERR_DEVICE,
                       "kvq_decode_attention_scratch: hipGetSymbolAddress of the scratch "
                       "array failed");
    g_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_ptr[dev];
  return KVQ_OK;
}

}  // namespace
}  // namespace kvq

extern "C" kvq_status kvq_decode_attention_scratch(const kvq_config* cfg, const kvq_cache* cache,
                                                   const void* q, const int32_t* q_pos,
                                                   float sm_scale, void* out, int32_t out_dtype,
                                                   void* stream) {
  float* ws = nullptr;
  kvq_status st = kvq::scratch_ptr(&ws);
  if (st != KVQ_OK) return st;
  // every partial slot the combine reads is written by this call's
  // streaming kernels first: nothing in the array needs clearing
  return kvq::decode_attention_impl(cfg, cache, q, q_pos, sm_scale, out, out_dtype, stream, ws,
                                    kvq::kScratchBytes);
}

// Split-K (flash-decoding) state merge shared by the decode kernels.
//
// Every workgroup handles a token range of one (sequence, KV head) and
// leaves, per query head, an unnormalized partial (o, m, l): the running
// maximum m of the base-2 scores, l = sum 2^(s - m) and o = sum 2^(s - m) v.
// The last workgroup of a (sequence, KV head) to finish -- found with an
// agent-scope atomic counter that it resets afterwards -- merges the
// partials with log-sum-exp weights and writes the output, so a decode step
// is a single launch.
#pragma once

#include "device_common.h"

namespace kvq {

__device__ __forceinline__ float* partial_rec(const DecodeArgs& a, int b, int j, int s) {
  return a.partial + (((int64_t)b * a.sh.Hq + j) * a.S_max + s) * (kHeadDim + 2);
}

__device__ __forceinline__ void store_out(const DecodeArgs& a, int64_t idx, float v) {
  if (a.out_dtype == KVQ_F32)
    static_cast<float*>(a.out)[idx] = v;
  else if (a.out_dtype == KVQ_F16)
    static_cast<uint16_t*>(a.out)[idx] = f2h_rn(v);
  else
    static_cast<uint16_t*>(a.out)[idx] = f2bf_rn(v);
}

// Called by all threads of the block after it has written its partials for
// every query head of (b, h).  ``flag`` is a block-shared int.
__device__ __forceinline__ void splitk_finish(const DecodeArgs& a, int b, int h, int* flag) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(&a.counters[b * a.sh.Hkv + h], 1u,
                                                __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    *flag = (old == (uint32_t)(a.splits - 1));
  }
  __syncthreads();
  if (!*flag) return;
  __threadfence();
  const int g = a.sh.g;
  for (int idx = threadIdx.x; idx < g * kHeadDim; idx += blockDim.x) {
    const int jj = idx / kHeadDim, c = idx % kHeadDim;
    const int j = h * g + jj;
    float M = -INFINITY;
    for (int s = 0; s < a.splits; ++s) M = fmaxf(M, partial_rec(a, b, j, s)[kHeadDim]);
    float L = 0.0f, O = 0.0f;
    if (M > -INFINITY) {
      for (int s = 0; s < a.splits; ++s) {
        const float* p = partial_rec(a, b, j, s);
        const float w = exp2f(p[kHeadDim] - M);
        L += w * p[kHeadDim + 1];
        O += w * p[c];
      }
    }
    store_out(a, ((int64_t)b * a.sh.Hq + j) * kHeadDim + c, L > 0.0f ? O / L : 0.0f);
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(&a.counters[b * a.sh.Hkv + h], 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace kvq

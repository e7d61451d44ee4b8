// Split-K merge of libkvq's decode: one thread per (query head, channel),
// two query heads per block of 256 threads.  For split s of head (b, j) the
// partial holds o_s[d], m_s, l_s (see splitk.h); the output is
//   out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,  M = max_s m_s,
// the log-sum-exp combination that makes split-K decoding exact.  Each
// thread reads the m_s and l_s of its head itself (the same addresses for
// the 128 threads of a head) together with its own o_s[c], sixteen splits
// at a time, and folds them in with a running maximum: no barriers, and one
// round trip to memory for up to sixteen splits.
#include <hip/hip_runtime.h>

#include "splitk.h"

namespace kvq {
namespace {

__global__ __launch_bounds__(256) void dec_combine_kernel(DecodeArgs a) {
  const int half = threadIdx.x >> 7, c = threadIdx.x & (kHeadDim - 1);
  const int S = a.n_partials;
  const int64_t heads = (int64_t)a.sh.B * a.sh.Hq;
  const int64_t hq = (int64_t)blockIdx.x * 2 + half;
  if (hq >= heads) return;
  const int b = (int)(hq / a.sh.Hq), j = (int)(hq % a.sh.Hq);
  const float* rec0 = partial_rec(a, b, j, 0);
  float M = -INFINITY, L = 0.f, O = 0.f;
  constexpr int kU = 16;   // splits per round trip
  for (int s0 = 0; s0 < S; s0 += kU) {
    float m[kU], l[kU], o[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const bool ok = s0 + u < S;
      const float* p = rec0 + (int64_t)(ok ? s0 + u : 0) * (kHeadDim + 2);
      m[u] = ok ? p[kHeadDim] : -INFINITY;
      l[u] = ok ? p[kHeadDim + 1] : 0.f;
      o[u] = ok ? p[c] : 0.f;
    }
    float mc = M;
#pragma unroll
    for (int u = 0; u < kU; ++u) mc = fmaxf(mc, m[u]);
    if (mc == -INFINITY) continue;   // no tokens in these splits yet
    const float r = M == -INFINITY ? 0.f : exp2f(M - mc);
    L *= r;
    O *= r;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const float w = m[u] == -INFINITY ? 0.f : exp2f(m[u] - mc);
      L = __builtin_fmaf(w, l[u], L);
      O = __builtin_fmaf(w, o[u], O);
    }
    M = mc;
  }
  store_out(a, hq * kHeadDim + c, L > 0.0f ? O / L : 0.0f);
}

}  // namespace

hipError_t launch_combine(const DecodeArgs& a, hipStream_t stream) {
  const int64_t heads = (int64_t)a.sh.B * a.sh.Hq;
  hipLaunchKernelGGL(dec_combine_kernel, dim3((unsigned)((heads + 1) / 2)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq

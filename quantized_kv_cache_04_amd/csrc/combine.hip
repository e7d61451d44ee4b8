// Split-K merge of libkvq's decode: one block of 256 threads merges two
// query heads (128 threads per head, one channel each).  For split s of head
// (b, j) the partial holds o_s[d], m_s, l_s (see splitk.h); the output is
//   out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,  M = max_s m_s,
// the log-sum-exp combination that makes split-K decoding exact.
#include <hip/hip_runtime.h>

#include "splitk.h"

namespace kvq {
namespace {

__global__ __launch_bounds__(256) void dec_combine_kernel(DecodeArgs a) {
  __shared__ float f_w[2][256];      // weight of each split
  __shared__ float f_red[2][2][2];   // [head of the block][wave of the head][max, sum]
  const int half = threadIdx.x >> 7, c = threadIdx.x & (kHeadDim - 1);
  const int w2 = (threadIdx.x >> 6) & 1, lane = threadIdx.x & 63;
  const int S = a.n_partials;
  const int64_t heads = (int64_t)a.sh.B * a.sh.Hq;
  const int64_t hq = (int64_t)blockIdx.x * 2 + half;
  const bool act = hq < heads;
  const int b = act ? (int)(hq / a.sh.Hq) : 0, j = act ? (int)(hq % a.sh.Hq) : 0;
  float m0 = -INFINITY, m1 = -INFINITY, l0 = 0.f, l1 = 0.f;
  if (act && c < S) {
    const float* p = partial_rec(a, b, j, c);
    m0 = p[kHeadDim];
    l0 = p[kHeadDim + 1];
  }
  if (act && c + 128 < S) {
    const float* p = partial_rec(a, b, j, c + 128);
    m1 = p[kHeadDim];
    l1 = p[kHeadDim + 1];
  }
  float mx = fmaxf(m0, m1);
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if (lane == 0) f_red[half][w2][0] = mx;
  __syncthreads();
  const float M = fmaxf(f_red[half][0][0], f_red[half][1][0]);
  const float w0 = (M > -INFINITY && m0 > -INFINITY) ? exp2f(m0 - M) : 0.f;
  const float w1 = (M > -INFINITY && m1 > -INFINITY) ? exp2f(m1 - M) : 0.f;
  if (c < S) f_w[half][c] = w0;
  if (c + 128 < S) f_w[half][c + 128] = w1;
  float ls = w0 * l0 + w1 * l1;
  for (int off = 32; off >= 1; off >>= 1) ls += __shfl_xor(ls, off, 64);
  if (lane == 0) f_red[half][w2][1] = ls;
  __syncthreads();
  const float L = f_red[half][0][1] + f_red[half][1][1];
  float O = 0.f;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = (act && s0 + u < S) ? partial_rec(a, b, j, s0 + u)[c] : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < S) O += f_w[half][s0 + u] * v[u];
  }
  if (act) store_out(a, hq * kHeadDim + c, L > 0.0f ? O / L : 0.0f);
}

}  // namespace

hipError_t launch_combine(const DecodeArgs& a, hipStream_t stream) {
  const int64_t heads = (int64_t)a.sh.B * a.sh.Hq;
  hipLaunchKernelGGL(dec_combine_kernel, dim3((unsigned)((heads + 1) / 2)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq

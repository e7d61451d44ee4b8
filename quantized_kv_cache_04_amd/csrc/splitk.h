// Split-K (flash-decoding) partial states shared by the decode kernels.
//
// Every workgroup handles a token range of one (sequence, KV head) and
// leaves, per query head, an unnormalized partial (o, m, l): the reference
// maximum m of the base-2 scores, l = sum 2^(s - m) and o = sum 2^(s - m) v.
// A second, small kernel merges the partials of all splits with
// log-sum-exp weights (dec_combine_kernel).  Keeping the merge in its own
// launch avoids device-scope fences in the streaming kernel: on a GPU whose
// L2 is split across chiplets such a fence writes back and invalidates the
// whole L2 of the chiplet.  (Merging in the last workgroup of each
// sequence and KV head measured slower both with a fence per workgroup and
// with the partial states stored and read at device scope, past the L2s:
// each workgroup then waits for its stores before it may count itself.)
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

}  // namespace kvq

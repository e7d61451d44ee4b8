// Launch of a decode streaming kernel with the caller's optional profiling
// events (kvq_set_decode_events): given, they are recorded at the kernel's
// own start and end by hipExtLaunchKernel, so that their interval is the
// kernel's execution alone, without the dispatch gap before it.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include "kvq_internal.h"

namespace kvq {

template <typename F>
inline void launch_timed(F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t s,
                         const DecodeArgs& a) {
  if (a.ev_start || a.ev_stop)
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, a.ev_start, a.ev_stop, 0u, a);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, a);
}

}  // namespace kvq

// fa_launch.h -- internal interface between the C ABI (fa_api.hip) and the
// kernels (fa_fwd_kernel.hip). Not installed; the public header is include/fa.h.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

int block_m();
int block_n(int d);
int threads_per_block();
int lds_bytes(int d);

// Enqueues the forward kernel; arguments were validated by the caller.
hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int N, int d, bool causal, float scale, bool bf16,
                      hipStream_t stream);

}  // namespace fa

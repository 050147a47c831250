// fa_launch.h -- internal interface between the C ABI (fa_api.hip) and the
// kernels (fa_fwd_kernel.hip). Not installed; the public header is include/fa.h.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

// Workgroup shape chosen for a problem: waves per workgroup, query rows per
// wave, and the resulting rows per workgroup and threads.
struct Shape {
    int waves;
    int rows_per_wave;
    int block_m;
    int threads;
};

Shape pick_shape(int B, int H, int n_queries, int d, bool causal);
int block_n(int d);
int lds_bytes(int d);

// Enqueues the forward kernel for Nq query rows against Nk keys per head;
// arguments were validated by the caller.
hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int Nq, int Nk, int d, bool causal, float scale, bool bf16,
                      hipStream_t stream);

}  // namespace fa

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

// Split launch for few query tiles (KV-cache decode): the key tiles of each
// 128-row query tile are divided into n_splits chunks whose partial results
// go to `workspace` (n_splits * B*H*Nq * (d + 1) floats) and are then merged
// into o and lse; arguments were validated by the caller.
hipError_t launch_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                            int H, int Nq, int Nk, int d, bool causal, float scale, bool bf16,
                            int n_splits, float* workspace, hipStream_t stream);
int split_rows_per_tile();

// Enqueues the backward pass (delta, dK/dV and dQ kernels); arguments were
// validated by the caller.
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int H, int N,
                      int d, bool causal, float scale, bool bf16, hipStream_t stream);

}  // namespace fa

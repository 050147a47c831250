// fa_launch.h -- internal interface between the C ABI (fa_api.hip) and the
// kernels (fa_fwd_kernel.hip, fa_fwd_masked.hip, fa_bwd_kernel.hip). Not installed; the public header is include/fa.h.
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

// Padding and sliding-window masks of a masked launch (fa_tiles.h, row_keys).
struct MaskArgs {
    int window_left;      // -1: unbounded
    int window_right;     // -1: unbounded; not used when causal
    const int* key_lens;  // device, [B] key counts (clamped into [0, Nk]), or nullptr
    int heads;            // H: head bh belongs to batch bh / H
};

Shape pick_shape(int B, int H, int n_queries, int d, bool causal);
// The shape of a masked launch: pick_shape's, except that d = 128 keeps 4 waves.
Shape pick_shape_masked(int B, int H, int n_queries, int d, bool causal);
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

// The same two launches with padding and window masks; rows that see no key
// get O = 0 and lse = -inf.
hipError_t launch_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                             int H, int Nq, int Nk, int d, bool causal, const MaskArgs& mask,
                             float scale, bool bf16, hipStream_t stream);
hipError_t launch_fwd_split_masked(const void* q, const void* k, const void* v, void* o, float* lse,
                                   int B, int H, int Nq, int Nk, int d, bool causal,
                                   const MaskArgs& mask, float scale, bool bf16, int n_splits,
                                   float* workspace, hipStream_t stream);

// Enqueues the backward pass (delta, dK/dV and dQ kernels); arguments were
// validated by the caller.
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int H, int N,
                      int d, bool causal, float scale, bool bf16, hipStream_t stream);

}  // namespace fa

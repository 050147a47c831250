// fa_launch.h -- internal interface between the C ABI (fa_api.hip) and the
// kernels. The forward launches are split over five sources by variant
// (fa_fwd_kernel.hip: no masks, head dim 64 or 128; fa_fwd_masked.hip: masks;
// fa_fwd_hdim.hip and fa_fwd_hdim_masked.hip: other head dims), built from
// the kernel template in fa_fwd_kernel.h, and fa_fwd_ks.hip, the key-split
// kernel of fa_fwd_ks.h for small grids (any head dim). The backward pass is in
// fa_bwd_kernel.h, launched from fa_bwd_kernel.hip (head dim 64 or 128) and
// fa_bwd_hdim.hip (other head dims). Not installed; the public header is include/fa.h.
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

// One forward launch, arguments already validated by the caller.
struct FwdArgs {
    const void *q, *k, *v;
    void* o;
    float* lse;
    int B, H, Nq, Nk;
    int d;            // head dim: 64 or 128, or a multiple of 8 below 128 (run padded)
    bool causal;
    float scale;
    bool bf16;
    bool masked;      // padding / window masks in effect (mask below)
    MaskArgs mask;
    bool split;       // split-key launch: n_splits chunks through workspace, then the merge
    int n_splits;
    float* workspace; // n_splits * B*H*Nq * (kernel_dim(d) + 1) floats
    hipStream_t stream;
};

// The head dim the kernel runs with: 64 or 128.
inline int kernel_dim(int d) { return d <= 64 ? 64 : 128; }
// The dims the forward kernel's MFMAs cover: d rounded up to a multiple of 32
// (32, 64, 96 or 128), at most kernel_dim(d).
inline int compute_dim(int d) { return (d + 31) / 32 * 32; }

// Whether an unmasked direct launch runs the key-split kernel (fa_fwd_ks.h):
// more than 32 query rows (fewer go to the split-key path), every 32-row
// workgroup resident at once (256 at head dims above 64, where one workgroup's
// 128-160 KB of LDS fills a CU, 512 below), and at most 2048 keys seen by the
// longest query block (causal: min(Nq, Nk)). Measured on MI355X against the
// direct and split launches (bf16, B*H from 1 to 64, 128 to 4096 query rows,
// 128 to 16384 keys): it is the fastest inside these bounds (B2 H4 N1000
// d64: 8.5 us against 13.7 direct and 15.9 split; N128: 4.1 against 4.8),
// while more workgroups or longer key ranges favour the direct launch or the
// split (more waves per key range).
inline bool uses_key_split(int B, int H, int Nq, int Nk, int d, bool causal)
{
    const int64_t blocks = (int64_t)B * H * ((Nq + 31) / 32);
    const int64_t keys = causal && Nq < Nk ? Nq : Nk;
    const int64_t resident = kernel_dim(d) == 64 ? 512 : 256;
    return Nq > 32 && blocks <= resident && keys <= 2048;
}

// LDS per key-split workgroup: two K (three when it computes 128 dims) and
// two V tiles of 32 keys for each of its four waves (the merge reuses less
// than that).
inline int ks_lds_bytes(int d) { return 4 * (compute_dim(d) == 128 ? 5 : 4) * 32 * kernel_dim(d) * 2; }

Shape pick_shape(int B, int H, int n_queries, int d, bool causal);
// The shape of a masked launch: pick_shape's, except that a kernel head dim
// of 128 keeps 4 waves.
Shape pick_shape_masked(int B, int H, int n_queries, int d, bool causal);
int block_n(int d);
// LDS per workgroup; stage_out: the launch stages its output through LDS (no
// split, head dim at least 64); q_tile: it also copies its Q tile there (8
// waves, no masks or padding).
int lds_bytes(int d, int waves, bool stage_out, bool q_tile);
int split_rows_per_tile();

// Enqueues the forward pass (one kernel, or the split kernel and the merge).
hipError_t launch_forward(const FwdArgs& a);
// The variants launch_forward picks from, one per source file.
hipError_t launch_forward_masked(const FwdArgs& a);
hipError_t launch_forward_hdim(const FwdArgs& a);
hipError_t launch_forward_hdim_masked(const FwdArgs& a);
// The key-split kernel for small grids (uses_key_split), any head dim.
hipError_t launch_forward_ks(const FwdArgs& a);

// fp32 inputs and outputs (d = 64 or 128): splits K and V into bf16 hi/lo
// parts in `workspace` (4 * B*H*Nk*d bf16 values), then one kernel.
hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
                          int Nq, int Nk, int d, bool causal, float scale, void* workspace, hipStream_t stream);

// Enqueues the backward pass (delta, dK/dV and dQ kernels); arguments were
// validated by the caller. mask: padding / window masks, or nullptr. d: 64 or
// 128, or a multiple of 8 below 128 (launch_bwd_hdim, run padded).
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int H, int Nq,
                      int Nk, int d, bool causal, float scale, bool bf16, const MaskArgs* mask,
                      hipStream_t stream);
hipError_t launch_bwd_hdim(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int H, int Nq,
                           int Nk, int d, bool causal, float scale, bool bf16, const MaskArgs* mask,
                           hipStream_t stream);

}  // namespace fa

/*
 * fa.h -- C ABI of libfa: fused attention forward (FlashAttention-2 form)
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation, from "How to optimise a Triton FlashAttention-2 kernel step
 * by step with a profiler" (sections "Where the last article left off" and
 * Round 4) and "Programming an attention kernel in Triton" (Kernel 4):
 *
 *   O   = softmax(scale * Q K^T [+ causal mask]) V
 *   lse = per-row logsumexp of scale * Q K^T over the visible keys (natural log)
 *
 * One workgroup owns a tile of query rows, streams K and V tiles through LDS
 * and keeps the running max, running sum and unnormalised output in fp32
 * registers (online softmax); O and lse are written once.
 *
 * Conventions shared by every entry point:
 *   - Tensors are dense, row-major: q and o [B, H, Nq, d], k and v
 *     [B, H, Nk, d], lse [B, H, Nq]. The *_qk entry points take Nq and Nk
 *     separately; the others are the self-attention case Nq = Nk = N. No
 *     strides are taken.
 *   - Device pointers are HIP device memory owned by the caller; libfa
 *     allocates nothing, frees nothing and keeps no pointer after a call.
 *   - A causal query row i attends to keys j <= i (absolute positions, as the
 *     keep test of "How to optimise a Triton FlashAttention-2 kernel step by
 *     step with a profiler", Round 4, "Causal tile-skipping": with Nq != Nk
 *     the diagonal starts at the top-left corner, and rows i >= Nk see every
 *     key).
 *   - Functions return an fa_status; nothing is thrown across the ABI.
 *     Argument errors are reported before any HIP call is made.
 */
#ifndef FA_H
#define FA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1, /* NULL/misaligned/overlapping pointer, bad size, dtype or scale */
    FA_ERR_UNSUPPORTED = 2, /* well-formed but not built: a head dim that is not a multiple of
                               8 from 8 to 128 (fp32 inputs: not 64 or 128) */
    FA_ERR_HIP = 3          /* the HIP runtime reported an error (see fa_status_string) */
} fa_status;

typedef enum {
    FA_DTYPE_F16 = 0,  /* IEEE binary16 inputs and output */
    FA_DTYPE_BF16 = 1  /* bfloat16 inputs and output */
} fa_dtype;

/*
 * fa_fwd -- attention forward pass.
 *
 *   q, k, v : device, [B, H, N, d] contiguous, element type `dtype`,
 *             16-byte aligned. Read only.
 *   o       : device, [B, H, N, d] contiguous, element type `dtype`,
 *             16-byte aligned, must not overlap q, k, v or lse. Every element
 *             is overwritten with O rounded to nearest-even.
 *   lse     : device, [B, H, N] fp32, 4-byte aligned, must not overlap the
 *             others. Every element is overwritten with the row's
 *             logsumexp in natural-log units (kept for a backward pass, as
 *             in "How to optimise a Triton FlashAttention-2 kernel step by
 *             step with a profiler", Round 4, "exp2").
 *   B, H, N : >= 1, with N*d*2 < 2^32 (one head below 4 GiB).
 *   d       : a multiple of 8 from 8 to 128 (other values: FA_ERR_UNSUPPORTED).
 *             64 and 128 have kernels of their own; any other d runs with
 *             the tiles of the d = 64 kernel (d < 64) or the d = 128 kernel,
 *             the missing dims held at zero on chip, so the result is that of
 *             head dim d; the matrix cores compute d rounded up to 32 dims
 *             (32, 64, 96 or 128). ("How to optimise a Triton
 *             FlashAttention-2 kernel step by step with a profiler" runs its
 *             tests over several shapes, input types and head dims, Round 3.)
 *   causal  : 0 or 1.
 *   scale   : finite and > 0; multiplies Q K^T before the softmax
 *             (1/sqrt(d) is the usual choice, the caller computes it).
 *   dtype   : an fa_dtype.
 *   stream  : hipStream_t to launch on (NULL: the default stream).
 *
 * The call is asynchronous: it enqueues one kernel on `stream` and returns.
 * Softmax and accumulation are fp32; P is rounded to `dtype` before the
 * P.V product. Results are deterministic (no atomics, no split over keys).
 */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
           int N, int d, int causal, float scale, int dtype, void *stream);

/*
 * fa_fwd_qk -- attention forward pass with Nq query rows and Nk keys per head
 * ("Programming an attention kernel in Triton", Kernel 4, validates such
 * mismatched lengths, down to a single query).
 *
 *   q, o    : device, [B, H, Nq, d] contiguous, element type `dtype`, 16-byte
 *             aligned (o is written, as in fa_fwd).
 *   k, v    : device, [B, H, Nk, d] contiguous, element type `dtype`, 16-byte
 *             aligned.
 *   lse     : device, [B, H, Nq] fp32, 4-byte aligned (written).
 *   Nq, Nk  : >= 1, with Nk*d*2 < 2^32 and Nq*d*2 < 2^32.
 * Everything else as fa_fwd, which is fa_fwd_qk with Nq = Nk = N.
 */
int fa_fwd_qk(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
              int Nq, int Nk, int d, int causal, float scale, int dtype, void *stream);

/*
 * Split-key forward, for problems with too few query tiles to fill the GPU
 * (KV-cache decode: a handful of query rows against a long key sequence).
 * The key tiles each 128-row query tile visits are divided into n_splits
 * contiguous chunks, one workgroup each; every chunk's normalised partial
 * output (fp32) and logsumexp go to a caller-owned workspace, and a second
 * kernel merges them exactly: lse = ln sum_s e^{lse_s},
 * O = sum_s e^{lse_s - lse} O_s. That merge is the running-max and
 * running-sum correction of the online softmax ("Programming an attention
 * kernel in Triton", "The wall, named honestly") applied once per chunk.
 * The profiler page names KV-cache decode as the next step ("Getting the
 * kernel correct, then benchmarking it honestly", closing paragraph).
 *
 * fa_split_count -- a suggested n_splits (>= 1), from timings on MI355X:
 *   for up to 32 query rows about 512 workgroups in all and chunks of at
 *   least two key tiles of 64; with more query rows at most 256 workgroups
 *   and chunks of at least 16 key tiles (8 for grids of at most 16
 *   workgroups); 1, the direct path, under 16 key tiles and wherever the
 *   direct entry points run their key-split kernel (more than 32 query rows,
 *   at most 2048 keys, every 32-row workgroup resident: at most 512 of them
 *   for d <= 64, 256 above; its four waves split each 32-row block's keys
 *   and merge on chip). A causal problem counts the min(Nq, Nk) keys its
 *   longest query tile sees. Returns 0 on invalid arguments.
 * fa_split_workspace_bytes -- bytes of workspace fa_fwd_split_qk needs:
 *   n_splits * B*H*Nq * (D + 1) * 4, with D = 64 for d <= 64 and 128
 *   otherwise (the kernel's head dim). Returns 0 on invalid arguments.
 * fa_fwd_split_qk -- arguments as fa_fwd_qk, plus:
 *   n_splits        : 1 .. ceil(Nk / 64).
 *   workspace       : device, >= fa_split_workspace_bytes(...) bytes,
 *                     16-byte aligned, owned by the caller, overlapping no
 *                     tensor argument. Its contents on entry do not matter;
 *                     on return it holds the partial results.
 *   workspace_bytes : its size.
 * Two kernels are enqueued on `stream`; calls that share a workspace must be
 * ordered on one stream. O and lse equal those of fa_fwd_qk up to rounding.
 */
int fa_split_count(int B, int H, int Nq, int Nk, int d, int causal);
int64_t fa_split_workspace_bytes(int B, int H, int Nq, int d, int n_splits);
int fa_fwd_split_qk(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                    int H, int Nq, int Nk, int d, int causal, float scale, int dtype, int n_splits,
                    void *workspace, int64_t workspace_bytes, void *stream);

/*
 * fa_fwd_split_qk_noalloc -- for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): fa_fwd_split_qk without the workspace arguments. The partial
 * results go to a scratch array of the library's own, FA_NOALLOC_SCRATCH_BYTES
 * of device memory on each GPU the call runs on, which that GPU holds until
 * the process ends. The call allocates nothing and frees nothing: on the
 * first call on a device (the current device) it looks up the array's
 * address there and keeps it. Arguments, results and ordering as
 * fa_fwd_split_qk. Returns FA_ERR_UNSUPPORTED, before any HIP call, when
 * fa_split_workspace_bytes(B, H, Nq, d, n_splits) exceeds
 * FA_NOALLOC_SCRATCH_BYTES (then call fa_fwd_split_qk with a workspace).
 * Every call on one GPU uses the same array and overwrites it: calls that can
 * overlap in time on one GPU (on different streams, or from several threads)
 * race and give wrong results; order them on one stream. Each call writes
 * every scratch entry it reads, so nothing needs clearing between calls.
 */
#define FA_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)
int fa_fwd_split_qk_noalloc(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                            int H, int Nq, int Nk, int d, int causal, float scale, int dtype,
                            int n_splits, void *stream);

/*
 * Padding masks and sliding windows. "How to optimise a Triton
 * FlashAttention-2 kernel step by step with a profiler", section "Future
 * articles", names them as the case where a query row can be left with no
 * visible key, which a finite mask sentinel gets wrong. Row i of batch b sees
 * key j iff
 *   j < key_lens[b]                         (padding; all Nk keys when NULL),
 *   j >= i - window_left                    (when window_left >= 0),
 *   j <= i             when causal,
 *   j <= i + window_right when not causal   (when window_right >= 0).
 * -1 leaves a window unbounded; window_right is not used when causal. A row
 * that sees no key gets O = 0 and lse = -infinity (the logsumexp of an empty
 * set), never NaN. Only the key tiles some row of a query tile can see are
 * visited, and only tiles at the edges of the visible band get the mask.
 *
 * fa_fwd_masked -- arguments as fa_fwd_qk, plus:
 *   window_left, window_right : >= -1.
 *   key_lens : device, [B] int32, 4-byte aligned, or NULL. Read by the kernel;
 *              values outside [0, Nk] are clamped into it. It must not
 *              overlap o or lse.
 * With no mask in effect (key_lens NULL, window_left -1, and causal or
 * window_right -1) the call is fa_fwd_qk.
 *
 * fa_fwd_split_masked -- the split-key launch of fa_fwd_split_qk with the same
 *   masks (KV-cache decode over batches of different cache lengths). Split
 *   count, workspace and ordering rules as fa_fwd_split_qk; key_lens must not
 *   overlap the workspace either.
 */
int fa_fwd_masked(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                  int Nq, int Nk, int d, int causal, int window_left, int window_right,
                  const int32_t *key_lens, float scale, int dtype, void *stream);
int fa_fwd_split_masked(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                        int H, int Nq, int Nk, int d, int causal, int window_left, int window_right,
                        const int32_t *key_lens, float scale, int dtype, int n_splits,
                        void *workspace, int64_t workspace_bytes, void *stream);

/*
 * fa_fwd_f32 -- attention forward for fp32 inputs and outputs ("How to
 * optimise a Triton FlashAttention-2 kernel step by step with a profiler",
 * Round 1: the test file includes fp32 inputs at D = 128, whose products
 * that page's kernel forms in a reduced-precision fp32 format).
 *
 * Each fp32 value x is split into hi = bf16(x) (round to nearest even) and
 * lo = bf16(x - hi), and every product of Q K^T and P V is formed on the bf16
 * matrix cores as hi*hi + hi*lo + lo*hi with fp32 accumulation: about 16
 * significant bits per product, at a third of the bf16 rate (the fp32 matrix
 * rate of gfx950 is a sixteenth). Softmax state and accumulation are fp32.
 *
 *   q, o      : device, [B, H, Nq, d] fp32, 16-byte aligned (o written).
 *   k, v      : device, [B, H, Nk, d] fp32, 16-byte aligned.
 *   lse       : device, [B, H, Nq] fp32 (written, natural log).
 *   d         : 64 or 128 (others: FA_ERR_UNSUPPORTED); Nk*d*4 < 2^32.
 *   workspace : device, >= fa_f32_workspace_bytes(B, H, Nk, d) bytes
 *               (8*B*H*Nk*d: the hi and lo parts of K and V in bf16),
 *               16-byte aligned, owned by the caller, overlapping no tensor
 *               argument; contents on entry do not matter.
 * causal, scale, stream as fa_fwd_qk. Three kernels are enqueued (the split
 * of K, the split of V, the attention kernel); deterministic.
 */
int64_t fa_f32_workspace_bytes(int B, int H, int Nk, int d);
int fa_fwd_f32(const float *q, const float *k, const float *v, float *o, float *lse, int B, int H,
               int Nq, int Nk, int d, int causal, float scale, void *workspace,
               int64_t workspace_bytes, void *stream);

/*
 * fa_bwd -- attention backward pass: the gradients of sum(dO * O) with respect
 * to q, k and v, where O = fa_fwd(q, k, v) with the same causal flag and
 * scale. "How to optimise a Triton FlashAttention-2 kernel step by step with
 * a profiler" names this pass as its next kernel (closing list): it consumes
 * the logsumexp the forward writes and accumulates in two directions. With
 * P_ij = exp(scale <q_i, k_j> - lse_i) over the visible keys:
 *   D_i = <dO_i, O_i>,  dS_ij = P_ij (<dO_i, v_j> - D_i),
 *   dV_j = sum_i P_ij dO_i,  dK_j = scale sum_i dS_ij q_i,
 *   dQ_i = scale sum_j dS_ij k_j.
 *
 *   q, k, v, o, dout : device, [B, H, N, d] contiguous, element type `dtype`,
 *                      16-byte aligned; o and lse as written by fa_fwd.
 *   lse              : device, [B, H, N] fp32, 4-byte aligned.
 *   dq, dk, dv       : device, [B, H, N, d], `dtype`, 16-byte aligned,
 *                      overwritten; no overlap with any other argument.
 *   delta            : device, [B, H, N] fp32, 16-byte aligned, owned by the
 *                      caller: scratch that receives D (libfa allocates
 *                      nothing).
 * Other arguments as fa_fwd, d included (a multiple of 8 from 8 to 128;
 * below 128 other than 64 the d = 64 or 128 kernels run with the missing
 * dims held at zero, computing d rounded up to 32 dims). Three kernels are
 * enqueued on `stream`; nothing uses
 * atomics, so results are deterministic.
 */
int fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
           const float *lse, void *dq, void *dk, void *dv, float *delta, int B, int H, int N, int d,
           int causal, float scale, int dtype, void *stream);

/*
 * fa_bwd_qk -- the backward pass for Nq query rows against Nk keys per head
 * (the gradients of fa_fwd_qk, same causal rule: key j is visible to row i
 * iff j <= i). q, o, dout, dq are [B, H, Nq, d]; lse and delta [B, H, Nq];
 * k, v, dk, dv [B, H, Nk, d]. Keys no row sees get dK = dV = 0. Other
 * arguments as fa_bwd, which is fa_bwd_qk with Nq = Nk = N. No output
 * (dq, dk, dv, delta) may overlap another output or an input.
 */
int fa_bwd_qk(const void *q, const void *k, const void *v, const void *o, const void *dout,
              const float *lse, void *dq, void *dk, void *dv, float *delta, int B, int H, int Nq,
              int Nk, int d, int causal, float scale, int dtype, void *stream);

/*
 * fa_bwd_masked -- the backward pass of fa_fwd_masked: the same padding
 * lengths and sliding windows (window_left, window_right, key_lens with the
 * meaning, clamping and overlap rules of fa_fwd_masked), o and lse as that
 * call wrote them. Keys that no row sees get dK = dV = 0; a row that sees no
 * key (O = 0, lse = -inf) gets dQ = 0 and adds nothing elsewhere. Other
 * arguments as fa_bwd_qk; with no mask in effect it is fa_bwd_qk.
 */
int fa_bwd_masked(const void *q, const void *k, const void *v, const void *o, const void *dout,
                  const float *lse, void *dq, void *dk, void *dv, float *delta, int B, int H, int Nq,
                  int Nk, int d, int causal, int window_left, int window_right,
                  const int32_t *key_lens, float scale, int dtype, void *stream);

/*
 * fa_status_string -- human-readable text for a status code. For FA_ERR_HIP
 * and FA_ERR_INVALID_ARG it names the HIP error or the failed check of the
 * last failing call on the calling thread. The returned pointer stays valid
 * until the next libfa call on the same thread.
 */
const char *fa_status_string(int status);

/*
 * fa_tile_counts -- (query tile, key tile) pairs of one head, for a tiling of
 * block_m query rows by block_n keys (host only, no HIP call). Causal
 * attention visits, for the query tile starting at q0, the key tiles that
 * need no mask (those ending at or before the block_n-aligned start of q0)
 * and then the tiles up to key min(q0 + block_m, N) - 1, which get the mask;
 * key tiles above the diagonal are never visited. Non-causal attention
 * masks only a ragged last key tile. This is the split described in
 * "How to optimise a Triton FlashAttention-2 kernel step by step with a
 * profiler", Round 4, "Causal tile-skipping".
 *
 *   counts[0] = all pairs, ceil(N/block_m) * ceil(N/block_n)
 *   counts[1] = visited pairs
 *   counts[2] = visited pairs that need no mask
 *   counts[3] = visited pairs that get the mask
 * Returns FA_ERR_INVALID_ARG for N < 1, non-positive tile sizes or NULL.
 */
int fa_tile_counts(int64_t N, int block_m, int block_n, int causal, int64_t counts[4]);

/* fa_tile_counts_qk -- the same for Nq query rows against Nk keys:
 * counts[0] = ceil(Nq/block_m) * ceil(Nk/block_n); fa_tile_counts is the
 * case Nq = Nk = N. */
int fa_tile_counts_qk(int64_t Nq, int64_t Nk, int block_m, int block_n, int causal,
                      int64_t counts[4]);

/* fa_tile_counts_masked -- the same for one batch under the masks of
 * fa_fwd_masked with key_len keys (0 <= key_len <= Nk): counts[1] the visited
 * pairs (key tiles holding a key some row of the query tile sees), counts[2]
 * those every row of the query tile sees in full (no mask), counts[3] the
 * rest. */
int fa_tile_counts_masked(int64_t Nq, int64_t Nk, int block_m, int block_n, int causal,
                          int64_t window_left, int64_t window_right, int64_t key_len,
                          int64_t counts[4]);

/* Launch plan of fa_fwd for a problem (host only, no HIP call). */
typedef struct {
    int block_m;            /* query rows per workgroup */
    int block_n;            /* keys per K/V tile in LDS */
    int threads;            /* threads per workgroup (wave64) */
    int lds_bytes;          /* LDS per workgroup */
    int64_t workgroups;     /* grid size */
    int64_t pairs_visited;  /* visited (query tile, key tile) pairs, all heads */
    double mfma_flops;      /* FLOPs the matrix cores execute, D the head dim
                               rounded up to a multiple of 32 (the dims the
                               forward kernel computes): 2*32*64*D for each block of
                               32 query rows x 64 keys of which a wave computes
                               S = Q K^T, and as much for each it computes P V.
                               Every visited tile pair counts, masked ones too,
                               except that in a causal tile a wave skips the key
                               tiles past its own rows (and under masks the
                               tiles its rows do not see) */
    double algo_flops;      /* 4*d per (query, key) pair of the visible region:
                               4*B*H*Nq*Nk*d non-causal; causal counts the area
                               below the diagonal, Nq*Nq/2 for Nq <= Nk and
                               Nk*Nk/2 + (Nq-Nk)*Nk otherwise, so that Nq = Nk
                               gives the pages' halved 4*B*H*N*N*d */
    double algo_bytes;      /* compulsory HBM bytes: q, k, v read and o written
                               once (2 bytes each: 4*B*H*(Nq+Nk)*d) plus lse */
} fa_plan_t;

/*
 * fa_plan -- fill `plan` for the given problem; the same argument rules as
 * fa_fwd apart from the pointers. Returns FA_OK, FA_ERR_INVALID_ARG or
 * FA_ERR_UNSUPPORTED.
 */
int fa_plan(int B, int H, int N, int d, int causal, int dtype, fa_plan_t *plan);

/* fa_plan_qk -- the plan of fa_fwd_qk; fa_plan is the case Nq = Nk = N. */
int fa_plan_qk(int B, int H, int Nq, int Nk, int d, int causal, int dtype, fa_plan_t *plan);

/* fa_plan_masked -- the plan of fa_fwd_masked. key_lens is a HOST array of B
 * values in [0, Nk] (or NULL). Here algo_flops is 4*d per visible (query,
 * key) pair counted exactly (the diagonal included), and algo_bytes reads q
 * and writes o and lse once and reads each key and value row that some row
 * sees once. */
int fa_plan_masked(int B, int H, int Nq, int Nk, int d, int causal, int window_left, int window_right,
                   const int32_t *key_lens, int dtype, fa_plan_t *plan);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */

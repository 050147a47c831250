// fa_fwd_kernel.h -- the attention forward kernel (FlashAttention-2 form) for
// gfx950, its epilogues, the merge of a split launch and the launch templates.
// One template covers every variant, chosen at compile time: SPLIT (the key
// tiles of a query tile divided over several workgroups, for decode), MASKS
// (padding lengths and sliding windows) and PADDED (head dims other than 64
// and 128, run with the missing dims held at zero). fa_fwd_kernel.hip,
// fa_fwd_masked.hip, fa_fwd_hdim.hip and fa_fwd_hdim_masked.hip instantiate
// the four MASKS x PADDED combinations, each with and without SPLIT.
//
// Method: "How to optimise a Triton FlashAttention-2 kernel step by step with
// a profiler" ("Where the last article left off", Round 1, Round 4): one
// workgroup per tile of query rows; K and V tiles stream through LDS; the
// running max m, running sum l and unnormalised O stay in fp32 registers and
// are rescaled when a tile raises the max (the online softmax named at the end
// of "Programming an attention kernel in Triton"); O and the logsumexp are
// written once.
//
// gfx950 mapping (our design, not the pages'):
//   * A workgroup is WAVES waves (4 or 8); each wave owns QB blocks of 32 whole
//     query rows, so row reductions never leave the wave (the pages' rule that
//     every warp must own whole rows, Round 0 / Round 1). The launches use
//     QB = 1, which keeps two waves per SIMD; the template's QB = 2 (each K and
//     V operand read feeding two MFMAs) needs more registers than that allows.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_{bf16,f16}: keys on the M axis, queries on N. In the
//     32x32 accumulator each lane holds 16 keys of ONE query, and the other 16
//     keys of that query sit in lane ^ 32. The row max and row sum are
//     in-lane plus one v_permlane32_swap, and the rescale of O by alpha is one
//     scalar per lane. Consecutive score MFMAs share their Q operand (the
//     32-key blocks of a tile run interleaved), which lowers operand toggling
//     and with it the energy per MFMA on this power-limited part.
//   * O^T += V^T P^T takes P^T straight from the score registers as the B
//     operand: the accumulator hands lane half h, element e the key
//     16t + 8(e/4) + 4h + (e%4), and the V^T operand is read in that key
//     order, so P never goes through LDS.
//   * Q is loaded once into registers in B-operand layout.
//   * K and V tiles go from HBM straight into LDS (buffer_load_dwordx4 ... lds,
//     16 bytes per lane, no staging registers), row-major and dense. The
//     16-byte chunks of each row are XOR-swizzled by a function of the row so
//     that the operand reads below hit distinct banks.
//   * K is read as the A operand of S^T = K Q^T with one ds_read_b128 per
//     MFMA. V is read as the A operand of O^T = V^T P^T with two
//     ds_read_b64_tr_b16: within each 16-lane group that instruction hands
//     lane j element (j mod 4) of the 8-byte chunk addressed by lane
//     4e + j/4, so 16 lanes addressing 4 keys x 4 dim-quads receive 4 keys of
//     one dim each: a transposed read of the row-major tile.
//   * Software pipeline over key tiles, two K and two V buffers in LDS:
//     iteration j computes the scores of tile j+1 on the matrix cores with
//     the exp2 work of tile j interleaved between those MFMAs in program
//     order (the two are independent, so the vector units run while the
//     matrix core does), then P_j V_j; the copies of K_{j+2} and V_{j+1}
//     are in flight meanwhile; one barrier per tile. The last tile runs
//     without a successor, so no score MFMA is wasted. The copies go through
//     a buffer descriptor bounded to the head, so the rows of a ragged last
//     tile past N arrive as zeros (and are masked). A wave raises its issue
//     priority while it runs that mixed score/exp block, so that the other
//     wave of its SIMD, then mostly in P.V MFMAs, fills the matrix core
//     around it. d=64 without masks splits the exp work of a tile by its two
//     32-key blocks over the score block and the previous tile's P.V block.
//   * exp2 with the softmax scale and log2(e) folded into one constant
//     (Round 4, "exp2"); the running max is kept in log2 units. The max is
//     updated lazily: a tile's P is taken against the running max and the
//     tile's own row max is reduced only when a partial row sum shows that P
//     grew past 2^12 (always on the first tile); O and l carry the same
//     factor, so O / l is unchanged.
//   * P is rounded to the input type after l has been summed from fp32 P
//     (Round 4, "The P cast").
//   * Causal attention visits no key tile above the diagonal and masks only
//     the diagonal tiles; non-causal attention masks only a ragged last tile
//     (Round 4, "Causal tile-skipping"). Masked scores are -inf; the running
//     max starts at a finite very negative value so a row with no visible key
//     in a tile never forms -inf - (-inf).
//   * Workgroup ids are remapped. Non-causal: all query tiles of one (b, h)
//     run on the same XCD (workgroups are dealt round-robin over the 8 XCDs,
//     each with its own L2), which keeps that head's K and V in one L2.
//     Causal: longest tiles of every head first, which balances the uneven
//     causal work over the XCDs.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"
#include "fa_tiles.h"

namespace fa {
namespace {

// blockIdx -> (b*H + h, query tile). Hardware id i runs on XCD i % 8 and
// the ids are dealt in order.
//  * Non-causal (equal tiles): each XCD gets a contiguous range of
//    head-major ids, so a head's query tiles share one L2.
//  * Causal (a tile's work grows with its index): tile-major, longest tiles
//    of all heads first, id i -> head i % BH. Greedy dispatch of
//    longest-first work then keeps every XCD busy to the end, and when BH is
//    a multiple of 8 every tile of a head still lands on one XCD.
//  * Padding lengths (the work of a head depends on its batch): the same
//    tile-major order, so that every XCD gets heads of every batch instead
//    of the contiguous range that would leave some XCDs all the long batches.
template <bool CAUSAL>
__device__ __forceinline__ void workgroup_tile(int n_qt, bool uneven_heads, uint32_t& bh, uint32_t& qt)
{
    const uint32_t nwg = gridDim.x, hw = blockIdx.x;
    if (CAUSAL || uneven_heads) {
        const uint32_t n_bh = nwg / (uint32_t)n_qt;
        bh = hw % n_bh;
        qt = (uint32_t)n_qt - 1 - hw / n_bh;
    } else {
        const uint32_t xcd = hw % kXcds, slot = hw / kXcds;
        const uint32_t per = nwg / kXcds, extra = nwg % kXcds;
        const uint32_t logical = xcd < extra ? xcd * (per + 1) + slot
                                             : extra * (per + 1) + (xcd - extra) * per + slot;
        bh = logical / (uint32_t)n_qt;
        qt = logical % (uint32_t)n_qt;
    }
}

// Non-causal launches with padding lengths: every query tile of a batch costs
// about the same, in proportion to the batch's key count, and dealing the
// batches interleaved leaves the long ones to finish alone at the end.
// Batches are taken longest first (largest key count, then lowest index),
// each batch's heads tile-major as above, so that greedy dispatch runs the
// longest work first. Each wave ranks the batches itself, one lane per batch
// (B <= 64); the ranks form a permutation, so exactly one lane matches.
__device__ __forceinline__ void padded_batch_tile(int n_qt, int heads, const int* key_lens, int n_keys,
                                                  uint32_t& bh, uint32_t& qt)
{
    const uint32_t per_batch = (uint32_t)heads * (uint32_t)n_qt;
    const int n_batch = (int)(gridDim.x / per_batch);
    const int want = (int)(blockIdx.x / per_batch);
    const uint32_t j = blockIdx.x % per_batch;
    const int lane = threadIdx.x & 63;
    const int mine = lane < n_batch ? min(max(key_lens[lane], 0), n_keys) : -1;
    int rank = 0;
    for (int u = 0; u < n_batch; ++u) {
        const int other = __builtin_amdgcn_readlane(mine, u);
        rank += (other > mine || (other == mine && u < lane)) ? 1 : 0;
    }
    const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < n_batch && rank == want);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit));
    bh = b * (uint32_t)heads + j % (uint32_t)heads;
    qt = j / (uint32_t)heads;
}

// Epilogue: O = O_acc / l in the input type, lse = (m + log2 l) * ln 2.
// EMPTY: rows may have seen no key (masks); such a row has l = 0 and gets
// O = 0 and lse = -inf.
// PADDED: rows are dm elements apart and only dims below dm are written.
template <typename T, int D, int QB, int DB, bool EMPTY, bool PADDED>
__device__ __forceinline__ void store_outputs(const f32x16 (&oacc)[QB][DB], const float (&m_run)[QB],
                                              const float (&l_run)[QB], const int (&qrow)[QB], int n_rows,
                                              T* __restrict__ oh, float* __restrict__ lseh, int hh, int dm)
{
    const int stride = PADDED ? dm : D;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l_tot = swap_halves_sum(l_run[qb]);
        if (qrow[qb] < n_rows) {
            const bool seen = !EMPTY || l_tot > 0.f;
            const float inv = seen ? 1.0f / l_tot : 0.f;
            T* orow = oh + (int64_t)qrow[qb] * stride;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    T vals[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) vals[t] = to_elem<T>(oacc[qb][db][4 * g + t] * inv);
                    u32x2 packed = __builtin_bit_cast(u32x2, vals);
                    const int col = db * 32 + 8 * g + 4 * hh;
                    if (!PADDED || col < dm) *(u32x2*)(orow + col) = packed;
                }
            }
            if (hh == 0) lseh[qrow[qb]] = seen ? (m_run[qb] + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
        }
    }
}

// Epilogue through LDS: each wave writes its 32 normalised rows to its own
// LDS region (rows D + 8 elements apart, 16-byte aligned), then reads them
// back a row per 16 lanes and stores 16 contiguous bytes per lane, so every
// store instruction writes four whole rows instead of 16 bytes of 32 rows.
// The caller has passed a barrier after its last LDS read of K and V.
// EMPTY: rows may have seen no key (masks): O = 0 and lse = -inf there.
// PADDED: rows are dm elements apart in memory and only dims below dm are
// written (dm a multiple of 8, so rows stay 16-byte aligned).
template <typename T, int D, int DB, bool EMPTY, bool PADDED>
__device__ __forceinline__ void store_outputs_staged(const f32x16 (&oacc)[1][DB], const float (&m_run)[1],
                                                     const float (&l_run)[1], const int (&qrow)[1], int row0,
                                                     int n_rows, T* __restrict__ oh, float* __restrict__ lseh,
                                                     int hh, int lane, uint16_t* __restrict__ stage, int dm)
{
    constexpr int RS = D + 8;  // LDS row stride in elements
    const float l_tot = swap_halves_sum(l_run[0]);
    const bool seen = !EMPTY || l_tot > 0.f;
    const float inv = seen ? 1.0f / l_tot : 0.f;
    const int l32 = lane & 31;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            T vals[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) vals[t] = to_elem<T>(oacc[0][db][4 * g + t] * inv);
            *(u32x2*)(stage + l32 * RS + db * 32 + 8 * g + 4 * hh) = __builtin_bit_cast(u32x2, vals);
        }
    }
    constexpr int CPR = D / 8;             // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;          // rows per read instruction
    const int rr = lane / CPR, cc = lane % CPR;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
        const int r = i * RPI + rr;
        const u32x4 x = *(const u32x4*)(stage + r * RS + cc * 8);
        const int stride = PADDED ? dm : D;
        if (row0 + r < n_rows && (!PADDED || cc * 8 < dm)) *(u32x4*)(oh + (int64_t)(row0 + r) * stride + cc * 8) = x;
    }
    if (qrow[0] < n_rows && hh == 0)
        lseh[qrow[0]] = seen ? (m_run[0] + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
}

// SPLIT: the key tiles of a query tile are divided into n_splits contiguous
// chunks, one workgroup each, and every workgroup writes the normalised
// partial output of its chunk (fp32) and the chunk's logsumexp to a
// workspace instead of O and lse; fa_merge_kernel combines them. This is for
// problems with too few query tiles to fill the GPU (KV-cache decode). A
// chunk's partial result is exact for its keys, and the merge is the online
// softmax identity applied once per chunk.
// Partial result of a key chunk: O_chunk = O_acc / l in fp32 and the chunk's
// logsumexp (natural log). A row that sees no key of the chunk gets O = 0
// and lse = -inf, which gives it weight zero in the merge.
template <int D, int QB, int DB>
__device__ __forceinline__ void store_partials(const f32x16 (&oacc)[QB][DB], const float (&m_run)[QB],
                                               const float (&l_run)[QB], const int (&qrow)[QB], int n_rows,
                                               float* __restrict__ ws_o, float* __restrict__ ws_lse, int hh)
{
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l_tot = swap_halves_sum(l_run[qb]);
        if (qrow[qb] < n_rows) {
            const bool seen = l_tot > 0.f;
            const float inv = seen ? 1.0f / l_tot : 0.f;
            float* orow = ws_o + (int64_t)qrow[qb] * D;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    typedef float f32x4 __attribute__((ext_vector_type(4)));
                    f32x4 vals;
#pragma unroll
                    for (int t = 0; t < 4; ++t) vals[t] = oacc[qb][db][4 * g + t] * inv;
                    *(f32x4*)(orow + db * 32 + 8 * g + 4 * hh) = vals;
                }
            }
            if (hh == 0) ws_lse[qrow[qb]] = seen ? (m_run[qb] + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
        }
    }
}

// Merge of the key chunks of a split launch, per query row:
// lse = ln sum_s exp(lse_s), O = sum_s exp(lse_s - lse) O_s. Each thread
// owns 8 consecutive dims of one row; rows are [B*H*Nq] in order. Chunks go
// in groups of 16 whose loads (logsumexps and partial outputs together) are
// all issued before any is used, so a call with up to 16 chunks makes one
// round of memory reads; later groups rescale the running sums to their
// larger maximum (the online-softmax update, once per group).
// The partial rows are D floats apart and hold the DC computed dims (a PADDED
// launch's dims past dm are zero there); O rows are dm elements apart and
// only dims below dm are written.
template <typename T, int D, int DC>
__global__ __launch_bounds__(256) void fa_merge_kernel(const float* __restrict__ ws_o,
                                                       const float* __restrict__ ws_lse, T* __restrict__ o,
                                                       float* __restrict__ lse, int64_t n_rows, int n_splits, int dm)
{
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    constexpr int TPR = DC / 8, G = 16;  // threads per row, chunks per group
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = t / TPR;
    const int c0 = (int)(t % TPR) * 8;
    if (row >= n_rows) return;
    float mx = -INFINITY, wsum = 0.f;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < n_splits; s0 += G) {
        float l[G];
        f32x4 a[G], b[G];
#pragma unroll
        for (int i = 0; i < G; ++i) {
            if (s0 + i < n_splits) {
                const float* src = ws_o + ((int64_t)(s0 + i) * n_rows + row) * D + c0;
                l[i] = ws_lse[(int64_t)(s0 + i) * n_rows + row];
                a[i] = *(const f32x4*)src;
                b[i] = *(const f32x4*)(src + 4);
            } else {
                l[i] = -INFINITY;
                a[i] = b[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
            }
        }
        float gm = mx;
#pragma unroll
        for (int i = 0; i < G; ++i) gm = fmaxf(gm, l[i]);
        if (gm == -INFINITY) continue;  // no chunk so far saw a key of this row
        // rescale what the earlier groups added (weight 0 when there were none)
        const float r = mx == -INFINITY ? 0.f : expf(mx - gm);
        wsum *= r;
        acc0 *= r;
        acc1 *= r;
        mx = gm;
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const float w = expf(l[i] - mx);  // exp(-inf) = 0 for absent or empty chunks
            wsum += w;
            acc0 += w * a[i];
            acc1 += w * b[i];
        }
    }
    const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
    T vals[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        vals[e] = to_elem<T>(acc0[e] * inv);
        vals[4 + e] = to_elem<T>(acc1[e] * inv);
    }
    if (c0 < dm) *(u32x4*)(o + row * dm + c0) = __builtin_bit_cast(u32x4, vals);
    if (c0 == 0) lse[row] = wsum > 0.f ? mx + logf(wsum) : -INFINITY;
}

// MASKS: padding lengths and sliding windows (fa_tiles.h, row_keys). The
// key tiles of a query tile are then [first, end) with a masked prefix (the
// left window edge), an unmasked middle and a masked suffix (diagonal, right
// window edge, padding); each wave computes only the tiles its own rows can
// see, and a row that sees nothing ends with O = 0 and lse = -inf.
// PADDED: the head dim dm (a multiple of 8 below D) is run with D; K/V
// lanes of the missing dims copy nothing and their LDS chunks stay zero, Q
// loads zeros there, and only dm dims of O are written.
template <typename T, int D, bool CAUSAL, int WAVES, int QB, bool SPLIT, bool MASKS, bool PADDED, int DC = D>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WAVES, 64 * WAVES),
                          amdgpu_waves_per_eu(2 / QB, 2 / QB)))
void fa_fwd_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                   T* __restrict__ o, float* __restrict__ lse, int Nq, int Nk, int n_qt, float c_log2,
                   int n_splits, float* __restrict__ ws_o, float* __restrict__ ws_lse, MaskArgs mask, int dm)
{
    typedef Cfg<D, WAVES, QB, DC> C;
    typedef typename Mma<T>::vec8 vec8;
    // kStaged: the epilogue goes through LDS (store_outputs_staged); padded head
    // dims below 64 measured 1% slower with it and keep the direct stores.
    constexpr bool kStaged = QB == 1 && !SPLIT && !(PADDED && D == 64);
    // kQlds: the 8-wave launches without masks, padding or split copy their Q
    // tile into LDS with the same whole-row copies as K and V and read the
    // operand from there, instead of 16-byte register loads from 32 rows.
    constexpr bool kQlds = kStaged && !MASKS && !PADDED && WAVES == 8;
    constexpr int kTilesQ = 4 * C::TILE + (kQlds ? C::BM * D : 0);
    constexpr int kSmem = kStaged && WAVES * 32 * (D + 8) > kTilesQ ? WAVES * 32 * (D + 8) : kTilesQ;
    __shared__ __attribute__((aligned(16))) uint16_t smem[kSmem];

    uint32_t bh, qt, split = 0;
    if (SPLIT) {
        const uint32_t rest = blockIdx.x / (uint32_t)n_splits;
        split = blockIdx.x % (uint32_t)n_splits;
        bh = rest / (uint32_t)n_qt;
        qt = rest % (uint32_t)n_qt;
    } else {
        const bool padded = MASKS && mask.key_lens != nullptr;
        if (!CAUSAL && padded && gridDim.x / ((uint32_t)mask.heads * (uint32_t)n_qt) <= 64)
            padded_batch_tile(n_qt, mask.heads, mask.key_lens, Nk, bh, qt);
        else
            workgroup_tile<CAUSAL>(n_qt, padded, bh, qt);
    }
    const int q0 = (int)qt * C::BM;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    const int dmem = PADDED ? dm : D;  // row length in memory
    const int64_t q_off = (int64_t)bh * Nq * dmem, kv_off = (int64_t)bh * Nk * dmem;
    const T* kh = k + kv_off;
    const T* vh = v + kv_off;
    // The exp2 work of tile j is interleaved with the score MFMAs of tile j+1
    // (scores_with_exp). The 4-wave shape computing 128 dims keeps them apart
    // in its split, masked and padded variants, which run out of registers
    // fused.
    constexpr bool kFuseExp = QB == 1 && fuses_exp(DC, WAVES, SPLIT, MASKS, PADDED);
    // d=64 without masks splits the exp work of a tile in two halves by its
    // 32-key blocks: the second block's goes between the next tile's score
    // MFMAs as above, the first block's between the MFMAs of the previous
    // tile's P.V, so both MFMA blocks carry vector work. The lazy-max test
    // still sees the whole tile before any of its P enters P.V. Measured +3%
    // at B4 H16 N4096 d=64 non-causal, causal unchanged; at d=128 the same
    // split ran 5% slower in every instruction order tried. Computing 96
    // dims, the direct non-causal kernels take it too (+1-1.7% at d = 80 and
    // 96; the causal and split ones spill with it). (With masks a wave can
    // start at a tile whose scores it never computed, which this order would
    // leave unmasked.)
    constexpr bool kSplitExp = kFuseExp && !MASKS && (D == 64 || (DC == 96 && !CAUSAL && !SPLIT));
    // While a wave runs a mixed score/exp block it gets issue priority over the
    // other wave of its SIMD, whose next instructions are then mostly P.V
    // MFMAs: the matrix core keeps taking the mixed block's MFMAs as they come
    // up and the vector work between them runs meanwhile. Measured +2.5% for
    // the 8-wave shapes, +3% for 4-wave d=128 and +1.5% for 4-wave d=64 with
    // the split above; 4-wave d=64 without the split ran 1-2% slower with it.
    constexpr bool kPrioMixed = WAVES == 8 || D == 128 || kSplitExp;
    // Row sums of a tile: d=64 and the kernels computing 96 dims add one
    // partial sum per 32-key block, in element order, and then the blocks (the
    // split above produces them apart); d=128 adds all 64 scores in element
    // order. Every path of a kernel (fused or not, first tile, rescaled tile)
    // uses the same order, so the masked and unmasked kernels of one head dim
    // agree bit for bit.
    constexpr bool kBS = D == 64 || DC == 96;

    int qrow[QB];
    vec8 qf[QB][C::DS];
    if (PADDED)
        load_q_padded<T, D, QB, C::DS>(q + q_off, dm, q0 + wave * QB * 32, Nq, l32, hh, qrow, qf);
    else if (!kQlds)
        load_q<T, D, QB, C::DS>(q + q_off, q0 + wave * QB * 32, Nq, l32, hh, qrow, qf);
    else
        qrow[0] = q0 + wave * 32 + l32;

    // key tiles [t0, t1) of the query tile, of which [u_lo, u_hi) need no mask
    int t0 = 0, t1, u_lo = 0, u_hi;
    int key_len = Nk;
    if (MASKS) {
        if (mask.key_lens) key_len = min(max(mask.key_lens[bh / (uint32_t)mask.heads], 0), Nk);
        const MaskedSpan ms = masked_span(q0, C::BM, C::BN, Nq, Nk, CAUSAL, mask.window_left,
                                          mask.window_right, key_len);
        t0 = (int)ms.first;
        t1 = (int)ms.end;
        u_lo = (int)ms.unmasked_begin;
        u_hi = (int)ms.unmasked_end;
    } else {
        const TileSpan span = tile_span(q0, C::BM, C::BN, Nq, Nk, CAUSAL);
        u_hi = (int)span.unmasked;
        t1 = (int)span.total;
    }
    // key tiles [jb, je) of this workgroup: all of them, or one chunk
    int jb = t0, je = t1;
    if (SPLIT) {
        const int per = (t1 - t0 + n_splits - 1) / n_splits;
        jb = min(t1, t0 + (int)split * per);
        je = min(t1, jb + per);
    }

    f32x16 oacc[QB][C::DB];
    float m_run[QB], l_run[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db) oacc[qb][db] = (f32x16){};
        m_run[qb] = -1e30f;
        l_run[qb] = 0.f;
    }

    // LDS: K tiles in buffers 0/1, V tiles in buffers 2/3. Iteration j reads
    // K_{j+1} (scores of the next tile) and V_j (P.V of this tile) while the
    // copies of K_{j+2} and V_{j+1} are in flight; one barrier per tile.
    auto kbuf = [&](int i) { return smem + (i & 1) * C::TILE; };
    auto vbuf = [&](int i) { return smem + (2 + (i & 1)) * C::TILE; };

    const uint32_t head_bytes = (uint32_t)Nk * (uint32_t)(dmem * 2);
    const rsrc_t krs = head_rsrc(kh, head_bytes), vrs = head_rsrc(vh, head_bytes);
    bool real_chunk = true;
    const uint32_t lane_off = PADDED ? tile_lane_offset_padded<D>(wave, lane, dm, real_chunk)
                                     : tile_lane_offset<D>(wave, lane);
    if (PADDED) zero_pad_chunks<D, WAVES, QB>(smem, 4, dm, tid);
    auto issue = [&](uint16_t* buf, rsrc_t src, int k0) {
        if (PADDED)
            issue_tile_padded<D, WAVES, QB>(buf, src, k0, wave, lane_off, real_chunk, dm);
        else
            issue_tile<D, WAVES, QB>(buf, src, k0, wave, lane_off);
    };
    // Causal: the key tiles this wave's rows can see form the prefix
    // [0, n_wave); in the diagonal tiles past it the wave only helps with the
    // copies and the barriers. In a split launch a wave whose rows all lie
    // past Nq computes nothing either.
    int n_wave = CAUSAL ? min(je, (q0 + (wave + 1) * QB * 32 - 1) / C::BN + 1) : je;
    if (SPLIT && q0 + wave * QB * 32 >= Nq) n_wave = jb;
    // Masks: the wave computes the tiles [w_lo, n_wave) its rows can see, and
    // each lane masks its row's keys outside [row_lo, row_hi). With the exp
    // work fused into the next tile's score MFMAs, scores are only computed
    // by a step that processes a tile, so the wave also takes the tile before
    // its first one: every key there lies below all its rows' ranges, the
    // mask turns whatever its score registers hold into -inf, and the tile
    // adds nothing to m, l or O.
    int w_lo = jb;
    int row_lo[QB], row_hi[QB];
    if (MASKS) {
        const int r0 = q0 + wave * QB * 32;
        if (r0 >= Nq) {
            n_wave = jb;
        } else {
            const MaskedSpan ws = masked_span(r0, QB * 32, C::BN, Nq, Nk, CAUSAL, mask.window_left,
                                              mask.window_right, key_len);
            w_lo = max(jb, (int)ws.first - (kFuseExp ? 1 : 0));
            n_wave = min(je, (int)ws.end);
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const RowKeys rk = row_keys(qrow[qb], Nk, CAUSAL, mask.window_left, mask.window_right, key_len);
            row_lo[qb] = (int)rk.lo;
            row_hi[qb] = (int)rk.hi;
        }
    }
    // G-mode limits: does this wave compute tile t?
    auto wave_sees = [&](int t) { return t < n_wave && (!MASKS || t >= w_lo); };
    auto apply_mask = [&](f32x16 (&sq)[C::KB], int j, int qb) {
        if (MASKS)
            mask_range<C::KB>(sq, j * C::BN, row_lo[qb], row_hi[qb], hh);
        else
            mask_scores<C::KB, CAUSAL>(sq, j * C::BN, qrow[qb], Nk, hh);
    };

    f32x16 sa[QB][C::KB], sb[QB][C::KB];
    // kSplitExp: P of the tile whose scores are in sa / sb (first block
    // filled one step ahead) and the first block's partial row sum
    vec8 pa[QB][C::KT], pb[QB][C::KT];
    float ra = 0.f, rb = 0.f;
    bool premax = false;  // m_run holds tile jb's row max (wave-uniform)
    if (MASKS) {
        // a wave's extra leading tile is masked without its scores having been
        // computed: give the registers a defined value
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb) sa[qb][kb] = sb[qb][kb] = (f32x16){};
    }
    if ((SPLIT || MASKS) && jb == je) {
        // an empty chunk, or a query tile that sees no key
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb) sa[qb][kb] = (f32x16){};
    } else {
        if constexpr (kQlds) {
            const rsrc_t qrs = head_rsrc(q + q_off, (uint32_t)Nq * (uint32_t)(D * 2));
#pragma unroll
            for (int r = 0; r < C::BM; r += C::BN) issue(smem + 4 * C::TILE + r * D, qrs, q0 + r);
        }
        issue(kbuf(jb), krs, jb * C::BN);
        issue(vbuf(jb), vrs, jb * C::BN);
        if (jb + 1 < je) issue(kbuf(jb + 1), krs, (jb + 1) * C::BN);
        stage_barrier();
        if constexpr (kQlds) {
#pragma unroll
            for (int ds = 0; ds < C::DS; ++ds)
                qf[0][ds] = k_operand<vec8, D>(smem + 4 * C::TILE, wave * 32 + l32, ds, hh);
        }
        // every wave processes an unmasked tile of a direct launch
        if ((!SPLIT && (!MASKS || (jb >= u_lo && jb < u_hi))) || wave_sees(jb)) {
            scores<T, D, QB, C::KB, C::DS>(sa, kbuf(jb), qf, l32, hh);
            // The running max starts at the first tile's own row max, so that
            // tile's exponentials are taken once: against the initial -1e30
            // they would fail the lazy-max test and be taken again. (A row
            // that sees none of the tile's keys keeps -1e30.)
            if (MASKS ? (jb < u_lo || jb >= u_hi) : jb >= u_hi) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) apply_mask(sa[qb], jb, qb);
            }
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) m_run[qb] = fmaxf(m_run[qb], row_max_log2<C::KB>(sa[qb], c_log2));
            premax = true;
            if constexpr (kSplitExp) ra = exp_range<T, C::KB, C::KT, 0, 16>(sa[0], m_run[0], c_log2, pa[0]);
        }
        stage_barrier();  // K_jb's buffer is refilled in the first iteration
    }

    // One tile that has a successor: sc holds the scores of tile j; sn
    // receives those of tile j+1.
    auto step = [&](auto masked, int j, f32x16 (&sc)[QB][C::KB], f32x16 (&sn)[QB][C::KB], vec8 (&pc)[QB][C::KT],
                    vec8 (&pn)[QB][C::KT], float& rc, float& rn) {
        // M: the tile gets the mask; G: per-wave limits apply (masked tiles,
        // and every tile of a split launch)
        constexpr bool M = decltype(masked)::value, G = M || SPLIT;
        // K_{j+2} is copied even past the last tile: the copy stays inside the
        // head (the descriptor reads zeros past it) and nothing reads that
        // buffer afterwards, and the step has no branch before its MFMAs.
        issue(kbuf(j), krs, (j + 2) * C::BN);
        issue(vbuf(j + 1), vrs, (j + 1) * C::BN);
        if constexpr (kSplitExp) {
            // sc is masked and its first block's P is in pc (rc): they were
            // made with the previous tile's P.V (or before the loop)
            if (!G || wave_sees(j)) {
                float rs[QB];
                if (!G || wave_sees(j + 1)) {
                    if constexpr (kPrioMixed) __builtin_amdgcn_s_setprio(1);
                    scores_with_exp<T, D, C::KB, C::DS, C::KT, 16, 32, kBS>(sn, kbuf(j + 1), qf, l32, hh, sc,
                                                                            m_run[0], c_log2, pc, rs);
                    order_scores_block<D, WAVES, QB, DC>();
                    pin_regs(pc[0][2]);
                    pin_regs(pc[0][3]);
                    pin_reg(rs[0]);
                    if constexpr (kPrioMixed) __builtin_amdgcn_s_setprio(0);
                } else {
                    rs[0] = exp_range<T, C::KB, C::KT, 16, 32>(sc[0], m_run[0], c_log2, pc[0]);
                }
                rs[0] = rc + rs[0];
                softmax_finish<T, QB, C::KB, C::DB, C::KT, kBS>(sc, oacc, m_run, l_run, c_log2, pc, rs,
                                                                !(premax && j == jb));
                if (!G || wave_sees(j + 1)) {
                    if (M || j + 1 >= u_hi) apply_mask(sn[0], j + 1, 0);
                    pv_with_exp<T, D, C::DB, C::KT, C::KB, 0, 16>(pc, vbuf(j), oacc, lane, hh, sn, m_run[0], c_log2,
                                                                  pn, rn);
                    order_pv_block<D, WAVES, QB, DC>();
                    pin_regs(pn[0][0]);
                    pin_regs(pn[0][1]);
                    pin_reg(rn);
                } else {
                    pv_tile<T, D, QB, C::DB, C::KT>(pc, vbuf(j), oacc, lane, hh);
                    order_pv_block<D, WAVES, QB, DC>();
                }
            }
        } else if constexpr (kFuseExp) {
            if (!G || wave_sees(j)) {
                if (M) apply_mask(sc[0], j, 0);
                vec8 p[QB][C::KT];
                float rs[QB];
                if (!G || wave_sees(j + 1)) {
                    if constexpr (kPrioMixed) __builtin_amdgcn_s_setprio(1);
                    scores_with_exp<T, D, C::KB, C::DS, C::KT, 0, C::KB * 16, kBS>(sn, kbuf(j + 1), qf, l32, hh,
                                                                                   sc, m_run[0], c_log2, p, rs);
                    order_scores_block<D, WAVES, QB, DC>();
                    if constexpr (kPrioMixed) __builtin_amdgcn_s_setprio(0);
                } else {
                    exp_tile<T, QB, C::KB, C::KT, kBS>(sc, m_run, c_log2, p, rs);
                }
                softmax_finish<T, QB, C::KB, C::DB, C::KT, kBS>(sc, oacc, m_run, l_run, c_log2, p, rs,
                                                                !(premax && j == jb));
                pv_tile<T, D, QB, C::DB, C::KT>(p, vbuf(j), oacc, lane, hh);
                order_pv_block<D, WAVES, QB, DC>();
            }
        } else {
            if (!G || wave_sees(j + 1)) {
                scores<T, D, QB, C::KB, C::DS>(sn, kbuf(j + 1), qf, l32, hh);
                order_scores_block<D, WAVES, QB, DC>();
            }
            if (!G || wave_sees(j)) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    if (M) apply_mask(sc[qb], j, qb);
                softmax_pv<T, D, QB, C::KB, C::DB, C::KT, kBS>(sc, vbuf(j), oacc, m_run, l_run, c_log2, lane, hh,
                                                            !(premax && j == jb));
                order_pv_block<D, WAVES, QB, DC>();
            }
        }
        stage_barrier();
    };
    typedef std::integral_constant<bool, false> unmasked_t;
    typedef std::integral_constant<bool, true> masked_t;

    // The last tile has no successor whose scores would be computed, so it
    // runs a step of its own. Before it: a masked prefix [jb, u_lo) (masks
    // only: the left window edge, one step at a time), then tiles up to u_hi
    // that need no mask, then the masked rest; those loops are unrolled by two
    // so the score registers alternate.
    auto last_step = [&](auto masked, int j, f32x16 (&sc)[QB][C::KB], vec8 (&pc)[QB][C::KT], float rc) {
        constexpr bool M = decltype(masked)::value, G = M || SPLIT;
        if constexpr (kSplitExp) {
            if (!G || wave_sees(j)) {
                float rs[QB];
                rs[0] = rc + exp_range<T, C::KB, C::KT, 16, 32>(sc[0], m_run[0], c_log2, pc[0]);
                softmax_finish<T, QB, C::KB, C::DB, C::KT, kBS>(sc, oacc, m_run, l_run, c_log2, pc, rs,
                                                                !(premax && j == jb));
                pv_tile<T, D, QB, C::DB, C::KT>(pc, vbuf(j), oacc, lane, hh);
                order_pv_block<D, WAVES, QB, DC>();
            }
        } else if (!G || wave_sees(j)) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                if (M) apply_mask(sc[qb], j, qb);
            softmax_pv<T, D, QB, C::KB, C::DB, C::KT, kBS>(sc, vbuf(j), oacc, m_run, l_run, c_log2, lane, hh,
                                                            !(premax && j == jb));
            order_pv_block<D, WAVES, QB, DC>();
        }
    };
    auto shift_scores = [&]() {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb) sa[qb][kb] = sb[qb][kb];
            if constexpr (kSplitExp) {
#pragma unroll
                for (int t = 0; t < C::KT; ++t) pa[qb][t] = pb[qb][t];
            }
        }
        ra = rb;
    };
    const int n_lead = je - 1;
    int j = jb;
    if (MASKS) {
        const int a_end = min(u_lo, n_lead);
        for (; j < a_end; ++j) {
            step(masked_t(), j, sa, sb, pa, pb, ra, rb);
            shift_scores();
        }
    }
    const int n_u = min(u_hi, n_lead);
    for (; j + 2 <= n_u; j += 2) {
        step(unmasked_t(), j, sa, sb, pa, pb, ra, rb);
        step(unmasked_t(), j + 1, sb, sa, pb, pa, rb, ra);
    }
    if (j < n_u) {
        step(unmasked_t(), j, sa, sb, pa, pb, ra, rb);
        ++j;
        shift_scores();
    }
    for (; j + 2 <= n_lead; j += 2) {
        step(masked_t(), j, sa, sb, pa, pb, ra, rb);
        step(masked_t(), j + 1, sb, sa, pb, pa, rb, ra);
    }
    if (j < n_lead) {
        step(masked_t(), j, sa, sb, pa, pb, ra, rb);
        ++j;
        shift_scores();
    }
    if (j < je) {
        if (j >= u_lo && j < u_hi)
            last_step(unmasked_t(), j, sa, pa, ra);
        else
            last_step(masked_t(), j, sa, pa, ra);
    }

    if (SPLIT) {
        const int64_t slot = ((int64_t)split * (gridDim.x / ((uint32_t)n_splits * (uint32_t)n_qt)) + bh) * Nq;
        store_partials<D, QB, C::DB>(oacc, m_run, l_run, qrow, Nq, ws_o + slot * D, ws_lse + slot, hh);
    } else if constexpr (kStaged) {
        __syncthreads();  // every wave is past its last read of K and V
        store_outputs_staged<T, D, C::DB, MASKS, PADDED>(oacc, m_run, l_run, qrow, q0 + wave * 32, Nq, o + q_off,
                                                         lse + (int64_t)bh * Nq, hh, lane, smem + wave * 32 * (D + 8),
                                                         dm);
    } else {
        store_outputs<T, D, QB, C::DB, MASKS, PADDED>(oacc, m_run, l_run, qrow, Nq, o + q_off,
                                                      lse + (int64_t)bh * Nq, hh, dm);
    }
}

template <typename T, int D, bool CAUSAL, int WAVES, int QB, bool MASKS, bool PADDED, int DC>
hipError_t launch_one(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                      int Nq, int Nk, float scale, const MaskArgs& mask, int dm, hipStream_t stream)
{
    typedef Cfg<D, WAVES, QB> C;
    const int n_qt = (Nq + C::BM - 1) / C::BM;
    const float c_log2 = scale * 1.4426950408889634f;
    dim3 grid((unsigned)((int64_t)n_qt * BH)), block(C::THREADS);
    hipLaunchKernelGGL((fa_fwd_kernel<T, D, CAUSAL, WAVES, QB, false, MASKS, PADDED, DC>), grid, block, 0, stream,
                       (const T*)q, (const T*)k, (const T*)v, (T*)o, lse, Nq, Nk, n_qt, c_log2, 1,
                       (float*)nullptr, (float*)nullptr, mask, dm);
    return hipGetLastError();
}

// Split launch (4-wave, 128-row workgroups) followed by the merge; the
// workspace holds n_splits * B*H*Nq partial rows of D floats and then as many
// logsumexps.
template <typename T, int D, bool CAUSAL, bool MASKS, bool PADDED, int DC>
hipError_t launch_split(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                        int Nq, int Nk, float scale, int n_splits, float* ws, const MaskArgs& mask,
                        int dm, hipStream_t stream)
{
    typedef Cfg<D, 4, 1> C;
    const int n_qt = (Nq + C::BM - 1) / C::BM;
    const float c_log2 = scale * 1.4426950408889634f;
    const int64_t n_rows = (int64_t)BH * Nq;
    float* ws_o = ws;
    float* ws_lse = ws + (int64_t)n_splits * n_rows * D;
    dim3 grid((unsigned)((int64_t)n_qt * BH * n_splits)), block(C::THREADS);
    hipLaunchKernelGGL((fa_fwd_kernel<T, D, CAUSAL, 4, 1, true, MASKS, PADDED, DC>), grid, block, 0, stream,
                       (const T*)q, (const T*)k, (const T*)v, (T*)o, lse, Nq, Nk, n_qt, c_log2, n_splits,
                       ws_o, ws_lse, mask, dm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t threads = n_rows * (DC / 8);
    dim3 mgrid((unsigned)((threads + 255) / 256)), mblock(256);
    hipLaunchKernelGGL((fa_merge_kernel<T, D, DC>), mgrid, mblock, 0, stream, (const float*)ws_o,
                       (const float*)ws_lse, (T*)o, lse, n_rows, n_splits, PADDED ? dm : D);
    return hipGetLastError();
}

template <typename T, int D, bool CAUSAL, bool MASKS, bool PADDED, int DC>
hipError_t launch_shape(const Shape& sh, const void* q, const void* k, const void* v, void* o,
                        float* lse, int BH, int Nq, int Nk, float scale, const MaskArgs& mask, int dm,
                        hipStream_t stream)
{
    // 8 waves for non-causal problems only (pick_shape), and never for masked
    // d=128: that kernel has no registers left for the per-row key ranges
    if constexpr (!CAUSAL && !(MASKS && D == 128)) {
        if (sh.waves == 8)
            return launch_one<T, D, CAUSAL, 8, 1, MASKS, PADDED, DC>(q, k, v, o, lse, BH, Nq, Nk, scale, mask, dm,
                                                                 stream);
    }
    return launch_one<T, D, CAUSAL, 4, 1, MASKS, PADDED, DC>(q, k, v, o, lse, BH, Nq, Nk, scale, mask, dm, stream);
}

template <typename T>
struct TypeTag {
    typedef T type;
};

// One forward launch of the MASKS / PADDED variant: dispatch on dtype, the
// kernel head dim, the computed dims and causality, then the direct or the
// split launch. A PADDED launch computes compute_dim(d) dims (d rounded up to
// 32): at d = 96 three quarters of the d = 128 kernel's MFMAs, at d <= 32
// half of the d = 64 kernel's.
template <bool MASKS, bool PADDED>
hipError_t launch_variant(const FwdArgs& a)
{
    const int BH = a.B * a.H;
    auto go = [&](auto t, auto dd, auto dc, auto cc) -> hipError_t {
        typedef typename decltype(t)::type T;
        constexpr int D = decltype(dd)::value, DC = decltype(dc)::value;
        constexpr bool CAUSAL = decltype(cc)::value;
        if (a.split)
            return launch_split<T, D, CAUSAL, MASKS, PADDED, DC>(a.q, a.k, a.v, a.o, a.lse, BH, a.Nq, a.Nk,
                                                                 a.scale, a.n_splits, a.workspace, a.mask, a.d,
                                                                 a.stream);
        const Shape sh = MASKS ? pick_shape_masked(a.B, a.H, a.Nq, a.d, a.causal)
                               : pick_shape(a.B, a.H, a.Nq, a.d, a.causal);
        return launch_shape<T, D, CAUSAL, MASKS, PADDED, DC>(sh, a.q, a.k, a.v, a.o, a.lse, BH, a.Nq, a.Nk,
                                                             a.scale, a.mask, a.d, a.stream);
    };
    auto by_compute = [&](auto t, auto dd, auto cc) -> hipError_t {
        constexpr int D = decltype(dd)::value;
        if constexpr (PADDED) {
            if (compute_dim(a.d) < D) return go(t, dd, std::integral_constant<int, D - 32>(), cc);
        }
        return go(t, dd, dd, cc);
    };
    auto by_causal = [&](auto t, auto dd) -> hipError_t {
        return a.causal ? by_compute(t, dd, std::true_type()) : by_compute(t, dd, std::false_type());
    };
    auto by_dim = [&](auto t) -> hipError_t {
        return kernel_dim(a.d) == 64 ? by_causal(t, std::integral_constant<int, 64>())
                                     : by_causal(t, std::integral_constant<int, 128>());
    };
    return a.bf16 ? by_dim(TypeTag<__bf16>()) : by_dim(TypeTag<_Float16>());
}

}  // namespace
}  // namespace fa

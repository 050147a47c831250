// fa_bwd_kernel.h -- attention backward (FlashAttention-2 form) for gfx950.
//
// The gradient of sum(dO * O) for O = softmax(scale * Q K^T [+ causal]) V,
// using the logsumexp L the forward wrote: "How to optimise a Triton
// FlashAttention-2 kernel step by step with a profiler" names this pass as the
// next kernel (closing list), a kernel that needs that L and accumulates in
// two directions. With P_ij = exp(scale * <q_i, k_j> - L_i):
//
//   D_i  = <dO_i, O_i>                (fa_bwd_delta_kernel)
//   dV_j = sum_i P_ij dO_i,  dK_j = scale * sum_i dS_ij q_i,
//          dS_ij = P_ij (<dO_i, v_j> - D_i)          (fa_bwd_dkdv_kernel)
//   dQ_i = scale * sum_j dS_ij k_j                    (fa_bwd_dq_kernel)
//
// The two accumulation directions get a kernel each, so nothing is summed
// with atomics and the results are deterministic; P and dS are recomputed in
// both. Both kernels reuse the forward's gfx950 layouts:
//   * dK/dV: a workgroup of 8 waves owns 256 keys (32 per wave) with K in
//     registers in B-operand layout and V rows in LDS, and streams 64-row
//     tiles of Q and dO (plus L and D) through LDS, shared by the 8 waves. S = Q K^T is computed with queries on the M axis and keys
//     on N, so each lane holds 16 queries of ONE key; P and dS then serve
//     directly as the B operands of dV^T += dO^T P and dK^T += Q^T dS, whose
//     A operands are transposed reads (ds_read_b64_tr_b16) of the row-major
//     dO and Q tiles, as V^T is read in the forward.
//   * dQ: a workgroup owns 128 query rows (32 per wave) with Q and dO in
//     registers, and streams 64-key tiles of K and V. S^T = K Q^T and
//     dP^T = V dO^T put one query per lane (the forward's score layout), and
//     dQ^T += K^T dS^T reads K^T transposed from the K tile.
//   * Causal: the dK/dV kernel starts at the first query tile that sees its
//     keys and masks only the diagonal tiles; the dQ kernel visits the
//     forward's key-tile range (Round 4, "Causal tile-skipping"). Waves skip
//     query or key blocks that lie wholly above the diagonal for their rows.
//   * N_q query rows against N_k keys, with the forward's top-left causal
//     rule (key j visible to row i iff j <= i): query-side tensors (q, dO, O,
//     L, D, dQ) have N_q rows per head, key-side ones (K, V, dK, dV) N_k.
//   * MASKS: the forward's padding lengths and sliding windows (fa_tiles.h,
//     row_keys). The rows that see key j form one interval [i_min(j),
//     i_max(j)]; a dK/dV workgroup visits only the query tiles whose rows see
//     one of its keys and masks P per element, and the dQ kernel takes the
//     forward's masked key-tile ranges. A row that sees no key (lse = -inf,
//     O = 0) gets P = 0 everywhere, so it adds nothing.
//   * PADDED: a head dim dm below the kernel's D (a multiple of 8), run as the
//     forward's padded launches: rows are dm elements apart in memory, the
//     copies of the missing dims are skipped and their LDS chunks hold zeros
//     written once, register loads of them are zero, and stores write the
//     first dm columns only. Zero dims add nothing to any dot product, so the
//     result is the d = dm gradient.
// The kernels are instantiated by fa_bwd_kernel.hip (D = 64, 128) and
// fa_bwd_hdim.hip (PADDED).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_launch.h"
#include "fa_tiles.h"

namespace fa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// D_i = <dO_i, O_i> in fp32; TPR = D/8 consecutive threads share a row of dm
// elements (dm <= D, a multiple of 8; chunks past dm count zero).
template <typename T, int D>
__global__ __launch_bounds__(256) void fa_bwd_delta_kernel(const T* __restrict__ o, const T* __restrict__ dout,
                                                           float* __restrict__ delta, int64_t n_rows, int dm)
{
    constexpr int TPR = D / 8;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = t / TPR;
    const int c0 = (int)(t % TPR) * 8;
    float acc = 0.f;
    if (row < n_rows && c0 < dm) {
        const u32x4 a = *(const u32x4*)(o + row * dm + c0);
        const u32x4 b = *(const u32x4*)(dout + row * dm + c0);
        typedef T t8 __attribute__((ext_vector_type(8)));
        const t8 av = __builtin_bit_cast(t8, a), bv = __builtin_bit_cast(t8, b);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += (float)av[e] * (float)bv[e];
    }
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (row < n_rows && (t % TPR) == 0) delta[row] = acc;
}

// Rows of a 32 x (32*DB) accumulator block set, lane = row (l % 32), register
// r = column 32*db + 8*(r/4) + 4*hh + (r%4): times `mul`, rounded, stored in
// rows dm elements apart. PADDED: only columns below dm (a multiple of 8, so
// a group of 4 lies wholly below or wholly past it).
template <typename T, int D, int DB, bool PADDED>
__device__ __forceinline__ void store_rows(const f32x16 (&acc)[DB], float mul, int row, int n_rows,
                                           T* __restrict__ out, int hh, int dm)
{
    if (row >= n_rows) return;
    T* orow = out + (int64_t)row * (PADDED ? dm : D);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            if (PADDED && db * 32 + 8 * g + 4 * hh >= dm) continue;
            T vals[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) vals[t] = to_elem<T>(acc[db][4 * g + t] * mul);
            *(u32x2*)(orow + db * 32 + 8 * g + 4 * hh) = __builtin_bit_cast(u32x2, vals);
        }
    }
}

// blockIdx -> (b*H + h, tile) with the forward's rules: head-major and
// XCD-contiguous without causality; tile-major, most work first, with it
// (reverse = the tile index whose work is largest comes first).
template <bool CAUSAL>
__device__ __forceinline__ void bwd_tile(int n_tiles, bool low_first, uint32_t& bh, uint32_t& tile)
{
    const uint32_t nwg = gridDim.x, hw = blockIdx.x;
    if (CAUSAL) {
        const uint32_t n_bh = nwg / (uint32_t)n_tiles;
        bh = hw % n_bh;
        const uint32_t r = hw / n_bh;
        tile = low_first ? r : (uint32_t)n_tiles - 1 - r;
    } else {
        const uint32_t xcd = hw % kXcds, slot = hw / kXcds;
        const uint32_t per = nwg / kXcds, extra = nwg % kXcds;
        const uint32_t logical = xcd < extra ? xcd * (per + 1) + slot
                                             : extra * (per + 1) + (xcd - extra) * per + slot;
        bh = logical / (uint32_t)n_tiles;
        tile = logical % (uint32_t)n_tiles;
    }
}

// ---------------------------------------------------------------- dK, dV
constexpr int kBwdWaves = 8;                // waves per dK/dV workgroup
constexpr int kBwdKeys = 32 * kBwdWaves;     // keys per dK/dV workgroup (32 per wave)
constexpr int kBwdRows = 64;                 // query rows per streamed tile

// Rows that see key j under the masks: i_min(j) <= i <= i_max(j), none when
// j is past the batch's key count (fa_tiles.h, row_keys, read per key).
struct KeyRows {
    int64_t first, last;  // empty when first > last
};

__device__ __forceinline__ KeyRows key_rows(int64_t j, bool causal, const MaskArgs& m, int64_t key_len)
{
    KeyRows r;
    r.first = causal ? j : (m.window_right >= 0 ? j - m.window_right : 0);
    if (r.first < 0) r.first = 0;
    r.last = m.window_left >= 0 ? j + m.window_left : INT64_MAX / 4;
    if (j >= key_len) r.last = r.first - 1;
    return r;
}

template <typename T, int D, bool CAUSAL, bool MASKS, bool PADDED, int DC = D>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kBwdWaves, 64 * kBwdWaves),
                          amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dkdv_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                        const T* __restrict__ dout, const float* __restrict__ lse,
                        const float* __restrict__ delta, T* __restrict__ dk, T* __restrict__ dv, int Nq,
                        int Nk, int n_kt, float scale, float c_log2, MaskArgs mask, int dm)
{
    typedef Cfg<D, kBwdWaves, 1, DC> C;  // 64-row copies by the whole workgroup, as the forward's tiles
    typedef typename Mma<T>::vec8 vec8;
    static_assert(C::BN == kBwdRows, "tile rows");
    constexpr int TILE = C::TILE;
    // per buffer: Q tile, dO tile (TILE elements each), L and D (64 floats each);
    // then the workgroup's V rows (kBwdKeys of them), read as B operands
    constexpr int BUF = 2 * TILE + 2 * kBwdRows * 2;  // in 2-byte units
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * BUF + (kBwdKeys / kBwdRows) * TILE];
    uint16_t* const vtile = smem + 2 * BUF;

    uint32_t bh, kt;
    bwd_tile<CAUSAL || MASKS>(n_kt, true, bh, kt);
    const int k0 = (int)kt * kBwdKeys;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    const int rs = PADDED ? dm : D;  // elements between rows in memory
    const int64_t q_off = (int64_t)bh * Nq * rs, kv_off = (int64_t)bh * Nk * rs;
    const int kw0 = k0 + 32 * wave;  // this wave's first key

    // K rows of this wave's keys in B-operand layout (rows >= Nk zero); V rows
    // go to LDS once and are read per MFMA (registers hold two waves per SIMD)
    int krow[1];
    vec8 kf[1][C::DS];
    if (PADDED)
        load_q_padded<T, D, 1, C::DS>(k + kv_off, dm, kw0, Nk, l32, hh, krow, kf);
    else
        load_q<T, D, 1, C::DS>(k + kv_off, kw0, Nk, l32, hh, krow, kf);

    f32x16 dk_acc[1][C::DB], dv_acc[1][C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) dk_acc[0][db] = dv_acc[0][db] = (f32x16){};

    const uint32_t q_bytes = (uint32_t)Nq * (rs * 2), row_bytes = (uint32_t)Nq * 4;
    const rsrc_t qrs = head_rsrc(q + q_off, q_bytes), drs = head_rsrc(dout + q_off, q_bytes);
    const rsrc_t lrs = head_rsrc(lse + (int64_t)bh * Nq, row_bytes);
    const rsrc_t ers = head_rsrc(delta + (int64_t)bh * Nq, row_bytes);
    bool real_chunk = true;
    const uint32_t lane_off =
        PADDED ? tile_lane_offset_padded<D>(wave, lane, dm, real_chunk) : tile_lane_offset<D>(wave, lane);
    auto copy_tile = [&](uint16_t* buf, rsrc_t src, int row0) {
        if (PADDED)
            issue_tile_padded<D, kBwdWaves, 1>(buf, src, row0, wave, lane_off, real_chunk, dm);
        else
            issue_tile<D, kBwdWaves, 1>(buf, src, row0, wave, lane_off);
    };
    const rsrc_t vrs = head_rsrc(v + kv_off, (uint32_t)Nk * (rs * 2));
#pragma unroll
    for (int i = 0; i < kBwdKeys / kBwdRows; ++i) copy_tile(vtile + i * TILE, vrs, k0 + i * kBwdRows);
    if (PADDED) {  // the dims past dm of the V rows and of both Q/dO buffers
        zero_pad_chunks<D, kBwdWaves, 1>(vtile, kBwdKeys / kBwdRows, dm, tid);
        zero_pad_chunks<D, kBwdWaves, 1>(smem, 2, dm, tid);
        zero_pad_chunks<D, kBwdWaves, 1>(smem + BUF, 2, dm, tid);
    }
    auto qbuf = [&](int i) { return smem + (i & 1) * BUF; };
    auto dbuf = [&](int i) { return smem + (i & 1) * BUF + TILE; };
    auto lbuf = [&](int i) { return (float*)(smem + (i & 1) * BUF + 2 * TILE); };
    auto ebuf = [&](int i) { return (float*)(smem + (i & 1) * BUF + 2 * TILE) + kBwdRows; };
    auto issue = [&](int t) {
        copy_tile(qbuf(t), qrs, t * kBwdRows);
        copy_tile(dbuf(t), drs, t * kBwdRows);
        if (wave == 0 && lane < 16) {  // 64 floats of L and of D: 16 lanes x 16 bytes
            copy16_to_lds(lrs, (uint16_t*)lbuf(t), (uint32_t)lane * 16, (uint32_t)t * kBwdRows * 4);
            copy16_to_lds(ers, (uint16_t*)ebuf(t), (uint32_t)lane * 16, (uint32_t)t * kBwdRows * 4);
        }
    };

    int n_qt = (Nq + kBwdRows - 1) / kBwdRows;
    // no earlier query row sees these keys; with fewer queries than keys a
    // causal key block can lie past every row (its gradients are zero)
    int t_begin = CAUSAL ? k0 / kBwdRows : 0;
    // masks: the rows that see a key of this block, and this lane's key's rows
    int key_len = Nk;
    int64_t my_first = 0, my_last = INT64_MAX / 4;
    if (MASKS) {
        if (mask.key_lens) key_len = min(max(mask.key_lens[bh / (uint32_t)mask.heads], 0), Nk);
        const int k1 = min(k0 + kBwdKeys, key_len);  // one past the block's last real key
        if (k1 <= k0) {
            n_qt = t_begin = 0;  // padding only: no row sees these keys
        } else {
            const KeyRows a = key_rows(k0, CAUSAL, mask, key_len), z = key_rows(k1 - 1, CAUSAL, mask, key_len);
            t_begin = (int)(a.first / kBwdRows);
            const int64_t r_end = min((int64_t)Nq, z.last + 1);
            n_qt = r_end > a.first ? (int)((r_end + kBwdRows - 1) / kBwdRows) : t_begin;
        }
        const KeyRows mine = key_rows(kw0 + l32, CAUSAL, mask, key_len);
        my_first = mine.first;
        my_last = mine.last;
    }
    // this wave's keys: the rows that see one of them (masks)
    int64_t wave_first = 0, wave_last = INT64_MAX / 4;
    if (MASKS) {
        const int kl = min(kw0 + 31, key_len - 1);
        if (kl < kw0) {
            wave_last = -1;  // all of this wave's keys are padding
        } else {
            wave_first = key_rows(kw0, CAUSAL, mask, key_len).first;
            wave_last = key_rows(kl, CAUSAL, mask, key_len).last;
        }
    }
    if (t_begin < n_qt) issue(t_begin);
    stage_barrier();
    for (int t = t_begin; t < n_qt; ++t) {
        if (t + 1 < n_qt) issue(t + 1);
        const uint16_t* qs = qbuf(t);
        const uint16_t* ds = dbuf(t);
        const float* ls = lbuf(t);
        const float* es = ebuf(t);
#pragma unroll
        for (int qb = 0; qb < kBwdRows / 32; ++qb) {
            const int qbase = t * kBwdRows + qb * 32;  // first query row of this block
            if (!MASKS && CAUSAL && qbase + 31 < kw0) continue;  // every query of the block precedes every key
            if (MASKS && (qbase + 31 < wave_first || qbase > wave_last)) continue;  // no row sees these keys
            // S = Q K^T and dP = dO V^T: queries on M, this wave's keys on N
            f32x16 s = (f32x16){}, dp = (f32x16){};
            const int row = qb * 32 + l32, vrow = 32 * wave + l32;
#pragma unroll
            for (int dsx = 0; dsx < C::DS; ++dsx) {
                const int chunk = ((2 * dsx + hh) ^ swz<D>(row)) * 8;
                const vec8 aq = as_vec8<vec8>(*(const u32x4*)(qs + row * D + chunk));
                const vec8 ad = as_vec8<vec8>(*(const u32x4*)(ds + row * D + chunk));
                const vec8 bv = as_vec8<vec8>(
                    *(const u32x4*)(vtile + vrow * D + ((2 * dsx + hh) ^ swz<D>(vrow)) * 8));
                s = Mma<T>::run(aq, kf[0][dsx], s);
                dp = Mma<T>::run(ad, bv, dp);
            }
            // register r holds query qb*32 + 8*(r/4) + 4*hh + (r%4) of the tile
            vec8 pk[2], dsk[2];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                typedef float f32x4 __attribute__((ext_vector_type(4)));
                const f32x4 lq = *(const f32x4*)(ls + qb * 32 + 8 * g + 4 * hh);
                const f32x4 dq = *(const f32x4*)(es + qb * 32 + 8 * g + 4 * hh);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g + e;
                    float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c_log2, -lq[e] * kLog2e));
                    const int qi = qbase + 8 * g + 4 * hh + e;
                    if (MASKS) {
                        if (qi < my_first || qi > my_last) p = 0.f;
                    } else if (CAUSAL && kw0 + l32 > qi) {
                        p = 0.f;
                    }
                    const float dsv = p * (dp[r] - dq[e]);
                    pk[r >> 3][r & 7] = to_elem<T>(p);
                    dsk[r >> 3][r & 7] = to_elem<T>(dsv);
                }
            }
            // dV^T += dO^T P and dK^T += Q^T dS (transposed tile reads)
            const vec8 p1[1][2] = {{pk[0], pk[1]}};
            const vec8 d1[1][2] = {{dsk[0], dsk[1]}};
            pv_tile<T, D, 1, C::DB, 2>(p1, ds + qb * 32 * D, dv_acc, lane, hh);
            pv_tile<T, D, 1, C::DB, 2>(d1, qs + qb * 32 * D, dk_acc, lane, hh);
            // keep the two query blocks apart: interleaved they need more
            // registers than two waves per SIMD have
            __builtin_amdgcn_sched_barrier(0);
        }
        stage_barrier();
    }
    store_rows<T, D, C::DB, PADDED>(dk_acc[0], scale, kw0 + l32, Nk, dk + kv_off, hh, dm);
    store_rows<T, D, C::DB, PADDED>(dv_acc[0], 1.0f, kw0 + l32, Nk, dv + kv_off, hh, dm);
}

// ---------------------------------------------------------------- dQ
template <typename T, int D, bool CAUSAL, bool MASKS, bool PADDED, int DC = D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dq_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                      const T* __restrict__ dout, const float* __restrict__ lse,
                      const float* __restrict__ delta, T* __restrict__ dq, int Nq, int Nk, int n_qt,
                      float scale, float c_log2, MaskArgs mask, int dm)
{
    typedef Cfg<D, 4, 1, DC> C;  // 128 query rows, 64-key tiles
    typedef typename Mma<T>::vec8 vec8;
    __shared__ __attribute__((aligned(16))) uint16_t smem[4 * C::TILE];

    uint32_t bh, qt;
    bwd_tile<CAUSAL || MASKS>(n_qt, false, bh, qt);
    const int q0 = (int)qt * C::BM;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    const int rs = PADDED ? dm : D;  // elements between rows in memory
    const int64_t q_off = (int64_t)bh * Nq * rs, kv_off = (int64_t)bh * Nk * rs;

    int qrow[1];
    vec8 qf[1][C::DS], df[1][C::DS];
    if (PADDED) {
        load_q_padded<T, D, 1, C::DS>(q + q_off, dm, q0 + wave * 32, Nq, l32, hh, qrow, qf);
        load_q_padded<T, D, 1, C::DS>(dout + q_off, dm, q0 + wave * 32, Nq, l32, hh, qrow, df);
    } else {
        load_q<T, D, 1, C::DS>(q + q_off, q0 + wave * 32, Nq, l32, hh, qrow, qf);
        load_q<T, D, 1, C::DS>(dout + q_off, q0 + wave * 32, Nq, l32, hh, qrow, df);
    }
    const bool row_ok = qrow[0] < Nq;
    float l2 = row_ok ? lse[(int64_t)bh * Nq + qrow[0]] * kLog2e : 0.f;
    // a row that saw no key (masks) has lse = -inf and every score masked:
    // any finite value gives P = 0 instead of -inf - (-inf)
    if (MASKS && !(l2 > -INFINITY)) l2 = 0.f;
    const float dd = row_ok ? delta[(int64_t)bh * Nq + qrow[0]] : 0.f;

    f32x16 dq_acc[1][C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) dq_acc[0][db] = (f32x16){};

    // key tiles [t0, t1), of which [u_lo, u_hi) need no mask (the forward's split)
    int t0 = 0, t1, u_lo = 0, u_hi, w_lo = 0, n_wave;
    int row_lo = 0, row_hi = 0, key_len = Nk;
    if (MASKS) {
        if (mask.key_lens) key_len = min(max(mask.key_lens[bh / (uint32_t)mask.heads], 0), Nk);
        const MaskedSpan ms = masked_span(q0, C::BM, C::BN, Nq, Nk, CAUSAL, mask.window_left,
                                          mask.window_right, key_len);
        t0 = (int)ms.first;
        t1 = (int)ms.end;
        u_lo = (int)ms.unmasked_begin;
        u_hi = (int)ms.unmasked_end;
        const int r0 = q0 + wave * 32;
        if (r0 >= Nq) {
            w_lo = n_wave = t0;
        } else {
            const MaskedSpan ws = masked_span(r0, 32, C::BN, Nq, Nk, CAUSAL, mask.window_left, mask.window_right,
                                              key_len);
            w_lo = max(t0, (int)ws.first);
            n_wave = min(t1, (int)ws.end);
        }
        const RowKeys rk = row_keys(qrow[0], Nk, CAUSAL, mask.window_left, mask.window_right, key_len);
        row_lo = (int)rk.lo;
        row_hi = (int)rk.hi;
    } else {
        const TileSpan span = tile_span(q0, C::BM, C::BN, Nq, Nk, CAUSAL);
        u_hi = (int)span.unmasked;
        t1 = (int)span.total;
        n_wave = CAUSAL ? min(t1, (q0 + (wave + 1) * 32 - 1) / C::BN + 1) : t1;
    }

    auto kbuf = [&](int i) { return smem + (i & 1) * C::TILE; };
    auto vbuf = [&](int i) { return smem + (2 + (i & 1)) * C::TILE; };
    const uint32_t head_bytes = (uint32_t)Nk * (rs * 2);
    const rsrc_t krs = head_rsrc(k + kv_off, head_bytes), vrs = head_rsrc(v + kv_off, head_bytes);
    bool real_chunk = true;
    const uint32_t lane_off =
        PADDED ? tile_lane_offset_padded<D>(wave, lane, dm, real_chunk) : tile_lane_offset<D>(wave, lane);
    auto copy_tile = [&](uint16_t* buf, rsrc_t src, int row0) {
        if (PADDED)
            issue_tile_padded<D, 4, 1>(buf, src, row0, wave, lane_off, real_chunk, dm);
        else
            issue_tile<D, 4, 1>(buf, src, row0, wave, lane_off);
    };
    if (PADDED) zero_pad_chunks<D, 4, 1>(smem, 4, dm, tid);  // both K and both V buffers
    if (t0 < t1) {
        copy_tile(kbuf(t0), krs, t0 * C::BN);
        copy_tile(vbuf(t0), vrs, t0 * C::BN);
    }
    stage_barrier();
    for (int j = t0; j < t1; ++j) {
        if (j + 1 < t1) {
            copy_tile(kbuf(j + 1), krs, (j + 1) * C::BN);
            copy_tile(vbuf(j + 1), vrs, (j + 1) * C::BN);
        }
        if (j < n_wave && j >= w_lo) {
            f32x16 s[1][C::KB], dp[1][C::KB];
            scores<T, D, 1, C::KB, C::DS>(s, kbuf(j), qf, l32, hh);
            scores<T, D, 1, C::KB, C::DS>(dp, vbuf(j), df, l32, hh);
            if (j < u_lo || j >= u_hi) {
                if (MASKS)
                    mask_range<C::KB>(s[0], j * C::BN, row_lo, row_hi, hh);
                else
                    mask_scores<C::KB, CAUSAL>(s[0], j * C::BN, qrow[0], Nk, hh);
            }
            vec8 dsk[1][C::KT];
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[0][kb][r], c_log2, -l2));
                    dsk[0][kb * 2 + (r >> 3)][r & 7] = to_elem<T>(p * (dp[0][kb][r] - dd));
                }
            }
            pv_tile<T, D, 1, C::DB, C::KT>(dsk, kbuf(j), dq_acc, lane, hh);
        }
        stage_barrier();
    }
    store_rows<T, D, C::DB, PADDED>(dq_acc[0], scale, qrow[0], Nq, dq + q_off, hh, dm);
}

// The three kernels for head dim dm (dm == D, or a multiple of 8 below D when
// PADDED), computing DC dims.
template <typename T, int D, bool CAUSAL, bool MASKS, bool PADDED, int DC>
hipError_t launch_bwd_typed(const void* q, const void* k, const void* v, const void* o, const void* dout,
                            const float* lse, void* dq, void* dk, void* dv, float* delta, int BH, int Nq,
                            int Nk, int dm, float scale, const MaskArgs& mask, hipStream_t stream)
{
    const int64_t n_rows = (int64_t)BH * Nq;
    const float c_log2 = scale * kLog2e;
    dim3 g0((unsigned)((n_rows * (D / 8) + 255) / 256)), b0(256);
    hipLaunchKernelGGL((fa_bwd_delta_kernel<T, D>), g0, b0, 0, stream, (const T*)o, (const T*)dout, delta,
                       n_rows, dm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n_kt = (Nk + kBwdKeys - 1) / kBwdKeys;
    dim3 g1((unsigned)((int64_t)n_kt * BH)), b1(64 * kBwdWaves);
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<T, D, CAUSAL, MASKS, PADDED, DC>), g1, b1, 0, stream, (const T*)q,
                       (const T*)k, (const T*)v, (const T*)dout, lse, (const float*)delta, (T*)dk, (T*)dv, Nq,
                       Nk, n_kt, scale, c_log2, mask, dm);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n_qt = (Nq + 127) / 128;
    dim3 g2((unsigned)((int64_t)n_qt * BH)), b2(256);
    hipLaunchKernelGGL((fa_bwd_dq_kernel<T, D, CAUSAL, MASKS, PADDED, DC>), g2, b2, 0, stream, (const T*)q,
                       (const T*)k, (const T*)v, (const T*)dout, lse, (const float*)delta, (T*)dq, Nq, Nk, n_qt,
                       scale, c_log2, mask, dm);
    return hipGetLastError();
}

template <typename T>
struct BwdType {
    typedef T type;
};

// Every (element type, kernel head dim, computed dims, causal, masks) instance
// for one PADDED value; d picks the kernel head dim (kernel_dim) and, PADDED,
// the computed dims (compute_dim: d rounded up to 32).
template <bool PADDED>
hipError_t launch_bwd_variant(const void* q, const void* k, const void* v, const void* o, const void* dout,
                              const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int H,
                              int Nq, int Nk, int d, bool causal, float scale, bool bf16, const MaskArgs* mask,
                              hipStream_t stream)
{
    const int BH = B * H;
    const MaskArgs none{-1, -1, nullptr, H};
    auto go = [&](auto t, auto dd, auto dc, auto cc, auto mm) -> hipError_t {
        typedef typename decltype(t)::type T;
        constexpr int D = decltype(dd)::value, DC = decltype(dc)::value;
        constexpr bool CAUSAL = decltype(cc)::value, MASKS = decltype(mm)::value;
        return launch_bwd_typed<T, D, CAUSAL, MASKS, PADDED, DC>(q, k, v, o, dout, lse, dq, dk, dv, delta, BH,
                                                                 Nq, Nk, d, scale, MASKS ? *mask : none, stream);
    };
    auto by_masks = [&](auto t, auto dd, auto dc, auto cc) -> hipError_t {
        return mask ? go(t, dd, dc, cc, std::true_type()) : go(t, dd, dc, cc, std::false_type());
    };
    auto by_causal = [&](auto t, auto dd, auto dc) -> hipError_t {
        return causal ? by_masks(t, dd, dc, std::true_type()) : by_masks(t, dd, dc, std::false_type());
    };
    auto by_compute = [&](auto t, auto dd) -> hipError_t {
        constexpr int D = decltype(dd)::value;
        if constexpr (PADDED) {
            if (compute_dim(d) < D) return by_causal(t, dd, std::integral_constant<int, D - 32>());
        }
        return by_causal(t, dd, dd);
    };
    auto by_dim = [&](auto t) -> hipError_t {
        return kernel_dim(d) == 64 ? by_compute(t, std::integral_constant<int, 64>())
                                   : by_compute(t, std::integral_constant<int, 128>());
    };
    return bf16 ? by_dim(BwdType<__bf16>()) : by_dim(BwdType<_Float16>());
}

}  // namespace
}  // namespace fa

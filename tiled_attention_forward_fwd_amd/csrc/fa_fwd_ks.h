// fa_fwd_ks.h -- the attention forward for small grids: a workgroup's four
// waves share one block of 32 query rows and split its key tiles four ways.
//
// The direct launch gives each wave 32 query rows and all their keys, so a
// problem with few query tiles (B*H*ceil(Nq/128) well below the 256 CUs) runs
// on a fraction of the chip and each wave walks every key tile in turn. The
// split-key launch shortens that walk but writes fp32 partials of every row
// and merges them in a second launch. Here the four waves of a workgroup take
// the same 32 rows and a contiguous quarter of the key tiles each, run the
// online softmax of "Programming an attention kernel in Triton" over their
// own tiles, and combine their (m, l, O) in LDS at the end with the same
// identity the split launch's merge applies (O = sum_w 2^(m_w - M) O_w /
// sum_w 2^(m_w - M) l_w, M the largest m_w): one launch, no HBM partials.
//
//  * Tiles are 32 keys; each wave streams its own tiles through its own K
//    and V buffers in LDS (the LDS DMA copies and swizzled layout of the
//    direct kernel), so waves never wait for each other before the merge.
//    Computing 128 dims, a wave issues the next tile's scores before this
//    tile's softmax (ks_pipelined).
//  * S^T = K Q^T, the lazy-max online softmax and O^T += V^T P^T are the
//    direct kernel's device code at one 32-key block per tile.
//  * Causal (top-left: row i sees keys j <= i) and ragged key counts mask the
//    tiles past the 32-row block's unmasked span, as in the direct kernel.
//  * PADDED: a head dim dm below the tile layout's D, the missing dims held at
//    zero in LDS and registers and only DC = dm rounded up to 32 computed.
#pragma once

#include "fa_fwd_kernel.h"

namespace fa {
namespace {

constexpr int kKsWaves = 4;  // waves per workgroup, one key quarter each
constexpr int kKsRows = 32;  // query rows per workgroup
constexpr int kKsKeys = 32;  // keys per per-wave K or V tile

// HBM -> LDS copy of keys [k0, k0 + 32) of one K or V head by one wave: copy
// i fills LDS chunks [64 i, 64 i + 64) of the tile, lane l the chunk 64 i + l,
// fetching the global chunk the swizzle places there (rows are row_bytes
// apart in memory). PADDED: chunks of the dims at or past dm are not copied
// (they hold zeros, ks_zero_pad).
template <int D, bool PADDED>
__device__ __forceinline__ void ks_copy_tile(uint16_t* buf, rsrc_t src, int k0, int lane, uint32_t row_bytes,
                                             int dm)
{
    constexpr int CPR = D / 8, COPIES = kKsKeys * CPR / 64;
#pragma unroll
    for (int i = 0; i < COPIES; ++i) {
        const int c = i * 64 + lane, r = c / CPR, lc = (c % CPR) ^ swz<D>(r);
        if (!PADDED || lc < dm / 8)
            copy16_to_lds(src, buf + i * 64 * 8, (uint32_t)r * row_bytes + (uint32_t)lc * 16,
                          (uint32_t)k0 * row_bytes);
    }
}

// Zeros the chunks of the dims at or past dm in n consecutive tiles of one
// wave (their swizzled positions are the same in every tile).
template <int D>
__device__ __forceinline__ void ks_zero_pad(uint16_t* buf0, int n, int lane, int dm)
{
    constexpr int CPR = D / 8;
    for (int c = lane; c < kKsKeys * CPR; c += 64) {
        const int r = c / CPR, lc = (c % CPR) ^ swz<D>(r);
        if (lc >= dm / 8)
            for (int t = 0; t < n; ++t) *(u32x4*)(buf0 + t * kKsKeys * D + c * 8) = (u32x4){0u, 0u, 0u, 0u};
    }
}

// Whether the kernel computing DC dims issues the next tile's scores before
// this tile's softmax (three K buffers). With 128 dims a workgroup's LDS
// fills a CU and its waves run one per SIMD, and the overlap within the wave
// measured 6-12% faster; with two waves per SIMD (64 dims and fewer) it was
// 2-5% slower, and computing 96 dims 2%.
constexpr bool ks_pipelined(int DC) { return DC == 128; }

// LDS of the key-split kernel, in 2-byte units: per wave two (three when
// pipelined) K and two V tiles; the merge then reuses the same memory for
// every wave's fp32 partial O (DB blocks of 16 registers x 64 lanes) and its
// 32 row maxima and sums.
template <int D, int DC>
constexpr int ks_lds_elems()
{
    constexpr int tiles = kKsWaves * (ks_pipelined(DC) ? 5 : 4) * kKsKeys * D;
    constexpr int merge = 2 * kKsWaves * ((DC / 32) * 16 * 64 + 2 * kKsRows);
    return tiles > merge ? tiles : merge;
}

template <typename T, int D, bool CAUSAL, bool PADDED, int DC>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kKsWaves, 64 * kKsWaves),
                          amdgpu_waves_per_eu(D == 128 ? 1 : 2, 2)))
void fa_fwd_ks_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                      T* __restrict__ o, float* __restrict__ lse, int Nq, int Nk, int n_qb, float c_log2, int dm)
{
    typedef Cfg<D, kKsWaves, 1, DC> C;  // DS and DB (its 64-key BN is not used here)
    typedef typename Mma<T>::vec8 vec8;
    constexpr int TILE = kKsKeys * D;  // elements of one 32-key tile
    __shared__ __attribute__((aligned(16))) uint16_t smem[ks_lds_elems<D, DC>()];

    uint32_t bh, qb;
    workgroup_tile<CAUSAL>(n_qb, false, bh, qb);
    const int q0 = (int)qb * kKsRows;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    const int dmem = PADDED ? dm : D;  // row length in memory
    const int64_t q_off = (int64_t)bh * Nq * dmem, kv_off = (int64_t)bh * Nk * dmem;

    int qrow[1];
    vec8 qf[1][C::DS];
    if (PADDED)
        load_q_padded<T, D, 1, C::DS>(q + q_off, dm, q0, Nq, l32, hh, qrow, qf);
    else
        load_q<T, D, 1, C::DS>(q + q_off, q0, Nq, l32, hh, qrow, qf);

    // the block's key tiles [0, n_t), of which [0, u_hi) need no mask; this
    // wave's share is the contiguous range [jb, je)
    const TileSpan span = tile_span(q0, kKsRows, kKsKeys, Nq, Nk, CAUSAL);
    const int u_hi = (int)span.unmasked, n_t = (int)span.total;
    const int per = (n_t + kKsWaves - 1) / kKsWaves;
    const int jb = min(n_t, wave * per), je = min(n_t, jb + per);

    constexpr bool kPipe = ks_pipelined(DC);
    constexpr int kKBufs = kPipe ? 3 : 2;
    uint16_t* const kb = smem + wave * (kKBufs + 2) * TILE;  // K buffers
    uint16_t* const vb = kb + kKBufs * TILE;                  // V buffers 0, 1
    const uint32_t row_bytes = (uint32_t)dmem * 2;
    const uint32_t head_bytes = (uint32_t)Nk * row_bytes;
    const rsrc_t krs = head_rsrc(k + kv_off, head_bytes), vrs = head_rsrc(v + kv_off, head_bytes);
    if (PADDED) ks_zero_pad<D>(kb, kKBufs + 2, lane, dm);

    f32x16 oacc[1][C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) oacc[0][db] = (f32x16){};
    float m_run[1] = {-1e30f}, l_run[1] = {0.f};

    // Tile j's K sits in K buffer (j - jb) % kKBufs and its V in V buffer
    // (j - jb) % 2. Each wave waits only for its own copies.
    auto kbuf = [&](int j) { return kb + ((j - jb) % kKBufs) * TILE; };
    auto vbuf = [&](int j) { return vb + ((j - jb) & 1) * TILE; };
    auto tile_scores = [&](f32x16 (&s)[1][1], int j) {
        scores<T, D, 1, 1, C::DS>(s, kbuf(j), qf, l32, hh);
        if (j >= u_hi) mask_scores<1, CAUSAL>(s[0], j * kKsKeys, qrow[0], Nk, hh);
    };
    if constexpr (kPipe) {
        // Step j computes the scores of tile j + 1 first and then the
        // softmax and P.V of tile j, so that the wave's exponentials run while
        // its score MFMAs are in flight; the copies of K_{j+2} and V_{j+1} are
        // issued at its start, after the wait for K_{j+1} and V_j.
        f32x16 sc[1][1];
        if (jb < je) {
            ks_copy_tile<D, PADDED>(kbuf(jb), krs, jb * kKsKeys, lane, row_bytes, dm);
            ks_copy_tile<D, PADDED>(vbuf(jb), vrs, jb * kKsKeys, lane, row_bytes, dm);
            if (jb + 1 < je) ks_copy_tile<D, PADDED>(kbuf(jb + 1), krs, (jb + 1) * kKsKeys, lane, row_bytes, dm);
            __builtin_amdgcn_s_waitcnt(0);
            asm volatile("" ::: "memory");
            tile_scores(sc, jb);
            // the first tile starts the running max at its own row max, so
            // its exponentials are taken once (no lazy-max check needed)
            m_run[0] = fmaxf(m_run[0], row_max_log2<1>(sc[0], c_log2));
        }
        for (int j = jb; j < je; ++j) {
            // K_{j+1} and V_j have landed; the buffers the next copies fill
            // were last read by the scores and the P.V of tile j - 1
            __builtin_amdgcn_s_waitcnt(0);
            asm volatile("" ::: "memory");
            if (j + 2 < je) ks_copy_tile<D, PADDED>(kbuf(j + 2), krs, (j + 2) * kKsKeys, lane, row_bytes, dm);
            if (j + 1 < je) ks_copy_tile<D, PADDED>(vbuf(j + 1), vrs, (j + 1) * kKsKeys, lane, row_bytes, dm);
            f32x16 sn[1][1];
            if (j + 1 < je) tile_scores(sn, j + 1);
            softmax_pv<T, D, 1, 1, C::DB, 2, false>(sc, vbuf(j), oacc, m_run, l_run, c_log2, lane, hh, j != jb);
            if (j + 1 < je) sc[0][0] = sn[0][0];
        }
    } else {
        if (jb < je) {
            ks_copy_tile<D, PADDED>(kbuf(jb), krs, jb * kKsKeys, lane, row_bytes, dm);
            ks_copy_tile<D, PADDED>(vbuf(jb), vrs, jb * kKsKeys, lane, row_bytes, dm);
        }
        for (int j = jb; j < je; ++j) {
            // tile j has landed (and the zeroed chunks are written); the
            // other buffers were last read by tile j - 1, whose reads have
            // completed
            __builtin_amdgcn_s_waitcnt(0);
            asm volatile("" ::: "memory");
            if (j + 1 < je) {
                ks_copy_tile<D, PADDED>(kbuf(j + 1), krs, (j + 1) * kKsKeys, lane, row_bytes, dm);
                ks_copy_tile<D, PADDED>(vbuf(j + 1), vrs, (j + 1) * kKsKeys, lane, row_bytes, dm);
            }
            f32x16 s[1][1];
            tile_scores(s, j);
            // the wave's first tile starts the running max at its own row
            // max, so its exponentials are taken once (no lazy-max check)
            if (j == jb) m_run[0] = fmaxf(m_run[0], row_max_log2<1>(s[0], c_log2));
            softmax_pv<T, D, 1, 1, C::DB, 2, false>(s, vbuf(j), oacc, m_run, l_run, c_log2, lane, hh, j != jb);
        }
    }

    // merge: every wave's partial O (its accumulator layout), row max m (log2
    // units) and row sum l go to LDS; wave w < DB then combines dim block w
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    float* const mo = (float*)smem;                         // [wave][db][r][lane]
    float* const mm = mo + kKsWaves * C::DB * 16 * 64;      // [wave][row] m
    float* const ml = mm + kKsWaves * kKsRows;              // [wave][row] l
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) mo[((wave * C::DB + db) * 16 + r) * 64 + lane] = oacc[0][db][r];
    const float l_tot = swap_halves_sum(l_run[0]);
    if (hh == 0) {
        mm[wave * kKsRows + l32] = m_run[0];
        ml[wave * kKsRows + l32] = l_tot;
    }
    __syncthreads();
    if (wave < C::DB) {
        const int db = wave;
        float mw[kKsWaves], big = -INFINITY;
#pragma unroll
        for (int w = 0; w < kKsWaves; ++w) {
            mw[w] = mm[w * kKsRows + l32];
            big = fmaxf(big, mw[w]);
        }
        float wt[kKsWaves], l_all = 0.f;
#pragma unroll
        for (int w = 0; w < kKsWaves; ++w) {
            wt[w] = __builtin_amdgcn_exp2f(mw[w] - big);  // 0 for a wave without keys (m = -1e30)
            l_all += wt[w] * ml[w * kKsRows + l32];
        }
        const float inv = 1.0f / l_all;
        if (qrow[0] < Nq) {
            T* orow = o + q_off + (int64_t)qrow[0] * dmem;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                T vals[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int r = 4 * g + t;
                    float acc = 0.f;
#pragma unroll
                    for (int w = 0; w < kKsWaves; ++w) acc += wt[w] * mo[((w * C::DB + db) * 16 + r) * 64 + lane];
                    vals[t] = to_elem<T>(acc * inv);
                }
                const int col = db * 32 + 8 * g + 4 * hh;
                if (!PADDED || col < dm) *(u32x2*)(orow + col) = __builtin_bit_cast(u32x2, vals);
            }
            if (db == 0 && hh == 0)
                lse[(int64_t)bh * Nq + qrow[0]] = (big + log2f(l_all)) * 0.69314718055994531f;
        }
    }
}

template <typename T, int D, bool CAUSAL, bool PADDED, int DC>
hipError_t launch_ks_typed(const FwdArgs& a)
{
    const int n_qb = (a.Nq + kKsRows - 1) / kKsRows;
    const float c_log2 = a.scale * 1.4426950408889634f;
    dim3 grid((unsigned)((int64_t)n_qb * a.B * a.H)), block(64 * kKsWaves);
    hipLaunchKernelGGL((fa_fwd_ks_kernel<T, D, CAUSAL, PADDED, DC>), grid, block, 0, a.stream, (const T*)a.q,
                       (const T*)a.k, (const T*)a.v, (T*)a.o, a.lse, a.Nq, a.Nk, n_qb, c_log2, a.d);
    return hipGetLastError();
}

}  // namespace
}  // namespace fa

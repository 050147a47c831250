// fa_device.h -- device building blocks shared by the attention kernels
// (forward and backward): MFMA wrappers, the LDS tile layout and its copies,
// the score and transposed-operand MFMA loops and their ordering hints. The
// layouts are described where they are defined and in the forward kernel's
// header comment. Included by the kernel sources only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;

template <typename T>
struct Mma;

template <>
struct Mma<__bf16> {
    typedef bf16x8 vec8;
    static __device__ __forceinline__ f32x16 run(vec8 a, vec8 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <>
struct Mma<_Float16> {
    typedef f16x8 vec8;
    static __device__ __forceinline__ f32x16 run(vec8 a, vec8 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

constexpr int kXcds = 8;  // XCDs of an MI355X

// Tile shape: head dim D, WAVES waves per workgroup, QB 32-row query blocks
// per wave, BN = 64 keys per K/V tile. DC: the dims the MFMAs cover, a
// multiple of 32 up to D; a head dim below D is padded with zeros to D in LDS
// (the layout and swizzle of D) but computed only up to DC, so the score
// k-steps and O^T blocks past it are never issued.
template <int D, int WAVES, int QB, int DC = D>
struct Cfg {
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(DC % 32 == 0 && DC >= 32 && DC <= D, "compute dims");
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int BM = 32 * QB * WAVES;    // query rows per workgroup
    static constexpr int BN = 64;                 // keys per tile
    static constexpr int CPR = D / 8;             // 16-byte chunks per row
    static constexpr int TILE = BN * D;           // elements of one K or V tile (dense)
    static constexpr int LDS_BYTES = 4 * TILE * 2;  // two K and two V tile buffers
    static constexpr int KB = BN / 32;            // 32-key blocks per tile
    static constexpr int DS = DC / 16;            // MFMA k-steps of S^T = K Q^T
    static constexpr int DB = DC / 32;            // 32-row blocks of O^T
    static constexpr int KT = BN / 16;            // MFMA k-steps of O^T += V^T P^T
    static constexpr int LOADS = BN * CPR / THREADS;  // 16-byte copies per thread, each of K and V
    static_assert(LOADS * THREADS == BN * CPR, "tile split");
    // rows between a lane's consecutive copies keep the swizzle (period 16)
    static_assert((64 * WAVES / CPR) % 16 == 0 || LOADS == 1, "copy stride");
};

// Chunk swizzle: 16-byte chunk c of tile row r is stored at chunk c ^ swz(r).
// The LDS has 64 four-byte banks; a 16-byte read is served 16 lanes at a
// time, an 8-byte read 32 lanes at a time.
//  * K operand (ds_read_b128): 16 consecutive rows read one logical chunk;
//    swz is a bijection on r mod 16 (d=128) or maps the 8 even and the 8 odd
//    rows (the two bank halves of a 128-byte row pair, d=64) to distinct
//    chunks, so the 16 lanes hit 16 distinct bank quads.
//  * V operand (ds_read_b64_tr_b16): a half-wave reads rows 4a..4a+3 at
//    logical chunks {4b, 4b+1} (lanes 0-15) and {4b+2, 4b+3} (lanes 16-31);
//    swz changes bits 2-3 between those rows and leaves bit 1 alone, so the
//    two lane groups fall in disjoint halves of the 64 banks.
// swz has period 16 in r (tile_lane_offset relies on it).
template <int D>
__device__ __forceinline__ int swz(int row)
{
    if (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
    const int m = (row >> 1) & 7;
    return ((m & 1) << 2) | ((m >> 1) & 3);
}

__device__ __forceinline__ float swap_halves_max(float x)
{
    // v_permlane32_swap exchanges lanes 0-31 of one operand with lanes 32-63
    // of the other; with both operands = x, the pair holds x[lane] and
    // x[lane ^ 32] in some order, which is all a symmetric reduction needs.
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float swap_halves_sum(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <typename V8>
__device__ __forceinline__ V8 as_vec8(u32x4 x)
{
    return __builtin_bit_cast(V8, x);
}

// K/V tiles are copied with the buffer form of the LDS DMA: a descriptor
// covering one head (base, size in bytes), a wave-uniform byte offset and one
// per-lane byte offset. Bytes at or past the head's size read as zero, so a
// ragged last tile is zero-filled and no copy can leave its head.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRawBufferWord3 = 0x00020000;  // raw (untyped) buffer, 32-bit data format

__device__ __forceinline__ rsrc_t head_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRawBufferWord3);
}

// 16 bytes per lane into LDS at lds_base + 16 * lane (lds_base wave-uniform).
// The builtin exists only in the device pass.
__device__ __forceinline__ void copy16_to_lds(rsrc_t r, uint16_t* lds_base, uint32_t lane_off,
                                              uint32_t tile_off)
{
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds_base, 16, lane_off, tile_off, 0, 0);
#endif
}

// HBM -> LDS copy of rows [k0, k0 + BN) of one K or V head. Wave w, copy i
// fills 64 consecutive LDS chunks; lane l fetches the global chunk that the
// swizzle places there. Copy i is 64*WAVES/CPR rows below copy 0, a multiple
// of the swizzle period, so every copy of a lane is one per-lane byte offset
// plus a wave-uniform k0 * D * 2 + i * WAVES * 64 * 16.
template <int D>
__device__ __forceinline__ uint32_t tile_lane_offset(int wave, int lane)
{
    const int c = wave * 64 + lane;
    const int r0 = c / (D / 8), pc = c % (D / 8);
    return (uint32_t)(r0 * D * 2 + (pc ^ swz<D>(r0)) * 16);
}

template <int D, int WAVES, int QB>
__device__ __forceinline__ void issue_tile(uint16_t* buf, rsrc_t src, int k0, int wave,
                                           uint32_t lane_off)
{
    typedef Cfg<D, WAVES, QB> C;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i)
        copy16_to_lds(src, buf + (i * WAVES + wave) * 64 * 8, lane_off,
                      (uint32_t)k0 * (D * 2) + i * (WAVES * 64 * 16));
}

// Waits for this thread's outstanding LDS copies and LDS reads, then for the
// whole workgroup.
__device__ __forceinline__ void stage_barrier()
{
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
}

template <typename T>
__device__ __forceinline__ T to_elem(float x);
template <>
__device__ __forceinline__ __bf16 to_elem<__bf16>(float x) { return (__bf16)x; }
template <>
__device__ __forceinline__ _Float16 to_elem<_Float16>(float x) { return (_Float16)x; }

// The K operand of S^T = K Q^T: key `row` of the tile, the 8 dims of
// k-step ds that lane half hh holds (one ds_read_b128).
template <typename V8, int D>
__device__ __forceinline__ V8 k_operand(const uint16_t* __restrict__ ks, int row, int ds, int hh)
{
    return as_vec8<V8>(*(const u32x4*)(ks + row * D + (((2 * ds + hh) ^ swz<D>(row)) * 8)));
}

// The V^T operand of O^T += V^T P^T for k-step t and dim block db (two
// transposed reads). Lane l = 16g + i: dim 32*db + (l % 32); elements 0..3
// are keys 16t + 4h + [0,4), elements 4..7 keys 16t + 8 + 4h + [0,4)
// (h = g/2), the key order of P^T. Each transposed read has lane i address
// key (base + i/4), dims 4*(i%4) + [0,4) of the group's 16 dims.
template <typename V8, int D>
__device__ __forceinline__ V8 vt_operand(const uint16_t* __restrict__ vts, int t, int db, int lane, int hh)
{
    const int gi = lane & 15, g1 = (lane >> 4) & 1;
    const int half = (gi & 1) * 4;
    const int key0 = 16 * t + 4 * hh + (gi >> 2);
    const int key1 = key0 + 8;
    const int chunk = 4 * db + 2 * g1 + ((gi & 3) >> 1);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(vts + key0 * D + ((chunk ^ swz<D>(key0)) * 8) + half));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(vts + key1 * D + ((chunk ^ swz<D>(key1)) * 8) + half));
    u32x4 w;
    w[0] = __builtin_bit_cast(u32x2, lo)[0];
    w[1] = __builtin_bit_cast(u32x2, lo)[1];
    w[2] = __builtin_bit_cast(u32x2, hi)[0];
    w[3] = __builtin_bit_cast(u32x2, hi)[1];
    return as_vec8<V8>(w);
}

// S^T = K Q^T for one key tile: s[qb][kb] holds keys 32*kb + (accumulator
// rows) of this lane's query in block qb. Each K operand read feeds QB MFMAs.
template <typename T, int D, int QB, int KB, int DS>
__device__ __forceinline__ void scores(f32x16 (&s)[QB][KB], const uint16_t* __restrict__ ks,
                                       const typename Mma<T>::vec8 (&qf)[QB][DS], int l32, int hh)
{
    typedef typename Mma<T>::vec8 vec8;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = (f32x16){};
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const vec8 a = k_operand<vec8, D>(ks, kb * 32 + l32, ds, hh);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[qb][kb] = Mma<T>::run(a, qf[qb][ds], s[qb][kb]);
        }
    }
}

// Row-sum update with two exponentials of a row. bf16: the fp32 values, in
// order. fp16: one v_dot2_f32_f16 of the rounded pair (the values the P.V
// product uses); fp16 rounding changes each term by at most 2^-11 of itself,
// so l and the logsumexp move by at most 2^-11 relative / 4.9e-4 absolute.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
template <typename T>
__device__ __forceinline__ float pair_sum(float acc, float x0, float x1, T, T)
{
    return (acc + x0) + x1;
}
template <>
__device__ __forceinline__ float pair_sum<_Float16>(float acc, float, float, _Float16 h0, _Float16 h1)
{
    const f16x2 v = {h0, h1}, one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(v, one, acc, false);
}

// exp2 / row-sum / convert of the score pair (e, e + 1) of one query row (e
// even; element e of the tile is accumulator block e / 16, row e % 16), into
// the P^T operand vector that holds it.
template <typename T, int KB, int KT>
__device__ __forceinline__ void exp_pair(const f32x16 (&s)[KB], int e, float m, float c_log2,
                                         typename Mma<T>::vec8 (&p)[KT], float& acc)
{
    const int eb = e >> 4, r = e & 15;  // r even: r and r + 1 share a P vector
    const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[eb][r], c_log2, -m));
    const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[eb][r + 1], c_log2, -m));
    const T h0 = to_elem<T>(x0), h1 = to_elem<T>(x1);
    p[eb * 2 + (r >> 3)][r & 7] = h0;
    p[eb * 2 + (r >> 3)][(r & 7) + 1] = h1;
    acc = pair_sum<T>(acc, x0, x1, h0, h1);
}

// Pairs [E0/2, E1/2) of a tile's scores spread evenly over N_MFMA slots;
// slot i gets the pairs [i*n/N_MFMA, (i+1)*n/N_MFMA).
// BS (block sums): the row sum goes into one partial sum per 32-key block
// (acc[e / 16]), each added in element order, and a tile's row sum is
// acc[0] + acc[1] + ...; otherwise every element goes into acc[0] in order.
template <typename T, int KB, int KT, int E0, int E1, int N_MFMA, bool BS>
__device__ __forceinline__ void exp_slot(int i, const f32x16 (&s)[KB], float m, float c_log2,
                                         typename Mma<T>::vec8 (&p)[KT], float (&acc)[KB])
{
    constexpr int n = (E1 - E0) / 2;
    static_assert(E0 % 2 == 0 && E1 % 2 == 0, "pairs");
#pragma unroll
    for (int q = i * n / N_MFMA; q < (i + 1) * n / N_MFMA; ++q)
        exp_pair<T, KB, KT>(s, E0 + 2 * q, m, c_log2, p, acc[BS ? (E0 + 2 * q) >> 4 : 0]);
}

template <int KB>
__device__ __forceinline__ float block_sums(const float (&acc)[KB])
{
    float r = acc[0];
#pragma unroll
    for (int kb = 1; kb < KB; ++kb) r += acc[kb];
    return r;
}

// The scores of the next tile fused with the exp2 work of this one: after
// each score MFMA come the exp2 / row-sum / convert of a few elements of the
// current tile (those in [E0, E1)), so the vector units work while the
// matrix core runs instead of after it (the two streams are independent).
// One 32-row block (QB = 1).
template <typename T, int D, int KB, int DS, int KT, int E0, int E1, bool BS>
__device__ __forceinline__ void scores_with_exp(f32x16 (&sn)[1][KB], const uint16_t* __restrict__ ks,
                                                const typename Mma<T>::vec8 (&qf)[1][DS], int l32, int hh,
                                                const f32x16 (&sc)[1][KB], float m, float c_log2,
                                                typename Mma<T>::vec8 (&p)[1][KT], float (&rs)[1])
{
    typedef typename Mma<T>::vec8 vec8;
    constexpr int n_mfma = KB * DS;
    constexpr int b0 = BS ? E0 >> 4 : 0, b1 = BS ? (E1 + 15) >> 4 : 1;  // partial sums in use
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sn[0][kb] = (f32x16){};
    float acc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) acc[kb] = 0.f;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const vec8 a = k_operand<vec8, D>(ks, kb * 32 + l32, ds, hh);
            sn[0][kb] = Mma<T>::run(a, qf[0][ds], sn[0][kb]);
            exp_slot<T, KB, KT, E0, E1, n_mfma, BS>(ds * KB + kb, sc[0], m, c_log2, p[0], acc);
        }
    }
    float r = acc[b0];
#pragma unroll
    for (int kb = b0 + 1; kb < b1; ++kb) r += acc[kb];
    rs[0] = r;
}

// exp2 work on the elements [E0, E1) of one tile without MFMAs between (a
// range within one 32-key block).
template <typename T, int KB, int KT, int E0, int E1>
__device__ __forceinline__ float exp_range(const f32x16 (&s)[KB], float m, float c_log2,
                                           typename Mma<T>::vec8 (&p)[KT])
{
    static_assert(E0 >> 4 == (E1 - 1) >> 4, "one block");
    float acc = 0.f;
#pragma unroll
    for (int e = E0; e < E1; e += 2) exp_pair<T, KB, KT>(s, e, m, c_log2, p, acc);
    return acc;
}

// Diagonal / ragged tiles: keys past N, and for causal attention keys after
// the lane's query, get score -inf.
template <int KB, bool CAUSAL>
__device__ __forceinline__ void mask_scores(f32x16 (&s)[KB], int k0, int qrow, int n_keys, int hh)
{
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool hide = key >= n_keys || (CAUSAL && key > qrow);
            if (hide) s[kb][r] = -INFINITY;
        }
    }
}

// Mask of a tile under padding and window masks: the lane's query row sees
// the keys [lo, hi) only (fa_tiles.h, row_keys).
template <int KB>
__device__ __forceinline__ void mask_range(f32x16 (&s)[KB], int k0, int lo, int hi, int hh)
{
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (key < lo || key >= hi) s[kb][r] = -INFINITY;
        }
    }
}

// Row max of one block of scores in log2 units (both lane halves of a row).
template <int KB>
__device__ __forceinline__ float row_max_log2(const f32x16 (&s)[KB], float c_log2)
{
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    return swap_halves_max(mx) * c_log2;
}

// P = 2^(s * c - m) of one tile, rounded to the input type after the fp32
// value has been added to the lane's partial row sum (Round 4, "The P cast").
template <typename T, int QB, int KB, int KT, bool BS>
__device__ __forceinline__ void exp_tile(const f32x16 (&s)[QB][KB], const float (&m_run)[QB], float c_log2,
                                         typename Mma<T>::vec8 (&p)[QB][KT], float (&rs)[QB])
{
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        float acc[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            acc[kb] = 0.f;
#pragma unroll
            for (int r = 0; r < 16; r += 2)
                exp_pair<T, KB, KT>(s[qb], kb * 16 + r, m_run[qb], c_log2, p[qb], acc[BS ? kb : 0]);
        }
        rs[qb] = BS ? block_sums<KB>(acc) : acc[0];
    }
}

// Online softmax with a lazily updated max. The exponentials of a tile are
// taken against the running max m of the earlier tiles; the row max of the
// tile itself is only needed when that makes some P large. The test is on the
// lane's partial row sum rs (32 of the tile's 64 keys), which bounds every P
// of the lane. The tile is accepted as it is while
//   * rs <= 2^12: P <= 2^12 is far inside the fp16/bf16 range, the
//     accumulators cannot overflow, and O / l and m + log2(l) are unchanged
//     because O and l carry the same factor; and
//   * rs <= 4 l, l the lane's running sum of the earlier tiles: no key of the
//     tile then carries more than 4/5 of the lane's sum so far. A key that
//     outweighs the rest of its row is accepted only while it sits at the
//     running max, where its P is 1 and rounds to the input type exactly; at
//     P = 2^k (0 < k <= 12) its rounding (up to 2^-8 of itself for bf16)
//     would move a row dominated by it by up to one output ulp.
// Otherwise (on the first tile, where m is still the initial -1e30, when the
// scores grew by more than about 2^12 over m, and when a tile's keys outweigh
// the row so far) the wave takes the true row max, rescales O and l by
// alpha = 2^(m_old - m_new) and recomputes the tile's P (the update of
// "Programming an attention kernel in Triton", online softmax). The branch is
// wave-uniform. A caller that set m to the first tile's own row max before
// its exponentials passes check = false for that tile: every P is then at
// most 1, the largest exactly 1, and neither rule can ask for a refresh.
// On iid N(0,1) inputs the second rule adds almost no refresh beyond that.
constexpr float kLaneSumBound = 4096.0f;
constexpr float kLaneSumGrowth = 4.0f;

template <typename T, int QB, int KB, int DB, int KT, bool BS>
__device__ __forceinline__ void softmax_finish(const f32x16 (&s)[QB][KB], f32x16 (&o)[QB][DB],
                                               float (&m_run)[QB], float (&l_run)[QB], float c_log2,
                                               typename Mma<T>::vec8 (&p)[QB][KT], float (&rs)[QB],
                                               bool check = true)
{
    bool bad = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
        bad = bad || !(rs[qb] <= kLaneSumBound) || rs[qb] > kLaneSumGrowth * l_run[qb];
    if (check && __builtin_amdgcn_ballot_w64(bad)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float mx = row_max_log2<KB>(s[qb], c_log2);
            const float m_new = fmaxf(m_run[qb], mx);
            const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
            m_run[qb] = m_new;
            l_run[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) o[qb][db] *= alpha;
        }
        exp_tile<T, QB, KB, KT, BS>(s, m_run, c_log2, p, rs);
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l_run[qb] += rs[qb];
}

template <typename T, int QB, int KB, int DB, int KT, bool BS>
__device__ __forceinline__ void softmax_tile(const f32x16 (&s)[QB][KB], f32x16 (&o)[QB][DB],
                                             float (&m_run)[QB], float (&l_run)[QB], float c_log2,
                                             typename Mma<T>::vec8 (&p)[QB][KT], bool check = true)
{
    float rs[QB];
    exp_tile<T, QB, KB, KT, BS>(s, m_run, c_log2, p, rs);
    softmax_finish<T, QB, KB, DB, KT, BS>(s, o, m_run, l_run, c_log2, p, rs, check);
}

// O^T += V^T P^T (operand layout at vt_operand). Each V operand feeds QB
// MFMAs; the t-major order consumes P in the order it is produced.
template <typename T, int D, int QB, int DB, int KT>
__device__ __forceinline__ void pv_tile(const typename Mma<T>::vec8 (&p)[QB][KT],
                                        const uint16_t* __restrict__ vts, f32x16 (&o)[QB][DB], int lane,
                                        int hh)
{
    typedef typename Mma<T>::vec8 vec8;
#pragma unroll
    for (int t = 0; t < KT; ++t) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const vec8 a = vt_operand<vec8, D>(vts, t, db, lane, hh);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) o[qb][db] = Mma<T>::run(a, p[qb][t], o[qb][db]);
        }
    }
}

// O^T += V^T P^T of this tile with the exp2 work of the elements [E0, E1)
// of the next tile's scores sn between the MFMAs (into pn, row sum in rs).
template <typename T, int D, int DB, int KT, int KB, int E0, int E1>
__device__ __forceinline__ void pv_with_exp(const typename Mma<T>::vec8 (&p)[1][KT],
                                            const uint16_t* __restrict__ vts, f32x16 (&o)[1][DB], int lane, int hh,
                                            const f32x16 (&sn)[1][KB], float m, float c_log2,
                                            typename Mma<T>::vec8 (&pn)[1][KT], float& rs)
{
    typedef typename Mma<T>::vec8 vec8;
    static_assert(E0 >> 4 == (E1 - 1) >> 4, "one block");
    constexpr int n_mfma = KT * DB;
    float acc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) acc[kb] = 0.f;
#pragma unroll
    for (int t = 0; t < KT; ++t) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const vec8 a = vt_operand<vec8, D>(vts, t, db, lane, hh);
            o[0][db] = Mma<T>::run(a, p[0][t], o[0][db]);
            exp_slot<T, KB, KT, E0, E1, n_mfma, true>(t * DB + db, sn[0], m, c_log2, pn[0], acc);
        }
    }
    rs = acc[E0 >> 4];
}

template <typename T, int D, int QB, int KB, int DB, int KT, bool BS>
__device__ __forceinline__ void softmax_pv(const f32x16 (&s)[QB][KB], const uint16_t* __restrict__ vts,
                                           f32x16 (&o)[QB][DB], float (&m_run)[QB],
                                           float (&l_run)[QB], float c_log2, int lane, int hh,
                                           bool check = true)
{
    typename Mma<T>::vec8 p[QB][KT];
    softmax_tile<T, QB, KB, DB, KT, BS>(s, o, m_run, l_run, c_log2, p, check);
    pv_tile<T, D, QB, DB, KT>(p, vts, o, lane, hh);
}

// Instruction order of a pipelined tile. The scores of the next tile are
// issued first (MFMAs that need only K and Q), keeping their K operand reads
// a few MFMAs ahead; then the P.V MFMAs follow with their transposed V reads
// issued ahead. Vector instructions keep their program order between the
// MFMAs (scores_with_exp places them).
template <int D, int WAVES, int QB, int DC = D>
__device__ __forceinline__ void order_scores_block()
{
    typedef Cfg<D, WAVES, QB, DC> C;
    constexpr int n_reads = C::KB * C::DS;  // one K read per QB MFMAs
    constexpr int lead = 4;
    __builtin_amdgcn_sched_group_barrier(0x100, lead, 0);
#pragma unroll
    for (int i = 0; i < n_reads - lead; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < lead; ++i) __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
}

template <int D, int WAVES, int QB, int DC = D>
__device__ __forceinline__ void order_pv_block()
{
    typedef Cfg<D, WAVES, QB, DC> C;
    constexpr int n_ops = C::DB * C::KT;  // two V reads per QB MFMAs
    constexpr int lead = 4;
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * lead, 0);
#pragma unroll
    for (int i = 0; i < n_ops - lead; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
#pragma unroll
    for (int i = 0; i < lead; ++i) __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
}

// Keeps the computation of x where it is written: an empty asm statement that
// takes x in registers and may change it. Without it the compiler sinks the
// exp work of a mixed block past the end of the block (into the next tile's
// step), where it no longer runs between MFMAs.
template <typename V>
__device__ __forceinline__ void pin_regs(V& x)
{
    u32x4 w = __builtin_bit_cast(u32x4, x);
    asm volatile("" : "+v"(w));
    x = __builtin_bit_cast(V, w);
}

__device__ __forceinline__ void pin_reg(float& x) { asm volatile("" : "+v"(x)); }

// Q fragments: B operand of S^T = K Q^T, query qrow[qb] = row0 + 32*qb +
// (lane % 32), dims 16*ds + 8*hh + [0, 8). Rows past N are zero (their
// outputs are not stored).
template <typename T, int D, int QB, int DS>
__device__ __forceinline__ void load_q(const T* __restrict__ qh, int row0, int n_rows, int l32, int hh,
                                       int (&qrow)[QB], typename Mma<T>::vec8 (&qf)[QB][DS])
{
    typedef typename Mma<T>::vec8 vec8;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        qrow[qb] = row0 + qb * 32 + l32;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (qrow[qb] < n_rows) x = *(const u32x4*)(qh + (int64_t)qrow[qb] * D + ds * 16 + hh * 8);
            qf[qb][ds] = as_vec8<vec8>(x);
        }
    }
}

// Head dims below the kernel's D (PADDED launches): the head's rows are dm
// elements apart in memory (dm a multiple of 8, dm < D) and the kernel runs
// with D, the missing dims held at zero. Q dims past dm load as zero.
template <typename T, int D, int QB, int DS>
__device__ __forceinline__ void load_q_padded(const T* __restrict__ qh, int dm, int row0, int n_rows, int l32,
                                              int hh, int (&qrow)[QB], typename Mma<T>::vec8 (&qf)[QB][DS])
{
    typedef typename Mma<T>::vec8 vec8;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        qrow[qb] = row0 + qb * 32 + l32;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            u32x4 x = {0u, 0u, 0u, 0u};
            const int c0 = ds * 16 + hh * 8;
            if (qrow[qb] < n_rows && c0 < dm) x = *(const u32x4*)(qh + (int64_t)qrow[qb] * dm + c0);
            qf[qb][ds] = as_vec8<vec8>(x);
        }
    }
}

// K/V copies of a PADDED launch: the lane's logical chunk (pc ^ swz) is a
// real one iff it lies below dm / 8; the other lanes copy nothing, and the
// LDS chunks they would fill hold zeros written once (zero_pad_chunks). The
// swizzle has period 16 in the row and consecutive copies of a lane are a
// multiple of 16 rows apart, so a lane's chunk is real for all its copies or
// for none.
template <int D>
__device__ __forceinline__ uint32_t tile_lane_offset_padded(int wave, int lane, int dm, bool& real)
{
    const int c = wave * 64 + lane;
    const int r0 = c / (D / 8), lc = (c % (D / 8)) ^ swz<D>(r0);
    real = lc < dm / 8;
    return (uint32_t)(r0 * dm * 2 + lc * 16);
}

template <int D, int WAVES, int QB>
__device__ __forceinline__ void issue_tile_padded(uint16_t* buf, rsrc_t src, int k0, int wave, uint32_t lane_off,
                                                  bool real, int dm)
{
    typedef Cfg<D, WAVES, QB> C;
    constexpr int rows_per_copy = WAVES * 64 / C::CPR;
    if (real) {
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i)
            copy16_to_lds(src, buf + (i * WAVES + wave) * 64 * 8, lane_off,
                          (uint32_t)(k0 + i * rows_per_copy) * (uint32_t)(dm * 2));
    }
}

// Zeros the LDS chunks of the dims past dm in n_tiles consecutive tile
// buffers (their positions are the same in every tile and no copy writes
// them).
template <int D, int WAVES, int QB>
__device__ __forceinline__ void zero_pad_chunks(uint16_t* buf0, int n_tiles, int dm, int tid)
{
    typedef Cfg<D, WAVES, QB> C;
    for (int c = tid; c < C::BN * C::CPR; c += C::THREADS) {
        const int r = c / C::CPR, lc = (c % C::CPR) ^ swz<D>(r);
        if (lc >= dm / 8)
            for (int t = 0; t < n_tiles; ++t) *(u32x4*)(buf0 + t * C::TILE + c * 8) = (u32x4){0u, 0u, 0u, 0u};
    }
}

}  // namespace
}  // namespace fa

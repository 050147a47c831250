// fa_fwd_kernel.hip -- attention forward (FlashAttention-2 form) for gfx950.
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
//   * A workgroup is 4 waves (256 threads) and owns 128 query rows; each wave
//     owns 32 whole rows, so row reductions never leave the wave (the pages'
//     rule that every warp must own whole rows, Round 0 / Round 1).
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_{bf16,f16}: keys on the M axis, queries on N. In the
//     32x32 accumulator each lane holds 16 keys of ONE query, and the other 16
//     keys of that query sit in lane ^ 32. The row max and row sum are
//     in-lane plus one v_permlane32_swap, and the rescale of O by alpha is one
//     scalar per lane.
//   * O^T += V^T P^T takes P^T straight from the score registers as the B
//     operand. The score accumulator hands each lane keys {8g + 4h + t}; V^T
//     is written to LDS with its keys permuted the same way, so every operand
//     is one 16-byte LDS read and P never goes through LDS.
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
//     iteration j computes the scores of tile j+1 on the matrix cores while
//     the vector units run the softmax of tile j, then P_j V_j; the copies of
//     K_{j+2} and V_{j+1} are in flight meanwhile; one barrier per tile. The
//     copies go through a buffer descriptor bounded to the head, so the rows
//     of a ragged last tile past N arrive as zeros (and are masked).
//   * exp2 with the softmax scale and log2(e) folded into one constant
//     (Round 4, "exp2"); the running max is kept in log2 units; the row max is
//     taken on the scaled scores so the maximal term is 2^0 = 1.
//   * P is rounded to the input type after l has been summed from fp32 P
//     (Round 4, "The P cast").
//   * Causal attention visits no key tile above the diagonal and masks only
//     the diagonal tiles; non-causal attention masks only a ragged last tile
//     (Round 4, "Causal tile-skipping"). Masked scores are -inf; the running
//     max starts at a finite very negative value so a row with no visible key
//     in a tile never forms -inf - (-inf).
//   * Workgroup ids are remapped so that all query tiles of one (b, h) run on
//     the same XCD (workgroups are dealt round-robin over the 8 XCDs, each with
//     its own L2), which keeps that head's K and V in one L2.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_launch.h"
#include "fa_tiles.h"

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

constexpr int kThreads = 256;  // 4 waves of 64
constexpr int kWaves = 4;
constexpr int kBlockM = 128;   // query rows per workgroup (32 per wave)
constexpr int kXcds = 8;       // XCDs of an MI355X

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int D>
struct Cfg {
    static_assert(D == 64 || D == 128, "head dim");
    static constexpr int BN = 64;                 // keys per tile
    static constexpr int CPR = D / 8;             // 16-byte chunks per row
    static constexpr int TILE = BN * D;           // elements of one K or V tile (dense)
    static constexpr int LDS_BYTES = 4 * TILE * 2;  // two K and two V tile buffers
    static constexpr int KB = BN / 32;            // 32-key blocks per tile
    static constexpr int DS = D / 16;             // MFMA k-steps of S^T = K Q^T
    static constexpr int DB = D / 32;             // 32-row blocks of O^T
    static constexpr int KT = BN / 16;            // MFMA k-steps of O^T += V^T P^T
    static constexpr int LOADS = BN * CPR / kThreads;  // 16-byte loads per thread, each of K and V
    static_assert(LOADS * kThreads == BN * CPR, "tile split");
    static_assert(BN * CPR % (64 * kWaves) == 0, "whole wave loads");
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
// Rows 256/CPR apart have the same swizzle (tile_lane_offset relies on it).
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

// HBM -> LDS copy of rows [k0, k0 + BN) of one K or V head. Wave w, load i
// fills 64 consecutive LDS chunks; lane l fetches the global chunk that the
// swizzle places there. Load i is 256/CPR rows below load 0, which leaves the
// swizzle unchanged, so every load of a lane is one per-lane byte offset plus
// a wave-uniform k0 * D * 2 + i * 4096.
template <int D>
__device__ __forceinline__ uint32_t tile_lane_offset(int wave, int lane)
{
    typedef Cfg<D> C;
    const int c = wave * 64 + lane;
    const int r0 = c / C::CPR, pc = c % C::CPR;
    return (uint32_t)(r0 * D * 2 + (pc ^ swz<D>(r0)) * 16);
}

template <int D>
__device__ __forceinline__ void issue_tile(uint16_t* buf, rsrc_t src, int k0, int wave,
                                           uint32_t lane_off)
{
    typedef Cfg<D> C;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i)
        copy16_to_lds(src, buf + (i * kWaves + wave) * 64 * 8, lane_off,
                      (uint32_t)k0 * (D * 2) + i * 4096);
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

// Largest growth of the row max, in log2 units, that the running state may
// absorb without rescaling O and l: P then reaches at most 2^8, far inside the
// fp16/bf16 range, and the final O / l is unchanged (both carry the same
// factor). Rescaling only when some row of the wave passes this keeps the
// O * alpha multiplies off the common path.
constexpr float kRescaleSlack = 8.0f;

// S^T = K Q^T for one key tile: s[kb] holds keys 32*kb + (accumulator rows)
// of this lane's query.
template <typename T, int D>
__device__ __forceinline__ void scores(f32x16 (&s)[Cfg<D>::KB], const uint16_t* __restrict__ ks,
                                       const typename Mma<T>::vec8 (&qf)[Cfg<D>::DS], int l32,
                                       int hh)
{
    typedef Cfg<D> C;
    typedef typename Mma<T>::vec8 vec8;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
        s[kb] = (f32x16){};
        const int row = kb * 32 + l32;
        const uint16_t* krow = ks + row * D;
        const int sw = swz<D>(row);
#pragma unroll
        for (int ds = 0; ds < C::DS; ++ds) {
            vec8 a = as_vec8<vec8>(*(const u32x4*)(krow + (((2 * ds + hh) ^ sw) * 8)));
            s[kb] = Mma<T>::run(a, qf[ds], s[kb]);
        }
    }
}

// Diagonal / ragged tiles: keys past N, and for causal attention keys after
// the lane's query, get score -inf.
template <int D, bool CAUSAL>
__device__ __forceinline__ void mask_scores(f32x16 (&s)[Cfg<D>::KB], int k0, int qrow, int N, int hh)
{
#pragma unroll
    for (int kb = 0; kb < Cfg<D>::KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool hide = key >= N || (CAUSAL && key > qrow);
            if (hide) s[kb][r] = -INFINITY;
        }
    }
}

// Online-softmax update for one tile of scores, then O^T += V^T P^T.
// Rows whose max grew past the slack trigger a wave-uniform rescale first.
template <typename T, int D>
__device__ __forceinline__ void rescale_if_needed(const f32x16 (&s)[Cfg<D>::KB],
                                                  f32x16 (&o)[Cfg<D>::DB], float& m_run,
                                                  float& l_run, float c_log2)
{
    typedef Cfg<D> C;
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = swap_halves_max(mx) * c_log2;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleSlack)) {
        // some row's max grew past the slack: move every row of the wave to
        // its true running max
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) o[db] *= alpha;
    }
}

template <typename T, int D>
__device__ __forceinline__ void softmax_pv(const f32x16 (&s)[Cfg<D>::KB],
                                           const uint16_t* __restrict__ vts,
                                           f32x16 (&o)[Cfg<D>::DB], float m_run, float& l_run,
                                           float c_log2, int lane, int hh)
{
    typedef Cfg<D> C;
    typedef typename Mma<T>::vec8 vec8;
    // P = 2^(s * c - m); l is summed from fp32 P, then P is rounded to the
    // input type for the P.V product (Round 4, "The P cast")
    vec8 p[C::KT];
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c_log2, -m_run));
            rs += e;
            p[kb * 2 + (r >> 3)][r & 7] = to_elem<T>(e);
        }
    }
    l_run += rs;

    // V^T operand, lane l = 16g + i: dim 32*db + (l % 32); elements 0..3 are
    // keys 16t + 4h + [0,4), elements 4..7 keys 16t + 8 + 4h + [0,4) (h = g/2),
    // the key order of P^T. Each of the two transposed reads has lane i address
    // key (base + i/4), dims 4*(i%4) + [0,4) of the group's 16 dims.
    const int gi = lane & 15, g1 = (lane >> 4) & 1;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
        const int chunk = 4 * db + 2 * g1 + ((gi & 3) >> 1);
        const int half = (gi & 1) * 4;
#pragma unroll
        for (int t = 0; t < C::KT; ++t) {
            const int key0 = 16 * t + 4 * hh + (gi >> 2);
            const int key1 = key0 + 8;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(vts + key0 * D + ((chunk ^ swz<D>(key0)) * 8) + half));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(vts + key1 * D + ((chunk ^ swz<D>(key1)) * 8) + half));
            u32x4 w;
            w[0] = __builtin_bit_cast(u32x2, lo)[0];
            w[1] = __builtin_bit_cast(u32x2, lo)[1];
            w[2] = __builtin_bit_cast(u32x2, hi)[0];
            w[3] = __builtin_bit_cast(u32x2, hi)[1];
            o[db] = Mma<T>::run(as_vec8<vec8>(w), p[t], o[db]);
        }
    }
}

template <typename T, int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void fa_fwd_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                   T* __restrict__ o, float* __restrict__ lse, int N, int n_qt, float c_log2)
{
    typedef Cfg<D> C;
    typedef typename Mma<T>::vec8 vec8;
    __shared__ __attribute__((aligned(16))) uint16_t smem[4 * C::TILE];

    // blockIdx -> (b*H + h, query tile), XCD-aware: hardware id i runs on XCD
    // i % 8; give each XCD a contiguous range of logical ids.
    const uint32_t nwg = gridDim.x, hw = blockIdx.x;
    const uint32_t xcd = hw % kXcds, slot = hw / kXcds;
    const uint32_t per = nwg / kXcds, extra = nwg % kXcds;
    const uint32_t logical = xcd < extra ? xcd * (per + 1) + slot
                                         : extra * (per + 1) + (xcd - extra) * per + slot;
    const uint32_t bh = logical / (uint32_t)n_qt;
    uint32_t qt = logical % (uint32_t)n_qt;
    if (CAUSAL) qt = (uint32_t)n_qt - 1 - qt;  // longest causal tiles first
    const int q0 = (int)qt * kBlockM;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    const int64_t head_off = (int64_t)bh * N * D;
    const T* qh = q + head_off;
    const T* kh = k + head_off;
    const T* vh = v + head_off;

    // Q fragment: B operand of S^T = K Q^T, query qrow, dims 16*ds + 8*hh + [0, 8).
    const int qrow = q0 + wave * 32 + l32;
    vec8 qf[C::DS];
#pragma unroll
    for (int ds = 0; ds < C::DS; ++ds) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (qrow < N) x = *(const u32x4*)(qh + (int64_t)qrow * D + ds * 16 + hh * 8);
        qf[ds] = as_vec8<vec8>(x);
    }

    const TileSpan span = tile_span(q0, kBlockM, C::BN, N, CAUSAL);
    const int n_unmasked = (int)span.unmasked, n_tiles = (int)span.total;

    f32x16 oacc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) oacc[db] = (f32x16){};
    float m_run = -1e30f, l_run = 0.f;

    // LDS: K tiles in buffers 0/1, V tiles in buffers 2/3. Iteration j reads
    // K_{j+1} (scores of the next tile) and V_j (P.V of this tile) while the
    // copies of K_{j+2} and V_{j+1} are in flight; one barrier per tile.
    auto kbuf = [&](int i) { return smem + (i & 1) * C::TILE; };
    auto vbuf = [&](int i) { return smem + (2 + (i & 1)) * C::TILE; };

    const uint32_t head_bytes = (uint32_t)N * (D * 2);
    const rsrc_t krs = head_rsrc(kh, head_bytes), vrs = head_rsrc(vh, head_bytes);
    const uint32_t lane_off = tile_lane_offset<D>(wave, lane);
    issue_tile<D>(kbuf(0), krs, 0, wave, lane_off);
    issue_tile<D>(vbuf(0), vrs, 0, wave, lane_off);
    if (n_tiles > 1) issue_tile<D>(kbuf(1), krs, C::BN, wave, lane_off);
    stage_barrier();
    f32x16 sa[C::KB], sb[C::KB];
    scores<T, D>(sa, kbuf(0), qf, l32, hh);
    stage_barrier();  // K_0's buffer is refilled in the first iteration

    // One tile: sc holds the scores of tile j; sn receives those of tile j+1
    // (past the last tile it reads a stale buffer and is never used).
    auto step = [&](auto masked, int j, f32x16 (&sc)[C::KB], f32x16 (&sn)[C::KB]) {
        if (j + 2 < n_tiles) issue_tile<D>(kbuf(j), krs, (j + 2) * C::BN, wave, lane_off);
        if (j + 1 < n_tiles) issue_tile<D>(vbuf(j + 1), vrs, (j + 1) * C::BN, wave, lane_off);
        if (decltype(masked)::value) mask_scores<D, CAUSAL>(sc, j * C::BN, qrow, N, hh);
        rescale_if_needed<T, D>(sc, oacc, m_run, l_run, c_log2);
        scores<T, D>(sn, kbuf(j + 1), qf, l32, hh);
        softmax_pv<T, D>(sc, vbuf(j), oacc, m_run, l_run, c_log2, lane, hh);
        stage_barrier();
    };
    typedef std::integral_constant<bool, false> unmasked_t;
    typedef std::integral_constant<bool, true> masked_t;

    // tiles [0, n_unmasked) need no mask, [n_unmasked, n_tiles) get it
    int j = 0;
    for (; j + 2 <= n_unmasked; j += 2) {
        step(unmasked_t(), j, sa, sb);
        step(unmasked_t(), j + 1, sb, sa);
    }
    if (j < n_unmasked) {
        step(unmasked_t(), j, sa, sb);
        ++j;
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) sa[kb] = sb[kb];
    }
    for (; j + 2 <= n_tiles; j += 2) {
        step(masked_t(), j, sa, sb);
        step(masked_t(), j + 1, sb, sa);
    }
    if (j < n_tiles) step(masked_t(), j, sa, sb);

    // Epilogue: O = O_acc / l in the input type, lse = (m + log2 l) * ln 2.
    const float l_tot = swap_halves_sum(l_run);
    if (qrow < N) {
        const float inv = 1.0f / l_tot;
        T* orow = o + head_off + (int64_t)qrow * D;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                T vals[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) vals[t] = to_elem<T>(oacc[db][4 * g + t] * inv);
                u32x2 packed = __builtin_bit_cast(u32x2, vals);
                *(u32x2*)(orow + db * 32 + 8 * g + 4 * hh) = packed;
            }
        }
        if (hh == 0) lse[(int64_t)bh * N + qrow] = (m_run + log2f(l_tot)) * 0.69314718055994531f;
    }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_one(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                      int N, float scale, hipStream_t stream)
{
    const int n_qt = (N + kBlockM - 1) / kBlockM;
    const float c_log2 = scale * 1.4426950408889634f;
    dim3 grid((unsigned)((int64_t)n_qt * BH)), block(kThreads);
    hipLaunchKernelGGL((fa_fwd_kernel<T, D, CAUSAL>), grid, block, 0, stream, (const T*)q,
                       (const T*)k, (const T*)v, (T*)o, lse, N, n_qt, c_log2);
    return hipGetLastError();
}

}  // namespace

int block_m() { return kBlockM; }
int block_n(int d) { return d == 64 ? Cfg<64>::BN : Cfg<128>::BN; }
int threads_per_block() { return kThreads; }
int lds_bytes(int d) { return d == 64 ? Cfg<64>::LDS_BYTES : Cfg<128>::LDS_BYTES; }

hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int N, int d, bool causal, float scale, bool bf16,
                      hipStream_t stream)
{
    const int BH = B * H;
#define FA_DISPATCH(T, D)                                                                      \
    return causal ? launch_one<T, D, true>(q, k, v, o, lse, BH, N, scale, stream)              \
                  : launch_one<T, D, false>(q, k, v, o, lse, BH, N, scale, stream)
    if (bf16) {
        if (d == 64) FA_DISPATCH(__bf16, 64);
        FA_DISPATCH(__bf16, 128);
    }
    if (d == 64) FA_DISPATCH(_Float16, 64);
    FA_DISPATCH(_Float16, 128);
#undef FA_DISPATCH
}

}  // namespace fa

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
//   * K tiles are copied to LDS with 128-bit loads and stores; V tiles are
//     loaded with 128-bit loads, transposed 4 keys x 8 dims in registers and
//     stored as V^T. Rows are padded by 16 bytes so the 32 lanes of an operand
//     read hit distinct banks. Two LDS stages: the next tile's global loads are
//     issued before the current tile's MFMAs, one barrier per tile.
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
constexpr int kBlockM = 128;   // query rows per workgroup (32 per wave)
constexpr int kXcds = 8;       // XCDs of an MI355X

template <int D>
struct Cfg {
    static_assert(D == 64 || D == 128, "head dim");
    static constexpr int BN = 8192 / D;           // keys per tile: 64 at d=128, 128 at d=64
    static constexpr int KSTRIDE = D + 8;         // LDS row of K, elements (16 B pad)
    static constexpr int VSTRIDE = BN + 8;        // LDS row of V^T, elements (16 B pad)
    static constexpr int K_ELEMS = BN * KSTRIDE;
    static constexpr int V_ELEMS = D * VSTRIDE;
    static constexpr int STAGE = K_ELEMS + V_ELEMS;
    static constexpr int LDS_BYTES = 2 * STAGE * 2;
    static constexpr int KB = BN / 32;            // 32-key blocks per tile
    static constexpr int DS = D / 16;             // MFMA k-steps of S^T = K Q^T
    static constexpr int DB = D / 32;             // 32-row blocks of O^T
    static constexpr int KT = BN / 16;            // MFMA k-steps of O^T += V^T P^T
    static constexpr int CPR = D / 8;             // 16-byte chunks per row
    static constexpr int K_CHUNKS = BN * CPR / kThreads;  // K chunks per thread
    static constexpr int V_ITEMS = (BN / 4) * CPR / kThreads;  // 4-key x 8-dim V blocks per thread
    static_assert(K_CHUNKS * kThreads == BN * CPR, "K tile split");
    static_assert(V_ITEMS * kThreads == (BN / 4) * CPR, "V tile split");
};

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

// Slot of key kappa (0..15) inside a 16-key group of a V^T row. Lane half h,
// element j of the P^T operand holds key 8*(j/4) + 4*h + (j%4) of the group
// (the order of the 32x32 accumulator rows), so slot 8*h + j holds that key.
__device__ __forceinline__ int vt_slot_of_4group(int g)  // g = kappa / 4, kappa multiple of 4
{
    return 8 * (g & 1) + 4 * (g >> 1);
}

template <typename T, int D>
struct TileRegs {
    u32x4 k[Cfg<D>::K_CHUNKS];
    u32x4 v[Cfg<D>::V_ITEMS][4];
};

// Global -> registers for the key tile starting at key k0. CHECK: the tile
// reaches past N, so rows >= N are replaced by zeros (only a ragged last tile).
template <typename T, int D, bool CHECK>
__device__ __forceinline__ void load_tile(TileRegs<T, D>& r, const T* __restrict__ kh,
                                          const T* __restrict__ vh, int k0, int N, int tid)
{
    typedef Cfg<D> C;
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < C::K_CHUNKS; ++i) {
        const int id = tid + i * kThreads;
        const int row = id / C::CPR, c8 = id % C::CPR;
        const int key = k0 + row;
        if (CHECK) {
            // clamped address, then select: no divergent branch around the load
            const int kc = key < N ? key : N - 1;
            const u32x4 x = *(const u32x4*)(kh + (int64_t)kc * D + c8 * 8);
            r.k[i] = key < N ? x : zero;
        } else {
            r.k[i] = *(const u32x4*)(kh + (int64_t)key * D + c8 * 8);
        }
    }
#pragma unroll
    for (int i = 0; i < C::V_ITEMS; ++i) {
        const int id = tid + i * kThreads;
        const int g4 = id / C::CPR, c8 = id % C::CPR;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int key = k0 + 4 * g4 + t;
            if (CHECK) {
                const int kc = key < N ? key : N - 1;
                const u32x4 x = *(const u32x4*)(vh + (int64_t)kc * D + c8 * 8);
                r.v[i][t] = key < N ? x : zero;
            } else {
                r.v[i][t] = *(const u32x4*)(vh + (int64_t)key * D + c8 * 8);
            }
        }
    }
}

template <typename T, int D>
__device__ __forceinline__ void load_tile_any(TileRegs<T, D>& r, const T* __restrict__ kh,
                                              const T* __restrict__ vh, int tile, int n_full,
                                              int N, int tid)
{
    if (tile < n_full)
        load_tile<T, D, false>(r, kh, vh, tile * Cfg<D>::BN, N, tid);
    else
        load_tile<T, D, true>(r, kh, vh, tile * Cfg<D>::BN, N, tid);
}

// Registers -> LDS stage: K row-major (padded), V transposed to V^T with the
// keys of each 16-key group permuted to the P^T operand order.
template <typename T, int D>
__device__ __forceinline__ void store_tile(const TileRegs<T, D>& r, uint16_t* __restrict__ ks,
                                           uint16_t* __restrict__ vts, int tid)
{
    typedef Cfg<D> C;
#pragma unroll
    for (int i = 0; i < C::K_CHUNKS; ++i) {
        const int id = tid + i * kThreads;
        const int row = id / C::CPR, c8 = id % C::CPR;
        *(u32x4*)(ks + row * C::KSTRIDE + c8 * 8) = r.k[i];
    }
#pragma unroll
    for (int i = 0; i < C::V_ITEMS; ++i) {
        const int id = tid + i * kThreads;
        const int g4 = id / C::CPR, c8 = id % C::CPR;
        const int slot = 16 * (g4 >> 2) + vt_slot_of_4group(g4 & 3);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int w = e >> 1;
            uint32_t a0 = r.v[i][0][w], a1 = r.v[i][1][w], a2 = r.v[i][2][w], a3 = r.v[i][3][w];
            u32x2 out;
            if (e & 1) {
                out[0] = (a0 >> 16) | (a1 & 0xffff0000u);
                out[1] = (a2 >> 16) | (a3 & 0xffff0000u);
            } else {
                out[0] = (a0 & 0xffffu) | (a1 << 16);
                out[1] = (a2 & 0xffffu) | (a3 << 16);
            }
            *(u32x2*)(vts + (c8 * 8 + e) * C::VSTRIDE + slot) = out;
        }
    }
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

// One key tile: S^T = K Q^T, mask (diagonal / ragged tiles only), online
// softmax update, O^T += V^T P^T.
template <typename T, int D, bool CAUSAL, bool MASKED>
__device__ __forceinline__ void attend_tile(const uint16_t* __restrict__ ks,
                                            const uint16_t* __restrict__ vts,
                                            const typename Mma<T>::vec8 (&qf)[Cfg<D>::DS],
                                            f32x16 (&o)[Cfg<D>::DB], float& m_run, float& l_run,
                                            float c_log2, int k0, int qrow, int N, int l32, int hh)
{
    typedef Cfg<D> C;
    typedef typename Mma<T>::vec8 vec8;

    f32x16 s[C::KB];
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
        s[kb] = (f32x16){};
        const uint16_t* krow = ks + (kb * 32 + l32) * C::KSTRIDE + hh * 8;
#pragma unroll
        for (int ds = 0; ds < C::DS; ++ds) {
            vec8 a = as_vec8<vec8>(*(const u32x4*)(krow + ds * 16));
            s[kb] = Mma<T>::run(a, qf[ds], s[kb]);
        }
    }

    if (MASKED) {
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
                const bool hide = key >= N || (CAUSAL && key > qrow);
                if (hide) s[kb][r] = -INFINITY;
            }
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = swap_halves_max(mx) * c_log2;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleSlack)) {
        // wave-uniform: some row's max grew past the slack; move every row of
        // the wave to its true running max
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) o[db] *= alpha;
    }

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

#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
        const uint16_t* vrow = vts + (db * 32 + l32) * C::VSTRIDE + hh * 8;
#pragma unroll
        for (int t = 0; t < C::KT; ++t) {
            vec8 a = as_vec8<vec8>(*(const u32x4*)(vrow + t * 16));
            o[db] = Mma<T>::run(a, p[t], o[db]);
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
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::STAGE];

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
    const int n_full = N / C::BN;  // key tiles wholly inside [0, N)

    f32x16 oacc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) oacc[db] = (f32x16){};
    float m_run = -1e30f, l_run = 0.f;

    TileRegs<T, D> regs;
    load_tile_any<T, D>(regs, kh, vh, 0, n_full, N, tid);
    store_tile<T, D>(regs, smem, smem + C::K_ELEMS, tid);
    __syncthreads();

    // Tiles [0, n_unmasked) need no mask, [n_unmasked, n_tiles) get it. The
    // next tile's global loads are in flight while the current one is used.
    int j = 0;
    for (; j < n_unmasked; ++j) {
        const bool more = j + 1 < n_tiles;
        if (more) load_tile_any<T, D>(regs, kh, vh, j + 1, n_full, N, tid);
        const uint16_t* ks = smem + (j & 1) * C::STAGE;
        attend_tile<T, D, CAUSAL, false>(ks, ks + C::K_ELEMS, qf, oacc, m_run, l_run, c_log2,
                                         j * C::BN, qrow, N, l32, hh);
        if (more) {
            uint16_t* nks = smem + ((j + 1) & 1) * C::STAGE;
            store_tile<T, D>(regs, nks, nks + C::K_ELEMS, tid);
        }
        __syncthreads();
    }
    for (; j < n_tiles; ++j) {
        const bool more = j + 1 < n_tiles;
        if (more) load_tile_any<T, D>(regs, kh, vh, j + 1, n_full, N, tid);
        const uint16_t* ks = smem + (j & 1) * C::STAGE;
        attend_tile<T, D, CAUSAL, true>(ks, ks + C::K_ELEMS, qf, oacc, m_run, l_run, c_log2,
                                        j * C::BN, qrow, N, l32, hh);
        if (more) {
            uint16_t* nks = smem + ((j + 1) & 1) * C::STAGE;
            store_tile<T, D>(regs, nks, nks + C::K_ELEMS, tid);
        }
        __syncthreads();
    }

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

// fa_fwd_f32.hip -- the attention forward for fp32 inputs and outputs.
//
// "How to optimise a Triton FlashAttention-2 kernel step by step with a
// profiler" (Round 1) runs its tests with fp32 inputs at D = 128, where the
// products go through the tensor cores in a reduced-precision fp32 format.
// On gfx950 the fp32 MFMA rate is 1/16 of the bf16 rate, so the products
// are formed from bf16 parts instead: every fp32 value x is split into
// hi = bf16(x) and lo = bf16(x - hi), which together hold about 16
// significant bits (|x - hi - lo| <= 2^-16 |x|), and a product is taken as
// hi*hi + hi*lo + lo*hi (the dropped lo*lo is below 2^-16 of it). That is
// three bf16 MFMAs, a third of the bf16 rate, with fp32 accumulation, and
// more precise than a 10-bit-mantissa product.
//
//   * A pre-pass splits K and V into four bf16 arrays (hi and lo of each)
//     in a caller-owned workspace of the same size as fp32 K and V; Q is
//     split once into registers when it is loaded.
//   * Scores: S^T = Kh Qh^T + Kh Ql^T + Kl Qh^T, each K operand read feeding
//     two or one MFMAs. The softmax is the one of the bf16/fp16 kernel
//     (exp2 with folded scale, lazily updated running max), with P split
//     into hi and lo parts from its fp32 value; O^T += Vh Ph + Vh Pl + Vl Ph.
//   * One 4-wave workgroup per 128 query rows, 32 rows per wave, 64-key
//     tiles; both stages of Kh, Kl, Vh, Vl sit in LDS (8 tiles, 128 KB at
//     d = 128), the next tile's copies in flight while this one is computed,
//     one barrier per tile. One wave per SIMD: the hi/lo operands need more
//     than 256 registers.
//   * Causal tile skipping, per-wave diagonal skip, XCD order and N_q != N_k
//     as in the bf16/fp16 kernel; O is written in fp32, lse in natural log.

#include "fa_fwd_kernel.h"

namespace fa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// hi = bf16(x) rounded to nearest even, lo = bf16(x - hi).
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo)
{
    hi = (__bf16)x;
    lo = (__bf16)(x - (float)hi);
}

// K or V (fp32, n elements, n a multiple of 4) into its hi and lo parts.
__global__ __launch_bounds__(256) void fa_split_f32_kernel(const float* __restrict__ src, __bf16* __restrict__ hi,
                                                           __bf16* __restrict__ lo, int64_t n4)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    const f32x4 x = ((const f32x4*)src)[i];
    __bf16 h[4], l[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) split_bf16(x[t], h[t], l[t]);
    ((u32x2*)hi)[i] = __builtin_bit_cast(u32x2, h);
    ((u32x2*)lo)[i] = __builtin_bit_cast(u32x2, l);
}

// S^T for one key tile from the hi/lo parts of K (LDS tiles) and Q.
template <int D, int KB, int DS>
__device__ __forceinline__ void scores_x3(f32x16 (&s)[KB], const uint16_t* __restrict__ kh,
                                          const uint16_t* __restrict__ kl, const bf16x8 (&qh)[DS],
                                          const bf16x8 (&ql)[DS], int l32, int hh)
{
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s[kb] = (f32x16){};
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const bf16x8 ah = k_operand<bf16x8, D>(kh, kb * 32 + l32, ds, hh);
            const bf16x8 al = k_operand<bf16x8, D>(kl, kb * 32 + l32, ds, hh);
            s[kb] = Mma<__bf16>::run(ah, qh[ds], s[kb]);
            s[kb] = Mma<__bf16>::run(ah, ql[ds], s[kb]);
            s[kb] = Mma<__bf16>::run(al, qh[ds], s[kb]);
        }
    }
}

// P = 2^(s c - m) with its hi and lo parts, and the lane's partial row sum of
// the fp32 values.
template <int KB, int KT>
__device__ __forceinline__ float exp_x3(const f32x16 (&s)[KB], float m, float c_log2, bf16x8 (&ph)[KT],
                                        bf16x8 (&pl)[KT])
{
    float acc = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c_log2, -m));
            acc += e;
            __bf16 h, l;
            split_bf16(e, h, l);
            ph[kb * 2 + (r >> 3)][r & 7] = h;
            pl[kb * 2 + (r >> 3)][r & 7] = l;
        }
    }
    return acc;
}

// O^T += V^T P^T from the hi/lo parts of V (LDS tiles) and P.
template <int D, int DB, int KT>
__device__ __forceinline__ void pv_x3(const bf16x8 (&ph)[KT], const bf16x8 (&pl)[KT], const uint16_t* __restrict__ vh,
                                      const uint16_t* __restrict__ vl, f32x16 (&o)[DB], int lane, int hh)
{
#pragma unroll
    for (int t = 0; t < KT; ++t) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const bf16x8 ah = vt_operand<bf16x8, D>(vh, t, db, lane, hh);
            const bf16x8 al = vt_operand<bf16x8, D>(vl, t, db, lane, hh);
            o[db] = Mma<__bf16>::run(ah, ph[t], o[db]);
            o[db] = Mma<__bf16>::run(ah, pl[t], o[db]);
            o[db] = Mma<__bf16>::run(al, ph[t], o[db]);
        }
    }
}

template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void fa_fwd_f32_kernel(const float* __restrict__ q, const __bf16* __restrict__ kh, const __bf16* __restrict__ kl,
                       const __bf16* __restrict__ vh, const __bf16* __restrict__ vl, float* __restrict__ o,
                       float* __restrict__ lse, int Nq, int Nk, int n_qt, float c_log2)
{
    typedef Cfg<D, 4, 1> C;
    // stage s holds Kh, Kl, Vh, Vl of one key tile at tiles 4s .. 4s + 3
    __shared__ __attribute__((aligned(16))) uint16_t smem[8 * C::TILE];

    uint32_t bh, qt;
    workgroup_tile<CAUSAL>(n_qt, false, bh, qt);
    const int q0 = (int)qt * C::BM;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    const int64_t q_off = (int64_t)bh * Nq * D, kv_off = (int64_t)bh * Nk * D;

    // Q: this lane's row, 8 dims per k-step, split into hi and lo
    const int qrow = q0 + wave * 32 + l32;
    bf16x8 qh[C::DS], ql[C::DS];
#pragma unroll
    for (int ds = 0; ds < C::DS; ++ds) {
        f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
        if (qrow < Nq) {
            const float* src = q + q_off + (int64_t)qrow * D + ds * 16 + hh * 8;
            x0 = *(const f32x4*)src;
            x1 = *(const f32x4*)(src + 4);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            __bf16 h, l;
            split_bf16(x0[t], h, l);
            qh[ds][t] = h;
            ql[ds][t] = l;
            split_bf16(x1[t], h, l);
            qh[ds][4 + t] = h;
            ql[ds][4 + t] = l;
        }
    }

    const TileSpan span = tile_span(q0, C::BM, C::BN, Nq, Nk, CAUSAL);
    const int n_unmasked = (int)span.unmasked, n_tiles = (int)span.total;
    const int n_wave = CAUSAL ? min(n_tiles, (q0 + (wave + 1) * 32 - 1) / C::BN + 1) : n_tiles;

    const uint32_t head_bytes = (uint32_t)Nk * (D * 2);
    const rsrc_t rs[4] = {head_rsrc(kh + kv_off, head_bytes), head_rsrc(kl + kv_off, head_bytes),
                          head_rsrc(vh + kv_off, head_bytes), head_rsrc(vl + kv_off, head_bytes)};
    const uint32_t lane_off = tile_lane_offset<D>(wave, lane);
    auto tile = [&](int j, int part) { return smem + (4 * (j & 1) + part) * C::TILE; };
    auto issue = [&](int j) {
#pragma unroll
        for (int part = 0; part < 4; ++part) issue_tile<D, 4, 1>(tile(j, part), rs[part], j * C::BN, wave, lane_off);
    };

    f32x16 oacc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) oacc[db] = (f32x16){};
    float m_run = -1e30f, l_run = 0.f;

    issue(0);
    stage_barrier();
    for (int j = 0; j < n_tiles; ++j) {
        if (j + 1 < n_tiles) issue(j + 1);
        if (j < n_wave) {
            f32x16 s[C::KB];
            scores_x3<D, C::KB, C::DS>(s, tile(j, 0), tile(j, 1), qh, ql, l32, hh);
            if (j >= n_unmasked) mask_scores<C::KB, CAUSAL>(s, j * C::BN, qrow, Nk, hh);
            bf16x8 ph[C::KT], pl[C::KT];
            float rsum = exp_x3<C::KB, C::KT>(s, m_run, c_log2, ph, pl);
            // the lazy max of the bf16/fp16 kernel (kLaneSumBound)
            if (__builtin_amdgcn_ballot_w64(!(rsum <= kLaneSumBound))) {
                const float m_new = fmaxf(m_run, row_max_log2<C::KB>(s, c_log2));
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < C::DB; ++db) oacc[db] *= alpha;
                rsum = exp_x3<C::KB, C::KT>(s, m_run, c_log2, ph, pl);
            }
            l_run += rsum;
            pv_x3<D, C::DB, C::KT>(ph, pl, tile(j, 2), tile(j, 3), oacc, lane, hh);
        }
        stage_barrier();
    }

    const float l_tot = swap_halves_sum(l_run);
    if (qrow < Nq) {
        const float inv = 1.0f / l_tot;
        float* orow = o + q_off + (int64_t)qrow * D;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 vals;
#pragma unroll
                for (int t = 0; t < 4; ++t) vals[t] = oacc[db][4 * g + t] * inv;
                *(f32x4*)(orow + db * 32 + 8 * g + 4 * hh) = vals;
            }
        }
        if (hh == 0) lse[(int64_t)bh * Nq + qrow] = (m_run + log2f(l_tot)) * 0.69314718055994531f;
    }
}

template <int D, bool CAUSAL>
hipError_t launch_f32_typed(const float* q, const float* k, const float* v, float* o, float* lse, int BH, int Nq,
                            int Nk, float scale, __bf16* ws, hipStream_t stream)
{
    const int64_t n = (int64_t)BH * Nk * D;
    __bf16 *kh = ws, *kl = ws + n, *vh = ws + 2 * n, *vl = ws + 3 * n;
    const int64_t n4 = n / 4;
    dim3 sgrid((unsigned)((n4 + 255) / 256)), sblock(256);
    hipLaunchKernelGGL(fa_split_f32_kernel, sgrid, sblock, 0, stream, k, kh, kl, n4);
    hipLaunchKernelGGL(fa_split_f32_kernel, sgrid, sblock, 0, stream, v, vh, vl, n4);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n_qt = (Nq + 127) / 128;
    dim3 grid((unsigned)((int64_t)n_qt * BH)), block(256);
    hipLaunchKernelGGL((fa_fwd_f32_kernel<D, CAUSAL>), grid, block, 0, stream, q, (const __bf16*)kh,
                       (const __bf16*)kl, (const __bf16*)vh, (const __bf16*)vl, o, lse, Nq, Nk, n_qt,
                       scale * 1.4426950408889634f);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
                          int Nq, int Nk, int d, bool causal, float scale, void* workspace, hipStream_t stream)
{
    const int BH = B * H;
    __bf16* ws = (__bf16*)workspace;
    if (d == 64)
        return causal ? launch_f32_typed<64, true>(q, k, v, o, lse, BH, Nq, Nk, scale, ws, stream)
                      : launch_f32_typed<64, false>(q, k, v, o, lse, BH, Nq, Nk, scale, ws, stream);
    return causal ? launch_f32_typed<128, true>(q, k, v, o, lse, BH, Nq, Nk, scale, ws, stream)
                  : launch_f32_typed<128, false>(q, k, v, o, lse, BH, Nq, Nk, scale, ws, stream);
}

}  // namespace fa

// fa_api.hip -- the C ABI of libfa (declared in include/fa.h): argument
// checks, launch plan, dispatch to the gfx950 kernels and error strings.
// Every argument check happens before the first HIP call, so misuse is
// reported without touching the device.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "fa.h"
#include "fa_launch.h"
#include "fa_tiles.h"

// The split workspace of fa_fwd_split_qk_noalloc: a scratch array of the
// library's own, one copy on each GPU (at its own address there), allocated
// with the code object and held until the process ends. Host code never
// passes `scratch` itself to a kernel (in host code the name stands for a
// host-side shadow): it looks up the device address on each GPU once
// (noalloc_scratch) and passes that.
static __device__ __align__(256) float scratch[FA_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

thread_local char g_msg[256];

int fail(int status, const char* what)
{
    snprintf(g_msg, sizeof g_msg, "%s", what);
    return status;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

// Shape/dtype checks shared by the forward entry points and the plans.
int check_problem(int B, int H, int Nq, int Nk, int d, int causal, int dtype)
{
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1)
        return fail(FA_ERR_INVALID_ARG, "B, H and the sequence lengths must be >= 1");
    if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16)
        return fail(FA_ERR_INVALID_ARG, "dtype must be FA_DTYPE_F16 or FA_DTYPE_BF16");
    if (d < 8 || d > 128 || d % 8 != 0)
        return fail(FA_ERR_UNSUPPORTED, "head dim must be a multiple of 8 from 8 to 128");
    const int64_t bh = (int64_t)B * H;
    const int64_t n_qt = ((int64_t)Nq + 127) / 128;  // the smallest workgroup tile
    if (bh > INT32_MAX || bh * n_qt > (int64_t)UINT32_MAX)
        return fail(FA_ERR_INVALID_ARG, "B*H*ceil(Nq/128) exceeds the grid limit");
    const int64_t n_max = Nq > Nk ? Nq : Nk;
    if (bh * n_max * d > INT64_MAX / 4) return fail(FA_ERR_INVALID_ARG, "B*H*N*d too large");
    if ((int64_t)n_max * d * 2 > (int64_t)UINT32_MAX)
        return fail(FA_ERR_INVALID_ARG, "one head (N*d*2 bytes) must be below 4 GiB");
    return FA_OK;
}

// Pointer, alignment, scale and overlap checks of the forward entry points.
int check_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq,
              int Nk, int d, int causal, float scale, int dtype)
{
    if (!q || !k || !v || !o || !lse) return fail(FA_ERR_INVALID_ARG, "NULL tensor pointer");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
        return fail(FA_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
    if (!aligned(lse, 4)) return fail(FA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
    const int rc = check_problem(B, H, Nq, Nk, d, causal, dtype);
    if (rc != FA_OK) return rc;
    if (!(scale > 0.f) || !isfinite(scale))
        return fail(FA_ERR_INVALID_ARG, "scale must be finite and > 0");
    const size_t qb = (size_t)B * H * Nq * d * 2, kb = (size_t)B * H * Nk * d * 2;
    const size_t lb = (size_t)B * H * Nq * 4;
    if (overlap(o, qb, q, qb) || overlap(o, qb, k, kb) || overlap(o, qb, v, kb))
        return fail(FA_ERR_INVALID_ARG, "o overlaps q, k or v");
    if (overlap(lse, lb, q, qb) || overlap(lse, lb, k, kb) || overlap(lse, lb, v, kb) ||
        overlap(lse, lb, o, qb))
        return fail(FA_ERR_INVALID_ARG, "lse overlaps q, k, v or o");
    return FA_OK;
}

// The split launch's own checks, after check_fwd.
int check_split(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                int Nq, int Nk, int d, int n_splits, void* workspace, int64_t workspace_bytes)
{
    if (!workspace) return fail(FA_ERR_INVALID_ARG, "NULL workspace pointer");
    if (!aligned(workspace, 16)) return fail(FA_ERR_INVALID_ARG, "the workspace must be 16-byte aligned");
    if (n_splits < 1 || n_splits > (Nk + 63) / 64)
        return fail(FA_ERR_INVALID_ARG, "n_splits must be between 1 and ceil(Nk / 64)");
    const int64_t need = (int64_t)n_splits * B * H * Nq * (fa::kernel_dim(d) + 1) * 4;
    if ((int64_t)B * H * ((Nq + 127) / 128) * n_splits > (int64_t)UINT32_MAX)
        return fail(FA_ERR_INVALID_ARG, "B*H*ceil(Nq/128)*n_splits exceeds the grid limit");
    if (workspace_bytes < need) return fail(FA_ERR_INVALID_ARG, "workspace too small");
    const size_t qb = (size_t)B * H * Nq * d * 2, kb = (size_t)B * H * Nk * d * 2;
    const size_t lb = (size_t)B * H * Nq * 4, wb = (size_t)need;
    if (overlap(workspace, wb, q, qb) || overlap(workspace, wb, k, kb) ||
        overlap(workspace, wb, v, kb) || overlap(workspace, wb, o, qb) ||
        overlap(workspace, wb, lse, lb))
        return fail(FA_ERR_INVALID_ARG, "the workspace overlaps a tensor argument");
    return FA_OK;
}

// Mask arguments: windows >= -1; key_lens (device, read by the kernel)
// 4-byte aligned and clear of everything the call writes.
int check_masks(int B, int H, int Nq, int d, int window_left, int window_right,
                const int32_t* key_lens, const void* o, const float* lse, const void* workspace,
                int64_t workspace_bytes)
{
    if (window_left < -1 || window_right < -1)
        return fail(FA_ERR_INVALID_ARG, "window_left and window_right must be >= -1");
    if (key_lens) {
        if (!aligned(key_lens, 4)) return fail(FA_ERR_INVALID_ARG, "key_lens must be 4-byte aligned");
        const size_t nb = (size_t)B * 4;
        if (overlap(key_lens, nb, o, (size_t)B * H * Nq * d * 2) ||
            overlap(key_lens, nb, lse, (size_t)B * H * Nq * 4) ||
            (workspace && overlap(key_lens, nb, workspace, (size_t)workspace_bytes)))
            return fail(FA_ERR_INVALID_ARG, "key_lens overlaps an output or the workspace");
    }
    return FA_OK;
}

// True when the masks hide nothing beyond the causal/tail masks of the
// unmasked kernels.
bool masks_off(int causal, int window_left, int window_right, const int32_t* key_lens)
{
    return !key_lens && window_left < 0 && (causal || window_right < 0);
}

fa::FwdArgs fwd_args(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                     int Nq, int Nk, int d, int causal, float scale, int dtype, void* stream)
{
    fa::FwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.B = B;
    a.H = H;
    a.Nq = Nq;
    a.Nk = Nk;
    a.d = d;
    a.causal = causal != 0;
    a.scale = scale;
    a.bf16 = dtype == FA_DTYPE_BF16;
    a.stream = (hipStream_t)stream;
    return a;
}

int hip_status(hipError_t e)
{
    if (e == hipSuccess) return FA_OK;
    snprintf(g_msg, sizeof g_msg, "HIP error %d: %s", (int)e, hipGetErrorString(e));
    return FA_ERR_HIP;
}

// Causal visible area below the diagonal in the pages' convention (N*N/2
// for a square problem).
double causal_area(double Nq, double Nk)
{
    return Nq <= Nk ? 0.5 * Nq * Nq : 0.5 * Nk * Nk + (Nq - Nk) * Nk;
}

// Device address of `scratch` on the current device, looked up with
// hipGetSymbolAddress on the first call there (with that device current) and
// kept per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_addr[kMaxDevices];

int noalloc_scratch(void** addr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kMaxDevices) return fail(FA_ERR_UNSUPPORTED, "device index past the scratch table (64)");
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e);
        if (!p) return fail(FA_ERR_HIP, "hipGetSymbolAddress returned no address for the scratch array");
        g_scratch_addr[dev] = p;
    }
    *addr = g_scratch_addr[dev];
    return FA_OK;
}

// Number of j in [a, b) that lie in [u0, u1) or in [w0, w1).
int64_t count_in_union(int64_t a, int64_t b, int64_t u0, int64_t u1, int64_t w0, int64_t w1)
{
    auto len = [a, b](int64_t lo, int64_t hi) {
        lo = lo > a ? lo : a;
        hi = hi < b ? hi : b;
        return hi > lo ? hi - lo : 0;
    };
    const int64_t both = len(u0 > w0 ? u0 : w0, u1 < w1 ? u1 : w1);
    return len(u0, u1) + len(w0, w1) - both;
}

// Masks of a plan (host values); key_len is the batch's key count.
struct PlanMasks {
    int64_t window_left, window_right, key_len;
};

// Blocks of 32 query rows x 64 keys for which the waves of the query tile at
// q0 execute S = Q K^T, plus those for which they execute P V, in a direct
// (unsplit) launch, following the forward kernel's loop (fa_fwd_kernel.h):
//  * the tile's key tiles are [jb, je), of which U = [u_lo, u_hi) run the
//    unmasked step, where every wave computes; in the other steps a wave
//    computes only the tiles W = [w_lo, n_wave) its own rows see;
//  * the scores of the first tile are computed before the loop, those of tile
//    j+1 in step j, and the P V of tile j in step j (the last tile in a step
//    of its own);
//  * a wave that fuses the exp work with the next scores computes the scores
//    of j+1 only in a step in which it computes tile j.
int64_t wave_blocks(int64_t q0, int waves, int64_t Nq, int64_t Nk, bool causal, const PlanMasks* m, int D,
                    int DC, bool padded)
{
    const int64_t BM = 32 * waves, BN = fa::block_n(D);
    int64_t jb, je, u_lo, u_hi;
    if (m) {
        const fa::MaskedSpan ms =
            fa::masked_span(q0, BM, BN, Nq, Nk, causal, m->window_left, m->window_right, m->key_len);
        jb = ms.first;
        je = ms.end;
        u_lo = ms.unmasked_begin;
        u_hi = ms.unmasked_end;
        if (jb == je) return 0;
    } else {
        const fa::TileSpan sp = fa::tile_span(q0, BM, BN, Nq, Nk, causal);
        jb = 0;
        je = sp.total;
        u_lo = 0;
        u_hi = sp.unmasked;
    }
    const bool fused = fa::fuses_exp(DC, waves, false, m != nullptr, padded);
    int64_t blocks = 0;
    for (int w = 0; w < waves; ++w) {
        int64_t n_wave = causal ? std::min(je, (q0 + (w + 1) * 32 - 1) / BN + 1) : je;
        int64_t w_lo = jb;
        if (m) {
            const int64_t r0 = q0 + w * 32;
            if (r0 >= Nq) {
                n_wave = jb;
            } else {
                const fa::MaskedSpan ws = fa::masked_span(r0, 32, BN, Nq, Nk, causal, m->window_left,
                                                          m->window_right, m->key_len);
                w_lo = std::max(jb, ws.first - (fused ? 1 : 0));
                n_wave = std::min(je, ws.end);
            }
        }
        const bool pre = (!m || (jb >= u_lo && jb < u_hi)) || (jb >= w_lo && jb < n_wave);
        const int64_t s_steps = fused ? count_in_union(jb, je - 1, u_lo, u_hi, w_lo, n_wave - 1)
                                      : count_in_union(jb, je - 1, u_lo, u_hi, w_lo - 1, n_wave - 1);
        const int64_t pv = count_in_union(jb, je, u_lo, u_hi, w_lo, n_wave);
        blocks += (pre ? 1 : 0) + s_steps + pv;
    }
    return blocks;
}

// FLOPs of one 32 x 64 block of S = Q K^T or of P V over the dims the
// forward kernel computes (d rounded up to 32).
double block_flops(int d) { return 2.0 * 32 * 64 * fa::compute_dim(d); }

int bwd_checked(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                void* dq, void* dk, void* dv, float* delta, int B, int H, int Nq, int Nk, int d, int causal,
                float scale, int dtype, const fa::MaskArgs* mask, void* stream)
{
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !delta)
        return fail(FA_ERR_INVALID_ARG, "NULL tensor pointer");
    const void* a16[] = {q, k, v, o, dout, dq, dk, dv, delta};
    for (const void* p : a16)
        if (!aligned(p, 16)) return fail(FA_ERR_INVALID_ARG, "tensors and delta must be 16-byte aligned");
    if (!aligned(lse, 4)) return fail(FA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
    const int rc = check_problem(B, H, Nq, Nk, d, causal, dtype);
    if (rc != FA_OK) return rc;
    if (!(scale > 0.f) || !isfinite(scale))
        return fail(FA_ERR_INVALID_ARG, "scale must be finite and > 0");
    // query side: q, o, dout, dq [Nq rows], lse and delta [Nq]; key side: k, v, dk, dv [Nk rows]
    const size_t qb = (size_t)B * H * Nq * d * 2, kb = (size_t)B * H * Nk * d * 2;
    const size_t lb = (size_t)B * H * Nq * 4;
    struct Buf {
        const void* p;
        size_t n;
    };
    const Buf ins[] = {{q, qb}, {k, kb}, {v, kb}, {o, qb}, {dout, qb}, {lse, lb}};
    const Buf outs[] = {{dq, qb}, {dk, kb}, {dv, kb}, {delta, lb}};
    for (const Buf& w : outs)
        for (const Buf& r : ins)
            if (overlap(w.p, w.n, r.p, r.n))
                return fail(FA_ERR_INVALID_ARG, "an output (dq, dk, dv or delta) overlaps an input");
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i].p, outs[i].n, outs[j].p, outs[j].n))
                return fail(FA_ERR_INVALID_ARG, "dq, dk, dv and delta overlap");
    if (mask) {
        const int rc2 = check_masks(B, H, Nq, d, mask->window_left, mask->window_right, mask->key_lens, dq,
                                    lse, nullptr, 0);
        if (rc2 != FA_OK) return rc2;
        const size_t nb = (size_t)B * 4;
        if (mask->key_lens && (overlap(mask->key_lens, nb, dk, kb) || overlap(mask->key_lens, nb, dv, kb) ||
                               overlap(mask->key_lens, nb, delta, lb)))
            return fail(FA_ERR_INVALID_ARG, "key_lens overlaps an output");
        if (masks_off(causal, mask->window_left, mask->window_right, mask->key_lens)) mask = nullptr;
    }
    return hip_status(fa::launch_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, Nq, Nk, d, causal != 0,
                                     scale, dtype == FA_DTYPE_BF16, mask, (hipStream_t)stream));
}


// Plan of a key-split launch (fa::uses_key_split): workgroups of 32 query
// rows and four waves, 32-key tiles each computed by one wave, so the MFMA
// work is S = Q K^T and P V of every visited 32 x 32 tile pair.
void key_split_plan(int B, int H, int Nq, int Nk, int d, int causal, fa_plan_t* plan)
{
    int64_t counts[4];
    fa_tile_counts_qk(Nq, Nk, 32, 32, causal, counts);
    const int64_t bh = (int64_t)B * H;
    plan->block_m = 32;
    plan->block_n = 32;
    plan->threads = 256;
    plan->lds_bytes = fa::ks_lds_bytes(d);
    plan->workgroups = bh * ((Nq + 31) / 32);
    plan->pairs_visited = bh * counts[1];
    plan->mfma_flops = 2.0 * (2.0 * 32 * 32 * fa::compute_dim(d)) * (double)counts[1] * (double)bh;
}

}  // namespace

extern "C" {

const char* fa_status_string(int status)
{
    switch (status) {
    case FA_OK:
        return "FA_OK";
    case FA_ERR_INVALID_ARG:
    case FA_ERR_UNSUPPORTED:
    case FA_ERR_HIP:
        return g_msg[0] ? g_msg : (status == FA_ERR_HIP ? "HIP error" : "invalid argument");
    default:
        return "unknown fa_status";
    }
}

int fa_tile_counts_qk(int64_t Nq, int64_t Nk, int block_m, int block_n, int causal,
                      int64_t counts[4])
{
    if (!counts || Nq < 1 || Nk < 1 || block_m < 1 || block_n < 1)
        return fail(FA_ERR_INVALID_ARG,
                    "fa_tile_counts: lengths and block sizes must be >= 1, counts non-NULL");
    const int64_t n_qt = (Nq + block_m - 1) / block_m, n_kt = (Nk + block_n - 1) / block_n;
    int64_t visited = 0, unmasked = 0;
    for (int64_t i = 0; i < n_qt; ++i) {
        const fa::TileSpan s = fa::tile_span(i * block_m, block_m, block_n, Nq, Nk, causal != 0);
        visited += s.total;
        unmasked += s.unmasked;
    }
    counts[0] = n_qt * n_kt;
    counts[1] = visited;
    counts[2] = unmasked;
    counts[3] = visited - unmasked;
    return FA_OK;
}

int fa_tile_counts(int64_t N, int block_m, int block_n, int causal, int64_t counts[4])
{
    return fa_tile_counts_qk(N, N, block_m, block_n, causal, counts);
}

int fa_plan_qk(int B, int H, int Nq, int Nk, int d, int causal, int dtype, fa_plan_t* plan)
{
    if (!plan) return fail(FA_ERR_INVALID_ARG, "plan is NULL");
    const int rc = check_problem(B, H, Nq, Nk, d, causal, dtype);
    if (rc != FA_OK) return rc;
    const double bh_all = (double)B * H;
    const double pairs_all = causal ? causal_area(Nq, Nk) : (double)Nq * (double)Nk;
    if (fa::uses_key_split(B, H, Nq, Nk, d, causal != 0)) {
        key_split_plan(B, H, Nq, Nk, d, causal, plan);
        plan->algo_flops = 4.0 * bh_all * pairs_all * d;
        plan->algo_bytes = 4.0 * bh_all * ((double)Nq + Nk) * d + 4.0 * bh_all * Nq;
        return FA_OK;
    }
    const fa::Shape sh = fa::pick_shape(B, H, Nq, d, causal != 0);
    const int bm = sh.block_m, bn = fa::block_n(d);
    int64_t counts[4];
    fa_tile_counts_qk(Nq, Nk, bm, bn, causal, counts);
    const int64_t bh = (int64_t)B * H;
    plan->block_m = bm;
    plan->block_n = bn;
    plan->threads = sh.threads;
    plan->lds_bytes = fa::lds_bytes(d, sh.waves, d >= 64, d == fa::kernel_dim(d) && sh.waves == 8);
    plan->workgroups = bh * ((Nq + bm - 1) / bm);
    plan->pairs_visited = bh * counts[1];
    // S = Q K^T and P V of every 32-row block a wave computes (waves skip the
    // causal tiles past their own rows), at the kernel's head dim
    const bool padded = d != fa::kernel_dim(d);
    int64_t blocks = 0;
    for (int64_t q0 = 0; q0 < Nq; q0 += bm)
        blocks += wave_blocks(q0, sh.waves, Nq, Nk, causal != 0, nullptr, fa::kernel_dim(d), fa::compute_dim(d),
                              padded);
    plan->mfma_flops = block_flops(d) * (double)blocks * (double)bh;
    const double pairs = causal ? causal_area(Nq, Nk) : (double)Nq * (double)Nk;
    plan->algo_flops = 4.0 * (double)bh * pairs * d;
    plan->algo_bytes = 4.0 * (double)bh * ((double)Nq + Nk) * d + 4.0 * (double)bh * Nq;
    return FA_OK;
}

int fa_tile_counts_masked(int64_t Nq, int64_t Nk, int block_m, int block_n, int causal,
                          int64_t window_left, int64_t window_right, int64_t key_len,
                          int64_t counts[4])
{
    g_msg[0] = 0;
    if (!counts || Nq < 1 || Nk < 1 || block_m < 1 || block_n < 1 || (causal != 0 && causal != 1) ||
        window_left < -1 || window_right < -1 || key_len < 0 || key_len > Nk)
        return fail(FA_ERR_INVALID_ARG, "fa_tile_counts_masked: invalid argument");
    const int64_t n_qt = (Nq + block_m - 1) / block_m, n_kt = (Nk + block_n - 1) / block_n;
    counts[0] = n_qt * n_kt;
    counts[1] = counts[2] = counts[3] = 0;
    for (int64_t i = 0; i < n_qt; ++i) {
        const fa::MaskedSpan s = fa::masked_span(i * block_m, block_m, block_n, Nq, Nk, causal != 0,
                                                 window_left, window_right, key_len);
        counts[1] += s.end - s.first;
        counts[2] += s.unmasked_end - s.unmasked_begin;
    }
    counts[3] = counts[1] - counts[2];
    return FA_OK;
}

int fa_plan_masked(int B, int H, int Nq, int Nk, int d, int causal, int window_left, int window_right,
                   const int32_t* key_lens, int dtype, fa_plan_t* plan)
{
    g_msg[0] = 0;
    if (!plan) return fail(FA_ERR_INVALID_ARG, "plan is NULL");
    const int rc = check_problem(B, H, Nq, Nk, d, causal, dtype);
    if (rc != FA_OK) return rc;
    if (window_left < -1 || window_right < -1)
        return fail(FA_ERR_INVALID_ARG, "window_left and window_right must be >= -1");
    if (key_lens)
        for (int b = 0; b < B; ++b)
            if (key_lens[b] < 0 || key_lens[b] > Nk)
                return fail(FA_ERR_INVALID_ARG, "key_lens values must lie in [0, Nk]");
    const bool off = masks_off(causal, window_left, window_right, key_lens);
    const fa::Shape sh = off ? fa::pick_shape(B, H, Nq, d, causal != 0)
                             : fa::pick_shape_masked(B, H, Nq, d, causal != 0);
    const int bm = sh.block_m, bn = fa::block_n(d);
    double pairs = 0, tiles = 0, keys_read = 0, blocks = 0;
    const bool padded = d != fa::kernel_dim(d);
    for (int b = 0; b < B; ++b) {
        const int64_t kl = key_lens ? key_lens[b] : Nk;
        int64_t counts[4];
        if (off)
            fa_tile_counts_qk(Nq, Nk, bm, bn, causal, counts);
        else
            fa_tile_counts_masked(Nq, Nk, bm, bn, causal, window_left, window_right, kl, counts);
        tiles += (double)counts[1];
        const PlanMasks pm{window_left, window_right, kl};
        for (int64_t q0 = 0; q0 < Nq; q0 += bm)
            blocks += (double)wave_blocks(q0, sh.waves, Nq, Nk, causal != 0, off ? nullptr : &pm,
                                          fa::kernel_dim(d), fa::compute_dim(d), padded);
        // visible (query, key) pairs, and the keys some row sees (the union
        // of the rows' ranges; lo and hi never decrease with the row)
        int64_t reach = 0;
        for (int64_t i = 0; i < Nq; ++i) {
            const fa::RowKeys r = fa::row_keys(i, Nk, causal != 0, window_left, window_right, kl);
            if (r.hi > r.lo) pairs += (double)(r.hi - r.lo);
            const int64_t from = r.lo > reach ? r.lo : reach;
            if (r.hi > from) keys_read += (double)(r.hi - from);
            if (r.hi > reach) reach = r.hi;
        }
    }
    plan->block_m = bm;
    plan->block_n = bn;
    plan->threads = sh.threads;
    plan->lds_bytes =
        fa::lds_bytes(d, sh.waves, d >= 64, off && d == fa::kernel_dim(d) && sh.waves == 8);
    plan->workgroups = (int64_t)B * H * ((Nq + bm - 1) / bm);
    plan->pairs_visited = (int64_t)(tiles * H);
    plan->mfma_flops = block_flops(d) * blocks * H;
    if (off && fa::uses_key_split(B, H, Nq, Nk, d, causal != 0))  // the launch the plain entry points take
        key_split_plan(B, H, Nq, Nk, d, causal, plan);
    plan->algo_flops = 4.0 * H * pairs * d;
    plan->algo_bytes = 4.0 * H * ((double)B * Nq + keys_read) * d + 4.0 * (double)B * H * Nq;
    return FA_OK;
}

int fa_plan(int B, int H, int N, int d, int causal, int dtype, fa_plan_t* plan)
{
    return fa_plan_qk(B, H, N, N, d, causal, dtype, plan);
}

int fa_fwd_qk(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
              int Nq, int Nk, int d, int causal, float scale, int dtype, void* stream)
{
    g_msg[0] = 0;
    const int rc = check_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype);
    if (rc != FA_OK) return rc;
    return hip_status(fa::launch_forward(fwd_args(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype,
                                                  stream)));
}

int fa_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                  int Nq, int Nk, int d, int causal, int window_left, int window_right,
                  const int32_t* key_lens, float scale, int dtype, void* stream)
{
    g_msg[0] = 0;
    int rc = check_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype);
    if (rc != FA_OK) return rc;
    rc = check_masks(B, H, Nq, d, window_left, window_right, key_lens, o, lse, nullptr, 0);
    if (rc != FA_OK) return rc;
    fa::FwdArgs a = fwd_args(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, stream);
    a.masked = !masks_off(causal, window_left, window_right, key_lens);
    a.mask = fa::MaskArgs{window_left, window_right, key_lens, H};
    return hip_status(fa::launch_forward(a));
}

int fa_split_count(int B, int H, int Nq, int Nk, int d, int causal)
{
    if (check_problem(B, H, Nq, Nk, d, causal, FA_DTYPE_BF16) != FA_OK) return 0;
    // Measured on MI355X (bf16, d = 64 and 128, B*H from 8 to 2048, 1 to
    // 4000 query rows, 512 to 16384 keys; every split count timed).
    //  * Under 16 key tiles the merge costs more than the split gains.
    //  * Causal: query row i sees keys [0, i], so the longest query tile sees
    //    min(Nq, Nk) keys; that is what a split could shorten.
    //  * Up to 32 query rows a workgroup has one computing wave and streams
    //    K/V: about 512 workgroups keep HBM busy, and chunks as short as two
    //    key tiles still pay. Small grids with long caches take 8 chunks,
    //    which also balances caches of different lengths (padding); grids
    //    past 128 tiles take 2 chunks from 64 key tiles on.
    //  * With more query rows every chunk writes fp32 partials of all its rows
    //    and the merge reads them back: the split and merge cost 5-12 us more
    //    than the direct launch, against 0.6 (d = 64) to 0.85 us (d = 128) per
    //    key tile taken off the longest workgroup. So at most 256 workgroups
    //    (one per CU; a second one on a CU shares its SIMDs and shortens
    //    nothing) and chunks of at least 16 key tiles, or 8 when the grid
    //    has at most 16 workgroups. At B2 H4 (8 heads, 8 to 63 query tiles
    //    each), N = 1000 to 4000, the direct launch is as fast or faster at
    //    every N; at B1 H2 N4096 d128 and B1 H1 N8192 d64 (64 workgroups) 4
    //    chunks take 0.5-0.6x its time, at B1 H16 Nq128 Nk1536 d128 (16
    //    workgroups) 8 chunks take 0.7x.
    const int64_t rows = fa::split_rows_per_tile();
    const int64_t rq = Nq < rows ? Nq : rows;
    const int64_t wgs = (int64_t)B * H * (((int64_t)Nq + rows - 1) / rows);
    const int64_t keys = causal && Nq < Nk ? Nq : Nk;
    const int64_t n_kt = (keys + 63) / 64;
    if (n_kt < 16) return 1;
    int64_t s;
    if (rq <= 32) {
        if (wgs <= 128) {
            s = (512 + wgs - 1) / wgs;
            const int64_t long_cache = n_kt / 16 < 8 ? n_kt / 16 : 8;
            if (s < long_cache) s = long_cache;
        } else {
            s = n_kt >= 64 ? 2 : 1;
        }
        if (s > n_kt / 2) s = n_kt / 2;
    } else {
        // the key-split kernel shortens the walk of small grids in one launch
        if (fa::uses_key_split(B, H, Nq, Nk, d, causal != 0)) return 1;
        s = 256 / wgs;
        const int64_t min_chunk = wgs <= 16 ? 8 : 16;
        if (s > n_kt / min_chunk) s = n_kt / min_chunk;
    }
    return (int)(s < 1 ? 1 : s);
}

int64_t fa_split_workspace_bytes(int B, int H, int Nq, int d, int n_splits)
{
    if (B < 1 || H < 1 || Nq < 1 || d < 8 || d > 128 || d % 8 != 0 || n_splits < 1) return 0;
    return (int64_t)n_splits * B * H * Nq * (fa::kernel_dim(d) + 1) * 4;
}

int fa_fwd_split_qk(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                    int Nq, int Nk, int d, int causal, float scale, int dtype, int n_splits,
                    void* workspace, int64_t workspace_bytes, void* stream)
{
    g_msg[0] = 0;
    int rc = check_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype);
    if (rc != FA_OK) return rc;
    rc = check_split(q, k, v, o, lse, B, H, Nq, Nk, d, n_splits, workspace, workspace_bytes);
    if (rc != FA_OK) return rc;
    fa::FwdArgs a = fwd_args(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, stream);
    a.split = true;
    a.n_splits = n_splits;
    a.workspace = (float*)workspace;
    return hip_status(fa::launch_forward(a));
}

int fa_fwd_split_qk_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                            int Nq, int Nk, int d, int causal, float scale, int dtype, int n_splits, void* stream)
{
    g_msg[0] = 0;
    int rc = check_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype);
    if (rc != FA_OK) return rc;
    if (n_splits < 1 || n_splits > (Nk + 63) / 64)
        return fail(FA_ERR_INVALID_ARG, "n_splits must be between 1 and ceil(Nk / 64)");
    if ((int64_t)B * H * ((Nq + 127) / 128) * n_splits > (int64_t)UINT32_MAX)
        return fail(FA_ERR_INVALID_ARG, "B*H*ceil(Nq/128)*n_splits exceeds the grid limit");
    const int64_t need = fa_split_workspace_bytes(B, H, Nq, d, n_splits);
    if (need > (int64_t)FA_NOALLOC_SCRATCH_BYTES)
        return fail(FA_ERR_UNSUPPORTED,
                    "the split workspace (n_splits*B*H*Nq*(D+1)*4 bytes) exceeds the static scratch "
                    "(FA_NOALLOC_SCRATCH_BYTES = 16 MiB); use fa_fwd_split_qk with a workspace");
    void* ws = nullptr;
    rc = noalloc_scratch(&ws);
    if (rc != FA_OK) return rc;
    fa::FwdArgs a = fwd_args(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, stream);
    a.split = true;
    a.n_splits = n_splits;
    a.workspace = (float*)ws;
    return hip_status(fa::launch_forward(a));
}

int fa_fwd_split_masked(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                        int H, int Nq, int Nk, int d, int causal, int window_left, int window_right,
                        const int32_t* key_lens, float scale, int dtype, int n_splits,
                        void* workspace, int64_t workspace_bytes, void* stream)
{
    g_msg[0] = 0;
    int rc = check_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype);
    if (rc != FA_OK) return rc;
    rc = check_split(q, k, v, o, lse, B, H, Nq, Nk, d, n_splits, workspace, workspace_bytes);
    if (rc != FA_OK) return rc;
    rc = check_masks(B, H, Nq, d, window_left, window_right, key_lens, o, lse, workspace,
                     workspace_bytes);
    if (rc != FA_OK) return rc;
    fa::FwdArgs a = fwd_args(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, stream);
    a.masked = !masks_off(causal, window_left, window_right, key_lens);
    a.mask = fa::MaskArgs{window_left, window_right, key_lens, H};
    a.split = true;
    a.n_splits = n_splits;
    a.workspace = (float*)workspace;
    return hip_status(fa::launch_forward(a));
}

int64_t fa_f32_workspace_bytes(int B, int H, int Nk, int d)
{
    if (B < 1 || H < 1 || Nk < 1 || (d != 64 && d != 128)) return 0;
    return (int64_t)8 * B * H * Nk * d;
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int Nq,
               int Nk, int d, int causal, float scale, void* workspace, int64_t workspace_bytes, void* stream)
{
    g_msg[0] = 0;
    if (!q || !k || !v || !o || !lse || !workspace)
        return fail(FA_ERR_INVALID_ARG, "NULL tensor or workspace pointer");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(workspace, 16))
        return fail(FA_ERR_INVALID_ARG, "q, k, v, o and the workspace must be 16-byte aligned");
    if (!aligned(lse, 4)) return fail(FA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
    const int rc = check_problem(B, H, Nq, Nk, d, causal, FA_DTYPE_BF16);
    if (rc != FA_OK) return rc;
    if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "fp32 inputs take head dim 64 or 128");
    if (!(scale > 0.f) || !isfinite(scale))
        return fail(FA_ERR_INVALID_ARG, "scale must be finite and > 0");
    const int64_t need = fa_f32_workspace_bytes(B, H, Nk, d);
    if (workspace_bytes < need) return fail(FA_ERR_INVALID_ARG, "workspace too small");
    if ((int64_t)Nk * d * 4 > (int64_t)UINT32_MAX)
        return fail(FA_ERR_INVALID_ARG, "one fp32 head (Nk*d*4 bytes) must be below 4 GiB");
    const size_t qb = (size_t)B * H * Nq * d * 4, kb = (size_t)B * H * Nk * d * 4;
    const size_t lb = (size_t)B * H * Nq * 4, wb = (size_t)need;
    if (overlap(o, qb, q, qb) || overlap(o, qb, k, kb) || overlap(o, qb, v, kb))
        return fail(FA_ERR_INVALID_ARG, "o overlaps q, k or v");
    if (overlap(lse, lb, q, qb) || overlap(lse, lb, k, kb) || overlap(lse, lb, v, kb) ||
        overlap(lse, lb, o, qb))
        return fail(FA_ERR_INVALID_ARG, "lse overlaps q, k, v or o");
    if (overlap(workspace, wb, q, qb) || overlap(workspace, wb, k, kb) || overlap(workspace, wb, v, kb) ||
        overlap(workspace, wb, o, qb) || overlap(workspace, wb, lse, lb))
        return fail(FA_ERR_INVALID_ARG, "the workspace overlaps a tensor argument");
    return hip_status(fa::launch_fwd_f32(q, k, v, o, lse, B, H, Nq, Nk, d, causal != 0, scale, workspace,
                                         (hipStream_t)stream));
}


int fa_bwd_qk(const void* q, const void* k, const void* v, const void* o, const void* dout,
              const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int H, int Nq, int Nk,
              int d, int causal, float scale, int dtype, void* stream)
{
    g_msg[0] = 0;
    return bwd_checked(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, Nq, Nk, d, causal, scale, dtype, nullptr,
                       stream);
}

int fa_bwd_masked(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int H, int Nq, int Nk,
                  int d, int causal, int window_left, int window_right, const int32_t* key_lens, float scale,
                  int dtype, void* stream)
{
    g_msg[0] = 0;
    const fa::MaskArgs mask{window_left, window_right, key_lens, H};
    return bwd_checked(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, Nq, Nk, d, causal, scale, dtype, &mask,
                       stream);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int H, int N, int d,
           int causal, float scale, int dtype, void* stream)
{
    return fa_bwd_qk(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, N, d, causal, scale, dtype, stream);
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
           int d, int causal, float scale, int dtype, void* stream)
{
    return fa_fwd_qk(q, k, v, o, lse, B, H, N, N, d, causal, scale, dtype, stream);
}

}  // extern "C"

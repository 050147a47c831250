/*
 * fa_oracle_bwd.c -- plain fp64 CPU reference for the attention backward pass.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite and the smoke check may load
 * this library. The GPU path never calls it, includes it or shares code with
 * it.
 *
 * The forward pass is O = softmax(scale * Q K^T [+ causal mask]) V, row by
 * row, with a causal row i seeing keys j <= min(i, Nk - 1) (the definition
 * fa_oracle.c follows). "How to optimise a Triton FlashAttention-2 kernel
 * step by step with a profiler" names the backward pass of FlashAttention-2
 * as the next kernel (closing list): it consumes the logsumexp the forward
 * writes and accumulates in two directions. Its result is the gradient of
 * the scalar sum(dO * O) with respect to Q, K and V for a given upstream
 * gradient dO, which for one head and the visible pairs (i, j) is the chain
 * rule through the softmax:
 *
 *   P_ij  = exp(s_ij) / sum_j' exp(s_ij'),   s_ij = scale * <q_i, k_j>
 *   dV_j  = sum_i P_ij dO_i
 *   dP_ij = <dO_i, v_j>
 *   D_i   = sum_j P_ij dP_ij  (= <dO_i, O_i>)
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale * sum_j dS_ij k_j
 *   dK_j  = scale * sum_i dS_ij q_i
 *
 * With padding lengths and sliding windows (fa_oracle_bwd_masked; the masks
 * of fa_oracle.c: key j is visible to row i of batch b iff j < key_len[b],
 * j >= i - window_left and j <= i (causal) or j <= i + window_right) the sums
 * run over each row's visible keys; a row that sees no key has O = 0, which
 * does not depend on q, k or v, so it adds nothing to any gradient and its
 * dQ is 0.
 *
 * P is formed here from this file's own fp64 softmax (max subtracted, two
 * passes), not from a stored logsumexp, and D from the fp64 O. Every product
 * and sum is in double; nothing is blocked or reordered beyond the steps
 * above. One thread owns one (b, h) head at a time, so the sums over rows
 * into dK and dV need no synchronisation.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const float *q, *k, *v, *dout;
    int64_t BH, H, Nq, Nk, d;
    int causal;
    int64_t win_left, win_right; /* -1: unbounded */
    const int64_t *key_lens;     /* NULL: every batch has Nk keys */
    double scale;
    double *dq, *dk, *dv;
    int64_t next;
    pthread_mutex_t lock;
    int status;
} bjob_t;

static int64_t visible(int64_t i, int64_t Nk, int causal)
{
    return causal ? (i + 1 < Nk ? i + 1 : Nk) : Nk;
}

/* The visible keys [*lo, *hi) of row i of batch b (hi <= lo: none). */
static void row_range(const bjob_t *job, int64_t b, int64_t i, int64_t *lo, int64_t *hi)
{
    int64_t h = visible(i, job->Nk, job->causal);
    if (!job->causal && job->win_right >= 0 && i + job->win_right + 1 < h)
        h = i + job->win_right + 1;
    if (job->key_lens && job->key_lens[b] < h)
        h = job->key_lens[b];
    int64_t l = 0;
    if (job->win_left >= 0 && i - job->win_left > 0)
        l = i - job->win_left;
    *lo = l;
    *hi = h;
}

static void head_bwd(const bjob_t *job, int64_t bh, double *p, double *dp, double *o)
{
    const int64_t Nq = job->Nq, Nk = job->Nk, d = job->d;
    const float *qh = job->q + bh * Nq * d, *kh = job->k + bh * Nk * d;
    const float *vh = job->v + bh * Nk * d, *doh = job->dout + bh * Nq * d;
    double *dqh = job->dq + bh * Nq * d, *dkh = job->dk + bh * Nk * d, *dvh = job->dv + bh * Nk * d;
    memset(dqh, 0, sizeof(double) * (size_t)(Nq * d));
    memset(dkh, 0, sizeof(double) * (size_t)(Nk * d));
    memset(dvh, 0, sizeof(double) * (size_t)(Nk * d));
    for (int64_t i = 0; i < Nq; ++i) {
        const float *qi = qh + i * d, *doi = doh + i * d;
        int64_t lo, hi;
        row_range(job, bh / job->H, i, &lo, &hi);
        if (hi <= lo)
            continue; /* no visible key: O_i = 0, no gradient */
        /* softmax row P_i. over the visible keys */
        double m = -INFINITY;
        for (int64_t j = lo; j < hi; ++j) {
            double acc = 0.0;
            for (int64_t c = 0; c < d; ++c)
                acc += (double)qi[c] * (double)kh[j * d + c];
            p[j] = job->scale * acc;
            if (p[j] > m)
                m = p[j];
        }
        double l = 0.0;
        for (int64_t j = lo; j < hi; ++j) {
            p[j] = exp(p[j] - m);
            l += p[j];
        }
        for (int64_t j = lo; j < hi; ++j)
            p[j] /= l;
        /* O_i and D_i = <dO_i, O_i> */
        for (int64_t c = 0; c < d; ++c)
            o[c] = 0.0;
        for (int64_t j = lo; j < hi; ++j)
            for (int64_t c = 0; c < d; ++c)
                o[c] += p[j] * (double)vh[j * d + c];
        double Di = 0.0;
        for (int64_t c = 0; c < d; ++c)
            Di += (double)doi[c] * o[c];
        /* dP_ij = <dO_i, v_j>; dS_ij = P_ij (dP_ij - D_i) */
        for (int64_t j = lo; j < hi; ++j) {
            double acc = 0.0;
            for (int64_t c = 0; c < d; ++c)
                acc += (double)doi[c] * (double)vh[j * d + c];
            dp[j] = p[j] * (acc - Di);
        }
        /* the three products */
        for (int64_t j = lo; j < hi; ++j) {
            for (int64_t c = 0; c < d; ++c) {
                dvh[j * d + c] += p[j] * (double)doi[c];
                dqh[i * d + c] += job->scale * dp[j] * (double)kh[j * d + c];
                dkh[j * d + c] += job->scale * dp[j] * (double)qi[c];
            }
        }
    }
}

static void *bworker(void *arg)
{
    bjob_t *job = (bjob_t *)arg;
    double *p = (double *)malloc(sizeof(double) * (size_t)job->Nk);
    double *dp = (double *)malloc(sizeof(double) * (size_t)job->Nk);
    double *o = (double *)malloc(sizeof(double) * (size_t)job->d);
    if (!p || !dp || !o) {
        pthread_mutex_lock(&job->lock);
        job->status = -2;
        pthread_mutex_unlock(&job->lock);
        free(p);
        free(dp);
        free(o);
        return NULL;
    }
    for (;;) {
        pthread_mutex_lock(&job->lock);
        int64_t bh = job->next++;
        pthread_mutex_unlock(&job->lock);
        if (bh >= job->BH)
            break;
        head_bwd(job, bh, p, dp, o);
    }
    free(p);
    free(dp);
    free(o);
    return NULL;
}

/*
 * fa_oracle_bwd_masked: dQ [B,H,Nq,d], dK and dV [B,H,Nk,d] (double) for
 * q [B,H,Nq,d], k, v [B,H,Nk,d] and dout [B,H,Nq,d] (fp32 arrays of
 * dtype-rounded values), with window_left / window_right (-1: unbounded;
 * window_right is not used when causal) and key_lens ([B] key counts in
 * 0..Nk, or NULL). Returns 0 on success, -1 on a bad argument, -2 when memory
 * runs out.
 */
int fa_oracle_bwd_masked(const float *q, const float *k, const float *v, const float *dout, int64_t B,
                         int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                         int64_t window_left, int64_t window_right, const int64_t *key_lens,
                         double scale, double *dq, double *dk, double *dv, int nthreads);

/* fa_oracle_bwd: fa_oracle_bwd_masked without masks. */
int fa_oracle_bwd(const float *q, const float *k, const float *v, const float *dout, int64_t B,
                  int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal, double scale,
                  double *dq, double *dk, double *dv, int nthreads)
{
    return fa_oracle_bwd_masked(q, k, v, dout, B, H, Nq, Nk, d, causal, -1, -1, NULL, scale, dq, dk,
                                dv, nthreads);
}

int fa_oracle_bwd_masked(const float *q, const float *k, const float *v, const float *dout, int64_t B,
                         int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                         int64_t window_left, int64_t window_right, const int64_t *key_lens,
                         double scale, double *dq, double *dk, double *dv, int nthreads)
{
    if (!q || !k || !v || !dout || !dq || !dk || !dv || B < 1 || H < 1 || Nq < 1 || Nk < 1 ||
        d < 1 || window_left < -1 || window_right < -1)
        return -1;
    if (key_lens)
        for (int64_t b = 0; b < B; ++b)
            if (key_lens[b] < 0 || key_lens[b] > Nk)
                return -1;
    bjob_t job;
    memset(&job, 0, sizeof(job));
    job.q = q;
    job.k = k;
    job.v = v;
    job.dout = dout;
    job.BH = B * H;
    job.H = H;
    job.win_left = window_left;
    job.win_right = window_right;
    job.key_lens = key_lens;
    job.Nq = Nq;
    job.Nk = Nk;
    job.d = d;
    job.causal = causal ? 1 : 0;
    job.scale = scale;
    job.dq = dq;
    job.dk = dk;
    job.dv = dv;
    pthread_mutex_init(&job.lock, NULL);
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > job.BH)
        nthreads = (int)job.BH;
    pthread_t *tids = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!tids) {
        pthread_mutex_destroy(&job.lock);
        return -2;
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tids[t], NULL, bworker, &job) != 0)
            break;
        ++started;
    }
    bworker(&job);
    for (int t = 1; t <= started; ++t)
        pthread_join(tids[t], NULL);
    free(tids);
    pthread_mutex_destroy(&job.lock);
    return job.status;
}

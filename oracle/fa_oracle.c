/*
 * fa_oracle.c -- plain fp64 CPU reference for the attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * bench's CPU-baseline leg may load this library. The GPU path never calls
 * it, includes it or shares code with it.
 *
 * What it computes, per batch b, head h and query row i (all independent),
 * for Nq query rows attending to Nk keys (Nq = Nk for self-attention):
 *
 *   s_j   = scale * sum_c q[b,h,i,c] * k[b,h,j,c]      for visible keys j
 *   O_i   = sum_j softmax(s)_j * v[b,h,j,:]
 *   lse_i = ln sum_j exp(s_j)
 *
 * The definition of attention with its scale applied to Q.K^T before the
 * softmax is the one in "Programming an attention kernel in Triton",
 * section "Kernel 4: bringing it together, a self-attention kernel"; the
 * max subtraction before the exponential is from the same page, "Kernel 3:
 * fused softmax". Every row sees keys 0..Nk-1, and a causal row i sees keys
 * j <= i among them: the keep test of the causal mask in "How to optimise a
 * Triton FlashAttention-2 kernel step by step with a profiler", Round 4,
 * "Causal tile-skipping", compares absolute key and query positions and
 * bounds keys by the key count, so with Nq != Nk the diagonal starts at the
 * top-left corner (row i >= Nk sees every key). Mismatched query and key
 * lengths are the shapes "Programming an attention kernel in Triton"
 * validates in "Kernel 4".
 *
 * Masks (fa_oracle_fwd_masked). "How to optimise a Triton FlashAttention-2
 * kernel step by step with a profiler", section "Future articles", notes that
 * a kernel with padding masks or sliding windows must handle rows with no
 * visible key, which its finite mask sentinel does not. Here a key is visible to row i
 * of batch b iff j < key_len[b] (padding), j >= i - window_left (when
 * window_left >= 0) and j <= i (causal) or j <= i + window_right (when not
 * causal and window_right >= 0). The visible keys of a row are one
 * contiguous range. A row with none has O = 0 and lse = -infinity (the sum
 * of no exponentials), which is the rule this oracle fixes for that case.
 *
 * The per-row
 * logsumexp is stored in natural-log units (same page, Round 4, "exp2": the
 * kernel converts its base-2 state back because its tests compare against a
 * natural-log logsumexp).
 *
 * Two evaluation orders are provided:
 *   - two-pass (tile_n == 0): all scores of a row, then their max, then the
 *     exponentials and the weighted sum. This is the plain definition.
 *   - online over key tiles (tile_n > 0): a running max m, running sum l and
 *     unnormalised output O, rescaled whenever a tile raises the max; the
 *     method named at the end of "Programming an attention kernel in
 *     Triton" ("The wall, named honestly") and kept as fp32 state by the
 *     FlashAttention-2 kernel of the profiler page ("Where the last article
 *     left off"). In exact arithmetic both orders give the same result.
 *
 * Inputs are fp32 arrays holding values that were already rounded to the
 * storage dtype (fp16/bf16 values are exact in fp32); every product and sum
 * is carried out in double. Nothing here is blocked, fused or reordered
 * beyond the steps named above.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ROWS_PER_ITEM 16

typedef struct {
    const float *q, *k, *v;
    int64_t B, H, Nq, Nk, d;
    int causal;
    double scale;
    const int64_t *rows; /* NULL: all rows 0..N-1 */
    int64_t win_left, win_right; /* -1: unbounded */
    const int64_t *key_lens;     /* NULL: every batch has Nk keys */
    int64_t n_rows;      /* rows per (b, h) in the output */
    int64_t tile_n;      /* 0: two-pass; > 0: online over key tiles */
    double *o, *lse;
    int64_t n_items;
    int64_t next_item; /* shared work counter */
    pthread_mutex_t lock;
    int status;
} job_t;

/* Score of query row i against key row j: scale * <q_i, k_j>, in double. */
static double score(const float *qi, const float *kj, int64_t d, double scale)
{
    double acc = 0.0;
    for (int64_t c = 0; c < d; ++c)
        acc += (double)qi[c] * (double)kj[c];
    return scale * acc;
}

/* Number of keys row i may attend to: all Nk, or keys 0..min(i, Nk-1) when
 * causal. */
static int64_t visible_keys(int64_t i, int64_t Nk, int causal)
{
    return causal ? (i + 1 < Nk ? i + 1 : Nk) : Nk;
}

/* The visible keys [*lo, *hi) of row i under the masks (see the header). */
static void visible_range(const job_t *job, int64_t b, int64_t i, int64_t *lo, int64_t *hi)
{
    int64_t h = visible_keys(i, job->Nk, job->causal);
    if (!job->causal && job->win_right >= 0 && i + job->win_right + 1 < h)
        h = i + job->win_right + 1;
    if (job->key_lens && job->key_lens[b] < h)
        h = job->key_lens[b];
    int64_t l = 0;
    if (job->win_left >= 0 && i - job->win_left > 0)
        l = i - job->win_left;
    *lo = l;
    *hi = h > l ? h : l;
}

/* The plain definition, evaluated in two passes over the scores. */
static void row_two_pass(const float *qi, const float *kh, const float *vh,
                         int64_t nvis, int64_t d, double scale, double *s,
                         double *o_row, double *lse_out)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < nvis; ++j) {
        s[j] = score(qi, kh + j * d, d, scale);
        if (s[j] > m)
            m = s[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < nvis; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    for (int64_t c = 0; c < d; ++c)
        o_row[c] = 0.0;
    for (int64_t j = 0; j < nvis; ++j) {
        const float *vj = vh + j * d;
        for (int64_t c = 0; c < d; ++c)
            o_row[c] += s[j] * (double)vj[c];
    }
    for (int64_t c = 0; c < d; ++c)
        o_row[c] /= l;
    *lse_out = m + log(l);
}

/* The same quantity with the online softmax: key tiles [t0, t0 + tile_n) in
 * order, each folded into the running (m, l, O). Keys at or past nvis are
 * masked out; a tile with no visible key is not visited. */
static void row_online(const float *qi, const float *kh, const float *vh,
                       int64_t nvis, int64_t d, double scale, int64_t tile_n,
                       double *s, double *o_row, double *lse_out)
{
    double m = 0.0, l = 0.0;
    int started = 0;
    for (int64_t c = 0; c < d; ++c)
        o_row[c] = 0.0;
    for (int64_t t0 = 0; t0 < nvis; t0 += tile_n) {
        int64_t t1 = t0 + tile_n < nvis ? t0 + tile_n : nvis;
        double m_tile = -INFINITY;
        for (int64_t j = t0; j < t1; ++j) {
            s[j - t0] = score(qi, kh + j * d, d, scale);
            if (s[j - t0] > m_tile)
                m_tile = s[j - t0];
        }
        double m_new = (!started || m_tile > m) ? m_tile : m;
        double alpha = started ? exp(m - m_new) : 0.0;
        l *= alpha;
        for (int64_t c = 0; c < d; ++c)
            o_row[c] *= alpha;
        for (int64_t j = t0; j < t1; ++j) {
            double p = exp(s[j - t0] - m_new);
            const float *vj = vh + j * d;
            l += p;
            for (int64_t c = 0; c < d; ++c)
                o_row[c] += p * (double)vj[c];
        }
        m = m_new;
        started = 1;
    }
    for (int64_t c = 0; c < d; ++c)
        o_row[c] /= l;
    *lse_out = m + log(l);
}

static void *worker(void *arg)
{
    job_t *job = (job_t *)arg;
    const int64_t d = job->d, Nq = job->Nq, Nk = job->Nk;
    int64_t scratch_n = job->tile_n > 0 ? job->tile_n : Nk;
    double *s = (double *)malloc(sizeof(double) * (size_t)scratch_n);
    if (!s) {
        pthread_mutex_lock(&job->lock);
        job->status = -2;
        pthread_mutex_unlock(&job->lock);
        return NULL;
    }
    const int64_t chunks = (job->n_rows + ROWS_PER_ITEM - 1) / ROWS_PER_ITEM;
    for (;;) {
        pthread_mutex_lock(&job->lock);
        int64_t item = job->next_item++;
        pthread_mutex_unlock(&job->lock);
        if (item >= job->n_items)
            break;
        int64_t bh = item / chunks;
        int64_t r0 = (item % chunks) * ROWS_PER_ITEM;
        int64_t r1 = r0 + ROWS_PER_ITEM < job->n_rows ? r0 + ROWS_PER_ITEM : job->n_rows;
        const float *qh = job->q + bh * Nq * d;
        const float *kh = job->k + bh * Nk * d;
        const float *vh = job->v + bh * Nk * d;
        for (int64_t r = r0; r < r1; ++r) {
            int64_t i = job->rows ? job->rows[r] : r;
            int64_t nvis = visible_keys(i, Nk, job->causal);
            double *o_row = job->o + (bh * job->n_rows + r) * d;
            double *lse_out = job->lse + bh * job->n_rows + r;
            int64_t k_lo = 0;
            if (job->win_left >= 0 || job->win_right >= 0 || job->key_lens) {
                int64_t k_hi;
                visible_range(job, bh / job->H, i, &k_lo, &k_hi);
                nvis = k_hi - k_lo;
                if (nvis == 0) { /* no visible key: O = 0, lse = -inf */
                    for (int64_t c = 0; c < d; ++c)
                        o_row[c] = 0.0;
                    *lse_out = -INFINITY;
                    continue;
                }
            }
            const float *kv0 = kh + k_lo * d, *vv0 = vh + k_lo * d;
            if (job->tile_n > 0)
                row_online(qh + i * d, kv0, vv0, nvis, d, job->scale, job->tile_n, s, o_row,
                           lse_out);
            else
                row_two_pass(qh + i * d, kv0, vv0, nvis, d, job->scale, s, o_row, lse_out);
        }
    }
    free(s);
    return NULL;
}

/*
 * fa_oracle_fwd_qk: O and lse for the query rows listed in `rows` (NULL =
 * every row) of every (b, h).
 *   q       : fp32, [B, H, Nq, d] contiguous (dtype-rounded values).
 *   k, v    : fp32, [B, H, Nk, d] contiguous.
 *   o       : double, [B, H, R, d] with R = n_rows (or Nq when rows is NULL).
 *   lse     : double, [B, H, R], natural log.
 *   tile_n  : 0 for the two-pass definition, > 0 for the online order.
 * Returns 0 on success, -1 on a bad argument, -2 when memory runs out.
 */
int fa_oracle_fwd_masked(const float *q, const float *k, const float *v, int64_t B, int64_t H,
                         int64_t Nq, int64_t Nk, int64_t d, int causal, int64_t window_left,
                         int64_t window_right, const int64_t *key_lens, double scale,
                         const int64_t *rows, int64_t n_rows, int64_t tile_n, double *o,
                         double *lse, int nthreads);

int fa_oracle_fwd_qk(const float *q, const float *k, const float *v, int64_t B, int64_t H,
                     int64_t Nq, int64_t Nk, int64_t d, int causal, double scale,
                     const int64_t *rows, int64_t n_rows, int64_t tile_n, double *o, double *lse,
                     int nthreads)
{
    return fa_oracle_fwd_masked(q, k, v, B, H, Nq, Nk, d, causal, -1, -1, NULL, scale, rows,
                                n_rows, tile_n, o, lse, nthreads);
}

/*
 * fa_oracle_fwd_masked: fa_oracle_fwd_qk with the masks of the header:
 * window_left / window_right (-1: unbounded; window_right is not used when
 * causal) and key_lens ([B] key counts, each in 0..Nk, or NULL).
 */
int fa_oracle_fwd_masked(const float *q, const float *k, const float *v, int64_t B, int64_t H,
                         int64_t Nq, int64_t Nk, int64_t d, int causal, int64_t window_left,
                         int64_t window_right, const int64_t *key_lens, double scale,
                         const int64_t *rows, int64_t n_rows, int64_t tile_n, double *o,
                         double *lse, int nthreads)
{
    if (window_left < -1 || window_right < -1)
        return -1;
    if (key_lens)
        for (int64_t b = 0; b < B; ++b)
            if (key_lens[b] < 0 || key_lens[b] > Nk)
                return -1;
    if (!q || !k || !v || !o || !lse || B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1 ||
        tile_n < 0)
        return -1;
    if (rows) {
        if (n_rows < 1)
            return -1;
        for (int64_t r = 0; r < n_rows; ++r)
            if (rows[r] < 0 || rows[r] >= Nq)
                return -1;
    } else {
        n_rows = Nq;
    }
    if (nthreads < 1)
        nthreads = 1;
    job_t job;
    memset(&job, 0, sizeof(job));
    job.q = q;
    job.k = k;
    job.v = v;
    job.B = B;
    job.H = H;
    job.Nq = Nq;
    job.Nk = Nk;
    job.win_left = window_left;
    job.win_right = window_right;
    job.key_lens = key_lens;
    job.d = d;
    job.causal = causal ? 1 : 0;
    job.scale = scale;
    job.rows = rows;
    job.n_rows = n_rows;
    job.tile_n = tile_n;
    job.o = o;
    job.lse = lse;
    job.n_items = B * H * ((n_rows + ROWS_PER_ITEM - 1) / ROWS_PER_ITEM);
    pthread_mutex_init(&job.lock, NULL);
    if (nthreads > job.n_items)
        nthreads = (int)job.n_items;
    pthread_t *tids = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!tids) {
        pthread_mutex_destroy(&job.lock);
        return -2;
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tids[t], NULL, worker, &job) != 0)
            break;
        ++started;
    }
    worker(&job);
    for (int t = 1; t <= started; ++t)
        pthread_join(tids[t], NULL);
    free(tids);
    pthread_mutex_destroy(&job.lock);
    return job.status;
}

/* fa_oracle_fwd: the self-attention case, Nq = Nk = N. */
int fa_oracle_fwd(const float *q, const float *k, const float *v, int64_t B, int64_t H,
                  int64_t N, int64_t d, int causal, double scale, const int64_t *rows,
                  int64_t n_rows, int64_t tile_n, double *o, double *lse, int nthreads)
{
    return fa_oracle_fwd_qk(q, k, v, B, H, N, N, d, causal, scale, rows, n_rows, tile_n, o, lse,
                            nthreads);
}

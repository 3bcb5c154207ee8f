/*
 * gqa_oracle.c -- float64 CPU oracle for causal grouped-query attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
 * definition that the HIP library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no code, header, table or helper with the GPU library, and the GPU library
 * never calls it.
 *
 * What it computes (one definition, written out):
 *
 *   For batch b, query head h and query row i, the key/value head is
 *   g = h / G with G = Hq / Hkv: consecutive query heads share one K/V head,
 *   the grouping that repeat_interleave(group_size) produces ("Grouped-Query
 *   Attention", section 5.1 "Queries, keys, and the shared group"; the same
 *   head mapping kvHead = h / groupSize appears in runCausalCachedHeads of
 *   makarna's attention_cached.go).
 *
 *   Query row i sits at absolute position p_i = pos0 + i.  Full-sequence
 *   prefill has pos0 = 0; cached decode has pos0 = startPos, the position of
 *   the first new token, and the key limit is p_i + 1 (makarna,
 *   CausalAttentionCached / runCausalCachedHeads: maxKeyPos = startPos+qi+1).
 *
 *   allowed(i,j) = !causal || j <= p_i     (Hesper "Causal Masking": 0 on and
 *                                           below the diagonal, -inf above)
 *                  and, with a local window W >= 1 (causal only),
 *                  j >= p_i - W + 1        (the multi-query primer's local
 *                                           attention, section 4.1: the current
 *                                           position and the W-1 before it)
 *   s_ij = scale * sum_d q[b,h,i,d] * k[b,g,j,d]
 *                                          (Riftco "Dataflow and shapes":
 *                                           scores = Q K^T / sqrt(d_h))
 *   m_i  = max over allowed j of s_ij
 *   w_ij = exp(s_ij - m_i) if allowed else exactly 0
 *   P_ij = w_ij / sum_j w_ij               (softmax over the key axis; masked
 *                                           entries get probability exactly 0,
 *                                           Riftco "The causal mask")
 *   out[b,h,i,:] = sum_j P_ij * v[b,g,j,:] (Riftco "Dataflow and shapes":
 *                                           context = probabilities @ values)
 *
 * Subtracting m_i before exp does not change P in exact arithmetic; it keeps
 * exp finite.  Everything is float64 with libm exp.  The full score row is
 * materialized (length Tk) before the softmax, as the "materialized"
 * algorithm of Riftco's "Two exact full-sequence algorithms" does; no tiling,
 * no online recurrence.
 *
 * Layout: q and out are [B, Hq, Tq, d]; k and v are [B, Hkv, Tk, d]; all
 * contiguous row-major float64.  Work is spread over threads by independent
 * (b, h) units, as makarna splits query heads over goroutines; each unit runs
 * the definition above unchanged.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
    const double *q, *k, *v;
    double *out;   /* [B,Hq,Tq,d] context, or NULL */
    double *probs; /* [B,Hq,Tq,Tk] probabilities, or NULL */
    int B, Hq, Hkv, Tq, Tk, d, causal;
    long pos0;
    long window; /* 0: no window */
    double scale;
    int nthreads;
    int tid;
} job_t;

/* The mask: may query position p see key j? */
static int allowed(const job_t *J, long p, long j) {
    if (J->causal && j > p) return 0;
    if (J->window > 0 && j < p - J->window + 1) return 0;
    return 1;
}

/* One (b, h) unit: every query row of query head h in batch b. */
static void run_unit(const job_t *J, int b, int h, double *row) {
    const int G = J->Hq / J->Hkv;
    const int g = h / G;
    const int d = J->d, Tq = J->Tq, Tk = J->Tk;
    const double *qh = J->q + ((size_t)b * J->Hq + h) * (size_t)Tq * d;
    const double *kg = J->k + ((size_t)b * J->Hkv + g) * (size_t)Tk * d;
    const double *vg = J->v + ((size_t)b * J->Hkv + g) * (size_t)Tk * d;
    for (int i = 0; i < Tq; ++i) {
        const long p = J->pos0 + i;
        const double *qi = qh + (size_t)i * d;
        /* scores of the allowed keys; the row is materialized in full */
        double m = -INFINITY;
        for (int j = 0; j < Tk; ++j) {
            if (!allowed(J, p, j)) {
                row[j] = -INFINITY; /* additive -inf mask */
                continue;
            }
            const double *kj = kg + (size_t)j * d;
            double s = 0.0;
            for (int e = 0; e < d; ++e) s += qi[e] * kj[e];
            s *= J->scale;
            row[j] = s;
            if (s > m) m = s;
        }
        /* softmax over the key axis: masked entries are exactly zero */
        double denom = 0.0;
        for (int j = 0; j < Tk; ++j) {
            row[j] = allowed(J, p, j) ? exp(row[j] - m) : 0.0;
            denom += row[j];
        }
        for (int j = 0; j < Tk; ++j) row[j] = row[j] / denom;
        if (J->probs) {
            double *pr = J->probs + (((size_t)b * J->Hq + h) * Tq + i) * (size_t)Tk;
            memcpy(pr, row, sizeof(double) * (size_t)Tk);
        }
        if (J->out) {
            double *o = J->out + (((size_t)b * J->Hq + h) * Tq + i) * (size_t)d;
            for (int e = 0; e < d; ++e) o[e] = 0.0;
            /* the sum runs over allowed keys only: a masked key's value row is
             * never read, so nothing after position p_i can reach row i (the
             * makarna loop stops at maxKeyPos the same way) */
            for (int j = 0; j < Tk; ++j) {
                if (!allowed(J, p, j)) continue;
                const double pj = row[j];
                const double *vj = vg + (size_t)j * d;
                for (int e = 0; e < d; ++e) o[e] += pj * vj[e];
            }
        }
    }
}

static void *worker(void *arg) {
    const job_t *J = (const job_t *)arg;
    double *row = (double *)malloc(sizeof(double) * (size_t)(J->Tk > 0 ? J->Tk : 1));
    if (!row) return (void *)1;
    const int units = J->B * J->Hq;
    for (int u = J->tid; u < units; u += J->nthreads) run_unit(J, u / J->Hq, u % J->Hq, row);
    free(row);
    return NULL;
}

/*
 * Returns 0 on success, -1 on invalid arguments, -2 on allocation/thread
 * failure.  nthreads <= 0 means one thread per online CPU.
 */
int oracle_attention(const double *q, const double *k, const double *v, double *out, double *probs,
                     int B, int Hq, int Hkv, int Tq, int Tk, int d, double scale, int causal,
                     long pos0, long window, int nthreads) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Tq < 0 || Tk < 0 || d <= 0 || Hq % Hkv != 0) return -1;
    if (causal != 0 && causal != 1) return -1;
    /* a local window is a restriction of causal attention; key p_i stays visible */
    if (window < 0 || (window > 0 && !causal)) return -1;
    /* every query row must have at least one allowed key */
    if (causal && Tq > 0 && (pos0 < 0 || pos0 + Tq > Tk)) return -1;
    if (!causal && Tq > 0 && Tk == 0) return -1;
    if (B == 0 || Tq == 0) return 0;
    if (nthreads <= 0) {
        long n = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = n > 0 ? (int)n : 1;
    }
    const int units = B * Hq;
    if (nthreads > units) nthreads = units;
    job_t *jobs = (job_t *)calloc((size_t)nthreads, sizeof(job_t));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return -2;
    }
    int rc = 0, started = 0;
    for (int t = 0; t < nthreads; ++t) {
        job_t J = {q, k, v, out, probs, B, Hq, Hkv, Tq, Tk, d, causal, pos0, window, scale, nthreads, t};
        jobs[t] = J;
        if (pthread_create(&th[t], NULL, worker, &jobs[t]) != 0) {
            rc = -2;
            break;
        }
        ++started;
    }
    for (int t = 0; t < started; ++t) {
        void *ret = NULL;
        pthread_join(th[t], &ret);
        if (ret) rc = -2;
    }
    free(jobs);
    free(th);
    return rc;
}

/* Number of threads oracle_attention would use for nthreads <= 0. */
int oracle_default_threads(void) {
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

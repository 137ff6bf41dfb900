/*
 * fp64 CPU oracle for the Kimi Delta Attention (KDA) recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the GPU product path may include,
 * link or call this file; only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark use it.  It shares no code with the HIP
 * library.
 *
 * What it computes (Kimi K3 technical-report digest on discuss.pytorch.kr,
 * section "Kimi Delta Attention", the per-head update equation):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t
 *
 * with q_t, k_t in R^{dk}, v_t in R^{dv}, S_t in R^{dk x dv}, alpha_t in
 * (0,1)^{dk} a per-key-channel retention and beta_t a scalar write strength
 * (same section, the sentence after the equation).  alpha_t is passed as its
 * logarithm g_t = log alpha_t (the bounded-decay section writes the gate as
 * g and alpha = exp(g)).
 *
 * The three stages follow the order the explainer on digitalbourgeois.tistory
 * ("How does KDA manage old information?") names: forget (decay), erase, write.
 *   forget: P = Diag(alpha_t) S_{t-1}          -- scales row i by alpha_{t,i}
 *   erase : E = (I - beta k k^T) P = P - beta k (k^T P)
 *   write : S_t = E + beta k v^T
 *   read  : o_t = S_t^T q_t                     -- uses the updated state
 * Each stage is the matrix product of the equation, evaluated with the
 * identity (I - beta k k^T) P = P - k (beta k^T P), so no dk x dk matrix is
 * formed.  This is the plain token-by-token definition: no chunking, no
 * blocking, no reordering of the sum beyond the loop order written here.
 *
 * All arithmetic is IEEE double.  Inputs arrive already widened to double by
 * the caller (bf16 and fp32 values widen exactly).
 *
 * Layouts (row-major, contiguous):
 *   q, k, g : [N, H, dk]      v : [N, H, dv]      beta : [N, H]
 *   cu_seqlens : int64 [nseq + 1], non-decreasing, cu[0] = 0, cu[nseq] = N
 *   init  : [nseq, H, dk, dv] or NULL (zero initial state)
 *   o     : [N, H, dv]        final : [nseq, H, dk, dv] (may be NULL)
 * Decode uses the same step on [B, H, ...] inputs and an in/out state
 * [B, H, dk, dv].
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* One token of the recurrence on the state S (dk x dv, row-major), in place.
 * Writes o (length dv).  scratch holds dv doubles. */
static void kda_token_step(double *S, int64_t dk, int64_t dv,
                           const double *q, const double *k, const double *v,
                           const double *g, double beta, double *o,
                           double *scratch) {
    /* forget: P = Diag(alpha) S, alpha_i = exp(g_i) scales key-channel row i */
    for (int64_t i = 0; i < dk; ++i) {
        const double a = exp(g[i]);
        double *row = S + i * dv;
        for (int64_t j = 0; j < dv; ++j) row[j] *= a;
    }
    /* erase: P <- P - k (beta k^T P);  kp = k^T P is a row vector of length dv */
    double *kp = scratch;
    for (int64_t j = 0; j < dv; ++j) kp[j] = 0.0;
    for (int64_t i = 0; i < dk; ++i) {
        const double *row = S + i * dv;
        for (int64_t j = 0; j < dv; ++j) kp[j] += k[i] * row[j];
    }
    for (int64_t i = 0; i < dk; ++i) {
        double *row = S + i * dv;
        const double bk = beta * k[i];
        for (int64_t j = 0; j < dv; ++j) row[j] -= bk * kp[j];
    }
    /* write: S <- E + beta k v^T */
    for (int64_t i = 0; i < dk; ++i) {
        double *row = S + i * dv;
        const double bk = beta * k[i];
        for (int64_t j = 0; j < dv; ++j) row[j] += bk * v[j];
    }
    /* read: o = S_t^T q */
    for (int64_t j = 0; j < dv; ++j) o[j] = 0.0;
    for (int64_t i = 0; i < dk; ++i) {
        const double *row = S + i * dv;
        for (int64_t j = 0; j < dv; ++j) o[j] += q[i] * row[j];
    }
}

typedef struct {
    const double *q, *k, *v, *g, *beta, *init;
    const int64_t *cu;
    int64_t nseq, H, dk, dv;
    double *o, *final_state;
    int64_t next_task;            /* shared work counter, guarded by lock */
    pthread_mutex_t lock;
    int decode;                   /* 1: one token per (b, h), state in/out */
    double *state;                /* decode: [B, H, dk, dv] */
} oracle_job;

static int64_t take_task(oracle_job *job) {
    pthread_mutex_lock(&job->lock);
    const int64_t t = job->next_task++;
    pthread_mutex_unlock(&job->lock);
    return t;
}

static void *worker(void *arg) {
    oracle_job *job = (oracle_job *)arg;
    const int64_t H = job->H, dk = job->dk, dv = job->dv;
    const int64_t ntask = job->nseq * H;
    double *S = (double *)malloc(sizeof(double) * (size_t)(dk * dv));
    double *scratch = (double *)malloc(sizeof(double) * (size_t)dv);
    if (!S || !scratch) { free(S); free(scratch); return (void *)1; }
    for (;;) {
        const int64_t task = take_task(job);
        if (task >= ntask) break;
        const int64_t s = task / H, h = task % H;
        if (job->decode) {
            /* decode: sequence s is batch row b; exactly one token. */
            double *st = job->state + (s * H + h) * dk * dv;
            const int64_t r = s * H + h;
            kda_token_step(st, dk, dv, job->q + r * dk, job->k + r * dk,
                           job->v + r * dv, job->g + r * dk, job->beta[r],
                           job->o + r * dv, scratch);
            continue;
        }
        if (job->init) memcpy(S, job->init + (s * H + h) * dk * dv, sizeof(double) * (size_t)(dk * dv));
        else memset(S, 0, sizeof(double) * (size_t)(dk * dv));
        for (int64_t t = job->cu[s]; t < job->cu[s + 1]; ++t) {
            const int64_t r = t * H + h;
            kda_token_step(S, dk, dv, job->q + r * dk, job->k + r * dk,
                           job->v + r * dv, job->g + r * dk, job->beta[r],
                           job->o + r * dv, scratch);
        }
        if (job->final_state)
            memcpy(job->final_state + (s * H + h) * dk * dv, S, sizeof(double) * (size_t)(dk * dv));
    }
    free(S);
    free(scratch);
    return NULL;
}

static int run_job(oracle_job *job, int nthreads) {
    if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    const int64_t ntask = job->nseq * job->H;
    if (nthreads > ntask) nthreads = (int)(ntask > 0 ? ntask : 1);
    job->next_task = 0;
    pthread_mutex_init(&job->lock, NULL);
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!tid) return -1;
    int rc = 0;
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&tid[i], NULL, worker, job) != 0) break;
        ++started;
    }
    /* Threads that did start drain every task; with none, run inline. */
    if (started == 0 && worker(job) != NULL) rc = -3;
    for (int i = 0; i < started; ++i) {
        void *ret = NULL;
        pthread_join(tid[i], &ret);
        if (ret) rc = -3;
    }
    free(tid);
    pthread_mutex_destroy(&job->lock);
    return rc;
}

/* Prefill over packed variable-length sequences.  Returns 0 on success,
 * a negative number on bad arguments or allocation failure.  nthreads <= 0
 * uses every online core. */
int kda_oracle_prefill_f64(const double *q, const double *k, const double *v,
                           const double *g, const double *beta,
                           const double *init_state, const int64_t *cu_seqlens,
                           int64_t nseq, int64_t H, int64_t dk, int64_t dv,
                           double *o, double *final_state, int nthreads) {
    if (nseq < 1 || H < 1 || dk < 1 || dv < 1 || !cu_seqlens || !o) return -10;
    if (cu_seqlens[0] != 0) return -11;
    for (int64_t s = 0; s < nseq; ++s)
        if (cu_seqlens[s + 1] < cu_seqlens[s]) return -12;
    oracle_job job;
    memset(&job, 0, sizeof(job));
    job.q = q; job.k = k; job.v = v; job.g = g; job.beta = beta;
    job.init = init_state; job.cu = cu_seqlens;
    job.nseq = nseq; job.H = H; job.dk = dk; job.dv = dv;
    job.o = o; job.final_state = final_state;
    job.decode = 0;
    return run_job(&job, nthreads);
}

/* One decode token for each of B x H heads; state [B, H, dk, dv] updated in
 * place, o [B, H, dv] written. */
int kda_oracle_decode_f64(const double *q, const double *k, const double *v,
                          const double *g, const double *beta, double *state,
                          int64_t B, int64_t H, int64_t dk, int64_t dv,
                          double *o, int nthreads) {
    if (B < 1 || H < 1 || dk < 1 || dv < 1 || !state || !o) return -10;
    oracle_job job;
    memset(&job, 0, sizeof(job));
    job.q = q; job.k = k; job.v = v; job.g = g; job.beta = beta;
    job.nseq = B; job.H = H; job.dk = dk; job.dv = dv;
    job.o = o; job.state = state;
    job.decode = 1;
    return run_job(&job, nthreads);
}

/* ----------------------------------------------------------------------
 * Reverse mode of the recurrence (the gradients a training step needs),
 * the chain rule taken through the four stages above in reverse order, one
 * (sequence, head) at a time, single-threaded (test sizes).
 *
 * For a loss L with dL/do_t = dO_t and dL/dS_final = dfinal, the adjoint
 * A = dL/dS is carried backwards from the last token:
 *   read   o_t = S_t^T q_t          : A += q_t dO_t^T,   dq_t = S_t dO_t
 *   write  S_t = E + beta k v^T     : dv_t = beta A^T k,  dbeta += (A^T k).v
 *   erase  E = P - beta k (k^T P)   : with e = A^T k and u = P^T k,
 *            dbeta -= e.u,  dk_t = beta A (v - u) - beta P e  (with the
 *            write's term),  dP = A - beta k e^T
 *   forget P = Diag(alpha) S_{t-1}  : dg_t[i] = sum_j dP[i][j] P[i][j]
 *            (d alpha_i / d g_i = alpha_i), A <- Diag(alpha) dP
 * and dinit = A after the first token.  The states S_{t-1} are recomputed by
 * the forward recurrence and kept for the whole sequence.
 *
 * Layouts as the forward; dO [N, H, dv]; dfinal [nseq, H, dk, dv] or NULL
 * (zero); outputs dq, dk, dg [N, H, dk], dv [N, H, dv], dbeta [N, H],
 * dinit [nseq, H, dk, dv] or NULL.  Returns 0, or a negative number on bad
 * arguments or allocation failure.
 */
int kda_oracle_backward_f64(const double *q, const double *k, const double *v,
                            const double *g, const double *beta,
                            const double *init_state, const int64_t *cu,
                            int64_t nseq, int64_t H, int64_t dk, int64_t dv,
                            const double *dO, const double *dfinal,
                            double *dq, double *dkk, double *dvv, double *dg,
                            double *dbeta, double *dinit) {
    if (nseq < 1 || H < 1 || dk < 1 || dv < 1 || !cu || !dO) return -10;
    if (cu[0] != 0) return -11;
    int64_t Tmax = 0;
    for (int64_t s = 0; s < nseq; ++s) {
        if (cu[s + 1] < cu[s]) return -12;
        if (cu[s + 1] - cu[s] > Tmax) Tmax = cu[s + 1] - cu[s];
    }
    const size_t blk = (size_t)(dk * dv);
    double *st = (double *)malloc(sizeof(double) * blk * (size_t)(Tmax + 1));  /* S_0 .. S_T */
    double *A = (double *)malloc(sizeof(double) * blk);
    double *P = (double *)malloc(sizeof(double) * blk);
    double *scr = (double *)malloc(sizeof(double) * (size_t)(dv > dk ? dv : dk) * 4);
    if (!st || !A || !P || !scr) { free(st); free(A); free(P); free(scr); return -20; }
    double *ob = scr, *e = scr + (dv > dk ? dv : dk), *u = e + (dv > dk ? dv : dk);
    for (int64_t s = 0; s < nseq; ++s) {
        for (int64_t h = 0; h < H; ++h) {
            const int64_t T = cu[s + 1] - cu[s];
            /* forward, keeping every state */
            if (init_state) memcpy(st, init_state + (s * H + h) * dk * dv, sizeof(double) * blk);
            else memset(st, 0, sizeof(double) * blk);
            for (int64_t t = 0; t < T; ++t) {
                const int64_t r = (cu[s] + t) * H + h;
                memcpy(st + (size_t)(t + 1) * blk, st + (size_t)t * blk, sizeof(double) * blk);
                kda_token_step(st + (size_t)(t + 1) * blk, dk, dv, q + r * dk, k + r * dk, v + r * dv,
                               g + r * dk, beta[r], ob, u);
            }
            /* adjoint of the final state */
            if (dfinal) memcpy(A, dfinal + (s * H + h) * dk * dv, sizeof(double) * blk);
            else memset(A, 0, sizeof(double) * blk);
            for (int64_t t = T - 1; t >= 0; --t) {
                const int64_t r = (cu[s] + t) * H + h;
                const double *qt = q + r * dk, *kt = k + r * dk, *vt = v + r * dv, *gt = g + r * dk;
                const double *dot = dO + r * dv;
                const double bt = beta[r];
                const double *Sp = st + (size_t)t * blk;       /* S_{t-1} */
                const double *Sn = st + (size_t)(t + 1) * blk; /* S_t */
                /* read */
                for (int64_t i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (int64_t j = 0; j < dv; ++j) {
                        A[i * dv + j] += qt[i] * dot[j];
                        acc += Sn[i * dv + j] * dot[j];
                    }
                    dq[r * dk + i] = acc;
                }
                /* forget (forward): P = Diag(alpha) S_{t-1}; w = k^T P (the erase's row vector) */
                for (int64_t i = 0; i < dk; ++i) {
                    const double a = exp(gt[i]);
                    for (int64_t j = 0; j < dv; ++j) P[i * dv + j] = a * Sp[i * dv + j];
                }
                for (int64_t j = 0; j < dv; ++j) {
                    double w = 0.0, ee = 0.0;
                    for (int64_t i = 0; i < dk; ++i) {
                        w += kt[i] * P[i * dv + j];
                        ee += kt[i] * A[i * dv + j];
                    }
                    u[j] = w;  /* k^T P */
                    e[j] = ee; /* A^T k */
                }
                /* write: S_t = E + beta k v^T */
                double db = 0.0;
                for (int64_t j = 0; j < dv; ++j) {
                    dvv[r * dv + j] = bt * e[j];
                    db += e[j] * vt[j];
                }
                /* erase: E = P - beta k (k^T P) = P - beta k u^T */
                for (int64_t j = 0; j < dv; ++j) db -= e[j] * u[j];
                dbeta[r] = db;
                for (int64_t i = 0; i < dk; ++i) {
                    /* d/dk of beta k v^T and of -beta k u^T with u = P^T k */
                    double acc = 0.0;
                    for (int64_t j = 0; j < dv; ++j)
                        acc += A[i * dv + j] * bt * (vt[j] - u[j]) - bt * P[i * dv + j] * e[j];
                    dkk[r * dk + i] = acc;
                }
                /* dP = A - beta k e^T; then the forget stage */
                for (int64_t i = 0; i < dk; ++i) {
                    const double a = exp(gt[i]);
                    double acc = 0.0;
                    for (int64_t j = 0; j < dv; ++j) {
                        const double dp = A[i * dv + j] - bt * kt[i] * e[j];
                        acc += dp * P[i * dv + j];
                        A[i * dv + j] = a * dp;
                    }
                    dg[r * dk + i] = acc;
                }
            }
            if (dinit) memcpy(dinit + (s * H + h) * dk * dv, A, sizeof(double) * blk);
        }
    }
    free(st); free(A); free(P); free(scr);
    return 0;
}

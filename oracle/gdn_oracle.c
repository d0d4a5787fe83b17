/*
 * Token-serial fp64 oracle for the gated delta rule.  TEST INFRASTRUCTURE ONLY:
 * nothing on the product path may link, load or call this file.  Only the test
 * suite, the smoke check and the CPU-baseline leg of the benchmark use it.
 *
 * What it computes, for every (batch b, head h) stream independently, with the
 * recurrent state S of shape [V, K] (rows: value channels, columns: key channels):
 *
 *     S <- S0 (or zeros)
 *     for t = 0 .. T-1:
 *         S   <- alpha_t * S (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *         o_t <- S q_t
 *     final_state <- S
 *
 * Sources (the pages of the method):
 *  - "Sparse Delta Memory: layer and kernels" (sparse-delta-memory 2.0.0 package
 *    description), section "What the layer computes": per token, the bank is first
 *    decayed, then read with the key, then written with beta times the prediction
 *    error, and the output is read with the query from the UPDATED bank.  Its
 *    section "Product-key top-k", paragraph on the dense limit, states that with
 *    every slot selected and l2-normalised weights the bank is the d_k x d_v state
 *    of the gated delta rule.  Transposing that bank gives S [V, K]; the token step
 *    above is exactly that sequence: S <- a S ; r = S k ; S <- S + b (v - r) k^T ;
 *    o = S q.
 *  - "OpenGDN 0.1.0" package description, section "Core operator reference":
 *    q, k are [B, T, H, K], v is [B, T, H, V], the gates are [B, T, H], the state
 *    is [B, H, V, K], and feeding final_state back as the next call's state is
 *    exact streaming continuation.  That section also names the token-by-token
 *    function as the correctness oracle.
 *
 * The reverse mode (gdn_oracle_bwd) is the vector-Jacobian product of that same
 * token loop, derived by hand (see the comment above it) and checked in the tests
 * against central finite differences and against float64 autograd of an
 * independent token loop.
 *
 * All arithmetic is IEEE double, in plain loops, with no blocking or reordering
 * beyond the token order.  Threads split the B*H independent streams.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *v, *alpha, *beta, *s0, *d_o, *d_sfinal;
    double *o, *s_final;
    double *dq, *dk, *dv, *dalpha, *dbeta, *d_s0;
    int64_t B, T, H, K, V;
    int64_t next;          /* next stream index to process (guarded by lock) */
    pthread_mutex_t lock;
    int failed;
} job_t;

static int64_t take_stream(job_t *j) {
    pthread_mutex_lock(&j->lock);
    int64_t s = j->next++;
    pthread_mutex_unlock(&j->lock);
    return s;
}

/* Element offsets in the row-major [B, T, H, D] and [B, H, V, K] layouts. */
static inline int64_t tok_off(const job_t *j, int64_t b, int64_t t, int64_t h, int64_t D) {
    return ((b * j->T + t) * j->H + h) * D;
}
static inline int64_t gate_off(const job_t *j, int64_t b, int64_t t, int64_t h) {
    return (b * j->T + t) * j->H + h;
}
static inline int64_t state_off(const job_t *j, int64_t b, int64_t h) {
    return (b * j->H + h) * j->V * j->K;
}

/* One token step of the recurrence, in place on S [V, K].  w is scratch of length V. */
static void token_step(double *S, double *w, const double *k, const double *v,
                       double a, double bt, int64_t K, int64_t V) {
    /* decayed read: w = (a S) k */
    for (int64_t i = 0; i < V; ++i) {
        double acc = 0.0;
        for (int64_t c = 0; c < K; ++c) acc += S[i * K + c] * k[c];
        w[i] = a * acc;
    }
    /* S <- a S + bt (v - w) k^T  ==  a S (I - bt k k^T) + bt v k^T */
    for (int64_t i = 0; i < V; ++i) {
        double e = bt * (v[i] - w[i]);
        for (int64_t c = 0; c < K; ++c) S[i * K + c] = a * S[i * K + c] + e * k[c];
    }
}

static void *fwd_worker(void *arg) {
    job_t *j = (job_t *)arg;
    const int64_t K = j->K, V = j->V;
    double *S = (double *)malloc(sizeof(double) * (size_t)(V * K));
    double *w = (double *)malloc(sizeof(double) * (size_t)V);
    if (!S || !w) { j->failed = 1; free(S); free(w); return NULL; }
    for (;;) {
        int64_t s = take_stream(j);
        if (s >= j->B * j->H) break;
        int64_t b = s / j->H, h = s % j->H;
        if (j->s0) memcpy(S, j->s0 + state_off(j, b, h), sizeof(double) * (size_t)(V * K));
        else memset(S, 0, sizeof(double) * (size_t)(V * K));
        for (int64_t t = 0; t < j->T; ++t) {
            const double *kt = j->k + tok_off(j, b, t, h, K);
            const double *vt = j->v + tok_off(j, b, t, h, V);
            const double *qt = j->q + tok_off(j, b, t, h, K);
            token_step(S, w, kt, vt, j->alpha[gate_off(j, b, t, h)], j->beta[gate_off(j, b, t, h)], K, V);
            double *ot = j->o + tok_off(j, b, t, h, V);
            for (int64_t i = 0; i < V; ++i) {
                double acc = 0.0;
                for (int64_t c = 0; c < K; ++c) acc += S[i * K + c] * qt[c];
                ot[i] = acc;
            }
        }
        if (j->s_final) memcpy(j->s_final + state_off(j, b, h), S, sizeof(double) * (size_t)(V * K));
    }
    free(S); free(w);
    return NULL;
}

static int run_threads(job_t *j, void *(*fn)(void *), int nthreads) {
    int64_t streams = j->B * j->H;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > streams) nthreads = (int)streams;
    pthread_mutex_init(&j->lock, NULL);
    j->next = 0;
    j->failed = 0;
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!tid) return -2;
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&tid[i], NULL, fn, j) != 0) break;
        ++started;
    }
    if (started == 0) fn(j);
    for (int i = 0; i < started; ++i) pthread_join(tid[i], NULL);
    free(tid);
    pthread_mutex_destroy(&j->lock);
    return j->failed ? -2 : 0;
}

static int check_dims(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V) {
    return (B >= 1 && T >= 0 && H >= 1 && K >= 1 && V >= 1) ? 0 : -1;
}

/*
 * Forward.  q, k: [B,T,H,K]; v, o: [B,T,H,V]; alpha, beta: [B,T,H];
 * s0, s_final: [B,H,V,K] (s0 NULL means zeros, s_final NULL means not wanted).
 * Returns 0 on success, -1 for invalid sizes or NULL required pointers, -2 when
 * out of host memory.
 */
int gdn_oracle_fwd(const double *q, const double *k, const double *v,
                   const double *alpha, const double *beta, const double *s0,
                   double *o, double *s_final,
                   int64_t B, int64_t T, int64_t H, int64_t K, int64_t V, int nthreads) {
    if (check_dims(B, T, H, K, V)) return -1;
    if (T > 0 && (!q || !k || !v || !alpha || !beta || !o)) return -1;
    job_t j;
    memset(&j, 0, sizeof(j));
    j.q = q; j.k = k; j.v = v; j.alpha = alpha; j.beta = beta; j.s0 = s0;
    j.o = o; j.s_final = s_final;
    j.B = B; j.T = T; j.H = H; j.K = K; j.V = V;
    return run_threads(&j, fwd_worker, nthreads);
}

/*
 * Reverse mode of the same token loop.  With G = dL/dS_t (everything downstream
 * of S_t) and S_prev = S_{t-1}, the token step S_t = a S_prev (I - b k k^T) + b v k^T,
 * o_t = S_t q_t gives, walking t from T-1 down to 0:
 *
 *     G      += dO_t q_t^T                 (o_t reads S_t)
 *     dq_t    = S_t^T dO_t
 *     dv_t    = b G k
 *     dbeta_t = (v - a S_prev k)^T G k
 *     dalpha_t= < G , S_prev (I - b k k^T) >_F
 *     dk_t    = b G^T v - a b (S_prev^T G + G^T S_prev) k
 *     G       = a G (I - b k k^T)          (gradient reaching S_prev)
 *
 * and d_s0 = G after the first token.  G starts at d_sfinal (zeros when NULL).
 * S_prev is recomputed segment by segment from fp64 checkpoints taken every
 * SEG tokens in a first forward sweep, so memory stays O(SEG * V * K) per thread.
 */
#define SEG 64

static void *bwd_worker(void *arg) {
    job_t *j = (job_t *)arg;
    const int64_t K = j->K, V = j->V, T = j->T;
    const int64_t VK = V * K;
    const int64_t nseg = (T + SEG - 1) / SEG;
    double *ckpt = (double *)malloc(sizeof(double) * (size_t)((nseg > 0 ? nseg : 1) * VK));
    double *seg = (double *)malloc(sizeof(double) * (size_t)((SEG + 1) * VK)); /* S_{t0-1} .. S_{t0+SEG-1} */
    double *G = (double *)malloc(sizeof(double) * (size_t)VK);
    double *w = (double *)malloc(sizeof(double) * (size_t)(V > K ? V : K));
    double *sk = (double *)malloc(sizeof(double) * (size_t)V);
    double *gk = (double *)malloc(sizeof(double) * (size_t)V);
    if (!ckpt || !seg || !G || !w || !sk || !gk) {
        j->failed = 1;
        free(ckpt); free(seg); free(G); free(w); free(sk); free(gk);
        return NULL;
    }
    for (;;) {
        int64_t s = take_stream(j);
        if (s >= j->B * j->H) break;
        int64_t b = s / j->H, h = s % j->H;
        /* forward sweep, keeping the state entering each segment */
        double *S = seg; /* reuse first slot as running state */
        if (j->s0) memcpy(S, j->s0 + state_off(j, b, h), sizeof(double) * (size_t)VK);
        else memset(S, 0, sizeof(double) * (size_t)VK);
        for (int64_t t = 0; t < T; ++t) {
            if (t % SEG == 0) memcpy(ckpt + (t / SEG) * VK, S, sizeof(double) * (size_t)VK);
            token_step(S, w, j->k + tok_off(j, b, t, h, K), j->v + tok_off(j, b, t, h, V),
                       j->alpha[gate_off(j, b, t, h)], j->beta[gate_off(j, b, t, h)], K, V);
        }
        if (j->d_sfinal) memcpy(G, j->d_sfinal + state_off(j, b, h), sizeof(double) * (size_t)VK);
        else memset(G, 0, sizeof(double) * (size_t)VK);
        for (int64_t sg = nseg - 1; sg >= 0; --sg) {
            int64_t t0 = sg * SEG;
            int64_t t1 = t0 + SEG < T ? t0 + SEG : T;
            /* seg[i] holds S_{t0+i-1}: seg[0] = state entering token t0 */
            memcpy(seg, ckpt + sg * VK, sizeof(double) * (size_t)VK);
            for (int64_t t = t0; t < t1; ++t) {
                double *nxt = seg + (t - t0 + 1) * VK;
                memcpy(nxt, seg + (t - t0) * VK, sizeof(double) * (size_t)VK);
                token_step(nxt, w, j->k + tok_off(j, b, t, h, K), j->v + tok_off(j, b, t, h, V),
                           j->alpha[gate_off(j, b, t, h)], j->beta[gate_off(j, b, t, h)], K, V);
            }
            for (int64_t t = t1 - 1; t >= t0; --t) {
                const double *Sp = seg + (t - t0) * VK;     /* S_{t-1} */
                const double *St = seg + (t - t0 + 1) * VK; /* S_t */
                const double *kt = j->k + tok_off(j, b, t, h, K);
                const double *vt = j->v + tok_off(j, b, t, h, V);
                const double *qt = j->q + tok_off(j, b, t, h, K);
                const double *dot = j->d_o + tok_off(j, b, t, h, V);
                const double a = j->alpha[gate_off(j, b, t, h)];
                const double bt = j->beta[gate_off(j, b, t, h)];
                double *dqt = j->dq + tok_off(j, b, t, h, K);
                double *dkt = j->dk + tok_off(j, b, t, h, K);
                double *dvt = j->dv + tok_off(j, b, t, h, V);
                /* G += dO q^T */
                for (int64_t i = 0; i < V; ++i)
                    for (int64_t c = 0; c < K; ++c) G[i * K + c] += dot[i] * qt[c];
                /* dq = S_t^T dO */
                for (int64_t c = 0; c < K; ++c) {
                    double acc = 0.0;
                    for (int64_t i = 0; i < V; ++i) acc += St[i * K + c] * dot[i];
                    dqt[c] = acc;
                }
                /* sk = S_prev k, gk = G k */
                for (int64_t i = 0; i < V; ++i) {
                    double a1 = 0.0, a2 = 0.0;
                    for (int64_t c = 0; c < K; ++c) {
                        a1 += Sp[i * K + c] * kt[c];
                        a2 += G[i * K + c] * kt[c];
                    }
                    sk[i] = a1;
                    gk[i] = a2;
                }
                /* dv = b G k ; dbeta = (v - a S_prev k) . (G k) */
                double db = 0.0;
                for (int64_t i = 0; i < V; ++i) {
                    dvt[i] = bt * gk[i];
                    db += (vt[i] - a * sk[i]) * gk[i];
                }
                j->dbeta[gate_off(j, b, t, h)] = db;
                /* dalpha = <G, S_prev> - b <G k, S_prev k> */
                double gs = 0.0, gksk = 0.0;
                for (int64_t i = 0; i < V; ++i) {
                    for (int64_t c = 0; c < K; ++c) gs += G[i * K + c] * Sp[i * K + c];
                    gksk += gk[i] * sk[i];
                }
                j->dalpha[gate_off(j, b, t, h)] = gs - bt * gksk;
                /* dk = b G^T v - a b (S_prev^T (G k) + G^T (S_prev k)) */
                for (int64_t c = 0; c < K; ++c) {
                    double gv = 0.0, sgk = 0.0, gsk = 0.0;
                    for (int64_t i = 0; i < V; ++i) {
                        gv += G[i * K + c] * vt[i];
                        sgk += Sp[i * K + c] * gk[i];
                        gsk += G[i * K + c] * sk[i];
                    }
                    dkt[c] = bt * gv - a * bt * (sgk + gsk);
                }
                /* G <- a G (I - b k k^T) = a (G - b (G k) k^T) */
                for (int64_t i = 0; i < V; ++i)
                    for (int64_t c = 0; c < K; ++c)
                        G[i * K + c] = a * (G[i * K + c] - bt * gk[i] * kt[c]);
            }
        }
        if (j->d_s0) memcpy(j->d_s0 + state_off(j, b, h), G, sizeof(double) * (size_t)VK);
    }
    free(ckpt); free(seg); free(G); free(w); free(sk); free(gk);
    return NULL;
}

/*
 * Reverse mode.  Same layouts as gdn_oracle_fwd; d_o is [B,T,H,V]; d_sfinal is
 * [B,H,V,K] or NULL (zeros).  Outputs dq, dk [B,T,H,K], dv [B,T,H,V],
 * dalpha, dbeta [B,T,H], d_s0 [B,H,V,K] (NULL skips it).  Gradients are taken
 * with respect to alpha and beta themselves.
 */
int gdn_oracle_bwd(const double *q, const double *k, const double *v,
                   const double *alpha, const double *beta, const double *s0,
                   const double *d_o, const double *d_sfinal,
                   double *dq, double *dk, double *dv, double *dalpha, double *dbeta,
                   double *d_s0,
                   int64_t B, int64_t T, int64_t H, int64_t K, int64_t V, int nthreads) {
    if (check_dims(B, T, H, K, V)) return -1;
    if (T > 0 && (!q || !k || !v || !alpha || !beta || !d_o || !dq || !dk || !dv || !dalpha || !dbeta))
        return -1;
    job_t j;
    memset(&j, 0, sizeof(j));
    j.q = q; j.k = k; j.v = v; j.alpha = alpha; j.beta = beta; j.s0 = s0;
    j.d_o = d_o; j.d_sfinal = d_sfinal;
    j.dq = dq; j.dk = dk; j.dv = dv; j.dalpha = dalpha; j.dbeta = dbeta; j.d_s0 = d_s0;
    j.B = B; j.T = T; j.H = H; j.K = K; j.V = V;
    return run_threads(&j, bwd_worker, nthreads);
}

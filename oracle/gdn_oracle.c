/*
 * Sequential fp64 oracle of the gated delta rule (test infrastructure only).
 *
 * This file is test infrastructure. Only the tests, the smoke check and the
 * CPU-baseline leg of the benchmark load it; the library under
 * gated_deltanet_chunked_03_amd/ never does, and shares no code with it.
 *
 * What it computes. The FlashQLA page ("FlashQLA: CP-/Bwd-friendly fused
 * linear attention kernels for GDN", section on optimising GDN chunked
 * prefill) speeds up the chunked prefill of the Gated DeltaNet recurrence but
 * never writes the recurrence down. It is the gated delta rule
 *     S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t
 * with S_t a d_v x d_k matrix, a_t = exp(g_t) the gate and b_t the write
 * strength. This oracle stores the transpose, a d_k x d_v matrix S, and for
 * every sequence and value head, in token order, applies
 *     S <- a_t S                     decay
 *     e <- v_t - S^T k_t             error of the decayed state's prediction
 *     S <- S + b_t k_t e^T           delta-rule rank-1 correction
 *     o_t <- scale * S^T q_t         read-out of the updated state
 * Transposing the formula gives these steps: the transposed right side is
 * a (I - b k k^T) S + b k v^T, and with S' = a S (the decayed stored state)
 * that equals S' + b k (v - S'^T k)^T.
 *
 * Value head h reads query/key head floor(h * h_qk / h_v) (contiguous groups).
 *
 * Layouts (row-major, all fp64):
 *   q, k            [T_total][h_qk][d_k]
 *   v, out          [T_total][h_v][d_v]
 *   g, beta         [T_total][h_v]
 *   states          [n_seqs][h_v][d_k][d_v]
 *   cu_seqlens      [n_seqs + 1] token offsets, cu_seqlens[0] = 0
 *   snaps           [n_seqs][h_v][n_snap][d_k][d_v]; snapshot j is the state
 *                   after the first j*snap_stride tokens of the sequence
 *                   (j = 0 is the initial state); written only when
 *                   j*snap_stride <= sequence length.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t n_seqs, h_qk, h_v, d_k, d_v;
    const int64_t* cu;
    const double *q, *k, *v, *g, *beta, *s0;
    double scale;
    double *out, *sfinal, *snaps;
    int64_t snap_stride, n_snap;
    int64_t next;               /* next work item, taken under the lock */
    pthread_mutex_t lock;
} job_t;

/* One (sequence, value head) scan, token by token. */
static void run_item(const job_t* J, int64_t item, double* S, double* e, double* u)
{
    const int64_t n = item / J->h_v, h = item % J->h_v;
    const int64_t hq = h * J->h_qk / J->h_v;
    const int64_t dk = J->d_k, dv = J->d_v;
    const int64_t t0 = J->cu[n], t1 = J->cu[n + 1];
    const int64_t sz = dk * dv;

    if (J->s0) memcpy(S, J->s0 + (n * J->h_v + h) * sz, sizeof(double) * sz);
    else memset(S, 0, sizeof(double) * sz);

    double* snap = J->snaps ? J->snaps + (n * J->h_v + h) * J->n_snap * sz : NULL;
    if (snap && J->n_snap > 0) memcpy(snap, S, sizeof(double) * sz);

    for (int64_t t = t0; t < t1; ++t) {
        const double* kt = J->k + (t * J->h_qk + hq) * dk;
        const double* qt = J->q + (t * J->h_qk + hq) * dk;
        const double* vt = J->v + (t * J->h_v + h) * dv;
        const double alpha = exp(J->g[t * J->h_v + h]);
        const double b = J->beta[t * J->h_v + h];

        /* decay */
        for (int64_t i = 0; i < sz; ++i) S[i] *= alpha;
        /* e = v - S^T k */
        for (int64_t j = 0; j < dv; ++j) u[j] = 0.0;
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < dv; ++j) u[j] += S[i * dv + j] * kt[i];
        for (int64_t j = 0; j < dv; ++j) e[j] = vt[j] - u[j];
        /* S += beta k e^T */
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < dv; ++j) S[i * dv + j] += b * kt[i] * e[j];
        /* o = scale S^T q */
        double* ot = J->out + (t * J->h_v + h) * dv;
        for (int64_t j = 0; j < dv; ++j) u[j] = 0.0;
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < dv; ++j) u[j] += S[i * dv + j] * qt[i];
        for (int64_t j = 0; j < dv; ++j) ot[j] = J->scale * u[j];

        if (snap && J->snap_stride > 0) {
            const int64_t done = t - t0 + 1;
            if (done % J->snap_stride == 0 && done / J->snap_stride < J->n_snap)
                memcpy(snap + (done / J->snap_stride) * sz, S, sizeof(double) * sz);
        }
    }
    if (J->sfinal) memcpy(J->sfinal + (n * J->h_v + h) * sz, S, sizeof(double) * sz);
}

static void* worker(void* arg)
{
    job_t* J = (job_t*)arg;
    const int64_t sz = J->d_k * J->d_v;
    double* S = (double*)malloc(sizeof(double) * sz);
    double* e = (double*)malloc(sizeof(double) * J->d_v);
    double* u = (double*)malloc(sizeof(double) * J->d_v);
    if (!S || !e || !u) { free(S); free(e); free(u); return (void*)1; }
    for (;;) {
        pthread_mutex_lock(&J->lock);
        const int64_t item = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (item >= J->n_seqs * J->h_v) break;
        run_item(J, item, S, e, u);
    }
    free(S); free(e); free(u);
    return NULL;
}

/* Returns 0 on success, -1 on bad arguments, -2 on allocation/thread failure. */
int gdn_oracle_fwd(int64_t n_seqs, const int64_t* cu_seqlens,
                   int64_t h_qk, int64_t h_v, int64_t d_k, int64_t d_v,
                   const double* q, const double* k, const double* v,
                   const double* g, const double* beta, double scale,
                   const double* initial_state, double* out, double* final_state,
                   int64_t snap_stride, int64_t n_snap, double* snaps,
                   int n_threads)
{
    if (n_seqs < 0 || h_qk <= 0 || h_v <= 0 || d_k <= 0 || d_v <= 0) return -1;
    if (h_v % h_qk != 0 || !cu_seqlens) return -1;
    if (cu_seqlens[n_seqs] > 0 && (!q || !k || !v || !g || !beta || !out)) return -1;
    for (int64_t n = 0; n < n_seqs; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;

    job_t J;
    memset(&J, 0, sizeof J);
    J.n_seqs = n_seqs; J.h_qk = h_qk; J.h_v = h_v; J.d_k = d_k; J.d_v = d_v;
    J.cu = cu_seqlens; J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta;
    J.s0 = initial_state; J.scale = scale; J.out = out; J.sfinal = final_state;
    J.snaps = snaps; J.snap_stride = snap_stride; J.n_snap = snaps ? n_snap : 0;
    pthread_mutex_init(&J.lock, NULL);

    if (n_threads < 1) n_threads = 1;
    if (n_threads > 256) n_threads = 256;
    pthread_t th[256];
    int started = 0, rc = 0;
    for (int i = 0; i < n_threads; ++i) {
        if (pthread_create(&th[i], NULL, worker, &J) != 0) break;
        ++started;
    }
    if (started == 0) { worker(&J); }
    for (int i = 0; i < started; ++i) {
        void* r = NULL;
        pthread_join(th[i], &r);
        if (r) rc = -2;
    }
    pthread_mutex_destroy(&J.lock);
    return rc;
}

/* ------------------------------------------------------------------------
 * Gradients of the same recurrence (reverse mode, fp64).
 *
 * The pages' title promises a backward-friendly design but prints no backward
 * formulas; the gradient of the sequential recurrence above is its plain
 * definition. Given dL/do_t for every token and dL/dS_final, it returns
 * dL/dq, dL/dk (per value head, before the heads of a query/key group are
 * summed), dL/dv, dL/dg, dL/dbeta and dL/dS_initial. The steps of one token
 * (forward: D = a S_prev, p = D^T k, w = b (v - p), S = D + k w^T,
 * o = scale S^T q) are undone in reverse order, with G the running dL/dS:
 *     G   += scale q do^T            read-out;  dq = scale S do
 *     dw   = G^T k                   through S = D + k w^T;  dk = G w
 *     db   = dw . (v - p)            through w = b (v - p)
 *     dv   = b dw,  dp = -b dw
 *     G   += k dp^T                  through p = D^T k;  dk += D dp
 *     dg   = <G, D>                  through D = a S_prev, a = exp(g)
 *     G    = a G                     dL/dS_prev
 * The states the reverse pass needs are recomputed from a checkpoint taken
 * every 64 tokens of the forward pass.
 *
 * Layouts: dq_part, dk_part [T_total][h_v][d_k]; dv [T_total][h_v][d_v];
 * dg, dbeta [T_total][h_v]; d_out like out; d_final and d_initial like the
 * states (d_final may be NULL for zero).
 * ------------------------------------------------------------------------ */
enum { kCk = 64 };

typedef struct {
    int64_t n_seqs, h_qk, h_v, d_k, d_v;
    const int64_t* cu;
    const double *q, *k, *v, *g, *beta, *s0, *dout, *dfinal;
    double scale;
    double *dq, *dk, *dv, *dg, *dbeta, *dinit;
    int64_t next;
    pthread_mutex_t lock;
} bjob_t;

/* One token forward: S <- a S + b k (v - a S^T k)^T (p receives a S^T k). */
static void fwd_token(const bjob_t* J, int64_t t, int64_t h, int64_t hq, double* S, double* p)
{
    const int64_t dk = J->d_k, dv = J->d_v;
    const double* kt = J->k + (t * J->h_qk + hq) * dk;
    const double* vt = J->v + (t * J->h_v + h) * dv;
    const double a = exp(J->g[t * J->h_v + h]), b = J->beta[t * J->h_v + h];
    for (int64_t i = 0; i < dk * dv; ++i) S[i] *= a;
    for (int64_t j = 0; j < dv; ++j) p[j] = 0.0;
    for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < dv; ++j) p[j] += S[i * dv + j] * kt[i];
    for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < dv; ++j) S[i * dv + j] += b * kt[i] * (vt[j] - p[j]);
}

typedef struct { double *ck, *blk, *G, *D, *p, *dw, *dp; int64_t n_ck; } bwork_t;

static void bwd_item(const bjob_t* J, int64_t item, bwork_t* W)
{
    const int64_t n = item / J->h_v, h = item % J->h_v;
    const int64_t hq = h * J->h_qk / J->h_v;
    const int64_t dk = J->d_k, dv = J->d_v, sz = dk * dv;
    const int64_t t0 = J->cu[n], t1 = J->cu[n + 1], len = t1 - t0;
    const int64_t nb = (len + kCk - 1) / kCk;
    double *ck = W->ck, *blk = W->blk, *G = W->G, *D = W->D, *p = W->p, *dw = W->dw, *dp = W->dp;

    /* forward pass: checkpoint b holds the state before token t0 + 64 b */
    if (J->s0) memcpy(ck, J->s0 + (n * J->h_v + h) * sz, sizeof(double) * sz);
    else memset(ck, 0, sizeof(double) * sz);
    for (int64_t b = 0; b + 1 < nb; ++b) {
        memcpy(ck + (b + 1) * sz, ck + b * sz, sizeof(double) * sz);
        for (int64_t t = t0 + b * kCk; t < t0 + (b + 1) * kCk; ++t) fwd_token(J, t, h, hq, ck + (b + 1) * sz, p);
    }

    if (J->dfinal) memcpy(G, J->dfinal + (n * J->h_v + h) * sz, sizeof(double) * sz);
    else memset(G, 0, sizeof(double) * sz);
    for (int64_t b = nb - 1; b >= 0; --b) {
        const int64_t ta = t0 + b * kCk, tb = (ta + kCk < t1) ? ta + kCk : t1;
        /* blk[i] = state after i tokens of the block */
        memcpy(blk, ck + b * sz, sizeof(double) * sz);
        for (int64_t t = ta; t < tb; ++t) {
            memcpy(blk + (t - ta + 1) * sz, blk + (t - ta) * sz, sizeof(double) * sz);
            fwd_token(J, t, h, hq, blk + (t - ta + 1) * sz, p);
        }
        for (int64_t t = tb - 1; t >= ta; --t) {
            const double* Sp = blk + (t - ta) * sz;
            const double* St = blk + (t - ta + 1) * sz;
            const double* kt = J->k + (t * J->h_qk + hq) * dk;
            const double* qt = J->q + (t * J->h_qk + hq) * dk;
            const double* vt = J->v + (t * J->h_v + h) * dv;
            const double* dot = J->dout + (t * J->h_v + h) * dv;
            const double a = exp(J->g[t * J->h_v + h]), bt = J->beta[t * J->h_v + h];
            double* dqt = J->dq + (t * J->h_v + h) * dk;
            double* dkt = J->dk + (t * J->h_v + h) * dk;
            double* dvt = J->dv + (t * J->h_v + h) * dv;

            /* read-out o = scale S^T q */
            for (int64_t i = 0; i < dk; ++i) {
                double s = 0.0;
                for (int64_t j = 0; j < dv; ++j) s += St[i * dv + j] * dot[j];
                dqt[i] = J->scale * s;
            }
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) G[i * dv + j] += J->scale * qt[i] * dot[j];
            /* D = a S_prev, p = D^T k, w = b (v - p) */
            for (int64_t i = 0; i < sz; ++i) D[i] = a * Sp[i];
            for (int64_t j = 0; j < dv; ++j) p[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) p[j] += D[i * dv + j] * kt[i];
            /* through S = D + k w^T */
            for (int64_t j = 0; j < dv; ++j) dw[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) dw[j] += G[i * dv + j] * kt[i];
            double db = 0.0;
            for (int64_t i = 0; i < dk; ++i) {
                double s = 0.0;
                for (int64_t j = 0; j < dv; ++j) s += G[i * dv + j] * bt * (vt[j] - p[j]);
                dkt[i] = s;
            }
            for (int64_t j = 0; j < dv; ++j) {
                db += dw[j] * (vt[j] - p[j]);
                dvt[j] = bt * dw[j];
                dp[j] = -bt * dw[j];
            }
            J->dbeta[t * J->h_v + h] = db;
            /* through p = D^T k */
            for (int64_t i = 0; i < dk; ++i) {
                double s = 0.0;
                for (int64_t j = 0; j < dv; ++j) {
                    G[i * dv + j] += kt[i] * dp[j];
                    s += D[i * dv + j] * dp[j];
                }
                dkt[i] += s;
            }
            /* through D = exp(g) S_prev */
            double dgt = 0.0;
            for (int64_t i = 0; i < sz; ++i) dgt += G[i] * D[i];
            J->dg[t * J->h_v + h] = dgt;
            for (int64_t i = 0; i < sz; ++i) G[i] *= a;
        }
    }
    if (J->dinit) memcpy(J->dinit + (n * J->h_v + h) * sz, G, sizeof(double) * sz);
}

static void* bwd_worker(void* arg)
{
    bjob_t* J = (bjob_t*)arg;
    const int64_t sz = J->d_k * J->d_v;
    int64_t maxlen = 0;
    for (int64_t n = 0; n < J->n_seqs; ++n)
        if (J->cu[n + 1] - J->cu[n] > maxlen) maxlen = J->cu[n + 1] - J->cu[n];
    bwork_t W;
    W.n_ck = (maxlen + kCk - 1) / kCk + 1;
    W.ck = (double*)malloc(sizeof(double) * sz * W.n_ck);
    W.blk = (double*)malloc(sizeof(double) * sz * (kCk + 1));
    W.G = (double*)malloc(sizeof(double) * sz);
    W.D = (double*)malloc(sizeof(double) * sz);
    W.p = (double*)malloc(sizeof(double) * J->d_v);
    W.dw = (double*)malloc(sizeof(double) * J->d_v);
    W.dp = (double*)malloc(sizeof(double) * J->d_v);
    void* rc = NULL;
    if (!W.ck || !W.blk || !W.G || !W.D || !W.p || !W.dw || !W.dp) rc = (void*)1;
    while (!rc) {
        pthread_mutex_lock(&J->lock);
        const int64_t item = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (item >= J->n_seqs * J->h_v) break;
        bwd_item(J, item, &W);
    }
    free(W.ck); free(W.blk); free(W.G); free(W.D); free(W.p); free(W.dw); free(W.dp);
    return rc;
}

/* Returns 0 on success, -1 on bad arguments, -2 on allocation/thread failure. */
int gdn_oracle_bwd(int64_t n_seqs, const int64_t* cu_seqlens,
                   int64_t h_qk, int64_t h_v, int64_t d_k, int64_t d_v,
                   const double* q, const double* k, const double* v,
                   const double* g, const double* beta, double scale,
                   const double* initial_state, const double* d_out, const double* d_final,
                   double* dq_part, double* dk_part, double* dv, double* dg, double* dbeta,
                   double* d_initial, int n_threads)
{
    if (n_seqs < 0 || h_qk <= 0 || h_v <= 0 || d_k <= 0 || d_v <= 0) return -1;
    if (h_v % h_qk != 0 || !cu_seqlens) return -1;
    if (cu_seqlens[n_seqs] > 0 && (!q || !k || !v || !g || !beta || !d_out || !dq_part || !dk_part ||
                                   !dv || !dg || !dbeta)) return -1;
    for (int64_t n = 0; n < n_seqs; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;

    bjob_t J;
    memset(&J, 0, sizeof J);
    J.n_seqs = n_seqs; J.h_qk = h_qk; J.h_v = h_v; J.d_k = d_k; J.d_v = d_v;
    J.cu = cu_seqlens; J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta;
    J.s0 = initial_state; J.dout = d_out; J.dfinal = d_final; J.scale = scale;
    J.dq = dq_part; J.dk = dk_part; J.dv = dv; J.dg = dg; J.dbeta = dbeta; J.dinit = d_initial;
    pthread_mutex_init(&J.lock, NULL);

    if (n_threads < 1) n_threads = 1;
    if (n_threads > 256) n_threads = 256;
    pthread_t th[256];
    int started = 0, rc = 0;
    for (int i = 0; i < n_threads; ++i) {
        if (pthread_create(&th[i], NULL, bwd_worker, &J) != 0) break;
        ++started;
    }
    if (started == 0 && bwd_worker(&J)) rc = -2;
    for (int i = 0; i < started; ++i) {
        void* r = NULL;
        pthread_join(th[i], &r);
        if (r) rc = -2;
    }
    pthread_mutex_destroy(&J.lock);
    return rc;
}

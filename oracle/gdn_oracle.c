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

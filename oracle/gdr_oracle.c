/*
 * Oracle for the gated delta rule forward pass: a plain, slow, per-token fp64
 * CPU recurrence.  TEST INFRASTRUCTURE ONLY: tests, the smoke check and the
 * benchmark's CPU-baseline leg use it; the product path never does.  It shares
 * no code, header or constant with the HIP library.
 *
 * What it computes.  The pages name the op `chunk_gated_delta_rule` with a
 * varlen `cu_seqlens` API, chunk size 64, an initial state and a final state
 * ("FlashQLA GDN backend produces different tokens from FLA Triton", Setup and
 * Observation; "Findings from integrating FlashQLA's Blackwell GDN kernels into
 * a JAX trainer", items 1-2).  They do not write the formula.  The recurrence
 * is the gated delta rule of Gated DeltaNet:
 *
 *     S_t = exp(g_t) * S_{t-1} * (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = scale * S_t q_t
 *
 * with S_t a dv x dk matrix.  The state is stored transposed, H_t = S_t^T
 * (dk x dv, row-major [dk][dv]), which is the layout of the initial and final
 * state tensors [N, Hv, dk, dv].  In that layout one step reads
 *
 *     H <- exp(g_t) H                 (decay first)
 *     p <- H^T k_t                    (what the state predicts for key k_t)
 *     d <- beta_t (v_t - p)           (delta-rule correction)
 *     H <- H + k_t d^T                (rank-1 write)
 *     o_t <- scale * H^T q_t          (read with the updated state)
 *
 * which expands to the matrix form above exactly.  A chunked evaluation
 * reaches the same result up to rounding order, so no chunking appears here.
 *
 * Segments.  Sequence n owns tokens [cu[n], cu[n+1]).  A segment of length 0
 * (a "ghost", a repeated offset in cu_seqlens: item 2 of the integration
 * report) reads nothing and writes nothing: its rows of ht keep whatever the
 * caller put there.  v-head h reads q/k head h / (Hv / Hk).
 *
 * Chunk-boundary states (optional).  Chunk c of sequence n holds its tokens
 * cu[n] + 64c .. min(cu[n] + 64(c+1), cu[n+1]) - 1; its state is H after the
 * last of them, stored at row off[n] + c, where off[n] = sum over m < n of
 * ceil(L_m / 64) (the prefix caching of the pages' `state_checkpoints`,
 * "feat(cake_kda): add paired recurrent training for SM100a and SM103a", the
 * follow-up's kept prefill surface).  The last chunk's state is ht.
 *
 * Layouts (all row-major, fp64):
 *   q, k  [T, Hk, dk]      v, o  [T, Hv, dv]      g, beta  [T, Hv]
 *   cu    [n_seq + 1]      h0, ht [n_seq, Hv, dk, dv]   (h0 NULL = zero state,
 *                                                          ht NULL = not written)
 *   hck   [NT, Hv, dk, dv] with NT = off[n_seq]     (NULL = not written)
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
    const double *q, *k, *v, *g, *beta, *h0;
    const int64_t *cu;
    double *o, *ht, *hck;
    const int64_t *off;  /* chunk offsets per sequence (hck only) */
    int64_t n_seq, T, Hk, Hv, dk, dv;
    double scale;
    int64_t *items;      /* work items n * Hv + h, longest segment first */
    int64_t n_items;
    int64_t next;        /* shared work counter */
    pthread_mutex_t lock;
} job_t;

/* One (sequence, v-head) pair, token by token. */
static void run_item(const job_t *J, int64_t n, int64_t h, double *H, double *p)
{
    const int64_t dk = J->dk, dv = J->dv, Hk = J->Hk, Hv = J->Hv;
    const int64_t hk = h / (Hv / Hk);
    const int64_t bos = J->cu[n], eos = J->cu[n + 1];
    if (eos <= bos) return;                       /* ghost: no read, no write */

    if (J->h0) memcpy(H, J->h0 + ((n * Hv + h) * dk) * dv, sizeof(double) * dk * dv);
    else memset(H, 0, sizeof(double) * dk * dv);

    for (int64_t t = bos; t < eos; ++t) {
        const double *kt = J->k + (t * Hk + hk) * dk;
        const double *qt = J->q + (t * Hk + hk) * dk;
        const double *vt = J->v + (t * Hv + h) * dv;
        const double a = exp(J->g[t * Hv + h]);
        const double b = J->beta[t * Hv + h];

        for (int64_t i = 0; i < dk * dv; ++i) H[i] *= a;

        for (int64_t j = 0; j < dv; ++j) p[j] = 0.0;
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < dv; ++j) p[j] += H[i * dv + j] * kt[i];

        for (int64_t j = 0; j < dv; ++j) p[j] = b * (vt[j] - p[j]);   /* p now holds d */

        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < dv; ++j) H[i * dv + j] += kt[i] * p[j];

        double *ot = J->o + (t * Hv + h) * dv;
        for (int64_t j = 0; j < dv; ++j) ot[j] = 0.0;
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < dv; ++j) ot[j] += H[i * dv + j] * qt[i];
        for (int64_t j = 0; j < dv; ++j) ot[j] *= J->scale;

        if (J->hck && ((t - bos + 1) % 64 == 0 || t == eos - 1)) {
            const int64_t c = (t - bos) / 64;
            memcpy(J->hck + (((J->off[n] + c) * Hv + h) * dk) * dv, H, sizeof(double) * dk * dv);
        }
    }
    if (J->ht) memcpy(J->ht + ((n * Hv + h) * dk) * dv, H, sizeof(double) * dk * dv);
}

static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    double *H = (double *)malloc(sizeof(double) * (size_t)(J->dk * J->dv + J->dv));
    if (!H) return (void *)1;
    double *p = H + J->dk * J->dv;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int64_t i = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (i >= J->n_items) break;
        const int64_t it = J->items[i];
        run_item(J, it / J->Hv, it % J->Hv, H, p);
    }
    free(H);
    return NULL;
}

static const job_t *g_sort_job;
static int by_length_desc(const void *a, const void *b)
{
    const job_t *J = g_sort_job;
    const int64_t ia = *(const int64_t *)a, ib = *(const int64_t *)b;
    const int64_t na = ia / J->Hv, nb = ib / J->Hv;
    const int64_t la = J->cu[na + 1] - J->cu[na], lb = J->cu[nb + 1] - J->cu[nb];
    if (la != lb) return la > lb ? -1 : 1;
    return ia < ib ? -1 : (ia > ib);
}

/* Threads actually used for a call with `requested` threads (<= 0: all cores). */
int gdr_oracle_threads(int requested, int64_t n_items)
{
    long n = requested > 0 ? requested : sysconf(_SC_NPROCESSORS_ONLN);
    if (n < 1) n = 1;
    if (n > n_items) n = n_items > 0 ? n_items : 1;
    return (int)n;
}

/*
 * Returns 0 on success, -1 on an argument the recurrence cannot take
 * (non-positive head sizes, Hv not a multiple of Hk, cu not non-decreasing
 * within [0, T]), -2 when memory or threads cannot be obtained.
 */
int gdr_oracle_fwd_chunks(const double *q, const double *k, const double *v, const double *g,
                          const double *beta, const int64_t *cu, int64_t n_seq, int64_t T,
                          int64_t Hk, int64_t Hv, int64_t dk, int64_t dv, const double *h0,
                          double *o, double *ht, double *hck, double scale, int n_threads);

int gdr_oracle_fwd(const double *q, const double *k, const double *v, const double *g,
                   const double *beta, const int64_t *cu, int64_t n_seq, int64_t T,
                   int64_t Hk, int64_t Hv, int64_t dk, int64_t dv, const double *h0,
                   double *o, double *ht, double scale, int n_threads)
{
    return gdr_oracle_fwd_chunks(q, k, v, g, beta, cu, n_seq, T, Hk, Hv, dk, dv, h0, o, ht,
                                 NULL, scale, n_threads);
}

/* The same, also writing the chunk-boundary states into hck (may be NULL). */
int gdr_oracle_fwd_chunks(const double *q, const double *k, const double *v, const double *g,
                          const double *beta, const int64_t *cu, int64_t n_seq, int64_t T,
                          int64_t Hk, int64_t Hv, int64_t dk, int64_t dv, const double *h0,
                          double *o, double *ht, double *hck, double scale, int n_threads)
{
    if (n_seq < 0 || T < 0 || Hk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || Hv % Hk != 0)
        return -1;
    if (n_seq == 0) return 0;
    if (cu[0] < 0) return -1;
    for (int64_t n = 0; n < n_seq; ++n)
        if (cu[n + 1] < cu[n] || cu[n + 1] > T) return -1;

    job_t J;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.h0 = h0;
    J.cu = cu; J.o = o; J.ht = ht; J.hck = hck;
    int64_t *off = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n_seq + 1));
    if (!off) return -2;
    off[0] = 0;
    for (int64_t n = 0; n < n_seq; ++n) off[n + 1] = off[n] + (cu[n + 1] - cu[n] + 63) / 64;
    J.off = off;
    J.n_seq = n_seq; J.T = T; J.Hk = Hk; J.Hv = Hv; J.dk = dk; J.dv = dv;
    J.scale = scale;
    J.n_items = n_seq * Hv;
    J.next = 0;
    J.items = (int64_t *)malloc(sizeof(int64_t) * (size_t)J.n_items);
    if (!J.items) {
        free(off);
        return -2;
    }
    for (int64_t i = 0; i < J.n_items; ++i) J.items[i] = i;
    g_sort_job = &J;
    qsort(J.items, (size_t)J.n_items, sizeof(int64_t), by_length_desc);
    pthread_mutex_init(&J.lock, NULL);

    const int nt = gdr_oracle_threads(n_threads, J.n_items);
    int rc = 0;
    if (nt == 1) {
        if (worker(&J)) rc = -2;
    } else {
        pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nt);
        int started = 0;
        if (!th) rc = -2;
        for (int i = 0; rc == 0 && i < nt; ++i) {
            if (pthread_create(&th[i], NULL, worker, &J) != 0) { rc = -2; break; }
            ++started;
        }
        for (int i = 0; i < started; ++i) {
            void *ret = NULL;
            pthread_join(th[i], &ret);
            if (ret) rc = -2;
        }
        free(th);
    }
    pthread_mutex_destroy(&J.lock);
    free(J.items);
    free(off);
    return rc;
}

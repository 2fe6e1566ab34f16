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
 * gdr_oracle_fwd_checkpoints does the same for pieces of `every` tokens in
 * place of 64 (that surface also keeps a `checkpoint_every_n_tokens`
 * argument, with checkpoint granularity 16): row off[n] + j holds H after
 * min((j+1) every, L_n) tokens, off[n] = sum over m < n of ceil(L_m / every).
 *
 * Layouts (all row-major, fp64):
 *   q, k  [T, Hk, dk]      v, o  [T, Hv, dv]      g, beta  [T, Hv]
 *   cu    [n_seq + 1]      h0, ht [n_seq, Hv, dk, dv]   (h0 NULL = zero state,
 *                                                          ht NULL = not written)
 *   hck   [NT, Hv, dk, dv] with NT = off[n_seq]     (NULL = not written)
 *   gk    [T, Hv, dk] per-channel log-gates (gdr_oracle_kda_fwd only; replaces g)
 */
#define _GNU_SOURCE   /* sched_getaffinity, CPU_COUNT */
#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
    const double *q, *k, *v, *g, *beta, *h0;
    const double *gk;    /* per-channel log-gates [T, Hv, dk], or NULL (scalar g) */
    const int64_t *cu;
    double *o, *ht, *hck;
    const int64_t *off;  /* checkpoint row offsets per sequence (hck only) */
    int64_t every;       /* tokens per checkpoint piece (hck only) */
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
        const double a = J->gk ? 1.0 : exp(J->g[t * Hv + h]);
        const double b = J->beta[t * Hv + h];

        for (int64_t i = 0; i < dk * dv; ++i) H[i] *= a;
        if (J->gk) {                              /* per-channel decay of the rows of H */
            const double *gt = J->gk + (t * Hv + h) * dk;
            for (int64_t i = 0; i < dk; ++i) {
                const double ai = exp(gt[i]);
                for (int64_t j = 0; j < dv; ++j) H[i * dv + j] *= ai;
            }
        }

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

        if (J->hck && ((t - bos + 1) % J->every == 0 || t == eos - 1)) {
            const int64_t c = (t - bos) / J->every;
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

/* Threads actually used for a call with `requested` threads (<= 0: the cores
 * this process may run on, at most OMP_NUM_THREADS when that is set). */
int gdr_oracle_threads(int requested, int64_t n_items)
{
    long n = requested;
    if (n <= 0) {
        cpu_set_t set;
        n = sched_getaffinity(0, sizeof(set), &set) == 0 ? CPU_COUNT(&set) : sysconf(_SC_NPROCESSORS_ONLN);
        const char *env = getenv("OMP_NUM_THREADS");
        const long cap = env ? strtol(env, NULL, 10) : 0;
        if (cap > 0 && cap < n) n = cap;
    }
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

static int run_fwd_job(const double *q, const double *k, const double *v, const double *g,
                       const double *g_channels, const double *beta, const int64_t *cu, int64_t n_seq,
                       int64_t T, int64_t Hk, int64_t Hv, int64_t dk, int64_t dv, const double *h0,
                       double *o, double *ht, double *hck, int64_t every, double scale, int n_threads);

/* The same, also writing the chunk-boundary states into hck (may be NULL). */
int gdr_oracle_fwd_chunks(const double *q, const double *k, const double *v, const double *g,
                          const double *beta, const int64_t *cu, int64_t n_seq, int64_t T,
                          int64_t Hk, int64_t Hv, int64_t dk, int64_t dv, const double *h0,
                          double *o, double *ht, double *hck, double scale, int n_threads)
{
    return run_fwd_job(q, k, v, g, NULL, beta, cu, n_seq, T, Hk, Hv, dk, dv, h0, o, ht, hck, 64,
                       scale, n_threads);
}

/* The same with checkpoints every `every` tokens (every >= 1) in place of 64. */
int gdr_oracle_fwd_checkpoints(const double *q, const double *k, const double *v, const double *g,
                               const double *beta, const int64_t *cu, int64_t n_seq, int64_t T,
                               int64_t Hk, int64_t Hv, int64_t dk, int64_t dv, const double *h0,
                               double *o, double *ht, double *hck, int64_t every, double scale,
                               int n_threads)
{
    if (every < 1) return -1;
    return run_fwd_job(q, k, v, g, NULL, beta, cu, n_seq, T, Hk, Hv, dk, dv, h0, o, ht, hck, every,
                       scale, n_threads);
}

/*
 * Per-channel gates (the KDA-style variant of "feat(cake_kda): add paired
 * recurrent training for SM100a and SM103a", whose raw gate carries one value
 * per key channel): the scalar decay exp(g_t) becomes diag(exp(g_t)) with
 * g_t in R^dk, applied to the rows of H (the key side):
 *
 *     S_t = S_{t-1} diag(exp(g_t)) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *
 * g_channels is [T, Hv, dk] (already the log-decay: the pages do not define
 * the transform that produces it from a raw gate).  Everything else is
 * gdr_oracle_fwd.
 */
int gdr_oracle_kda_fwd(const double *q, const double *k, const double *v, const double *g_channels,
                       const double *beta, const int64_t *cu, int64_t n_seq, int64_t T, int64_t Hk,
                       int64_t Hv, int64_t dk, int64_t dv, const double *h0, double *o, double *ht,
                       double scale, int n_threads)
{
    if (!g_channels) return -1;
    return run_fwd_job(q, k, v, NULL, g_channels, beta, cu, n_seq, T, Hk, Hv, dk, dv, h0, o, ht, NULL,
                       64, scale, n_threads);
}

static int run_fwd_job(const double *q, const double *k, const double *v, const double *g,
                       const double *g_channels, const double *beta, const int64_t *cu, int64_t n_seq,
                       int64_t T, int64_t Hk, int64_t Hv, int64_t dk, int64_t dv, const double *h0,
                       double *o, double *ht, double *hck, int64_t every, double scale, int n_threads)
{
    if (n_seq < 0 || T < 0 || Hk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || Hv % Hk != 0)
        return -1;
    if (n_seq == 0) return 0;
    if (cu[0] < 0) return -1;
    for (int64_t n = 0; n < n_seq; ++n)
        if (cu[n + 1] < cu[n] || cu[n + 1] > T) return -1;

    job_t J;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.h0 = h0;
    J.gk = g_channels;
    J.cu = cu; J.o = o; J.ht = ht; J.hck = hck;
    int64_t *off = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n_seq + 1));
    if (!off) return -2;
    off[0] = 0;
    for (int64_t n = 0; n < n_seq; ++n) off[n + 1] = off[n] + (cu[n + 1] - cu[n] + every - 1) / every;
    J.off = off;
    J.every = every;
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

/*
 * Backward pass (reverse-mode derivative of the same per-token recurrence).
 *
 * Given upstream gradients do = dL/do [T, Hv, dv] and dht = dL/dht
 * [n_seq, Hv, dk, dv] (NULL = zero), it returns dL/d of every input: dq, dk
 * [T, Hk, dk] (summed over the v-heads that share a q/k head), dv [T, Hv, dv],
 * dg, dbeta [T, Hv] and dh0 [n_seq, Hv, dk, dv].  The pages list this as the
 * other half of the kernel family (the bit-reproducible backward of "Findings
 * from integrating FlashQLA's Blackwell GDN kernels into a JAX trainer",
 * opening summary and items 3-4); they give no formula, so the derivative is
 * taken of the recurrence above, one token at a time, in reverse order.  For
 * token t with state H_prev before it (a = exp(g_t), b = beta_t):
 *
 *   forward   Hd = a H_prev,  p = Hd^T k,  d = b (v - p),  H = Hd + k d^T,
 *             o = scale H^T q
 *   reverse   dq  = scale H do          dH += scale q do^T
 *             dd  = dH^T k              dk  = dH d
 *             dv  = b dd                dbeta = dd . (v - p)
 *             dp  = -b dd               dHd = dH + k dp^T,  dk += Hd dp
 *             dg  = <dHd, Hd>           dH  = a dHd        (the gradient of H_prev)
 *
 * The states H_prev are recomputed from per-chunk copies kept during one
 * forward sweep (64 tokens at a time), which changes nothing in the values.
 * Tokens outside every segment get zero gradients; a length-0 segment reads
 * nothing and writes nothing (its dh0 rows keep the caller's bytes), as in the
 * forward pass.  dh0 is written whether or not h0 was given (NULL h0 means the
 * zero state, whose gradient is still defined); dh0 NULL = not written.
 */
typedef struct {
    const double *q, *k, *v, *g, *beta, *h0, *dout, *dht;
    const int64_t *cu;
    double *dqv, *dkv;   /* [T, Hv, dk] per v-head, summed over groups afterwards */
    double *dv, *dg, *dbeta, *dh0;
    int64_t n_seq, T, Hk, Hv, dk, dv_;
    double scale;
    int64_t *items;
    int64_t n_items;
    int64_t next;
    pthread_mutex_t lock;
} bjob_t;

static void bwd_item(const bjob_t *J, int64_t n, int64_t h, double *ws)
{
    const int64_t dk = J->dk, dv = J->dv_, Hk = J->Hk, Hv = J->Hv;
    const int64_t hk = h / (Hv / Hk);
    const int64_t bos = J->cu[n], eos = J->cu[n + 1];
    if (eos <= bos) return;
    const int64_t L = eos - bos, nc = (L + 63) / 64, S = dk * dv;

    /* ws: chunk-start states [nc][S], per-token states of one chunk [65][S], dH, dHd, vectors */
    double *Hs = ws;
    double *Hc = Hs + nc * S;
    double *dH = Hc + 65 * S;
    double *dHd = dH + S;
    double *p = dHd + S, *d = p + dv, *dd = d + dv, *dp = dd + dv;

    /* forward sweep keeping the state at every chunk start */
    double *H = Hc;
    if (J->h0) memcpy(H, J->h0 + ((n * Hv + h) * dk) * dv, sizeof(double) * S);
    else memset(H, 0, sizeof(double) * S);
    for (int64_t t = bos; t < eos; ++t) {
        if ((t - bos) % 64 == 0) memcpy(Hs + ((t - bos) / 64) * S, H, sizeof(double) * S);
        const double *kt = J->k + (t * Hk + hk) * dk;
        const double *vt = J->v + (t * Hv + h) * dv;
        const double a = exp(J->g[t * Hv + h]), b = J->beta[t * Hv + h];
        for (int64_t i = 0; i < S; ++i) H[i] *= a;
        for (int64_t j = 0; j < dv; ++j) p[j] = 0.0;
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < dv; ++j) p[j] += H[i * dv + j] * kt[i];
        for (int64_t j = 0; j < dv; ++j) d[j] = b * (vt[j] - p[j]);
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < dv; ++j) H[i * dv + j] += kt[i] * d[j];
    }

    if (J->dht) memcpy(dH, J->dht + ((n * Hv + h) * dk) * dv, sizeof(double) * S);
    else memset(dH, 0, sizeof(double) * S);

    for (int64_t c = nc - 1; c >= 0; --c) {
        const int64_t t0 = bos + 64 * c, t1 = (t0 + 64 < eos) ? t0 + 64 : eos;
        /* Hc[i] = state before token t0 + i */
        memcpy(Hc, Hs + c * S, sizeof(double) * S);
        for (int64_t t = t0; t < t1; ++t) {
            const double *Hp = Hc + (t - t0) * S;
            double *Hn = Hc + (t - t0 + 1) * S;
            const double *kt = J->k + (t * Hk + hk) * dk;
            const double *vt = J->v + (t * Hv + h) * dv;
            const double a = exp(J->g[t * Hv + h]), b = J->beta[t * Hv + h];
            for (int64_t i = 0; i < S; ++i) Hn[i] = a * Hp[i];
            for (int64_t j = 0; j < dv; ++j) p[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) p[j] += Hn[i * dv + j] * kt[i];
            for (int64_t j = 0; j < dv; ++j) d[j] = b * (vt[j] - p[j]);
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) Hn[i * dv + j] += kt[i] * d[j];
        }
        for (int64_t t = t1 - 1; t >= t0; --t) {
            const double *Hp = Hc + (t - t0) * S;       /* H_prev */
            const double *Ht = Hc + (t - t0 + 1) * S;   /* H after token t */
            const double *kt = J->k + (t * Hk + hk) * dk;
            const double *qt = J->q + (t * Hk + hk) * dk;
            const double *vt = J->v + (t * Hv + h) * dv;
            const double *dot = J->dout + (t * Hv + h) * dv;
            const double a = exp(J->g[t * Hv + h]), b = J->beta[t * Hv + h];
            double *dqt = J->dqv + (t * Hv + h) * dk;
            double *dkt = J->dkv + (t * Hv + h) * dk;

            /* recompute p and d from H_prev */
            for (int64_t j = 0; j < dv; ++j) p[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) p[j] += a * Hp[i * dv + j] * kt[i];
            for (int64_t j = 0; j < dv; ++j) d[j] = b * (vt[j] - p[j]);

            /* o = scale H^T q */
            for (int64_t i = 0; i < dk; ++i) {
                double s = 0.0;
                for (int64_t j = 0; j < dv; ++j) s += Ht[i * dv + j] * dot[j];
                dqt[i] = J->scale * s;
            }
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) dH[i * dv + j] += J->scale * qt[i] * dot[j];

            /* H = Hd + k d^T */
            for (int64_t j = 0; j < dv; ++j) dd[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) dd[j] += dH[i * dv + j] * kt[i];
            for (int64_t i = 0; i < dk; ++i) {
                double s = 0.0;
                for (int64_t j = 0; j < dv; ++j) s += dH[i * dv + j] * d[j];
                dkt[i] = s;
            }

            /* d = b (v - p) */
            double db = 0.0;
            for (int64_t j = 0; j < dv; ++j) {
                J->dv[(t * Hv + h) * dv + j] = b * dd[j];
                db += dd[j] * (vt[j] - p[j]);
                dp[j] = -b * dd[j];
            }
            J->dbeta[t * Hv + h] = db;

            /* p = Hd^T k with Hd = a H_prev */
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) dHd[i * dv + j] = dH[i * dv + j] + kt[i] * dp[j];
            for (int64_t i = 0; i < dk; ++i) {
                double s = 0.0;
                for (int64_t j = 0; j < dv; ++j) s += a * Hp[i * dv + j] * dp[j];
                dkt[i] += s;
            }

            /* Hd = a H_prev */
            double dgt = 0.0;
            for (int64_t i = 0; i < S; ++i) dgt += dHd[i] * a * Hp[i];
            J->dg[t * Hv + h] = dgt;
            for (int64_t i = 0; i < S; ++i) dH[i] = a * dHd[i];
        }
    }
    if (J->dh0) memcpy(J->dh0 + ((n * Hv + h) * dk) * dv, dH, sizeof(double) * S);
}

static void *bwd_worker(void *arg)
{
    bjob_t *J = (bjob_t *)arg;
    int64_t max_nc = 1;
    for (int64_t n = 0; n < J->n_seq; ++n) {
        const int64_t nc = (J->cu[n + 1] - J->cu[n] + 63) / 64;
        if (nc > max_nc) max_nc = nc;
    }
    const int64_t S = J->dk * J->dv_;
    double *ws = (double *)malloc(sizeof(double) * (size_t)((max_nc + 67) * S + 4 * J->dv_));
    if (!ws) return (void *)1;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int64_t i = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (i >= J->n_items) break;
        const int64_t it = J->items[i];
        bwd_item(J, it / J->Hv, it % J->Hv, ws);
    }
    free(ws);
    return NULL;
}

static const bjob_t *g_sort_bjob;
static int by_length_desc_b(const void *a, const void *b)
{
    const bjob_t *J = g_sort_bjob;
    const int64_t ia = *(const int64_t *)a, ib = *(const int64_t *)b;
    const int64_t na = ia / J->Hv, nb = ib / J->Hv;
    const int64_t la = J->cu[na + 1] - J->cu[na], lb = J->cu[nb + 1] - J->cu[nb];
    if (la != lb) return la > lb ? -1 : 1;
    return ia < ib ? -1 : (ia > ib);
}

/*
 * Returns 0 on success, -1 on a bad argument (as gdr_oracle_fwd), -2 when
 * memory or threads cannot be obtained.  dq, dk, dv, dg, dbeta are fully
 * written (zero outside segments); h0, dht and dh0 may be NULL.
 */
int gdr_oracle_bwd(const double *q, const double *k, const double *v, const double *g,
                   const double *beta, const int64_t *cu, int64_t n_seq, int64_t T,
                   int64_t Hk, int64_t Hv, int64_t dk, int64_t dv, const double *h0,
                   const double *dout, const double *dht, double *dq, double *dk_out,
                   double *dv_out, double *dg, double *dbeta, double *dh0, double scale,
                   int n_threads)
{
    if (n_seq < 0 || T < 0 || Hk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || Hv % Hk != 0)
        return -1;
    if (n_seq > 0 && cu[0] < 0) return -1;
    for (int64_t n = 0; n < n_seq; ++n)
        if (cu[n + 1] < cu[n] || cu[n + 1] > T) return -1;

    memset(dq, 0, sizeof(double) * (size_t)(T * Hk * dk));
    memset(dk_out, 0, sizeof(double) * (size_t)(T * Hk * dk));
    memset(dv_out, 0, sizeof(double) * (size_t)(T * Hv * dv));
    memset(dg, 0, sizeof(double) * (size_t)(T * Hv));
    memset(dbeta, 0, sizeof(double) * (size_t)(T * Hv));
    if (n_seq == 0) return 0;

    bjob_t J;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.h0 = h0; J.dout = dout; J.dht = dht;
    J.cu = cu; J.dv = dv_out; J.dg = dg; J.dbeta = dbeta; J.dh0 = dh0;
    J.n_seq = n_seq; J.T = T; J.Hk = Hk; J.Hv = Hv; J.dk = dk; J.dv_ = dv;
    J.scale = scale;
    J.dqv = (double *)calloc((size_t)(T * Hv * dk) + 1, sizeof(double));
    J.dkv = (double *)calloc((size_t)(T * Hv * dk) + 1, sizeof(double));
    J.n_items = n_seq * Hv;
    J.next = 0;
    J.items = (int64_t *)malloc(sizeof(int64_t) * (size_t)J.n_items);
    if (!J.dqv || !J.dkv || !J.items) {
        free(J.dqv); free(J.dkv); free(J.items);
        return -2;
    }
    for (int64_t i = 0; i < J.n_items; ++i) J.items[i] = i;
    g_sort_bjob = &J;
    qsort(J.items, (size_t)J.n_items, sizeof(int64_t), by_length_desc_b);
    pthread_mutex_init(&J.lock, NULL);

    const int nt = gdr_oracle_threads(n_threads, J.n_items);
    int rc = 0;
    if (nt == 1) {
        if (bwd_worker(&J)) rc = -2;
    } else {
        pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nt);
        int started = 0;
        if (!th) rc = -2;
        for (int i = 0; rc == 0 && i < nt; ++i) {
            if (pthread_create(&th[i], NULL, bwd_worker, &J) != 0) { rc = -2; break; }
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

    /* q and k are shared by the Hv / Hk v-heads of a group: their gradients add */
    const int64_t G = Hv / Hk;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t h = 0; h < Hv; ++h)
            for (int64_t i = 0; i < dk; ++i) {
                dq[(t * Hk + h / G) * dk + i] += J.dqv[(t * Hv + h) * dk + i];
                dk_out[(t * Hk + h / G) * dk + i] += J.dkv[(t * Hv + h) * dk + i];
            }
    free(J.dqv);
    free(J.dkv);
    free(J.items);
    return rc;
}

/*
 * Simple GLA CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, fp64, token-by-token evaluation of the head-wise gated linear
 * attention recurrence.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library; the GPU product path
 * never links, loads or calls it, and it shares no code, header or constant
 * with the GPU library.
 *
 * What is computed (page "flash-linear-attention 中的 Simple GLA" (xxqk.cn),
 * section 一, the recurrence and the naive_recurrent_simple_gla description;
 * section 二 for the argument conventions):
 *
 *     S_t = exp(g_t) * S_{t-1} + k_t v_t^T           (K x V state per head)
 *     o_t = scale * S_t^T q_t                       (uses the updated state)
 *
 * The printed recurrence lost its '=' and '+' in extraction; it is read as
 * S_{t+1} = g_{t+1} (.) S_t + K_{t+1} V_{t+1}^T with g the per-head scalar
 * gate.  The API passes the gate in log space (section 二: g are log forget
 * gates, g_gamma is a head-wise log decay), so the multiplier is exp(g).
 *
 * Sequences: dense input is B rows of T tokens; packed (varlen) input has
 * B == 1 and cu_seqlens[N+1] marking sequence n as tokens
 * [cu_seqlens[n], cu_seqlens[n+1]) (section 二, FlashAttention convention).
 * Every sequence starts from initial_state[n] (or zeros) and its state after
 * its last token is final_state[n].
 *
 * Decode step (section 四, the fused_recurrent path for short inputs): one
 * token per sequence, S <- exp(g) S + k v^T in place, o = scale S^T q, with g
 * per (sequence, head) or a per-head constant g_gamma.
 *
 * Grouped kv heads (the relinear pages, GQA: k and v have Hkv heads and query
 * head h reads kv head h / (H / Hkv), the contiguous grouping of repeat_kv):
 * every query head keeps its own state and gate; only the k and v rows are
 * shared by the H / Hkv query heads of a group.
 *
 * Parity pins for this file live in tests/test_oracle_pins.py.  The
 * SGLA_ORACLE_MUTANT macro (default 0) exists only so that the test suite can
 * build deliberately wrong copies of this file and show that the pins catch
 * each planted mistake; the shipped build never defines it.
 */
#ifndef SGLA_ORACLE_MUTANT
#define SGLA_ORACLE_MUTANT 0
#endif
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t bos, len;   /* token range of the sequence, in packed token index */
    int64_t seq;        /* sequence index: row of initial_state / final_state */
    int head;
} unit_t;

typedef struct {
    int T_row;          /* unused for packed input */
    int H, Hkv, K, V;
    const double *q, *k, *v, *g, *g_gamma, *h0;
    double scale;
    double *o, *ht;
    const unit_t *units;
    int64_t n_units;
    int64_t next;       /* next unit to take (guarded by mu) */
    pthread_mutex_t mu;
} fwd_job_t;

/* One (sequence, head) recurrence, token by token. */
static void run_unit(const fwd_job_t *J, const unit_t *u, double *S)
{
    const int H = J->H, Hkv = J->Hkv, K = J->K, V = J->V, h = u->head;
#if SGLA_ORACLE_MUTANT == 8
    const int hk = h % Hkv;                 /* planted: interleaved grouping */
#else
    const int hk = h / (H / Hkv);           /* kv head of query head h */
#endif
    const size_t KV = (size_t)K * V;
#if SGLA_ORACLE_MUTANT == 3
    if (J->h0)
        memcpy(S, J->h0 + ((size_t)u->seq * H + (H - 1 - h)) * KV, KV * sizeof(double));
#else
    if (J->h0)
        memcpy(S, J->h0 + ((size_t)u->seq * H + h) * KV, KV * sizeof(double));
#endif
    else
        memset(S, 0, KV * sizeof(double));

    for (int64_t i = 0; i < u->len; ++i) {
        const int64_t t = u->bos + i;
        const double *qt = J->q + ((size_t)t * H + h) * K;
        const double *kt = J->k + ((size_t)t * Hkv + hk) * K;
        const double *vt = J->v + ((size_t)t * Hkv + hk) * V;
        double logg = 0.0;
#if SGLA_ORACLE_MUTANT == 4
        if (J->g) logg = J->g[(size_t)h * J->T_row + (t % (J->T_row > 0 ? J->T_row : 1))];
#else
        if (J->g) logg = J->g[(size_t)t * H + h];
#endif
        else if (J->g_gamma) logg = J->g_gamma[h];
        const double gamma = exp(logg);
        double *ot = J->o + ((size_t)t * H + h) * V;
#if SGLA_ORACLE_MUTANT == 2
        for (int b = 0; b < V; ++b) ot[b] = 0.0;
        for (int a = 0; a < K; ++a)
            for (int b = 0; b < V; ++b) ot[b] += S[(size_t)a * V + b] * qt[a];
#endif

        /* state update: decay the previous state, then add k_t v_t^T */
        for (int a = 0; a < K; ++a) {
            double *row = S + (size_t)a * V;
            const double ka = kt[a];
            for (int b = 0; b < V; ++b)
#if SGLA_ORACLE_MUTANT == 1
                row[b] = gamma * (row[b] + ka * vt[b]);
#else
                row[b] = gamma * row[b] + ka * vt[b];
#endif
        }
#if SGLA_ORACLE_MUTANT != 2
        /* output from the updated state: o_t[b] = scale * sum_a S[a][b] q_t[a] */
        for (int b = 0; b < V; ++b) ot[b] = 0.0;
        for (int a = 0; a < K; ++a) {
            const double *row = S + (size_t)a * V;
#if SGLA_ORACLE_MUTANT == 6
            const double qa = kt[a];
#else
            const double qa = qt[a];
#endif
            for (int b = 0; b < V; ++b) ot[b] += row[b] * qa;
        }
#endif
#if SGLA_ORACLE_MUTANT != 5
        for (int b = 0; b < V; ++b) ot[b] *= J->scale;
#endif
    }
    if (J->ht)
        memcpy(J->ht + ((size_t)u->seq * H + h) * KV, S, KV * sizeof(double));
}

static void *fwd_worker(void *arg)
{
    fwd_job_t *J = (fwd_job_t *)arg;
    double *S = (double *)malloc((size_t)J->K * J->V * sizeof(double));
    if (!S) return (void *)1;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int64_t i = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (i >= J->n_units) break;
        run_unit(J, &J->units[i], S);
    }
    free(S);
    return NULL;
}

/*
 * Forward over all sequences and heads.
 *   q : [B, T, H, K]   k : [B, T, Hkv, K]   v : [B, T, Hkv, V]   o : [B, T, H, V]
 *   (packed: B = 1, T = total tokens; Hkv divides H; Hkv = H is plain MHA)
 *   g    : [B, T, H] log gates, or NULL
 *   g_gamma : [H] per-head log decay, or NULL (at most one of g / g_gamma;
 *             neither means no decay)
 *   h0, ht : [N, H, K, V] or NULL; N = B (dense) or num_seqs (packed)
 *   cu_seqlens : [num_seqs + 1] token offsets (packed) or NULL (dense)
 * Returns 0 on success, negative on a malformed argument.
 */
int sgla_oracle_fwd(int B, int T, int H, int Hkv, int K, int V,
                    const double *q, const double *k, const double *v,
                    const double *g, const double *g_gamma, double scale,
                    const double *h0, const int64_t *cu_seqlens, int num_seqs,
                    double *o, double *ht, int nthreads)
{
    if (B < 0 || T < 0 || H <= 0 || K <= 0 || V <= 0) return -1;
    if (Hkv <= 0 || H % Hkv != 0) return -6;
    if (g && g_gamma) return -2;
    if (cu_seqlens && B != 1) return -3;
    int N = cu_seqlens ? num_seqs : B;
    if (N < 0) return -1;
    int64_t n_units = (int64_t)N * H;
    unit_t *units = (unit_t *)malloc((size_t)(n_units > 0 ? n_units : 1) * sizeof(unit_t));
    if (!units) return -4;
    for (int n = 0; n < N; ++n) {
        int64_t bos, len;
        if (cu_seqlens) {
            bos = cu_seqlens[n];
            len = cu_seqlens[n + 1] - cu_seqlens[n];
            if (len < 0 || bos < 0 || cu_seqlens[n + 1] > (int64_t)T) { free(units); return -5; }
        } else {
            bos = (int64_t)n * T;
            len = T;
        }
        for (int h = 0; h < H; ++h) {
            unit_t *u = &units[(int64_t)n * H + h];
            u->bos = bos; u->len = len; u->seq = n; u->head = h;
        }
    }
    fwd_job_t J;
    J.T_row = T; J.H = H; J.Hkv = Hkv; J.K = K; J.V = V;
    J.q = q; J.k = k; J.v = v; J.g = g; J.g_gamma = g_gamma; J.h0 = h0;
    J.scale = scale; J.o = o; J.ht = ht; J.units = units; J.n_units = n_units; J.next = 0;
    pthread_mutex_init(&J.mu, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    int started = 0, rc = 0;
    for (int i = 1; i < nthreads; ++i)
        if (pthread_create(&th[started], NULL, fwd_worker, &J) == 0) ++started;
    if (fwd_worker(&J) != NULL) rc = -4;
    for (int i = 0; i < started; ++i) {
        void *r = NULL;
        pthread_join(th[i], &r);
        if (r != NULL) rc = -4;
    }
    pthread_mutex_destroy(&J.mu);
    free(units);
    return rc;
}

typedef struct {
    int H, Hkv, K, V;
    const double *q, *k, *v, *g, *g_gamma;
    double scale;
    double *S, *o;
    int64_t n_units, next;
    pthread_mutex_t mu;
} step_job_t;

static void *step_worker(void *arg)
{
    step_job_t *J = (step_job_t *)arg;
    const int K = J->K, V = J->V;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int64_t u = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (u >= J->n_units) break;
        /* unit u = (sequence n, head h) flattened as n * H + h; its k and v
         * rows are those of kv head h / (H / Hkv) of sequence n */
        const int64_t n = u / J->H;
        const int h = (int)(u % J->H);
        const int64_t ukv = n * J->Hkv + h / (J->H / J->Hkv);
        const double *qt = J->q + (size_t)u * K;
        const double *kt = J->k + (size_t)ukv * K;
        const double *vt = J->v + (size_t)ukv * V;
#if SGLA_ORACLE_MUTANT == 9
        const double logg = J->g ? J->g[u] : (J->g_gamma ? J->g_gamma[n % J->H] : 0.0);
#else
        const double logg = J->g ? J->g[u] : (J->g_gamma ? J->g_gamma[h] : 0.0);
#endif
        const double gamma = exp(logg);
        double *S = J->S + (size_t)u * K * V;
        double *ot = J->o + (size_t)u * V;
        for (int a = 0; a < K; ++a)
            for (int b = 0; b < V; ++b)
#if SGLA_ORACLE_MUTANT == 7
                S[(size_t)a * V + b] = gamma * S[(size_t)a * V + b] + kt[b % K] * vt[a % V];
#else
                S[(size_t)a * V + b] = gamma * S[(size_t)a * V + b] + kt[a] * vt[b];
#endif
        for (int b = 0; b < V; ++b) ot[b] = 0.0;
        for (int a = 0; a < K; ++a)
            for (int b = 0; b < V; ++b) ot[b] += S[(size_t)a * V + b] * qt[a];
        for (int b = 0; b < V; ++b) ot[b] *= J->scale;
    }
    return NULL;
}

/*
 * One decode step for N sequences x H heads.
 *   q : [N, H, K]  k : [N, Hkv, K]  v : [N, Hkv, V]  o : [N, H, V]
 *   g : [N, H] log gate, or g_gamma : [H] per-head log decay (at most one;
 *       neither means no decay)
 *   S : [N, H, K, V], updated in place.
 */
int sgla_oracle_step(int N, int H, int Hkv, int K, int V,
                     const double *q, const double *k, const double *v,
                     const double *g, const double *g_gamma, double scale,
                     double *S, double *o, int nthreads)
{
    if (N < 0 || H <= 0 || K <= 0 || V <= 0 || !S) return -1;
    if (g && g_gamma) return -2;
    if (Hkv <= 0 || H % Hkv != 0) return -6;
    step_job_t J;
    J.H = H; J.Hkv = Hkv; J.K = K; J.V = V; J.q = q; J.k = k; J.v = v; J.g = g;
    J.g_gamma = g_gamma;
    J.scale = scale; J.S = S; J.o = o;
    J.n_units = (int64_t)N * H; J.next = 0;
    pthread_mutex_init(&J.mu, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    int started = 0;
    for (int i = 1; i < nthreads; ++i)
        if (pthread_create(&th[started], NULL, step_worker, &J) == 0) ++started;
    step_worker(&J);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    pthread_mutex_destroy(&J.mu);
    return 0;
}

/*
 * Chunk-local cumulative log gate, pre-scaled by 1/ln 2 (page "flash-linear-
 * attention 中的 Simple GLA", section 三: the chunk_local_cumsum call with
 * the RCP_LN2 scale, one scalar sequence per head).  For token t of a
 * sequence that starts at bos, the chunk starts at
 * c0 = bos + floor((t - bos) / chunk) * chunk and
 *     gc[t][h] = (sum_{j = c0..t} g[j][h]) / ln 2.
 *   g, gc : [B, T, H];  cu_seqlens as for sgla_oracle_fwd.
 */
int sgla_oracle_chunk_local_cumsum(int B, int T, int H, const double *g,
                                   const int64_t *cu_seqlens, int num_seqs,
                                   int chunk, double *gc)
{
    if (B < 0 || T < 0 || H <= 0 || chunk <= 0) return -1;
    if (cu_seqlens && B != 1) return -3;
    const int N = cu_seqlens ? num_seqs : B;
    const double ln2 = log(2.0);
    for (int n = 0; n < N; ++n) {
        const int64_t bos = cu_seqlens ? cu_seqlens[n] : (int64_t)n * T;
        const int64_t eos = cu_seqlens ? cu_seqlens[n + 1] : (int64_t)(n + 1) * T;
        for (int h = 0; h < H; ++h) {
            double run = 0.0;
            for (int64_t t = bos; t < eos; ++t) {
                if ((t - bos) % chunk == 0) run = 0.0;
                run += g[(size_t)t * H + h];
                gc[(size_t)t * H + h] = run / ln2;
            }
        }
    }
    return 0;
}

/*
 * Backward of sgla_oracle_fwd (page "flash-linear-attention 中的 Simple GLA",
 * section 三: the backward produces the q, k, v and gate gradients and the
 * initial-state gradient from an fp32 state trajectory; section 五: its tests
 * compare dq, dk, dv, dg and dh0 with the naive recurrent reference).
 *
 * Gradients of   L = sum_t <do_t, o_t> + sum_n <dht_n, final_state_n>
 * by reverse-mode differentiation of the token recurrence itself.  Forward,
 * keeping every state S_0 (initial) .. S_L:  S_t = gamma_t S_{t-1} + k_t v_t^T
 * with gamma_t = exp(g_t).  Then in reverse, with D the gradient with respect
 * to S_t:
 *     D    = dht (or 0)                       before the last token
 *     D   += scale q_t do_t^T                 (o_t = scale S_t^T q_t)
 *     dq_t = scale S_t do_t
 *     dk_t = D v_t ,   dv_t = D^T k_t         (S_t receives k_t v_t^T)
 *     dg_t = gamma_t <D, S_{t-1}>             (d gamma_t / d g_t = gamma_t)
 *     D    = gamma_t D                        (now the gradient of S_{t-1})
 * and dh0 = D after the first token.  With g_gamma the gradient of g_gamma[h]
 * is the sum of dg_t over every token of every sequence of head h.  Plain
 * multi-head input (k and v with H heads).
 */
typedef struct {
    int H, K, V;
    const double *q, *k, *v, *g, *g_gamma, *h0, *dout, *dht;
    double scale;
    double *dq, *dk, *dv, *dg, *dh0;
    double *gamma_part;   /* [n_units] sum of dg_t of the unit (g_gamma) */
    const unit_t *units;
    int64_t n_units, next;
    int64_t max_len;
    pthread_mutex_t mu;
} bwd_job_t;

static void bwd_unit(const bwd_job_t *J, int64_t ui, double *Sall, double *D)
{
    const unit_t *u = &J->units[ui];
    const int H = J->H, K = J->K, V = J->V, h = u->head;
    const int64_t KV = (int64_t)K * V;
    /* forward, keeping S_0 .. S_len */
    double *S0 = Sall;
    const double *h0 = J->h0 ? J->h0 + (u->seq * H + h) * KV : NULL;
    for (int64_t i = 0; i < KV; ++i) S0[i] = h0 ? h0[i] : 0.0;
    for (int64_t s = 0; s < u->len; ++s) {
        const int64_t t = u->bos + s;
        const double *kt = J->k + ((size_t)t * H + h) * K;
        const double *vt = J->v + ((size_t)t * H + h) * V;
        const double logg = J->g ? J->g[(size_t)t * H + h] : (J->g_gamma ? J->g_gamma[h] : 0.0);
        const double gamma = exp(logg);
        const double *Sp = Sall + s * KV;
        double *Sn = Sall + (s + 1) * KV;
        for (int a = 0; a < K; ++a)
            for (int b = 0; b < V; ++b)
                Sn[(int64_t)a * V + b] = gamma * Sp[(int64_t)a * V + b] + kt[a] * vt[b];
    }
    /* reverse */
    const double *dht = J->dht ? J->dht + (u->seq * H + h) * KV : NULL;
    for (int64_t i = 0; i < KV; ++i) D[i] = dht ? dht[i] : 0.0;
    double gsum = 0.0;
    for (int64_t s = u->len - 1; s >= 0; --s) {
        const int64_t t = u->bos + s;
        const double *qt = J->q + ((size_t)t * H + h) * K;
        const double *kt = J->k + ((size_t)t * H + h) * K;
        const double *vt = J->v + ((size_t)t * H + h) * V;
        const double *dot = J->dout + ((size_t)t * H + h) * V;
        const double logg = J->g ? J->g[(size_t)t * H + h] : (J->g_gamma ? J->g_gamma[h] : 0.0);
        const double gamma = exp(logg);
        const double *St = Sall + (s + 1) * KV;
        const double *Sp = Sall + s * KV;
        double *dqt = J->dq + ((size_t)t * H + h) * K;
        double *dkt = J->dk + ((size_t)t * H + h) * K;
        double *dvt = J->dv + ((size_t)t * H + h) * V;
#if SGLA_ORACLE_MUTANT != 12
        for (int a = 0; a < K; ++a)
            for (int b = 0; b < V; ++b) D[(int64_t)a * V + b] += J->scale * qt[a] * dot[b];
#endif
        for (int a = 0; a < K; ++a) {
            double x = 0.0;
            for (int b = 0; b < V; ++b) x += St[(int64_t)a * V + b] * dot[b];
            dqt[a] = J->scale * x;
        }
        for (int a = 0; a < K; ++a) {
            double x = 0.0;
            for (int b = 0; b < V; ++b) x += D[(int64_t)a * V + b] * vt[b];
            dkt[a] = x;
        }
        for (int b = 0; b < V; ++b) {
            double x = 0.0;
            for (int a = 0; a < K; ++a) x += D[(int64_t)a * V + b] * kt[a];
            dvt[b] = x;
        }
#if SGLA_ORACLE_MUTANT == 12
        for (int a = 0; a < K; ++a)
            for (int b = 0; b < V; ++b) D[(int64_t)a * V + b] += J->scale * qt[a] * dot[b];
#endif
        double inner = 0.0;
#if SGLA_ORACLE_MUTANT == 11
        for (int64_t i = 0; i < KV; ++i) inner += D[i] * St[i];
#else
        for (int64_t i = 0; i < KV; ++i) inner += D[i] * Sp[i];
#endif
        const double dgt = gamma * inner;
        if (J->dg) J->dg[(size_t)t * H + h] = dgt;
        gsum += dgt;
#if SGLA_ORACLE_MUTANT != 10
        for (int64_t i = 0; i < KV; ++i) D[i] *= gamma;
#endif
    }
    if (J->dh0) {
        double *d0 = J->dh0 + (u->seq * H + h) * KV;
        for (int64_t i = 0; i < KV; ++i) d0[i] = D[i];
    }
    J->gamma_part[ui] = gsum;
}

static void *bwd_worker(void *arg)
{
    bwd_job_t *J = (bwd_job_t *)arg;
    const int64_t KV = (int64_t)J->K * J->V;
    double *Sall = (double *)malloc((size_t)(J->max_len + 1) * KV * sizeof(double));
    double *D = (double *)malloc((size_t)KV * sizeof(double));
    if (!Sall || !D) { free(Sall); free(D); return (void *)1; }
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int64_t i = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (i >= J->n_units) break;
        bwd_unit(J, i, Sall, D);
    }
    free(Sall);
    free(D);
    return NULL;
}

/*
 * Backward over all sequences and heads (multi-head: k, v have H heads).
 *   q, k, dq, dk : [B, T, H, K]   v, dout, dv : [B, T, H, V]
 *   g, dg : [B, T, H] or NULL;  g_gamma, dg_gamma : [H] or NULL
 *   h0, dht, dh0 : [N, H, K, V] or NULL (dht NULL = no loss on the final state)
 *   cu_seqlens : [num_seqs + 1] or NULL, as for sgla_oracle_fwd.
 * dq, dk, dv are required; dg is written when given (g given), dg_gamma when
 * given (g_gamma given), dh0 when given.  Returns 0, or negative on a
 * malformed argument.
 */
int sgla_oracle_bwd(int B, int T, int H, int K, int V,
                    const double *q, const double *k, const double *v,
                    const double *g, const double *g_gamma, double scale,
                    const double *h0, const int64_t *cu_seqlens, int num_seqs,
                    const double *dout, const double *dht,
                    double *dq, double *dk, double *dv, double *dg, double *dg_gamma,
                    double *dh0, int nthreads)
{
    if (B < 0 || T < 0 || H <= 0 || K <= 0 || V <= 0) return -1;
    if (g && g_gamma) return -2;
    if (cu_seqlens && B != 1) return -3;
    if (!dq || !dk || !dv) return -1;
    int N = cu_seqlens ? num_seqs : B;
    if (N < 0) return -1;
    int64_t n_units = (int64_t)N * H;
    unit_t *units = (unit_t *)malloc((size_t)(n_units > 0 ? n_units : 1) * sizeof(unit_t));
    double *part = (double *)calloc((size_t)(n_units > 0 ? n_units : 1), sizeof(double));
    if (!units || !part) { free(units); free(part); return -4; }
    int64_t max_len = 0;
    for (int n = 0; n < N; ++n) {
        int64_t bos, len;
        if (cu_seqlens) {
            bos = cu_seqlens[n];
            len = cu_seqlens[n + 1] - cu_seqlens[n];
            if (len < 0 || bos < 0 || cu_seqlens[n + 1] > (int64_t)T) { free(units); free(part); return -5; }
        } else {
            bos = (int64_t)n * T;
            len = T;
        }
        if (len > max_len) max_len = len;
        for (int h = 0; h < H; ++h) {
            unit_t *u = &units[(int64_t)n * H + h];
            u->bos = bos; u->len = len; u->seq = n; u->head = h;
        }
    }
    bwd_job_t J;
    J.H = H; J.K = K; J.V = V;
    J.q = q; J.k = k; J.v = v; J.g = g; J.g_gamma = g_gamma; J.h0 = h0; J.dout = dout; J.dht = dht;
    J.scale = scale; J.dq = dq; J.dk = dk; J.dv = dv; J.dg = g ? dg : NULL; J.dh0 = dh0;
    J.gamma_part = part; J.units = units; J.n_units = n_units; J.next = 0; J.max_len = max_len;
    pthread_mutex_init(&J.mu, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    int started = 0, rc = 0;
    for (int i = 1; i < nthreads; ++i)
        if (pthread_create(&th[started], NULL, bwd_worker, &J) == 0) ++started;
    if (bwd_worker(&J) != NULL) rc = -4;
    for (int i = 0; i < started; ++i) {
        void *r = NULL;
        pthread_join(th[i], &r);
        if (r != NULL) rc = -4;
    }
    pthread_mutex_destroy(&J.mu);
    if (rc == 0 && g_gamma && dg_gamma) {
        for (int h = 0; h < H; ++h) {
            double s = 0.0;
            for (int n = 0; n < N; ++n) s += part[(int64_t)n * H + h];
            dg_gamma[h] = s;
        }
    }
    free(units);
    free(part);
    return rc;
}

/*
 * Elementwise-gate GLA (the general GLA the Simple GLA page contrasts with:
 * its gate decays every state element independently; the relinear pages pass
 * fla's chunk_gla a gate vector over the key dimension, of which the
 * head-wise scalar gate is the special case):
 *
 *     S_t = diag(exp(gk_t)) S_{t-1} + k_t v_t^T ,    o_t = scale * S_t^T q_t
 *
 * with gk_t a log gate per (token, head, key): row a of the state decays by
 * exp(gk_t[a]).
 *   q, gk : [B, T, H, K]   k : [B, T, Hkv, K]   v : [B, T, Hkv, V]
 *   o : [B, T, H, V]   h0, ht : [N, H, K, V] or NULL; cu_seqlens as above.
 */
typedef struct {
    int H, Hkv, K, V;
    const double *q, *k, *v, *gk, *h0;
    double scale;
    double *o, *ht;
    const unit_t *units;
    int64_t n_units, next;
    pthread_mutex_t mu;
} gla_job_t;

static void *gla_worker(void *arg)
{
    gla_job_t *J = (gla_job_t *)arg;
    const int H = J->H, Hkv = J->Hkv, K = J->K, V = J->V;
    double *S = (double *)malloc((size_t)K * V * sizeof(double));
    if (!S) return (void *)1;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int64_t i = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (i >= J->n_units) break;
        const unit_t *u = &J->units[i];
        const int h = u->head;
#if SGLA_ORACLE_MUTANT == 13
        const int hk = h % Hkv;
#else
        const int hk = h / (H / Hkv);
#endif
        const double *h0 = J->h0 ? J->h0 + ((size_t)u->seq * H + h) * K * V : NULL;
        for (int64_t e = 0; e < (int64_t)K * V; ++e) S[e] = h0 ? h0[e] : 0.0;
        for (int64_t s = 0; s < u->len; ++s) {
            const int64_t t = u->bos + s;
            const double *qt = J->q + ((size_t)t * H + h) * K;
            const double *gt = J->gk + ((size_t)t * H + h) * K;
            const double *kt = J->k + ((size_t)t * Hkv + hk) * K;
            const double *vt = J->v + ((size_t)t * Hkv + hk) * V;
            for (int a = 0; a < K; ++a) {
                const double decay = exp(gt[a]);
                for (int b = 0; b < V; ++b) {
#if SGLA_ORACLE_MUTANT == 14
                    /* planted: gate indexed by the value column */
                    S[(int64_t)a * V + b] = exp(gt[b % K]) * S[(int64_t)a * V + b] + kt[a] * vt[b];
#else
                    S[(int64_t)a * V + b] = decay * S[(int64_t)a * V + b] + kt[a] * vt[b];
#endif
                }
            }
            double *ot = J->o + ((size_t)t * H + h) * V;
            for (int b = 0; b < V; ++b) {
                double acc = 0.0;
                for (int a = 0; a < K; ++a) acc += S[(int64_t)a * V + b] * qt[a];
                ot[b] = J->scale * acc;
            }
        }
        if (J->ht) {
            double *ht = J->ht + ((size_t)u->seq * H + h) * K * V;
            for (int64_t e = 0; e < (int64_t)K * V; ++e) ht[e] = S[e];
        }
    }
    free(S);
    return NULL;
}

int sgla_oracle_gla_fwd(int B, int T, int H, int Hkv, int K, int V,
                        const double *q, const double *k, const double *v, const double *gk,
                        double scale, const double *h0, const int64_t *cu_seqlens, int num_seqs,
                        double *o, double *ht, int nthreads)
{
    if (B < 0 || T < 0 || H <= 0 || K <= 0 || V <= 0 || !gk) return -1;
    if (Hkv <= 0 || H % Hkv != 0) return -6;
    if (cu_seqlens && B != 1) return -3;
    int N = cu_seqlens ? num_seqs : B;
    if (N < 0) return -1;
    int64_t n_units = (int64_t)N * H;
    unit_t *units = (unit_t *)malloc((size_t)(n_units > 0 ? n_units : 1) * sizeof(unit_t));
    if (!units) return -4;
    for (int n = 0; n < N; ++n) {
        int64_t bos, len;
        if (cu_seqlens) {
            bos = cu_seqlens[n];
            len = cu_seqlens[n + 1] - cu_seqlens[n];
            if (len < 0 || bos < 0 || cu_seqlens[n + 1] > (int64_t)T) { free(units); return -5; }
        } else {
            bos = (int64_t)n * T;
            len = T;
        }
        for (int hh = 0; hh < H; ++hh) {
            unit_t *u = &units[(int64_t)n * H + hh];
            u->bos = bos; u->len = len; u->seq = n; u->head = hh;
        }
    }
    gla_job_t J;
    J.H = H; J.Hkv = Hkv; J.K = K; J.V = V;
    J.q = q; J.k = k; J.v = v; J.gk = gk; J.h0 = h0; J.scale = scale; J.o = o; J.ht = ht;
    J.units = units; J.n_units = n_units; J.next = 0;
    pthread_mutex_init(&J.mu, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    int started = 0, rc = 0;
    for (int i = 1; i < nthreads; ++i)
        if (pthread_create(&th[started], NULL, gla_worker, &J) == 0) ++started;
    if (gla_worker(&J) != NULL) rc = -4;
    for (int i = 0; i < started; ++i) {
        void *r = NULL;
        pthread_join(th[i], &r);
        if (r != NULL) rc = -4;
    }
    pthread_mutex_destroy(&J.mu);
    free(units);
    return rc;
}

/*
 * Parallel form (page "flash-linear-attention 中的 Simple GLA", section 二:
 * the parallel entry builds the decayed attention matrix A explicitly;
 * section 五: its test compares that A with a directly built decay matrix).
 * Per batch row b and query head h, with G_t = g_0 + ... + g_t (g_t = g_gamma[h]
 * for the data-independent decay, 0 when neither gate is given):
 *
 *     A[i][j] = scale * (q_i . k_j) * exp(G_i - G_j)   for j <= i,  else 0
 *     o_i     = sum_j A[i][j] v_j
 *
 * which is the recurrence above unrolled from a zero state: exp(G_i - G_j)
 * is the product of the gates of tokens j+1 .. i.
 *   q [B, T, H, K], k [B, T, Hkv, K], v [B, T, Hkv, V], g [B, T, H] or NULL,
 *   g_gamma [H] or NULL; o [B, T, H, V]; attn [B, H, T, T] or NULL.
 * Dense input only (no initial state, no final state).
 */
typedef struct {
    int T, H, Hkv, K, V;
    const double *q, *k, *v, *g, *g_gamma;
    double scale;
    double *o, *attn;
    int64_t n_units, next;
    pthread_mutex_t mu;
} par_job_t;

static void *par_worker(void *arg)
{
    par_job_t *J = (par_job_t *)arg;
    const int T = J->T, H = J->H, Hkv = J->Hkv, K = J->K, V = J->V;
    double *G = (double *)malloc((size_t)(T > 0 ? T : 1) * sizeof(double));
    if (!G) return (void *)1;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int64_t u = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (u >= J->n_units) break;
        const int64_t b = u / H;
        const int h = (int)(u % H);
        const int hk = h / (H / Hkv);
        double run = 0.0;
        for (int t = 0; t < T; ++t) {
            const double gt = J->g ? J->g[((size_t)b * T + t) * H + h]
                                   : (J->g_gamma ? J->g_gamma[h] : 0.0);
            run += gt;
            G[t] = run;
        }
        double *A = J->attn ? J->attn + (size_t)u * T * T : NULL;
        for (int i = 0; i < T; ++i) {
            const double *qi = J->q + (((size_t)b * T + i) * H + h) * K;
            double *oi = J->o + (((size_t)b * T + i) * H + h) * V;
            for (int c = 0; c < V; ++c) oi[c] = 0.0;
            for (int j = 0; j < T; ++j) {
#if SGLA_ORACLE_MUTANT == 15
                /* planted: strictly causal mask, the token's own term dropped */
                const int keep = j < i;
#else
                const int keep = j <= i;
#endif
                double a = 0.0;
                if (keep) {
                    const double *kj = J->k + (((size_t)b * T + j) * Hkv + hk) * K;
                    double dot = 0.0;
                    for (int e = 0; e < K; ++e) dot += qi[e] * kj[e];
#if SGLA_ORACLE_MUTANT == 16
                    /* planted: the key token's own gate counted in the decay */
                    const double gj = G[j] - (j > 0 ? G[j - 1] : 0.0);
                    a = J->scale * dot * exp(G[i] - G[j] + gj);
#else
                    a = J->scale * dot * exp(G[i] - G[j]);
#endif
                    const double *vj = J->v + (((size_t)b * T + j) * Hkv + hk) * V;
                    for (int c = 0; c < V; ++c) oi[c] += a * vj[c];
                }
                if (A) A[(size_t)i * T + j] = a;
            }
        }
    }
    free(G);
    return NULL;
}

int sgla_oracle_parallel(int B, int T, int H, int Hkv, int K, int V,
                         const double *q, const double *k, const double *v,
                         const double *g, const double *g_gamma, double scale,
                         double *o, double *attn, int nthreads)
{
    if (B < 0 || T < 0 || H <= 0 || K <= 0 || V <= 0) return -1;
    if (Hkv <= 0 || H % Hkv != 0) return -6;
    if (g && g_gamma) return -2;
    par_job_t J;
    J.T = T; J.H = H; J.Hkv = Hkv; J.K = K; J.V = V;
    J.q = q; J.k = k; J.v = v; J.g = g; J.g_gamma = g_gamma; J.scale = scale;
    J.o = o; J.attn = attn; J.n_units = (int64_t)B * H; J.next = 0;
    pthread_mutex_init(&J.mu, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    int started = 0, rc = 0;
    for (int i = 1; i < nthreads; ++i)
        if (pthread_create(&th[started], NULL, par_worker, &J) == 0) ++started;
    if (par_worker(&J) != NULL) rc = -4;
    for (int i = 0; i < started; ++i) {
        void *r = NULL;
        pthread_join(th[i], &r);
        if (r != NULL) rc = -4;
    }
    pthread_mutex_destroy(&J.mu);
    return rc;
}

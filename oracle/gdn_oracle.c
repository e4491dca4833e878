/*
 * gdn_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU statement of the gated delta rule, written to be
 * checked against its definition by eye.  Only the test suite, the smoke check
 * and the CPU-baseline leg of the benchmark may load it; the GPU library never
 * links, calls or includes anything from here, and nothing here comes from the
 * GPU library.
 *
 * What it computes (the Gated DeltaNet recurrence, Yang, Kautz and Hatamizadeh,
 * "Gated Delta Networks: Improving Mamba2 with Delta Rule", ICLR 2025; the pages
 * name the kernel family that implements it, gated_delta_rule_*, in the module
 * doc of ssm_gdn_tc_route.rs and of ssm_gdn_woa.rs):
 *
 *     S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t q_t
 *
 * S_t is dv x dk.  This file stores h = S^T (dk rows, dv columns, row-major),
 * the layout the pages' state buffers use (dk*dv fp32 per head, ssm_gdn_woa.rs,
 * the shared-memory size of the verify launch).  Expanding the product gives the
 * token step used below:
 *
 *     h      <- alpha_t h                       (decay first)
 *     p_j     = sum_i h[i][j] k_t[i]            (prediction of the decayed state)
 *     delta_j = beta_t (v_t[j] - p_j)
 *     h[i][j] += k_t[i] delta_j
 *     o_t[j]  = sum_i h[i][j] q_t[i]           (the updated state answers q_t)
 *
 * alpha_t = exp(log_g[t]); no scale is applied to q.  Multi-head: v-head vh
 * reads k-head vh / (Hv/Hk) (contiguous groups, as the v-head grouping of
 * ssm_ba_gates_hopper.rs, "the index model", pairs a group with its v-heads).
 *
 * Every input is read exactly as fp64 (the caller widens bf16/fp32 values,
 * which is exact), and all arithmetic is fp64.  Threads split the independent
 * (sequence, v-head) pairs; each pair runs strictly in token order.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* One (sequence, v-head) walk over L tokens.
 *   q, k      : row r of this head at q + r*qk_row (dk values)
 *   v         : row r at v + r*v_row (dv values)
 *   log_g,beta: row r at [r*gb_row]
 *   h         : dk*dv state, updated in place
 *   out       : row r at out + r*out_row (dv values), may be NULL
 *   states    : if not NULL, the state after token r is copied to states + r*dk*dv
 */
static void token_walk(const double* q, const double* k, const double* v,
                       const double* log_g, const double* beta,
                       long qk_row, long v_row, long gb_row, long out_row,
                       double* h, double* out, double* states,
                       long L, int dk, int dv, double* p /* dv scratch */)
{
    for (long t = 0; t < L; ++t) {
        const double* kt = k + t * qk_row;
        const double* qt = q + t * qk_row;
        const double* vt = v + t * v_row;
        const double alpha = exp(log_g[t * gb_row]);
        const double b = beta[t * gb_row];

        for (long e = 0; e < (long)dk * dv; ++e) h[e] *= alpha;

        for (int j = 0; j < dv; ++j) p[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) p[j] += h[(long)i * dv + j] * kt[i];

        for (int j = 0; j < dv; ++j) p[j] = b * (vt[j] - p[j]); /* p now holds delta */

        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) h[(long)i * dv + j] += kt[i] * p[j];

        if (out) {
            double* ot = out + t * out_row;
            for (int j = 0; j < dv; ++j) ot[j] = 0.0;
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) ot[j] += h[(long)i * dv + j] * qt[i];
        }
        if (states) memcpy(states + t * (long)dk * dv, h, sizeof(double) * (size_t)dk * dv);
    }
}

/* ------------------------------------------------------------------------- */
/* Prefill: B sequences, dense ([B][T] rows) or packed (cu_seqlens).          */

typedef struct {
    const double *q, *k, *v, *log_g, *beta, *h0;
    double *out, *h_final;
    int B, T, Hk, Hv, dk, dv;
    const int64_t* cu;
    const int32_t* heads; /* v-heads to compute, or NULL for all */
    int n_heads;
    long n_jobs, next_job;
    pthread_mutex_t lock;
} prefill_ctx;

static void prefill_job(prefill_ctx* c, long job, double* h, double* p)
{
    const int b = (int)(job / c->n_heads);
    const int hslot = (int)(job % c->n_heads);
    const int vh = c->heads ? c->heads[hslot] : hslot;
    const int kh = vh / (c->Hv / c->Hk);
    const long dkdv = (long)c->dk * c->dv;
    long r0, L;
    if (c->cu) { r0 = c->cu[b]; L = c->cu[b + 1] - c->cu[b]; }
    else       { r0 = (long)b * c->T; L = c->T; }

    if (c->h0) memcpy(h, c->h0 + ((long)b * c->Hv + vh) * dkdv, sizeof(double) * (size_t)dkdv);
    else       memset(h, 0, sizeof(double) * (size_t)dkdv);

    token_walk(c->q + (r0 * c->Hk + kh) * c->dk,
               c->k + (r0 * c->Hk + kh) * c->dk,
               c->v + (r0 * c->Hv + vh) * c->dv,
               c->log_g + r0 * c->Hv + vh,
               c->beta + r0 * c->Hv + vh,
               (long)c->Hk * c->dk, (long)c->Hv * c->dv, c->Hv, (long)c->Hv * c->dv,
               h, c->out ? c->out + (r0 * c->Hv + vh) * c->dv : NULL, NULL,
               L, c->dk, c->dv, p);

    if (c->h_final)
        memcpy(c->h_final + ((long)b * c->Hv + vh) * dkdv, h, sizeof(double) * (size_t)dkdv);
}

static void* prefill_worker(void* arg)
{
    prefill_ctx* c = (prefill_ctx*)arg;
    double* h = (double*)malloc(sizeof(double) * (size_t)c->dk * c->dv);
    double* p = (double*)malloc(sizeof(double) * (size_t)c->dv);
    for (;;) {
        pthread_mutex_lock(&c->lock);
        long job = c->next_job++;
        pthread_mutex_unlock(&c->lock);
        if (job >= c->n_jobs) break;
        prefill_job(c, job, h, p);
    }
    free(h);
    free(p);
    return NULL;
}

/*
 * Returns 0 on success, -1 on a shape error.
 * q, k: [N][Hk][dk]; v, out: [N][Hv][dv]; log_g, beta: [N][Hv];
 * h0, h_final: [B][Hv][dk][dv] (either may be NULL; NULL h0 means zeros).
 * Dense input (cu_seqlens == NULL): N = B*T.  Packed: N = cu_seqlens[B].
 * heads: optional list of v-heads to compute (others are not written).
 */
int gdn_oracle_prefill(const double* q, const double* k, const double* v,
                       const double* log_g, const double* beta, const double* h0,
                       double* out, double* h_final,
                       int B, int T, int Hk, int Hv, int dk, int dv,
                       const int64_t* cu_seqlens, const int32_t* heads, int n_heads,
                       int nthreads)
{
    if (B < 0 || T < 0 || Hk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || Hv % Hk != 0) return -1;
    prefill_ctx c;
    c.q = q; c.k = k; c.v = v; c.log_g = log_g; c.beta = beta; c.h0 = h0;
    c.out = out; c.h_final = h_final;
    c.B = B; c.T = T; c.Hk = Hk; c.Hv = Hv; c.dk = dk; c.dv = dv;
    c.cu = cu_seqlens;
    c.heads = heads;
    c.n_heads = heads ? n_heads : Hv;
    c.n_jobs = (long)B * c.n_heads;
    c.next_job = 0;
    pthread_mutex_init(&c.lock, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > c.n_jobs) nthreads = (int)(c.n_jobs > 0 ? c.n_jobs : 1);
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, prefill_worker, &c);
    prefill_worker(&c);
    for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&c.lock);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Decode verify of K draft rows per sequence (ssm_gdn_woa.rs, doc of
 * gdn_decode_wy4_woa and gdn_wy4_fold): the K rows of sequence b are the
 * same recurrence run from that sequence's state.  The oracle returns the
 * outputs of all K rows and the state after each prefix, so that the state
 * a fold with na accepted rows must leave is states_after[na] (na = 0 is the
 * untouched state).
 *
 * states   : [B][Hv][dk][dv]   (the state of each sequence before verify)
 * q, k     : [B*K][Hk][dk];  v, out: [B*K][Hv][dv];  gate, beta: [B*K][Hv]
 * after    : [B][K+1][Hv][dk][dv]
 */
int gdn_oracle_decode(const double* states, const double* q, const double* k,
                      const double* v, const double* gate, const double* beta,
                      double* out, double* after,
                      int B, int K, int Hk, int Hv, int dk, int dv)
{
    if (B < 0 || K <= 0 || Hk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || Hv % Hk != 0) return -1;
    const long dkdv = (long)dk * dv;
    double* h = (double*)malloc(sizeof(double) * (size_t)dkdv);
    double* p = (double*)malloc(sizeof(double) * (size_t)dv);
    double* st = (double*)malloc(sizeof(double) * (size_t)(dkdv * K));
    for (int b = 0; b < B; ++b)
        for (int vh = 0; vh < Hv; ++vh) {
            const int kh = vh / (Hv / Hk);
            const long r0 = (long)b * K;
            memcpy(h, states + ((long)b * Hv + vh) * dkdv, sizeof(double) * (size_t)dkdv);
            /* after[b][0][vh] = the state before any row */
            memcpy(after + (((long)b * (K + 1) + 0) * Hv + vh) * dkdv, h,
                   sizeof(double) * (size_t)dkdv);
            token_walk(q + (r0 * Hk + kh) * dk, k + (r0 * Hk + kh) * dk,
                       v + (r0 * Hv + vh) * dv, gate + r0 * Hv + vh, beta + r0 * Hv + vh,
                       (long)Hk * dk, (long)Hv * dv, Hv, (long)Hv * dv,
                       h, out + (r0 * Hv + vh) * dv, st, K, dk, dv, p);
            for (int r = 1; r <= K; ++r)
                memcpy(after + (((long)b * (K + 1) + r) * Hv + vh) * dkdv,
                       st + (long)(r - 1) * dkdv, sizeof(double) * (size_t)dkdv);
        }
    free(h);
    free(p);
    free(st);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* The gate/beta producer (the BA projection) ahead of the recurrence.
 *
 * The pages give its launcher and index model (ssm_ba_gates_hopper.rs, the
 * launcher of dense_gemm_ba_gates_prefill_hopper and "the index model"): every
 * token's activation row (k values) is multiplied by n = 2*nv weight rows,
 * and output n lands, by ba_gates_slot, in the token's output row
 * [gate(nv) | beta(nv)]: with G = vheads_per_group, group = n / (2G) and
 * w = n % (2G), the first G outputs of a group are beta of v-heads
 * group*G + w and the next G the gates of v-heads group*G + (w - G).
 *
 * The activation of the two halves is not printed on the pages; the reading
 * taken (from the names a_log and dt_bias the launcher passes) is the usual
 * Gated DeltaNet gating:
 *     gate = -exp(a_log[vh]) * softplus(y + dt_bias[vh])   (log of alpha)
 *     beta = 1 / (1 + exp(-y))
 * with softplus(z) = log(1 + exp(z)), evaluated as max(z, 0) + log1p(exp(-|z|)),
 * the same number without overflow.
 *
 * x   : [m][x_stride] (the first k values of a row are used)
 * w   : [n][k]
 * out : [m][out_stride]; columns 0..nv-1 gate, nv..2nv-1 beta
 * Returns 0, or -1 on a shape error.
 */
static double softplus(double z) { return (z > 0.0 ? z : 0.0) + log1p(exp(-fabs(z))); }

int gdn_oracle_ba_gates(const double* x, const double* w, const double* a_log,
                        const double* dt_bias, double* out, int m, int n, int k,
                        long x_stride, long out_stride, int nv, int G)
{
    if (m < 0 || k <= 0 || nv <= 0 || G <= 0 || n != 2 * nv || nv % G != 0 ||
        x_stride < k || out_stride < 2L * nv)
        return -1;
    for (int t = 0; t < m; ++t) {
        const double* xt = x + (long)t * x_stride;
        double* ot = out + (long)t * out_stride;
        for (int o = 0; o < n; ++o) {
            double y = 0.0;
            for (int i = 0; i < k; ++i) y += xt[i] * w[(long)o * k + i];
            const int group = o / (2 * G), within = o % (2 * G);
            if (within < G) {
                const int vh = group * G + within;
                ot[nv + vh] = 1.0 / (1.0 + exp(-y));
            } else {
                const int vh = group * G + (within - G);
                ot[vh] = -exp(a_log[vh]) * softplus(y + dt_bias[vh]);
            }
        }
    }
    return 0;
}

/*
 * Gated DeltaNet forward and backward: plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header or constant with the HIP
 * library.
 *
 * What it computes (the method's plain definition, token by token, no
 * chunking, no blocking, no reordering):
 *
 *   The gated delta rule S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T)
 *   + beta_t v_t k_t^T and o_t = scale * S_t q_t, as stated for the Gated
 *   DeltaNet layer that the FlashQLA pages optimise (agentlenshq.com,
 *   "GDN chunked prefill" and "AutoCP" sections: gates alpha = exp(g) lie in
 *   (0,1); aisparkup.com "high-level API": q,k [B,T,H_q,K], v [B,T,H_v,V],
 *   g and beta [B,T,H_v], scale, initial_state, output_final_state,
 *   cu_seqlens).  The pages never print the recurrence; the formula above is
 *   the one the GDN layer defines and every quantity the pages name (W, U,
 *   S, V', O, M, g, A, h) is derived from it.
 *
 * State orientation: we keep H = S^T, a K x V matrix, because the state
 * tensors are laid out [N, H_v, K, V].  Expanding the product form,
 *
 *   H <- a H                        (decay first)
 *   u  = beta (v - H^T k)           (delta-rule residual, a V-vector)
 *   H <- H + k u^T
 *   o  = scale H^T q
 *
 * which is exactly S_t = a S_{t-1} (I - beta k k^T) + beta v k^T transposed.
 *
 * Grouped heads: v-head j reads q/k head floor(j / (H_v / H_qk)).
 * Varlen: cu_seqlens (int32, N+1 offsets, B == 1) splits the packed token
 * axis into independent sequences, each starting from its own initial state.
 *
 * Inputs are passed as double arrays (the exact bf16 / float32 input values
 * widen to double without rounding; finite-difference checks perturb them in
 * double); all arithmetic is double.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t B, T;
    int Hqk, Hv, K, V, N;
    const double *q, *k, *v, *g, *beta, *h0;
    const int32_t *cu;
    double scale;
    double *o, *ht;
    int next_unit; /* shared work counter */
    pthread_mutex_t lock;
} fwd_job;

/* Token rows [r0, r1) of the flattened [B*T] axis that sequence n covers. */
static void seq_rows(const fwd_job *J, int n, int64_t *r0, int64_t *r1)
{
    if (J->cu) {
        *r0 = J->cu[n];
        *r1 = J->cu[n + 1];
    } else {
        *r0 = (int64_t)n * J->T;
        *r1 = (int64_t)(n + 1) * J->T;
    }
}

static void fwd_unit(const fwd_job *J, int n, int j, double *H, double *p, double *u)
{
    const int K = J->K, V = J->V;
    const int grp = J->Hv / J->Hqk;
    const int i = j / grp;
    int64_t r0, r1;
    seq_rows(J, n, &r0, &r1);

    if (J->h0) {
        const double *s = J->h0 + ((int64_t)n * J->Hv + j) * K * V;
        for (int e = 0; e < K * V; ++e) H[e] = (double)s[e];
    } else {
        memset(H, 0, sizeof(double) * (size_t)K * V);
    }

    for (int64_t r = r0; r < r1; ++r) {
        const double *kt = J->k + (r * J->Hqk + i) * K;
        const double *qt = J->q + (r * J->Hqk + i) * K;
        const double *vt = J->v + (r * J->Hv + j) * V;
        const double a = exp((double)J->g[r * J->Hv + j]);
        const double b = (double)J->beta[r * J->Hv + j];

        /* decay */
        for (int e = 0; e < K * V; ++e) H[e] *= a;
        /* p = H^T k */
        for (int c = 0; c < V; ++c) p[c] = 0.0;
        for (int d = 0; d < K; ++d) {
            const double kd = (double)kt[d];
            const double *row = H + (size_t)d * V;
            for (int c = 0; c < V; ++c) p[c] += row[c] * kd;
        }
        /* u = beta (v - p) ; H += k u^T */
        for (int c = 0; c < V; ++c) u[c] = b * ((double)vt[c] - p[c]);
        for (int d = 0; d < K; ++d) {
            const double kd = (double)kt[d];
            double *row = H + (size_t)d * V;
            for (int c = 0; c < V; ++c) row[c] += kd * u[c];
        }
        /* o = scale H^T q */
        double *ot = J->o + (r * J->Hv + j) * V;
        for (int c = 0; c < V; ++c) p[c] = 0.0;
        for (int d = 0; d < K; ++d) {
            const double qd = (double)qt[d];
            const double *row = H + (size_t)d * V;
            for (int c = 0; c < V; ++c) p[c] += row[c] * qd;
        }
        for (int c = 0; c < V; ++c) ot[c] = J->scale * p[c];
    }

    if (J->ht) {
        double *dst = J->ht + ((int64_t)n * J->Hv + j) * K * V;
        memcpy(dst, H, sizeof(double) * (size_t)K * V);
    }
}

static void *fwd_worker(void *arg)
{
    fwd_job *J = (fwd_job *)arg;
    const int units = J->N * J->Hv;
    double *H = (double *)malloc(sizeof(double) * (size_t)J->K * J->V);
    double *p = (double *)malloc(sizeof(double) * (size_t)J->V);
    double *u = (double *)malloc(sizeof(double) * (size_t)J->V);
    if (!H || !p || !u) {
        free(H); free(p); free(u);
        return (void *)1;
    }
    for (;;) {
        pthread_mutex_lock(&J->lock);
        const int w = J->next_unit++;
        pthread_mutex_unlock(&J->lock);
        if (w >= units) break;
        fwd_unit(J, w / J->Hv, w % J->Hv, H, p, u);
    }
    free(H); free(p); free(u);
    return NULL;
}

/*
 * gdn_oracle_fwd: returns 0 on success, -1 on invalid arguments, -2 on an
 * allocation or thread failure.
 *   q, k   double [B, T, Hqk, K]      v  double [B, T, Hv, V]
 *   g, beta double [B, T, Hv]         h0 double [N, Hv, K, V] or NULL
 *   cu_seqlens int32 [N+1] or NULL (then N must equal B)
 *   o  double  [B, T, Hv, V]          ht double [N, Hv, K, V] or NULL
 */
int gdn_oracle_fwd(int64_t B, int64_t T, int Hqk, int Hv, int K, int V,
                   const double *q, const double *k, const double *v,
                   const double *g, const double *beta, double scale,
                   const double *h0, const int32_t *cu_seqlens, int N,
                   double *o, double *ht, int n_threads)
{
    if (B < 0 || T < 0 || Hqk <= 0 || Hv <= 0 || K <= 0 || V <= 0 || N < 0) return -1;
    if (Hv % Hqk != 0) return -1;
    if (cu_seqlens) {
        if (B != 1 || cu_seqlens[0] != 0 || cu_seqlens[N] != T) return -1;
        for (int n = 0; n < N; ++n)
            if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    } else if (N != B) {
        return -1;
    }
    fwd_job J;
    J.B = B; J.T = T; J.Hqk = Hqk; J.Hv = Hv; J.K = K; J.V = V; J.N = N;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.h0 = h0;
    J.cu = cu_seqlens; J.scale = scale; J.o = o; J.ht = ht;
    J.next_unit = 0;
    pthread_mutex_init(&J.lock, NULL);

    if (n_threads < 1) n_threads = 1;
    if (n_threads > N * Hv) n_threads = N * Hv > 0 ? N * Hv : 1;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
    if (!th) return -2;
    int started = 0, rc = 0;
    for (int t = 0; t < n_threads; ++t) {
        if (pthread_create(&th[t], NULL, fwd_worker, &J) != 0) { rc = -2; break; }
        ++started;
    }
    for (int t = 0; t < started; ++t) {
        void *ret = NULL;
        pthread_join(th[t], &ret);
        if (ret) rc = -2;
    }
    free(th);
    pthread_mutex_destroy(&J.lock);
    return rc;
}

/*
 * gdn_oracle_chunk_cumsum: chunk-local running sum of the log-gates, the
 * transformed g that the low-level forward returns (aisparkup.com,
 * "low-level API").  Chunks of `chunk` tokens start at every sequence start;
 * the sum restarts at each chunk start.  g and out are [B, T, H] (double).
 */
int gdn_oracle_chunk_cumsum(int64_t B, int64_t T, int H, int chunk,
                            const double *g, const int32_t *cu_seqlens, int N,
                            double *out)
{
    if (B < 0 || T < 0 || H <= 0 || chunk <= 0 || N < 0) return -1;
    if (cu_seqlens) {
        if (B != 1 || cu_seqlens[0] != 0 || cu_seqlens[N] != T) return -1;
        for (int n = 0; n < N; ++n)
            if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    } else if (N != B) {
        return -1;
    }
    for (int n = 0; n < N; ++n) {
        int64_t r0 = cu_seqlens ? cu_seqlens[n] : (int64_t)n * T;
        int64_t r1 = cu_seqlens ? cu_seqlens[n + 1] : (int64_t)(n + 1) * T;
        for (int h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int64_t r = r0; r < r1; ++r) {
                if ((r - r0) % chunk == 0) acc = 0.0;
                acc += (double)g[r * H + h];
                out[r * H + h] = acc;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ backward
 *
 * Reverse-mode derivative of the same per-token loop (the chunked backward
 * that the FlashQLA pages announce -- agentlenshq.com blog, title and
 * "performance benchmarks"; aisparkup.com wiki, "key features" -- computes
 * exactly these gradients; the pages print no formula for them).  For a
 * scalar loss with upstream gradients dO = dL/do and dHT = dL/d final_state,
 * one forward token step
 *
 *     Hh = a H_prev,  r = v - Hh^T k,  u = beta r,  H = Hh + k u^T,
 *     o  = scale H^T q
 *
 * is undone in reverse order of its statements:
 *
 *     dH  += scale q dO^T            dq   = scale H dO
 *     dk   = dH u                    du   = dH^T k
 *     dbeta = du . r                 dr   = beta du
 *     dv   = dr                      dk  -= Hh dr
 *     dHh  = dH - k dr^T
 *     dg   = a <dHh, H_prev>         dH   = a dHh     (a = exp(g))
 *
 * starting from dH = dHT (or 0) after the last token; dH after the first
 * token is dL/d initial_state.  H_prev is recomputed from states stored every
 * CKPT tokens, so memory is O(len / CKPT) states per (sequence, v-head).
 * dq and dk are returned per v-head; the caller sums a group's v-heads.
 */
#define CKPT 64

typedef struct {
    fwd_job f;               /* shapes and forward inputs (o, ht unused) */
    const double *dO, *dht;  /* [B,T,Hv,V], [N,Hv,K,V] or NULL */
    double *dq, *dk;         /* per v-head: [B,T,Hv,K] */
    double *dv;              /* [B,T,Hv,V] */
    double *dg, *dbeta;      /* [B,T,Hv] */
    double *dh0;             /* [N,Hv,K,V] */
} bwd_job;

/* One forward token step on H (K x V), in place. */
static void token_step(const fwd_job *J, int64_t r, int i, int j, double *H, double *p)
{
    const int K = J->K, V = J->V;
    const double *kt = J->k + (r * J->Hqk + i) * K;
    const double *vt = J->v + (r * J->Hv + j) * V;
    const double a = exp(J->g[r * J->Hv + j]);
    const double b = J->beta[r * J->Hv + j];
    for (size_t e = 0; e < (size_t)K * V; ++e) H[e] *= a;
    for (int c = 0; c < V; ++c) p[c] = 0.0;
    for (int d = 0; d < K; ++d)
        for (int c = 0; c < V; ++c) p[c] += H[(size_t)d * V + c] * kt[d];
    for (int c = 0; c < V; ++c) p[c] = b * (vt[c] - p[c]);
    for (int d = 0; d < K; ++d)
        for (int c = 0; c < V; ++c) H[(size_t)d * V + c] += kt[d] * p[c];
}

typedef struct {
    double *ck;   /* checkpoints: states before every CKPT-th token */
    double *hs;   /* states inside one block: (CKPT + 1) x K x V */
    double *dH, *Hh, *vecs;
    size_t ck_cap;
} bwd_ws;

static int bwd_unit(const bwd_job *B, int n, int j, bwd_ws *w)
{
    const fwd_job *J = &B->f;
    const int K = J->K, V = J->V;
    const size_t KV = (size_t)K * V;
    const int i = j / (J->Hv / J->Hqk);
    int64_t r0, r1;
    seq_rows(J, n, &r0, &r1);
    const int64_t len = r1 - r0;
    const int64_t nb = (len + CKPT - 1) / CKPT;
    if ((size_t)(nb > 0 ? nb : 1) > w->ck_cap) {
        free(w->ck);
        w->ck_cap = (size_t)(nb > 0 ? nb : 1);
        w->ck = (double *)malloc(sizeof(double) * KV * w->ck_cap);
        if (!w->ck) { w->ck_cap = 0; return -2; }
    }
    double *p = w->vecs, *r = w->vecs + V, *du = w->vecs + 2 * V, *dk = w->vecs + 3 * V;

    /* forward pass, keeping a state every CKPT tokens */
    double *H = w->hs;
    if (J->h0) {
        const double *s = J->h0 + ((int64_t)n * J->Hv + j) * KV;
        for (size_t e = 0; e < KV; ++e) H[e] = s[e];
    } else {
        memset(H, 0, sizeof(double) * KV);
    }
    for (int64_t t = 0; t < len; ++t) {
        if (t % CKPT == 0) memcpy(w->ck + (size_t)(t / CKPT) * KV, H, sizeof(double) * KV);
        token_step(J, r0 + t, i, j, H, p);
    }

    double *dH = w->dH;
    if (B->dht) {
        const double *s = B->dht + ((int64_t)n * J->Hv + j) * KV;
        for (size_t e = 0; e < KV; ++e) dH[e] = s[e];
    } else {
        memset(dH, 0, sizeof(double) * KV);
    }

    for (int64_t blk = nb - 1; blk >= 0; --blk) {
        const int64_t t0 = blk * CKPT;
        const int64_t t1 = (t0 + CKPT < len) ? t0 + CKPT : len;
        /* states before each token of the block: hs[m] = state before token t0 + m */
        memcpy(w->hs, w->ck + (size_t)blk * KV, sizeof(double) * KV);
        for (int64_t t = t0; t < t1; ++t) {
            double *dst = w->hs + (size_t)(t - t0 + 1) * KV;
            memcpy(dst, w->hs + (size_t)(t - t0) * KV, sizeof(double) * KV);
            token_step(J, r0 + t, i, j, dst, p);
        }
        for (int64_t t = t1 - 1; t >= t0; --t) {
            const int64_t row = r0 + t;
            const double *Hp = w->hs + (size_t)(t - t0) * KV;     /* H_prev */
            const double *Ht = w->hs + (size_t)(t - t0 + 1) * KV; /* H after the token */
            const double *kt = J->k + (row * J->Hqk + i) * K;
            const double *qt = J->q + (row * J->Hqk + i) * K;
            const double *vt = J->v + (row * J->Hv + j) * V;
            const double *dot = B->dO + (row * J->Hv + j) * V;
            const double a = exp(J->g[row * J->Hv + j]);
            const double b = J->beta[row * J->Hv + j];
            double *Hh = w->Hh;
            for (size_t e = 0; e < KV; ++e) Hh[e] = a * Hp[e];
            /* r = v - Hh^T k ; u = beta r (kept in p) */
            for (int c = 0; c < V; ++c) r[c] = 0.0;
            for (int d = 0; d < K; ++d)
                for (int c = 0; c < V; ++c) r[c] += Hh[(size_t)d * V + c] * kt[d];
            for (int c = 0; c < V; ++c) { r[c] = vt[c] - r[c]; p[c] = b * r[c]; }

            /* o = scale H^T q */
            double *dqt = B->dq + (row * J->Hv + j) * K;
            for (int d = 0; d < K; ++d) {
                double acc = 0.0;
                for (int c = 0; c < V; ++c) acc += Ht[(size_t)d * V + c] * dot[c];
                dqt[d] = J->scale * acc;
            }
            for (int d = 0; d < K; ++d)
                for (int c = 0; c < V; ++c) dH[(size_t)d * V + c] += J->scale * qt[d] * dot[c];

            /* H = Hh + k u^T */
            for (int d = 0; d < K; ++d) {
                double acc = 0.0;
                for (int c = 0; c < V; ++c) acc += dH[(size_t)d * V + c] * p[c];
                dk[d] = acc;
            }
            for (int c = 0; c < V; ++c) du[c] = 0.0;
            for (int d = 0; d < K; ++d)
                for (int c = 0; c < V; ++c) du[c] += dH[(size_t)d * V + c] * kt[d];

            /* u = beta r */
            double db = 0.0;
            for (int c = 0; c < V; ++c) db += du[c] * r[c];
            B->dbeta[row * J->Hv + j] = db;
            /* dr = beta du, reusing du */
            for (int c = 0; c < V; ++c) du[c] *= b;

            /* r = v - Hh^T k */
            double *dvt = B->dv + (row * J->Hv + j) * V;
            for (int c = 0; c < V; ++c) dvt[c] = du[c];
            for (int d = 0; d < K; ++d) {
                double acc = 0.0;
                for (int c = 0; c < V; ++c) acc += Hh[(size_t)d * V + c] * du[c];
                dk[d] -= acc;
            }
            double *dkt = B->dk + (row * J->Hv + j) * K;
            for (int d = 0; d < K; ++d) dkt[d] = dk[d];
            /* dHh = dH - k dr^T (in place in dH) */
            for (int d = 0; d < K; ++d)
                for (int c = 0; c < V; ++c) dH[(size_t)d * V + c] -= kt[d] * du[c];

            /* Hh = a H_prev */
            double da = 0.0;
            for (size_t e = 0; e < KV; ++e) da += dH[e] * Hp[e];
            B->dg[row * J->Hv + j] = a * da;
            for (size_t e = 0; e < KV; ++e) dH[e] *= a;
        }
    }
    memcpy(B->dh0 + ((int64_t)n * J->Hv + j) * KV, dH, sizeof(double) * KV);
    return 0;
}

static void *bwd_worker(void *arg)
{
    bwd_job *B = (bwd_job *)arg;
    fwd_job *J = &B->f;
    const int units = J->N * J->Hv;
    const size_t KV = (size_t)J->K * J->V;
    bwd_ws w;
    w.ck = NULL;
    w.ck_cap = 0;
    w.hs = (double *)malloc(sizeof(double) * KV * (CKPT + 1));
    w.dH = (double *)malloc(sizeof(double) * KV);
    w.Hh = (double *)malloc(sizeof(double) * KV);
    w.vecs = (double *)malloc(sizeof(double) * (size_t)(3 * J->V + J->K));
    void *ret = NULL;
    if (!w.hs || !w.dH || !w.Hh || !w.vecs) {
        ret = (void *)1;
    } else {
        for (;;) {
            pthread_mutex_lock(&J->lock);
            const int u = J->next_unit++;
            pthread_mutex_unlock(&J->lock);
            if (u >= units) break;
            if (bwd_unit(B, u / J->Hv, u % J->Hv, &w) != 0) { ret = (void *)1; break; }
        }
    }
    free(w.ck); free(w.hs); free(w.dH); free(w.Hh); free(w.vecs);
    return ret;
}

/*
 * gdn_oracle_bwd: gradients of L = <dO, o> + <dht, final_state> with respect
 * to every input of gdn_oracle_fwd.  Same shapes and conventions as the
 * forward; dht may be NULL (no gradient flows into the final state).
 * Outputs (double): dq, dk per v-head [B, T, Hv, K]; dv [B, T, Hv, V];
 * dg, dbeta [B, T, Hv]; dh0 [N, Hv, K, V] (written even when h0 is NULL:
 * the gradient with respect to a zero initial state).
 * Returns 0, -1 on invalid arguments, -2 on an allocation or thread failure.
 */
int gdn_oracle_bwd(int64_t Bsz, int64_t T, int Hqk, int Hv, int K, int V,
                   const double *q, const double *k, const double *v,
                   const double *g, const double *beta, double scale,
                   const double *h0, const int32_t *cu_seqlens, int N,
                   const double *dO, const double *dht,
                   double *dq, double *dk, double *dv, double *dg, double *dbeta, double *dh0,
                   int n_threads)
{
    if (Bsz < 0 || T < 0 || Hqk <= 0 || Hv <= 0 || K <= 0 || V <= 0 || N < 0) return -1;
    if (Hv % Hqk != 0 || !dO || !dq || !dk || !dv || !dg || !dbeta || !dh0) return -1;
    if (cu_seqlens) {
        if (Bsz != 1 || cu_seqlens[0] != 0 || cu_seqlens[N] != T) return -1;
        for (int n = 0; n < N; ++n)
            if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    } else if (N != Bsz) {
        return -1;
    }
    bwd_job B;
    fwd_job *J = &B.f;
    J->B = Bsz; J->T = T; J->Hqk = Hqk; J->Hv = Hv; J->K = K; J->V = V; J->N = N;
    J->q = q; J->k = k; J->v = v; J->g = g; J->beta = beta; J->h0 = h0;
    J->cu = cu_seqlens; J->scale = scale; J->o = NULL; J->ht = NULL;
    J->next_unit = 0;
    B.dO = dO; B.dht = dht; B.dq = dq; B.dk = dk; B.dv = dv; B.dg = dg; B.dbeta = dbeta; B.dh0 = dh0;
    pthread_mutex_init(&J->lock, NULL);

    if (n_threads < 1) n_threads = 1;
    if (n_threads > N * Hv) n_threads = N * Hv > 0 ? N * Hv : 1;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
    if (!th) return -2;
    int started = 0, rc = 0;
    for (int t = 0; t < n_threads; ++t) {
        if (pthread_create(&th[t], NULL, bwd_worker, &B) != 0) { rc = -2; break; }
        ++started;
    }
    for (int t = 0; t < started; ++t) {
        void *ret = NULL;
        pthread_join(th[t], &ret);
        if (ret) rc = -2;
    }
    free(th);
    pthread_mutex_destroy(&J->lock);
    return rc;
}

/*
 * Gated DeltaNet forward: plain fp64 CPU oracle.
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
 * Inputs are passed as float32 arrays holding the exact input values (bf16
 * values are exactly representable in float32); all arithmetic is double.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t B, T;
    int Hqk, Hv, K, V, N;
    const float *q, *k, *v, *g, *beta, *h0;
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
        const float *s = J->h0 + ((int64_t)n * J->Hv + j) * K * V;
        for (int e = 0; e < K * V; ++e) H[e] = (double)s[e];
    } else {
        memset(H, 0, sizeof(double) * (size_t)K * V);
    }

    for (int64_t r = r0; r < r1; ++r) {
        const float *kt = J->k + (r * J->Hqk + i) * K;
        const float *qt = J->q + (r * J->Hqk + i) * K;
        const float *vt = J->v + (r * J->Hv + j) * V;
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
 *   q, k   float32 [B, T, Hqk, K]     v  float32 [B, T, Hv, V]
 *   g, beta float32 [B, T, Hv]        h0 float32 [N, Hv, K, V] or NULL
 *   cu_seqlens int32 [N+1] or NULL (then N must equal B)
 *   o  double  [B, T, Hv, V]          ht double [N, Hv, K, V] or NULL
 */
int gdn_oracle_fwd(int64_t B, int64_t T, int Hqk, int Hv, int K, int V,
                   const float *q, const float *k, const float *v,
                   const float *g, const float *beta, double scale,
                   const float *h0, const int32_t *cu_seqlens, int N,
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
 * the sum restarts at each chunk start.  g and out are [B, T, H] (float32
 * in, double out).
 */
int gdn_oracle_chunk_cumsum(int64_t B, int64_t T, int H, int chunk,
                            const float *g, const int32_t *cu_seqlens, int N,
                            double *out)
{
    if (B < 0 || T < 0 || H <= 0 || chunk <= 0 || N < 0) return -1;
    if (!cu_seqlens && N != B) return -1;
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

/*
 * Drives the fp64 oracle (oracle/gdn_oracle.c, built by the host compiler
 * with AddressSanitizer and UndefinedBehaviorSanitizer) over seeded random
 * small problems: dense batches with B > 1, packed sequences with empty and
 * one-token members, grouped heads, with and without initial and final
 * states, one and several threads.  Every buffer is allocated at exactly its
 * documented size, so a read or write past any of them is reported by the
 * sanitizer.  The driver also asserts that every output is finite, that the
 * thread count does not change a single bit of the results, and that invalid
 * arguments are refused.  Exit status 0 means every check held.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int gdn_oracle_fwd(int64_t B, int64_t T, int Hqk, int Hv, int K, int V,
                   const double *q, const double *k, const double *v,
                   const double *g, const double *beta, double scale,
                   const double *h0, const int32_t *cu_seqlens, int N,
                   double *o, double *ht, int n_threads);
int gdn_oracle_bwd(int64_t Bsz, int64_t T, int Hqk, int Hv, int K, int V,
                   const double *q, const double *k, const double *v,
                   const double *g, const double *beta, double scale,
                   const double *h0, const int32_t *cu_seqlens, int N,
                   const double *dO, const double *dht,
                   double *dq, double *dk, double *dv, double *dg, double *dbeta, double *dh0,
                   int n_threads);
int gdn_oracle_chunk_cumsum(int64_t B, int64_t T, int H, int chunk,
                            const double *g, const int32_t *cu_seqlens, int N,
                            double *out);

static int g_failures = 0;
#define CHECK(x) do { if (!(x)) { fprintf(stderr, "check failed (line %d): %s\n", __LINE__, #x); ++g_failures; } } while (0)

/* splitmix64: a small seeded generator, enough for test inputs */
static uint64_t g_state = 20261202u;
static uint64_t next_u64(void)
{
    uint64_t z = (g_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}
static double unif(void) { return (double)(next_u64() >> 11) * (1.0 / 9007199254740992.0); }
static int uni(int lo, int hi) { return lo + (int)(next_u64() % (uint64_t)(hi - lo + 1)); }

static double *rand_buf(size_t n, double lo, double hi)
{
    double *p = (double *)malloc(n ? n * sizeof(double) : 1);
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * unif();
    return p;
}
static double *nan_buf(size_t n)
{
    double *p = (double *)malloc(n ? n * sizeof(double) : 1);
    for (size_t i = 0; i < n; ++i) p[i] = NAN;
    return p;
}
static int all_finite(const double *p, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(p[i])) return 0;
    return 1;
}
static int same_bits(const double *a, const double *b, size_t n) { return n == 0 || memcmp(a, b, n * sizeof(double)) == 0; }

static void one_case(int it)
{
    const int Hqk = uni(1, 3), grp = uni(1, 3), Hv = Hqk * grp;
    const int K = uni(1, 9), V = uni(1, 9);
    int64_t B, T;
    int N;
    int32_t *cu = NULL;
    if (uni(0, 1)) {
        N = uni(0, 6);
        cu = (int32_t *)malloc(sizeof(int32_t) * (size_t)(N + 1));
        cu[0] = 0;
        for (int n = 0; n < N; ++n) cu[n + 1] = cu[n] + (uni(0, 3) == 0 ? uni(0, 1) : uni(2, 150));
        B = 1;
        T = cu[N];
    } else {
        B = uni(0, 3);
        T = uni(0, 150);
        N = (int)B;
    }
    const size_t rows = (size_t)(B * T);
    const size_t nst = (size_t)N * Hv * K * V;
    double *q = rand_buf(rows * Hqk * K, -1, 1), *k = rand_buf(rows * Hqk * K, -0.5, 0.5);
    double *v = rand_buf(rows * Hv * V, -1, 1), *g = rand_buf(rows * Hv, -0.3, 0.0);
    double *beta = rand_buf(rows * Hv, 0.0, 1.0);
    const int use_h0 = uni(0, 1), use_ht = uni(0, 1), use_dht = uni(0, 1);
    double *h0 = use_h0 ? rand_buf(nst, -0.1, 0.1) : NULL;
    const double scale = 1.0 / sqrt((double)K);
    const int threads = uni(2, 4);

    /* forward, one thread and several */
    double *o1 = nan_buf(rows * Hv * V), *o2 = nan_buf(rows * Hv * V);
    double *ht1 = use_ht ? nan_buf(nst) : NULL, *ht2 = use_ht ? nan_buf(nst) : NULL;
    CHECK(gdn_oracle_fwd(B, T, Hqk, Hv, K, V, q, k, v, g, beta, scale, h0, cu, N, o1, ht1, 1) == 0);
    CHECK(gdn_oracle_fwd(B, T, Hqk, Hv, K, V, q, k, v, g, beta, scale, h0, cu, N, o2, ht2, threads) == 0);
    CHECK(all_finite(o1, rows * Hv * V));
    CHECK(same_bits(o1, o2, rows * Hv * V));
    if (use_ht) {
        CHECK(all_finite(ht1, nst));
        CHECK(same_bits(ht1, ht2, nst));
    }

    /* backward, one thread and several */
    double *dO = rand_buf(rows * Hv * V, -1, 1);
    double *dht = use_dht ? rand_buf(nst, -0.1, 0.1) : NULL;
    double *dq[2], *dk[2], *dv[2], *dg[2], *db[2], *dh0[2];
    for (int r = 0; r < 2; ++r) {
        dq[r] = nan_buf(rows * Hv * K); dk[r] = nan_buf(rows * Hv * K); dv[r] = nan_buf(rows * Hv * V);
        dg[r] = nan_buf(rows * Hv); db[r] = nan_buf(rows * Hv); dh0[r] = nan_buf(nst);
        CHECK(gdn_oracle_bwd(B, T, Hqk, Hv, K, V, q, k, v, g, beta, scale, h0, cu, N, dO, dht,
                             dq[r], dk[r], dv[r], dg[r], db[r], dh0[r], r == 0 ? 1 : threads) == 0);
    }
    CHECK(all_finite(dq[0], rows * Hv * K) && all_finite(dk[0], rows * Hv * K) && all_finite(dv[0], rows * Hv * V));
    CHECK(all_finite(dg[0], rows * Hv) && all_finite(db[0], rows * Hv) && all_finite(dh0[0], nst));
    CHECK(same_bits(dq[0], dq[1], rows * Hv * K) && same_bits(dk[0], dk[1], rows * Hv * K));
    CHECK(same_bits(dv[0], dv[1], rows * Hv * V) && same_bits(dg[0], dg[1], rows * Hv));
    CHECK(same_bits(db[0], db[1], rows * Hv) && same_bits(dh0[0], dh0[1], nst));

    /* chunk-local cumulative sum of the gates */
    double *cs = nan_buf(rows * Hv);
    const int chunk = uni(1, 70);
    CHECK(gdn_oracle_chunk_cumsum(B, T, Hv, chunk, g, cu, N, cs) == 0);
    CHECK(all_finite(cs, rows * Hv));

    /* invalid arguments are refused */
    if (Hqk > 1)  /* H_v not a multiple of H_qk */
        CHECK(gdn_oracle_fwd(B, T, Hqk, Hv + 1, K, V, q, k, v, g, beta, scale, NULL, cu, N, o1, NULL, 1) == -1);
    if (cu && N > 0) {
        cu[N] += 1;
        CHECK(gdn_oracle_fwd(B, T, Hqk, Hv, K, V, q, k, v, g, beta, scale, h0, cu, N, o1, ht1, 1) == -1);
        CHECK(gdn_oracle_bwd(B, T, Hqk, Hv, K, V, q, k, v, g, beta, scale, h0, cu, N, dO, dht,
                             dq[0], dk[0], dv[0], dg[0], db[0], dh0[0], 1) == -1);
        CHECK(gdn_oracle_chunk_cumsum(B, T, Hv, chunk, g, cu, N, cs) == -1);
        cu[N] -= 1;
    }
    if (!cu) CHECK(gdn_oracle_fwd(B, T, Hqk, Hv, K, V, q, k, v, g, beta, scale, h0, NULL, N + 1, o1, ht1, 1) == -1);

    free(q); free(k); free(v); free(g); free(beta); free(h0); free(o1); free(o2); free(ht1); free(ht2);
    free(dO); free(dht); free(cs); free(cu);
    for (int r = 0; r < 2; ++r) { free(dq[r]); free(dk[r]); free(dv[r]); free(dg[r]); free(db[r]); free(dh0[r]); }
    (void)it;
}

int main(int argc, char **argv)
{
    const int iters = argc > 1 ? atoi(argv[1]) : 300;
    for (int it = 0; it < iters; ++it) one_case(it);
    printf("oracle driver: %d cases, %d failed checks\n", iters, g_failures);
    return g_failures == 0 ? 0 : 1;
}

/*
 * Drives every entry point of the CPU oracle on edge shapes (k = 0, V = 1,
 * N = 0, P = 0, B = 0, ragged lengths past both ends, ids outside the
 * vocabulary, a tree whose path rows are partly unused) with every input and
 * output in a heap buffer of exactly its documented size, plus the argument
 * checks.  Built together with the oracle's source under
 * -fsanitize=address,undefined by tests/test_sanitizers.py, which fails on any
 * sanitizer report or a nonzero exit.  Exit 1 on an unexpected status.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* The oracle's entry points (it has no header). */
int oracle_verify_stochastic(const void *, const void *, int, const int32_t *, const float *,
                             double, int, int, int, int32_t *, int32_t *, double *, double *,
                             double *);
int oracle_verify_stochastic_filtered(const void *, const void *, int, const int32_t *,
                                      const float *, double, int, double, double, int, int, int,
                                      int32_t *, int32_t *, double *, double *, double *,
                                      double *);
int oracle_verify_stochastic_ragged(const void *, const void *, int, const int32_t *,
                                    const int32_t *, const float *, double, int, int, int,
                                    int32_t *, int32_t *, double *, double *, double *);
void oracle_philox_uniforms(uint64_t, uint64_t, int, int, float *);
int oracle_verify_greedy(const void *, int, const int32_t *, int, int, int, int32_t *,
                         int32_t *, int32_t *);
int oracle_verify_greedy_ragged(const void *, int, const int32_t *, const int32_t *, int, int,
                                int, int32_t *, int32_t *, int32_t *);
int oracle_verify_tree(const void *, int, const int32_t *, const int32_t *, int, int, int, int,
                       int, int32_t *, int32_t *, int32_t *, int32_t *);
int oracle_verify_tree_stochastic(const void *, const void *, int, const int32_t *,
                                  const int32_t *, const float *, double, int, int, int, int,
                                  int, int32_t *, int32_t *, int32_t *, double *);

enum { F32 = 0, BF16 = 1, OK = 0, BAD = 1 };

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static uint32_t next_u32(void) {
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (uint32_t)(rng >> 11);
}
static float uniform01(void) { return (float)(next_u32() >> 8) / 16777216.0f; }

/* A heap block of exactly n elements of size sz (malloc(0) when n == 0, so
 * any access to an empty array is reported). */
static void *block(size_t n, size_t sz) {
    void *p = malloc(n * sz);
    if (!p && n) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static void *logits(int dtype, size_t n) {
    if (dtype == F32) {
        float *p = block(n, 4);
        for (size_t i = 0; i < n; ++i) p[i] = 6.0f * uniform01() - 3.0f;
        return p;
    }
    uint16_t *p = block(n, 2);
    for (size_t i = 0; i < n; ++i) {
        const float f = 6.0f * uniform01() - 3.0f;
        uint32_t bits;
        memcpy(&bits, &f, 4);
        p[i] = (uint16_t)(bits >> 16);
    }
    return p;
}

/* ids in [-1, V]: mostly in range, a few outside on either side. */
static int32_t *ids(size_t n, int V) {
    int32_t *p = block(n, 4);
    for (size_t i = 0; i < n; ++i) {
        const uint32_t r = next_u32() % 16;
        p[i] = r == 0 ? -1 : r == 1 ? V : (int32_t)(next_u32() % (uint32_t)V);
    }
    return p;
}

static float *uniforms(size_t n) {
    float *p = block(n, 4);
    for (size_t i = 0; i < n; ++i) p[i] = uniform01();
    return p;
}

static void expect(int rc, int want, const char *what, int a, int b, int c) {
    if (rc != want) {
        fprintf(stderr, "%s(%d, %d, %d): status %d, expected %d\n", what, a, b, c, rc, want);
        exit(1);
    }
}

static void linear(int dtype, int B, int k, int V) {
    void *t = logits(dtype, (size_t)B * (k + 1) * V);
    void *d = logits(dtype, (size_t)B * k * V);
    int32_t *x = ids((size_t)B * k, V);
    float *u = uniforms((size_t)B * (k + 1));
    int32_t *lens = block((size_t)B, 4);
    for (int b = 0; b < B; ++b) lens[b] = (int32_t)(next_u32() % (uint32_t)(k + 3)) - 1;
    int32_t *out = block((size_t)B * (k + 1), 4), *acc = block((size_t)B, 4);
    int32_t *amax = block((size_t)B * (k + 1), 4);
    double *P = block((size_t)B * k, 8), *Q = block((size_t)B * k, 8);
    double *mg = block((size_t)B * (k + 1), 8), *fm = block((size_t)B, 8);

    expect(oracle_verify_stochastic(t, d, dtype, x, u, 0.8, B, k, V, out, acc, P, Q, mg), OK,
           "stochastic", B, k, V);
    expect(oracle_verify_stochastic(t, d, dtype, x, u, 1.0, B, k, V, out, acc, NULL, NULL, NULL),
           OK, "stochastic without optional outputs", B, k, V);
    const struct { int top_k; double top_p, min_p; } filters[] = {
        {0, 1.0, 0.0}, {1, 1.0, 0.0}, {3, 0.5, 0.0}, {0, 0.9, 0.1}, {V + 5, 1.0, 1.0}};
    for (size_t f = 0; f < sizeof filters / sizeof filters[0]; ++f)
        expect(oracle_verify_stochastic_filtered(t, d, dtype, x, u, 0.7, filters[f].top_k,
                                                 filters[f].top_p, filters[f].min_p, B, k, V, out,
                                                 acc, P, Q, mg, fm),
               OK, "filtered", B, k, V);
    expect(oracle_verify_stochastic_ragged(t, d, dtype, x, lens, u, 1.3, B, k, V, out, acc, P, Q,
                                           mg),
           OK, "ragged", B, k, V);
    expect(oracle_verify_greedy(t, dtype, x, B, k, V, out, acc, amax), OK, "greedy", B, k, V);
    expect(oracle_verify_greedy(t, dtype, x, B, k, V, out, acc, NULL), OK, "greedy", B, k, V);
    expect(oracle_verify_greedy_ragged(t, dtype, x, lens, B, k, V, out, acc, amax), OK,
           "greedy ragged", B, k, V);

    /* argument checks */
    expect(oracle_verify_stochastic(t, d, dtype, x, u, 0.0, B, k, V, out, acc, P, Q, mg), BAD,
           "stochastic T = 0", B, k, V);
    expect(oracle_verify_stochastic(t, d, 7, x, u, 1.0, B, k, V, out, acc, P, Q, mg), BAD,
           "stochastic dtype 7", B, k, V);
    expect(oracle_verify_stochastic_filtered(t, d, dtype, x, u, 1.0, 0, 1.5, 0.0, B, k, V, out,
                                             acc, P, Q, mg, fm),
           BAD, "filtered top_p 1.5", B, k, V);
    expect(oracle_verify_stochastic_filtered(t, d, dtype, x, u, 1.0, -1, 1.0, 0.0, B, k, V, out,
                                             acc, P, Q, mg, fm),
           BAD, "filtered top_k -1", B, k, V);

    free(t); free(d); free(x); free(u); free(lens); free(out); free(acc); free(amax);
    free(P); free(Q); free(mg); free(fm);
}

/* A random tree over nodes 0..N (parent[n] < n) and P path rows of length L:
 * row r lists the root-first chain to a random node, truncated to L entries
 * and padded with -1; every third row is unused (first entry -1 or N + 1). */
static void tree(int dtype, int B, int N, int P, int L, int V) {
    void *t = logits(dtype, (size_t)B * (N + 1) * V);
    void *d = logits(dtype, (size_t)B * (N + 1) * V);
    int32_t *nt = ids((size_t)B * (N + 1), V);
    int32_t *paths = block((size_t)B * P * L, 4);
    int32_t *parent = block((size_t)N + 1, 4), *chain = block((size_t)N + 1, 4);
    for (int b = 0; b < B; ++b) {
        for (int n = 1; n <= N; ++n) parent[n] = (int32_t)(next_u32() % (uint32_t)n);
        for (int r = 0; r < P; ++r) {
            int32_t *row = paths + ((size_t)b * P + r) * L;
            for (int j = 0; j < L; ++j) row[j] = -1;
            if (r % 3 == 2) {
                row[0] = (r % 2) ? -1 : N + 1;
                continue;
            }
            int len = 0;
            for (int n = (int)(next_u32() % (uint32_t)(N + 1)); ; n = parent[n]) {
                chain[len++] = n;
                if (n == 0) break;
            }
            for (int j = 0; j < L && j < len; ++j) row[j] = chain[len - 1 - j];
        }
    }
    float *u = uniforms((size_t)B * (N + 1));
    int32_t *out = block((size_t)B * L, 4), *acc = block((size_t)B, 4);
    int32_t *best = block((size_t)B, 4), *nodes = block((size_t)B * L, 4);
    double *mg = block((size_t)B * (N + 1), 8);

    expect(oracle_verify_tree(t, dtype, nt, paths, B, N, P, L, V, out, acc, best, nodes), OK,
           "tree", B, N, P);
    expect(oracle_verify_tree(t, dtype, nt, paths, B, N, P, L, V, out, acc, NULL, NULL), OK,
           "tree without optional outputs", B, N, P);
    expect(oracle_verify_tree_stochastic(t, d, dtype, nt, paths, u, 0.9, B, N, P, L, V, out, acc,
                                         nodes, mg),
           OK, "tree stochastic", B, N, P);
    expect(oracle_verify_tree_stochastic(t, d, dtype, nt, paths, u, 1.0, B, N, P, L, V, out, acc,
                                         NULL, NULL),
           OK, "tree stochastic without optional outputs", B, N, P);
    expect(oracle_verify_tree(t, dtype, nt, paths, B, N, P, 0, V, out, acc, best, nodes), BAD,
           "tree L = 0", B, N, P);
    expect(oracle_verify_tree_stochastic(t, d, dtype, nt, paths, u, -1.0, B, N, P, L, V, out,
                                         acc, nodes, mg),
           BAD, "tree stochastic T = -1", B, N, P);

    free(t); free(d); free(nt); free(paths); free(parent); free(chain); free(u); free(out);
    free(acc); free(best); free(nodes); free(mg);
}

int main(void) {
    static const int lin[][3] = {{1, 0, 1}, {3, 0, 5},  {1, 1, 1},   {2, 1, 2},
                                 {3, 2, 7}, {2, 4, 33}, {0, 3, 5},   {4, 5, 64},
                                 {1, 8, 3}, {2, 3, 257}, {5, 64, 2}, {1, 2, 1000}};
    for (int dtype = 0; dtype < 2; ++dtype)
        for (size_t i = 0; i < sizeof lin / sizeof lin[0]; ++i)
            linear(dtype, lin[i][0], lin[i][1], lin[i][2]);

    static const int tr[][5] = {{1, 0, 0, 1, 1}, {2, 0, 1, 1, 4}, {2, 3, 0, 2, 4},
                                {2, 5, 3, 4, 9}, {1, 6, 2, 1, 3}, {3, 9, 6, 3, 17},
                                {0, 4, 2, 3, 5}, {2, 12, 7, 13, 40}, {1, 1, 1, 2, 1}};
    for (int dtype = 0; dtype < 2; ++dtype)
        for (size_t i = 0; i < sizeof tr / sizeof tr[0]; ++i)
            tree(dtype, tr[i][0], tr[i][1], tr[i][2], tr[i][3], tr[i][4]);

    static const int ph[][2] = {{0, 0}, {1, 1}, {3, 5}, {2, 65}};
    for (size_t i = 0; i < sizeof ph / sizeof ph[0]; ++i) {
        float *u = block((size_t)ph[i][0] * ph[i][1], 4);
        oracle_philox_uniforms(12345u, 7u * i, ph[i][0], ph[i][1], u);
        for (size_t j = 0; j < (size_t)ph[i][0] * ph[i][1]; ++j)
            if (!(u[j] >= 0.0f && u[j] < 1.0f)) {
                fprintf(stderr, "philox uniform %g out of [0, 1)\n", u[j]);
                return 1;
            }
        free(u);
    }
    printf("oracle edge shapes: ok\n");
    return 0;
}

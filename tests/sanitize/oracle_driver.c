/* Drives the C part of the oracle under AddressSanitizer and UndefinedBehaviorSanitizer:
 * every grid, the four quantize kinds on values that include ties, signed zeros, values
 * past the grid's range and binary32 subnormals, and the exact-sum search on tensors with
 * tiny and huge elements (the extreme exponent buckets).  Checks only properties that hold
 * by construction (codes in range, the sign bit, the bucket sum of one element).  Exits
 * non-zero on a failed check; the sanitizers abort on any memory error or undefined
 * behaviour. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_minifloat_value(int e, int m, int b, int code);
void orc_minifloat_grid(int e, int m, int b, double* out);
void orc_quantize(const float* x, const float* r, int64_t n, int grid_kind, const double* grid, int ng,
                  uint8_t* codes);
void orc_candidate_sse(const float* w, int64_t n, const double* g, int ng, float c, uint64_t* out);
void orc_search_sse(const float* w, int64_t n, const double* grids, int nf, int ng, const float* clips, int nc,
                    uint64_t* out);
int orc_exp_min(void);
int orc_nbucket(void);

static int fail = 0;
#define CHECK(c) do { if (!(c)) { printf("FAIL line %d: %s\n", __LINE__, #c); fail = 1; } } while (0)

int main(void) {
    const int fmts[][3] = {{1, 2, 1}, {2, 1, 1}, {3, 0, 1}, {2, 3, 1}, {3, 2, 3}, {4, 3, 7}, {5, 2, 15}};
    double grid[256];
    enum { N = 4096 };
    float* x = malloc(N * sizeof(float));
    float* r = malloc(N * sizeof(float));
    uint8_t* codes = malloc(N);
    uint32_t s = 12345u;
    for (int i = 0; i < N; i++) {
        s = s * 1664525u + 1013904223u;
        float v = ldexpf((float)(s >> 8) / 16777216.0f, (int)(s % 40) - 30);
        if (s & 1u) v = -v;
        if (i % 97 == 0) v = 0.0f;
        if (i % 89 == 0) v = -0.0f;
        if (i % 83 == 0) v = 1e-40f;   /* binary32 subnormal */
        if (i % 79 == 0) v = 3.0e38f;  /* past every grid's range */
        x[i] = v;
        r[i] = (i % 13 == 0) ? 0.0f : ldexpf(1.0f, (int)(i % 7) - 3);
    }
    for (int f = 0; f < 7; f++) {
        const int e = fmts[f][0], m = fmts[f][1], b = fmts[f][2], ng = 1 << (e + m);
        orc_minifloat_grid(e, m, b, grid);
        for (int c = 1; c < ng; c++) CHECK(grid[c] > grid[c - 1]);
        const int kind = e + m == 3 ? 0 : e + m == 7 ? 2 : 3;
        const int sbit = kind == 0 ? 3 : kind == 2 ? 7 : 5;
        orc_quantize(x, r, N, kind, grid, ng, codes);
        for (int i = 0; i < N; i++) {
            CHECK((codes[i] & ((1 << sbit) - 1)) < ng);
            CHECK(((codes[i] >> sbit) & 1) == (signbit(x[i]) ? 1 : 0));
            CHECK(codes[i] >> (sbit + 1) == 0);
        }
        /* ties: every midpoint between neighbours, and its neighbours */
        for (int c = 0; c + 1 < ng; c++) {
            float t[3], one[3] = {1.0f, 1.0f, 1.0f};
            uint8_t q[3];
            t[1] = (float)((grid[c] + grid[c + 1]) / 2);
            t[0] = nextafterf(t[1], 0.0f);
            t[2] = nextafterf(t[1], 1e30f);
            orc_quantize(t, one, 3, kind, grid, ng, q);
            CHECK(q[0] <= q[1] && q[1] <= q[2]);
        }
    }
    /* the 16-entry signed lookup grid (kind 1) */
    double lut[16];
    for (int i = 0; i < 16; i++) lut[i] = (i - 7.5) / 8.0;
    orc_quantize(x, r, N, 1, lut, 16, codes);
    for (int i = 0; i < N; i++) CHECK(codes[i] < 16);

    /* exact-sum search: tiny and huge elements reach the extreme buckets */
    const int nb = orc_nbucket();
    float w[6] = {1e-45f, -1e-45f, 3.0e38f, -2.5f, 0.0f, 1.0f};
    float clips[2] = {1.0f, 3.0e38f};
    double g3[3 * 8];
    orc_minifloat_grid(1, 2, 1, g3);
    orc_minifloat_grid(2, 1, 1, g3 + 8);
    orc_minifloat_grid(3, 0, 1, g3 + 16);
    uint64_t* out = calloc((size_t)3 * 2 * nb * 2, sizeof(uint64_t));
    orc_search_sse(w, 6, g3, 3, 8, clips, 2, out);
    /* one element: the buckets hold exactly its squared error's significand */
    uint64_t* one = calloc((size_t)nb * 2, sizeof(uint64_t));
    float w1 = 0.75f;
    orc_candidate_sse(&w1, 1, g3 + 8, 8, 6.0f, one);
    int nonzero = 0;
    for (int j = 0; j < nb; j++) nonzero += (one[2 * j] | one[2 * j + 1]) != 0;
    CHECK(nonzero <= 1);
    CHECK(orc_exp_min() < -1074);
    free(one);
    free(out);
    free(codes);
    free(r);
    free(x);
    printf("oracle: %s\n", fail ? "FAILURES" : "all checks passed");
    return fail;
}

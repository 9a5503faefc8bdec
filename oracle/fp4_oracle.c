/*
 * CPU oracle for low-bit floating-point quantization -- TEST INFRASTRUCTURE ONLY.
 *
 * Only tests, the smoke check and the benchmark's CPU-baseline leg may load this
 * library.  It shares no code, header, table or helper with the HIP library; it is
 * plain C, built with -O2 -ffp-contract=off (no fused multiply-add, no fast-math),
 * so every float expression below is rounded exactly as written (IEEE binary32 /
 * binary64, round-to-nearest-even, subnormals kept).
 *
 * Sources (web pages, cited by title and section):
 *  [FP4-LLM] "首个支持4-bit浮点量化的LLM来了" (811yy.cn), a summary of the LLM-FP4
 *            paper: floating-point value formula with sign s, exponent field p in
 *            [0, 2^e-1], mantissa bits d_i and bias b; "scale and clip" eqs. (2)-(3);
 *            bias from the range, eq. (4); "compare and quantize", eq. (5); the
 *            format/range search; the pre-shifted exponent bias.
 *  [NF4]     "量化技术详解" (aidocs.cortexgrid.cn), section NF4: 4-bit grid at the
 *            quantiles of the normal distribution.
 * The formulas on [FP4-LLM] did not survive text extraction; the readings used here
 * (IEEE-style minifloat with subnormals and no reserved inf/NaN codes, nearest grid
 * point with exact ties to the even code) are forced by the E2M1 magnitude set
 * {0, 0.5, 1, 1.5, 2, 3, 4, 6} and are listed with the others in the design notes.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

/* Magnitude of minifloat code c = p<<m | d for exponent bits e, mantissa bits m,
 * integer bias b [FP4-LLM, FP value formula]:
 *   p == 0 : 2^(1-b) * d / 2^m            (subnormal)
 *   p >= 1 : 2^(p-b) * (1 + d / 2^m)      (normal; the top exponent is an ordinary
 *                                           binade, nothing is reserved)            */
double orc_minifloat_value(int e, int m, int b, int code) {
    int p = code >> m;
    int d = code & ((1 << m) - 1);
    (void)e;
    if (p == 0) return ldexp((double)d, 1 - b - m);
    return ldexp((double)((1 << m) + d), p - b - m);
}

/* Enumerate every magnitude of the (e,m,b) grid: out[c] for c = 0 .. 2^(e+m)-1. */
void orc_minifloat_grid(int e, int m, int b, double* out) {
    for (int c = 0; c < (1 << (e + m)); c++) out[c] = orc_minifloat_value(e, m, b, c);
}

/* a - b = *s + *e exactly (TwoSum with -b; binary64, no FMA contraction). */
static void two_diff(double a, double b, double* s, double* e) {
    double d = a - b;
    double bb = d - a;
    *s = d;
    *e = (a - (d - bb)) + (-b - bb);
}

/* Exact sign of |v - a| - |v - b|: each difference is kept as an unevaluated sum
 * hi + lo (hi the rounded difference), and such pairs compare lexicographically.     */
static int exact_dist_cmp(double v, double a, double b) {
    double sa, ea, sb, eb;
    two_diff(v, a, &sa, &ea);
    two_diff(v, b, &sb, &eb);
    if (sa < 0 || (sa == 0 && ea < 0)) { sa = -sa; ea = -ea; }
    if (sb < 0 || (sb == 0 && eb < 0)) { sb = -sb; eb = -eb; }
    if (sa != sb) return sa < sb ? -1 : 1;
    if (ea != eb) return ea < eb ? -1 : 1;
    return 0;
}

/* Brute-force nearest grid point ("compare and quantize", [FP4-LLM] eq. (5)):
 * returns the index c in [0, n) minimising |v - grid[c]|, an exact tie going to the
 * even index.  v has already been clipped to the grid's range ("scale and clip",
 * eq. (2)).  Rounded binary64 distances decide whenever they differ (rounding is
 * monotone, so their order is the exact order); equal rounded distances are compared
 * exactly, so a false tie (e.g. a tiny |v| at the zero midpoint of a symmetric
 * lookup grid) cannot occur.                                                         */
static int nearest(double v, const double* grid, int n) {
    int best = 0;
    double bd = fabs(v - grid[0]);
    for (int c = 1; c < n; c++) {
        double dc = fabs(v - grid[c]);
        int take = 0;
        if (dc < bd) take = 1;
        else if (dc == bd) {
            int r = exact_dist_cmp(v, grid[c], grid[best]);
            take = r < 0 || (r == 0 && (c % 2 == 0) && (best % 2 != 0));
        }
        if (take) { best = c; bd = dc; }
    }
    return best;
}

/* Quantize x[i] with per-element multiplier r[i]: y = fl32(x * r) ("scale", the
 * multiplier being the reciprocal of the scale), clip to the grid's range, then
 *  grid_kind 0 (minifloat, sign-magnitude): code = signbit(x)<<3 | nearest(min(|y|,
 *      Qmax)) over the ng magnitudes, Qmax = grid[ng-1];
 *  grid_kind 1 (16-entry signed lookup grid, e.g. NF4): code = nearest(clip(y,
 *      grid[0], grid[ng-1])) over the ng sorted signed values;
 *  grid_kind 2 (8-bit minifloat, sign-magnitude): as kind 0 with the sign in bit 7;
 *  grid_kind 3 (6-bit minifloat, sign-magnitude): as kind 0 with the sign in bit 5.
 * Non-finite x is not a valid input.                                                */
void orc_quantize(const float* x, const float* r, int64_t n, int grid_kind,
                  const double* grid, int ng, uint8_t* codes) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        float y = x[i] * r[i];
        if (grid_kind == 0 || grid_kind == 2 || grid_kind == 3) {
            int s = signbit(x[i]) ? 1 : 0;
            double v = fmin(fabs((double)y), grid[ng - 1]);
            int c = nearest(v, grid, ng);
            codes[i] = (uint8_t)((s << (grid_kind == 0 ? 3 : grid_kind == 2 ? 7 : 5)) | c);
        } else {
            double v = fmax(fmin((double)y, grid[ng - 1]), grid[0]);
            codes[i] = (uint8_t)nearest(v, grid, ng);
        }
    }
}

/* --------------------------------------------------------------------------------
 * Format and clip-range search ([FP4-LLM], the search-based FP quantization: pick the
 * exponent/mantissa split and the quantization range that minimise the quantization
 * error of a tensor).
 *
 * For one tensor w[0..n), its amax, and one candidate (grid magnitudes g[0..ng), Qmax
 * = g[ng-1], clip value c):
 *     s = fl32(c / Qmax);  r = fl32(1 / s)  (r = 0 when s == 0)
 *     code_i = nearest(min(fl32(|w_i| * r), Qmax));    deq_i = fl32(g[code_i] * s)
 *     SSE = sum_i (|w_i| - deq_i)^2         (the sign is shared, so this equals
 *                                             (w_i - dequant(q_i))^2)
 * Each difference is exact in binary64 (two binary32 values) and so is its square
 * (at most 2*26 significant bits); the sum is accumulated EXACTLY: every term
 * T * 2^E (T a 53-bit integer) is added into an integer bucket for its exponent E.
 * The caller turns the buckets into the correctly rounded binary64 value, so the
 * result does not depend on any summation order.
 * -------------------------------------------------------------------------------- */
#define ORC_EXP_MIN (-1100)
#define ORC_NBUCKET 2100

static void add_exact(double t, unsigned __int128* acc) {
    if (t == 0.0) return;
    uint64_t bits;
    memcpy(&bits, &t, 8);
    int biased = (int)((bits >> 52) & 0x7ff);
    uint64_t mant = bits & ((1ull << 52) - 1);
    int E;
    if (biased == 0) { E = -1074; }                 /* subnormal binary64 */
    else { mant |= (1ull << 52); E = biased - 1075; }
    acc[E - ORC_EXP_MIN] += (unsigned __int128)mant;
}

/* SSE buckets for one candidate; acc has ORC_NBUCKET entries, each written as two
 * uint64 (low, high) into out[2*j], out[2*j+1].                                     */
void orc_candidate_sse(const float* w, int64_t n, const double* g, int ng, float c,
                       uint64_t* out) {
    static const int nb = ORC_NBUCKET;
    unsigned __int128 acc[ORC_NBUCKET];
    memset(acc, 0, sizeof(acc));
    float qmax = (float)g[ng - 1];
    float s = c / qmax;
    float r = (s == 0.0f) ? 0.0f : 1.0f / s;
    for (int64_t i = 0; i < n; i++) {
        float a = fabsf(w[i]);
        float y = a * r;
        int code = nearest(fmin((double)y, g[ng - 1]), g, ng);
        float deq = (float)g[code] * s;
        double d = (double)a - (double)deq;
        add_exact(d * d, acc);
    }
    for (int j = 0; j < nb; j++) {
        out[2 * j] = (uint64_t)acc[j];
        out[2 * j + 1] = (uint64_t)(acc[j] >> 64);
    }
}

/* All candidates of one tensor: clips[j] for j < nc and each of nf grids (grids is
 * nf x 8 magnitudes).  out has nf*nc*ORC_NBUCKET*2 uint64; candidates are processed
 * in parallel, each one independently and exactly.                                  */
void orc_search_sse(const float* w, int64_t n, const double* grids, int nf, int ng,
                    const float* clips, int nc, uint64_t* out) {
    #pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < nf * nc; t++) {
        int f = t / nc, j = t % nc;
        orc_candidate_sse(w, n, grids + (int64_t)f * ng, ng, clips[j],
                          out + (int64_t)t * ORC_NBUCKET * 2);
    }
}

int orc_exp_min(void) { return ORC_EXP_MIN; }
int orc_nbucket(void) { return ORC_NBUCKET; }

// Host layer of libfp4: argument validation (before any launch), grid tables, and
// dispatch to the HIP kernels.  Every entry point of include/fp4.h is defined here.
#include <hip/hip_runtime.h>
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/fp4.h"
#include "fp4_internal.h"

using namespace fp4;

namespace {

thread_local char g_err[512] = "";

fp4_status fail(fp4_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

fp4_status ok() {
    g_err[0] = 0;
    return FP4_OK;
}

fp4_status hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(FP4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

// value of minifloat magnitude code c (canonical bias 1): p == 0 subnormal d/2^m,
// p >= 1 normal 2^(p-1) (1 + d/2^m)
double minifloat_value(int m, int c) {
    int p = c >> m, d = c & ((1 << m) - 1);
    if (p == 0) return std::ldexp((double)d, -m);
    return std::ldexp(1.0 + std::ldexp((double)d, -m), p - 1);
}

bool f16_exact(float v) {
    _Float16 h = (_Float16)v;
    return (float)h == v;
}

fp4_status make_grid(const fp4_grid& g, QGrid* q) {
    std::memset(q, 0, sizeof(*q));
    if (g.reserved != 0) return fail(FP4_ERR_INVALID_ARG, "fp4_grid.reserved must be 0");
    if (g.kind == FP4_GRID_MINIFLOAT && ((g.e == 4 && g.m == 3) || (g.e == 5 && g.m == 2))) {
        q->kind = 0;  // OCP FP8: E4M3 (bias 7, max 448) or E5M2 (bias 15, max 57344)
        q->e = g.e;
        q->m = g.m;
        q->bits = 8;
        q->qmax = g.e == 4 ? 448.0f : 57344.0f;
        return FP4_OK;
    }
    if (g.kind == FP4_GRID_MINIFLOAT && ((g.e == 2 && g.m == 3) || (g.e == 3 && g.m == 2))) {
        q->kind = 0;  // OCP FP6: E2M3 (bias 1, max 7.5) or E3M2 (bias 3, max 28)
        q->e = g.e;
        q->m = g.m;
        q->bits = 6;
        q->qmax = g.e == 2 ? 7.5f : 28.0f;
        return FP4_OK;
    }
    if (g.kind == FP4_GRID_MINIFLOAT) {
        if (g.e < 1 || g.m < 0 || g.e + g.m != 3)
            return fail(FP4_ERR_UNSUPPORTED, "minifloat grid needs e >= 1 and e + m == 3, or FP8 E4M3 / E5M2 (got e=%d m=%d)",
                        g.e, g.m);
        q->kind = 0;
        q->bits = 4;
        q->e = g.e;
        q->m = g.m;
        q->is_e2m1 = (g.e == 2 && g.m == 1);
        for (int c = 0; c < 8; c++) q->val[c] = (float)minifloat_value(g.m, c);
        for (int i = 0; i < 7; i++) q->thr[i] = (float)((minifloat_value(g.m, i) + minifloat_value(g.m, i + 1)) / 2);
        q->qmax = q->val[7];
        return FP4_OK;
    }
    if (g.kind == FP4_GRID_LUT16) {
        for (int i = 0; i < 16; i++) {
            if (!std::isfinite(g.lut[i]) || !f16_exact(g.lut[i]))
                return fail(FP4_ERR_INVALID_ARG, "lut[%d] must be finite and exact in binary16", i);
            if (i > 0 && !(g.lut[i] > g.lut[i - 1])) return fail(FP4_ERR_INVALID_ARG, "lut must be strictly increasing");
        }
        q->kind = 1;
        q->bits = 4;
        for (int i = 0; i < 16; i++) q->val[i] = g.lut[i];
        for (int i = 0; i < 15; i++) q->thr[i] = (float)(((double)g.lut[i] + (double)g.lut[i + 1]) / 2);
        q->qmax = std::fmax(std::fabs(g.lut[0]), std::fabs(g.lut[15]));
        if (!(q->qmax > 0)) return fail(FP4_ERR_INVALID_ARG, "lut has no nonzero value");
        return FP4_OK;
    }
    if (g.kind == FP4_GRID_TWO_MODE) {
        // E2M1 (mode 0) magnitudes and midpoints in [0, 8) / [0, 7), E1M2 (mode 1) in [8, 16) / [7, 14)
        q->kind = 2;
        q->bits = 4;
        for (int c = 0; c < 8; c++) {
            q->val[c] = (float)minifloat_value(1, c);
            q->val[8 + c] = (float)minifloat_value(2, c);
        }
        for (int i = 0; i < 7; i++) {
            q->thr[i] = (float)((minifloat_value(1, i) + minifloat_value(1, i + 1)) / 2);
            q->thr[7 + i] = (float)((minifloat_value(2, i) + minifloat_value(2, i + 1)) / 2);
        }
        q->qmax = q->val[7];
        return FP4_OK;
    }
    return fail(FP4_ERR_INVALID_ARG, "unknown grid kind %d", g.kind);
}

fp4_status check_gran(const fp4_gran& g, int64_t cols) {
    if (g.reserved != 0) return fail(FP4_ERR_INVALID_ARG, "fp4_gran.reserved must be 0");
    if (g.mode < FP4_SCALE_TENSOR || g.mode > FP4_SCALE_GROUP) return fail(FP4_ERR_INVALID_ARG, "bad scale mode %d", g.mode);
    if (g.scale_dtype != FP4_F32 && g.scale_dtype != FP4_F16)
        return fail(FP4_ERR_INVALID_ARG, "scale dtype must be FP4_F32 or FP4_F16");
    if (g.mode == FP4_SCALE_TENSOR && g.scale_dtype != FP4_F32)
        return fail(FP4_ERR_UNSUPPORTED, "per-tensor scales are f32 only");
    if (g.mode == FP4_SCALE_GROUP) {
        if (!is_pow2(g.group) || g.group < 8 || g.group > 512)
            return fail(FP4_ERR_UNSUPPORTED, "group must be a power of two in [8, 512] (got %d)", g.group);
        if (cols % g.group != 0) return fail(FP4_ERR_INVALID_ARG, "cols (%lld) must be a multiple of group %d",
                                             (long long)cols, g.group);
    }
    return FP4_OK;
}

int64_t units_of(const fp4_gran& g, int64_t rows, int64_t cols) {
    return g.mode == FP4_SCALE_TENSOR ? 1 : (g.mode == FP4_SCALE_ROW ? rows : rows * (cols / g.group));
}

}  // namespace

extern "C" {

const char* fp4_status_string(fp4_status s) {
    switch (s) {
        case FP4_OK: return "FP4_OK";
        case FP4_ERR_INVALID_ARG: return "FP4_ERR_INVALID_ARG";
        case FP4_ERR_UNSUPPORTED: return "FP4_ERR_UNSUPPORTED";
        case FP4_ERR_ALIGNMENT: return "FP4_ERR_ALIGNMENT";
        case FP4_ERR_WORKSPACE: return "FP4_ERR_WORKSPACE";
        case FP4_ERR_HIP: return "FP4_ERR_HIP";
        default: return "FP4_ERR_UNKNOWN";
    }
}

const char* fp4_last_error(void) { return g_err; }

fp4_status fp4_calibrate(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ld, int32_t reduce,
                         int32_t group, int64_t first_rows, float* amax_out, void* stream) {
    if (!amax_out || (!x && rows != 0 && cols != 0)) return fail(FP4_ERR_INVALID_ARG, "null pointer");
    if (x_dtype != FP4_F32 && x_dtype != FP4_BF16) return fail(FP4_ERR_INVALID_ARG, "x_dtype must be FP4_F32 or FP4_BF16");
    if (rows < 0 || cols < 0 || ld < cols) return fail(FP4_ERR_INVALID_ARG, "bad sizes rows=%lld cols=%lld ld=%lld",
                                                       (long long)rows, (long long)cols, (long long)ld);
    if (reduce < FP4_REDUCE_TENSOR || reduce > FP4_REDUCE_ROW_GROUP) return fail(FP4_ERR_INVALID_ARG, "bad reduce %d", reduce);
    if (reduce == FP4_REDUCE_ROW_GROUP) {
        if (!is_pow2(group) || group < 8 || group > 512) return fail(FP4_ERR_UNSUPPORTED, "group must be a power of two in [8, 512]");
        if (cols % group) return fail(FP4_ERR_INVALID_ARG, "cols must be a multiple of group");
    }
    if (!aligned16(x) || (reinterpret_cast<uintptr_t>(amax_out) & 3u))
        return fail(FP4_ERR_ALIGNMENT, "x must be 16-byte aligned and amax_out 4-byte aligned");
    int64_t r = (first_rows > 0 && first_rows < rows) ? first_rows : rows;
    int esz = x_dtype == FP4_BF16 ? 2 : 4;
    int vec = ((ld * esz) % 16 == 0) && (cols % 8 == 0);
    return hip_status(launch_calibrate(x, x_dtype == FP4_BF16, r, cols, ld, reduce, group, amax_out, vec,
                                       (hipStream_t)stream),
                      "fp4_calibrate");
}

fp4_status fp4_quantize_pack(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ldx, fp4_grid grid,
                             fp4_gran gran, const float* amax_in, const float* tensor_scale, const int8_t* col_shift,
                             uint8_t* packed, int64_t ldp, void* scales_out, void* stream) {
    const bool empty = rows == 0 || cols == 0;
    if ((!x || !packed) && !empty) return fail(FP4_ERR_INVALID_ARG, "null pointer");
    if (x_dtype != FP4_F32 && x_dtype != FP4_BF16) return fail(FP4_ERR_INVALID_ARG, "x_dtype must be FP4_F32 or FP4_BF16");
    if (rows < 0 || cols < 0 || (cols & 1) || ldx < cols || ldp < cols / 2)
        return fail(FP4_ERR_INVALID_ARG, "bad sizes (cols must be even, ldx >= cols, ldp >= cols/2)");
    QGrid q;
    fp4_status st = make_grid(grid, &q);
    if (st) return st;
    if ((st = check_gran(gran, cols))) return st;
    if (q.bits != 4) {
        if (ldp < cols * q.bits / 8) return fail(FP4_ERR_INVALID_ARG, "ldp below the code bytes of a row (cols * bits / 8)");
        if (cols % 8 != 0 || (q.bits == 6 && ldp % 2 != 0))
            return fail(FP4_ERR_UNSUPPORTED, "FP8/FP6 quantization needs cols % 8 == 0 (FP6: ldp even)");
    }
    if (q.kind == 2 && (gran.mode != FP4_SCALE_GROUP || col_shift))
        return fail(FP4_ERR_UNSUPPORTED, "the two-mode grid needs GROUP scales and no column shifts");
    if (tensor_scale && gran.mode != FP4_SCALE_TENSOR) return fail(FP4_ERR_INVALID_ARG, "tensor_scale needs TENSOR mode");
    if (tensor_scale && scales_out && (const void*)tensor_scale == scales_out)
        return fail(FP4_ERR_INVALID_ARG, "tensor_scale and scales_out must not alias");
    if (!aligned16(x) || !aligned16(packed) || !aligned16(col_shift))
        return fail(FP4_ERR_ALIGNMENT, "x, packed and col_shift must be 16-byte aligned");
    if (empty && gran.mode != FP4_SCALE_TENSOR) return ok();  // nothing to quantize, no scale unit
    if (!scales_out && !tensor_scale) return fail(FP4_ERR_INVALID_ARG, "scales_out may be NULL only with tensor_scale");
    int esz = x_dtype == FP4_BF16 ? 2 : 4;
    QuantParams p{};
    p.x = x;
    p.ldx = ldx;
    p.x_bf16 = x_dtype == FP4_BF16;
    p.mode = gran.mode;
    p.rows = rows;
    p.cols = cols;
    p.packed = packed;
    p.ldp = ldp;
    p.group = gran.mode == FP4_SCALE_GROUP ? gran.group : 0;
    p.scale_f16 = gran.scale_dtype == FP4_F16;
    p.amax_in = amax_in;
    p.tensor_scale = tensor_scale;
    p.scales_out = scales_out;
    p.col_shift = col_shift;
    p.shift_sign = -1;
    p.vec = ((ldx * esz) % 16 == 0) && (cols % 8 == 0) && (ldp % (q.bits == 8 ? 8 : 4) == 0);  // FP6 stores 16-bit words
    p.g = q;
    hipStream_t s = (hipStream_t)stream;
    if (gran.mode == FP4_SCALE_TENSOR && !tensor_scale) {
        // per-tensor scale from the amax: reduce into scales_out (as scratch), quantize
        // reading that amax, then overwrite it with s = amax / Qmax
        float* sc = reinterpret_cast<float*>(scales_out);
        if (amax_in) {
            p.tensor_amax = amax_in;
        } else {
            hipError_t e = launch_calibrate(x, p.x_bf16, rows, cols, ldx, FP4_REDUCE_TENSOR, 0, sc, p.vec, s);
            if (e != hipSuccess) return hip_status(e, "fp4_quantize_pack/amax");
            p.tensor_amax = sc;
        }
        hipError_t e = launch_quantize(p, s);
        if (e != hipSuccess) return hip_status(e, "fp4_quantize_pack");
        return hip_status(launch_tensor_scale_finalize(p.tensor_amax, sc, q.qmax, s), "fp4_quantize_pack/scale");
    }
    return hip_status(launch_quantize(p, s), "fp4_quantize_pack");
}

fp4_status fp4_dequantize(const uint8_t* packed, int64_t rows, int64_t cols, int64_t ldp, fp4_grid grid, fp4_gran gran,
                          const void* scales, const int8_t* col_shift, float* out, int64_t ldo, void* stream) {
    if (rows < 0 || cols < 0 || (cols & 1) || ldp < cols / 2 || ldo < cols) return fail(FP4_ERR_INVALID_ARG, "bad sizes");
    if (rows == 0 || cols == 0) return ok();
    if (!packed || !scales || !out) return fail(FP4_ERR_INVALID_ARG, "null pointer");
    QGrid q;
    fp4_status st = make_grid(grid, &q);
    if (st) return st;
    if (q.bits != 4 && ldp < cols * q.bits / 8) return fail(FP4_ERR_INVALID_ARG, "ldp below the code bytes of a row");
    if (q.bits == 6 && cols % 4 != 0) return fail(FP4_ERR_INVALID_ARG, "FP6 rows hold whole groups of four codes");
    if ((st = check_gran(gran, cols))) return st;
    if (q.kind == 2 && gran.mode != FP4_SCALE_GROUP) return fail(FP4_ERR_UNSUPPORTED, "the two-mode grid needs GROUP scales");
    return hip_status(launch_dequantize(packed, rows, cols, ldp, q, gran.mode, gran.group, scales,
                                        gran.scale_dtype == FP4_F16, col_shift, out, ldo, (hipStream_t)stream),
                      "fp4_dequantize");
}

fp4_status fp4_preshift_weights(const float* w, int64_t n, int64_t k, int64_t ldw, const float* chan_amax,
                                fp4_grid act_grid, fp4_grid w_grid, fp4_gran w_gran, int8_t* shift_out,
                                float* act_scale_out, uint8_t* w_packed, int64_t ldp, void* w_scales, void* stream) {
    if (!w || !chan_amax || !shift_out || !act_scale_out || !w_packed || !w_scales)
        return fail(FP4_ERR_INVALID_ARG, "null pointer");
    if (n < 0 || k <= 0 || (k & 1) || ldw < k || ldp < k / 2) return fail(FP4_ERR_INVALID_ARG, "bad sizes");
    QGrid qa, qw;
    fp4_status st = make_grid(act_grid, &qa);
    if (st) return st;
    if ((st = make_grid(w_grid, &qw))) return st;
    if ((st = check_gran(w_gran, k))) return st;
    if (w_gran.mode == FP4_SCALE_TENSOR) return fail(FP4_ERR_UNSUPPORTED, "pre-shifted weights need ROW or GROUP scales");
    if (qa.kind == 2 || qw.kind == 2) return fail(FP4_ERR_UNSUPPORTED, "pre-shift with the two-mode grid is not implemented");
    if (qw.bits != 4) {
        if (ldp < k * qw.bits / 8) return fail(FP4_ERR_INVALID_ARG, "ldp below the code bytes of a row (k * bits / 8)");
        if (k % 8 != 0 || (qw.bits == 6 && ldp % 2 != 0))
            return fail(FP4_ERR_UNSUPPORTED, "FP8/FP6 weights need k % 8 == 0 (FP6: ldp even)");
    }
    if (!aligned16(w) || !aligned16(w_packed) || !aligned16(shift_out))
        return fail(FP4_ERR_ALIGNMENT, "w, w_packed and shift_out must be 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_preshift_factors(chan_amax, k, qa.qmax, shift_out, act_scale_out, s);
    if (e != hipSuccess) return hip_status(e, "fp4_preshift_weights/factors");
    QuantParams p{};
    p.x = w;
    p.ldx = ldw;
    p.x_bf16 = 0;
    p.mode = w_gran.mode;
    p.rows = n;
    p.cols = k;
    p.packed = w_packed;
    p.ldp = ldp;
    p.group = w_gran.mode == FP4_SCALE_GROUP ? w_gran.group : 0;
    p.scale_f16 = w_gran.scale_dtype == FP4_F16;
    p.scales_out = w_scales;
    p.col_shift = shift_out;
    p.shift_sign = +1;
    p.vec = ((ldw * 4) % 16 == 0) && (k % 8 == 0) && (ldp % (qw.bits == 8 ? 8 : 4) == 0);
    p.g = qw;
    return hip_status(launch_quantize(p, s), "fp4_preshift_weights/quantize");
}

size_t fp4_search_workspace_size(int64_t ntensors, int64_t numel, int32_t nformats, int32_t nclips) {
    if (ntensors < 0 || numel < 0 || nformats < 1 || nclips < 1) return 0;
    return search_workspace_bytes(ntensors, numel, nformats, nclips);
}

// candidate list and clip range shared by both search entry points
static fp4_status search_candidates(const int32_t* formats_em, int32_t nformats, int32_t nclips, float clip_lo,
                                    float clip_hi, SearchCandidates* c) {
    if (!formats_em) return fail(FP4_ERR_INVALID_ARG, "null pointer");
    if (nformats < 1 || nformats > 8 || nclips < 2 || (int64_t)nformats * nclips > 512)
        return fail(FP4_ERR_UNSUPPORTED, "need 1..8 formats, >= 2 clips, at most 512 candidates");
    if (!(clip_lo > 0.0f) || !(clip_hi >= clip_lo) || !(clip_hi <= 1.0f))
        return fail(FP4_ERR_INVALID_ARG, "need 0 < clip_lo <= clip_hi <= 1");
    *c = SearchCandidates{};
    c->nformats = nformats;
    c->nclips = nclips;
    for (int f = 0; f < nformats; f++) {
        int e = formats_em[2 * f], m = formats_em[2 * f + 1];
        if (e < 1 || m < 0 || e + m != 3) return fail(FP4_ERR_UNSUPPORTED, "format %d: need e >= 1 and e + m == 3", f);
        c->fmt_e[f] = e;
        c->fmt_m[f] = m;
        c->fmt_qmax[f] = (float)minifloat_value(m, 7);
    }
    return FP4_OK;
}

static fp4_status search_workspace_check(int64_t units, int64_t numel, const SearchCandidates& c, void* workspace,
                                         size_t ws_bytes) {
    size_t need = search_workspace_bytes(units, numel, c.nformats, c.nclips);
    if (!workspace || ws_bytes < need)
        return fail(FP4_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : 0);
    if (!aligned16(workspace)) return fail(FP4_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
    return FP4_OK;
}

fp4_status fp4_search_format(const float* w, int64_t ntensors, int64_t numel, const int32_t* formats_em,
                             int32_t nformats, int32_t nclips, float clip_lo, float clip_hi,
                             fp4_search_result* results, uint8_t* packed, void* workspace, size_t ws_bytes,
                             void* stream) {
    if (!w || !formats_em || !results || !packed) return fail(FP4_ERR_INVALID_ARG, "null pointer");
    if (ntensors < 0 || numel <= 0 || numel % 16 != 0)
        return fail(FP4_ERR_INVALID_ARG, "numel must be a positive multiple of 16");
    SearchCandidates c;
    fp4_status st = search_candidates(formats_em, nformats, nclips, clip_lo, clip_hi, &c);
    if (st) return st;
    if (!aligned16(w) || !aligned16(packed) || !aligned16(results))
        return fail(FP4_ERR_ALIGNMENT, "w, packed and results must be 16-byte aligned");
    if ((st = search_workspace_check(ntensors, numel, c, workspace, ws_bytes))) return st;
    SearchInput in{w, 0, 1, numel, ntensors, numel, 1};
    return hip_status(launch_search(in, c, (double)clip_lo, (double)clip_hi, results, packed, numel / 2, workspace,
                                    (hipStream_t)stream),
                      "fp4_search_format");
}

fp4_status fp4_search_format_static(const float* w, int64_t ntensors, int64_t numel, const int32_t* formats_em,
                                    int32_t nformats, int32_t nclips, float clip_lo, float clip_hi,
                                    fp4_search_result* results, uint8_t* packed, void* stream) {
    if (!w || !formats_em || !results || !packed) return fail(FP4_ERR_INVALID_ARG, "null pointer");
    if (ntensors < 0 || numel <= 0 || numel % 16 != 0)
        return fail(FP4_ERR_INVALID_ARG, "numel must be a positive multiple of 16");
    SearchCandidates c;
    fp4_status st = search_candidates(formats_em, nformats, nclips, clip_lo, clip_hi, &c);
    if (st) return st;
    if (!aligned16(w) || !aligned16(packed) || !aligned16(results))
        return fail(FP4_ERR_ALIGNMENT, "w, packed and results must be 16-byte aligned");
    const size_t need = search_workspace_bytes(ntensors, numel, c.nformats, c.nclips);
    if (need > kSearchScratchBytes)
        return fail(FP4_ERR_WORKSPACE, "this search needs %zu bytes of scratch; the static scratch holds %zu "
                    "(use fp4_search_format with a workspace)", need, kSearchScratchBytes);
    if (ntensors == 0) return ok();
    void* ws = nullptr;
    if ((st = hip_status(search_scratch(&ws), "fp4_search_format_static: scratch address"))) return st;
    SearchInput in{w, 0, 1, numel, ntensors, numel, 1};
    return hip_status(launch_search(in, c, (double)clip_lo, (double)clip_hi, results, packed, numel / 2, ws,
                                    (hipStream_t)stream),
                      "fp4_search_format_static");
}

fp4_status fp4_search_activations(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                                  int32_t unit, int64_t first_rows, const int32_t* formats_em, int32_t nformats,
                                  int32_t nclips, float clip_lo, float clip_hi, fp4_search_result* results,
                                  uint8_t* packed, int64_t ldp, void* workspace, size_t ws_bytes, void* stream) {
    if (!x || !formats_em || !results || !packed) return fail(FP4_ERR_INVALID_ARG, "null pointer");
    if (x_dtype != FP4_F32 && x_dtype != FP4_BF16) return fail(FP4_ERR_INVALID_ARG, "x_dtype must be F32 or BF16");
    if (rows < 0 || cols <= 0 || cols % 16 != 0) return fail(FP4_ERR_INVALID_ARG, "cols must be a positive multiple of 16");
    if (ldx < cols || ldx % 4 != 0) return fail(FP4_ERR_ALIGNMENT, "ldx must be >= cols and a multiple of 4");
    if (ldp < cols / 2 || ldp % 4 != 0) return fail(FP4_ERR_ALIGNMENT, "ldp must be >= cols/2 and a multiple of 4");
    if (unit != FP4_SCALE_TENSOR && unit != FP4_SCALE_ROW) return fail(FP4_ERR_INVALID_ARG, "unit must be TENSOR or ROW");
    SearchCandidates c;
    fp4_status st = search_candidates(formats_em, nformats, nclips, clip_lo, clip_hi, &c);
    if (st) return st;
    if (!aligned16(x) || !aligned16(packed) || !aligned16(results))
        return fail(FP4_ERR_ALIGNMENT, "x, packed and results must be 16-byte aligned");
    const int64_t t = unit == FP4_SCALE_ROW ? 1 : (first_rows > 0 && first_rows < rows ? first_rows : rows);
    if (rows == 0) return ok();
    const int64_t units = unit == FP4_SCALE_ROW ? rows : 1;
    if ((st = search_workspace_check(units, t * cols, c, workspace, ws_bytes))) return st;
    SearchInput in{x, x_dtype == FP4_BF16, unit == FP4_SCALE_ROW, ldx, rows, cols, t};
    return hip_status(launch_search(in, c, (double)clip_lo, (double)clip_hi, results, packed, ldp, workspace,
                                    (hipStream_t)stream),
                      "fp4_search_activations");
}

fp4_status fp4_gemm(const fp4_gemm_desc* d, void* stream) {
    if (!d) return fail(FP4_ERR_INVALID_ARG, "null descriptor");
    if (d->M < 0 || d->N < 0 || d->K <= 0 || (d->K & 1)) return fail(FP4_ERR_INVALID_ARG, "bad sizes");
    if (d->M == 0 || d->N == 0) return ok();  // empty output: nothing to do
    if (!d->a || !d->w || !d->w_scales || !d->y) return fail(FP4_ERR_INVALID_ARG, "null pointer");
    if (d->ldw < d->K / 2 || d->ldy < d->N) return fail(FP4_ERR_INVALID_ARG, "bad leading dimensions");
    if (d->y_dtype != FP4_BF16 && d->y_dtype != FP4_F32) return fail(FP4_ERR_INVALID_ARG, "y_dtype must be BF16 or F32");
    if (d->reserved1) return fail(FP4_ERR_INVALID_ARG, "reserved fields must be 0");
    if (d->a_scale_mode != FP4_SCALE_TENSOR && d->a_scale_mode != FP4_SCALE_ROW)
        return fail(FP4_ERR_INVALID_ARG, "a_scale_mode must be TENSOR or ROW");
    GemmParams p{};
    fp4_status st = make_grid(d->w_grid, &p.wg);
    if (st) return st;
    if ((st = check_gran(d->w_gran, d->K))) return st;
    p.M = d->M;
    p.N = d->N;
    p.K = d->K;
    p.a_kind = d->a_kind;
    p.a = d->a;
    p.lda = d->lda;
    p.a_scale = d->a_scale;
    p.a_row = d->a_scale_mode == FP4_SCALE_ROW;
    p.w = d->w;
    p.ldw = d->ldw;
    p.w_mode = d->w_gran.mode;
    p.w_group = d->w_gran.mode == FP4_SCALE_GROUP ? d->w_gran.group : 0;
    p.w_scale_f16 = d->w_gran.scale_dtype == FP4_F16;
    p.w_scales = d->w_scales;
    p.y = d->y;
    p.ldy = d->ldy;
    p.y_bf16 = d->y_dtype == FP4_BF16;
    hipStream_t s = (hipStream_t)stream;
    if (!aligned16(d->a) || !aligned16(d->w) || (d->ldw % 16) != 0)
        return fail(FP4_ERR_ALIGNMENT, "a and w must be 16-byte aligned and ldw a multiple of 16");

    if (p.wg.kind == 2 && (d->w_gran.mode != FP4_SCALE_GROUP || d->a_kind == FP4_PACKED))
        return fail(FP4_ERR_UNSUPPORTED, "two-mode weights need GROUP scales and f32/bf16 activations");
    if (p.a_row && (d->a_kind != FP4_PACKED || p.wg.kind != 0))
        return fail(FP4_ERR_UNSUPPORTED, "per-token activation scales are taken by the products of two minifloat grids only");
    if (p.wg.bits != 4 && d->a_kind == FP4_PACKED) {
        // both operands FP8 / FP6 on the f8f6f4 matrix cores: E4M3 x E4M3 on the
        // persistent kernel, every other pair (W6A6 among them) on the tiled one
        QGrid qa;
        if ((st = make_grid(d->a_grid, &qa))) return st;
        if (qa.kind != 0)
            return fail(FP4_ERR_UNSUPPORTED, "FP8 / FP6 weights with packed activations need minifloat activations");
        if (!d->a_scale) return fail(FP4_ERR_INVALID_ARG, "packed activations need a_scale");
        if (d->K % 32 != 0) return fail(FP4_ERR_UNSUPPORTED, "K must be a multiple of 32");
        if (d->lda < d->K * qa.bits / 8 || d->ldw < d->K * p.wg.bits / 8 || d->lda % 16 != 0)
            return fail(FP4_ERR_ALIGNMENT, "FP8 / FP6 rows: lda, ldw >= the code bytes of a row, lda a multiple of 16");
        // weight scales: f32 per tensor or per output row, or f32 / f16 per row and group of
        // G codes along K (G a multiple of 64 dividing K: the tiled kernel, E4M3 x E4M3 too)
        const bool grp = d->w_gran.mode == FP4_SCALE_GROUP;
        if (grp) {
            if (d->w_gran.group % 64 != 0 || d->K % d->w_gran.group != 0)
                return fail(FP4_ERR_UNSUPPORTED,
                            "group-scaled FP8 / FP6 weights need a group that is a multiple of 64 and divides K");
            if (256 * (d->K / d->w_gran.group) * 4 >= 0x7fff0000)
                return fail(FP4_ERR_UNSUPPORTED, "too many weight groups per row");
        } else if (d->w_gran.scale_dtype != FP4_F32) {
            return fail(FP4_ERR_UNSUPPORTED, "FP8 / FP6 products need f32 TENSOR or ROW weight scales, or GROUP scales");
        }
        p.ag = qa;
        if (!grp && p.wg.bits == 8 && p.wg.e == 4 && qa.bits == 8 && qa.e == 4)
            return hip_status(launch_w8a8_fp8(p, s), "fp4_gemm/w8a8");
        if (!grp && p.wg.bits == 8 && p.wg.e == 5 && qa.bits == 8 && qa.e == 5)
            return hip_status(launch_w8a8_e5m2(p, s), "fp4_gemm/w8a8-e5m2");
        if (!grp && p.wg.bits == 8 && qa.bits == 8 && p.wg.e != qa.e)
            return hip_status(launch_w8a8_mixed(p, s), "fp4_gemm/w8a8-mixed");
        if (!grp && p.wg.bits == 6 && qa.bits == 6 && p.wg.e == qa.e && w6a6_fits(p))
            return hip_status(launch_w6a6_fp6(p, s), "fp4_gemm/w6a6");
        // E4M3 x E4M3 with group-128 scales: the persistent kernel, when its operands fit
        if (grp && p.wg.bits == 8 && p.wg.e == 4 && qa.bits == 8 && qa.e == 4 && w8a8_group_fits(p))
            return hip_status(launch_w8a8_fp8_group(p, s), "fp4_gemm/w8a8-group");
        if (256 * std::max(d->lda, d->ldw) >= 0x7fff0000)
            return fail(FP4_ERR_UNSUPPORTED, "FP8 / FP6 rows longer than 8 MiB are not supported");
        return hip_status(launch_f8f6_gemm(p, s), "fp4_gemm/f8f6");
    }
    if (p.wg.bits != 4) {
        if (d->ldw < d->K * p.wg.bits / 8) return fail(FP4_ERR_INVALID_ARG, "ldw below the code bytes of a row");
        if (p.wg.bits == 6 && d->K % 4 != 0) return fail(FP4_ERR_INVALID_ARG, "FP6 rows hold whole groups of four codes");
    }
    if (d->a_kind == FP4_F32 || d->a_kind == FP4_BF16) {
        if (d->lda < d->K) return fail(FP4_ERR_INVALID_ARG, "lda < K");
        // 4-bit minifloat weights E1M2, E2M1, E3M0: the bf16 matrix-core kernels
        const bool mini4 = p.wg.kind == 0 && p.wg.bits == 4 && p.wg.e >= 1 && p.wg.e <= 3;
        bool mfma = d->a_kind == FP4_BF16 && mini4 && d->K % 128 == 0 && (d->lda * 2) % 16 == 0 &&
                    (d->w_gran.mode != FP4_SCALE_GROUP || d->w_gran.group % 128 == 0);
        // FP8 / FP6 weights: the small-batch matrix-core kernel, else the VALU kernel
        if (p.wg.bits != 4) {
            if (d->a_kind == FP4_BF16 && d->K % 128 == 0 && (d->lda * 2) % 16 == 0 && d->M <= 16 &&
                (d->w_gran.mode != FP4_SCALE_GROUP || d->w_gran.group == 128))
                return hip_status(launch_w8a16_small(p, s), "fp4_gemm/w8a16");
            return hip_status(launch_w4a16_valu(p, s), "fp4_gemm/w8a16_valu");
        }
        // two-mode weights: the small-batch matrix-core kernel (group 128), else the VALU kernel
        if (p.wg.kind == 2 && d->a_kind == FP4_BF16 && d->K % 128 == 0 && (d->lda * 2) % 16 == 0 &&
            d->w_gran.group == 128 && d->M <= 16)
            return hip_status(launch_w4a16_two_mode(p, s), "fp4_gemm/w4a16_two_mode");
        if (mfma) return hip_status(launch_w4a16_mfma(p, s), "fp4_gemm/w4a16");
        return hip_status(launch_w4a16_valu(p, s), "fp4_gemm/w4a16_valu");
    }
    if (d->a_kind != FP4_PACKED) return fail(FP4_ERR_INVALID_ARG, "a_kind must be F32, BF16 or PACKED");
    if (!d->a_scale) return fail(FP4_ERR_INVALID_ARG, "packed activations need a_scale");
    if ((st = make_grid(d->a_grid, &p.ag))) return st;
    const bool w4_mini = p.wg.kind == 0 && p.wg.bits == 4, a4_mini = p.ag.kind == 0 && p.ag.bits == 4;
    if ((p.ag.kind == 0 && p.ag.bits != 4 && w4_mini) || (w4_mini && a4_mini && !(p.wg.is_e2m1 && p.ag.is_e2m1))) {
        // FP8 / FP6 activations with 4-bit minifloat weights, and the 4-bit pairs with an
        // E1M2 or E3M0 operand (rewritten as FP8 E4M3 in LDS): the tiled f8f6f4 kernel
        if (d->K % 32 != 0) return fail(FP4_ERR_UNSUPPORTED, "K must be a multiple of 32");
        if (d->lda < d->K * p.ag.bits / 8 || d->lda % 16 != 0)
            return fail(FP4_ERR_ALIGNMENT, "packed rows: lda >= the code bytes of a row, a multiple of 16");
        if (d->w_gran.mode == FP4_SCALE_GROUP || d->w_gran.scale_dtype != FP4_F32)
            return fail(FP4_ERR_UNSUPPORTED, "FP8 / FP6 products need f32 TENSOR or ROW weight scales");
        if (256 * std::max(d->lda, d->ldw) >= 0x7fff0000)
            return fail(FP4_ERR_UNSUPPORTED, "FP8 / FP6 rows longer than 8 MiB are not supported");
        return hip_status(launch_f8f6_gemm(p, s), "fp4_gemm/f8f6");
    }
    if (d->lda < d->K / 2 || d->lda % 16 != 0) return fail(FP4_ERR_ALIGNMENT, "packed lda must be >= K/2 and a multiple of 16");
    if (!p.ag.is_e2m1) return fail(FP4_ERR_UNSUPPORTED, "packed activations must be E2M1");
    if (d->K % 32 != 0) return fail(FP4_ERR_UNSUPPORTED, "K must be a multiple of 32");
    if (p.wg.is_e2m1) {
        if (d->w_gran.mode == FP4_SCALE_GROUP || d->w_gran.scale_dtype != FP4_F32)
            return fail(FP4_ERR_UNSUPPORTED, "E2M1 x E2M1 needs f32 TENSOR or ROW weight scales");
        // quarter-integer partial sums below 36 K stay exact in fp32 while 36 K < 2^22
        if (d->K > 116508) return fail(FP4_ERR_UNSUPPORTED, "E2M1 x E2M1 needs K <= 116508 (exact fp32 accumulation)");
        return hip_status(launch_w4a4_fp4(p, s), "fp4_gemm/w4a4");
    }
    if (p.wg.kind == 1) {
        if (d->w_gran.mode != FP4_SCALE_GROUP || d->w_gran.group % 64 != 0 || d->K % 64 != 0)
            return fail(FP4_ERR_UNSUPPORTED, "lookup-grid weights need GROUP scales with group a multiple of 64");
        return hip_status(launch_w4a4_lut(p, s), "fp4_gemm/w4a4_lut");
    }
    return fail(FP4_ERR_UNSUPPORTED, "unsupported pair of weight and activation grids");
}

// Standard normal quantile: the x with Phi(x) = 0.5 erfc(-x / sqrt 2) = p, by bisection
// in binary64 until the bracket cannot shrink (monotone, so the last midpoint is within
// one binary64 step of the root for 0 < p < 1).
static double normal_quantile(double p) {
    double lo = -40.0, hi = 40.0;
    for (int i = 0; i < 200; i++) {
        const double mid = 0.5 * (lo + hi);
        if (mid == lo || mid == hi) break;
        if (0.5 * std::erfc(-mid / std::sqrt(2.0)) < p) lo = mid;
        else hi = mid;
    }
    return 0.5 * (lo + hi);
}

// Round a binary64 value in the binary16 normal range to the nearest binary16 value,
// ties to even (11 significant bits; the current rounding mode is round-to-nearest-even).
static double round_to_f16(double v) {
    int e = 0;
    const double f = std::frexp(v, &e);  // v = f 2^e, 0.5 <= |f| < 1
    return std::ldexp(std::nearbyint(std::ldexp(f, 11)), e - 11);
}

fp4_status fp4_nf4_grid(fp4_grid* out) {
    if (!out) return fail(FP4_ERR_INVALID_ARG, "null grid");
    std::memset(out, 0, sizeof(*out));
    out->kind = FP4_GRID_LUT16;
    const double z = normal_quantile(15.5 / 16.0);
    for (int i = 0; i < 16; i++) out->lut[i] = (float)round_to_f16(normal_quantile((i + 0.5) / 16.0) / z);
    return ok();
}

fp4_status fp4_set_split_limit(int64_t bytes) {
    set_split_limit(bytes);
    return ok();
}

fp4_status fp4_gemm_swiglu_quant(const fp4_swiglu_desc* d, void* stream) {
    if (!d) return fail(FP4_ERR_INVALID_ARG, "null descriptor");
    if (d->M < 0 || d->N < 0 || d->K <= 0) return fail(FP4_ERR_INVALID_ARG, "bad sizes");
    if (d->N % 32 != 0) return fail(FP4_ERR_UNSUPPORTED, "N must be a multiple of 32");
    if (d->K % 32 != 0) return fail(FP4_ERR_UNSUPPORTED, "K must be a multiple of 32");
    if (d->K > 116508) return fail(FP4_ERR_UNSUPPORTED, "K <= 116508 (exact fp32 accumulation)");
    if (d->M == 0 || d->N == 0) return ok();
    if (!d->a || !d->a_scale || !d->w_gate || !d->w_up || !d->s_gate || !d->s_up || !d->out_scale ||
        !d->h_packed)
        return fail(FP4_ERR_INVALID_ARG, "null pointer");
    if (d->lda < d->K / 2 || d->ldw < d->K / 2 || d->ldh < d->N / 2)
        return fail(FP4_ERR_INVALID_ARG, "bad leading dimensions");
    if (!aligned16(d->a) || !aligned16(d->w_gate) || !aligned16(d->w_up) || !aligned16(d->h_packed) ||
        d->lda % 16 != 0 || d->ldw % 16 != 0 || d->ldh % 16 != 0)
        return fail(FP4_ERR_ALIGNMENT, "a, w_gate, w_up, h_packed 16-byte aligned; lda, ldw, ldh multiples of 16");
    GemmParams p{};
    p.M = d->M;
    p.N = d->N;
    p.K = d->K;
    p.a_kind = FP4_PACKED;
    p.a = d->a;
    p.lda = d->lda;
    p.a_scale = d->a_scale;
    p.w = d->w_gate;
    p.ldw = d->ldw;
    p.w_mode = FP4_SCALE_ROW;
    p.w_scales = d->s_gate;
    p.y = d->h_packed;
    p.ldy = d->ldh;
    GluParams g{d->w_up, d->s_up, d->out_scale, d->out_shift};
    return hip_status(launch_w4a4_swiglu(p, g, (hipStream_t)stream), "fp4_gemm_swiglu_quant");
}

}  // extern "C"

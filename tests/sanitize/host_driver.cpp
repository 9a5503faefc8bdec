// Drives the host layer (fp4_api.cpp) through every entry point under AddressSanitizer
// and UndefinedBehaviorSanitizer, on the CPU: the kernel launchers are replaced by stubs
// that count calls, so every validation and routing path runs without a GPU.  Device
// pointers are fake, 16-byte aligned addresses; the host layer must never dereference
// them (the sanitizers would report it).  Exits non-zero on an unexpected status.
#include <cmath>
#include <cstdio>
#include <cstring>

#include "../../include/fp4.h"
#include "../../bit_floating_point_amd/csrc/fp4_internal.h"

static int g_calls = 0;

extern "C" const char* hipGetErrorString(hipError_t) { return "stub"; }

namespace fp4 {
#define STUB(...) { (void)sizeof(#__VA_ARGS__); ++g_calls; return hipSuccess; }
hipError_t launch_calibrate(const void*, int, int64_t, int64_t, int64_t, int, int, float*, int, hipStream_t) STUB()
hipError_t launch_quantize(const QuantParams& p, hipStream_t) {
    if (p.rows <= 0 || p.cols <= 0 || !p.packed) std::abort();
    ++g_calls;
    return hipSuccess;
}
hipError_t launch_tensor_scale_finalize(const float*, float*, float, hipStream_t) STUB()
hipError_t launch_dequantize(const uint8_t*, int64_t, int64_t, int64_t, const QGrid&, int, int, const void*, int,
                             const int8_t*, float*, int64_t, hipStream_t) STUB()
hipError_t launch_preshift_factors(const float*, int64_t, float, int8_t*, float*, hipStream_t) STUB()
hipError_t launch_w4a16_mfma(const GemmParams&, hipStream_t) STUB()
hipError_t launch_w4a16_valu(const GemmParams&, hipStream_t) STUB()
hipError_t launch_w4a16_two_mode(const GemmParams&, hipStream_t) STUB()
hipError_t launch_w8a16_small(const GemmParams&, hipStream_t) STUB()
hipError_t launch_w4a4_fp4(const GemmParams&, hipStream_t) STUB()
hipError_t launch_w8a8_fp8(const GemmParams&, hipStream_t) STUB()
hipError_t launch_w8a8_e5m2(const GemmParams&, hipStream_t) STUB()
hipError_t launch_w8a8_mixed(const GemmParams&, hipStream_t) STUB()
bool w6a6_fits(const GemmParams& p) { return p.K % 128 == 0; }
hipError_t launch_w6a6_fp6(const GemmParams&, hipStream_t) STUB()
bool w8a8_group_fits(const GemmParams& p) { return p.w_group == 128 && p.K % 128 == 0; }
hipError_t launch_w8a8_fp8_group(const GemmParams&, hipStream_t) STUB()
hipError_t launch_f8f6_gemm(const GemmParams&, hipStream_t) STUB()
hipError_t launch_w4a4_lut(const GemmParams&, hipStream_t) STUB()
hipError_t launch_w4a4_swiglu(const GemmParams&, const GluParams&, hipStream_t) STUB()
hipError_t launch_search(const SearchInput&, const SearchCandidates&, double, double, void*, uint8_t*, int64_t, void*,
                         hipStream_t) STUB()
void set_split_limit(int64_t) {}
size_t search_workspace_bytes(int64_t ntensors, int64_t numel, int32_t nformats, int32_t nclips) {
    return (size_t)(ntensors * nformats * nclips) * 4096 + (size_t)numel / 64 + 256;
}
hipError_t search_scratch(void** ptr) {
    *ptr = reinterpret_cast<void*>(0x7000000);
    return hipSuccess;
}
}  // namespace fp4

static int g_fail = 0;
static void expect(const char* what, fp4_status got, fp4_status want) {
    const char* msg = fp4_last_error();
    if (std::strlen(msg) > 4096) std::abort();
    if (got != want) {
        std::printf("FAIL %s: got %d (%s), want %d; last error: %s\n", what, got, fp4_status_string(got), want, msg);
        g_fail = 1;
    }
}

static void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }
static fp4_grid mini(int e, int m) {
    fp4_grid g;
    std::memset(&g, 0, sizeof g);
    g.kind = FP4_GRID_MINIFLOAT;
    g.e = e;
    g.m = m;
    return g;
}
static fp4_grid lut() {
    fp4_grid g;
    std::memset(&g, 0, sizeof g);
    g.kind = FP4_GRID_LUT16;
    for (int i = 0; i < 16; i++) g.lut[i] = (i - 7.5f) / 8.0f;
    return g;
}
static fp4_grid two_mode() {
    fp4_grid g;
    std::memset(&g, 0, sizeof g);
    g.kind = FP4_GRID_TWO_MODE;
    return g;
}
static fp4_gran gran(int mode, int group = 0, int sd = FP4_F32) {
    fp4_gran g;
    std::memset(&g, 0, sizeof g);
    g.mode = mode;
    g.group = group;
    g.scale_dtype = sd;
    return g;
}

int main() {
    for (int s = -2; s < 8; s++) (void)std::strlen(fp4_status_string(s));

    // NF4 grid (host arithmetic)
    expect("nf4 null", fp4_nf4_grid(nullptr), FP4_ERR_INVALID_ARG);
    fp4_grid nf4;
    expect("nf4", fp4_nf4_grid(&nf4), FP4_OK);
    if (nf4.lut[0] != -1.0f || nf4.lut[15] != 1.0f) g_fail = 1;

    // calibrate
    float* amax = static_cast<float*>(P(0x100000));
    expect("calibrate null", fp4_calibrate(nullptr, FP4_F32, 4, 64, 64, FP4_REDUCE_TENSOR, 0, 0, amax, nullptr),
           FP4_ERR_INVALID_ARG);
    for (int red = 0; red < 3; red++)
        for (int dt : {FP4_F32, FP4_BF16})
            expect("calibrate", fp4_calibrate(P(0x200000), dt, 37, 256, 264, red, red == 2 ? 64 : 0, red == 1 ? 9 : 0,
                                              amax, nullptr), FP4_OK);
    expect("calibrate bad reduce", fp4_calibrate(P(0x200000), FP4_F32, 4, 64, 64, 7, 0, 0, amax, nullptr),
           FP4_ERR_INVALID_ARG);

    // quantize / dequantize over grids and granularities
    const fp4_grid grids[] = {mini(2, 1), mini(1, 2), mini(3, 0), nf4, lut(), two_mode(), mini(4, 3), mini(5, 2),
                              mini(2, 3), mini(3, 2)};
    const fp4_gran grans[] = {gran(FP4_SCALE_TENSOR), gran(FP4_SCALE_ROW), gran(FP4_SCALE_ROW, 0, FP4_F16),
                              gran(FP4_SCALE_GROUP, 128, FP4_F16), gran(FP4_SCALE_GROUP, 64), gran(FP4_SCALE_GROUP, 8)};
    for (const fp4_grid& g : grids)
        for (const fp4_gran& gr : grans)
            for (int dt : {FP4_F32, FP4_BF16}) {
                const int bits = g.kind == FP4_GRID_MINIFLOAT && g.e + g.m == 7 ? 8
                                 : g.kind == FP4_GRID_MINIFLOAT && g.e + g.m == 5 ? 6 : 4;
                const int64_t cols = 1024, ldp = cols * bits / 8;
                fp4_status st = fp4_quantize_pack(P(0x300000), dt, 33, cols, cols, g, gr, nullptr, nullptr, nullptr,
                                                  static_cast<uint8_t*>(P(0x400000)), ldp, P(0x500000), nullptr);
                if (st != FP4_OK && st != FP4_ERR_UNSUPPORTED) expect("quantize", st, FP4_OK);
                st = fp4_dequantize(static_cast<uint8_t*>(P(0x400000)), 33, cols, ldp, g, gr, P(0x500000), nullptr,
                                    static_cast<float*>(P(0x600000)), cols, nullptr);
                if (st != FP4_OK && st != FP4_ERR_UNSUPPORTED) expect("dequantize", st, FP4_OK);
            }
    expect("quantize null", fp4_quantize_pack(nullptr, FP4_F32, 1, 8, 8, mini(2, 1), gran(0), nullptr, nullptr,
                                              nullptr, static_cast<uint8_t*>(P(0x400000)), 4, P(0x500000), nullptr),
           FP4_ERR_INVALID_ARG);
    fp4_grid bad = mini(2, 1);
    bad.reserved = 3;
    expect("quantize reserved", fp4_quantize_pack(P(0x300000), FP4_F32, 1, 8, 8, bad, gran(0), nullptr, nullptr,
                                                  nullptr, static_cast<uint8_t*>(P(0x400000)), 4, P(0x500000),
                                                  nullptr), FP4_ERR_INVALID_ARG);
    fp4_grid unsorted = lut();
    unsorted.lut[3] = 5.0f;
    expect("quantize unsorted lut", fp4_quantize_pack(P(0x300000), FP4_F32, 1, 64, 64, unsorted, gran(0), nullptr,
                                                      nullptr, nullptr, static_cast<uint8_t*>(P(0x400000)), 32,
                                                      P(0x500000), nullptr), FP4_ERR_INVALID_ARG);

    // pre-shift
    expect("preshift", fp4_preshift_weights(static_cast<const float*>(P(0x700000)), 256, 512, 512,
                                            static_cast<const float*>(P(0x800000)), mini(2, 1), mini(2, 1),
                                            gran(FP4_SCALE_ROW), static_cast<int8_t*>(P(0x900000)),
                                            static_cast<float*>(P(0xa00000)), static_cast<uint8_t*>(P(0xb00000)), 256,
                                            P(0xc00000), nullptr), FP4_OK);
    expect("preshift nf4", fp4_preshift_weights(static_cast<const float*>(P(0x700000)), 256, 512, 512,
                                                static_cast<const float*>(P(0x800000)), mini(2, 1), nf4,
                                                gran(FP4_SCALE_GROUP, 64), static_cast<int8_t*>(P(0x900000)),
                                                static_cast<float*>(P(0xa00000)), static_cast<uint8_t*>(P(0xb00000)),
                                                256, P(0xc00000), nullptr), FP4_OK);

    // search
    const int32_t fmts[] = {1, 2, 2, 1, 3, 0};
    const size_t ws = fp4_search_workspace_size(4, 4096, 3, 100);
    expect("search", fp4_search_format(static_cast<const float*>(P(0xd00000)), 4, 4096, fmts, 3, 100, 0.5f, 1.0f,
                                       static_cast<fp4_search_result*>(P(0xe00000)),
                                       static_cast<uint8_t*>(P(0xf00000)), P(0x1000000), ws, nullptr), FP4_OK);
    expect("search small workspace", fp4_search_format(static_cast<const float*>(P(0xd00000)), 4, 4096, fmts, 3, 100,
                                                       0.5f, 1.0f, static_cast<fp4_search_result*>(P(0xe00000)),
                                                       static_cast<uint8_t*>(P(0xf00000)), P(0x1000000), ws - 1,
                                                       nullptr), FP4_ERR_WORKSPACE);
    const int32_t bad_fmts[] = {0, 3};
    expect("search bad format", fp4_search_format(static_cast<const float*>(P(0xd00000)), 4, 4096, bad_fmts, 1, 100,
                                                  0.5f, 1.0f, static_cast<fp4_search_result*>(P(0xe00000)),
                                                  static_cast<uint8_t*>(P(0xf00000)), P(0x1000000), ws, nullptr),
           FP4_ERR_UNSUPPORTED);
    expect("search static", fp4_search_format_static(static_cast<const float*>(P(0xd00000)), 2, 4096, fmts, 3, 10,
                                                     0.5f, 1.0f, static_cast<fp4_search_result*>(P(0xe00000)),
                                                     static_cast<uint8_t*>(P(0xf00000)), nullptr), FP4_OK);
    for (int unit : {FP4_SCALE_TENSOR, FP4_SCALE_ROW}) {
        const size_t wsa = fp4_search_workspace_size(unit == FP4_SCALE_ROW ? 64 : 1, 64 * 512, 3, 100);
        expect("search activations", fp4_search_activations(P(0x1100000), FP4_BF16, 64, 512, 512, unit, 32, fmts, 3,
                                                            100, 0.5f, 1.0f,
                                                            static_cast<fp4_search_result*>(P(0xe00000)),
                                                            static_cast<uint8_t*>(P(0xf00000)), 256, P(0x1000000),
                                                            wsa, nullptr), FP4_OK);
    }

    // gemm: W4A16 and W4A4 over grids, scale modes and split limits
    fp4_gemm_desc d;
    expect("gemm null", fp4_gemm(nullptr, nullptr), FP4_ERR_INVALID_ARG);
    for (int64_t lim : {(int64_t)0, (int64_t)-5, (int64_t)1 << 20, (int64_t)1 << 40}) {
        fp4_set_split_limit(lim);
        for (int a_kind : {FP4_F32, FP4_BF16, FP4_PACKED})
            for (const fp4_grid& wg : grids)
                for (const fp4_grid& ag : {mini(2, 1), mini(1, 2), mini(3, 0), mini(4, 3), mini(2, 3)})
                    for (int mode : {FP4_SCALE_TENSOR, FP4_SCALE_ROW, FP4_SCALE_GROUP})
                        for (int M : {1, 16, 300}) {
                            std::memset(&d, 0, sizeof d);
                            const int wbits = wg.kind == FP4_GRID_MINIFLOAT && wg.e + wg.m == 7 ? 8
                                              : wg.kind == FP4_GRID_MINIFLOAT && wg.e + wg.m == 5 ? 6 : 4;
                            const int abits = ag.e + ag.m == 7 ? 8 : ag.e + ag.m == 5 ? 6 : 4;
                            d.M = M;
                            d.N = 520;
                            d.K = 1024;
                            d.a_kind = a_kind;
                            d.a_scale_mode = (a_kind == FP4_PACKED && M == 300) ? FP4_SCALE_ROW : FP4_SCALE_TENSOR;
                            d.a = P(0x2000000);
                            d.lda = a_kind == FP4_PACKED ? d.K * abits / 8 : d.K;
                            d.a_grid = ag;
                            d.a_scale = static_cast<const float*>(P(0x2100000));
                            d.w = static_cast<const uint8_t*>(P(0x2200000));
                            d.ldw = d.K * wbits / 8;
                            d.w_grid = wg;
                            d.w_gran = mode == FP4_SCALE_GROUP ? gran(mode, 128, FP4_F16) : gran(mode);
                            d.w_scales = P(0x2300000);
                            d.y = P(0x2400000);
                            d.ldy = d.N;
                            d.y_dtype = M == 16 ? FP4_F32 : FP4_BF16;
                            const fp4_status st = fp4_gemm(&d, nullptr);
                            if (st != FP4_OK && st != FP4_ERR_UNSUPPORTED) expect("gemm", st, FP4_OK);
                        }
    }
    fp4_set_split_limit(0);
    std::memset(&d, 0, sizeof d);
    d.M = 4; d.N = 64; d.K = 256; d.a_kind = FP4_PACKED; d.a = P(0x2000000); d.lda = 136; d.a_grid = mini(2, 1);
    d.a_scale = static_cast<const float*>(P(0x2100000)); d.w = static_cast<const uint8_t*>(P(0x2200000));
    d.ldw = 128; d.w_grid = mini(2, 1); d.w_gran = gran(FP4_SCALE_ROW); d.w_scales = P(0x2300000);
    d.y = P(0x2400000); d.ldy = 64; d.y_dtype = FP4_BF16;
    expect("gemm lda alignment", fp4_gemm(&d, nullptr), FP4_ERR_ALIGNMENT);
    d.lda = 128;
    d.K = 200000;
    d.lda = d.ldw = 100000;
    expect("gemm K too large", fp4_gemm(&d, nullptr), FP4_ERR_UNSUPPORTED);

    // fused SwiGLU
    fp4_swiglu_desc sd;
    std::memset(&sd, 0, sizeof sd);
    sd.M = 64; sd.N = 256; sd.K = 512; sd.a = static_cast<const uint8_t*>(P(0x3000000)); sd.lda = 256;
    sd.a_scale = static_cast<const float*>(P(0x3100000)); sd.w_gate = static_cast<const uint8_t*>(P(0x3200000));
    sd.w_up = static_cast<const uint8_t*>(P(0x3300000)); sd.ldw = 256; sd.s_gate = static_cast<const float*>(P(0x3400000));
    sd.s_up = static_cast<const float*>(P(0x3500000)); sd.out_scale = static_cast<const float*>(P(0x3600000));
    sd.h_packed = static_cast<uint8_t*>(P(0x3700000)); sd.ldh = 128;
    expect("swiglu", fp4_gemm_swiglu_quant(&sd, nullptr), FP4_OK);
    sd.N = 48;
    expect("swiglu N", fp4_gemm_swiglu_quant(&sd, nullptr), FP4_ERR_UNSUPPORTED);
    expect("swiglu null", fp4_gemm_swiglu_quant(nullptr, nullptr), FP4_ERR_INVALID_ARG);

    std::printf("host layer: %d launches reached the stubs, %s\n", g_calls, g_fail ? "FAILURES" : "all statuses as expected");
    return g_fail || g_calls < 100;
}

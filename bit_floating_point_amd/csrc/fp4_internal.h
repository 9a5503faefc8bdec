// Internal declarations shared by the host layer (fp4_api.cpp) and the HIP kernels.
// Nothing here is part of the public ABI (include/fp4.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4 {

// A 4-bit grid as the kernels see it.  Codes come from a compare ladder against the
// midpoints between neighbouring grid values ([FP4-LLM] "compare and quantize",
// eq. (5)): code = number of midpoints below y, where a value exactly on the
// midpoint between codes i-1 and i counts for the even one of the two.
//   kind 0 (minifloat, sign-magnitude): val[0..7] magnitudes, thr[0..6] midpoints,
//          applied to |y|; the sign bit of y becomes bit 3.
//   kind 1 (LUT16, signed):             val[0..15], thr[0..14], applied to y.
//   kind 2 (two-mode, per group):       E2M1 val[0..7] / thr[0..6] (mode 0) and E1M2
//          val[8..15] / thr[7..13] (mode 1); the mode is the sign bit of the group scale.
//   bits 8 (kind 0, e + m == 7): the OCP FP8 formats E4M3 / E5M2, one code per byte
//          (sign in bit 7), rounded arithmetically; val/thr unused.
struct QGrid {
    int32_t kind;
    int32_t e, m;
    int32_t is_e2m1;   // minifloat E2M1: the gfx950 FP4 converts apply
    float qmax;        // largest magnitude
    float val[16];
    float thr[15];
    int32_t bits;      // 4, or 8 for FP8
};

struct QuantParams {
    const void* x;
    int64_t ldx;           // elements
    int32_t x_bf16;
    int32_t mode;          // 0 tensor, 1 row, 2 group
    int64_t rows, cols;
    uint8_t* packed;
    int64_t ldp;           // bytes
    int32_t group;
    int32_t scale_f16;
    const float* amax_in;        // per scale unit, or null
    const float* tensor_scale;   // tensor mode: fixed scale s, or null
    const float* tensor_amax;    // tensor mode: amax (when tensor_scale is null)
    void* scales_out;            // per unit (f32/f16), may be null in tensor mode
    const int8_t* col_shift;     // or null
    int32_t shift_sign;          // -1: multiplier r * 2^-k ; +1: input x * 2^k
    int32_t vec;                 // 16-byte vector path allowed
    QGrid g;
};

hipError_t launch_fill_zero_u32(uint32_t* p, int64_t n, hipStream_t s);
hipError_t launch_calibrate(const void* x, int x_bf16, int64_t rows, int64_t cols,
                            int64_t ld, int reduce, int group, float* out, int vec,
                            hipStream_t s);
hipError_t launch_quantize(const QuantParams& p, hipStream_t s);
hipError_t launch_tensor_scale_finalize(const float* amax, float* scales_out, float qmax, hipStream_t s);
hipError_t launch_dequantize(const uint8_t* packed, int64_t rows, int64_t cols, int64_t ldp,
                             const QGrid& g, int mode, int group, const void* scales,
                             int scale_f16, const int8_t* col_shift, float* out,
                             int64_t ldo, hipStream_t s);
hipError_t launch_preshift_factors(const float* chan_amax, int64_t k, float act_qmax,
                                   int8_t* shift_out, float* act_scale_out, hipStream_t s);

// quantized GEMMs (Y = X W^T)
struct GemmParams {
    int64_t M, N, K;
    int32_t a_kind;       // 0 f32, 1 bf16, 3 packed
    const void* a;
    int64_t lda;
    QGrid ag;
    const float* a_scale;
    int32_t a_row;        // packed activations: one scale per row (token) of A
    const uint8_t* w;
    int64_t ldw;
    QGrid wg;
    int32_t w_mode;       // 0 tensor, 1 row, 2 group
    int32_t w_group;
    int32_t w_scale_f16;
    const void* w_scales;
    void* y;
    int64_t ldy;
    int32_t y_bf16;
};
hipError_t launch_w4a16_mfma(const GemmParams& p, hipStream_t s);
hipError_t launch_w4a16_valu(const GemmParams& p, hipStream_t s);
hipError_t launch_w4a16_two_mode(const GemmParams& p, hipStream_t s);  // M <= 16, bf16, group 128
hipError_t launch_w8a16_small(const GemmParams& p, hipStream_t s);     // FP8 weights, M <= 16, bf16
hipError_t launch_w4a4_fp4(const GemmParams& p, hipStream_t s);
void set_split_limit(int64_t bytes);  // 0: the 32-bit buffer range
hipError_t launch_w8a8_fp8(const GemmParams& p, hipStream_t s);  // FP8 E4M3 x E4M3
hipError_t launch_w8a8_e5m2(const GemmParams& p, hipStream_t s); // FP8 E5M2 x E5M2
hipError_t launch_w8a8_mixed(const GemmParams& p, hipStream_t s); // E4M3 x E5M2 either way
bool w6a6_fits(const GemmParams& p);                                // FP6 x FP6, one format
hipError_t launch_w6a6_fp6(const GemmParams& p, hipStream_t s);
bool w8a8_group_fits(const GemmParams& p);                          // E4M3 x E4M3, group-128 scales
hipError_t launch_w8a8_fp8_group(const GemmParams& p, hipStream_t s);
// every other pair of FP8 (E4M3, E5M2) / FP6 (E2M3, E3M2) operands, W6A6 among them
int f8f6_format_code(const QGrid& g);  // MFMA operand format, or -1
hipError_t launch_f8f6_gemm(const GemmParams& p, hipStream_t s);
hipError_t launch_w4a4_lut(const GemmParams& p, hipStream_t s);
// W4A4 gate/up products with SwiGLU and the next layer's activation quantization in
// the epilogue: p.w / p.w_scales are the gate weights and row scales, p.y the E2M1 codes
struct GluParams {
    const uint8_t* w_up;
    const float* s_up;
    const float* out_scale;   // next layer's per-tensor activation scale
    const int8_t* out_shift;  // its per-column shifts, or null
};
hipError_t launch_w4a4_swiglu(const GemmParams& p, const GluParams& gp, hipStream_t s);

// format search
struct SearchCandidates {
    int32_t nformats, nclips;
    int32_t fmt_e[8], fmt_m[8];
    float fmt_qmax[8];
};
size_t search_workspace_bytes(int64_t ntensors, int64_t numel, int32_t nformats,
                              int32_t nclips);
// search input: a row-major [rows, cols] matrix; units are its rows (per_row_units) or
// its first unit_rows rows as one unit (then every row is packed with that winner)
struct SearchInput {
    const void* x;
    int32_t bf16;
    int32_t per_row_units;
    int64_t ld;  // elements
    int64_t rows, cols;
    int64_t unit_rows;
};
hipError_t launch_search(const SearchInput& in, const SearchCandidates& c, double clip_lo, double clip_hi,
                         void* results, uint8_t* packed, int64_t ldp, void* ws, hipStream_t s);
// The allocation-free search's scratch: a file-scope device array of this many bytes,
// one copy per GPU; search_scratch() returns the current device's copy (looked up on the
// first call on each device).
constexpr size_t kSearchScratchBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;
hipError_t search_scratch(void** ptr);

}  // namespace fp4

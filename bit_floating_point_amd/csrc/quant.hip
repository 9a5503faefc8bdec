// Calibration, quantize + pack, dequantize and the pre-shift factors for gfx950.
//
// Method ([FP4-LLM] = "首个支持4-bit浮点量化的LLM来了" page, 811yy.cn):
//   scale and clip (eqs. (2)-(3)): s = amax / Qmax, y = x * (1/s) clipped to +-Qmax;
//   compare and quantize (eq. (5)): nearest grid point, ties to the even code;
//   pre-shifted exponent bias: per-channel maxima -> per-tensor a times 2^k.
// Two 4-bit codes per byte ("为什么我们需要4-bit浮点量化" page, section 2.2).  Also the
// two-mode grid ("HiFloat4格式" page, section 2.1: E2M1 or E1M2 per group, one control
// bit) and the OCP FP8 / FP6 grids (the FP8 key layers and 8/6/4-bit precision of the
// [FP4-LLM] page), one code per byte or four codes in three bytes.
//
// Memory path: every thread owns 8 consecutive elements of a row (one 16-byte load
// for bf16, two for f32) and writes their 4 packed bytes with one 32-bit store, so a
// wavefront moves 1-2 KiB per load instruction, fully coalesced.  Scale reductions
// are lane shuffles inside the wavefront (group <= 512) or an LDS reduction over the
// workgroup (per-row scales).  HBM-bound: no LDS staging, no re-read except the second
// pass over one row in per-row mode (L2-resident).
#include "fp4_device.h"

namespace fp4 {

constexpr int kThreads = 256;
constexpr int kChunk = kThreads * 8;  // elements of a row per workgroup pass

__device__ __forceinline__ float max_abs8(const float v[8]) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) m = fmaxf(m, fabsf(v[i]));
    return m;
}

// Max over the aligned 16-lane group (one 128-element group of 8 elements per lane)
// with DPP lane permutes, all in VALU: swap neighbours, swap pairs, mirror within 8,
// mirror within 16.
__device__ __forceinline__ float dpp_max16(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
    return v;
}

// Max over the whole wavefront: 16-lane groups by DPP, then the four group maxima read
// out with readlane (the result is uniform).
__device__ __forceinline__ float dpp_wave_max(float v) {
    v = dpp_max16(v);
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

__global__ void fill_zero_u32_kernel(uint32_t* p, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

hipError_t launch_fill_zero_u32(uint32_t* p, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(fill_zero_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

// ------------------------------------------------------------------ calibrate ----
// TENSOR: one workgroup per (row, 2048-column chunk); wave max -> atomicMax on the
// float bit pattern (|x| >= 0, so unsigned order equals float order; max is exact and
// order-free, so the result does not depend on the launch geometry).
template <bool VEC, bool BF16>
__global__ void __launch_bounds__(kThreads) amax_tensor_kernel(const void* x, int64_t cols, int64_t ld, int64_t chunks,
                                                               float* out) {
    int64_t b = blockIdx.x;
    int64_t row = b / chunks;
    int64_t col = (b % chunks) * kChunk + threadIdx.x * 8;
    const char* rp = reinterpret_cast<const char*>(x) + row * ld * (BF16 ? 2 : 4);
    float v[8];
    load8<VEC, BF16>(rp, col, cols, v);
    float m = dpp_wave_max(max_abs8(v));
    if ((threadIdx.x & 63) == 0) atomicMax(reinterpret_cast<unsigned int*>(out), __float_as_uint(m));
}

// COLUMN: per-column max over the first `rows` rows.  A thread owns 8 columns and a
// strip of 32 rows (all 32 loads issued before the first max); one atomicMax per column
// per strip.
template <bool VEC, bool BF16>
__global__ void __launch_bounds__(kThreads) amax_column_kernel(const void* x, int64_t rows, int64_t cols, int64_t ld,
                                                               float* out) {
    constexpr int kStrip = 32;
    int64_t col = (int64_t)blockIdx.x * kChunk + threadIdx.x * 8;
    int64_t r0 = (int64_t)blockIdx.y * kStrip;
    if (col >= cols) return;
    Raw8 raw[kStrip];
#pragma unroll
    for (int r = 0; r < kStrip; r++) {
        int64_t rr = r0 + r < rows ? r0 + r : rows - 1;  // a repeated row does not change a max
        raw[r] = load_raw8<VEC, BF16>(reinterpret_cast<const char*>(x) + rr * ld * (BF16 ? 2 : 4), col, cols);
    }
    float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < kStrip; r++) {
        float v[8];
        raw8_to_float<BF16>(raw[r], v);
#pragma unroll
        for (int i = 0; i < 8; i++) m[i] = fmaxf(m[i], fabsf(v[i]));
    }
#pragma unroll
    for (int i = 0; i < 8; i++)
        if (col + i < cols) atomicMax(reinterpret_cast<unsigned int*>(out) + col + i, __float_as_uint(m[i]));
}

// ROW_GROUP: per (row, group) max; a group spans group/8 aligned lanes.
template <bool VEC, bool BF16>
__global__ void __launch_bounds__(kThreads) amax_rowgroup_kernel(const void* x, int64_t cols, int64_t ld,
                                                                 int64_t chunks, int group, float* out) {
    int64_t b = blockIdx.x;
    int64_t row = b / chunks;
    int64_t col = (b % chunks) * kChunk + threadIdx.x * 8;
    const char* rp = reinterpret_cast<const char*>(x) + row * ld * (BF16 ? 2 : 4);
    float v[8];
    load8<VEC, BF16>(rp, col, cols, v);
    int lanes = group >> 3;
    float m = group_max(max_abs8(v), lanes);
    if (col < cols && ((threadIdx.x & (lanes - 1)) == 0)) out[row * (cols / group) + col / group] = m;
}

template <bool VEC, bool BF16>
static void calibrate_launch(const void* x, int64_t rows, int64_t cols, int64_t ld, int reduce, int group, float* out,
                             hipStream_t s) {
    int64_t chunks = (cols + kChunk - 1) / kChunk;
    if (reduce == 0) {
        hipLaunchKernelGGL((amax_tensor_kernel<VEC, BF16>), dim3((unsigned)(rows * chunks)), dim3(kThreads), 0, s, x,
                           cols, ld, chunks, out);
    } else if (reduce == 1) {
        dim3 grid((unsigned)chunks, (unsigned)((rows + 31) / 32));
        hipLaunchKernelGGL((amax_column_kernel<VEC, BF16>), grid, dim3(kThreads), 0, s, x, rows, cols, ld, out);
    } else {
        hipLaunchKernelGGL((amax_rowgroup_kernel<VEC, BF16>), dim3((unsigned)(rows * chunks)), dim3(kThreads), 0, s, x,
                           cols, ld, chunks, group, out);
    }
}

hipError_t launch_calibrate(const void* x, int x_bf16, int64_t rows, int64_t cols, int64_t ld, int reduce, int group,
                            float* out, int vec, hipStream_t s) {
    if (reduce == 0 || reduce == 1) {
        hipError_t e = launch_fill_zero_u32(reinterpret_cast<uint32_t*>(out), reduce == 0 ? 1 : cols, s);
        if (e != hipSuccess) return e;
    }
    if (rows == 0 || cols == 0) return hipSuccess;
    if (vec && x_bf16) calibrate_launch<true, true>(x, rows, cols, ld, reduce, group, out, s);
    else if (vec) calibrate_launch<true, false>(x, rows, cols, ld, reduce, group, out, s);
    else if (x_bf16) calibrate_launch<false, true>(x, rows, cols, ld, reduce, group, out, s);
    else calibrate_launch<false, false>(x, rows, cols, ld, reduce, group, out, s);
    return hipGetLastError();
}

// ------------------------------------------------------------------ quantize -----
__device__ __forceinline__ void store_codes(uint8_t* prow, int64_t col, int64_t cols, uint32_t w, bool vec) {
    if (vec && col + 8 <= cols) {
        *reinterpret_cast<uint32_t*>(prow + col / 2) = w;
    } else {
        for (int j = 0; j < 4; j++)
            if (col + 2 * j < cols) prow[col / 2 + j] = (uint8_t)(w >> (8 * j));
    }
}

// Column shifts of the 8 elements at col, raw (8 int8 in two words).
template <bool VEC>
__device__ __forceinline__ uint2 load_shift8(const QuantParams& p, int64_t col) {
    if (VEC) return col < p.cols ? *reinterpret_cast<const uint2*>(p.col_shift + col) : make_uint2(0, 0);
    uint32_t w[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 8; i++)
        if (col + i < p.cols) w[i >> 2] |= (uint32_t)(uint8_t)p.col_shift[col + i] << (8 * (i & 3));
    return make_uint2(w[0], w[1]);
}

__device__ __forceinline__ int shift_of(uint2 k, int i) {
    return (int)(int8_t)((i < 4 ? k.x : k.y) >> (8 * (i & 3)));
}

// Input side of the pre-shift (weights): x' = x * 2^k, exact.
__device__ __forceinline__ void shift_inputs(float v[8], uint2 k) {
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = ldexpf(v[i], shift_of(k, i));
}

// y = fl32(x * r), or fl32(x * (r * 2^-k)) with the activation-side pre-shift.
__device__ __forceinline__ void scale_values(float v[8], float r, bool shifted, uint2 k) {
    if (shifted) {
#pragma unroll
        for (int i = 0; i < 8; i++) v[i] = v[i] * ldexpf(r, -shift_of(k, i));
    } else {
#pragma unroll
        for (int i = 0; i < 8; i++) v[i] = v[i] * r;
    }
}

__device__ __forceinline__ void store_scale(const QuantParams& p, int64_t unit, float s) {
    if (p.scale_f16) reinterpret_cast<__half*>(p.scales_out)[unit] = __float2half_rn(s);
    else reinterpret_cast<float*>(p.scales_out)[unit] = s;
}

// TENSOR and GROUP modes.  The (row, 2048-column chunk) units are processed U per
// workgroup: every load of the U units (values and shifts) is issued before any
// arithmetic, so a lane has U x 16 B (bf16) or U x 32 B (f32) in flight.
template <bool VEC, bool BF16, int U>
__global__ void __launch_bounds__(kThreads) quantize_chunk_kernel(QuantParams p, int64_t chunks, int64_t nunits) {
    const bool has_k = p.col_shift != nullptr;
    Raw8 raw[U];
    uint2 kk[U];
    int64_t row[U], col[U];
#pragma unroll
    for (int i = 0; i < U; i++) {
        int64_t u = (int64_t)blockIdx.x * U + i;
        if (u >= nunits) u = nunits - 1;  // a duplicate of the last unit writes the same bytes
        row[i] = u / chunks;
        col[i] = (u % chunks) * kChunk + threadIdx.x * 8;
        raw[i] = load_raw8<VEC, BF16>(reinterpret_cast<const char*>(p.x) + row[i] * p.ldx * (BF16 ? 2 : 4), col[i],
                                      p.cols);
        kk[i] = has_k ? load_shift8<VEC>(p, col[i]) : make_uint2(0, 0);
    }
    float tensor_r = 0.0f;
    if (p.mode == 0) {
        float s = p.tensor_scale ? p.tensor_scale[0] : p.tensor_amax[0] / p.g.qmax;
        tensor_r = recip_or_zero(s);
        if (blockIdx.x == 0 && threadIdx.x == 0 && p.tensor_scale && p.scales_out)
            reinterpret_cast<float*>(p.scales_out)[0] = s;
    }
#pragma unroll
    for (int i = 0; i < U; i++) {
        float v[8];
        raw8_to_float<BF16>(raw[i], v);
        if (has_k && p.shift_sign > 0) shift_inputs(v, kk[i]);
        float r = tensor_r;
        if (p.mode != 0) {
            int lanes = p.group >> 3;
            int64_t unit = row[i] * (p.cols / p.group) + col[i] / p.group;
            float amax;
            if (p.amax_in) amax = (col[i] < p.cols) ? p.amax_in[unit] : 0.0f;
            else amax = group_max(max_abs8(v), lanes);
            float s = amax / p.g.qmax;
            if (p.scale_f16) s = round_f16(s);
            r = recip_or_zero(s);
            if (col[i] < p.cols && (threadIdx.x & (lanes - 1)) == 0 && p.scales_out) store_scale(p, unit, s);
        }
        scale_values(v, r, has_k && p.shift_sign < 0, kk[i]);
        uint32_t w = pack8(v, p.g);
        if (col[i] < p.cols) store_codes(p.packed + row[i] * p.ldp, col[i], p.cols, w, VEC);
    }
}

// the 8 codes of the scaled values y at columns col .. col + 7 of a row on an FP8 grid
// (8 bytes) or an FP6 grid (6 bytes as three 16-bit words; cols is a multiple of 8, so a
// lane's 6 bytes are whole)
template <bool VEC, int E, int M>
__device__ __forceinline__ void store_wide8(const QuantParams& p, int64_t row, int64_t col, const float y[8]) {
    if (E + M == 7) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            lo |= wide_code<E, M>(y[k]) << (8 * k);
            hi |= wide_code<E, M>(y[k + 4]) << (8 * k);
        }
        if (col < p.cols) {
            uint8_t* dst = p.packed + row * p.ldp + col;
            if (VEC) *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
            else
                for (int k = 0; k < 8 && col + k < p.cols; k++) dst[k] = (uint8_t)((k < 4 ? lo : hi) >> (8 * (k & 3)));
        }
    } else {
        uint64_t bits = 0;
#pragma unroll
        for (int k = 0; k < 8; k++) bits |= (uint64_t)wide_code<E, M>(y[k]) << (6 * k);
        if (col < p.cols) {
            uint16_t* dst = reinterpret_cast<uint16_t*>(p.packed + row * p.ldp + col / 8 * 6);
            dst[0] = (uint16_t)bits;
            dst[1] = (uint16_t)(bits >> 16);
            dst[2] = (uint16_t)(bits >> 32);
        }
    }
}

// TENSOR and GROUP modes with an OCP 8-bit (one code per byte) or 6-bit (a bit stream,
// four codes in three bytes) grid: the same units and scales as quantize_chunk_kernel,
// codes by wide_code; a lane stores its 8 codes as 8 bytes or as three 16-bit words.
template <bool VEC, bool BF16, int U, int E, int M>
__global__ void __launch_bounds__(kThreads) quantize_wide_kernel(QuantParams p, int64_t chunks, int64_t nunits) {
    Raw8 raw[U];
    int64_t row[U], col[U];
    uint2 kk[U];
    const bool has_k = p.col_shift != nullptr;
#pragma unroll
    for (int i = 0; i < U; i++) {
        int64_t u = (int64_t)blockIdx.x * U + i;
        if (u >= nunits) u = nunits - 1;  // a duplicate of the last unit writes the same bytes
        row[i] = u / chunks;
        col[i] = (u % chunks) * kChunk + threadIdx.x * 8;
        raw[i] = load_raw8<VEC, BF16>(reinterpret_cast<const char*>(p.x) + row[i] * p.ldx * (BF16 ? 2 : 4), col[i],
                                      p.cols);
        kk[i] = has_k ? load_shift8<VEC>(p, col[i]) : make_uint2(0, 0);
    }
    float tensor_r = 0.0f;
    if (p.mode == 0) {
        float s = p.tensor_scale ? p.tensor_scale[0] : p.tensor_amax[0] / p.g.qmax;
        tensor_r = recip_or_zero(s);
        if (blockIdx.x == 0 && threadIdx.x == 0 && p.tensor_scale && p.scales_out)
            reinterpret_cast<float*>(p.scales_out)[0] = s;
    }
#pragma unroll
    for (int i = 0; i < U; i++) {
        float v[8];
        raw8_to_float<BF16>(raw[i], v);
        if (has_k && p.shift_sign > 0) shift_inputs(v, kk[i]);  // pre-shifted weights W' = W 2^k
        float r = tensor_r;
        if (p.mode != 0) {
            const int lanes = p.group >> 3;
            const int64_t unit = row[i] * (p.cols / p.group) + col[i] / p.group;
            float amax;
            if (p.amax_in) amax = (col[i] < p.cols) ? p.amax_in[unit] : 0.0f;
            else amax = group_max(max_abs8(v), lanes);
            float s = amax / p.g.qmax;
            if (p.scale_f16) s = round_f16(s);
            r = recip_or_zero(s);
            if (col[i] < p.cols && (threadIdx.x & (lanes - 1)) == 0 && p.scales_out) store_scale(p, unit, s);
        }
        scale_values(v, r, has_k && p.shift_sign < 0, kk[i]);  // activations: r 2^-k per column
        store_wide8<VEC, E, M>(p, row[i], col[i], v);
    }
}

// GROUP mode, group 128, f32 input, on an OCP 8-bit or 6-bit grid: the load pattern of
// quantize_e2m1_g128_f32_kernel (wavefront w of a (row, 4096-column) unit takes columns
// c0 + 512 w + 256 h + 4 l .. + 3 in its load h, every load instruction 1 KiB contiguous,
// a 128-element group is 32 lanes of one load), codes by wide_code.  FP8: a lane stores
// its 4 codes as one 4-byte word.  FP6: a lane's 4 codes are 24 bits; a DPP swap gives
// each even lane its odd neighbour's 24 bits and the even lane stores the pair's 6 bytes
// as three 16-bit words.  Loads and code stores are nontemporal.  The arithmetic is that
// of quantize_wide_kernel.
template <int E, int M>
__global__ void __launch_bounds__(512) quantize_wide_g128_f32_kernel(QuantParams p, int chunks) {
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = blockIdx.x / chunks;
    const int64_t c0 = (int64_t)(blockIdx.x - row * chunks) * 4096 + wave * 512 + 4 * lane;
    const float* xr = reinterpret_cast<const float*>(p.x) + (int64_t)row * p.ldx;
    f32x4v v[2];
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const int64_t c = c0 + 256 * h;
        v[h] = c < p.cols ? __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(xr + c)) : f32x4v{0, 0, 0, 0};
    }
    const int64_t gpr = p.cols / 128;  // groups per row
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const int64_t c = c0 + 256 * h;
        float m = fmaxf(fmaxf(fabsf(v[h][0]), fabsf(v[h][1])), fmaxf(fabsf(v[h][2]), fabsf(v[h][3])));
        m = dpp_max16(m);
        m = fmaxf(m, __shfl_xor(m, 16, 64));
        float s = m / p.g.qmax;
        if (p.scale_f16) s = round_f16(s);
        const float r = recip_or_zero(s);
        uint32_t code[4];
#pragma unroll
        for (int i = 0; i < 4; i++) code[i] = wide_code<E, M>(v[h][i] * r);
        if (E + M == 7) {
            if (c < p.cols) {  // cols is a multiple of 128: the whole group is in range
                if ((lane & 31) == 0 && p.scales_out) store_scale(p, (int64_t)row * gpr + c / 128, s);
                const uint32_t w = code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
                __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(p.packed + (int64_t)row * p.ldp + c));
            }
        } else {
            const uint32_t b24 = code[0] | (code[1] << 6) | (code[2] << 12) | (code[3] << 18);
            const uint32_t nb = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)b24, 0xB1, 0xF, 0xF, false);
            if (c < p.cols) {
                if ((lane & 31) == 0 && p.scales_out) store_scale(p, (int64_t)row * gpr + c / 128, s);
                if ((lane & 1) == 0) {
                    const uint64_t bits = (uint64_t)b24 | ((uint64_t)nb << 24);
                    uint16_t* dst = reinterpret_cast<uint16_t*>(p.packed + (int64_t)row * p.ldp + c / 4 * 3);
                    __builtin_nontemporal_store((uint16_t)bits, dst);
                    __builtin_nontemporal_store((uint16_t)(bits >> 16), dst + 1);
                    __builtin_nontemporal_store((uint16_t)(bits >> 32), dst + 2);
                }
            }
        }
    }
}

// GROUP mode with the two-mode grid ([HiFloat4] section 2.1: per group the E2M1 or the
// E1M2 layout, one control bit).  Per group both candidates are formed -- s_m =
// fl32(amax / Qmax_m) (binary16-rounded for f16 scales), codes of y = fl32(x * fl32(1/s_m))
// (E2M1 by the FP4 convert, E1M2 as min(rint(4|y|), 7)) -- and the squared errors
// sum (|x| - fl32(g * s_m))^2 compared: every difference is exact in binary32 and its
// square exact in binary64, the per-element difference of the two squares is rounded
// once to binary64, summed in binary64 over each lane's 8 values and in double-double
// over the group's lanes (a butterfly that leaves the same sum in every lane).  The sign
// of the sum is the exact comparison's unless the two errors agree to about 2^-49 of
// their size.  E1M2 wins when the sum is positive; its scale is stored negated (the mode bit
// is the scale's sign bit).
template <bool VEC, bool BF16, int U>
__global__ void __launch_bounds__(kThreads) quantize_two_mode_kernel(QuantParams p, int64_t chunks, int64_t nunits) {
    Raw8 raw[U];
    int64_t row[U], col[U];
#pragma unroll
    for (int i = 0; i < U; i++) {
        int64_t u = (int64_t)blockIdx.x * U + i;
        if (u >= nunits) u = nunits - 1;  // a duplicate of the last unit writes the same bytes
        row[i] = u / chunks;
        col[i] = (u % chunks) * kChunk + threadIdx.x * 8;
        raw[i] = load_raw8<VEC, BF16>(reinterpret_cast<const char*>(p.x) + row[i] * p.ldx * (BF16 ? 2 : 4), col[i],
                                      p.cols);
    }
    const int lanes = p.group >> 3;
#pragma unroll
    for (int i = 0; i < U; i++) {
        float v[8];
        raw8_to_float<BF16>(raw[i], v);
        const int64_t unit = row[i] * (p.cols / p.group) + col[i] / p.group;
        float amax;
        if (p.amax_in) amax = (col[i] < p.cols) ? p.amax_in[unit] : 0.0f;
        else amax = group_max(max_abs8(v), lanes);
        float s0 = amax / p.g.val[7], s1 = amax / p.g.val[15];
        if (p.scale_f16) {
            s0 = round_f16(s0);
            s1 = round_f16(s1);
        }
        const float r0 = recip_or_zero(s0), r1 = recip_or_zero(s1);
        float y0[8];
#pragma unroll
        for (int k = 0; k < 8; k++) y0[k] = v[k] * r0;
        uint32_t w0 = 0;  // E2M1 codes by the FP4 convert (nearest, ties to even, +-6)
        w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, y0[0], y0[1], 1.0f, 0);
        w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, y0[2], y0[3], 1.0f, 1);
        w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, y0[4], y0[5], 1.0f, 2);
        w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, y0[6], y0[7], 1.0f, 3);
        // their magnitudes back from the codes
        float g0[8];
        {
            const auto a0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w0, 1.0f, 0);
            const auto a1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w0, 1.0f, 1);
            const auto a2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w0, 1.0f, 2);
            const auto a3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w0, 1.0f, 3);
            g0[0] = a0[0]; g0[1] = a0[1]; g0[2] = a1[0]; g0[3] = a1[1];
            g0[4] = a2[0]; g0[5] = a2[1]; g0[6] = a3[0]; g0[7] = a3[1];
        }
        uint32_t w1 = 0;
        double diff = 0.0;
#pragma unroll
        for (int k = 0; k < 8; k++) {
            const float y1 = v[k] * r1;
            const float d1c = fminf(rintf(fabsf(y1) * 4.0f), 7.0f);
            w1 |= ((__float_as_uint(y1) >> 31) << 3 | (uint32_t)d1c) << (4 * k);
            // q = fl32(g * s) is the dequantized value; |x| - q is formed in binary64, where
            // it is exact (q = 0, or |x| and q are binary32 values within a factor of 2 of
            // each other: at most 26 significant bits), and so is its square (at most 52);
            // the difference of the two squares is rounded once
            const double a = (double)fabsf(v[k]);
            const double d0 = a - (double)(fabsf(g0[k]) * s0), d1 = a - (double)((d1c * 0.25f) * s1);
            diff += d0 * d0 - d1 * d1;
        }
        DD acc{diff, 0.0};
        for (int o = 1; o < lanes; o <<= 1) acc = dd_add(acc, DD{__shfl_xor(acc.hi, o, 64), __shfl_xor(acc.lo, o, 64)});
        const bool e1m2 = acc.hi > 0.0 || (acc.hi == 0.0 && acc.lo > 0.0);
        if (col[i] < p.cols) {
            store_codes(p.packed + row[i] * p.ldp, col[i], p.cols, e1m2 ? w1 : w0, VEC);
            if ((threadIdx.x & (lanes - 1)) == 0) store_scale(p, unit, e1m2 ? -s1 : s0);
        }
    }
}

// GROUP mode with 128-element groups, the E2M1 grid, no column shifts, rows a multiple
// of 8 elements: the same arithmetic as quantize_chunk_kernel, specialised (group
// maximum by DPP instead of lane shuffles through LDS, no per-element grid dispatch).
// U (row, T*8-column chunk) units per workgroup of T threads, all loads issued first;
// one unit per workgroup measured fastest (the most workgroups in flight).
template <bool BF16, int U, int T>
__global__ void __launch_bounds__(T) quantize_e2m1_g128_kernel(QuantParams p, int chunks, int nunits) {
    Raw8 raw[U];
    int row[U], col[U];
#pragma unroll
    for (int i = 0; i < U; i++) {
        int u = blockIdx.x * U + i;
        if (u >= nunits) u = nunits - 1;  // a duplicate of the last unit writes the same bytes
        row[i] = u / chunks;
        col[i] = (u - row[i] * chunks) * (T * 8) + threadIdx.x * 8;
        raw[i] = load_raw8<true, BF16>(reinterpret_cast<const char*>(p.x) + (int64_t)row[i] * p.ldx * (BF16 ? 2 : 4),
                                       col[i], p.cols);
    }
    const int64_t gpr = p.cols / 128;  // groups per row
#pragma unroll
    for (int i = 0; i < U; i++) {
        float v[8];
        raw8_to_float<BF16>(raw[i], v);
        const float amax = dpp_max16(max_abs8(v));
        float s = amax / p.g.qmax;
        if (p.scale_f16) s = round_f16(s);
        const float r = recip_or_zero(s);
        if (col[i] < p.cols) {
            if ((threadIdx.x & 15) == 0 && p.scales_out) store_scale(p, (int64_t)row[i] * gpr + col[i] / 128, s);
#pragma unroll
            for (int k = 0; k < 8; k++) v[k] = v[k] * r;
            uint32_t w = 0;
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], 1.0f, 0);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
            *reinterpret_cast<uint32_t*>(p.packed + (int64_t)row[i] * p.ldp + col[i] / 2) = w;
        }
    }
}

// The f32 variant of quantize_e2m1_g128_kernel with every load instruction reading
// 1 KiB contiguous (whole 128-byte lines; a lane's two 16-byte pieces 1 KiB apart, not
// adjacent): wavefront w of a (row, 2048-column) unit takes columns c0 + 512 w + 256 h +
// 4 l .. + 3 in its load h = 0, 1, so a 128-element group is 32 lanes of one load (the
// group maximum: the 16-lane DPP maximum, then one exchange between the two rows of
// 16).  Loads and code stores bypass the caches' retention (nontemporal): the weights
// are read and the codes written once.  The arithmetic is that of the kernel above.
template <int T, int U>
__global__ void __launch_bounds__(T) quantize_e2m1_g128_f32_kernel(QuantParams p, int chunks, int nunits) {
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    f32x4v v[2 * U];
    int row[U];
    int64_t c0[U];
#pragma unroll
    for (int i = 0; i < U; i++) {
        int u = blockIdx.x * U + i;
        if (u >= nunits) u = nunits - 1;  // a duplicate of the last unit writes the same bytes
        row[i] = u / chunks;
        c0[i] = (int64_t)(u - row[i] * chunks) * (T * 8) + wave * 512 + 4 * lane;
        const float* xr = reinterpret_cast<const float*>(p.x) + (int64_t)row[i] * p.ldx;
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int64_t c = c0[i] + 256 * h;
            v[2 * i + h] = c < p.cols ? __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(xr + c))
                                      : f32x4v{0, 0, 0, 0};
        }
    }
    const int64_t gpr = p.cols / 128;  // groups per row
#pragma unroll
    for (int j = 0; j < 2 * U; j++) {
        const int i = j >> 1, h = j & 1;
        const int64_t c = c0[i] + 256 * h;
        float m = fmaxf(fmaxf(fabsf(v[j][0]), fabsf(v[j][1])), fmaxf(fabsf(v[j][2]), fabsf(v[j][3])));
        m = dpp_max16(m);
        m = fmaxf(m, __shfl_xor(m, 16, 64));
        float s = m / p.g.qmax;
        if (p.scale_f16) s = round_f16(s);
        const float r = recip_or_zero(s);
        if (c < p.cols) {  // cols is a multiple of 128: the whole group is in range
            if ((lane & 31) == 0 && p.scales_out) store_scale(p, (int64_t)row[i] * gpr + c / 128, s);
            uint32_t w = 0;
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[j][0] * r, v[j][1] * r, 1.0f, 0);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[j][2] * r, v[j][3] * r, 1.0f, 1);
            __builtin_nontemporal_store((uint16_t)w,
                                        reinterpret_cast<uint16_t*>(p.packed + (int64_t)row[i] * p.ldp + c / 2));
        }
    }
}

// TENSOR mode with the E2M1 grid (optionally with the activation-side column shifts
// r * 2^-k), rows a multiple of 8 elements: the arithmetic of quantize_chunk_kernel,
// specialised, one (row, T*8-column chunk) unit per workgroup.
template <bool BF16, bool SHIFT, int T>
__global__ void __launch_bounds__(T) quantize_e2m1_tensor_kernel(QuantParams p, int chunks) {
    const int u = blockIdx.x;
    const int row = u / chunks;
    const int col = (u - row * chunks) * (T * 8) + threadIdx.x * 8;
    const Raw8 raw =
        load_raw8<true, BF16>(reinterpret_cast<const char*>(p.x) + (int64_t)row * p.ldx * (BF16 ? 2 : 4), col, p.cols);
    const uint2 kk = SHIFT ? load_shift8<true>(p, col) : make_uint2(0, 0);
    const float s = p.tensor_scale ? p.tensor_scale[0] : p.tensor_amax[0] / p.g.qmax;
    const float r = recip_or_zero(s);
    if (blockIdx.x == 0 && threadIdx.x == 0 && p.tensor_scale && p.scales_out)
        reinterpret_cast<float*>(p.scales_out)[0] = s;
    if (col < p.cols) {
        float v[8];
        raw8_to_float<BF16>(raw, v);
        scale_values(v, r, SHIFT, kk);
        uint32_t w = 0;
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], 1.0f, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
        *reinterpret_cast<uint32_t*>(p.packed + (int64_t)row * p.ldp + col / 2) = w;
    }
}

// ROW mode, rows of at most R * 2048 elements: one workgroup per row, the row held in
// registers (one HBM read), max reduced across the workgroup, then quantized.
template <bool VEC, bool BF16, int R>
__global__ void __launch_bounds__(kThreads) quantize_row_reg_kernel(QuantParams p) {
    __shared__ float red[kThreads / 64];
    const int64_t row = blockIdx.x;
    const char* rp = reinterpret_cast<const char*>(p.x) + row * p.ldx * (BF16 ? 2 : 4);
    const bool has_k = p.col_shift != nullptr;
    Raw8 raw[R];
    uint2 kk[R];
#pragma unroll
    for (int c = 0; c < R; c++) {
        int64_t col = (int64_t)c * kChunk + threadIdx.x * 8;
        raw[c] = load_raw8<VEC, BF16>(rp, col, p.cols);
        kk[c] = has_k ? load_shift8<VEC>(p, col) : make_uint2(0, 0);
    }
    float v[R][8];
    float m = 0.0f;
#pragma unroll
    for (int c = 0; c < R; c++) {
        raw8_to_float<BF16>(raw[c], v[c]);
        if (has_k && p.shift_sign > 0) shift_inputs(v[c], kk[c]);
        m = fmaxf(m, max_abs8(v[c]));
    }
    float amax;
    if (p.amax_in) {
        amax = p.amax_in[row];
    } else {
        m = dpp_wave_max(m);
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
        __syncthreads();
        amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    }
    float s = amax / p.g.qmax;
    if (p.scale_f16) s = round_f16(s);
    float r = recip_or_zero(s);
    if (threadIdx.x == 0 && p.scales_out) store_scale(p, row, s);
#pragma unroll
    for (int c = 0; c < R; c++) {
        int64_t col = (int64_t)c * kChunk + threadIdx.x * 8;
        if (col >= p.cols) continue;
        scale_values(v[c], r, has_k && p.shift_sign < 0, kk[c]);
        uint32_t w = pack8(v[c], p.g);
        store_codes(p.packed + row * p.ldp, col, p.cols, w, VEC);
    }
}

// TENSOR mode with the E2M1 grid on bf16 input (the activations; optionally with the
// column shifts r * 2^-k): U (row, 2048-column) units per workgroup of 256 threads, lane
// l of wavefront w taking columns 512 w + 8 l .. + 7 of each, so every load instruction
// reads 1 KiB contiguous.  Buffer loads (zeros past the row, no lane-dependent branch
// around a load) that bypass the caches' retention, all U issued before any arithmetic;
// 4-byte code stores, also nontemporal.  The arithmetic is that of
// quantize_e2m1_tensor_kernel.
template <bool SHIFT, int U>
__global__ void __launch_bounds__(kThreads) quantize_e2m1_tensor_bf16_kernel(QuantParams p, int chunks, int nunits) {
    typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
    const __amdgpu_buffer_rsrc_t rx = buf_make(p.x, (int64_t)p.rows * p.ldx * 2);
    const __amdgpu_buffer_rsrc_t rk = buf_make(p.col_shift, SHIFT ? p.cols : 0);
    u32x4v raw[U];
    uint2 kk[U];
    int row[U];
    int64_t col[U];
#pragma unroll
    for (int i = 0; i < U; i++) {
        int u = blockIdx.x * U + i;
        if (u >= nunits) u = nunits - 1;  // a duplicate of the last unit writes the same bytes
        row[i] = u / chunks;
        col[i] = (int64_t)(u - row[i] * chunks) * 2048 + threadIdx.x * 8;
        const uint32_t off = col[i] < p.cols ? (uint32_t)(((int64_t)row[i] * p.ldx + col[i]) * 2) : kOOB;
        raw[i] = __builtin_bit_cast(u32x4v, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 2));
        if (SHIFT) {
            const uint32_t ko = col[i] < p.cols ? (uint32_t)col[i] : kOOB;
            kk[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rk, ko, 0, 0));
        }
    }
    const float s = p.tensor_scale ? p.tensor_scale[0] : p.tensor_amax[0] / p.g.qmax;
    const float r = recip_or_zero(s);
    if (blockIdx.x == 0 && threadIdx.x == 0 && p.tensor_scale && p.scales_out)
        reinterpret_cast<float*>(p.scales_out)[0] = s;
#pragma unroll
    for (int i = 0; i < U; i++) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            v[2 * j] = __uint_as_float(raw[i][j] << 16);
            v[2 * j + 1] = __uint_as_float(raw[i][j] & 0xffff0000u);
        }
        scale_values(v, r, SHIFT, SHIFT ? kk[i] : make_uint2(0, 0));
        uint32_t w = 0;
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], 1.0f, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
        if (col[i] < p.cols)
            __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(p.packed + (int64_t)row[i] * p.ldp + col[i] / 2));
    }
}

// ROW mode, E2M1, f32 input, rows of at most NB * 1024 elements: one workgroup per row
// with every load instruction reading 1 KiB contiguous (whole 128-byte lines): load b of
// lane l of wavefront w takes columns 1024 b + 256 w + 4 l .. + 3.  The loads are buffer
// loads (offsets past the row read zeros, so no load sits under a lane-dependent
// branch) that bypass the caches' retention; the row stays in registers (one HBM read).
// SH = 1: the weights' pre-shift x' = x * 2^k, applied as the row is loaded (before the
// row maximum); SH = -1: the activation-side y = fl32(x * fl32(r * 2^-k)); SH = 0: no
// shifts.  Codes are stored as 16-bit pieces.  The arithmetic is that of
// quantize_row_reg_kernel.
template <int NB, int SH>
__global__ void __launch_bounds__(kThreads) quantize_e2m1_row_f32_kernel(QuantParams p) {
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    __shared__ float red[kThreads / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t row = blockIdx.x;
    const __amdgpu_buffer_rsrc_t rx = buf_make(reinterpret_cast<const float*>(p.x) + row * p.ldx, p.cols * 4);
    const __amdgpu_buffer_rsrc_t rk = buf_make(p.col_shift, SH ? p.cols : 0);
    f32x4v v[NB];
    uint32_t kk[SH < 0 ? NB : 1];
    float m = 0.0f;
#pragma unroll
    for (int b = 0; b < NB; b++) {
        const uint32_t c = 1024 * b + 256 * wave + 4 * lane;
        v[b] = __builtin_bit_cast(f32x4v, __builtin_amdgcn_raw_buffer_load_b128(rx, 4 * c, 0, 2));
        if (SH != 0) {
            const uint32_t k = __builtin_amdgcn_raw_buffer_load_b32(rk, c, 0, 0);
            if (SH > 0) {
#pragma unroll
                for (int i = 0; i < 4; i++) v[b][i] = __builtin_amdgcn_ldexpf(v[b][i], (int)(int8_t)(k >> (8 * i)));
            } else {
                kk[b] = k;
            }
        }
#pragma unroll
        for (int i = 0; i < 4; i++) m = fmaxf(m, fabsf(v[b][i]));
    }
    float amax;
    if (p.amax_in) {
        amax = p.amax_in[row];
    } else {
        m = dpp_wave_max(m);
        if (lane == 0) red[wave] = m;
        __syncthreads();
        amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    }
    float s = amax / p.g.qmax;
    if (p.scale_f16) s = round_f16(s);
    const float r = recip_or_zero(s);
    if (threadIdx.x == 0 && p.scales_out) store_scale(p, row, s);
#pragma unroll
    for (int b = 0; b < NB; b++) {
        const int64_t c = 1024 * b + 256 * wave + 4 * lane;
        float y[4];
#pragma unroll
        for (int i = 0; i < 4; i++)
            y[i] = SH < 0 ? v[b][i] * __builtin_amdgcn_ldexpf(r, -(int)(int8_t)(kk[b] >> (8 * i))) : v[b][i] * r;
        uint32_t w = 0;
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], 1.0f, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
        if (c < p.cols)  // cols is a multiple of 8: the 4 columns are in range together
            __builtin_nontemporal_store((uint16_t)w, reinterpret_cast<uint16_t*>(p.packed + row * p.ldp + c / 2));
    }
}

// ROW mode, E2M1, bf16 input (per-token activation scales), rows of at most NB * 2048
// elements: the f32 kernel above with 8 values (16 bytes) per lane and load, lane l of
// wavefront w taking columns 2048 b + 512 w + 8 l .. + 7 of load b (1 KiB contiguous per
// load instruction); 4-byte code stores.  SH as above.
template <int NB, int SH>
__global__ void __launch_bounds__(kThreads) quantize_e2m1_row_bf16_kernel(QuantParams p) {
    typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
    __shared__ float red[kThreads / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t row = blockIdx.x;
    const __amdgpu_buffer_rsrc_t rx = buf_make(reinterpret_cast<const uint16_t*>(p.x) + row * p.ldx, p.cols * 2);
    const __amdgpu_buffer_rsrc_t rk = buf_make(p.col_shift, SH ? p.cols : 0);
    float v[NB][8];
    uint2 kk[SH < 0 ? NB : 1];
    float m = 0.0f;
#pragma unroll
    for (int b = 0; b < NB; b++) {
        const uint32_t c = 2048 * b + 512 * wave + 8 * lane;
        const u32x4v raw = __builtin_bit_cast(u32x4v, __builtin_amdgcn_raw_buffer_load_b128(rx, 2 * c, 0, 2));
#pragma unroll
        for (int j = 0; j < 4; j++) {
            v[b][2 * j] = __uint_as_float(raw[j] << 16);
            v[b][2 * j + 1] = __uint_as_float(raw[j] & 0xffff0000u);
        }
        if (SH != 0) {
            const uint2 k = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rk, c, 0, 0));
            if (SH > 0) shift_inputs(v[b], k);
            else kk[b] = k;
        }
#pragma unroll
        for (int i = 0; i < 8; i++) m = fmaxf(m, fabsf(v[b][i]));
    }
    float amax;
    if (p.amax_in) {
        amax = p.amax_in[row];
    } else {
        m = dpp_wave_max(m);
        if (lane == 0) red[wave] = m;
        __syncthreads();
        amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    }
    float s = amax / p.g.qmax;
    if (p.scale_f16) s = round_f16(s);
    const float r = recip_or_zero(s);
    if (threadIdx.x == 0 && p.scales_out) store_scale(p, row, s);
#pragma unroll
    for (int b = 0; b < NB; b++) {
        const int64_t c = 2048 * b + 512 * wave + 8 * lane;
        scale_values(v[b], r, SH < 0, SH < 0 ? kk[b] : make_uint2(0, 0));
        uint32_t w = 0;
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[b][0], v[b][1], 1.0f, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[b][2], v[b][3], 1.0f, 1);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[b][4], v[b][5], 1.0f, 2);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[b][6], v[b][7], 1.0f, 3);
        if (c < p.cols)  // cols is a multiple of 8: the 8 columns are in range together
            __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(p.packed + row * p.ldp + c / 2));
    }
}

// ROW mode for longer rows: pass 1 reduces the row max, pass 2 re-reads (L2) and
// quantizes.
template <bool VEC, bool BF16>
__global__ void __launch_bounds__(kThreads) quantize_row_kernel(QuantParams p) {
    __shared__ float red[kThreads / 64];
    const int64_t row = blockIdx.x;
    const char* rp = reinterpret_cast<const char*>(p.x) + row * p.ldx * (BF16 ? 2 : 4);
    const bool has_k = p.col_shift != nullptr;
    float amax;
    if (p.amax_in) {
        amax = p.amax_in[row];
    } else {
        float m = 0.0f;
        for (int64_t c0 = 0; c0 < p.cols; c0 += kChunk) {
            int64_t col = c0 + threadIdx.x * 8;
            float v[8];
            load8<VEC, BF16>(rp, col, p.cols, v);
            if (has_k && p.shift_sign > 0) shift_inputs(v, load_shift8<VEC>(p, col));
            m = fmaxf(m, max_abs8(v));
        }
        m = dpp_wave_max(m);
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
        __syncthreads();
        amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    }
    float s = amax / p.g.qmax;
    if (p.scale_f16) s = round_f16(s);
    float r = recip_or_zero(s);
    if (threadIdx.x == 0 && p.scales_out) store_scale(p, row, s);
    for (int64_t c0 = 0; c0 < p.cols; c0 += kChunk) {
        int64_t col = c0 + threadIdx.x * 8;
        if (col >= p.cols) continue;
        float v[8];
        load8<VEC, BF16>(rp, col, p.cols, v);
        uint2 k = has_k ? load_shift8<VEC>(p, col) : make_uint2(0, 0);
        if (has_k && p.shift_sign > 0) shift_inputs(v, k);
        scale_values(v, r, has_k && p.shift_sign < 0, k);
        uint32_t w = pack8(v, p.g);
        store_codes(p.packed + row * p.ldp, col, p.cols, w, VEC);
    }
}

// ROW mode on an FP8 / FP6 grid: one workgroup per row, the row's amax (or amax_in[row])
// in a first pass, s = amax / Qmax (binary16-rounded for f16 scales), then the codes of
// y = fl32(x * fl32(1/s)) in a second pass, as the 4-bit row kernel does.
template <bool VEC, bool BF16, int E, int M>
__global__ void __launch_bounds__(kThreads) quantize_wide_row_kernel(QuantParams p) {
    __shared__ float red[kThreads / 64];
    const int64_t row = blockIdx.x;
    const char* rp = reinterpret_cast<const char*>(p.x) + row * p.ldx * (BF16 ? 2 : 4);
    const bool has_k = p.col_shift != nullptr;
    float amax;
    if (p.amax_in) {
        amax = p.amax_in[row];
    } else {
        float m = 0.0f;
        for (int64_t c0 = 0; c0 < p.cols; c0 += kChunk) {
            float v[8];
            load8<VEC, BF16>(rp, c0 + threadIdx.x * 8, p.cols, v);
            if (has_k && p.shift_sign > 0) shift_inputs(v, load_shift8<VEC>(p, c0 + threadIdx.x * 8));
            m = fmaxf(m, max_abs8(v));
        }
        m = dpp_wave_max(m);
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
        __syncthreads();
        amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    }
    float s = amax / p.g.qmax;
    if (p.scale_f16) s = round_f16(s);
    const float r = recip_or_zero(s);
    if (threadIdx.x == 0 && p.scales_out) store_scale(p, row, s);
    for (int64_t c0 = 0; c0 < p.cols; c0 += kChunk) {
        const int64_t col = c0 + threadIdx.x * 8;
        if (col >= p.cols) continue;
        float v[8];
        load8<VEC, BF16>(rp, col, p.cols, v);
        const uint2 k = has_k ? load_shift8<VEC>(p, col) : make_uint2(0, 0);
        if (has_k && p.shift_sign > 0) shift_inputs(v, k);
        scale_values(v, r, has_k && p.shift_sign < 0, k);
        store_wide8<VEC, E, M>(p, row, col, v);
    }
}

__global__ void tensor_scale_finalize_kernel(const float* amax, float* scales_out, float qmax) {
    scales_out[0] = amax[0] / qmax;
}

hipError_t launch_tensor_scale_finalize(const float* amax, float* scales_out, float qmax, hipStream_t s) {
    hipLaunchKernelGGL(tensor_scale_finalize_kernel, dim3(1), dim3(1), 0, s, amax, scales_out, qmax);
    return hipGetLastError();
}

template <int SH>
static void row_bf16_launch(const QuantParams& p, dim3 grid, hipStream_t s) {
    if (p.cols <= 2 * 2048) hipLaunchKernelGGL((quantize_e2m1_row_bf16_kernel<2, SH>), grid, dim3(kThreads), 0, s, p);
    else if (p.cols <= 3 * 2048) hipLaunchKernelGGL((quantize_e2m1_row_bf16_kernel<3, SH>), grid, dim3(kThreads), 0, s, p);
    else if (p.cols <= 4 * 2048) hipLaunchKernelGGL((quantize_e2m1_row_bf16_kernel<4, SH>), grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((quantize_e2m1_row_bf16_kernel<7, SH>), grid, dim3(kThreads), 0, s, p);
}

template <int SH>
static void row_f32_launch(const QuantParams& p, dim3 grid, hipStream_t s) {
    if (p.cols <= 4 * 1024) hipLaunchKernelGGL((quantize_e2m1_row_f32_kernel<4, SH>), grid, dim3(kThreads), 0, s, p);
    else if (p.cols <= 6 * 1024) hipLaunchKernelGGL((quantize_e2m1_row_f32_kernel<6, SH>), grid, dim3(kThreads), 0, s, p);
    else if (p.cols <= 8 * 1024) hipLaunchKernelGGL((quantize_e2m1_row_f32_kernel<8, SH>), grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((quantize_e2m1_row_f32_kernel<14, SH>), grid, dim3(kThreads), 0, s, p);
}

template <bool VEC, bool BF16>
static void quantize_launch(const QuantParams& p, hipStream_t s) {
    constexpr int QT = 256;  // threads of the E2M1 group-128 kernel
    if (p.mode == 1 && p.g.bits != 4) {
        dim3 grid((unsigned)p.rows);
        if (p.g.e == 4) hipLaunchKernelGGL((quantize_wide_row_kernel<VEC, BF16, 4, 3>), grid, dim3(kThreads), 0, s, p);
        else if (p.g.e == 5) hipLaunchKernelGGL((quantize_wide_row_kernel<VEC, BF16, 5, 2>), grid, dim3(kThreads), 0, s, p);
        else if (p.g.e == 2) hipLaunchKernelGGL((quantize_wide_row_kernel<VEC, BF16, 2, 3>), grid, dim3(kThreads), 0, s, p);
        else hipLaunchKernelGGL((quantize_wide_row_kernel<VEC, BF16, 3, 2>), grid, dim3(kThreads), 0, s, p);
    } else if (p.mode == 1) {
        dim3 grid((unsigned)p.rows);
        if (VEC && !BF16 && p.g.is_e2m1 && p.cols <= 14 * 1024) {
            if (!p.col_shift) row_f32_launch<0>(p, grid, s);
            else if (p.shift_sign > 0) row_f32_launch<1>(p, grid, s);
            else row_f32_launch<-1>(p, grid, s);
        } else if (VEC && BF16 && p.g.is_e2m1 && p.cols <= 7 * 2048) {
            if (!p.col_shift) row_bf16_launch<0>(p, grid, s);
            else if (p.shift_sign > 0) row_bf16_launch<1>(p, grid, s);
            else row_bf16_launch<-1>(p, grid, s);
        } else if (p.cols <= 4 * kChunk) hipLaunchKernelGGL((quantize_row_reg_kernel<VEC, BF16, 4>), grid, dim3(kThreads), 0, s, p);
        else if (p.cols <= 8 * kChunk) hipLaunchKernelGGL((quantize_row_reg_kernel<VEC, BF16, 8>), grid, dim3(kThreads), 0, s, p);
        else hipLaunchKernelGGL((quantize_row_kernel<VEC, BF16>), grid, dim3(kThreads), 0, s, p);
    } else {
        constexpr int U = 2;
        int64_t chunks = (p.cols + kChunk - 1) / kChunk;
        int64_t nunits = p.rows * chunks;
        dim3 grid((unsigned)((nunits + U - 1) / U));
        const bool wide_g128 = VEC && !BF16 && p.g.bits != 4 && p.mode == 2 && p.group == 128 && !p.col_shift &&
                               !p.amax_in && p.cols % 128 == 0 && p.rows * ((p.cols + 4095) / 4096) < (1LL << 31) &&
                               p.cols < (1LL << 30);
        if (wide_g128) {
            const int wchunks = (int)((p.cols + 4095) / 4096);
            const dim3 wg((unsigned)(p.rows * wchunks));
            if (p.g.e == 4) hipLaunchKernelGGL((quantize_wide_g128_f32_kernel<4, 3>), wg, dim3(512), 0, s, p, wchunks);
            else if (p.g.e == 5) hipLaunchKernelGGL((quantize_wide_g128_f32_kernel<5, 2>), wg, dim3(512), 0, s, p, wchunks);
            else if (p.g.e == 2) hipLaunchKernelGGL((quantize_wide_g128_f32_kernel<2, 3>), wg, dim3(512), 0, s, p, wchunks);
            else hipLaunchKernelGGL((quantize_wide_g128_f32_kernel<3, 2>), wg, dim3(512), 0, s, p, wchunks);
        } else if (p.g.bits != 4 && p.g.e == 4)
            hipLaunchKernelGGL((quantize_wide_kernel<VEC, BF16, U, 4, 3>), grid, dim3(kThreads), 0, s, p, chunks, nunits);
        else if (p.g.bits != 4 && p.g.e == 5)
            hipLaunchKernelGGL((quantize_wide_kernel<VEC, BF16, U, 5, 2>), grid, dim3(kThreads), 0, s, p, chunks, nunits);
        else if (p.g.bits != 4 && p.g.e == 2)
            hipLaunchKernelGGL((quantize_wide_kernel<VEC, BF16, U, 2, 3>), grid, dim3(kThreads), 0, s, p, chunks, nunits);
        else if (p.g.bits != 4)
            hipLaunchKernelGGL((quantize_wide_kernel<VEC, BF16, U, 3, 2>), grid, dim3(kThreads), 0, s, p, chunks, nunits);
        else if (p.g.kind == 2)
            hipLaunchKernelGGL((quantize_two_mode_kernel<VEC, BF16, U>), grid, dim3(kThreads), 0, s, p, chunks, nunits);
        else if (VEC && p.mode == 2 && p.group == 128 && p.g.is_e2m1 && !p.col_shift && !p.amax_in &&
            p.rows * ((p.cols + QT * 8 - 1) / (QT * 8)) < (1LL << 30) && p.cols < (1LL << 30)) {
            const int64_t qchunks = (p.cols + QT * 8 - 1) / (QT * 8), qunits = p.rows * qchunks;
            if (BF16)
                hipLaunchKernelGGL((quantize_e2m1_g128_kernel<BF16, 1, QT>), dim3((unsigned)qunits), dim3(QT), 0, s, p,
                                   (int)qchunks, (int)qunits);
            else {
                // 512 threads, one (row, 4096-column) unit per workgroup: measured fastest of
                // 256 / 512 / 1024 threads with one or two units (33.5 us at 11008 x 4096)
                constexpr int FT = 512, FU = 1;
                const int64_t fchunks = (p.cols + FT * 8 - 1) / (FT * 8), funits = p.rows * fchunks;
                hipLaunchKernelGGL((quantize_e2m1_g128_f32_kernel<FT, FU>), dim3((unsigned)((funits + FU - 1) / FU)),
                                   dim3(FT), 0, s, p, (int)fchunks, (int)funits);
            }
        }
        else if (VEC && p.mode == 0 && p.g.is_e2m1 && !p.amax_in && (!p.col_shift || p.shift_sign < 0) &&
                 p.rows * ((p.cols + QT * 8 - 1) / (QT * 8)) < (1LL << 30) && p.cols < (1LL << 30)) {
            const int64_t qchunks = (p.cols + QT * 8 - 1) / (QT * 8), qunits = p.rows * qchunks;
#ifndef TBF_U
#define TBF_U 4
#endif
            if (BF16 && p.rows * p.ldx * 2 < 0x7fff0000LL) {
                constexpr int TU = TBF_U;  // measured: 1 / 2 / 4 units at 0.47 / 0.49 / 0.49 (2048x4096),
                                           // 0.65 / 0.69 / 0.76 (4096x13824) of HBM
                const dim3 g((unsigned)((qunits + TU - 1) / TU));
                if (p.col_shift)
                    hipLaunchKernelGGL((quantize_e2m1_tensor_bf16_kernel<true, TU>), g, dim3(kThreads), 0, s, p,
                                       (int)qchunks, (int)qunits);
                else
                    hipLaunchKernelGGL((quantize_e2m1_tensor_bf16_kernel<false, TU>), g, dim3(kThreads), 0, s, p,
                                       (int)qchunks, (int)qunits);
            } else if (p.col_shift)
                hipLaunchKernelGGL((quantize_e2m1_tensor_kernel<BF16, true, QT>), dim3((unsigned)qunits), dim3(QT), 0, s,
                                   p, (int)qchunks);
            else
                hipLaunchKernelGGL((quantize_e2m1_tensor_kernel<BF16, false, QT>), dim3((unsigned)qunits), dim3(QT), 0,
                                   s, p, (int)qchunks);
        } else
            hipLaunchKernelGGL((quantize_chunk_kernel<VEC, BF16, U>), grid, dim3(kThreads), 0, s, p, chunks, nunits);
    }
}

hipError_t launch_quantize(const QuantParams& p, hipStream_t s) {
    if (p.rows == 0 || p.cols == 0) return hipSuccess;
    if (p.vec && p.x_bf16) quantize_launch<true, true>(p, s);
    else if (p.vec) quantize_launch<true, false>(p, s);
    else if (p.x_bf16) quantize_launch<false, true>(p, s);
    else quantize_launch<false, false>(p, s);
    return hipGetLastError();
}

// ------------------------------------------------------------------ dequantize ---
__global__ void __launch_bounds__(kThreads) dequantize_kernel(const uint8_t* packed, int64_t cols, int64_t ldp,
                                                              QGrid g, int mode, int group, const void* scales,
                                                              int scale_f16, const int8_t* col_shift, float* out,
                                                              int64_t ldo, int64_t chunks) {
    int64_t b = blockIdx.x;
    int64_t row = b / chunks;
    int64_t col = (b % chunks) * kChunk + threadIdx.x * 8;
    if (col >= cols) return;
    const uint8_t* prow = packed + row * ldp;
    for (int i = 0; i < 8 && col + i < cols; i++) {
        int64_t c = col + i;
        uint32_t code = g.bits == 8 ? prow[c] : g.bits == 6 ? code6_at(prow, c) : (prow[c >> 1] >> (4 * (c & 1))) & 15u;
        int64_t unit = mode == 0 ? 0 : (mode == 1 ? row : row * (cols / group) + c / group);
        float sc = scale_f16 ? __half2float(reinterpret_cast<const __half*>(scales)[unit])
                             : reinterpret_cast<const float*>(scales)[unit];
        float v;
        if (g.bits != 4) {
            v = wide_value_rt(code, g.e) * sc;
        } else if (g.kind == 2) {  // two-mode: the scale's sign bit picks E1M2 (val[8..15]) over E2M1
            const float m = g.val[(signbit(sc) ? 8 : 0) + (code & 7)] * fabsf(sc);
            v = (code & 8) ? -m : m;
        } else {
            v = grid_value(code, g) * sc;
        }
        if (col_shift) v = ldexpf(v, (int)col_shift[c]);
        out[row * ldo + c] = v;
    }
}

hipError_t launch_dequantize(const uint8_t* packed, int64_t rows, int64_t cols, int64_t ldp, const QGrid& g,
                             int mode, int group, const void* scales, int scale_f16, const int8_t* col_shift,
                             float* out, int64_t ldo, hipStream_t s) {
    if (rows == 0 || cols == 0) return hipSuccess;
    int64_t chunks = (cols + kChunk - 1) / kChunk;
    hipLaunchKernelGGL(dequantize_kernel, dim3((unsigned)(rows * chunks)), dim3(kThreads), 0, s, packed, cols, ldp,
                       g, mode, group, scales, scale_f16, col_shift, out, ldo, chunks);
    return hipGetLastError();
}

// ------------------------------------------------------------------ pre-shift ----
// One workgroup: c_max = max_k c[k]; a = fl32(c_max / Qmax); k_j = smallest j with
// c_max * 2^j >= c[j].  With c = f * 2^E, f in [0.5, 1): k = E_c - E_max + (f_max < f_c),
// exact; 0 for c == 0; clamped at -64.
__global__ void __launch_bounds__(1024) preshift_factors_kernel(const float* c, int64_t k, float act_qmax,
                                                                int8_t* shift_out, float* act_scale_out) {
    __shared__ float red[16];
    float m = 0.0f;
    for (int64_t j = threadIdx.x; j < k; j += blockDim.x) m = fmaxf(m, c[j]);
    m = dpp_wave_max(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    float cmax = 0.0f;
    for (int i = 0; i < (int)(blockDim.x >> 6); i++) cmax = fmaxf(cmax, red[i]);
    if (threadIdx.x == 0) act_scale_out[0] = cmax / act_qmax;
    int em;
    float fm = frexpf(cmax, &em);
    for (int64_t j = threadIdx.x; j < k; j += blockDim.x) {
        float cj = c[j];
        int ej;
        float fj = frexpf(cj, &ej);
        int kk = ej - em + (fm < fj ? 1 : 0);
        if (kk < -64) kk = -64;
        if (cj == 0.0f) kk = 0;
        shift_out[j] = (int8_t)kk;
    }
}

hipError_t launch_preshift_factors(const float* chan_amax, int64_t k, float act_qmax, int8_t* shift_out,
                                   float* act_scale_out, hipStream_t s) {
    hipLaunchKernelGGL(preshift_factors_kernel, dim3(1), dim3(1024), 0, s, chan_amax, k, act_qmax, shift_out,
                       act_scale_out);
    return hipGetLastError();
}

}  // namespace fp4

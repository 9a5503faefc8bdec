// Device-side helpers for the gfx950 kernels: element loads, the 4-bit code ladder,
// nibble packing and wave-level reductions.  Built with -ffp-contract=off so every
// float expression rounds exactly as written; fused multiply-adds are explicit.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>
#include "fp4_internal.h"

namespace fp4 {

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) { return __uint_as_float(b << 16); }

// 8 consecutive elements of a row as floats; elements at col >= cols read as 0.
template <bool VEC>
__device__ __forceinline__ void load8(const void* row_ptr, int x_bf16, int64_t col, int64_t cols,
                                      float v[8]) {
    if (VEC && col + 8 <= cols) {
        if (x_bf16) {
            uint4 q = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(row_ptr) + col);
            uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int i = 0; i < 4; i++) {
                v[2 * i] = __uint_as_float(w[i] << 16);
                v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
            }
        } else {
            const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(row_ptr) + col);
            float4 a = p[0], b = p[1];
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
            v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; i++) {
            float t = 0.0f;
            if (col + i < cols) {
                if (x_bf16) t = bf16_bits_to_float(reinterpret_cast<const uint16_t*>(row_ptr)[col + i]);
                else t = reinterpret_cast<const float*>(row_ptr)[col + i];
            }
            v[i] = t;
        }
    }
}

// Magnitude code of a minifloat grid by the compare ladder: count the midpoints below
// a (a = |y|); exactly on the midpoint between codes i-1 and i the even code wins.
__device__ __forceinline__ uint32_t ladder7(float a, const float* thr) {
    uint32_t c = 0;
#pragma unroll
    for (int i = 1; i <= 7; i++) c += (i & 1) ? (a > thr[i - 1]) : (a >= thr[i - 1]);
    return c;
}

__device__ __forceinline__ uint32_t ladder15(float y, const float* thr) {
    uint32_t c = 0;
#pragma unroll
    for (int i = 1; i <= 15; i++) c += (i & 1) ? (y > thr[i - 1]) : (y >= thr[i - 1]);
    return c;
}

// 4-bit code of y (already multiplied by the reciprocal scale).
__device__ __forceinline__ uint32_t code_of(float y, const QGrid& g) {
    if (g.kind == 0) {
        uint32_t s = (__float_as_uint(y) >> 31) << 3;
        return s | ladder7(fabsf(y), g.thr);
    }
    return ladder15(y, g.thr);
}

// Eight codes -> one 32-bit word, element 2j in the low nibble of byte j.
__device__ __forceinline__ uint32_t pack8(const float y[8], const QGrid& g) {
    if (g.is_e2m1) {
        // gfx950 v_cvt_scalef32_pk_fp4_f32 with scale 1.0: nearest E2M1 value, ties to
        // the even code, saturating at +-6, sign kept (-0 -> 0x8); checked against
        // the compare ladder on every binary32 input.
        uint32_t w = 0;
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], 1.0f, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], 1.0f, 2);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], 1.0f, 3);
        return w;
    }
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) w |= code_of(y[i], g) << (4 * i);
    return w;
}

// Reciprocal of a scale; 0 for a zero scale (an all-zero unit quantizes to +-0).
__device__ __forceinline__ float recip_or_zero(float s) { return s == 0.0f ? 0.0f : 1.0f / s; }

__device__ __forceinline__ float round_f16(float s) { return __half2float(__float2half_rn(s)); }

// max over aligned groups of `width` lanes (width a power of two <= 64)
__device__ __forceinline__ float group_max(float v, int width) {
    for (int o = 1; o < width; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Decoded value of a 4-bit code (sign applied, no scale).
__device__ __forceinline__ float grid_value(uint32_t c, const QGrid& g) {
    if (g.kind == 0) {
        float v = g.val[c & 7];
        return (c & 8) ? -v : v;
    }
    return g.val[c & 15];
}

}  // namespace fp4

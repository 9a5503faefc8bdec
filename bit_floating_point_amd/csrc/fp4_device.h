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

// 8 consecutive elements of a row, loaded raw (bf16 bits or f32 bits) so that every
// load of a thread can be issued before the first conversion waits for data.
struct Raw8 {
    uint4 a, b;  // bf16: a holds the 8 values; f32: a = elements 0-3, b = elements 4-7
};

template <bool VEC, bool BF16>
__device__ __forceinline__ Raw8 load_raw8(const void* row_ptr, int64_t col, int64_t cols) {
    Raw8 r;
    r.a = make_uint4(0, 0, 0, 0);
    r.b = make_uint4(0, 0, 0, 0);
    if (VEC) {
        // vector path: cols is a multiple of 8, so a chunk is either whole or absent
        if (col < cols) {
            if (BF16) {
                r.a = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(row_ptr) + col);
            } else {
                const uint4* q = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(row_ptr) + col);
                r.a = q[0];
                r.b = q[1];
            }
        }
    } else {
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            w[i] = 0;
            if (col + i < cols) {
                if (BF16) w[i] = reinterpret_cast<const uint16_t*>(row_ptr)[col + i];
                else w[i] = __float_as_uint(reinterpret_cast<const float*>(row_ptr)[col + i]);
            }
        }
        if (BF16) {
            r.a = make_uint4(w[0] | (w[1] << 16), w[2] | (w[3] << 16), w[4] | (w[5] << 16), w[6] | (w[7] << 16));
        } else {
            r.a = make_uint4(w[0], w[1], w[2], w[3]);
            r.b = make_uint4(w[4], w[5], w[6], w[7]);
        }
    }
    return r;
}

template <bool BF16>
__device__ __forceinline__ void raw8_to_float(const Raw8& r, float v[8]) {
    if (BF16) {
        const uint32_t w[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    } else {
        v[0] = __uint_as_float(r.a.x); v[1] = __uint_as_float(r.a.y);
        v[2] = __uint_as_float(r.a.z); v[3] = __uint_as_float(r.a.w);
        v[4] = __uint_as_float(r.b.x); v[5] = __uint_as_float(r.b.y);
        v[6] = __uint_as_float(r.b.z); v[7] = __uint_as_float(r.b.w);
    }
}

template <bool VEC, bool BF16>
__device__ __forceinline__ void load8(const void* row_ptr, int64_t col, int64_t cols, float v[8]) {
    raw8_to_float<BF16>(load_raw8<VEC, BF16>(row_ptr, col, cols), v);
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

// OCP 8- and 6-bit minifloats: E4M3 (bias 7, largest code 0x7E = 448, the all-ones code
// is NaN), E5M2 (bias 15, largest 0x7B = 57344, exponent 31 is inf/NaN), E2M3 (bias 1,
// largest 7.5) and E3M2 (bias 3, largest 28), the last two with no reserved code; the
// sign sits above the e + m magnitude bits.
template <int E, int M>
struct Wide {
    static constexpr int BIAS = E == 4 ? 7 : E == 5 ? 15 : E == 2 ? 1 : 3;
    static constexpr uint32_t MAXC = E == 4 ? 0x7Eu : E == 5 ? 0x7Bu : 31u;
    static constexpr float QMAX = E == 4 ? 448.0f : E == 5 ? 57344.0f : E == 2 ? 7.5f : 28.0f;
};

// Code of y: nearest value, ties to the even code, saturating at the largest finite
// value, sign of y on top.  Below the smallest normal the magnitude code is
// rint(|y| / 2^(1 - bias - m)) (2^m is the smallest normal's code); above it the binary32
// significand is rounded to m bits (nearest-even, carries into the exponent) and its
// exponent re-biased.
template <int E, int M>
__device__ __forceinline__ uint32_t wide_code(float y) {
    constexpr int BIAS = Wide<E, M>::BIAS;
    constexpr uint32_t MAXC = Wide<E, M>::MAXC;
    const float a = fminf(fabsf(y), Wide<E, M>::QMAX);
    uint32_t c;
    if (a < __builtin_ldexpf(1.0f, 1 - BIAS)) {
        c = (uint32_t)rintf(a * __builtin_ldexpf(1.0f, BIAS - 1 + M));
    } else {
        uint32_t u = __float_as_uint(a);
        u += (1u << (22 - M)) - 1u + ((u >> (23 - M)) & 1u);
        c = (u >> (23 - M)) - ((uint32_t)(127 - BIAS) << M);
    }
    return ((__float_as_uint(y) >> 31) << (E + M)) | (c < MAXC ? c : MAXC);
}

// Value of a code (sign applied), exact.
template <int E, int M>
__device__ __forceinline__ float wide_value(uint32_t c) {
    constexpr int BIAS = Wide<E, M>::BIAS;
    const int ex = (int)((c >> M) & ((1u << E) - 1u)), mant = (int)(c & ((1u << M) - 1u));
    const float v = ex == 0 ? ldexpf((float)mant, 1 - BIAS - M) : ldexpf((float)((1 << M) + mant), ex - BIAS - M);
    return ((c >> (E + M)) & 1u) ? -v : v;
}

// Value of a code of an 8- or 6-bit grid (e, m)
__device__ __forceinline__ float wide_value_rt(uint32_t c, int e) {
    switch (e) {
        case 4: return wide_value<4, 3>(c);
        case 5: return wide_value<5, 2>(c);
        case 2: return wide_value<2, 3>(c);
        default: return wide_value<3, 2>(c);
    }
}

// Code k of a row of 6-bit codes (bit stream, code k in bits [6 k, 6 k + 6)); codes
// 4 j + 1 and 4 j + 2 straddle two bytes of their 3-byte group, the others do not.
__device__ __forceinline__ uint32_t code6_at(const uint8_t* row, int64_t k) {
    const int64_t bit = 6 * k, b = bit >> 3;
    const int sh = (int)(bit & 7);
    uint32_t v = row[b];
    if (sh > 2) v |= (uint32_t)row[b + 1] << 8;
    return (v >> sh) & 63u;
}

// Double-double sums (binary64 pairs, TwoSum error terms): about 100 bits, enough to
// decide comparisons of sums of exact binary64 terms except near-exact ties.  dd_add is
// commutative bit for bit (the TwoSum error term is exact whatever the operand order),
// so a butterfly leaves the same sum in every lane.
struct DD { double hi, lo; };

__device__ __forceinline__ DD dd_add_d(DD a, double b) {
    double s = a.hi + b;
    double bb = s - a.hi;
    double e = (a.hi - (s - bb)) + (b - bb);
    return DD{s, a.lo + e};
}

__device__ __forceinline__ DD dd_add(DD a, DD b) {
    double s = a.hi + b.hi;
    double bb = s - a.hi;
    double e = (a.hi - (s - bb)) + (b.hi - bb);
    double lo = e + (a.lo + b.lo);
    double h = s + lo;
    double l = lo - (h - s);
    return DD{h, l};
}

// Decoded value of a 4-bit code (sign applied, no scale).
__device__ __forceinline__ float grid_value(uint32_t c, const QGrid& g) {
    if (g.kind == 0) {
        float v = g.val[c & 7];
        return (c & 8) ? -v : v;
    }
    return g.val[c & 15];
}

// ---- buffer resources and direct-to-LDS loads --------------------------------------
// Raw buffer resource (stride 0): loads at byte offsets >= `bytes` return zeros, so
// rows and chunks past the end of an operand need no branch.  Offsets are 32-bit;
// kOOB is an offset past the end of any buffer this library builds.
constexpr uint32_t kOOB = 0x80000000u;
constexpr int kBufWord3 = 0x00020000;
typedef int i32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4v buf_words(const void* base, int64_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return i32x4v{(int)(uint32_t)a, (int)(uint32_t)(a >> 32), (int)bytes, kBufWord3};
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_make(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufWord3);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// One direct-to-LDS 16-byte buffer load per lane: lane l writes LDS bytes
// [lds_base + 16 l, lds_base + 16 l + 16).  Issued from inline assembly so that the
// compiler's wait-count pass, which cannot tell LDS regions apart, does not add a full
// wait before every LDS read; callers wait for these loads explicitly.  M0 is declared
// clobbered: no code of these kernels keeps a value in it (clang warns that it will not
// preserve a reserved register across the statement, which is fine).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(i32x4v rsrc, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
                 :
                 : "v"(voff), "s"(lds_base), "s"(rsrc)
                 : "memory", "m0");
}
// The same load into LDS byte base + off, M0 formed inside the asm: `base` is one
// long-lived register and `off` a constant the compiler can rematerialise, so a kernel
// issuing loads into many fixed LDS slots does not hold every slot address live.
__device__ __forceinline__ void dma16_at(i32x4v rsrc, uint32_t voff, uint32_t base, uint32_t off) {
    asm volatile("s_add_u32 m0, %1, %2\n\tbuffer_load_dwordx4 %0, %3, 0 offen lds"
                 :
                 : "v"(voff), "s"(base), "s"(off), "s"(rsrc)
                 : "memory", "m0", "scc");
}
#pragma clang diagnostic pop

}  // namespace fp4

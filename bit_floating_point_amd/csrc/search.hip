// Format and clip-range search ([FP4-LLM] search-based FP quantization: choose the
// exponent/mantissa split and the quantization range per tensor by minimising the
// quantization error), followed by packing each tensor with its winner.
//
// Pipeline per call (all on the caller's stream):
//   1. amax per tensor (atomicMax on float bits: exact, order-free);
//   2. candidate evaluation: a workgroup keeps 8192 values of one tensor in VGPRs (32
//      per lane) and sweeps every (format, clip) candidate over them.  Per element:
//      y = fl32(|w| * r), nearest grid point (E2M1: gfx950 FP4 convert pair; E1M2:
//      round-to-nearest-even of 4y; E3M0: exponent/mantissa test), deq = fl32(g * s),
//      d = |w| - deq in binary64 (exact), d*d (exact), added with TwoSum into a
//      double-double accumulator.  Double-double partials are reduced across the
//      wavefront, accumulated per candidate in LDS, and written per workgroup;
//   3. one workgroup per tensor combines the partials in a fixed order, rounds
//      (hi + lo) / numel once, and takes the argmin (exact ties: earliest candidate);
//   4. every tensor is packed with its winning format and scale.
// The double-double sum carries ~100 bits, so the rounded mean equals the correctly
// rounded mean of the exact sum (what the CPU reference computes with an exact
// integer accumulator) except when the exact value lies within ~2^-80 relative of a
// rounding boundary.  The work is VALU-bound (binary64 add throughput).
#include "fp4_device.h"

namespace fp4 {

constexpr int kSThreads = 256;
constexpr int kSPer = 32;                      // values per lane
constexpr int kSChunk = kSThreads * kSPer;     // 8192 values per pass
constexpr int kMaxCand = 512;   // formats x clips per call (LDS holds one double-double per wavefront each)

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

static int64_t search_blocks_per_tensor(int64_t numel) {
    int64_t b = (numel + 4 * kSChunk - 1) / (4 * kSChunk);
    if (b < 1) b = 1;
    if (b > 64) b = 64;
    return b;
}

size_t search_workspace_bytes(int64_t ntensors, int64_t numel, int32_t nformats, int32_t nclips) {
    int64_t nb = search_blocks_per_tensor(numel);
    size_t amax = (size_t)((ntensors * 4 + 255) / 256 * 256);
    return amax + (size_t)ntensors * nb * nformats * nclips * sizeof(DD);
}

__global__ void __launch_bounds__(kSThreads) search_amax_kernel(const float* w, int64_t numel, float* amax) {
    int64_t t = blockIdx.y;
    const float* p = w + t * numel;
    float m = 0.0f;
    for (int64_t i = ((int64_t)blockIdx.x * kSThreads + threadIdx.x) * 4; i < numel;
         i += (int64_t)gridDim.x * kSThreads * 4) {
        if (i + 4 <= numel) {
            float4 v = *reinterpret_cast<const float4*>(p + i);
            m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        } else {
            for (int64_t k = i; k < numel; k++) m = fmaxf(m, fabsf(p[k]));
        }
    }
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) atomicMax(reinterpret_cast<unsigned int*>(amax) + t, __float_as_uint(m));
}

// nearest E3M0 magnitude code of y >= 0 (values 0, 1, 2, ..., 64); exact midpoints go
// to the even code
__device__ __forceinline__ uint32_t e3m0_code(float y) {
    uint32_t u = __float_as_uint(y);
    int E = (int)(u >> 23) - 127;
    uint32_t mant = u & 0x7fffffu;
    int c;
    if (y <= 0.5f) c = 0;
    else if (y < 1.0f) c = 1;
    else {
        int up = (mant > 0x400000u) || (mant == 0x400000u && (E & 1) == 0);
        c = E + 1 + up;
    }
    return (uint32_t)(c > 7 ? 7 : c);
}


__device__ __forceinline__ uint32_t e1m2_code(float y) { return (uint32_t)fminf(rintf(y * 4.0f), 7.0f); }

// Nearest E3M0 grid value to y >= 0 without branches (same decisions as e3m0_code):
// y <= 0.5 gives 0; otherwise adding 0x3fffff plus the exponent's low bit to the bit
// pattern carries into the exponent exactly when the mantissa rounds up (past the
// midpoint 1.5 * 2^E, or on it when the code E + 2 is even), the exponent is clamped
// to the codes 1..7 (values 1..64), and NaN or infinity saturate like the code does.
__device__ __forceinline__ float e3m0_round(float y) {
    const uint32_t u = __float_as_uint(y);
    const uint32_t t = u + 0x3fffffu + ((u >> 23) & 1u);
    uint32_t x = t >> 23;
    x = x < 127u ? 127u : (x > 133u ? 133u : x);
    return u > 0x3f000000u ? __uint_as_float(x << 23) : 0.0f;
}

struct Cand { float s, r; };

template <int FMT>  // 0 E1M2, 1 E2M1, 2 E3M0
__device__ __forceinline__ DD eval_candidate(const float (&v)[kSPer], float s, float r) {
    DD acc{0.0, 0.0};
#pragma unroll
    for (int i = 0; i < kSPer; i += 2) {
        float y0 = v[i] * r, y1 = v[i + 1] * r;
        float g0, g1;
        if (FMT == 1) {
            uint32_t b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y0, y1, 1.0f, 0);
            auto gv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(b, 1.0f, 0);
            g0 = gv[0];
            g1 = gv[1];
        } else if (FMT == 0) {
            // the E1M2 code min(rint(4y), 7) kept as a float: code * 0.25 exactly
            g0 = fminf(rintf(y0 * 4.0f), 7.0f) * 0.25f;
            g1 = fminf(rintf(y1 * 4.0f), 7.0f) * 0.25f;
        } else {
            g0 = e3m0_round(y0);
            g1 = e3m0_round(y1);
        }
        float q0 = g0 * s, q1 = g1 * s;
        double d0 = (double)v[i] - (double)q0;
        double d1 = (double)v[i + 1] - (double)q1;
        acc = dd_add_d(acc, d0 * d0);
        acc = dd_add_d(acc, d1 * d1);
    }
    return acc;
}

__device__ __forceinline__ DD wave_dd_sum(DD a) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        DD b{__shfl_xor(a.hi, o, 64), __shfl_xor(a.lo, o, 64)};
        a = dd_add(a, b);
    }
    return a;
}

__global__ void __launch_bounds__(kSThreads) search_eval_kernel(const float* w, int64_t numel, SearchCandidates sc,
                                                                double lo, double hi, const float* amax_t,
                                                                DD* part) {
    __shared__ Cand cand[kMaxCand];
    __shared__ DD acc[kSThreads / 64][kMaxCand];
    const int64_t t = blockIdx.y;
    const int nb = gridDim.x;
    const int ncand = sc.nformats * sc.nclips;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float amax = amax_t[t];
    for (int c = threadIdx.x; c < ncand; c += kSThreads) {
        int f = c / sc.nclips, j = c % sc.nclips;
        double ratio = lo + (hi - lo) * (double)j / (double)(sc.nclips - 1);
        float clip = amax * (float)ratio;
        float s = clip / sc.fmt_qmax[f];
        cand[c] = Cand{s, recip_or_zero(s)};
        for (int wv = 0; wv < kSThreads / 64; wv++) acc[wv][c] = DD{0.0, 0.0};
    }
    __syncthreads();
    const float* p = w + t * numel;
    for (int64_t base = (int64_t)blockIdx.x * kSChunk; base < numel; base += (int64_t)nb * kSChunk) {
        float v[kSPer];
        // lane-interleaved 16-byte loads: value i of lane L sits at base + (i/4)*1024 + L*4 + i%4
#pragma unroll
        for (int i = 0; i < kSPer; i += 4) {
            int64_t k = base + (int64_t)(i / 4) * (kSThreads * 4) + threadIdx.x * 4;
            if (k + 4 <= numel) {
                float4 q = *reinterpret_cast<const float4*>(p + k);
                v[i] = fabsf(q.x); v[i + 1] = fabsf(q.y); v[i + 2] = fabsf(q.z); v[i + 3] = fabsf(q.w);
            } else {
#pragma unroll
                for (int u = 0; u < 4; u++) v[i + u] = (k + u < numel) ? fabsf(p[k + u]) : 0.0f;
            }
        }
        // padding values are 0: they quantize to 0 exactly and add nothing
        for (int f = 0; f < sc.nformats; f++) {
            const int e = sc.fmt_e[f];
            for (int j = 0; j < sc.nclips; j++) {
                const int c = f * sc.nclips + j;
                const Cand cd = cand[c];
                DD d;
                if (e == 2) d = eval_candidate<1>(v, cd.s, cd.r);
                else if (e == 1) d = eval_candidate<0>(v, cd.s, cd.r);
                else d = eval_candidate<2>(v, cd.s, cd.r);
                d = wave_dd_sum(d);
                if (lane == 0) acc[wave][c] = dd_add(acc[wave][c], d);
            }
        }
    }
    __syncthreads();
    for (int c = threadIdx.x; c < ncand; c += kSThreads) {
        DD s = acc[0][c];
        for (int wv = 1; wv < kSThreads / 64; wv++) s = dd_add(s, acc[wv][c]);
        part[((int64_t)t * nb + blockIdx.x) * ncand + c] = s;
    }
}

struct SearchResultDev {
    int32_t e, m, clip_index, format_index;
    float clip, scale, amax, reserved;
    double bias, mse, mse_runner_up;
};

__global__ void __launch_bounds__(1024) search_reduce_kernel(SearchCandidates sc, double lo, double hi, int nb,
                                                             int64_t numel, const float* amax_t, const DD* part,
                                                             SearchResultDev* results) {
    __shared__ double mse[kMaxCand];
    __shared__ int best_s[1];
    const int64_t t = blockIdx.x;
    const int ncand = sc.nformats * sc.nclips;
    const double n = (double)numel;
    for (int c = threadIdx.x; c < ncand; c += blockDim.x) {
        DD s{0.0, 0.0};
        for (int b = 0; b < nb; b++) s = dd_add(s, part[((int64_t)t * nb + b) * ncand + c]);
        double q1 = s.hi / n;
        double rem = fma(-q1, n, s.hi);
        mse[c] = q1 + (rem + s.lo) / n;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int best = 0;
        for (int c = 1; c < ncand; c++)
            if (mse[c] < mse[best]) best = c;
        double runner = __builtin_inf();
        for (int c = 0; c < ncand; c++)
            if (c != best && mse[c] < runner) runner = mse[c];
        int f = best / sc.nclips, j = best % sc.nclips;
        float amax = amax_t[t];
        double ratio = lo + (hi - lo) * (double)j / (double)(sc.nclips - 1);
        float clip = amax * (float)ratio;
        float s = clip / sc.fmt_qmax[f];
        SearchResultDev r;
        r.e = sc.fmt_e[f];
        r.m = sc.fmt_m[f];
        r.clip_index = j;
        r.format_index = f;
        r.clip = clip;
        r.scale = s;
        r.amax = amax;
        r.reserved = 0.0f;
        r.bias = s > 0.0f ? 1.0 - log2((double)s) : __builtin_inf();
        r.mse = mse[best];
        r.mse_runner_up = runner;
        results[t] = r;
        best_s[0] = best;
    }
}

// pack every tensor with its winner: TENSOR scale s, y = fl32(w * fl32(1/s))
__global__ void __launch_bounds__(256) search_pack_kernel(const float* w, int64_t numel, int64_t total8,
                                                          const SearchResultDev* results, uint8_t* packed) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total8) return;
    int64_t el = i * 8;
    int64_t t = el / numel;
    const SearchResultDev r = results[t];
    float rc = recip_or_zero(r.scale);
    float4 a = *reinterpret_cast<const float4*>(w + el);
    float4 b = *reinterpret_cast<const float4*>(w + el + 4);
    float y[8] = {a.x * rc, a.y * rc, a.z * rc, a.w * rc, b.x * rc, b.y * rc, b.z * rc, b.w * rc};
    uint32_t word = 0;
    if (r.e == 2) {
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, y[0], y[1], 1.0f, 0);
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, y[2], y[3], 1.0f, 1);
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, y[4], y[5], 1.0f, 2);
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, y[6], y[7], 1.0f, 3);
    } else {
#pragma unroll
        for (int k = 0; k < 8; k++) {
            uint32_t sgn = (__float_as_uint(y[k]) >> 31) << 3;
            float ay = fabsf(y[k]);
            uint32_t c = r.e == 1 ? e1m2_code(ay) : e3m0_code(ay);
            word |= (sgn | c) << (4 * k);
        }
    }
    *reinterpret_cast<uint32_t*>(packed + el / 2) = word;
}

hipError_t launch_search(const float* w, int64_t ntensors, int64_t numel, const SearchCandidates& c,
                         double clip_lo, double clip_hi, void* results, uint8_t* packed, void* ws, hipStream_t s) {
    if (ntensors == 0) return hipSuccess;
    float* amax = reinterpret_cast<float*>(ws);
    size_t amax_bytes = (size_t)((ntensors * 4 + 255) / 256 * 256);
    DD* part = reinterpret_cast<DD*>(reinterpret_cast<char*>(ws) + amax_bytes);
    hipError_t e = launch_fill_zero_u32(reinterpret_cast<uint32_t*>(amax), ntensors, s);
    if (e != hipSuccess) return e;
    int64_t ab = (numel + kSThreads * 4 * 8 - 1) / (kSThreads * 4 * 8);
    if (ab > 256) ab = 256;
    if (ab < 1) ab = 1;
    hipLaunchKernelGGL(search_amax_kernel, dim3((unsigned)ab, (unsigned)ntensors), dim3(kSThreads), 0, s, w, numel,
                       amax);
    int64_t nb = search_blocks_per_tensor(numel);
    hipLaunchKernelGGL(search_eval_kernel, dim3((unsigned)nb, (unsigned)ntensors), dim3(kSThreads), 0, s, w, numel, c,
                       clip_lo, clip_hi, amax, part);
    hipLaunchKernelGGL(search_reduce_kernel, dim3((unsigned)ntensors), dim3(1024), 0, s, c, clip_lo, clip_hi, (int)nb,
                       numel, amax, part, reinterpret_cast<SearchResultDev*>(results));
    int64_t total8 = ntensors * numel / 8;
    if (total8 > 0)
        hipLaunchKernelGGL(search_pack_kernel, dim3((unsigned)((total8 + 255) / 256)), dim3(256), 0, s, w, numel,
                           total8, reinterpret_cast<const SearchResultDev*>(results), packed);
    return hipGetLastError();
}

}  // namespace fp4

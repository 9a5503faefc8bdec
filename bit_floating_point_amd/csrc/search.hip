// Format and clip-range search ([FP4-LLM] search-based FP quantization: choose the
// exponent/mantissa split and the quantization range by minimising the quantization
// error, for weights and for activations), followed by packing with the winner.
//
// Search units over a row-major [rows, cols] matrix (f32 or bf16, leading dimension ld):
// unit u covers rows [u R, u R + R) (R = 1: one unit per row -- a weight tensor per row
// of a stacked batch, or one activation token; R = T: the first T rows as one tensor --
// the calibration tokens of an activation tensor).  Element i of a unit is row
// u R + i / cols, column i % cols.
//
// Pipeline per call (all on the caller's stream):
//   1. amax per unit (atomicMax on float bits: exact, order-free);
//   2. candidate evaluation: a workgroup keeps 256 PER values of one unit in VGPRs (PER
//      per lane, a multiple of 4 from 8 to 32 chosen to pad the unit least) and sweeps every
//      (format, clip) candidate over them.  Per element:
//      y = fl32(|w| * r), nearest grid point (E2M1: gfx950 FP4 convert pair; E1M2:
//      round-to-nearest-even of 4y; E3M0: exponent/mantissa test), deq = fl32(g * s),
//      d = |w| - deq in binary64 (exact), d*d (exact), added with TwoSum into a
//      double-double accumulator.  Double-double partials are reduced across the
//      wavefront, accumulated per candidate in LDS, and written per workgroup;
//   3. one workgroup per unit combines the partials in a fixed order, rounds
//      (hi + lo) / numel once, and takes the argmin (exact ties: earliest candidate);
//   4. every row is packed with its unit's winning format and scale (R = T: every row of
//      the matrix, the rows past T included, with the one calibration winner).
// The double-double sum carries ~100 bits, so the rounded mean equals the correctly
// rounded mean of the exact sum (what the CPU reference computes with an exact
// integer accumulator) except when the exact value lies within ~2^-80 relative of a
// rounding boundary.  The work is VALU-bound (binary64 add throughput).
#include <algorithm>

#include <mutex>

#include "fp4_device.h"

namespace fp4 {

constexpr int kSThreads = 256;
constexpr int kSPerMax = 32;                   // values per lane, at most
constexpr int kSChunk = kSThreads * kSPerMax;  // 8192 values per pass, at most
constexpr int kMaxCand = 512;   // formats x clips per call (LDS holds one double-double per wavefront each)

// Workgroups per unit: up to 4 passes of 8192 values each (at most 64 workgroups); when
// the units give fewer than 768 workgroups (3 per CU), more of them, down to 3072 values
// (12 per lane, the most for which a wavefront still evaluates four candidates at a
// time) each.  (Down to 8 per lane, the search over one 128 x 5120 unit ran 5% slower:
// each candidate's wavefront sum is amortised over fewer values.)
static int64_t search_blocks(int64_t units, int64_t numel) {
    int64_t b = (numel + 4 * kSChunk - 1) / (4 * kSChunk);
    if (b < 1) b = 1;
    if (b > 64) b = 64;
    const int64_t want = (768 + units - 1) / std::max<int64_t>(units, 1);
    const int64_t most = (numel + kSThreads * 12 - 1) / (kSThreads * 12);
    return std::max(b, std::min(want, most));
}

size_t search_workspace_bytes(int64_t ntensors, int64_t numel, int32_t nformats, int32_t nclips) {
    int64_t nb = search_blocks(ntensors, numel);
    size_t amax = (size_t)((ntensors * 4 + 255) / 256 * 256);
    return amax + (size_t)ntensors * nb * nformats * nclips * sizeof(DD);
}

// The search's view of its input: unit u's element i (a multiple of 4; cols is a
// multiple of 16, so 4 consecutive elements share a row) and the 3 after it.
struct SearchSrc {
    const void* x;
    int32_t bf16;
    int64_t ld;         // elements
    int64_t cols;
    int64_t unit_rows;  // R
    int64_t numel;      // R * cols
};

__device__ __forceinline__ float4 src_load4(const SearchSrc& s, int64_t u, int64_t i) {
    int64_t row, col;
    if (s.unit_rows == 1) {
        row = u;
        col = i;
    } else {
        row = u * s.unit_rows + i / s.cols;
        col = i % s.cols;
    }
    const int64_t off = row * s.ld + col;
    if (s.bf16) {
        const uint2 b = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(s.x) + off);
        return make_float4(__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xffff0000u), __uint_as_float(b.y << 16),
                           __uint_as_float(b.y & 0xffff0000u));
    }
    return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(s.x) + off);
}

__global__ void __launch_bounds__(kSThreads) search_amax_kernel(SearchSrc src, float* amax) {
    const int64_t t = blockIdx.y;
    float m = 0.0f;
    for (int64_t i = ((int64_t)blockIdx.x * kSThreads + threadIdx.x) * 4; i < src.numel;
         i += (int64_t)gridDim.x * kSThreads * 4) {
        const float4 v = src_load4(src, t, i);
        m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
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

template <int FMT, int PER>  // FMT 0 E1M2, 1 E2M1, 2 E3M0
__device__ __forceinline__ DD eval_candidate(const float (&v)[PER], float s, float r) {
    DD acc{0.0, 0.0};
#pragma unroll
    for (int i = 0; i < PER; i += 2) {
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

// the wavefront sums of four double-doubles, their butterflies interleaved (independent
// chains, so each step's shuffles and adds overlap the others' latency)
__device__ __forceinline__ void wave_dd_sum4(DD (&d)[4]) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        DD b[4];
#pragma unroll
        for (int q = 0; q < 4; q++) b[q] = DD{__shfl_xor(d[q].hi, o, 64), __shfl_xor(d[q].lo, o, 64)};
#pragma unroll
        for (int q = 0; q < 4; q++) d[q] = dd_add(d[q], b[q]);
    }
}

// candidates c0 .. c0 + nclips - 1 of one format over this lane's values; lane 0 adds
// each wavefront sum to the wavefront's LDS accumulator.  With few values per lane
// (workgroups then hold few wavefronts per SIMD to hide latency) four candidates at a
// time, their reductions interleaved; with many, one at a time (four would cost
// occupancy in registers).
template <int FMT, int PER>
__device__ __forceinline__ void eval_clips(const float (&v)[PER], const Cand* cand, int c0, int nclips, DD* accw,
                                           int lane) {
    int j = 0;
    for (; PER <= 12 && j + 4 <= nclips; j += 4) {
        DD d[4];
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const Cand cd = cand[c0 + j + q];
            d[q] = eval_candidate<FMT, PER>(v, cd.s, cd.r);
        }
        wave_dd_sum4(d);
        if (lane == 0) {
#pragma unroll
            for (int q = 0; q < 4; q++) accw[c0 + j + q] = dd_add(accw[c0 + j + q], d[q]);
        }
    }
    for (; j < nclips; j++) {
        const Cand cd = cand[c0 + j];
        DD d = wave_dd_sum(eval_candidate<FMT, PER>(v, cd.s, cd.r));
        if (lane == 0) accw[c0 + j] = dd_add(accw[c0 + j], d);
    }
}

template <int PER>
__global__ void __launch_bounds__(kSThreads) search_eval_kernel(SearchSrc src, SearchCandidates sc, double lo,
                                                                double hi, const float* amax_t, DD* part) {
    constexpr int CHUNK = kSThreads * PER;
    const int64_t numel = src.numel;
    __shared__ Cand cand[kMaxCand];
    __shared__ DD acc[kSThreads / 64][kMaxCand];
    const int64_t t = blockIdx.y;
    const int nb = gridDim.x;
    const int ncand = sc.nformats * sc.nclips;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float amax = amax_t[t];
    // formats [f0, f1) of this workgroup: all, or (gridDim.z == nformats) format blockIdx.z
    const int f0 = gridDim.z == 1 ? 0 : (int)blockIdx.z;
    const int f1 = gridDim.z == 1 ? sc.nformats : f0 + 1;
    for (int c = f0 * sc.nclips + threadIdx.x; c < f1 * sc.nclips; c += kSThreads) {
        int f = c / sc.nclips, j = c % sc.nclips;
        double ratio = lo + (hi - lo) * (double)j / (double)(sc.nclips - 1);
        float clip = amax * (float)ratio;
        float s = clip / sc.fmt_qmax[f];
        cand[c] = Cand{s, recip_or_zero(s)};
        for (int wv = 0; wv < kSThreads / 64; wv++) acc[wv][c] = DD{0.0, 0.0};
    }
    __syncthreads();
    for (int64_t base = (int64_t)blockIdx.x * CHUNK; base < numel; base += (int64_t)nb * CHUNK) {
        float v[PER];
        // lane-interleaved 4-element loads: value i of lane L is element base + (i/4)*1024 + L*4 + i%4
        // (numel is a multiple of 4, so a group is wholly inside or wholly past the unit)
#pragma unroll
        for (int i = 0; i < PER; i += 4) {
            const int64_t k = base + (int64_t)(i / 4) * (kSThreads * 4) + threadIdx.x * 4;
            float4 q = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (k < numel) q = src_load4(src, t, k);
            v[i] = fabsf(q.x); v[i + 1] = fabsf(q.y); v[i + 2] = fabsf(q.z); v[i + 3] = fabsf(q.w);
        }
        // padding values are 0: they quantize to 0 exactly and add nothing
        for (int f = f0; f < f1; f++) {
            const int e = sc.fmt_e[f];
            const int c0 = f * sc.nclips;
            if (e == 2) eval_clips<1, PER>(v, cand, c0, sc.nclips, acc[wave], lane);
            else if (e == 1) eval_clips<0, PER>(v, cand, c0, sc.nclips, acc[wave], lane);
            else eval_clips<2, PER>(v, cand, c0, sc.nclips, acc[wave], lane);
        }
    }
    __syncthreads();
    for (int c = f0 * sc.nclips + threadIdx.x; c < f1 * sc.nclips; c += kSThreads) {
        DD s = acc[0][c];
        for (int wv = 1; wv < kSThreads / 64; wv++) s = dd_add(s, acc[wv][c]);
        part[((int64_t)t * ncand + c) * nb + blockIdx.x] = s;
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
    // few partials: one thread per candidate adds them in order; many: one wavefront per
    // candidate, lane l adding partials l, l + 64, ..., then the wavefront's butterfly
    // (either way a fixed order for a given nb).  A wavefront takes four candidates at a
    // time, their loads and butterflies interleaved: one at a time, each candidate waited
    // for its loads and its six dependent shuffle steps in turn (70 us for one unit of 300
    // candidates x 320 partials).
    if (nb <= 16) {
        for (int c = threadIdx.x; c < ncand; c += blockDim.x) {
            DD s{0.0, 0.0};
            for (int b = 0; b < nb; b++) s = dd_add(s, part[((int64_t)t * ncand + c) * nb + b]);
            const double q1 = s.hi / n;
            const double rem = fma(-q1, n, s.hi);
            mse[c] = q1 + (rem + s.lo) / n;
        }
    } else {
        const int lane = threadIdx.x & 63, nw = blockDim.x >> 6;
        for (int c0 = threadIdx.x >> 6; c0 < ncand; c0 += 4 * nw) {
            DD d[4];
#pragma unroll
            for (int q = 0; q < 4; q++) d[q] = DD{0.0, 0.0};
            for (int b = lane; b < nb; b += 64) {
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const int c = c0 + q * nw;  // uniform per wavefront
                    if (c < ncand) d[q] = dd_add(d[q], part[((int64_t)t * ncand + c) * nb + b]);
                }
            }
            wave_dd_sum4(d);
            if (lane != 0) continue;
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int c = c0 + q * nw;
                if (c >= ncand) continue;
                const double q1 = d[q].hi / n;
                const double rem = fma(-q1, n, d[q].hi);
                mse[c] = q1 + (rem + d[q].lo) / n;
            }
        }
    }
    __syncthreads();
    // argmin (the smallest MSE, exact ties to the earliest candidate) and the runner-up's
    // MSE, over the candidates by the first wavefront: each lane scans every 64th, then a
    // butterfly (a single thread scanning all of them in turn took ~30 us)
    if (threadIdx.x >= 64) return;
    const int l = threadIdx.x;
    double bv = __builtin_inf();
    int best = ncand;  // none yet
    for (int c = l; c < ncand; c += 64)
        if (best == ncand || mse[c] < bv) bv = mse[c], best = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(best, o, 64);
        if (ov < bv || (ov == bv && oi < best)) bv = ov, best = oi;
    }
    double runner = __builtin_inf();
    for (int c = l; c < ncand; c += 64)
        if (c != best && mse[c] < runner) runner = mse[c];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) runner = fmin(runner, __shfl_xor(runner, o, 64));
    if (l == 0) {
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

// pack every row with its unit's winner (scale s of the unit), y = fl32(x * fl32(1/s));
// 8 elements per thread, rows x cols/8 threads
__global__ void __launch_bounds__(256) search_pack_kernel(SearchSrc src, int64_t rows, int per_row_units,
                                                          const SearchResultDev* results, uint8_t* packed,
                                                          int64_t ldp) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t c8 = src.cols / 8;
    if (i >= rows * c8) return;
    const int64_t row = i / c8, col = (i % c8) * 8;
    const SearchResultDev r = results[per_row_units ? row : 0];
    const float rc = recip_or_zero(r.scale);
    SearchSrc one = src;
    one.unit_rows = 1;
    const float4 a = src_load4(one, row, col);
    const float4 b = src_load4(one, row, col + 4);
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
    *reinterpret_cast<uint32_t*>(packed + row * ldp + col / 2) = word;
}

// values per lane for a unit of numel elements: the fewest padded elements over whole
// passes of 256 PER, the larger PER on a tie
static int search_per(int64_t numel, int64_t nb) {
    int best = 32;
    int64_t best_pad = -1;
    for (int per = 32; per >= 8; per -= 4) {
        const int64_t chunk = (int64_t)kSThreads * per * nb;
        const int64_t pad = (numel + chunk - 1) / chunk * chunk - numel;
        if (best_pad < 0 || pad < best_pad) {
            best = per;
            best_pad = pad;
        }
    }
    return best;
}

// Scratch of the allocation-free search entry point: one copy per GPU, held until the
// process ends.  Host code never uses the array's name as an address (on the host it
// stands for the symbol, not for device memory): it looks up each device's copy with
// hipGetSymbolAddress, once per device with that device current, and passes the
// returned pointer to the kernels.
static __device__ __align__(256) uint8_t scratch[kSearchScratchBytes];

hipError_t search_scratch(void** ptr) {
    static std::mutex mu;
    static void* addr[kMaxDevices];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_search(const SearchInput& in, const SearchCandidates& c, double clip_lo, double clip_hi,
                         void* results, uint8_t* packed, int64_t ldp, void* ws, hipStream_t s) {
    const int64_t units = in.per_row_units ? in.rows : 1;
    if (in.rows == 0) return hipSuccess;
    SearchSrc src;
    src.x = in.x;
    src.bf16 = in.bf16;
    src.ld = in.ld;
    src.cols = in.cols;
    src.unit_rows = in.per_row_units ? 1 : in.unit_rows;
    src.numel = src.unit_rows * in.cols;
    float* amax = reinterpret_cast<float*>(ws);
    const size_t amax_bytes = (size_t)((units * 4 + 255) / 256 * 256);
    DD* part = reinterpret_cast<DD*>(reinterpret_cast<char*>(ws) + amax_bytes);
    hipError_t e = launch_fill_zero_u32(reinterpret_cast<uint32_t*>(amax), units, s);
    if (e != hipSuccess) return e;
    int64_t ab = (src.numel + kSThreads * 4 * 8 - 1) / (kSThreads * 4 * 8);
    if (ab > 256) ab = 256;
    if (ab < 1) ab = 1;
    hipLaunchKernelGGL(search_amax_kernel, dim3((unsigned)ab, (unsigned)units), dim3(kSThreads), 0, s, src, amax);
    const int64_t nb = search_blocks(units, src.numel);
    // fewer workgroups than 3 per CU: one per format as well (the values are loaded once per format)
    const dim3 grid((unsigned)nb, (unsigned)units, units * nb < 768 ? (unsigned)c.nformats : 1u);
    switch (search_per(src.numel, nb)) {
        case 8:
            hipLaunchKernelGGL(search_eval_kernel<8>, grid, dim3(kSThreads), 0, s, src, c, clip_lo, clip_hi, amax, part);
            break;
        case 12:
            hipLaunchKernelGGL(search_eval_kernel<12>, grid, dim3(kSThreads), 0, s, src, c, clip_lo, clip_hi, amax, part);
            break;
        case 16:
            hipLaunchKernelGGL(search_eval_kernel<16>, grid, dim3(kSThreads), 0, s, src, c, clip_lo, clip_hi, amax, part);
            break;
        case 20:
            hipLaunchKernelGGL(search_eval_kernel<20>, grid, dim3(kSThreads), 0, s, src, c, clip_lo, clip_hi, amax, part);
            break;
        case 24:
            hipLaunchKernelGGL(search_eval_kernel<24>, grid, dim3(kSThreads), 0, s, src, c, clip_lo, clip_hi, amax, part);
            break;
        case 28:
            hipLaunchKernelGGL(search_eval_kernel<28>, grid, dim3(kSThreads), 0, s, src, c, clip_lo, clip_hi, amax, part);
            break;
        default:
            hipLaunchKernelGGL(search_eval_kernel<32>, grid, dim3(kSThreads), 0, s, src, c, clip_lo, clip_hi, amax, part);
    }
    hipLaunchKernelGGL(search_reduce_kernel, dim3((unsigned)units), dim3(1024), 0, s, c, clip_lo, clip_hi, (int)nb,
                       src.numel, amax, part, reinterpret_cast<SearchResultDev*>(results));
    const int64_t total8 = in.rows * (in.cols / 8);
    if (total8 > 0)
        hipLaunchKernelGGL(search_pack_kernel, dim3((unsigned)((total8 + 255) / 256)), dim3(256), 0, s, src, in.rows,
                           in.per_row_units, reinterpret_cast<const SearchResultDev*>(results), packed, ldp);
    return hipGetLastError();
}

}  // namespace fp4

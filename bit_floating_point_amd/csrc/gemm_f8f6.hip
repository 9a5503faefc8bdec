// Quantized GEMM with both operands in the OCP FP8 / FP6 formats, on gfx950's f8f6f4
// matrix cores:  Y[m, n] = fl32(acc[m, n] * fl32(a * s_n)),  acc = sum_k A_q[m, k] W_q[n, k]
// in fp32 by the MFMA.  Scales are factored out of the low-bit product as the
// FP4-LLM paper's efficient matrix multiplication section describes (one activation
// scale a per tensor or one per row of A, one weight scale per tensor or per output
// row); the progressive 8/6/4-bit formats come from the low-bit FP overview's FP8/FP6
// sections.
//
// Formats (the MFMA's operand format codes): 0 FP8 E4M3, 1 FP8 E5M2, 2 FP6 E2M3,
// 3 FP6 E3M2, 4 FP4 E2M1; and 5 E1M2, 6 E3M0 (the 4-bit grids the format search can
// choose that have no format code: rewritten as E4M3 on their way into LDS).  FP8 rows hold one code per byte, FP4 rows two (low nibble
// first); FP6 rows are a bit stream, code k in bits [6 k, 6 k + 6) of the row, so 16
// consecutive codes starting at a multiple of 16 are 12 contiguous bytes, half of the
// six registers of an FP6 MFMA operand.
//
// Tiling: a workgroup (four wavefronts) computes a 128 x 256 tile of Y (128 rows of A,
// 256 rows of W); each wavefront a 64 x 128 block as 2 x 4 MFMAs of 32 x 32 x 64.  A
// step covers 128 codes of K (two MFMA K-blocks): every thread loads its share of a
// later step's units into registers while the MFMAs run on the current step from LDS,
// then stores the next step's units into the other of two LDS buffers; one barrier per
// step.  The waits are the compiler's own.  Units past K are zeros, so the padding of a
// row adds nothing.
//
// Group-scaled FP8 / FP6 weights (GRP: one scale per output row and group of G codes of
// K, G a multiple of 64 dividing K, [W8A8] section 2.2's group size 128 among them):
//   Y[m, n] = fl32(T[m, n] * a_m),  T = sum over groups g of s[n, g] * P_g[m, n]
// where P_g is the group's fp32 MFMA sum, folded into T with one fused multiply-add per
// group (T = fma(P_g, s[n, g], T), group order) after the MFMA K-block that ends the
// group.  The scales of a step's two K-blocks (256 columns each) ride in LDS with the
// step's operand units.
//
// The E4M3 x E4M3 and E2M1 x E2M1 pairs have their own persistent kernel
// (gemm_w4a4.hip); this kernel takes every other pair with an FP8 or FP6 operand, W6A6
// among them, and every group-scaled FP8 / FP6 weight (E4M3 x E4M3 included).
#include "fp4_device.h"
#include "fp4_internal.h"

#include <algorithm>

namespace fp4 {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 256;  // rows of A and of W per tile
constexpr int kStepCodes = 128;
// steps of units held in registers (two: three or four measured no faster, so the
// loop is not bound by load latency)
constexpr int kSets = 2;

// A step of a row is 8 units: FP8 16-byte pieces (32 codes), FP6 12-byte runs or FP4
// 8-byte runs (16 codes).  Each unit is staged in its own 16-byte LDS slot (row stride 8 slots + 16
// bytes of padding, so the 16-byte fragment reads of 16 consecutive rows hit distinct
// banks).  With K a multiple of 32 a row ends on a unit boundary, so a unit is either
// wholly inside the row or wholly past it.
// F = 5 (E1M2) and 6 (E3M0): the 4-bit grids that have no matrix-core format of their
// own.  Their rows are loaded as FP4 rows are (8-byte runs of 16 codes) and every code is
// rewritten on its way into LDS as the FP8 E4M3 byte of the same value (every E1M2 and
// E3M0 value is an E4M3 value), staged and multiplied as E4M3 (format code 0).
template <int F>
struct Fmt {
    static constexpr bool expand = F >= 5;                     // 4-bit codes staged as E4M3
    static constexpr int bits = F < 2 ? 8 : (F < 4 ? 6 : (expand ? 8 : 4));  // bits per staged code
    static constexpr int lbits = expand ? 4 : bits;            // bits per loaded code
    static constexpr int code = expand ? 0 : F;                // MFMA operand format
    static constexpr int step_bytes = kStepCodes * lbits / 8;  // 128, 96 or 64 bytes loaded per step
    static constexpr int unit_bytes = step_bytes / 8;          // 16, 12 or 8
    static constexpr int stride = 8 * 16 + 16;                 // LDS row stride (bytes)
    // LDS slot of unit j.  The matrix cores pair the two operands' values in a fixed K
    // order that differs by format (measured on gfx950 with one-hot operands): an FP8
    // operand's 32 values are codes 32 hk + i of the 64-code K-block, i = 0..31; an FP6
    // (and FP4) operand's are two runs of 16, codes 16 hk + i and 32 + 16 hk + i.  FP8
    // pieces stay in order; FP6 / FP4 runs are placed so that lane half hk of K-block h finds
    // its two runs (4 h + hk, 4 h + 2 + hk) in slots 4 h + 2 hk and 4 h + 2 hk + 1.
    static __device__ __forceinline__ int slot(int j) {
        return bits == 8 ? j : 4 * (j >> 2) + 2 * (j & 1) + ((j >> 1) & 1);
    }
};

// Operand of K-block h for lane half hk: slots 4 h + 2 hk and 4 h + 2 hk + 1 of the row
// (an FP6 slot holds 12 code bytes and 4 unused ones, an FP4 slot 8 and 8).  The same
// slots line up every pair of formats.
template <int F>
__device__ __forceinline__ i32x8 frag(const uint8_t* row, int h, int hk) {
    const uint4 u = *reinterpret_cast<const uint4*>(row + 64 * h + 32 * hk);
    const uint4 v = *reinterpret_cast<const uint4*>(row + 64 * h + 32 * hk + 16);
    if constexpr (Fmt<F>::bits == 8)
        return i32x8{(int)u.x, (int)u.y, (int)u.z, (int)u.w, (int)v.x, (int)v.y, (int)v.z, (int)v.w};
    else if constexpr (Fmt<F>::bits == 6)
        return i32x8{(int)u.x, (int)u.y, (int)u.z, (int)v.x, (int)v.y, (int)v.z, 0, 0};
    else
        return i32x8{(int)u.x, (int)u.y, (int)v.x, (int)v.y, 0, 0, 0, 0};
}

// one unit of a row, `valid` code bytes of the row remaining from it on; a unit past K
// (valid <= 0) loads zeros, and so does one in a row past the tile's end (past its
// buffer range).  The offset is a select, not a branch: a load under a divergent branch
// would be waited for inside it, one load at a time.
template <int F>
__device__ __forceinline__ uint4 unit_load(__amdgpu_buffer_rsrc_t r, int64_t row_off, int64_t valid) {
    const uint32_t off = valid > 0 ? (uint32_t)row_off : kOOB;
    if constexpr (Fmt<F>::lbits == 8) {
        return buf_load16(r, off);
    } else if constexpr (Fmt<F>::lbits == 6) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 0);
        return make_uint4(v[0], v[1], v[2], 0u);
    } else {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        return make_uint4(v[0], v[1], 0u, 0u);
    }
}

// E4M3 bytes of the eight magnitudes of a 4-bit grid, bytes 0..3 and 4..7 of a lookup
// table for v_perm: E1M2 {0, .25, .5, .75, 1, 1.25, 1.5, 1.75}, E3M0 {0, 1, 2, 4, ..., 64}.
template <int F>
struct E4m3Table {
    static constexpr uint32_t lo = F == 5 ? 0x34302800u : 0x48403800u;
    static constexpr uint32_t hi = F == 5 ? 0x3e3c3a38u : 0x68605850u;
};

// 16 codes (8 bytes, code 2b in the low nibble of byte b) -> their 16 E4M3 bytes in code
// order: the magnitude picks a table byte, the code's sign bit becomes bit 7.
template <int F>
__device__ __forceinline__ uint4 expand16(uint4 u) {
    const uint32_t in[2] = {u.x, u.y};
    uint32_t out[4];
#pragma unroll
    for (int d = 0; d < 2; d++) {
        const uint32_t w = in[d];
        const uint32_t ev = __builtin_amdgcn_perm(E4m3Table<F>::hi, E4m3Table<F>::lo, w & 0x07070707u) |
                            ((w & 0x08080808u) << 4);  // codes 0, 2, 4, 6 of the dword
        const uint32_t od = __builtin_amdgcn_perm(E4m3Table<F>::hi, E4m3Table<F>::lo, (w >> 4) & 0x07070707u) |
                            (w & 0x80808080u);         // codes 1, 3, 5, 7
        out[2 * d] = __builtin_amdgcn_perm(od, ev, 0x05010400u);
        out[2 * d + 1] = __builtin_amdgcn_perm(od, ev, 0x07030602u);
    }
    return make_uint4(out[0], out[1], out[2], out[3]);
}

template <int F>
__device__ __forceinline__ uint4 staged(uint4 u) {
    if constexpr (Fmt<F>::expand) return expand16<F>(u);
    else return u;
}

}  // namespace

template <int FW, int FA, bool GRP>
__global__ void __launch_bounds__(256) f8f6_gemm_kernel(GemmParams p, int grid_m, int ntiles) {
    using WA = Fmt<FA>;
    using WW = Fmt<FW>;
    constexpr int LA = kBM * 8 / 256, LW = kBN * 8 / 256;  // units per thread and step
    constexpr int SA = kBM * WA::stride, SW = kBN * WW::stride;               // LDS bytes per buffer
    constexpr int SG = GRP ? 2 * kBN * 4 : 0;  // GRP: the 256 columns' f32 scales of the step's two K-blocks
    constexpr int BUF = SA + SW + SG;
    // register sets of units (GRP: one, the running sums take the registers of the second)
    constexpr int NSET = GRP ? 1 : kSets;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * BUF];

    // workgroups go round-robin over the eight XCDs; give each XCD a contiguous run of
    // tiles so the ones sharing operand rows meet in the same L2
    int t = blockIdx.x;
    const int full8 = ntiles / 8 * 8;
    if (t < full8) t = (t % 8) * (full8 / 8) + t / 8;
    const int64_t m0 = (int64_t)(t % grid_m) * kBM, n0 = (int64_t)(t / grid_m) * kBN;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int r32 = lane & 31, hk = lane >> 5;

    const int64_t rows_a = std::min<int64_t>(kBM, p.M - m0), rows_w = std::min<int64_t>(kBN, p.N - n0);
    const __amdgpu_buffer_rsrc_t rA =
        buf_make(reinterpret_cast<const uint8_t*>(p.a) + m0 * p.lda, rows_a * p.lda);
    const __amdgpu_buffer_rsrc_t rW = buf_make(p.w + n0 * p.ldw, rows_w * p.ldw);
    const int64_t bytes_a = p.K * WA::lbits / 8, bytes_w = p.K * WW::lbits / 8;  // code bytes per row
    const int nsteps = (int)((p.K + kStepCodes - 1) / kStepCodes);
    // GRP: this thread's column tid of the tile; its scale of group g at (tid * ngroups + g)
    // of a buffer over the tile's rows of scales (out of range past N: zeros)
    const int ngroups = GRP ? (int)(p.K / p.w_group) : 1;
    const int esz = p.w_scale_f16 ? 2 : 4;
    const __amdgpu_buffer_rsrc_t rS =
        buf_make(reinterpret_cast<const uint8_t*>(p.w_scales) + (GRP ? n0 * ngroups * esz : 0),
                 GRP ? rows_w * ngroups * esz : 0);

    // NSET register sets of units: set t % NSET holds step t; the loads of step
    // t + NSET are issued while step t is computed and stored into LDS at the end of
    // step t + NSET - 1
    uint4 ra[NSET][LA], rw[NSET][LW];
    float rs[NSET][2];  // GRP: this thread's column's scales for the two K-blocks of a step
    auto sload = [&](float (&v)[2], int s) {
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int g = (int)(((int64_t)s * kStepCodes + 64 * h) / p.w_group);  // K-blocks past K: g >= ngroups
            const uint32_t off = g < ngroups ? (uint32_t)((tid * ngroups + g) * esz) : kOOB;
            if (p.w_scale_f16) {
                const short b = __builtin_amdgcn_raw_buffer_load_b16(rS, off, 0, 0);
                v[h] = (float)__builtin_bit_cast(_Float16, b);
            } else {
                v[h] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rS, off, 0, 0));
            }
        }
    };
    auto gload = [&](uint4 (&a)[LA], uint4 (&w)[LW], int s) {
#pragma unroll
        for (int i = 0; i < LA; i++) {
            const int q = tid + 256 * i, row = q >> 3, j = q & 7;
            const int64_t kb = (int64_t)s * WA::step_bytes + WA::unit_bytes * j;
            a[i] = unit_load<FA>(rA, row * p.lda + kb, bytes_a - kb);
        }
#pragma unroll
        for (int i = 0; i < LW; i++) {
            const int q = tid + 256 * i, row = q >> 3, j = q & 7;
            const int64_t kb = (int64_t)s * WW::step_bytes + WW::unit_bytes * j;
            w[i] = unit_load<FW>(rW, row * p.ldw + kb, bytes_w - kb);
        }
    };
    auto sstore = [&](uint8_t* buf, const float (&v)[2]) {
        float* sg = reinterpret_cast<float*>(buf + SA + SW);
        sg[tid] = v[0];
        sg[kBN + tid] = v[1];
    };
    auto lstore = [&](uint8_t* buf, const uint4 (&a)[LA], const uint4 (&w)[LW]) {
#pragma unroll
        for (int i = 0; i < LA; i++) {
            const int q = tid + 256 * i, row = q >> 3, j = q & 7;
            *reinterpret_cast<uint4*>(buf + row * WA::stride + 16 * WA::slot(j)) = staged<FA>(a[i]);
        }
#pragma unroll
        for (int i = 0; i < LW; i++) {
            const int q = tid + 256 * i, row = q >> 3, j = q & 7;
            *reinterpret_cast<uint4*>(buf + SA + row * WW::stride + 16 * WW::slot(j)) = staged<FW>(w[i]);
        }
    };

    f32x16 acc[4][2];
    f32x16 tot[GRP ? 4 : 1][2];  // GRP: the sum over finished groups
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[j][i][v] = 0.0f;
    if constexpr (GRP) {
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int v = 0; v < 16; v++) tot[j][i][v] = 0.0f;
    }
    // GRP: K-block h of step t ends a group: T = fma(P, s[n, g], T) for every value, then
    // P = 0.  Value v of block (j, i) is column wn*128 + 32 j + 8 (v/4) + 4 hk + v%4 of the
    // tile.  (K-blocks past K end "groups" whose scale is 0 and whose P is 0: T stays.)
    auto fold = [&](const uint8_t* cur, int h) {
        const float* sg = reinterpret_cast<const float*>(cur + SA + SW) + h * kBN;
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const float4 s4 = *reinterpret_cast<const float4*>(&sg[wn * 128 + 32 * j + 8 * g + 4 * hk]);
                const float sc[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
                for (int i = 0; i < 2; i++)
#pragma unroll
                    for (int c = 0; c < 4; c++) {
                        tot[j][i][4 * g + c] = __builtin_fmaf(acc[j][i][4 * g + c], sc[c], tot[j][i][4 * g + c]);
                        acc[j][i][4 * g + c] = 0.0f;
                    }
            }
    };

    auto compute = [&](const uint8_t* cur, int t) {
#pragma unroll
        for (int h = 0; h < 2; h++) {
            i32x8 fa[2], fw[4];
#pragma unroll
            for (int i = 0; i < 2; i++) fa[i] = frag<FA>(cur + (wm * 64 + 32 * i + r32) * WA::stride, h, hk);
#pragma unroll
            for (int j = 0; j < 4; j++) fw[j] = frag<FW>(cur + SA + (wn * 128 + 32 * j + r32) * WW::stride, h, hk);
#pragma unroll
            for (int j = 0; j < 4; j++)
#pragma unroll
                for (int i = 0; i < 2; i++)
                    acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fw[j], fa[i], acc[j][i], WW::code,
                                                                               WA::code, 0, 127, 0, 127);
            if constexpr (GRP) {
                if (((int64_t)t * kStepCodes + 64 * (h + 1)) % p.w_group == 0) fold(cur, h);
            }
        }
        // keep the MFMAs ahead of the waits for the next units
        __builtin_amdgcn_sched_barrier(0);
    };

    // steps rounded up to a multiple of NSET; the loads of steps past K read zeros and
    // the extra steps add nothing.  Loop body without branches: every load and store is
    // unconditional.  Step t is computed from LDS buffer t % 2.
#pragma unroll
    for (int u = 0; u < NSET; u++) {
        gload(ra[u], rw[u], u);
        if constexpr (GRP) sload(rs[u], u);
    }
    lstore(smem, ra[0], rw[0]);
    if constexpr (GRP) sstore(smem, rs[0]);
    __syncthreads();
    for (int s = 0; s < nsteps; s += NSET) {
#pragma unroll
        for (int u = 0; u < NSET; u++) {
            const int t = s + u;
            uint8_t* const cur = smem + (t & 1) * BUF;
            uint8_t* const nxt = smem + ((t + 1) & 1) * BUF;
            gload(ra[u], rw[u], t + NSET);
            if constexpr (GRP) sload(rs[u], t + NSET);
            compute(cur, t);
            lstore(nxt, ra[(u + 1) % NSET], rw[(u + 1) % NSET]);
            if constexpr (GRP) sstore(nxt, rs[(u + 1) % NSET]);
            __syncthreads();
        }
    }

    // epilogue: lane (r32, hk) of block (j, i) holds Y[m][n .. n + 3] for
    // m = m0 + wm*64 + 32 i + r32 and n = n0 + wn*128 + 32 j + 8 g + 4 hk, g = 0..3
    const float a_scale = p.a_scale[0];
    const float* ws = reinterpret_cast<const float*>(p.w_scales);
    const bool vec_ok = ((p.ldy & 3) == 0) && ((reinterpret_cast<uintptr_t>(p.y) & 15) == 0);
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const int64_t n = n0 + wn * 128 + 32 * j + 8 * g + 4 * hk;
            float sn[4];
#pragma unroll
            for (int c = 0; c < 4; c++) sn[c] = GRP ? 1.0f : (p.w_mode == 1 ? ws[n + c < p.N ? n + c : p.N - 1] : ws[0]);
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const int64_t m = m0 + wm * 64 + 32 * i + r32;
                if (m >= p.M) continue;
                // one activation scale, or one per row (token) of A: y = fl32(acc * fl32(a_m * s_n))
                const float am = p.a_row ? p.a_scale[m] : a_scale;
                // GRP: y = fl32(T * a_m)
                float y[4];
#pragma unroll
                for (int c = 0; c < 4; c++)
                    y[c] = GRP ? tot[GRP ? j : 0][i][4 * g + c] * am : acc[j][i][4 * g + c] * (am * sn[c]);
                const bool vec = vec_ok && n + 3 < p.N;
                if (p.y_bf16) {
                    __bf16* yp = reinterpret_cast<__bf16*>(p.y) + m * p.ldy + n;
                    __bf16 h4[4] = {(__bf16)y[0], (__bf16)y[1], (__bf16)y[2], (__bf16)y[3]};
                    if (vec) {
                        *reinterpret_cast<uint2*>(yp) = __builtin_bit_cast(uint2, h4);
                    } else {
#pragma unroll
                        for (int c = 0; c < 4; c++)
                            if (n + c < p.N) yp[c] = h4[c];
                    }
                } else {
                    float* yp = reinterpret_cast<float*>(p.y) + m * p.ldy + n;
                    if (vec) {
                        *reinterpret_cast<float4*>(yp) = make_float4(y[0], y[1], y[2], y[3]);
                    } else {
#pragma unroll
                        for (int c = 0; c < 4; c++)
                            if (n + c < p.N) yp[c] = y[c];
                    }
                }
            }
        }
}

namespace {

template <int FW, int FA>
hipError_t launch_pair(const GemmParams& p, hipStream_t s) {
    const int64_t gm = (p.M + kBM - 1) / kBM, gn = (p.N + kBN - 1) / kBN;
    if constexpr (FW <= 3) {  // FP8 / FP6 weights: group scales
        if (p.w_mode == 2) {
            hipLaunchKernelGGL((f8f6_gemm_kernel<FW, FA, true>), dim3((unsigned)(gm * gn)), dim3(256), 0, s, p,
                               (int)gm, (int)(gm * gn));
            return hipGetLastError();
        }
    }
    if (p.w_mode == 2) return hipErrorInvalidValue;
    hipLaunchKernelGGL((f8f6_gemm_kernel<FW, FA, false>), dim3((unsigned)(gm * gn)), dim3(256), 0, s, p, (int)gm,
                       (int)(gm * gn));
    return hipGetLastError();
}

template <int FW>
hipError_t launch_w(const GemmParams& p, int fa, hipStream_t s) {
    switch (fa) {
        case 0: return launch_pair<FW, 0>(p, s);
        case 1: return launch_pair<FW, 1>(p, s);
        case 2: return launch_pair<FW, 2>(p, s);
        case 3: return launch_pair<FW, 3>(p, s);
        case 4: return launch_pair<FW, 4>(p, s);
        case 5: return launch_pair<FW, 5>(p, s);
        default: return launch_pair<FW, 6>(p, s);
    }
}

}  // namespace

// MFMA operand format code of an FP8 / FP6 / FP4 grid: 0 E4M3, 1 E5M2, 2 E2M3, 3 E3M2,
// 4 E2M1
int f8f6_format_code(const QGrid& g) {
    if (g.kind != 0) return -1;
    if (g.bits == 4) return g.is_e2m1 ? 4 : (g.e == 1 ? 5 : (g.e == 3 ? 6 : -1));
    if (g.bits == 8) return g.e == 4 && g.m == 3 ? 0 : (g.e == 5 && g.m == 2 ? 1 : -1);
    if (g.bits == 6) return g.e == 2 && g.m == 3 ? 2 : (g.e == 3 && g.m == 2 ? 3 : -1);
    return -1;
}

hipError_t launch_f8f6_gemm(const GemmParams& p, hipStream_t s) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    const int fw = f8f6_format_code(p.wg), fa = f8f6_format_code(p.ag);
    if (fw < 0 || fa < 0) return hipErrorInvalidValue;
    // per-tile buffer ranges are 32-bit: a tile's rows must span less than 2 GiB
    if ((int64_t)kBN * std::max(p.lda, p.ldw) >= 0x7fff0000) return hipErrorInvalidValue;
    if ((p.M + kBM - 1) / kBM * ((p.N + kBN - 1) / kBN) >= (int64_t)1 << 31) return hipErrorInvalidValue;
    // group scales: G a multiple of 64 dividing K; a tile's scales within the 32-bit range
    if (p.w_mode == 2 && (p.w_group < 64 || p.w_group % 64 != 0 || p.K % p.w_group != 0 ||
                          (int64_t)kBN * (p.K / p.w_group) * 4 >= 0x7fff0000))
        return hipErrorInvalidValue;
    switch (fw) {
        case 0: return launch_w<0>(p, fa, s);
        case 1: return launch_w<1>(p, fa, s);
        case 2: return launch_w<2>(p, fa, s);
        case 3: return launch_w<3>(p, fa, s);
        case 4: return launch_w<4>(p, fa, s);
        case 5: return launch_w<5>(p, fa, s);
        default: return launch_w<6>(p, fa, s);
    }
}

}  // namespace fp4

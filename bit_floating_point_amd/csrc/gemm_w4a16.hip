// W4A16: Y[m, n] = sum_u s[n, u] * sum_{k in u} x[m, k] * g(c[n, k])
// (scales factored out of the low-bit inner product: [FP4-LLM] "efficient matrix
// multiplication"; [W8A8] section 2.2 quantized_matmul; group size 128).
//
// Decode GEMV / small GEMM (M <= 16 per tile) for bf16 activations and E2M1 weights:
// HBM-bound on the packed weights.  A workgroup owns 16 output columns n and splits
// K over its 4 wavefronts.  Per 128-wide K chunk a lane streams 16 bytes (32 codes)
// of one weight row with a single 128-bit load, turns them into bf16 with the gfx950
// FP4->bf16 convert (exact), and feeds four bf16 16x16x32 MFMAs.  The 4-bit codes of
// one lane are the B operand of those MFMAs under a fixed permutation of K that the
// activation operand uses too, so no shuffles are needed.  Each scale group's partial
// sum is kept apart and multiplied by its scale in fp32 before it joins the total.
// The 4 wavefront partials are combined through LDS in a fixed order.
//
// A second, plain VALU kernel covers f32 activations and the other grids.
#include "fp4_device.h"

namespace fp4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kW16Waves = 4;
constexpr int kBatch = 4;  // K chunks in flight per wavefront

__device__ __forceinline__ bf16x8 decode_e2m1_bf16(uint32_t w) {
    // byte b of w holds codes 2b (low nibble) and 2b+1
    uint32_t o[4];
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1));
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2));
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3));
    return __builtin_bit_cast(bf16x8, o);
}

// Scale loads return raw bits; the conversion waits until the value is used, so a
// batch's loads are all in flight together.
template <bool SF16>
__device__ __forceinline__ uint32_t load_scale_raw(const GemmParams& p, int64_t idx) {
    if (SF16) return reinterpret_cast<const uint16_t*>(p.w_scales)[idx];
    return reinterpret_cast<const uint32_t*>(p.w_scales)[idx];
}

template <bool SF16>
__device__ __forceinline__ float scale_value(uint32_t raw) {
    if (SF16) return __half2float(__ushort_as_half((unsigned short)raw));
    return __uint_as_float(raw);
}

// T = 16-column tiles per wavefront (the activation registers are reused across them)
// G1: group scales with exactly one 128-wide chunk per group (group size 128)
template <int MODE, int T, bool SF16, bool G1>  // MODE 0 tensor, 1 row, 2 group
__global__ void __launch_bounds__(256) w4a16_mfma_kernel(GemmParams p) {
    __shared__ f32x4 part[kW16Waves - 1][T][64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int q = lane >> 4, r16 = lane & 15;
    const int64_t n0 = (int64_t)blockIdx.x * 16 * T;
    const int64_t m0 = (int64_t)blockIdx.y * 16;
    const int64_t m = m0 + r16;
    const bool m_ok = m < p.M;

    const int nchunks = (int)(p.K / 128);
    const int c_begin = nchunks * wave / kW16Waves;
    const int c_end = nchunks * (wave + 1) / kW16Waves;
    const int cpg = (MODE == 2 && !G1) ? p.w_group / 128 : 1;
    const int64_t ngroups = MODE == 2 ? p.K / p.w_group : 1;

    int64_t n[T];
    bool n_ok[T];
    const uint8_t* wrow[T];
#pragma unroll
    for (int t = 0; t < T; t++) {
        n[t] = n0 + t * 16 + r16;
        n_ok[t] = n[t] < p.N;
        wrow[t] = p.w + (n_ok[t] ? n[t] : 0) * p.ldw + q * 16;
    }
    const uint16_t* xrow = reinterpret_cast<const uint16_t*>(p.a) + (m_ok ? m : 0) * p.lda + q * 32;

    f32x4 total[T], gacc[T];
#pragma unroll
    for (int t = 0; t < T; t++) total[t] = gacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int c0 = c_begin; c0 < c_end; c0 += kBatch) {
        // issue every load of the batch before any arithmetic: weights, group scales and
        // activations are all independent of the MFMA chain
        uint4 wv[kBatch][T];
        uint4 xv[kBatch][4];
        uint32_t sc[kBatch][T];
        bool valid[kBatch];
        // Every load is unconditional: rows beyond N or M were pointed at row 0 above and
        // chunks past the wavefront's range re-read its last chunk (their codes are then
        // zeroed).  Values of rows beyond N or M only reach outputs that are never
        // stored.  No load sits inside a branch, which would force a wait on all loads
        // in flight.
#pragma unroll
        for (int b = 0; b < kBatch; b++) {
            valid[b] = c0 + b < c_end;
            const int c = valid[b] ? c0 + b : c_end - 1;
#pragma unroll
            for (int t = 0; t < T; t++) {
                wv[b][t] = *reinterpret_cast<const uint4*>(wrow[t] + (int64_t)c * 64);
                if (MODE == 2) sc[b][t] = load_scale_raw<SF16>(p, (n_ok[t] ? n[t] : 0) * ngroups + (G1 ? c : c / cpg));
            }
#pragma unroll
            for (int j = 0; j < 4; j++) xv[b][j] = *reinterpret_cast<const uint4*>(xrow + (int64_t)c * 128 + j * 8);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < kBatch; b++) {
            const int c = c0 + b;
#pragma unroll
            for (int t = 0; t < T; t++) {
                const uint4 w = valid[b] ? wv[b][t] : make_uint4(0, 0, 0, 0);
                const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
                f32x4 acc = G1 ? f32x4{0.f, 0.f, 0.f, 0.f} : gacc[t];
#pragma unroll
                for (int j = 0; j < 4; j++)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xv[b][j]),
                                                                  decode_e2m1_bf16(wd[j]), acc, 0, 0, 0);
                if (G1) {
                    // one group per chunk: scale its partial sum and add it (no branch)
                    const float sv = scale_value<SF16>(sc[b][t]);
#pragma unroll
                    for (int i = 0; i < 4; i++) total[t][i] = __builtin_fmaf(acc[i], sv, total[t][i]);
                } else {
                    gacc[t] = acc;
                }
            }
            if (MODE == 2 && !G1 && valid[b] && (c + 1) % cpg == 0) {
#pragma unroll
                for (int t = 0; t < T; t++) {
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        total[t][i] = __builtin_fmaf(gacc[t][i], scale_value<SF16>(sc[b][t]), total[t][i]);
                    gacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < T; t++) {
        if (MODE == 2 && !G1 && c_end > c_begin && (c_end % cpg) != 0) {
            // this wavefront's range ends inside a group: scale its share of that group
            float s = n_ok[t] ? scale_value<SF16>(load_scale_raw<SF16>(p, n[t] * ngroups + (c_end - 1) / cpg)) : 0.0f;
#pragma unroll
            for (int i = 0; i < 4; i++) total[t][i] = __builtin_fmaf(gacc[t][i], s, total[t][i]);
        }
        if (MODE != 2) {
            float s = n_ok[t] ? scale_value<SF16>(load_scale_raw<SF16>(p, MODE == 1 ? n[t] : 0)) : 0.0f;
#pragma unroll
            for (int i = 0; i < 4; i++) total[t][i] = gacc[t][i] * s;
        }
        if (wave > 0) part[wave - 1][t][lane] = total[t];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int t = 0; t < T; t++) {
#pragma unroll
            for (int w = 0; w < kW16Waves - 1; w++) {
                f32x4 o = part[w][t][lane];
#pragma unroll
                for (int i = 0; i < 4; i++) total[t][i] += o[i];
            }
            // D layout of a 16x16 MFMA: lane holds rows 4*(lane/16) + i of column lane%16
            if (!n_ok[t]) continue;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                int64_t mm = m0 + 4 * q + i;
                if (mm < p.M) {
                    if (p.y_bf16) reinterpret_cast<__bf16*>(p.y)[mm * p.ldy + n[t]] = (__bf16)total[t][i];
                    else reinterpret_cast<float*>(p.y)[mm * p.ldy + n[t]] = total[t][i];
                }
            }
        }
    }
}

template <int T, bool SF16>
static void launch_w16(const GemmParams& p, hipStream_t s) {
    dim3 grid((unsigned)((p.N + 16 * T - 1) / (16 * T)), (unsigned)((p.M + 15) / 16));
    if (p.w_mode == 2 && p.w_group == 128) hipLaunchKernelGGL((w4a16_mfma_kernel<2, T, SF16, true>), grid, dim3(256), 0, s, p);
    else if (p.w_mode == 2) hipLaunchKernelGGL((w4a16_mfma_kernel<2, T, SF16, false>), grid, dim3(256), 0, s, p);
    else if (p.w_mode == 1) hipLaunchKernelGGL((w4a16_mfma_kernel<1, T, SF16, false>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((w4a16_mfma_kernel<0, T, SF16, false>), grid, dim3(256), 0, s, p);
}

// ---------------------------------------------------------------------------------
// Decode GEMV for M <= 8 (the latency-critical case).  The activations (M x K bf16,
// at most 64 KB) are staged once per workgroup in LDS; each wavefront then issues the
// loads of all its weight chunks (up to 8 x 16 B per lane) and their group scales at
// once, so a CU keeps its whole share of the weight stream in flight and pays one
// HBM round trip instead of one per batch.  A fragments come from LDS (rows >= M read
// row 0: they only feed output rows that are never stored).
constexpr int kGemvChunks = 8;  // weight chunks per wavefront per round

template <int MODE, bool SF16, int XPT>  // MODE 0 tensor, 1 row, 2 group of 128
__global__ void __launch_bounds__(256) w4a16_gemv_kernel(GemmParams p) {
    extern __shared__ uint4 xs[];  // [M][K/8] 16-byte vectors of bf16
    __shared__ f32x4 part[kW16Waves - 1][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q = lane >> 4, r16 = lane & 15;
    const int64_t n = (int64_t)blockIdx.x * 16 + r16;
    const bool n_ok = n < p.N;
    const int64_t nrow = n_ok ? n : 0;
    const int kv = (int)(p.K / 8);  // 16-byte vectors per activation row
    const int xvec = (int)p.M * kv;
    const int nchunks = (int)(p.K / 128);
    const int c_begin = nchunks * wave / kW16Waves;
    const int c_end = nchunks * (wave + 1) / kW16Waves;
    const int64_t ngroups = MODE == 2 ? p.K / 128 : 1;
    const uint8_t* wrow = p.w + nrow * p.ldw + q * 16;
    const uint16_t* X = reinterpret_cast<const uint16_t*>(p.a);

    // 1. activation loads first (L2-resident, shared by every workgroup)
    uint4 xr[XPT];
#pragma unroll
    for (int i = 0; i < XPT; i++) {
        int idx = tid + 256 * i;
        idx = idx < xvec ? idx : xvec - 1;  // past the activations: re-read the last vector
        unsigned r = (unsigned)idx / (unsigned)kv, cc = (unsigned)idx % (unsigned)kv;
        xr[i] = *reinterpret_cast<const uint4*>(X + (int64_t)r * p.lda + (int64_t)cc * 8);
    }
    // 2. the first round of weight chunks and scales (loads and LDS stores are
    // unconditional -- a chunk past the range re-reads a valid one, a vector past the
    // activations goes to a spare LDS slot -- so no load is sunk into a branch where it
    // would be waited for at once)
    uint4 wv[kGemvChunks];
    uint32_t sc[kGemvChunks];
#pragma unroll
    for (int b = 0; b < kGemvChunks; b++) {
        int c = c_begin + b < c_end ? c_begin + b : c_end - 1;
        c = c < 0 ? 0 : c;
        wv[b] = *reinterpret_cast<const uint4*>(wrow + (int64_t)c * 64);
        if (MODE == 2) sc[b] = load_scale_raw<SF16>(p, nrow * ngroups + c);
    }
    // 3. activations into LDS
#pragma unroll
    for (int i = 0; i < XPT; i++) {
        int idx = tid + 256 * i;
        xs[idx < xvec ? idx : xvec + tid] = xr[i];
    }
    __syncthreads();

    const int xrow = (r16 < p.M ? r16 : 0) * kv;
    f32x4 total = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = c_begin; c0 < c_end; c0 += kGemvChunks) {
#pragma unroll
        for (int b = 0; b < kGemvChunks; b++) {
            const int c = c0 + b;
            const bool valid = c < c_end;
            const uint4 w = valid ? wv[b] : make_uint4(0, 0, 0, 0);
            const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
            const int cc = valid ? c : c_begin;
            f32x4 acc = MODE == 2 ? f32x4{0.f, 0.f, 0.f, 0.f} : total;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                uint4 a = xs[xrow + cc * 16 + q * 4 + j];
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), decode_e2m1_bf16(wd[j]),
                                                              acc, 0, 0, 0);
            }
            if (MODE == 2) {
                const float sv = valid ? scale_value<SF16>(sc[b]) : 0.0f;
#pragma unroll
                for (int i = 0; i < 4; i++) total[i] = __builtin_fmaf(acc[i], sv, total[i]);
            } else {
                total = acc;
            }
        }
        if (c0 + kGemvChunks < c_end) {
#pragma unroll
            for (int b = 0; b < kGemvChunks; b++) {
                int c = c0 + kGemvChunks + b < c_end ? c0 + kGemvChunks + b : c_end - 1;
                wv[b] = *reinterpret_cast<const uint4*>(wrow + (int64_t)c * 64);
                if (MODE == 2) sc[b] = load_scale_raw<SF16>(p, nrow * ngroups + c);
            }
        }
    }
    if (MODE != 2) {
        float s = scale_value<SF16>(load_scale_raw<SF16>(p, MODE == 1 ? nrow : 0));
#pragma unroll
        for (int i = 0; i < 4; i++) total[i] = total[i] * s;
    }
    if (wave > 0) part[wave - 1][lane] = total;
    __syncthreads();
    if (wave == 0 && n_ok) {
#pragma unroll
        for (int w = 0; w < kW16Waves - 1; w++) {
            f32x4 o = part[w][lane];
#pragma unroll
            for (int i = 0; i < 4; i++) total[i] += o[i];
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
            int64_t mm = 4 * q + i;
            if (mm < p.M) {
                if (p.y_bf16) reinterpret_cast<__bf16*>(p.y)[mm * p.ldy + n] = (__bf16)total[i];
                else reinterpret_cast<float*>(p.y)[mm * p.ldy + n] = total[i];
            }
        }
    }
}

template <int MODE, bool SF16>
static void launch_gemv(const GemmParams& p, hipStream_t s) {
    dim3 grid((unsigned)((p.N + 15) / 16));
    size_t lds = (size_t)p.M * p.K * 2 + 256 * 16;  // activations + one spare slot per thread
    int xpt = (int)((p.M * p.K / 8 + 255) / 256);
    if (xpt <= 2) hipLaunchKernelGGL((w4a16_gemv_kernel<MODE, SF16, 2>), grid, dim3(256), lds, s, p);
    else if (xpt <= 4) hipLaunchKernelGGL((w4a16_gemv_kernel<MODE, SF16, 4>), grid, dim3(256), lds, s, p);
    else if (xpt <= 8) hipLaunchKernelGGL((w4a16_gemv_kernel<MODE, SF16, 8>), grid, dim3(256), lds, s, p);
    else hipLaunchKernelGGL((w4a16_gemv_kernel<MODE, SF16, 16>), grid, dim3(256), lds, s, p);
}

hipError_t launch_w4a16_mfma(const GemmParams& p, hipStream_t s) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    const bool gemv = p.M <= 8 && p.M * p.K <= 32768 && (p.w_mode != 2 || p.w_group == 128);
    if (gemv) {
        const int mode = p.w_mode;
        if (p.w_scale_f16) {
            if (mode == 2) launch_gemv<2, true>(p, s);
            else if (mode == 1) launch_gemv<1, true>(p, s);
            else launch_gemv<0, true>(p, s);
        } else {
            if (mode == 2) launch_gemv<2, false>(p, s);
            else if (mode == 1) launch_gemv<1, false>(p, s);
            else launch_gemv<0, false>(p, s);
        }
        return hipGetLastError();
    }
    // larger M: reuse each activation fragment for two weight tiles
    if (p.M > 8) {
        if (p.w_scale_f16) launch_w16<2, true>(p, s);
        else launch_w16<2, false>(p, s);
    } else {
        if (p.w_scale_f16) launch_w16<1, true>(p, s);
        else launch_w16<1, false>(p, s);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Plain VALU kernel: one thread per output element, any grid, f32 or bf16
// activations, any scale granularity.  Used for small problems (and as the general
// case): per scale unit the partial sum of x * g(c) is formed with fp32 FMAs and then
// multiplied by the unit's scale.
__global__ void __launch_bounds__(256) w4a16_valu_kernel(GemmParams p) {
    int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= p.M * p.N) return;
    int64_t m = idx / p.N, n = idx % p.N;
    const uint8_t* wr = p.w + n * p.ldw;
    int64_t unit = p.w_mode == 2 ? p.w_group : p.K;
    float total = 0.0f;
    for (int64_t k0 = 0; k0 < p.K; k0 += unit) {
        float part = 0.0f;
        for (int64_t k = k0; k < k0 + unit; k++) {
            uint32_t c = (wr[k >> 1] >> (4 * (k & 1))) & 15u;
            float xv = p.a_kind == 1 ? bf16_bits_to_float(reinterpret_cast<const uint16_t*>(p.a)[m * p.lda + k])
                                     : reinterpret_cast<const float*>(p.a)[m * p.lda + k];
            part = __builtin_fmaf(xv, grid_value(c, p.wg), part);
        }
        int64_t u = p.w_mode == 0 ? 0 : (p.w_mode == 1 ? n : n * (p.K / p.w_group) + k0 / p.w_group);
        float s = p.w_scale_f16 ? __half2float(reinterpret_cast<const __half*>(p.w_scales)[u])
                                : reinterpret_cast<const float*>(p.w_scales)[u];
        total = __builtin_fmaf(part, s, total);
    }
    if (p.y_bf16) reinterpret_cast<__bf16*>(p.y)[m * p.ldy + n] = (__bf16)total;
    else reinterpret_cast<float*>(p.y)[m * p.ldy + n] = total;
}

hipError_t launch_w4a16_valu(const GemmParams& p, hipStream_t s) {
    int64_t n = p.M * p.N;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(w4a16_valu_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace fp4

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

struct U4 { uint32_t v[4]; };

__device__ __forceinline__ bf16x8 decode_e2m1_bf16(uint32_t w) {
    // byte b of w holds codes 2b (low nibble) and 2b+1
    uint32_t o[4];
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1));
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2));
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3));
    return __builtin_bit_cast(bf16x8, o);
}

template <int MODE>  // 0 tensor, 1 row, 2 group
__global__ void __launch_bounds__(256) w4a16_mfma_kernel(GemmParams p) {
    __shared__ f32x4 part[kW16Waves - 1][64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t m0 = (int64_t)blockIdx.y * 16;
    const int64_t n = n0 + (lane & 15);
    const int q = lane >> 4;
    const int64_t m = m0 + (lane & 15);
    const bool n_ok = n < p.N;
    const bool m_ok = m < p.M;

    const int64_t nchunks = p.K / 128;
    const int64_t c_begin = nchunks * wave / kW16Waves;
    const int64_t c_end = nchunks * (wave + 1) / kW16Waves;
    const int chunks_per_group = MODE == 2 ? p.w_group / 128 : 1;
    const int64_t ngroups = MODE == 2 ? p.K / p.w_group : 1;

    const uint8_t* wrow = p.w + (n_ok ? n : 0) * p.ldw + q * 16;
    const uint16_t* xrow = reinterpret_cast<const uint16_t*>(p.a) + (m_ok ? m : 0) * p.lda + q * 32;

    f32x4 total = {0.f, 0.f, 0.f, 0.f};
    f32x4 gacc = {0.f, 0.f, 0.f, 0.f};

    for (int64_t c0 = c_begin; c0 < c_end; c0 += kBatch) {
        uint4 wv[kBatch];
        uint4 xv[kBatch][4];
#pragma unroll
        for (int b = 0; b < kBatch; b++) {
            int64_t c = c0 + b;
            if (c < c_end && n_ok) wv[b] = *reinterpret_cast<const uint4*>(wrow + c * 64);
            else wv[b] = make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; j++) {
                if (c < c_end && m_ok) xv[b][j] = *reinterpret_cast<const uint4*>(xrow + c * 128 + j * 8);
                else xv[b][j] = make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int b = 0; b < kBatch; b++) {
            int64_t c = c0 + b;
            if (c >= c_end) break;
            uint32_t wd[4] = {wv[b].x, wv[b].y, wv[b].z, wv[b].w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                bf16x8 bop = decode_e2m1_bf16(wd[j]);
                bf16x8 aop = __builtin_bit_cast(bf16x8, xv[b][j]);
                gacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, bop, gacc, 0, 0, 0);
            }
            if (MODE == 2) {
                if ((c + 1) % chunks_per_group == 0) {
                    int64_t g = c / chunks_per_group;
                    float s = 0.0f;
                    if (n_ok) s = p.w_scale_f16 ? __half2float(reinterpret_cast<const __half*>(p.w_scales)[n * ngroups + g])
                                                : reinterpret_cast<const float*>(p.w_scales)[n * ngroups + g];
#pragma unroll
                    for (int i = 0; i < 4; i++) total[i] = __builtin_fmaf(gacc[i], s, total[i]);
                    gacc = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
    }
    if (MODE == 2 && c_end > c_begin && (c_end % chunks_per_group) != 0) {
        // this wavefront's range ends inside a group: scale its share of that group
        int64_t g = (c_end - 1) / chunks_per_group;
        float s = 0.0f;
        if (n_ok) s = p.w_scale_f16 ? __half2float(reinterpret_cast<const __half*>(p.w_scales)[n * ngroups + g])
                                    : reinterpret_cast<const float*>(p.w_scales)[n * ngroups + g];
#pragma unroll
        for (int i = 0; i < 4; i++) total[i] = __builtin_fmaf(gacc[i], s, total[i]);
    }
    if (MODE != 2) {
        float s = 0.0f;
        if (n_ok) {
            int64_t u = MODE == 1 ? n : 0;
            s = p.w_scale_f16 ? __half2float(reinterpret_cast<const __half*>(p.w_scales)[u])
                              : reinterpret_cast<const float*>(p.w_scales)[u];
        }
#pragma unroll
        for (int i = 0; i < 4; i++) total[i] = gacc[i] * s;
    }
    if (wave > 0) part[wave - 1][lane] = total;
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int w = 0; w < kW16Waves - 1; w++) {
            f32x4 o = part[w][lane];
#pragma unroll
            for (int i = 0; i < 4; i++) total[i] += o[i];
        }
        // D layout of a 16x16 MFMA: lane holds rows 4*(lane/16) + i of column lane%16
        if (n_ok) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                int64_t mm = m0 + 4 * q + i;
                if (mm < p.M) {
                    float v = total[i];
                    if (p.y_bf16) {
                        __bf16 h = (__bf16)v;
                        reinterpret_cast<__bf16*>(p.y)[mm * p.ldy + n] = h;
                    } else {
                        reinterpret_cast<float*>(p.y)[mm * p.ldy + n] = v;
                    }
                }
            }
        }
    }
}

hipError_t launch_w4a16_mfma(const GemmParams& p, hipStream_t s) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    dim3 grid((unsigned)((p.N + 15) / 16), (unsigned)((p.M + 15) / 16));
    if (p.w_mode == 2) hipLaunchKernelGGL(w4a16_mfma_kernel<2>, grid, dim3(256), 0, s, p);
    else if (p.w_mode == 1) hipLaunchKernelGGL(w4a16_mfma_kernel<1>, grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL(w4a16_mfma_kernel<0>, grid, dim3(256), 0, s, p);
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

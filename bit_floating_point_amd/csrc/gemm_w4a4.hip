// W4A4 prefill GEMM on the gfx950 FP4 matrix cores:
//   Y[m, n] = fl32(acc[m, n] * fl32(a * s_n)),  acc = sum_k A_q[m, k] * W_q[n, k]
// with A_q, W_q E2M1 codes ([FP4-LLM] FP quantization of weights and activations,
// the scaling factors taken out of the low-bit product: "efficient matrix
// multiplication"; per-tensor activation scale a from the pre-shifted exponent bias,
// per-output-channel weight scale s_n).  Every E2M1 product is a multiple of 1/4
// below 36 in magnitude, so acc is exact in fp32 for any K < 2^17 and any order of
// accumulation: the result is bit-reproducible.
//
// Tiling for CDNA4: a 256-thread workgroup (2x2 wavefronts) computes a BM x BN tile of
// Y; each wavefront a (BM/2) x (BN/2) sub-tile as a grid of 16x16 accumulators fed by
// v_mfma_scale_f32_16x16x128_f8f6f4 (both operands FP4, unit E8M0 scales).  K advances
// 128 codes (64 bytes per row) per step.  Packed codes stream HBM -> VGPR -> LDS with
// 16-byte loads, double-buffered in LDS (one barrier per step); the 16-byte segments of
// a row are XOR-swizzled so a wavefront's 128-bit LDS reads hit distinct banks.  The
// FP4 operand layout of the MFMA is "lane l holds 32 consecutive codes of row l%16",
// which is exactly a 16-byte read of a K-contiguous packed row.
#include "fp4_device.h"

namespace fp4 {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBKBytes = 64;  // 128 codes per K step

__device__ __forceinline__ int swz(int row, int seg) { return row * kBKBytes + ((seg ^ ((row >> 1) & 3)) << 4); }

template <int BM, int BN>
__global__ void __launch_bounds__(256) w4a4_fp4_kernel(GemmParams p, int grid_m) {
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int LA = BM * 4 / 256, LB = BN * 4 / 256;  // 16-byte loads per thread per step
    __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * kBKBytes];
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * kBKBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int bm = blockIdx.x % grid_m;
    const int bn = blockIdx.x / grid_m;
    const int64_t m0 = (int64_t)bm * BM, n0 = (int64_t)bn * BN;
    const int64_t nk = (p.K + 127) / 128;
    const uint8_t* A = reinterpret_cast<const uint8_t*>(p.a);

    // Loads are unconditional (out-of-range rows and K tails read a valid address and
    // are then zeroed with a select), so the main loop is one basic block and the
    // scheduler keeps the LDS stores after the MFMAs.
    uint4 ra[LA], rb[LB];
    auto gload = [&](int64_t kb) {
#pragma unroll
        for (int i = 0; i < LA; i++) {
            int s = tid + 256 * i, row = s >> 2, seg = s & 3;
            int64_t gm = m0 + row, kc = kb * 128 + seg * 32;
            bool ok = gm < p.M && kc < p.K;
            uint4 v = *reinterpret_cast<const uint4*>(ok ? A + gm * p.lda + kb * kBKBytes + seg * 16 : A);
            ra[i] = ok ? v : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < LB; i++) {
            int s = tid + 256 * i, row = s >> 2, seg = s & 3;
            int64_t gn = n0 + row, kc = kb * 128 + seg * 32;
            bool ok = gn < p.N && kc < p.K;
            uint4 v = *reinterpret_cast<const uint4*>(ok ? p.w + gn * p.ldw + kb * kBKBytes + seg * 16 : p.w);
            rb[i] = ok ? v : make_uint4(0, 0, 0, 0);
        }
    };
    auto sstore = [&](int st) {
#pragma unroll
        for (int i = 0; i < LA; i++) {
            int s = tid + 256 * i, row = s >> 2, seg = s & 3;
            *reinterpret_cast<uint4*>(&sA[st][swz(row, seg)]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < LB; i++) {
            int s = tid + 256 * i, row = s >> 2, seg = s & 3;
            *reinterpret_cast<uint4*>(&sB[st][swz(row, seg)]) = rb[i];
        }
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    gload(0);
    sstore(0);
    __syncthreads();
    const int q = lane >> 4, r16 = lane & 15;
    for (int64_t kb = 0; kb < nk; kb++) {
        const int st = (int)(kb & 1);
        gload(kb + 1 < nk ? kb + 1 : kb);  // the last step reloads itself into the idle stage
        i32x8 af[TM];
#pragma unroll
        for (int i = 0; i < TM; i++) {
            uint4 v = *reinterpret_cast<const uint4*>(&sA[st][swz(wm * WM + i * 16 + r16, q)]);
            af[i] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        }
#pragma unroll
        for (int j = 0; j < TN; j++) {
            uint4 v = *reinterpret_cast<const uint4*>(&sB[st][swz(wn * WN + j * 16 + r16, q)]);
            i32x8 bf = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < TM; i++)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bf, acc[i][j], 4, 4, 0, 127, 0, 127);
        }
        // keep the LDS stores (which wait for this step's global loads) after the MFMAs,
        // so the loads for step kb+1 overlap the matrix work of step kb
        __builtin_amdgcn_sched_barrier(0);
        sstore(st ^ 1);
        __syncthreads();
    }

    // epilogue: y = fl32(acc * fl32(a * s_n)); lane holds rows 4*(lane/16)+t of column lane%16
    const float a = p.a_scale[0];
#pragma unroll
    for (int j = 0; j < TN; j++) {
        int64_t n = n0 + wn * WN + j * 16 + r16;
        if (n >= p.N) continue;
        float sn = p.w_mode == 1 ? reinterpret_cast<const float*>(p.w_scales)[n]
                                 : reinterpret_cast<const float*>(p.w_scales)[0];
        float f = a * sn;
#pragma unroll
        for (int i = 0; i < TM; i++) {
#pragma unroll
            for (int t = 0; t < 4; t++) {
                int64_t m = m0 + wm * WM + i * 16 + q * 4 + t;
                if (m < p.M) {
                    float y = acc[i][j][t] * f;
                    if (p.y_bf16) reinterpret_cast<__bf16*>(p.y)[m * p.ldy + n] = (__bf16)y;
                    else reinterpret_cast<float*>(p.y)[m * p.ldy + n] = y;
                }
            }
        }
    }
}

hipError_t launch_w4a4_fp4(const GemmParams& p, hipStream_t s) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    int64_t gm256 = (p.M + 255) / 256, gn256 = (p.N + 255) / 256;
    if (gm256 * gn256 >= 384) {
        hipLaunchKernelGGL((w4a4_fp4_kernel<256, 256>), dim3((unsigned)(gm256 * gn256)), dim3(256), 0, s, p,
                           (int)gm256);
    } else {
        int64_t gm = (p.M + 127) / 128, gn = (p.N + 127) / 128;
        hipLaunchKernelGGL((w4a4_fp4_kernel<128, 128>), dim3((unsigned)(gm * gn)), dim3(256), 0, s, p, (int)gm);
    }
    return hipGetLastError();
}

}  // namespace fp4

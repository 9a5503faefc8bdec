// W4A4 GEMM with a 16-entry lookup grid on the weights (NF4: "量化技术详解" page,
// section NF4, levels at quantiles of the normal distribution) and E2M1 activations
// with the pre-shifted per-tensor scale a:
//   Y[m, n] = a * sum_g s[n, g] * sum_{k in g} A_q[m, k] * G[c[n, k]]
// Scales stay outside the low-bit products ([FP4-LLM] "efficient matrix
// multiplication"): each K group's partial sum is formed on the matrix cores and only
// then multiplied by its fp32 block scale.
//
// gfx950 has no matrix instruction for an arbitrary 16-value grid, so both operands
// are decoded to f16 in registers (E2M1 via the FP4->f16 convert; the lookup grid via
// byte permutes of a 32-byte table held in scalar registers; both exact because the
// grid values are binary16 numbers) and fed to v_mfma_f32_16x16x32_f16.
// Tiling: 128x128 output tile per 256-thread workgroup, 64x64 per wavefront (4x4
// accumulators), K step = one 64-code group; packed codes staged in LDS, double
// buffered, 8-byte segments XOR-swizzled against bank conflicts.
#include "fp4_device.h"

namespace fp4 {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kLutBM = 128, kLutBN = 128, kLutBK = 64;  // BK in codes
constexpr int kRowBytes = kLutBK / 2;                    // 32

__device__ __forceinline__ int swz8(int row, int q) { return row * kRowBytes + ((q ^ ((row >> 2) & 3)) << 3); }

__device__ __forceinline__ f16x8 decode_e2m1_f16(uint32_t w) {
    uint32_t o[4];
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1));
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2));
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3));
    return __builtin_bit_cast(f16x8, o);
}

// byte lookup T[idx] for the 4 byte-indices (0..15) of idx; T is 16 bytes in 4 words
__device__ __forceinline__ uint32_t lut_bytes(uint32_t idx, const uint32_t T[4]) {
    uint32_t i7 = idx & 0x07070707u;
    uint32_t lo = __builtin_amdgcn_perm(T[1], T[0], i7);
    uint32_t hi = __builtin_amdgcn_perm(T[3], T[2], i7);
    uint32_t msk = ((idx >> 3) & 0x01010101u) * 0xFFu;
    return (hi & msk) | (lo & ~msk);
}

// 8 lookup-grid codes (element 2j in the low nibble of byte j) -> 8 f16 values
__device__ __forceinline__ f16x8 decode_lut_f16(uint32_t w, const uint32_t TL[4], const uint32_t TH[4]) {
    uint32_t ev = w & 0x0F0F0F0Fu, od = (w >> 4) & 0x0F0F0F0Fu;
    uint32_t eL = lut_bytes(ev, TL), eH = lut_bytes(ev, TH);
    uint32_t oL = lut_bytes(od, TL), oH = lut_bytes(od, TH);
    uint32_t e01 = __builtin_amdgcn_perm(eH, eL, 0x05010400u);  // f16(x0) | f16(x2) << 16
    uint32_t e23 = __builtin_amdgcn_perm(eH, eL, 0x07030602u);  // f16(x4) | f16(x6) << 16
    uint32_t o01 = __builtin_amdgcn_perm(oH, oL, 0x05010400u);  // f16(x1) | f16(x3) << 16
    uint32_t o23 = __builtin_amdgcn_perm(oH, oL, 0x07030602u);  // f16(x5) | f16(x7) << 16
    uint32_t o[4];
    o[0] = __builtin_amdgcn_perm(o01, e01, 0x05040100u);
    o[1] = __builtin_amdgcn_perm(o01, e01, 0x07060302u);
    o[2] = __builtin_amdgcn_perm(o23, e23, 0x05040100u);
    o[3] = __builtin_amdgcn_perm(o23, e23, 0x07060302u);
    return __builtin_bit_cast(f16x8, o);
}

__global__ void __launch_bounds__(256) w4a4_lut_kernel(GemmParams p, int grid_m) {
    __shared__ __attribute__((aligned(16))) uint8_t sA[2][kLutBM * kRowBytes];
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][kLutBN * kRowBytes];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int64_t m0 = (int64_t)(blockIdx.x % grid_m) * kLutBM;
    const int64_t n0 = (int64_t)(blockIdx.x / grid_m) * kLutBN;
    const int64_t nk = p.K / kLutBK;
    const int steps_per_group = p.w_group / kLutBK;
    const int64_t ngroups = p.K / p.w_group;
    const uint8_t* A = reinterpret_cast<const uint8_t*>(p.a);

    // f16 bit patterns of the 16 grid values, split into low and high byte tables
    uint32_t TL[4] = {0, 0, 0, 0}, TH[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 16; i++) {
        uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)p.wg.val[i]);
        TL[i >> 2] |= (h & 0xffu) << (8 * (i & 3));
        TH[i >> 2] |= (h >> 8) << (8 * (i & 3));
    }

    // global -> LDS: 128 rows x 32 bytes per operand = 256 x 16 B, one load per thread
    const int lrow = tid >> 1, lseg = tid & 1;
    uint4 ra, rb;
    // unconditional loads (out-of-range rows read row 0 and are zeroed by a select): one
    // basic block per K step, so the LDS stores stay after the MFMAs
    auto gload = [&](int64_t kb) {
        int64_t gm = m0 + lrow, gn = n0 + lrow;
        bool oka = gm < p.M, okb = gn < p.N;
        uint4 va = *reinterpret_cast<const uint4*>(A + (oka ? gm : 0) * p.lda + kb * kRowBytes + lseg * 16);
        uint4 vb = *reinterpret_cast<const uint4*>(p.w + (okb ? gn : 0) * p.ldw + kb * kRowBytes + lseg * 16);
        ra = oka ? va : make_uint4(0, 0, 0, 0);
        rb = okb ? vb : make_uint4(0, 0, 0, 0);
    };
    auto sstore = [&](int st) {
        // the 16-byte segment holds two 8-byte units q = 2*lseg, 2*lseg+1
        *reinterpret_cast<uint2*>(&sA[st][swz8(lrow, 2 * lseg)]) = make_uint2(ra.x, ra.y);
        *reinterpret_cast<uint2*>(&sA[st][swz8(lrow, 2 * lseg + 1)]) = make_uint2(ra.z, ra.w);
        *reinterpret_cast<uint2*>(&sB[st][swz8(lrow, 2 * lseg)]) = make_uint2(rb.x, rb.y);
        *reinterpret_cast<uint2*>(&sB[st][swz8(lrow, 2 * lseg + 1)]) = make_uint2(rb.z, rb.w);
    };

    f32x4 acc[4][4], blk[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = blk[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int q = lane >> 4, r16 = lane & 15;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int64_t kb = 0; kb < nk; kb++) {
        const int st = (int)(kb & 1);
        gload(kb + 1 < nk ? kb + 1 : kb);
        // lane holds codes [q*16, q*16+16) of its row: sub-step u uses the u-th 8
        f16x8 af[4][2];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            uint2 v = *reinterpret_cast<const uint2*>(&sA[st][swz8(wm * 64 + i * 16 + r16, q)]);
            af[i][0] = decode_e2m1_f16(v.x);
            af[i][1] = decode_e2m1_f16(v.y);
        }
#pragma unroll
        for (int j = 0; j < 4; j++) {
            uint2 v = *reinterpret_cast<const uint2*>(&sB[st][swz8(wn * 64 + j * 16 + r16, q)]);
            f16x8 b0 = decode_lut_f16(v.x, TL, TH);
            f16x8 b1 = decode_lut_f16(v.y, TL, TH);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                blk[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i][0], b0, blk[i][j], 0, 0, 0);
                blk[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i][1], b1, blk[i][j], 0, 0, 0);
            }
        }
        if ((kb + 1) % steps_per_group == 0) {
            int64_t g = kb / steps_per_group;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                int64_t n = n0 + wn * 64 + j * 16 + r16;
                float s = 0.0f;
                if (n < p.N) s = p.w_scale_f16 ? __half2float(reinterpret_cast<const __half*>(p.w_scales)[n * ngroups + g])
                                               : reinterpret_cast<const float*>(p.w_scales)[n * ngroups + g];
#pragma unroll
                for (int i = 0; i < 4; i++) {
#pragma unroll
                    for (int t = 0; t < 4; t++) acc[i][j][t] = __builtin_fmaf(blk[i][j][t], s, acc[i][j][t]);
                    blk[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
        // keep the LDS stores (which wait for this step's global loads) after the MFMAs,
        // so the loads for step kb+1 overlap the matrix work of step kb
        __builtin_amdgcn_sched_barrier(0);
        sstore(st ^ 1);
        __syncthreads();
    }

    const float a = p.a_scale[0];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        int64_t n = n0 + wn * 64 + j * 16 + r16;
        if (n >= p.N) continue;
#pragma unroll
        for (int i = 0; i < 4; i++) {
#pragma unroll
            for (int t = 0; t < 4; t++) {
                int64_t m = m0 + wm * 64 + i * 16 + q * 4 + t;
                if (m < p.M) {
                    float y = acc[i][j][t] * a;
                    if (p.y_bf16) reinterpret_cast<__bf16*>(p.y)[m * p.ldy + n] = (__bf16)y;
                    else reinterpret_cast<float*>(p.y)[m * p.ldy + n] = y;
                }
            }
        }
    }
}

hipError_t launch_w4a4_lut(const GemmParams& p, hipStream_t s) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    int64_t gm = (p.M + kLutBM - 1) / kLutBM, gn = (p.N + kLutBN - 1) / kLutBN;
    hipLaunchKernelGGL(w4a4_lut_kernel, dim3((unsigned)(gm * gn)), dim3(256), 0, s, p, (int)gm);
    return hipGetLastError();
}

}  // namespace fp4

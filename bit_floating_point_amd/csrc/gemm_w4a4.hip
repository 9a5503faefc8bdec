// W4A4 prefill GEMM on the gfx950 FP4 matrix cores:
//   Y[m, n] = fl32(acc[m, n] * fl32(a * s_n)),  acc = sum_k A_q[m, k] * W_q[n, k]
// with A_q, W_q E2M1 codes ([FP4-LLM] FP quantization of weights and activations,
// the scaling factors taken out of the low-bit product: "efficient matrix
// multiplication"; per-tensor activation scale a from the pre-shifted exponent bias,
// per-output-channel weight scale s_n).  Every E2M1 product is a multiple of 1/4
// at most 36 in magnitude, so every partial sum is a quarter-integer below 36 K; for
// K <= 116508 (36 K < 2^22) all of them are exact in fp32, in any order of
// accumulation: the result is bit-reproducible.
//
// Tiling for CDNA4: a 256-thread workgroup (2x2 wavefronts) computes a BM x BN tile of
// Y (256x256 when the grid of such tiles fills the chip, else 128x128); each wavefront
// a (BM/2) x (BN/2) sub-tile as a grid of 32x32 accumulators.  K advances 128 codes
// (64 bytes per row) per step through a four-stage LDS ring fed by direct-to-LDS loads.
#include <algorithm>

#include "fp4_device.h"

namespace fp4 {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBKBytes = 64;  // 128 codes per K step

__device__ __forceinline__ int swz(int row, int seg) { return row * kBKBytes + ((seg ^ ((row >> 1) & 3)) << 4); }

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Operands move HBM -> LDS with gfx950's direct-to-LDS buffer loads (no staging
// registers): lane l of a wavefront writes LDS bytes [16 l, 16 l + 16) of a 1 KiB block,
// so each lane fetches the global 16-byte piece that belongs at that slot of the
// XOR-swizzled tile (the 16-byte segments of a row are permuted by row so that the
// 128-bit LDS reads of a wavefront spread over all banks).  Rows past M or N and K
// tails get an offset past the buffer's end, which the hardware returns as zeros.
// Four LDS stages: the loads for step k+3 are issued while step k is computed.
//
// 32x32x64 FP4 MFMAs (the 16x16x128 form issues at only the FP8 rate on gfx950), with
// operands swapped -- D = W_tile * A_tile^T -- so a lane's accumulator holds 4
// consecutive output columns of one row.  FP4 operand layout: lane l holds 32
// consecutive codes (16 B) of row l%32 at K offset 32*(l/32); D layout: lane l, value v
// holds D[8*(v/4) + 4*(l/32) + v%4][l%32].  A bf16 result tile is staged in LDS and
// written with whole-row 16-byte stores.

// Wait until at most N direct-to-LDS loads of this thread are in flight and every LDS
// read of this wavefront has returned, then meet the workgroup barrier.  The LDS reads
// must be complete: after the barrier other wavefronts start loads into the stage
// those reads came from.  One asm block, so the compiler cannot move the reads past it.
#define FP4_SYNC(N) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory")

template <int BM, int BN>
__global__ void __launch_bounds__(256) w4a4_fp4_kernel(GemmParams p, int grid_m) {
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int LA = BM * 4 / 256, LB = BN * 4 / 256;  // 16-byte pieces per thread per step
    constexpr int STAGE = (BM + BN) * kBKBytes;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * STAGE];
    uint8_t* const st0 = smem;
    uint8_t* const st1 = smem + STAGE;
    uint8_t* const st2 = smem + 2 * STAGE;
    uint8_t* const st3 = smem + 3 * STAGE;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int bm = blockIdx.x % grid_m;
    const int bn = blockIdx.x / grid_m;
    const int64_t m0 = (int64_t)bm * BM, n0 = (int64_t)bn * BN;
    const int nk = (int)((p.K + 127) / 128);

    // buffer resources (base, stride 0, size in bytes, format word)
    const i32x4v rsA = buf_words(p.a, p.M * p.lda);
    const i32x4v rsB = buf_words(p.w, p.N * p.ldw);
    // the global piece behind this lane's LDS slot, for each of its LA + LB loads: slot
    // s = (4 i + wave) * 64 + lane holds row s/4, swizzled segment s%4 (see swz)
    uint32_t offA[LA], offB[LB];
    int segk[LA > LB ? LA : LB];
#pragma unroll
    for (int i = 0; i < LA; i++) {
        int sidx = (4 * i + wave) * 64 + lane, row = sidx >> 2;
        int seg = (sidx & 3) ^ ((row >> 1) & 3);
        segk[i] = seg * 32;
        offA[i] = (m0 + row < p.M) ? (uint32_t)((m0 + row) * p.lda + seg * 16) : kOOB;
    }
#pragma unroll
    for (int i = 0; i < LB; i++) {
        int sidx = (4 * i + wave) * 64 + lane, row = sidx >> 2;
        int seg = (sidx & 3) ^ ((row >> 1) & 3);
        offB[i] = (n0 + row < p.N) ? (uint32_t)((n0 + row) * p.ldw + seg * 16) : kOOB;
    }

    // The step count is rounded up to a multiple of 4 (the stage rotation); steps past
    // the last real one load zeros (out-of-range offsets) and add nothing.
    const int nk4 = (nk + 3) & ~3;

    f32x16 acc[TN][TM];
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[j][i][v] = 0.0f;
    const int r32 = lane & 31, hk = lane >> 5;

// direct-to-LDS loads of step KB into stage array STG
#define FP4_DMA(STG, KB)                                                                                   \
    do {                                                                                                   \
        const int kb_ = (KB);                                                                              \
        _Pragma("unroll") for (int i = 0; i < LA; i++) {                                                   \
            uint32_t off = (kb_ * 128 + segk[i] < p.K) ? offA[i] + (uint32_t)kb_ * kBKBytes : kOOB;        \
            dma16(rsA, off, __builtin_amdgcn_readfirstlane(                                                \
                                (uint32_t)(uintptr_t)&STG[(4 * i + wave) * 1024]));                       \
        }                                                                                                  \
        _Pragma("unroll") for (int i = 0; i < LB; i++) {                                                   \
            uint32_t off = (kb_ * 128 + segk[i] < p.K) ? offB[i] + (uint32_t)kb_ * kBKBytes : kOOB;        \
            dma16(rsB, off, __builtin_amdgcn_readfirstlane(                                                \
                                (uint32_t)(uintptr_t)&STG[BM * kBKBytes + (4 * i + wave) * 1024]));       \
        }                                                                                                  \
    } while (0)

// the MFMAs of one step from stage array STG
#define FP4_COMPUTE(STG)                                                                                   \
    do {                                                                                                   \
        _Pragma("unroll") for (int h = 0; h < 2; h++) {                                                    \
            i32x8 af[TM];                                                                                  \
            _Pragma("unroll") for (int i = 0; i < TM; i++) {                                               \
                uint4 v = *reinterpret_cast<const uint4*>(&STG[swz(wm * WM + i * 32 + r32, 2 * h + hk)]);  \
                af[i] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};                        \
            }                                                                                              \
            _Pragma("unroll") for (int j = 0; j < TN; j++) {                                               \
                uint4 v = *reinterpret_cast<const uint4*>(                                                 \
                    &STG[BM * kBKBytes + swz(wn * WN + j * 32 + r32, 2 * h + hk)]);                         \
                i32x8 bf = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};                     \
                _Pragma("unroll") for (int i = 0; i < TM; i++) acc[j][i] =                                 \
                    __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf, af[i], acc[j][i], 4, 4, 0, 127, 0, 127); \
            }                                                                                              \
        }                                                                                                  \
    } while (0)

    constexpr int PER_STEP = LA + LB;  // direct-to-LDS loads per step and thread
    FP4_DMA(st0, 0);
    FP4_DMA(st1, 1);
    FP4_DMA(st2, 2);
    // phase kb: wait until step kb landed (steps kb+1 and kb+2 may still be in flight),
    // barrier, start step kb+3 into the stage that phase kb-1 read, compute step kb
    for (int kb = 0; kb < nk4; kb += 4) {
        FP4_SYNC(2 * PER_STEP);
        FP4_DMA(st3, kb + 3);
        FP4_COMPUTE(st0);
        FP4_SYNC(2 * PER_STEP);
        FP4_DMA(st0, kb + 4);
        FP4_COMPUTE(st1);
        FP4_SYNC(2 * PER_STEP);
        FP4_DMA(st1, kb + 5);
        FP4_COMPUTE(st2);
        FP4_SYNC(2 * PER_STEP);
        FP4_DMA(st2, kb + 6);
        FP4_COMPUTE(st3);
    }
#undef FP4_DMA
#undef FP4_COMPUTE
    // drain the (zero) loads still in flight before the workgroup exits
    FP4_SYNC(0);

    // epilogue: y = fl32(acc * fl32(a * s_n)); value v of lane l holds output row
    // m = l%32 (+ tile offsets) and column n = 8*(v/4) + 4*(l/32) + v%4.  All scale
    // loads are issued first.
    const float a = p.a_scale[0];
    float f[TN][4][4];
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
        for (int g = 0; g < 4; g++)
#pragma unroll
            for (int t = 0; t < 4; t++) {
                int64_t n = n0 + wn * WN + j * 32 + 8 * g + 4 * hk + t;
                n = n < p.N ? n : p.N - 1;
                f[j][g][t] = reinterpret_cast<const float*>(p.w_scales)[p.w_mode == 1 ? n : 0];
            }
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
        for (int g = 0; g < 4; g++)
#pragma unroll
            for (int t = 0; t < 4; t++) f[j][g][t] = a * f[j][g][t];

    if (p.y_bf16 && BM * BN * 2 <= 4 * STAGE) {
        // bf16: stage the tile in LDS (row stride BN*2 bytes, 16-byte chunks XOR-swizzled
        // by row), then write whole rows with 16-byte stores
        constexpr int CH = BN / 8;  // 16-byte chunks per tile row
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int i = 0; i < TM; i++) {
                const int ml = wm * WM + i * 32 + r32;
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    const int nl = wn * WN + j * 32 + 8 * g + 4 * hk;  // multiple of 4
                    __bf16 h4[4];
#pragma unroll
                    for (int t = 0; t < 4; t++) h4[t] = (__bf16)(acc[j][i][4 * g + t] * f[j][g][t]);
                    const int chunk = (nl >> 3) ^ (ml & (CH - 1));
                    *reinterpret_cast<uint2*>(smem + ml * (BN * 2) + chunk * 16 + (nl & 4) * 2) =
                        __builtin_bit_cast(uint2, h4);
                }
            }
        __syncthreads();
        for (int idx = tid; idx < BM * CH; idx += 256) {
            const int ml = idx / CH, c = idx % CH;
            const int64_t m = m0 + ml, n = n0 + c * 8;
            if (m >= p.M || n >= p.N) continue;
            const uint4 v = *reinterpret_cast<const uint4*>(smem + ml * (BN * 2) + ((c ^ (ml & (CH - 1))) * 16));
            __bf16* yp = reinterpret_cast<__bf16*>(p.y) + m * p.ldy + n;
            if (n + 8 <= p.N && ((reinterpret_cast<uintptr_t>(yp) & 15) == 0)) {
                *reinterpret_cast<uint4*>(yp) = v;
            } else {
                const __bf16* hv = reinterpret_cast<const __bf16*>(&v);
                for (int t = 0; t < 8; t++)
                    if (n + t < p.N) yp[t] = hv[t];
            }
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < TN; j++) {
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const int64_t nb = n0 + wn * WN + j * 32 + 8 * g + 4 * hk;
#pragma unroll
            for (int i = 0; i < TM; i++) {
                const int64_t m = m0 + wm * WM + i * 32 + r32;
                if (m >= p.M) continue;
                float y[4];
#pragma unroll
                for (int t = 0; t < 4; t++) y[t] = acc[j][i][4 * g + t] * f[j][g][t];
                if (p.y_bf16) {
                    __bf16* yp = reinterpret_cast<__bf16*>(p.y) + m * p.ldy + nb;
                    for (int t = 0; t < 4; t++)
                        if (nb + t < p.N) yp[t] = (__bf16)y[t];
                } else {
                    float* yp = reinterpret_cast<float*>(p.y) + m * p.ldy + nb;
                    if (nb + 4 <= p.N && ((reinterpret_cast<uintptr_t>(yp) & 15) == 0)) {
                        *reinterpret_cast<float4*>(yp) = make_float4(y[0], y[1], y[2], y[3]);
                    } else {
                        for (int t = 0; t < 4; t++)
                            if (nb + t < p.N) yp[t] = y[t];
                    }
                }
            }
        }
    }
}

// Buffer offsets are 32-bit and kOOB marks "past the end", so one launch covers at most
// kMaxBufBytes of A and of W; larger operands are split into row blocks (multiples of
// 256 rows, whole tiles either way), each launched on pointers advanced to its start.
constexpr int64_t kMaxBufBytes = 0x7fff0000;

static hipError_t launch_block(const GemmParams& p, hipStream_t s) {
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

hipError_t launch_w4a4_fp4(const GemmParams& p, hipStream_t s) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    const int64_t mstep = std::max<int64_t>(256, kMaxBufBytes / std::max<int64_t>(p.lda, 1) / 256 * 256);
    const int64_t nstep = std::max<int64_t>(256, kMaxBufBytes / std::max<int64_t>(p.ldw, 1) / 256 * 256);
    const size_t ysz = p.y_bf16 ? 2 : 4;
    for (int64_t m0 = 0; m0 < p.M; m0 += mstep) {
        for (int64_t n0 = 0; n0 < p.N; n0 += nstep) {
            GemmParams q = p;
            q.M = std::min(mstep, p.M - m0);
            q.N = std::min(nstep, p.N - n0);
            q.a = reinterpret_cast<const uint8_t*>(p.a) + m0 * p.lda;
            q.w = p.w + n0 * p.ldw;
            if (p.w_mode == 1) q.w_scales = reinterpret_cast<const float*>(p.w_scales) + n0;
            q.y = reinterpret_cast<uint8_t*>(p.y) + (m0 * p.ldy + n0) * ysz;
            hipError_t e = launch_block(q, s);
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace fp4

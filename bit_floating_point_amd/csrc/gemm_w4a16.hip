// W4A16: Y[m, n] = sum_u s[n, u] * sum_{k in u} x[m, k] * g(c[n, k])
// (scales factored out of the low-bit inner product: [FP4-LLM] "efficient matrix
// multiplication"; [W8A8] section 2.2 quantized_matmul; group size 128).
//
// Two bf16-activation, 4-bit-minifloat-weight kernels run on the bf16 matrix cores;
// both are HBM-bound on the packed weights.  Per 128-wide K chunk a lane streams 16
// bytes (32 codes) of one weight row with a single 128-bit load, turns them into bf16
// (E2M1 with the gfx950 FP4->bf16 convert, E1M2 and E3M0 through the FP8 convert; all
// exact), and feeds four bf16 16x16x32 MFMAs.  The 4-bit
// codes of one lane are the B operand of those MFMAs under a fixed permutation of K
// that the activation operand uses too, so no shuffles are needed.  Each scale group's
// partial sum is kept apart and multiplied by its scale in fp32 before it joins the
// total; the wavefront partials are combined through LDS in a fixed order.
//  * w4a16_small_kernel (M <= 16, the decode case): activations staged in LDS per
//    wavefront, all of a batch's weight loads in flight at once.  Its variants also
//    take two-mode weights (E2M1 or E1M2 per group, by the scale's sign bit) and the
//    OCP FP8 / FP6 weights (W8A16 / W6A16), each decoded exactly to bf16.
//  * w4a16_mfma_kernel (any M, 16-row tiles along M): activation fragments loaded
//    straight from memory, for shapes the small kernel does not take.
//
// A third, plain VALU kernel covers f32 activations and the other grids and shapes.
#include "fp4_device.h"

namespace fp4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x32 __attribute__((ext_vector_type(32)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kW16Waves = 4;
constexpr int kBatch = 4;  // K chunks in flight per wavefront

// Small-M path geometry (host and device): per-wavefront X region in 16-byte vectors,
// padded to whole 64-lane loads, and the workgroup's dynamic LDS (at most 136 KiB, which
// leaves room for the static partial-sum array within the CU's 160 KiB).
constexpr int kSmallWavesPerGroup = 8;
constexpr size_t kSmallMaxLds = 136 * 1024;
// The region also holds the wavefront's T partial-sum vectors per lane after its loop.
// Wavefronts own whole pairs of 128-wide K chunks (the last pair may be a single chunk).
__host__ __device__ inline int small_chunk_begin(int64_t nchunks, int wave) {
    return (int)(2 * (((nchunks + 1) / 2) * wave / kSmallWavesPerGroup));
}
__host__ __device__ inline int small_region(int64_t M, int64_t nchunks, int T) {
    const int64_t per_wave = 2 * (((nchunks + 1) / 2 + kSmallWavesPerGroup - 1) / kSmallWavesPerGroup);
    const int64_t r = (M * per_wave * 16 + 63) / 64 * 64;
    return (int)(r > 64 * T ? r : 64 * T);
}
inline size_t small_lds_bytes(int64_t M, int64_t K, int T) {
    return (size_t)kSmallWavesPerGroup * small_region(M, K / 128, T) * 16;
}

__device__ __forceinline__ bf16x8 decode_e2m1_bf16(uint32_t w) {
    // byte b of w holds codes 2b (low nibble) and 2b+1
    uint32_t o[4];
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1));
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2));
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3));
    return __builtin_bit_cast(bf16x8, o);
}

// 8 E1M2 or E3M0 codes -> 8 bf16 values, exact, through the FP8 E4M3 convert: the
// nibble's sign becomes bit 7 of a byte and its magnitude code c goes to
//  E1M2 (GE = 1): bits 0..2, the E4M3 subnormal c * 2^-9; the convert's scale 2^7 makes
//       it c / 4, which is the E1M2 value of c (c / 4 below 1, 1 + (c - 4) / 4 above);
//  E3M0 (GE = 3): bits 3..5, the E4M3 value 2^(c - 7) (zero for c = 0); the scale 2^6
//       makes it 2^(c - 1).
// GE = 2 is E2M1, which the FP4 convert takes directly.
template <int GE>
__device__ __forceinline__ bf16x8 decode_mini4_bf16(uint32_t w) {
    if constexpr (GE == 2) {
        return decode_e2m1_bf16(w);
    } else {
        static_assert(GE == 1 || GE == 3, "4-bit minifloat weights: E1M2, E2M1 or E3M0");
        constexpr int SH = GE == 3 ? 3 : 0;
        constexpr float kScale = GE == 3 ? 64.0f : 128.0f;
        const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;  // codes 0,2,4,6 / 1,3,5,7
        const uint32_t blo = ((lo & 0x07070707u) << SH) | ((lo & 0x08080808u) << 4);
        const uint32_t bhi = ((hi & 0x07070707u) << SH) | ((hi & 0x08080808u) << 4);
        const uint32_t d0 = __builtin_amdgcn_perm(bhi, blo, 0x05010400u);  // codes 0..3 in byte order
        const uint32_t d1 = __builtin_amdgcn_perm(bhi, blo, 0x07030602u);  // codes 4..7
        uint32_t o[4];
        o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, kScale, false));
        o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, kScale, true));
        o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, kScale, false));
        o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, kScale, true));
        return __builtin_bit_cast(bf16x8, o);
    }
}

// 8 two-mode codes -> 8 bf16 values, exact, in one pass for either grid: the magnitude
// code c goes to bits 0..2 of an FP8 E4M3 byte for E1M2 (the subnormal c * 2^-9, scale 2^7
// as above) or to bits 2..4 for E2M1: exponent field p of the E2M1 code then lands in the
// E4M3 exponent's low bits and its mantissa bit in the top mantissa bit, so the byte is
// 2^-6 times the E2M1 value (p = 0: the subnormal m * 2^-7; p >= 1: 2^(p - 7) (1 + m / 2)),
// and the scale 2^6 restores it.  The shift and the scale are per lane (the grid of the
// lane's scale group).
__device__ __forceinline__ bf16x8 decode_two_mode_bf16(uint32_t w, bool e1m2) {
    const uint32_t sh = e1m2 ? 0u : 2u;
    const float sc = e1m2 ? 128.0f : 64.0f;
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;  // codes 0,2,4,6 / 1,3,5,7
    const uint32_t blo = ((lo & 0x07070707u) << sh) | ((lo & 0x08080808u) << 4);
    const uint32_t bhi = ((hi & 0x07070707u) << sh) | ((hi & 0x08080808u) << 4);
    const uint32_t d0 = __builtin_amdgcn_perm(bhi, blo, 0x05010400u);  // codes 0..3 in byte order
    const uint32_t d1 = __builtin_amdgcn_perm(bhi, blo, 0x07030602u);  // codes 4..7
    uint32_t o[4];
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, sc, false));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, sc, true));
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, sc, false));
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, sc, true));
    return __builtin_bit_cast(bf16x8, o);
}

// The 16-byte pieces of two chunk loads e (rows r16 / 2) and o (rows 8 + r16 / 2),
// swapped between neighbouring lanes 2i, 2i + 1 so that each lane ends up with both
// chunks of one row: lane 2i keeps e (row i, chunk 2j) and takes its neighbour's e
// (row i, chunk 2j + 1); lane 2i + 1 takes its neighbour's o (row 8 + i, chunk 2j) and
// keeps o (row 8 + i, chunk 2j + 1).  One DPP quad permutation [1, 0, 3, 2] per dword.
__device__ __forceinline__ void pair_swap(uint4& e, uint4& o, bool odd) {
    uint32_t ev[4] = {e.x, e.y, e.z, e.w}, ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint32_t send = odd ? ev[i] : ov[i];
        const uint32_t got = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send, 0xB1, 0xF, 0xF, false);
        const uint32_t first = odd ? got : ev[i], second = odd ? ov[i] : got;
        ev[i] = first;
        ov[i] = second;
    }
    e = make_uint4(ev[0], ev[1], ev[2], ev[3]);
    o = make_uint4(ov[0], ov[1], ov[2], ov[3]);
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
// GE: exponent bits of the 4-bit minifloat weights (1 E1M2, 2 E2M1, 3 E3M0)
template <int MODE, int T, bool SF16, bool G1, int GE = 2>  // MODE 0 tensor, 1 row, 2 group
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
                                                                  decode_mini4_bf16<GE>(wd[j]), acc, 0, 0, 0);
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

template <int T, bool SF16, int GE>
static void launch_w16(const GemmParams& p, hipStream_t s) {
    dim3 grid((unsigned)((p.N + 16 * T - 1) / (16 * T)), (unsigned)((p.M + 15) / 16));
    if (p.w_mode == 2 && p.w_group == 128) hipLaunchKernelGGL((w4a16_mfma_kernel<2, T, SF16, true, GE>), grid, dim3(256), 0, s, p);
    else if (p.w_mode == 2) hipLaunchKernelGGL((w4a16_mfma_kernel<2, T, SF16, false, GE>), grid, dim3(256), 0, s, p);
    else if (p.w_mode == 1) hipLaunchKernelGGL((w4a16_mfma_kernel<1, T, SF16, false, GE>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((w4a16_mfma_kernel<0, T, SF16, false, GE>), grid, dim3(256), 0, s, p);
}

// ---------------------------------------------------------------------------------
// Decode GEMV / small batch, M <= 16 (the latency-critical case).  A workgroup of
// kSmallWaves wavefronts owns 16*T output columns; wavefront w owns 1/kSmallWaves of K.
//  * Each wavefront stages only its own K range of X (all M rows) in LDS with
//    direct-to-LDS loads, so no workgroup barrier precedes the main loop and chunk b is
//    computed as soon as its weights land.  X bytes cost vector-memory issue slots like
//    the weights do; the T column tiles of a wavefront share one staged copy.
//  * Weights and scales come through buffer loads (offsets past the end read zeros), a
//    batch of kSmallChunks chunks x T tiles at once; with group-128 scales the batch's
//    scales of a row are one vector load (SV).
//  * A fragments are read from LDS; rows >= M read row M-1 (they only feed output rows
//    that are never stored).
// The per-chunk MFMA sums, their scaling and the cross-wavefront sum are the same
// operations in the same order as in the kernel above.
constexpr int kSmallWaves = kSmallWavesPerGroup;
constexpr int kSmallChunks = 4;  // K chunks per wavefront per batch

// TWO: two-mode weights (group 128): a group is E1M2 when the sign bit of its scale is
// set, E2M1 otherwise, and is scaled by the scale's magnitude.
// W8 = 4 / 5: OCP FP8 E4M3 / E5M2 weights, one byte per code: a lane's 32 codes of a
// chunk are two 16-byte loads, converted to bf16 with the gfx950 FP8 converts (exact).
// W8 = 2 / 3: OCP FP6 E2M3 / E3M2 weights, a bit stream of 6-bit codes: a lane's 32
// codes are 24 bytes (a 16-byte and an 8-byte load, which the compiler cannot merge or
// split, so the wait counts below stay exact), converted at once by the 32-value FP6
// converts (exact).
// GE: exponent bits of 4-bit minifloat weights (1 E1M2, 2 E2M1, 3 E3M0) when W8 = 0.
template <int MODE, bool SF16, bool SV, int T, bool TWO = false, int W8 = 0, int GE = 2>  // MODE 0 tensor, 1 row, 2 group of 128
__global__ void __launch_bounds__(kSmallWaves * 64) w4a16_small_kernel(GemmParams p) {
    constexpr int NW = kSmallWaves, CH = kSmallChunks;
    extern __shared__ uint4 xs[];  // per wavefront: [M][its K range / 8] bf16 vectors
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q = lane >> 4, r16 = lane & 15;
    const int64_t n0 = (int64_t)blockIdx.x * 16 * T;
    const int nchunks = (int)(p.K / 128);
    const int c_begin = small_chunk_begin(nchunks, wave);
    const int c_end = min(nchunks, small_chunk_begin(nchunks, wave + 1));
    // X vectors of one row in this wavefront's range (at least one chunk, so that a
    // wavefront with an empty range still forms valid addresses)
    const int nvw = c_end - c_begin > 0 ? (c_end - c_begin) * 16 : 16;
    const int xw = (int)p.M * nvw;
    const int region = small_region(p.M, nchunks, T);
    const int wbase = wave * region;
    const int64_t ngroups = MODE == 2 ? p.K / 128 : 1;
    constexpr int SB = SF16 ? 2 : 4;       // bytes per scale
    constexpr int SVB = CH * SB;           // bytes of one batch's scales of a row (8 or 16)
    const __amdgpu_buffer_rsrc_t rsW = buf_make(p.w, p.N * p.ldw);
    const __amdgpu_buffer_rsrc_t rsS = buf_make(p.w_scales, p.N * ngroups * SB);
    // PAIRS (4-bit weights, one tile per wavefront): each load instruction reads whole
    // 128-byte lines.  Chunks 2j and 2j + 1 of a row are one 128-byte piece; the load of
    // chunk 2j reads the pieces of the tile's rows 0..7, that of chunk 2j + 1 those of rows
    // 8..15, lane (q, r16) the 16 bytes at (r16 % 2) * 64 + 16 q of row r16 / 2 (+ 8).  One
    // swap between neighbouring lanes (pair_swap) then leaves lane (q, r16) with quarter q
    // of both chunks of the row rho = r16 / 2 + 8 (r16 % 2), so column r16 of the tile's
    // MFMAs is weight row rho.  Measured 1.5-3% faster at M = 1 and 4 (11008 x 4096); with
    // three tiles per wavefront the swaps cost more than the loads gain, so those keep
    // rho = r16 and 64 bytes of 16 rows per load, as FP8 / FP6 weights do.
    constexpr bool PAIRS = !W8 && T == 1;
    const int rho = PAIRS ? (r16 >> 1) + 8 * (r16 & 1) : r16;
    uint32_t wrow[T], wrow2[T], srow[T];
    bool n_ok[T];
#pragma unroll
    for (int t = 0; t < T; t++) {
        const int64_t n = n0 + 16 * t + rho;
        n_ok[t] = n < p.N;
        constexpr int LB = W8 >= 4 ? 32 : W8 ? 24 : 16;  // bytes of a lane's 32 codes
        if (!PAIRS) {
            wrow[t] = n_ok[t] ? (uint32_t)(n * p.ldw + q * LB) : kOOB;
        } else {
            const int64_t re = n0 + 16 * t + (r16 >> 1), ro = re + 8;
            const int in = (r16 & 1) * 64 + q * 16;
            wrow[t] = re < p.N ? (uint32_t)(re * p.ldw + in) : kOOB;
            wrow2[t] = ro < p.N ? (uint32_t)(ro * p.ldw + in) : kOOB;
        }
        srow[t] = n_ok[t] ? (uint32_t)(n * ngroups * SB) : kOOB;
    }

    // 1. this wavefront's X into its LDS region: load i puts vector 64 i + l of the
    //    region (row m = v / nvw, vector v % nvw of the range) at lane l; vectors past
    //    the range read zeros into the region's padding
    {
        const i32x4v rs = buf_words(p.a, (((int64_t)p.M - 1) * p.lda + p.K) * 2);
        for (int i = 0; 64 * i < region; i++) {
            const int v = lane + 64 * i;
            const int m = (unsigned)v / (unsigned)nvw, cc = v - m * nvw;
            const uint32_t off = v < xw ? (uint32_t)((m * p.lda + (c_begin * 16 + cc) * 8) * 2) : kOOB;
            dma16(rs, off, __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&xs[wbase + 64 * i]));
        }
    }
    // 2. a batch of weights and scales; chunks past the range are loaded too (they
    //    belong to the next range or read zeros) and contribute nothing
    uint4 wv[CH][T], wv2[CH][T];  // wv2: the second 16 bytes of FP8 codes
    uint4 w6a[CH][T];             // FP6: bytes 0..15 of 24
    uint2 w6b[CH][T];             // FP6: bytes 16..23
    uint4 sv[T];
    uint32_t sc[CH][T];
    auto load_batch = [&](int cs) {
        if (MODE == 2 && SV) {
#pragma unroll
            for (int t = 0; t < T; t++) {
                if (SVB == 8) {
                    const uint2 u = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rsS, srow[t] + cs * SB, 0, 0));
                    sv[t] = make_uint4(u.x, u.y, 0, 0);
                } else {
                    sv[t] = buf_load16(rsS, srow[t] + cs * SB);
                }
            }
        }
#pragma unroll
        for (int b = 0; b < CH; b++) {
#pragma unroll
            for (int t = 0; t < T; t++) {
                if (W8 == 2 || W8 == 3) {
                    w6a[b][t] = buf_load16(rsW, wrow[t] + (uint32_t)(cs + b) * 96);
                    w6b[b][t] = __builtin_bit_cast(
                        uint2, __builtin_amdgcn_raw_buffer_load_b64(rsW, wrow[t] + (uint32_t)(cs + b) * 96 + 16, 0, 0));
                } else {
                    if (W8) {
                        wv[b][t] = buf_load16(rsW, wrow[t] + (uint32_t)(cs + b) * 128);
                        wv2[b][t] = buf_load16(rsW, wrow[t] + (uint32_t)(cs + b) * 128 + 16);
                    } else if (PAIRS) {  // cs is even: chunk cs + b is of parity b
                        wv[b][t] = buf_load16(rsW, ((b & 1) ? wrow2[t] : wrow[t]) + (uint32_t)(cs / 2 + b / 2) * 128);
                    } else {
                        wv[b][t] = buf_load16(rsW, wrow[t] + (uint32_t)(cs + b) * 64);
                    }
                }
                if (MODE == 2 && !SV) {
                    const uint32_t off = srow[t] + (uint32_t)(cs + b) * SB;
                    sc[b][t] = SF16 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rsS, off, 0, 0)
                                    : __builtin_amdgcn_raw_buffer_load_b32(rsS, off, 0, 0);
                }
            }
        }
    };
    load_batch(c_begin);
    // 3. the X loads are the oldest in flight: wait until only the batch's loads remain
    // Counted as the fewest instructions the compiler can make of the batch: the 16-byte
    // weight loads (FP6: 16 + 8 bytes) cannot be merged, but a tile's CH adjacent scale
    // loads can become one; counting too few only waits for some batch loads as well.
    constexpr int kLater = CH * T * (W8 ? 2 : 1) + (MODE == 2 ? T : 0);
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(kLater) : "memory");

    const int xrow = wbase + (r16 < p.M ? r16 : (int)p.M - 1) * nvw - c_begin * 16;
    f32x4 total[T];
#pragma unroll
    for (int t = 0; t < T; t++) total[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c0 = c_begin; c0 < c_end; c0 += CH) {
        if (MODE == 2 && SV) {
#pragma unroll
            for (int t = 0; t < T; t++) {
                const uint32_t sw[4] = {sv[t].x, sv[t].y, sv[t].z, sv[t].w};
#pragma unroll
                for (int b = 0; b < CH; b++) sc[b][t] = SF16 ? ((sw[b >> 1] >> (16 * (b & 1))) & 0xffffu) : sw[b];
            }
        }
#pragma unroll
        for (int b = 0; b < CH; b++) {
            const int c = c0 + b;
            const bool valid = c < c_end;
            const int cc = valid ? c : c_begin;
            if (PAIRS && (b & 1) == 0) {
#pragma unroll
                for (int t = 0; t < T; t++) pair_swap(wv[b][t], wv[b + 1][t], (r16 & 1) != 0);
            }
            uint4 xa[4];
#pragma unroll
            for (int j = 0; j < 4; j++) xa[j] = xs[xrow + cc * 16 + q * 4 + j];
#pragma unroll
            for (int t = 0; t < T; t++) {
                const uint32_t wd[4] = {wv[b][t].x, wv[b][t].y, wv[b][t].z, wv[b][t].w};
                f32x4 acc = MODE == 2 ? f32x4{0.f, 0.f, 0.f, 0.f} : total[t];
                constexpr uint32_t kSign = SF16 ? 0x8000u : 0x80000000u;
                const bool e1m2 = TWO && (sc[b][t] & kSign) != 0;
                bf16x32 w32;
                if (W8 == 2 || W8 == 3) {
                    typedef unsigned v6u __attribute__((ext_vector_type(6)));
                    const v6u src = v6u{w6a[b][t].x, w6a[b][t].y, w6a[b][t].z, w6a[b][t].w, w6b[b][t].x, w6b[b][t].y};
                    if (W8 == 2) w32 = __builtin_amdgcn_cvt_scalef32_pk32_bf16_fp6(src, 1.0f);
                    else w32 = __builtin_amdgcn_cvt_scalef32_pk32_bf16_bf6(src, 1.0f);
                }
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    bf16x8 wf;
                    if (W8 == 2 || W8 == 3) {
                        wf = bf16x8{w32[8 * j], w32[8 * j + 1], w32[8 * j + 2], w32[8 * j + 3], w32[8 * j + 4],
                                    w32[8 * j + 5], w32[8 * j + 6], w32[8 * j + 7]};
                    } else if (W8) {
                        // K values 8 j .. 8 j + 7 of the lane's 32: bytes 8 j .. of the two loads
                        const uint4 h = j < 2 ? wv[b][t] : wv2[b][t];
                        const uint32_t d0 = (j & 1) ? h.z : h.x, d1 = (j & 1) ? h.w : h.y;
                        uint32_t o[4];
                        if (W8 == 4) {
                            o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false));
                            o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true));
                            o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false));
                            o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true));
                        } else {
                            o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d0, 1.0f, false));
                            o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d0, 1.0f, true));
                            o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d1, 1.0f, false));
                            o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d1, 1.0f, true));
                        }
                        wf = __builtin_bit_cast(bf16x8, o);
                    } else if (TWO) {
                        wf = decode_two_mode_bf16(wd[j], e1m2);
                    } else {
                        wf = decode_mini4_bf16<GE>(wd[j]);
                    }
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[j]), wf, acc, 0, 0, 0);
                }
                if (MODE == 2) {
                    const float s = valid ? scale_value<SF16>(TWO ? (sc[b][t] & ~kSign) : sc[b][t]) : 0.0f;
#pragma unroll
                    for (int i = 0; i < 4; i++) total[t][i] = __builtin_fmaf(acc[i], s, total[t][i]);
                } else {
                    total[t] = valid ? acc : total[t];
                }
            }
        }
        if (c0 + CH < c_end) load_batch(c0 + CH);
    }
#pragma unroll
    for (int t = 0; t < T; t++) {
        if (MODE != 2) {
            const float s = scale_value<SF16>(load_scale_raw<SF16>(p, MODE == 1 ? (n_ok[t] ? n0 + 16 * t + rho : 0) : 0));
#pragma unroll
            for (int i = 0; i < 4; i++) total[t][i] = total[t][i] * s;
        }
        // partial sums into this wavefront's own region (its X is no longer read)
        if (wave > 0) xs[wbase + t * 64 + lane] = __builtin_bit_cast(uint4, total[t]);
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int t = 0; t < T; t++) {
#pragma unroll
            for (int w = 0; w < NW - 1; w++) {
                const f32x4 o = __builtin_bit_cast(f32x4, xs[(w + 1) * region + t * 64 + lane]);
#pragma unroll
                for (int i = 0; i < 4; i++) total[t][i] += o[i];
            }
            if (!n_ok[t]) continue;
            const int64_t n = n0 + 16 * t + rho;
            // D layout of a 16x16 MFMA: lane holds rows 4*(lane/16) + i of column lane%16
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int64_t mm = 4 * q + i;
                if (mm < p.M) {
                    if (p.y_bf16) reinterpret_cast<__bf16*>(p.y)[mm * p.ldy + n] = (__bf16)total[t][i];
                    else reinterpret_cast<float*>(p.y)[mm * p.ldy + n] = total[t][i];
                }
            }
        }
    }
}

template <int MODE, bool SF16, bool SV, int T, bool TWO = false, int W8 = 0, int GE = 2>
static hipError_t launch_small_t(const GemmParams& p, hipStream_t s) {
    const size_t lds = small_lds_bytes(p.M, p.K, T);
    auto kern = w4a16_small_kernel<MODE, SF16, SV, T, TWO, W8, GE>;
    // the dynamic-LDS limit is a kernel attribute, set once per device
    static bool attr_set[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64 || !attr_set[dev]) {
        e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSmallMaxLds);
        if (e != hipSuccess) return e;
        if (dev >= 0 && dev < 64) attr_set[dev] = true;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)((p.N + 16 * T - 1) / (16 * T))), dim3(kSmallWaves * 64), lds, s, p);
    return hipGetLastError();
}

template <int MODE, bool SF16, bool SV, bool TWO = false, int W8 = 0, int GE = 2>
static hipError_t launch_small_sv(const GemmParams& p, hipStream_t s) {
    // M <= 4: one 16-column tile per wavefront (more workgroups, X is small);
    // larger M: three tiles share each staged X
    return p.M <= 4 ? launch_small_t<MODE, SF16, SV, 1, TWO, W8, GE>(p, s) : launch_small_t<MODE, SF16, SV, 3, TWO, W8, GE>(p, s);
}

template <bool SF16, bool TWO = false, int W8 = 0, int GE = 2>
static hipError_t launch_small(const GemmParams& p, hipStream_t s) {
    if (p.w_mode == 2) {
        const int64_t nchunks = p.K / 128;
        // one vector load per batch needs 4-byte aligned scale rows and batch starts
        const bool sv = SF16 ? (nchunks % (2 * kSmallWaves) == 0 && (reinterpret_cast<uintptr_t>(p.w_scales) & 3) == 0)
                             : (reinterpret_cast<uintptr_t>(p.w_scales) & 3) == 0;
        return sv ? launch_small_sv<2, SF16, true, TWO, W8, GE>(p, s) : launch_small_sv<2, SF16, false, TWO, W8, GE>(p, s);
    }
    if (p.w_mode == 1) return launch_small_sv<1, SF16, false, false, W8, GE>(p, s);
    return launch_small_sv<0, SF16, false, false, W8, GE>(p, s);
}

static bool small_fits(const GemmParams& p) {
    const int64_t ngroups = p.w_mode == 2 ? p.K / 128 : 1;
    const int64_t sbytes = p.w_scale_f16 ? 2 : 4;
    return p.M <= 16 && (p.w_mode != 2 || p.w_group == 128) && small_lds_bytes(p.M, p.K, 4) <= kSmallMaxLds &&
           // 32-bit buffer offsets
           p.N * p.ldw < kOOB && p.N * ngroups * sbytes < kOOB && ((p.M - 1) * p.lda + p.K) * 2 < (int64_t)kOOB;
}

hipError_t launch_w8a16_small(const GemmParams& p, hipStream_t s) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    if (!small_fits(p) || (p.wg.bits == 6 && p.ldw % 8 != 0)) return launch_w4a16_valu(p, s);
    if (p.wg.bits == 6) {
        if (p.wg.e == 2) return p.w_scale_f16 ? launch_small<true, false, 2>(p, s) : launch_small<false, false, 2>(p, s);
        return p.w_scale_f16 ? launch_small<true, false, 3>(p, s) : launch_small<false, false, 3>(p, s);
    }
    if (p.wg.e == 4) return p.w_scale_f16 ? launch_small<true, false, 4>(p, s) : launch_small<false, false, 4>(p, s);
    return p.w_scale_f16 ? launch_small<true, false, 5>(p, s) : launch_small<false, false, 5>(p, s);
}

hipError_t launch_w4a16_two_mode(const GemmParams& p, hipStream_t s) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    if (!small_fits(p)) return launch_w4a16_valu(p, s);
    return p.w_scale_f16 ? launch_small<true, true>(p, s) : launch_small<false, true>(p, s);
}

template <int GE>
static hipError_t launch_w4a16_mfma_ge(const GemmParams& p, hipStream_t s) {
    if (small_fits(p))
        return p.w_scale_f16 ? launch_small<true, false, 0, GE>(p, s) : launch_small<false, false, 0, GE>(p, s);
    // larger M: reuse each activation fragment for two weight tiles
    if (p.M > 8) {
        if (p.w_scale_f16) launch_w16<2, true, GE>(p, s);
        else launch_w16<2, false, GE>(p, s);
    } else {
        if (p.w_scale_f16) launch_w16<1, true, GE>(p, s);
        else launch_w16<1, false, GE>(p, s);
    }
    return hipGetLastError();
}
hipError_t launch_w4a16_mfma(const GemmParams& p, hipStream_t s) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    if (p.wg.e == 1) return launch_w4a16_mfma_ge<1>(p, s);
    if (p.wg.e == 3) return launch_w4a16_mfma_ge<3>(p, s);
    return launch_w4a16_mfma_ge<2>(p, s);
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
        int64_t u = p.w_mode == 0 ? 0 : (p.w_mode == 1 ? n : n * (p.K / p.w_group) + k0 / p.w_group);
        float s = p.w_scale_f16 ? __half2float(reinterpret_cast<const __half*>(p.w_scales)[u])
                                : reinterpret_cast<const float*>(p.w_scales)[u];
        // two-mode grid: the scale's sign bit picks E1M2 (val[8..15]) over E2M1 (val[0..7])
        const int vbase = (p.wg.kind == 2 && signbit(s)) ? 8 : 0;
        if (p.wg.kind == 2) s = fabsf(s);
        float part = 0.0f;
        for (int64_t k = k0; k < k0 + unit; k++) {
            uint32_t c = p.wg.bits == 8 ? wr[k] : p.wg.bits == 6 ? code6_at(wr, k) : (wr[k >> 1] >> (4 * (k & 1))) & 15u;
            float xv = p.a_kind == 1 ? bf16_bits_to_float(reinterpret_cast<const uint16_t*>(p.a)[m * p.lda + k])
                                     : reinterpret_cast<const float*>(p.a)[m * p.lda + k];
            float g;
            if (p.wg.bits != 4) {
                g = wide_value_rt(c, p.wg.e);
            } else if (p.wg.kind == 2) {
                g = p.wg.val[vbase + (c & 7)];
                if (c & 8) g = -g;
            } else {
                g = grid_value(c, p.wg);
            }
            part = __builtin_fmaf(xv, g, part);
        }
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

// W4A4 GEMM with a 16-entry lookup grid on the weights (NF4: "量化技术详解" page,
// section NF4, levels at quantiles of the normal distribution) and E2M1 activations
// with the pre-shifted per-tensor scale a:
//   Y[m, n] = a * sum_g s[n, g] * sum_{k in g} A_q[m, k] * G[c[n, k]]
//
// gfx950 has no matrix instruction for an arbitrary 16-value grid, so the products run
// on v_mfma_f32_32x32x16_f16 with fp32 accumulation, both operands as f16:
//  * activations: E2M1 -> f16 with the FP4 convert (exact);
//  * weights: G[c] by byte permutes of a table held in registers (exact: the grid values
//    are binary16), times the group scale taken relative to a power of two of the row:
//    w = fl16(G[c] * fl16(s[n, g] * 2^-e_n)) with 2^e_n the power of two just above the
//    row's largest group scale, so no scaled weight overflows and only groups whose scale
//    is far below the row's largest can reach f16 subnormals.  2^e_n and a are applied
//    to the fp32 result (exactly).  Folding the scale into the expanded weights keeps
//    the group scales out of the per-output arithmetic: one multiply per weight per
//    workgroup instead of one per output element and group.
// The weights are expanded once per workgroup and K step into LDS in MFMA fragment order
// (each 16-byte operand of lane l of a 32-row tile and K16 block at byte 16 l of a 1 KiB
// block), so every fragment read is one linear wavefront read.  The activations are
// expanded the same way on 256x256 tiles; on 128x128 tiles they stay packed in LDS and
// every wavefront converts its own fragments (a quarter of the LDS bytes, more VALU per
// wavefront: better where several workgroups share a CU).  Two LDS stages: while step k's
// MFMAs run, each wavefront expands a quarter of step k+1 after every K16 block of MFMAs
// (interleaved so that the VALU work overlaps the matrix work); packed codes for step
// k+2 are loaded meanwhile.  The MFMAs take the K values of a step in the order block kk,
// lane half h: codes 32 h + 8 kk .. +7 (the same order on both operands).
#include <algorithm>

#include "fp4_device.h"

namespace fp4 {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kLutBK = 64;  // K codes per step (one 64-code group)

// 8 E2M1 codes (element 2j in the low nibble of byte j) -> 8 f16 values, exact
__device__ __forceinline__ uint4 decode_e2m1_f16x8(uint32_t w) {
    uint4 o;
    o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0));
    o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1));
    o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2));
    o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3));
    return o;
}

// byte lookup T[idx] for the 4 byte-indices (0..15) of idx; T is 16 bytes in 4 words
__device__ __forceinline__ uint32_t lut_bytes(uint32_t idx, const uint32_t T[4]) {
    const uint32_t i7 = idx & 0x07070707u;
    const uint32_t lo = __builtin_amdgcn_perm(T[1], T[0], i7);  // T[i & 7] for i < 8
    const uint32_t hi = __builtin_amdgcn_perm(T[3], T[2], i7);  // T[8 + (i & 7)]
    // byte j from lo (selector j) or hi (selector 4 + j) by bit 3 of index byte j
    const uint32_t sel = ((idx >> 1) & 0x04040404u) | 0x03020100u;
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// 8 lookup-grid codes -> 8 f16 grid values (exact: the grid values are binary16)
__device__ __forceinline__ uint4 decode_lut_f16x8(uint32_t w, const uint32_t TL[4], const uint32_t TH[4]) {
    const uint32_t ev = w & 0x0F0F0F0Fu, od = (w >> 4) & 0x0F0F0F0Fu;
    const uint32_t eL = lut_bytes(ev, TL), eH = lut_bytes(ev, TH);
    const uint32_t oL = lut_bytes(od, TL), oH = lut_bytes(od, TH);
    const uint32_t e01 = __builtin_amdgcn_perm(eH, eL, 0x05010400u);  // f16(x0) | f16(x2) << 16
    const uint32_t e23 = __builtin_amdgcn_perm(eH, eL, 0x07030602u);  // f16(x4) | f16(x6) << 16
    const uint32_t o01 = __builtin_amdgcn_perm(oH, oL, 0x05010400u);  // f16(x1) | f16(x3) << 16
    const uint32_t o23 = __builtin_amdgcn_perm(oH, oL, 0x07030602u);  // f16(x5) | f16(x7) << 16
    uint4 o;
    o.x = __builtin_amdgcn_perm(o01, e01, 0x05040100u);
    o.y = __builtin_amdgcn_perm(o01, e01, 0x07060302u);
    o.z = __builtin_amdgcn_perm(o23, e23, 0x05040100u);
    o.w = __builtin_amdgcn_perm(o23, e23, 0x07060302u);
    return o;
}

// Slot of fragment position s (0..63) in a 1 KiB block of expanded f16 operands: s for
// s < 32, s ^ 12 above.  A thread expands the two halves of one row into positions j and
// j + 32 and neighbouring lanes take neighbouring rows, so the lanes of a 128-bit LDS
// write meet positions j and j + 32 together: unswizzled they lie 512 bytes apart, on the
// same banks.  With the XOR, the slots of any 8 or 16 neighbouring lanes differ modulo 8
// or 16 (the groups in which 128-bit accesses are served), for these writes and for the
// fragment reads (lane l at position l) alike.
__device__ __forceinline__ int frag_slot(int s) { return s ^ (((s >> 5) & 1) * 12); }

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t mul_f16x2(uint32_t a, f16x2 s) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, a) * s);
}

template <int BM, int BN, bool PK>
__global__ void __launch_bounds__(256) w4a4_lut_kernel(GemmParams p, int grid_m) {
    constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
    constexpr int A_BYTES = PK ? BM * kLutBK / 2 : BM * kLutBK * 2, B_BYTES = BN * kLutBK * 2;  // per stage
    constexpr int STAGE = A_BYTES + B_BYTES;
    constexpr int PA = BM * 2 / 256, PB = BN * 2 / 256;  // 16-byte packed pieces per thread per step
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];
    __shared__ float rowfac[BN];  // 2^e_n for the tile's weight rows

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int64_t m0 = (int64_t)(blockIdx.x % grid_m) * BM;
    const int64_t n0 = (int64_t)(blockIdx.x / grid_m) * BN;
    const int nk = (int)(p.K / kLutBK);
    const int steps_per_group = p.w_group / kLutBK;
    const int64_t ngroups = p.K / p.w_group;
    const int sb = p.w_scale_f16 ? 2 : 4;

    // f16 bit patterns of the 16 grid values, split into low and high byte tables
    uint32_t TL[4] = {0, 0, 0, 0}, TH[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)p.wg.val[i]);
        TL[i >> 2] |= (h & 0xffu) << (8 * (i & 3));
        TH[i >> 2] |= (h >> 8) << (8 * (i & 3));
    }

    const __amdgpu_buffer_rsrc_t rsA = buf_make(p.a, p.M * p.lda);
    const __amdgpu_buffer_rsrc_t rsW = buf_make(p.w, p.N * p.ldw);
    const __amdgpu_buffer_rsrc_t rsS = buf_make(p.w_scales, p.N * ngroups * sb);

    // the weight rows' power of two: e_n with max_g s[n, g] * 2^-e_n in [0.5, 1).  Row r's
    // scales are read in 16-byte pieces, eight loads in flight (pieces past the row read
    // another row's scales or zeros: they are masked out)
    for (int r = tid; r < BN; r += 256) {
        const int64_t n = n0 + r;
        float mx = 0.0f;
        if (n < p.N) {
            // the row's bytes [lo, hi) of the scale array, read from a 16-byte aligned start
            const int64_t lo = n * ngroups * sb, hi = lo + ngroups * sb;
            for (int64_t b = lo & ~(int64_t)15; b < hi; b += 8 * 16) {
                uint4 v[8];
#pragma unroll
                for (int u = 0; u < 8; u++) v[u] = buf_load16(rsS, (uint32_t)(b + 16 * u));
#pragma unroll
                for (int u = 0; u < 8; u++) {
                    const uint32_t w4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        const int64_t at = b + 16 * u + 4 * q;  // byte offset of this word
                        if (p.w_scale_f16) {
                            const float s0 = __half2float(__ushort_as_half((unsigned short)(w4[q] & 0xffffu)));
                            const float s1 = __half2float(__ushort_as_half((unsigned short)(w4[q] >> 16)));
                            if (at >= lo && at < hi) mx = fmaxf(mx, s0);
                            if (at + 2 >= lo && at + 2 < hi) mx = fmaxf(mx, s1);
                        } else {
                            if (at >= lo && at < hi) mx = fmaxf(mx, __uint_as_float(w4[q]));
                        }
                    }
                }
            }
        }
        int e = 0;
        if (mx > 0.0f) (void)frexpf(mx, &e);
        rowfac[r] = ldexpf(1.0f, e);
    }

    // packed pieces of this thread: piece q covers row q/2, codes 32*(q%2) .. +31 of a step
    uint32_t offA[PA], offB[PB];
    int rowA[PA], kA[PA], rowB[PB], kB[PB];
#pragma unroll
    for (int i = 0; i < PA; i++) {
        const int q = tid + 256 * i;
        rowA[i] = q >> 1;
        kA[i] = (q & 1) * 32;
        offA[i] = (m0 + rowA[i] < p.M) ? (uint32_t)((m0 + rowA[i]) * p.lda + (q & 1) * 16) : kOOB;
    }
#pragma unroll
    for (int i = 0; i < PB; i++) {
        const int q = tid + 256 * i;
        rowB[i] = q >> 1;
        kB[i] = (q & 1) * 32;
        offB[i] = (n0 + rowB[i] < p.N) ? (uint32_t)((n0 + rowB[i]) * p.ldw + (q & 1) * 16) : kOOB;
    }
    __syncthreads();
    // 2^-e_n of this thread's weight rows (folded into the decoded weights)
    float rinv[PB];
#pragma unroll
    for (int i = 0; i < PB; i++) rinv[i] = 1.0f / rowfac[rowB[i]];

    uint4 ra[PA], rb[PB];
    uint32_t rs[PB];
    auto gload = [&](int k) {
#pragma unroll
        for (int i = 0; i < PA; i++) ra[i] = buf_load16(rsA, offA[i] + (uint32_t)k * 32);
#pragma unroll
        for (int i = 0; i < PB; i++) {
            rb[i] = buf_load16(rsW, offB[i] + (uint32_t)k * 32);
            const int64_t g = k / steps_per_group;
            const uint32_t off = n0 + rowB[i] < p.N ? (uint32_t)(((n0 + rowB[i]) * ngroups + g) * sb) : kOOB;
            rs[i] = p.w_scale_f16 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rsS, off, 0, 0)
                                  : __builtin_amdgcn_raw_buffer_load_b32(rsS, off, 0, 0);
        }
    };
    // LDS per stage: the activation codes packed, 32 B per row (row-major, the two 16-byte
    // halves of a row swapped when bit 3 of the row is set, so a wavefront's 16-byte reads
    // of 32 rows hit distinct banks); the weights expanded to f16 in MFMA fragment order:
    // per K16 block kk and 32-row tile t a 1 KiB block whose 16-byte slot frag_slot(l)
    // holds row 32 t + l%32, K values 32 (l/32) + 8 kk .. +7 of the step.  The MFMAs take K in
    // that order (block kk, lane half h: codes 32 h + 8 kk .. +7) on both operands.
    // Decode + store chunk c (8 codes) of every weight piece of this thread into stage
    // st; with chunk 0 the activation pieces are stored as they are.
    auto dstore_chunk = [&](int st, int c) {
        uint8_t* sa = smem + st * STAGE;
        uint8_t* sw = sa + A_BYTES;
        if (PK) {
            if (c == 0) {
#pragma unroll
                for (int i = 0; i < PA; i++) {
                    const int r = rowA[i], h = kA[i] / 32;
                    *reinterpret_cast<uint4*>(sa + r * 32 + ((h ^ ((r >> 3) & 1)) << 4)) = ra[i];
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < PA; i++) {
                const uint32_t w[4] = {ra[i].x, ra[i].y, ra[i].z, ra[i].w};
                const int h = kA[i] / 32, r = rowA[i];
                *reinterpret_cast<uint4*>(sa + ((c * (BM / 32) + (r >> 5)) * 64 + frag_slot((r & 31) + 32 * h)) * 16) =
                    decode_e2m1_f16x8(w[c]);
            }
        }
#pragma unroll
        for (int i = 0; i < PB; i++) {
            const float s = p.w_scale_f16 ? __half2float(__ushort_as_half((unsigned short)rs[i])) : __uint_as_float(rs[i]);
            const _Float16 sh = (_Float16)(s * rinv[i]);
            const f16x2 s2 = {sh, sh};
            const uint32_t w[4] = {rb[i].x, rb[i].y, rb[i].z, rb[i].w};
            const int hh = kB[i] / 32, r = rowB[i];
            uint4 v = decode_lut_f16x8(w[c], TL, TH);
            v.x = mul_f16x2(v.x, s2); v.y = mul_f16x2(v.y, s2);
            v.z = mul_f16x2(v.z, s2); v.w = mul_f16x2(v.w, s2);
            *reinterpret_cast<uint4*>(sw + ((c * (BN / 32) + (r >> 5)) * 64 + frag_slot((r & 31) + 32 * hh)) * 16) = v;
        }
    };
    auto dstore = [&](int st) {
#pragma unroll
        for (int c = 0; c < 4; c++) dstore_chunk(st, c);
    };

    f32x16 acc[TN][TM];
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[j][i][v] = 0.0f;

    // one step: for each K16 block, its MFMAs, then a quarter of the next step's decode
    // (independent of the MFMAs, so it runs while they execute)
    auto step = [&](int st) {
        const uint8_t* sa = smem + st * STAGE;
        const uint8_t* sw = sa + A_BYTES;
        // this lane's activation codes of the step for its TM row tiles: word kk = the 8
        // codes of K16 block kk in its half
        uint4 apk[TM];
        if (PK) {
#pragma unroll
            for (int i = 0; i < TM; i++) {
                const int r = wm * WM + i * 32 + (lane & 31);
                apk[i] = *reinterpret_cast<const uint4*>(sa + r * 32 + (((lane >> 5) ^ ((r >> 3) & 1)) << 4));
            }
        }
#pragma unroll
        for (int kk = 0; kk < 4; kk++) {
            f16x8 af[TM];
#pragma unroll
            for (int i = 0; i < TM; i++) {
                if (PK) {
                    const uint32_t w4[4] = {apk[i].x, apk[i].y, apk[i].z, apk[i].w};
                    af[i] = __builtin_bit_cast(f16x8, decode_e2m1_f16x8(w4[kk]));
                } else {
                    af[i] = __builtin_bit_cast(
                        f16x8, *reinterpret_cast<const uint4*>(sa + ((kk * (BM / 32) + wm * TM + i) * 64 + frag_slot(lane)) * 16));
                }
            }
#pragma unroll
            for (int j = 0; j < TN; j++) {
                const f16x8 bf = __builtin_bit_cast(f16x8, *reinterpret_cast<const uint4*>(sw + ((kk * (BN / 32) + wn * TN + j) * 64 + frag_slot(lane)) * 16));
#pragma unroll
                for (int i = 0; i < TM; i++) acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf, af[i], acc[j][i], 0, 0, 0);
            }
            dstore_chunk(st ^ 1, kk);
            // interleave: each MFMA is followed by decode work, which then runs while the
            // MFMA executes
#pragma unroll
            for (int x = 0; x < TM * TN; x++) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four VALU
            }
        }
    };

    gload(0);
    dstore(0);
    gload(1);
    __syncthreads();
    // step k computes stage k%2 and fills stage (k+1)%2 with step k+1 (loaded during
    // step k-1); the loads for step k+2 are issued afterwards.  Past the last step the
    // loads read zeros or unused codes and the decoded stage is never read.
    for (int k = 0; k < nk; k++) {
        step(k & 1);
        gload(k + 2);
        __syncthreads();
    }

    // epilogue: y = fl32(acc * fl32(a * 2^e_n)); value v of lane l holds output row
    // m = l%32 (+ tile offsets) and column n = 8*(v/4) + 4*(l/32) + v%4
    const float a = p.a_scale[0];
    const int r32 = lane & 31, hk = lane >> 5;
#pragma unroll
    for (int j = 0; j < TN; j++) {
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const int nl = wn * WN + j * 32 + 8 * g + 4 * hk;
            float f[4];
#pragma unroll
            for (int t = 0; t < 4; t++) f[t] = a * rowfac[nl + t];
            const int64_t nb = n0 + nl;
#pragma unroll
            for (int i = 0; i < TM; i++) {
                const int64_t m = m0 + wm * WM + i * 32 + r32;
                if (m >= p.M) continue;
                float y[4];
#pragma unroll
                for (int t = 0; t < 4; t++) y[t] = acc[j][i][4 * g + t] * f[t];
                if (p.y_bf16) {
                    __bf16* yp = reinterpret_cast<__bf16*>(p.y) + m * p.ldy + nb;
                    if (nb + 4 <= p.N && ((reinterpret_cast<uintptr_t>(yp) & 7) == 0)) {
                        __bf16 h4[4] = {(__bf16)y[0], (__bf16)y[1], (__bf16)y[2], (__bf16)y[3]};
                        *reinterpret_cast<uint2*>(yp) = __builtin_bit_cast(uint2, h4);
                    } else {
                        for (int t = 0; t < 4; t++)
                            if (nb + t < p.N) yp[t] = (__bf16)y[t];
                    }
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

static int lut_cu_count() {
    static int counts[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (counts[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        counts[dev] = n;
    }
    return counts[dev];
}
static void lut256(const GemmParams& p, hipStream_t s) {
    const int64_t gm = (p.M + 255) / 256, gn = (p.N + 255) / 256;
    hipLaunchKernelGGL((w4a4_lut_kernel<256, 256, false>), dim3((unsigned)(gm * gn)), dim3(256), 0, s, p, (int)gm);
}
static void lut128(const GemmParams& p, hipStream_t s) {
    const int64_t gm = (p.M + 127) / 128, gn = (p.N + 127) / 128;
    hipLaunchKernelGGL((w4a4_lut_kernel<128, 128, true>), dim3((unsigned)(gm * gn)), dim3(256), 0, s, p, (int)gm);
}
// Whole rounds of 256x256 tiles (one workgroup per CU at a time); the column block left
// for a partial last round, and grids with fewer 256x256 tiles than CUs, as 128x128
// tiles with packed activations in LDS (several workgroups per CU).
static hipError_t launch_lut_block(const GemmParams& p, hipStream_t s) {
    const int64_t gm256 = (p.M + 255) / 256, gn256 = (p.N + 255) / 256, t256 = gm256 * gn256;
    const int64_t cus = lut_cu_count();
    if (t256 < cus) {
        lut128(p, s);
        return hipGetLastError();
    }
    const int64_t n1 = std::min<int64_t>(p.N, (t256 / cus) * cus / gm256 * 256);
    if (n1 >= p.N || t256 % cus == 0) {
        lut256(p, s);
        return hipGetLastError();
    }
    GemmParams q = p;
    q.N = n1;
    lut256(q, s);
    const int64_t srow = (p.K / p.w_group) * (p.w_scale_f16 ? 2 : 4);  // scale bytes per weight row
    q = p;
    q.N = p.N - n1;
    q.w = p.w + n1 * p.ldw;
    q.w_scales = reinterpret_cast<const uint8_t*>(p.w_scales) + n1 * srow;
    q.y = reinterpret_cast<uint8_t*>(p.y) + n1 * (p.y_bf16 ? 2 : 4);
    lut128(q, s);
    return hipGetLastError();
}

// Buffer offsets are 32-bit and kOOB marks "past the end", so one launch covers at most
// kLutMaxBufBytes of A, of W and of the scales; larger operands are split into row
// blocks (multiples of 256 rows), each launched on pointers advanced to its start.
constexpr int64_t kLutMaxBufBytes = 0x7fff0000;

hipError_t launch_w4a4_lut(const GemmParams& p, hipStream_t s) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    const int64_t srow = (p.K / p.w_group) * (p.w_scale_f16 ? 2 : 4);  // scale bytes per weight row
    const int64_t mstep = std::max<int64_t>(256, kLutMaxBufBytes / std::max<int64_t>(p.lda, 1) / 256 * 256);
    const int64_t nstep = std::max<int64_t>(
        256, std::min(kLutMaxBufBytes / std::max<int64_t>(p.ldw, 1), kLutMaxBufBytes / std::max<int64_t>(srow, 1)) / 256 * 256);
    const size_t ysz = p.y_bf16 ? 2 : 4;
    for (int64_t m0 = 0; m0 < p.M; m0 += mstep) {
        for (int64_t n0 = 0; n0 < p.N; n0 += nstep) {
            GemmParams q = p;
            q.M = std::min(mstep, p.M - m0);
            q.N = std::min(nstep, p.N - n0);
            q.a = reinterpret_cast<const uint8_t*>(p.a) + m0 * p.lda;
            q.w = p.w + n0 * p.ldw;
            q.w_scales = reinterpret_cast<const uint8_t*>(p.w_scales) + n0 * srow;
            q.y = reinterpret_cast<uint8_t*>(p.y) + (m0 * p.ldy + n0) * ysz;
            const hipError_t e = launch_lut_block(q, s);
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace fp4

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
// Tiling for CDNA4: a workgroup computes BM x BN tiles of Y (256x256 for whole rounds
// of tiles, 256x128 or 128x128 for the column block of a partial last round, 128x256 or
// 128x128 for small grids) with 2x4 wavefronts (256x256, 128x256: two per SIMD) or 2x2;
// each wavefront a
// (BM/2) x (BN/4 or BN/2) sub-tile as a grid of 32x32 accumulators.  K advances 128 codes (64 bytes per row) per step
// through a four-stage LDS ring fed by direct-to-LDS loads.  One workgroup per compute
// unit loops over tiles (each XCD over its own range of them, so that an XCD reads
// about an eighth of W); the load ring runs on across tile boundaries, so the next
// tile's first steps load while the last ones of the current tile are computed and
// while its epilogue writes its outputs.
//
// The same kernel also runs the LLaMA MLP's gate/up pair with SwiGLU and the next
// layer's E2M1 quantization in the epilogue (GLU), and the FP8 E4M3 x E4M3 product
// (F8: one code per byte, 64-code steps; fp32 sums not exact, so held to a tolerance;
// E5M2 x E5M2 and the mixed FP8 pairs too) with tensor or row weight scales or, on
// 128x256 tiles, one scale per row and group of 64 or 128 ([W8A8] section 2.2's group
// size) codes (F8 = 12 / 13, 2 / 3 for f32 / f16 scales) or f32 scales per 256 (F8 = 14),
// and FP6 x FP6 of one format (F8 = 8 / 9: 96-byte rows of 128-code steps, 128x128 tiles).
#include <algorithm>
#include <atomic>

#include "fp4_device.h"

namespace fp4 {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBKBytes = 64;  // 128 codes per K step

// A stage row is 64 bytes (four 16-byte segments); segment seg of row r sits in slot
// seg ^ ((r >> 2) & 3).  The 128-bit fragment reads are served 16 lanes at a time, the
// lanes of a group reading 16 consecutive rows at the same segment: rows r, r + 4, r + 8,
// r + 12 share their position in the 256-byte bank row and the XOR with r / 4 sends them
// to four different slots, so the 16 reads cover all 64 banks once.  (An XOR with r / 2
// repeats every 8 rows and left every group 2-way conflicted: half of all LDS cycles
// were bank-conflict cycles in the counters.)
__device__ __forceinline__ int swz(int row, int seg) { return row * kBKBytes + ((seg ^ ((row >> 2) & 3)) << 4); }

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Operands move HBM -> LDS with gfx950's direct-to-LDS buffer loads (no staging
// registers): lane l of a wavefront writes LDS bytes [16 l, 16 l + 16) of a 1 KiB block,
// so each lane fetches the global 16-byte piece that belongs at that slot of the
// XOR-swizzled tile (the 16-byte segments of a row are permuted by row so that the
// 128-bit LDS reads of a wavefront spread over all banks).  Rows past M or N and K
// tails get an offset past the buffer's end, which the hardware returns as zeros.
// Four LDS stages: the loads for step k+4 are issued while step k is computed.
//
// 32x32x64 FP4 MFMAs (the 16x16x128 form issues at only the FP8 rate on gfx950), with
// operands swapped -- D = W_tile * A_tile^T -- so a lane's accumulator holds 4
// consecutive output columns of one row.  FP4 operand layout: lane l holds 32
// consecutive codes (16 B) of row l%32 at K offset 32*(l/32); D layout: lane l, value v
// holds D[8*(v/4) + 4*(l/32) + v%4][l%32].  A bf16 result tile is staged in each
// wavefront's own LDS area and written with 16-byte stores.

// Wait until at most N direct-to-LDS loads of this thread are in flight and every LDS
// read of this wavefront has returned, then meet the workgroup barrier.  The LDS reads
// must be complete: after the barrier other wavefronts start loads into the stage
// those reads came from.  One asm block, so the compiler cannot move the reads past it.
#define FP4_SYNC(N) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory")

// Read an accumulator from its AGPR (keeps the accumulators in AGPRs across the tile loop)
__device__ __forceinline__ float agpr_read(float a) {
    float v;
    asm("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
    return v;
}

// Wait for every outstanding memory operation of this thread (loads and stores), every
// LDS read, and the workgroup barrier.
#define FP4_SYNC_ALL() asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" : : : "memory")
// Wait for this wavefront's LDS operations and meet the workgroup barrier.
#define FP4_BAR() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory")
// Wait for this wavefront's LDS operations.
#define FP4_LDS_WAIT() asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory")
// Meet the workgroup barrier (separates two load groups; waits for nothing).
#define FP4_BARRIER_ONLY() asm volatile("s_barrier" : : : "memory")
// One buffer store at an offset past the end of `none` (a buffer of size zero): the
// hardware discards it, and counts it among this thread's outstanding memory operations
// until it completes, in issue order with the others.
__device__ __forceinline__ void discarded_store(i32x4v none) {
    asm volatile("buffer_store_dword %0, %1, %2, 0 offen" : : "v"(0), "v"(kOOB), "s"(none) : "memory");
}

// e^x as a fixed sequence of binary32 operations (bit-reproducible on any IEEE
// binary32 implementation of the same sequence; built without contraction): t =
// fl(x * log2 e), n = rint(t), f = t - n (exact), 2^f by its degree-7 Taylor polynomial
// ((ln 2)^i / i!, rounded to binary32) in Horner form, times 2^n.  Relative error below
// 1e-5 for |x| <= 88.
__device__ __forceinline__ float exp_f32(float x) {
    const float t = x * 0x1.715476p+0f;
    const float n = rintf(t);
    const float f = t - n;
    float q = 0x1.ffcbfcp-17f;
    q = q * f + 0x1.430912p-13f;
    q = q * f + 0x1.5d87fep-10f;
    q = q * f + 0x1.3b2ab6p-7f;
    q = q * f + 0x1.c6b08ep-5f;
    q = q * f + 0x1.ebfbe0p-3f;
    q = q * f + 0x1.62e430p-1f;
    q = q * f + 1.0f;
    return ldexpf(q, (int)fminf(fmaxf(n, -300.0f), 300.0f));
}
// SiLU(x) = x / (1 + e^-x), the division correctly rounded
__device__ __forceinline__ float silu_f32(float x) { return x / (1.0f + exp_f32(-x)); }

// GLU = false: Y = the W4A4 product through the fixed epilogue (bf16 or f32).
// GLU = true: a tile's B rows [0, BN/2) are gate rows and [BN/2, BN) the up rows of the
// same BN/2 output columns; each wavefront computes the gate and the up products of the
// same rows and BN/4 output columns, and its epilogue writes E2M1 codes of
// h = fl32(SiLU(y_gate) * y_up) quantized with the next layer's scale and shifts.
// F8 = 1: OCP FP8 E4M3 operands (one code per byte; no SwiGLU): a step is 64 codes (the
// same 64 bytes per row), one 32x32x64 FP8 MFMA K-block whose lane fragment is the two
// 16-byte segments 2 hk, 2 hk + 1 (read as the two "halves" of the FP4 pipeline).
// NWV = 4 or 8 wavefronts per workgroup in a 2 x NWV/2 grid (rows x columns of the
// tile): with 8, two wavefronts share each SIMD, so one's LDS fragment reads overlap the
// other's MFMAs (each holds a (BM/2) x (BN/4) sub-tile, half the accumulators).
template <int BM, int BN, bool GLU, int F8 = 0, int NWV = 4>
__global__ void __launch_bounds__(64 * NWV) w4a4_fp4_kernel(GemmParams p, int grid_m, int ntiles, GluParams gp) {
    constexpr int CPB = F8 ? 1 : 2;  // codes per byte
    // F8 = 2 / 3: E4M3 weights with one f32 / f16 scale per output row and group of 128
    // codes along K (12 / 13: groups of 64, 14: f32 scales per 256): each group's MFMA sum
    // P_g (GS 64-code K-blocks) is folded into a running sum T = fma(P_g, s[n, g], T) once
    // the group's last MFMA has issued, and the epilogue gives y = fl32(T * a_m)
    constexpr bool GRP = F8 == 2 || F8 == 3 || (F8 >= 12 && F8 <= 15);
    constexpr bool GF16 = F8 == 3 || F8 == 13 || F8 == 15;
    constexpr int GS = (F8 == 12 || F8 == 13) ? 1 : (F8 == 14 || F8 == 15) ? 4 : 2;  // steps per group
    // F8 = 4 / 5 / 6: OCP FP8 E5M2 x E5M2, E4M3 weights x E5M2 activations, E5M2 weights x
    // E4M3 activations (the MFMA's format codes: 0 E4M3, 1 E5M2; both formats take the same
    // K order in the matrix cores), tensor or row weight scales; the other FP8 instances are
    // E4M3 x E4M3
    constexpr int FCW = (F8 == 4 || F8 == 6) ? 1 : 0, FCA = (F8 == 4 || F8 == 5) ? 1 : 0;
    // F8 = 8 / 9: FP6 E2M3 / E3M2 on both operands (128x128 tiles, 4 wavefronts).  A step
    // is 128 codes, 96 bytes per row (six 16-byte segments); a lane's fragment of a 64-code
    // K-block is the 24 bytes [48 H + 24 hk, +24) of its row, read as three 8-byte pieces.
    // Both operands take the same order of K, so the product is the same as in the matrix
    // cores' own FP6 order.  Segment g of stage row r sits in slot (g + 3 ((r >> 3) & 1)) % 6:
    // rows r and r + 8 (the same banks at a 96-byte row stride) then differ by 12 banks.
    constexpr bool F6 = F8 == 8 || F8 == 9;
    constexpr int FC6 = F8 == 9 ? 3 : 2;
    constexpr int RB = F6 ? 96 : kBKBytes;  // bytes per row and step
    constexpr int NSEG = RB / 16;
    static_assert(!F6 || (BM == 128 && BN == 128 && NWV == 4 && !GLU), "FP6: 128x128 tiles");
    static_assert(!GRP || (BM == 128 && BN == 256 && NWV == 8 && !GLU), "group-scaled FP8: 128x256 tiles");
    constexpr int WM = BM / 2, WN = BN / (NWV / 2);
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int LA = BM * NSEG / (64 * NWV), LB = BN * NSEG / (64 * NWV);  // 16-byte pieces per thread per step
    constexpr int STAGE = (BM + BN) * RB;
    // four operand stages, per tile parity a block of per-column weight scales and the
    // tile's per-row (per-token) activation scales, 1 KiB each (GLU: gate scales, up
    // scales and the output shifts), and each wavefront's output staging area (32 rows x
    // WN/2 bf16 columns; GLU: its columns' multipliers and 32 rows of codes)
    constexpr int SCL_BYTES = GLU ? 3072 : 2048;
    constexpr int STG_BYTES = GLU ? 2048 : 32 * WN;
    constexpr int ON = GLU ? BN / 2 : BN;  // output columns per tile
    // GRP: two blocks of the tile's group scales (256 columns x 16 bytes: the 16 bytes of a
    // column's scale row from the first group of a four-step group on), and 1 KiB that the
    // scale loads of the wavefronts without a column share write and no one reads
    constexpr int GS_BYTES = GRP ? 9 * 1024 : 0;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * STAGE + 2 * SCL_BYTES + NWV * STG_BYTES + GS_BYTES];
    constexpr int BOFF = BM * RB;  // a stage: its A block, then its B block
    uint8_t* const st0 = smem;
    uint8_t* const st1 = smem + STAGE;
    uint8_t* const st2 = smem + 2 * STAGE;
    uint8_t* const st3 = smem + 3 * STAGE;
    uint8_t* const scl = smem + 4 * STAGE;
    uint8_t* const stg_base = smem + 4 * STAGE + 2 * SCL_BYTES;
    uint8_t* const stg = stg_base + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * STG_BYTES;
    uint8_t* const gsb = smem + 4 * STAGE + 2 * SCL_BYTES + NWV * STG_BYTES;  // GRP scale blocks

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wavefront
    const int wm = wave & 1, wn = wave >> 1;
    const int r32 = lane & 31, hk = lane >> 5;
    const int nk = F6 ? (int)(p.K / 128) : (int)((p.K + 64 * CPB - 1) / (64 * CPB));
    const int kK = (int)p.K;  // 32-bit bound checks (rows are below 2^31 bytes; K far smaller)
    // The step count per tile is rounded up to a multiple of 4 (the stage rotation);
    // steps past the last real one load zeros (out-of-range offsets) and add nothing.
    const int nk4 = (nk + 3) & ~3;

    const i32x4v rsA = buf_words(p.a, p.M * p.lda);
    const i32x4v rsB = buf_words(p.w, p.N * p.ldw);
    const i32x4v rsB2 = GLU ? buf_words(gp.w_up, p.N * p.ldw) : rsB;
    const i32x4v rsS = buf_words(p.w_scales, p.w_mode == 1 ? p.N * 4 : 4);
    const i32x4v rsS2 = GLU ? buf_words(gp.s_up, p.N * 4) : rsS;
    const i32x4v rsK = (GLU && gp.out_shift) ? buf_words(gp.out_shift, p.N) : buf_words(p.w_scales, 0);
    const i32x4v rsR = buf_words(p.a_scale, p.a_row ? p.M * 4 : 0);  // per-token scales
    // read before any store of this kernel, so they can come through the scalar cache
    const float a_scale = p.a_scale[0];
    const float s_tensor = reinterpret_cast<const float*>(p.w_scales)[0];
    const float r_out = GLU ? recip_or_zero(gp.out_scale[0]) : 0.0f;  // next layer's fl32(1 / a')

    // Loads run ahead of the MFMAs through the tiles of this workgroup (tile t covers
    // rows bm*BM.., columns bn*BN.. with bm = t % grid_m, bn = t / grid_m; the tiles of a
    // workgroup in turn: tile_of below).  State of the load stream: its tile dt, and per
    // load the global piece behind this lane's LDS slot (slot s = (NWV i + wave) * 64 +
    // lane holds row s/4, swizzled segment s%4; see swz).
    int segk[LA > LB ? LA : LB];
#pragma unroll
    for (int i = 0; i < (LA > LB ? LA : LB); i++) {
        if constexpr (F6) {  // bytes: the segment stored in slot sidx % 6 of row sidx / 6
            const int sidx = (NWV * i + wave) * 64 + lane, row = sidx / 6;
            segk[i] = ((sidx - 6 * row + 3 * ((row >> 3) & 1)) % 6) * 16;
        } else {
            int sidx = (NWV * i + wave) * 64 + lane, row = sidx >> 2;
            segk[i] = ((sidx & 3) ^ ((row >> 2) & 3)) * 16 * CPB;  // codes (the segment stored in slot sidx % 4)
        }
    }
    uint32_t offA[LA], offB[LB], offS, offK, offR, offG = kOOB;
    // GRP: scale bytes per element and per output row (K / (64 GS) groups)
    constexpr int gsz = GF16 ? 2 : 4;
    const int64_t grow = GRP ? p.K / (64 * GS) * gsz : 0;
    const i32x4v rsG = buf_words(p.w_scales, GRP ? p.N * grow : 0);
    // Tile order.  Workgroups are dispatched to the 8 XCDs in turn (workgroup b on XCD
    // b % 8), each XCD with its own L2.  When the grid is a multiple of 8, XCD x takes the
    // column blocks [grid_n x / 8, grid_n (x + 1) / 8) and its workgroups share that
    // block's tiles in turn, ordered in panels of P row blocks: panel by panel, and within
    // a panel column by column.  The tiles an XCD computes at the same time then form a
    // compact block (4 row blocks x 8 column blocks for 32 workgroups), whose operand
    // row and column blocks are fetched from HBM about once per round instead of all row
    // blocks for every two columns.  Where whole columns per XCD would give some
    // workgroup more tiles than an even split of the tiles does (few columns), XCD x takes
    // the tiles [ntiles x / 8, ntiles (x + 1) / 8) of the column-major order instead.
    // Otherwise (a grid that is not a multiple of 8) workgroup b takes tiles b, b + grid, ...
    constexpr int kXcds = 8;
#ifndef FP4_PANEL
#define FP4_PANEL 4
#endif
    const bool xcd_order = gridDim.x % kXcds == 0;
    const int xcd = blockIdx.x % kXcds, xwg = blockIdx.x / kXcds, xwgs = gridDim.x / kXcds;
    const int grid_n = ntiles / grid_m;
    const int c_first = (int)((int64_t)grid_n * xcd / kXcds);
    const int c_cnt = (int)((int64_t)grid_n * (xcd + 1) / kXcds) - c_first;
    const int pan = grid_m < FP4_PANEL ? grid_m : FP4_PANEL;
    const int full_rows = grid_m / pan * pan;  // rows in whole panels
    // tiles per workgroup at most, whole columns per XCD against an even split
    const int64_t by_cols = ((grid_n + kXcds - 1) / kXcds * (int64_t)grid_m + xwgs - 1) / xwgs;
    const int64_t by_tiles = (((int64_t)ntiles + kXcds - 1) / kXcds + xwgs - 1) / xwgs;
    const bool panels = by_cols <= by_tiles;
    const int x_first = (int)((int64_t)ntiles * xcd / kXcds);
    const int x_count = panels ? grid_m * c_cnt : (int)((int64_t)ntiles * (xcd + 1) / kXcds) - x_first;
    auto tile_of = [&](int k) -> int {  // this workgroup's k-th tile, or ntiles once done
        if (!xcd_order) {
            const int64_t t = blockIdx.x + (int64_t)k * gridDim.x;
            return t < ntiles ? (int)t : ntiles;
        }
        const int64_t u64 = xwg + (int64_t)k * xwgs;
        if (u64 >= x_count) return ntiles;
        const int u = (int)u64;
        if (!panels) return x_first + u;
        int row, col;
        if (u < full_rows * c_cnt) {
            const int pn = u / (pan * c_cnt), v = u - pn * pan * c_cnt;
            col = v / pan;
            row = pn * pan + (v - col * pan);
        } else {  // the last panel, grid_m % pan rows
            const int h = grid_m - full_rows, v = u - full_rows * c_cnt;
            col = v / h;
            row = full_rows + (v - col * h);
        }
        return (c_first + col) * grid_m + row;
    };
    int dk = 0, dt = tile_of(0), dpar = 0;
    auto load_tile = [&](int t) {
        const bool ok = t < ntiles;
        const int64_t m0 = (int64_t)(t % grid_m) * BM, n0 = (int64_t)(t / grid_m) * ON;
#pragma unroll
        for (int i = 0; i < LA; i++) {
            int row = F6 ? ((NWV * i + wave) * 64 + lane) / 6 : ((NWV * i + wave) * 64 + lane) >> 2;
            offA[i] = (ok && m0 + row < p.M) ? (uint32_t)((m0 + row) * p.lda + (F6 ? segk[i] : segk[i] / CPB)) : kOOB;
        }
#pragma unroll
        for (int i = 0; i < LB; i++) {
            int row = F6 ? ((NWV * i + wave) * 64 + lane) / 6 : ((NWV * i + wave) * 64 + lane) >> 2;
            if (GLU && i >= LB / 2) row -= BN / 2;  // up rows (their own buffer)
            offB[i] = (ok && n0 + row < p.N) ? (uint32_t)((n0 + row) * p.ldw + (F6 ? segk[i] : segk[i] / CPB)) : kOOB;
        }
        offS = (ok && p.w_mode == 1 && n0 + 4 * lane < p.N && 4 * lane < ON) ? (uint32_t)((n0 + 4 * lane) * 4) : kOOB;
        offK = (ok && 16 * lane < ON && n0 + 16 * lane < p.N) ? (uint32_t)(n0 + 16 * lane) : kOOB;
        offR = (ok && p.a_row && 4 * lane < BM && m0 + 4 * lane < p.M) ? (uint32_t)((m0 + 4 * lane) * 4) : kOOB;
        if constexpr (GRP) {  // wavefronts 0..3: column 64 wave + lane of the tile
            const int64_t n = n0 + 64 * wave + lane;
            offG = (ok && wave < 4 && n < p.N) ? (uint32_t)(n * grow) : kOOB;
        }
    };
    load_tile(dt);
    // this wavefront's LDS slot base: load piece i of a stage goes to stage + (NWV i + wave) KiB
    const uint32_t wave_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&smem[wave * 1024]);

// direct-to-LDS loads of step KB of the load stream's tile into stage array STG
#define FP4_DMAK(STG, KB)                                                                                  \
    do {                                                                                                   \
        const int kb_ = (KB);                                                                              \
        const uint32_t st_ = (uint32_t)((STG) - smem);                                                     \
        _Pragma("unroll") for (int i = 0; i < LA; i++) {                                                   \
            uint32_t off = (F6 ? kb_ < nk : kb_ * 64 * CPB + segk[i] < kK) ? offA[i] + (uint32_t)kb_ * RB : kOOB; \
            dma16_at(rsA, off, wave_lds, st_ + (uint32_t)(NWV * i * 1024));                                \
        }                                                                                                  \
        _Pragma("unroll") for (int i = 0; i < LB; i++) {                                                   \
            uint32_t off = (F6 ? kb_ < nk : kb_ * 64 * CPB + segk[i] < kK) ? offB[i] + (uint32_t)kb_ * RB : kOOB; \
            dma16_at((GLU && i >= LB / 2) ? rsB2 : rsB, off, wave_lds, st_ + (uint32_t)(BOFF + NWV * i * 1024)); \
        }                                                                                                  \
    } while (0)
// the load stream's tile's 256 column scales into scales block dpar, and its BM
// per-token activation scales after them (zeros without them); all wavefronts load the
// same bytes, so every thread issues the same number of loads.  The epilogue reads the
// per-token scales from LDS: a register load there would need a full vmcnt(0) wait,
// which would also wait for the next tile's first four steps.
#define FP4_DMAS()                                                                                         \
    do {                                                                                                   \
        const uint32_t sb_ = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&scl[dpar * SCL_BYTES]); \
        dma16(rsS, offS, sb_);                                                                             \
        if (GLU) {                                                                                         \
            dma16(rsS2, offS, sb_ + 1024);                                                                 \
            dma16(rsK, offK, sb_ + 2048);                                                                  \
        } else {                                                                                           \
            dma16(rsR, offR, sb_ + 1024);                                                                  \
        }                                                                                                  \
    } while (0)
// GRP: the group scales of the four-step group that starts at step KB (a multiple of 4)
// of the load stream's tile into scale block BLK: 16 bytes of each column's scale row
// from group KB / GS on (f32: four groups, f16: eight; the four steps use the first
// 4 / GS).  Every thread issues one load (wavefronts 4..7 an out-of-range one into the
// unread KiB), so that all threads issue the same number of memory operations.
#define FP4_DMAG(KB, BLK)                                                                                  \
    do {                                                                                                   \
        if constexpr (GRP) {                                                                               \
            const uint32_t go_ = offG == kOOB ? kOOB : offG + (uint32_t)((KB) / GS * gsz);                 \
            const uint32_t gb_ = (uint32_t)(uintptr_t)gsb + (wave < 4 ? (BLK) * 4096 + wave * 1024 : 8192); \
            dma16(rsG, go_, __builtin_amdgcn_readfirstlane(gb_));                                          \
        }                                                                                                  \
    } while (0)
// the load stream moves on to this workgroup's next tile
#define FP4_NEXT_TILE()                                                                                    \
    do {                                                                                                   \
        dt = tile_of(++dk);                                                                                \
        dpar ^= 1;                                                                                         \
        load_tile(dt);                                                                                     \
    } while (0)

// fragments of half H of a step (K codes 64 H .. 64 H + 63 under the stage's segment
// order): FA[i] for A (rows), FB[j] for W (columns), 16 bytes each.  B row of fragment
// j: wn * WN + 32 j; GLU: fragments [0, TN/2) are gate rows wn * WN/2 + 32 j and
// [TN/2, TN) the up rows of the same columns.
#define FP4_READH(STG, H, FA, FB)                                                                          \
    do {                                                                                                   \
        const int sg_ = F8 ? 2 * hk + (H) : 2 * (H) + hk;                                                  \
        _Pragma("unroll") for (int i = 0; i < TM; i++) FA[i] =                                             \
            *reinterpret_cast<const uint4*>(&STG[swz(wm * WM + i * 32 + r32, sg_)]);                       \
        _Pragma("unroll") for (int j = 0; j < TN; j++) FB[j] =                                             \
            *reinterpret_cast<const uint4*>(&STG[BOFF + swz(brow(j) + r32, sg_)]);                         \
    } while (0)
// the MFMAs of one half step from fragment registers, with the LDS reads of the next
// half step (issued just before) spread between them
#define FP4_MMAH(FA, FB)                                                                                   \
    do {                                                                                                   \
        _Pragma("unroll") for (int j = 0; j < TN; j++) {                                                   \
            const uint4 v = FB[j];                                                                         \
            const i32x8 bf = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};                   \
            _Pragma("unroll") for (int i = 0; i < TM; i++) {                                               \
                const uint4 u = FA[i];                                                                     \
                const i32x8 af = i32x8{(int)u.x, (int)u.y, (int)u.z, (int)u.w, 0, 0, 0, 0};                \
                acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf, af, acc[j][i], 4, 4, 0, 127, 0, 127); \
            }                                                                                              \
        }                                                                                                  \
        _Pragma("unroll") for (int g = 0; g < TM + TN; g++) {                                              \
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                             \
            __builtin_amdgcn_sched_group_barrier(0x008, (TM * TN + TM + TN - 1) / (TM + TN), 0);           \
        }                                                                                                  \
    } while (0)

    auto brow = [&](int j) {
        return GLU ? (j / (TN / 2)) * (BN / 2) + wn * (WN / 2) + (j % (TN / 2)) * 32 : wn * WN + j * 32;
    };
// FP8: the MFMAs of the step held in registers (lo 16 bytes in x, hi 16 bytes in y),
// refilling each fragment with step SN's as soon as its last MFMA has issued: the B
// fragments of column block j after that block's MFMAs, the A fragments at the end.
#define FP4_MMA8(SN)                                                                                       \
    do {                                                                                                   \
        _Pragma("unroll") for (int j = 0; j < TN; j++) {                                                   \
            const i32x8 bf = i32x8{(int)xb[j].x, (int)xb[j].y, (int)xb[j].z, (int)xb[j].w,                 \
                                   (int)yb[j].x, (int)yb[j].y, (int)yb[j].z, (int)yb[j].w};                \
            _Pragma("unroll") for (int i = 0; i < TM; i++) {                                               \
                const i32x8 af = i32x8{(int)xa[i].x, (int)xa[i].y, (int)xa[i].z, (int)xa[i].w,             \
                                       (int)ya[i].x, (int)ya[i].y, (int)ya[i].z, (int)ya[i].w};            \
                acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf, af, acc[j][i], FCW, FCA, 0, 127, 0, 127); \
            }                                                                                              \
            xb[j] = *reinterpret_cast<const uint4*>(&SN[BOFF + swz(brow(j) + r32, 2 * hk)]);               \
            yb[j] = *reinterpret_cast<const uint4*>(&SN[BOFF + swz(brow(j) + r32, 2 * hk + 1)]);           \
        }                                                                                                  \
        _Pragma("unroll") for (int i = 0; i < TM; i++) {                                                   \
            xa[i] = *reinterpret_cast<const uint4*>(&SN[swz(wm * WM + i * 32 + r32, 2 * hk)]);             \
            ya[i] = *reinterpret_cast<const uint4*>(&SN[swz(wm * WM + i * 32 + r32, 2 * hk + 1)]);         \
        }                                                                                                  \
    } while (0)
// FP6: LDS byte of the 8-byte piece at byte B (a multiple of 8) of stage row R
    auto f6_at = [&](int R, int B) { return R * 96 + (((B >> 4) + 3 * ((R >> 3) & 1)) % 6) * 16 + (B & 8); };
// FP6: both K-blocks of a step, three 8-byte pieces per fragment
#define FP6_READ(STG)                                                                                      \
    do {                                                                                                   \
        _Pragma("unroll") for (int i = 0; i < TM; i++)                                                     \
            _Pragma("unroll") for (int h = 0; h < 2; h++)                                                  \
                _Pragma("unroll") for (int m = 0; m < 3; m++) fa6[i][h][m] =                               \
                    *reinterpret_cast<const uint2*>(&STG[f6_at(wm * WM + i * 32 + r32, 48 * h + 24 * hk + 8 * m)]); \
        _Pragma("unroll") for (int j = 0; j < TN; j++)                                                     \
            _Pragma("unroll") for (int h = 0; h < 2; h++)                                                  \
                _Pragma("unroll") for (int m = 0; m < 3; m++) fb6[j][h][m] =                               \
                    *reinterpret_cast<const uint2*>(&STG[BOFF + f6_at(brow(j) + r32, 48 * h + 24 * hk + 8 * m)]); \
    } while (0)
// FP6: the step's MFMAs from registers, refilling each fragment with step SN's as soon as
// its last MFMA has issued (the W fragments of column block j after that block's MFMAs,
// the A fragments at the end)
#define FP6_MMA(SN)                                                                                        \
    do {                                                                                                   \
        _Pragma("unroll") for (int j = 0; j < TN; j++) {                                                   \
            _Pragma("unroll") for (int h = 0; h < 2; h++) {                                                \
                const i32x8 bf = i32x8{(int)fb6[j][h][0].x, (int)fb6[j][h][0].y, (int)fb6[j][h][1].x,      \
                                       (int)fb6[j][h][1].y, (int)fb6[j][h][2].x, (int)fb6[j][h][2].y, 0, 0}; \
                _Pragma("unroll") for (int i = 0; i < TM; i++) {                                           \
                    const i32x8 af = i32x8{(int)fa6[i][h][0].x, (int)fa6[i][h][0].y, (int)fa6[i][h][1].x,  \
                                           (int)fa6[i][h][1].y, (int)fa6[i][h][2].x, (int)fa6[i][h][2].y, 0, 0}; \
                    acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf, af, acc[j][i], FC6, FC6, 0, 127, 0, 127); \
                }                                                                                          \
            }                                                                                              \
            _Pragma("unroll") for (int h = 0; h < 2; h++)                                                  \
                _Pragma("unroll") for (int m = 0; m < 3; m++) fb6[j][h][m] =                               \
                    *reinterpret_cast<const uint2*>(&SN[BOFF + f6_at(brow(j) + r32, 48 * h + 24 * hk + 8 * m)]); \
        }                                                                                                  \
        _Pragma("unroll") for (int i = 0; i < TM; i++)                                                     \
            _Pragma("unroll") for (int h = 0; h < 2; h++)                                                  \
                _Pragma("unroll") for (int m = 0; m < 3; m++) fa6[i][h][m] =                               \
                    *reinterpret_cast<const uint2*>(&SN[f6_at(wm * WM + i * 32 + r32, 48 * h + 24 * hk + 8 * m)]); \
    } while (0)
// FP8: the MFMAs of the step in registers, without reads
#define FP4_MMA8_REGS()                                                                                    \
    do {                                                                                                   \
        _Pragma("unroll") for (int j = 0; j < TN; j++) {                                                   \
            const i32x8 bf = i32x8{(int)xb[j].x, (int)xb[j].y, (int)xb[j].z, (int)xb[j].w,                 \
                                   (int)yb[j].x, (int)yb[j].y, (int)yb[j].z, (int)yb[j].w};                \
            _Pragma("unroll") for (int i = 0; i < TM; i++) {                                               \
                const i32x8 af = i32x8{(int)xa[i].x, (int)xa[i].y, (int)xa[i].z, (int)xa[i].w,             \
                                       (int)ya[i].x, (int)ya[i].y, (int)ya[i].z, (int)ya[i].w};            \
                acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf, af, acc[j][i], FCW, FCA, 0, 127, 0, 127); \
            }                                                                                              \
        }                                                                                                  \
    } while (0)
    f32x16 acc[TN][TM];
    uint2 fa6[F6 ? TM : 1][2][3], fb6[F6 ? TN : 1][2][3];  // FP6 fragments of a step
    f32x16 tot[GRP ? TN : 1][GRP ? TM : 1];  // GRP: the sum over the tile's finished groups
    int gcnt = 0;  // GRP: four-step groups computed so far (their scale block is gcnt % 2)
    constexpr int PER_STEP = LA + LB;  // operand loads per step and thread (+2 or +3 with the scales)
    // 16-byte output stores per thread of a staged epilogue (32 rows x WN bf16 columns
    // per wavefront and row block)
    constexpr int CH = WN / 8;  // 16-byte chunks per staged row
    constexpr int ST_PER = 32 * CH / 64;
    constexpr int STORES = TM * ST_PER;
    static_assert(2 * PER_STEP + STORES <= 63, "wait count out of range");
    uint4 xa[TM], xb[TN], ya[TM], yb[TN];
    // Prologue: the first four steps, one load group each (a barrier between groups, as
    // between the phases below).  The first three waits of every tile count, after the
    // awaited step's loads, the next two steps' loads and the previous tile's STORES output
    // stores; before the first tile the same number of stores is issued here, through a
    // buffer of size zero (the hardware discards every store out of a buffer's range, and
    // counts it like any other).  Then wait as every phase does: for the third most recent
    // group (step 1, and step 0 and the scales before it).
    FP4_DMAG(0, 0);
    FP4_DMAK(st0, 0);
    FP4_DMAS();
    FP4_BARRIER_ONLY();
    FP4_DMAK(st1, 1);
    FP4_BARRIER_ONLY();
    FP4_DMAK(st2, 2);
    FP4_BARRIER_ONLY();
    FP4_DMAK(st3, 3);
    {
        const i32x4v none = buf_words(p.a, 0);
#pragma unroll
        for (int i = 0; i < STORES; i++) discarded_store(none);
    }
    FP4_SYNC(2 * PER_STEP + STORES);
    if (!GRP && !F6) FP4_READH(st0, 0, xa, xb);
    if (F8 && BM * BN < 256 * 256 && !GRP && !F6) FP4_READH(st0, 1, ya, yb);
    if constexpr (F6) FP6_READ(st0);

    // Compute stream: tile ct.  Global step s (counted across this workgroup's tiles;
    // every tile has a multiple of 4 steps) lives in stage s % 4.  Phase q: the first
    // half of step q is in registers; read its second half while computing the first;
    // wait until step q+1 landed and every wavefront has read step q (its stage is
    // free), start the load step four ahead into that stage (in a tile's last group: the
    // next tile's first steps), read the first half of step q+1 while computing the
    // second half of step q.  Memory operations of a thread complete in issue order
    // (loads and stores alike), so "step q+1 landed" is "at most the operations issued
    // after it outstanding": the next two steps' loads, and in the first three phases
    // of a tile also the previous tile's output stores.  (A step with the scales has two
    // or three loads more; that only makes a wait longer.)
// (FP8: all of step q is in registers at the start of its phase; wait and meet the
// barrier first -- step q+1 landed, every wavefront holds step q -- start the load into
// q's stage, then run q's MFMAs while reading step q+1 into the registers they free.)
// 256x256 FP8 tiles have no registers to spare for that (spills would break the load
// counting of the waits): there the second halves are read just before the MFMAs.
#define FP4_PHASE(W, SQ, SN, D, PH)                                                                        \
    do {                                                                                                   \
        if constexpr (F6) {                                                                                \
            FP4_SYNC(W);                                                                                   \
            D;                                                                                             \
            FP6_MMA(SN);                                                                                   \
        } else if constexpr (GRP) {                                                                        \
            /* the step's fragments read just before its MFMAs: nothing is held across */             \
            /* the barrier (the running sums take the registers)                        */             \
            FP4_READH(SQ, 0, xa, xb);                                                                      \
            FP4_READH(SQ, 1, ya, yb);                                                                      \
            FP4_MMA8_REGS();                                                                               \
            if constexpr (((PH) + 1) % GS == 0) FP4_FOLD((PH) / GS);                                       \
            FP4_SYNC(W);                                                                                   \
            D;                                                                                             \
        } else if constexpr (F8 && BM * BN < 256 * 256) {                                                  \
            FP4_SYNC(W);                                                                                   \
            D;                                                                                             \
            FP4_MMA8(SN);                                                                                  \
        } else if constexpr (F8) {                                                                         \
            FP4_READH(SQ, 1, ya, yb);                                                                      \
            FP4_MMA8_REGS();                                                                               \
            FP4_SYNC(W);                                                                                   \
            D;                                                                                             \
            FP4_READH(SN, 0, xa, xb);                                                                      \
        } else if constexpr (NWV == 8) {                                                                   \
            /* two wavefronts per SIMD hide each other's fragment reads: one set of      */              \
            /* fragment registers, each half read just before its MFMAs                  */              \
            FP4_MMAH(xa, xb);                                                                              \
            FP4_READH(SQ, 1, xa, xb);                                                                      \
            FP4_MMAH(xa, xb);                                                                              \
            FP4_SYNC(W);                                                                                   \
            D;                                                                                             \
            FP4_READH(SN, 0, xa, xb);                                                                      \
        } else {                                                                                           \
            FP4_READH(SQ, 1, ya, yb);                                                                      \
            FP4_MMAH(xa, xb);                                                                              \
            FP4_SYNC(W);                                                                                   \
            D;                                                                                             \
            FP4_READH(SN, 0, xa, xb);                                                                      \
            FP4_MMAH(ya, yb);                                                                              \
        }                                                                                                  \
    } while (0)
#define FP4_GROUP(W0, W1, W2, D0, D1, D2, D3)                                                              \
    do {                                                                                                   \
        FP4_PHASE(W0, st0, st1, D0, 0);                                                                    \
        FP4_PHASE(W1, st1, st2, D1, 1);                                                                    \
        FP4_PHASE(W2, st2, st3, D2, 2);                                                                    \
        FP4_PHASE(2 * PER_STEP, st3, st0, D3, 3);                                                          \
        if constexpr (GRP) gcnt++;                                                                         \
    } while (0)
// GRP: fold group GG of the current four-step group (the MFMA sums of its GS steps) into the running
// sums: value v of block (j, i) is column wn * WN + 32 j + 8 (v/4) + 4 hk + v%4 of the
// tile; its scale is element GG of that column's 16 bytes in scale block gcnt % 2.  The
// accumulators start the next group at zero.  (Steps past K read zero operands: their
// sums are zero and leave T unchanged.)
#define FP4_FOLD(GG)                                                                                       \
    do {                                                                                                   \
        const uint8_t* gs_ = gsb + (gcnt & 1) * 4096 + (GG) * gsz;                                         \
        _Pragma("unroll") for (int j = 0; j < TN; j++) {                                                   \
            _Pragma("unroll") for (int g = 0; g < 4; g++) {                                                \
                float sc_[4];                                                                              \
                _Pragma("unroll") for (int c = 0; c < 4; c++) {                                            \
                    const uint8_t* a_ = gs_ + (wn * WN + 32 * j + 8 * g + 4 * hk + c) * 16;                \
                    if constexpr (GF16) sc_[c] = __half2float(*reinterpret_cast<const __half*>(a_));       \
                    else sc_[c] = *reinterpret_cast<const float*>(a_);                                     \
                }                                                                                          \
                _Pragma("unroll") for (int i = 0; i < TM; i++)                                             \
                    _Pragma("unroll") for (int c = 0; c < 4; c++) {                                        \
                        tot[j][i][4 * g + c] = __builtin_fmaf(acc[j][i][4 * g + c], sc_[c], tot[j][i][4 * g + c]); \
                        acc[j][i][4 * g + c] = 0.0f;                                                       \
                    }                                                                                      \
                /* four scales live at a time: the VGPRs are taken by the operand pipeline */             \
                __builtin_amdgcn_sched_barrier(0);                                                         \
            }                                                                                              \
        }                                                                                                  \
    } while (0)
    constexpr int WR = 2 * PER_STEP + STORES, WN2 = 2 * PER_STEP;
    const int ngroups = nk4 / 4;
    int ck = 0, ct = tile_of(0), cpar = 0;
    for (;;) {
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int v = 0; v < 16; v++) acc[j][i][v] = 0.0f;
        if constexpr (GRP) {
#pragma unroll
            for (int j = 0; j < TN; j++)
#pragma unroll
                for (int i = 0; i < TM; i++)
#pragma unroll
                    for (int v = 0; v < 16; v++) tot[j][i][v] = 0.0f;
        }
        if (ngroups == 1) {
            FP4_NEXT_TILE();
            FP4_GROUP(WR, WR, WR, { FP4_DMAG(0, (gcnt + 1) & 1); FP4_DMAK(st0, 0); FP4_DMAS(); }, FP4_DMAK(st1, 1),
                      FP4_DMAK(st2, 2), FP4_DMAK(st3, 3));
        } else {
            FP4_GROUP(WR, WR, WR, { FP4_DMAG(4, (gcnt + 1) & 1); FP4_DMAK(st0, 4); }, FP4_DMAK(st1, 5),
                      FP4_DMAK(st2, 6), FP4_DMAK(st3, 7));
            for (int g = 1; g < ngroups - 1; g++)
                FP4_GROUP(WN2, WN2, WN2, { FP4_DMAG(4 * g + 4, (gcnt + 1) & 1); FP4_DMAK(st0, 4 * g + 4); },
                          FP4_DMAK(st1, 4 * g + 5), FP4_DMAK(st2, 4 * g + 6), FP4_DMAK(st3, 4 * g + 7));
            FP4_NEXT_TILE();
            FP4_GROUP(WN2, WN2, WN2, { FP4_DMAG(0, (gcnt + 1) & 1); FP4_DMAK(st0, 0); FP4_DMAS(); }, FP4_DMAK(st1, 1),
                      FP4_DMAK(st2, 2), FP4_DMAK(st3, 3));
        }

        // The epilogue's lane-dependent values are derived again here from a copy of the
        // lane index the compiler cannot see through, so they are not computed before the
        // main loop and held (in registers it needs) across it.
        int lane_e = lane;
        asm volatile("" : "+v"(lane_e));
        const int r32 = lane_e & 31, hk = lane_e >> 5;
        // epilogue of tile ct: y = fl32(acc * fl32(a * s_n)); value v of lane l holds
        // row 32 i + l%32 and column 32 j + 8 (v/4) + 4 (l/32) + v%4 of this wavefront's
        // sub-tile.
        const int64_t m0 = (int64_t)(ct % grid_m) * BM, n0 = (int64_t)(ct / grid_m) * ON;
        const float* sc = reinterpret_cast<const float*>(scl + cpar * SCL_BYTES);
        const float* asc = reinterpret_cast<const float*>(scl + cpar * SCL_BYTES + 1024);  // per-token scales
        if constexpr (GLU) {
            // This wavefront's BN/4 output columns c0 + [0, WN/2) of rows wm * WM + [0, WM):
            // gate accumulators acc[jj], up accumulators acc[jj + TN/2].  First lane l puts
            // column c0 + l's multipliers fl32(a * s_gate), fl32(a * s_up) and
            // fl32(r' * 2^-k') in this wavefront's area; then per 32x32 block: h =
            // fl32(SiLU(y_gate) * y_up), times the multiplier, converted to E2M1 codes
            // (nearest, ties to even, +-6), 32 rows x 16 bytes staged and stored.  Rows past
            // M and 32-column blocks past N are not stored.
            constexpr int WC = WN / 2;  // output columns per wavefront
            const int c0 = wn * WC;
            const int8_t* kq = reinterpret_cast<const int8_t*>(scl + cpar * SCL_BYTES + 2048);
            float* const mul_g = reinterpret_cast<float*>(stg);
            float* const mul_u = mul_g + WC;
            float* const mul_k = mul_g + 2 * WC;
            uint8_t* const cst = stg + 1024;
            if (lane < WC) {
                mul_g[lane] = a_scale * sc[c0 + lane];
                mul_u[lane] = a_scale * sc[256 + c0 + lane];
                mul_k[lane] = ldexpf(r_out, -(int)kq[c0 + lane]);
            }
            FP4_LDS_WAIT();
#pragma unroll
            for (int i = 0; i < TM; i++) {
#pragma unroll
                for (int jj = 0; jj < TN / 2; jj++) {
#pragma unroll
                    for (int g = 0; g < 4; g++) {
                        const int cl = jj * 32 + 8 * g + 4 * hk;  // column within this wavefront's
                        const float4 fg = *reinterpret_cast<const float4*>(&mul_g[cl]);
                        const float4 fu = *reinterpret_cast<const float4*>(&mul_u[cl]);
                        const float4 fk = *reinterpret_cast<const float4*>(&mul_k[cl]);
                        const float fg4[4] = {fg.x, fg.y, fg.z, fg.w}, fu4[4] = {fu.x, fu.y, fu.z, fu.w};
                        const float fk4[4] = {fk.x, fk.y, fk.z, fk.w};
                        float v[4];
#pragma unroll
                        for (int t = 0; t < 4; t++) {
                            const float yg = agpr_read(acc[jj][i][4 * g + t]) * fg4[t];
                            const float yu = agpr_read(acc[jj + TN / 2][i][4 * g + t]) * fu4[t];
                            v[t] = (silu_f32(yg) * yu) * fk4[t];
                        }
                        uint32_t w = 0;
                        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], 1.0f, 0);
                        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
                        *reinterpret_cast<uint16_t*>(cst + r32 * 16 + 4 * g + 2 * hk) = (uint16_t)w;
                    }
                    FP4_LDS_WAIT();
                    const int64_t m = m0 + wm * WM + i * 32 + lane;
                    const int64_t nc = n0 + c0 + jj * 32;
                    if (lane < 32 && m < p.M && nc < p.N) {
                        const uint4 c16 = *reinterpret_cast<const uint4*>(cst + lane * 16);
                        *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(p.y) + m * p.ldy + nc / 2) = c16;
                    }
                    FP4_LDS_WAIT();
                }
            }
            FP4_SYNC_ALL();
        } else {
            const bool full = m0 + BM <= p.M && n0 + BN <= p.N;
            if (p.y_bf16 && full && (p.ldy & 7) == 0 && p.ldy < (1 << 26) &&
                (reinterpret_cast<uintptr_t>(p.y) & 15) == 0) {
                // bf16 whole tile: staged in this wavefront's own LDS area, 32 rows x WN/2
                // columns at a time (16-byte chunks XOR-swizzled by row), written out as whole
                // 16-byte pieces.  The stores are not waited for: the first three waits of the
                // next tile count them.  Addresses: a per-lane 32-bit part plus a
                // wavefront-uniform row offset.
                // The scales are read from LDS once per tile (the rows' activation scales) and
                // once per column half (the columns'), not once per 4-column group: each read
                // is a round trip every wavefront of the CU waits for at the same time.  No
                // wait separates the staging writes, the read-back and the next block's writes:
                // a wavefront's LDS operations are performed in issue order, and the stores
                // wait for the read-back data they take.
                constexpr int CH2 = WN / 16;    // 16-byte chunks per staged row (WN/2 columns)
                constexpr int RPQ = 64 / CH2;   // rows per read-back pass
                const int xw = (r32 & (CH2 - 1)) << 4;
                const int rl = lane / CH2, cl = lane % CH2;
                const uint32_t goff = (uint32_t)(rl * p.ldy * 2 + cl * 16);
                char* const ytile = reinterpret_cast<char*>(p.y) + ((m0 + wm * WM) * p.ldy + n0 + wn * WN) * 2;
                const bool col_scales = p.w_mode == 1, row_scales = p.a_row != 0;
                // this lane's rows' activation scales (one per token, or the tensor's)
                float am[TM];
    #pragma unroll
                for (int i = 0; i < TM; i++) {
                    const float v = asc[wm * WM + i * 32 + r32];
                    am[i] = row_scales ? v : a_scale;
                }
    #pragma unroll
                for (int jh = 0; jh < 2; jh++) {
                    float4 s4[TN / 2][4];  // this lane's columns' weight scales in this half
    #pragma unroll
                    for (int jj = 0; jj < TN / 2; jj++)
    #pragma unroll
                        for (int g = 0; g < 4; g++) {
                            const float4 v = *reinterpret_cast<const float4*>(&sc[wn * WN + (jh * (TN / 2) + jj) * 32 + 8 * g + 4 * hk]);
                            s4[jj][g] = col_scales ? v : make_float4(s_tensor, s_tensor, s_tensor, s_tensor);
                        }
    #pragma unroll
                    for (int i = 0; i < TM; i++) {
    #pragma unroll
                        for (int jj = 0; jj < TN / 2; jj++)
    #pragma unroll
                            for (int g = 0; g < 4; g++) {
                                const int j = jh * (TN / 2) + jj;
                                const float4 s = s4[jj][g];
                                const float f[4] = {am[i] * s.x, am[i] * s.y, am[i] * s.z, am[i] * s.w};
                                __bf16 h4[4];
    #pragma unroll
                                for (int t = 0; t < 4; t++)
                                    h4[t] = GRP ? (__bf16)(tot[GRP ? j : 0][GRP ? i : 0][4 * g + t] * am[i])
                                                : (__bf16)(agpr_read(acc[j][i][4 * g + t]) * f[t]);
                                *reinterpret_cast<uint2*>(stg + r32 * (WN) + (((jj * 4 + g) << 4) ^ xw) + hk * 8) =
                                    __builtin_bit_cast(uint2, h4);
                            }
    #pragma unroll
                        for (int q = 0; q < 32 * CH2 / 64; q++) {
                            const int row = q * RPQ + rl;
                            const uint4 v = *reinterpret_cast<const uint4*>(stg + row * WN + ((cl ^ (row & (CH2 - 1))) << 4));
                            *reinterpret_cast<uint4*>(ytile + (int64_t)(i * 32 + q * RPQ) * p.ldy * 2 + jh * WN + goff) = v;
                        }
                    }
                }
            } else {
                // edge tiles, f32 output, unaligned rows: stores straight from registers,
                // then a full wait (their number does not fit the wait counts above)
    #pragma unroll
                for (int j = 0; j < TN; j++)
    #pragma unroll
                    for (int g = 0; g < 4; g++) {
                        const int nl = wn * WN + j * 32 + 8 * g + 4 * hk;
                        const int64_t n = n0 + nl;
                        float4 s4 = make_float4(s_tensor, s_tensor, s_tensor, s_tensor);
                        if (p.w_mode == 1) {
                            if (full) {
                                s4 = *reinterpret_cast<const float4*>(&sc[nl]);
                            } else {  // scales straight from memory; columns past N are not stored
                                const float* ws = reinterpret_cast<const float*>(p.w_scales);
                                s4.x = ws[n < p.N ? n : p.N - 1];
                                s4.y = ws[n + 1 < p.N ? n + 1 : p.N - 1];
                                s4.z = ws[n + 2 < p.N ? n + 2 : p.N - 1];
                                s4.w = ws[n + 3 < p.N ? n + 3 : p.N - 1];
                            }
                        }
                        const bool vec = full && (p.ldy & 3) == 0 && (reinterpret_cast<uintptr_t>(p.y) & 15) == 0;
    #pragma unroll
                        for (int i = 0; i < TM; i++) {
                            const int64_t m = m0 + wm * WM + i * 32 + r32;
                            const float am = p.a_row ? asc[wm * WM + i * 32 + r32] : a_scale;  // 0 past M
                            const float f0 = am * s4.x, f1 = am * s4.y, f2 = am * s4.z, f3 = am * s4.w;
                            float y0, y1, y2, y3;
                            if constexpr (GRP) {  // y = fl32(T * a_m)
                                y0 = tot[j][i][4 * g] * am, y1 = tot[j][i][4 * g + 1] * am;
                                y2 = tot[j][i][4 * g + 2] * am, y3 = tot[j][i][4 * g + 3] * am;
                            } else {
                                y0 = agpr_read(acc[j][i][4 * g]) * f0, y1 = agpr_read(acc[j][i][4 * g + 1]) * f1;
                                y2 = agpr_read(acc[j][i][4 * g + 2]) * f2, y3 = agpr_read(acc[j][i][4 * g + 3]) * f3;
                            }
                            if (p.y_bf16) {
                                __bf16* yp = reinterpret_cast<__bf16*>(p.y) + m * p.ldy + n;
                                __bf16 h4[4] = {(__bf16)y0, (__bf16)y1, (__bf16)y2, (__bf16)y3};
                                if (vec) {
                                    *reinterpret_cast<uint2*>(yp) = __builtin_bit_cast(uint2, h4);
                                } else if (m < p.M) {
                                    if (n < p.N) yp[0] = h4[0];
                                    if (n + 1 < p.N) yp[1] = h4[1];
                                    if (n + 2 < p.N) yp[2] = h4[2];
                                    if (n + 3 < p.N) yp[3] = h4[3];
                                }
                            } else {
                                float* yp = reinterpret_cast<float*>(p.y) + m * p.ldy + n;
                                if (vec) {
                                    *reinterpret_cast<float4*>(yp) = make_float4(y0, y1, y2, y3);
                                } else if (m < p.M) {
                                    if (n < p.N) yp[0] = y0;
                                    if (n + 1 < p.N) yp[1] = y1;
                                    if (n + 2 < p.N) yp[2] = y2;
                                    if (n + 3 < p.N) yp[3] = y3;
                                }
                            }
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                FP4_SYNC_ALL();
            }
        }
        ct = tile_of(++ck);
        if (ct >= ntiles) break;
        cpar ^= 1;
    }
#undef FP4_DMAK
#undef FP4_DMAS
#undef FP4_NEXT_TILE
#undef FP4_GROUP
#undef FP4_READH
#undef FP4_MMAH
#undef FP4_MMA8
#undef FP4_MMA8_REGS
#undef FP4_PHASE
#undef FP6_READ
#undef FP6_MMA
#undef FP4_FOLD
#undef FP4_DMAG
    // drain the (zero) loads still in flight before the workgroup exits
    FP4_SYNC_ALL();
}

// Buffer offsets are 32-bit and kOOB marks "past the end", so one launch covers at most
// kMaxBufBytes of A and of W; larger operands are split into row blocks (multiples of
// 256 rows, whole tiles either way), each launched on pointers advanced to its start.
constexpr int64_t kMaxBufBytes = 0x7fff0000;
// 256 x 256 E2M1 tiles run 8 wavefronts (measured 6% faster than 4 on the LLaMA-13B
// prefill layer, bit-identical)
constexpr int kBigTileWaves = 8;

// one workgroup per compute unit (each holds the whole LDS ring), looping over tiles
static int cu_count() {
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

// 256 x 256 and 128 x 256 tiles run 8 wavefronts (2 per SIMD), smaller tiles 4.  (FP8
// 256 x 256 tiles: 4 to 10% faster with 8 than with 4 on the LLaMA-13B QKV shape; E2M1
// 128 x 256 tiles at 2048 x 4096 x 4096: 5% faster with 8 than two rounds of 128 x 128,
// 6% slower with 4.  Bit-identical.)
template <int BM, int BN, int F8 = 0>
static void launch_cfg(const GemmParams& p, hipStream_t s, int64_t cus) {
    const int64_t gm = (p.M + BM - 1) / BM, gn = (p.N + BN - 1) / BN, nt = gm * gn;
    constexpr int NWV = BN == 256 ? kBigTileWaves : 4;
    hipLaunchKernelGGL((w4a4_fp4_kernel<BM, BN, false, F8, NWV>), dim3((unsigned)std::min(nt, cus)), dim3(64 * NWV), 0,
                       s, p, (int)gm, (int)nt, GluParams{});
}
static GemmParams column_block(const GemmParams& p, int64_t n0, int64_t n1) {
    GemmParams q = p;
    q.N = n1 - n0;
    q.w = p.w + n0 * p.ldw;
    if (p.w_mode == 1) q.w_scales = reinterpret_cast<const float*>(p.w_scales) + n0;
    q.y = reinterpret_cast<uint8_t*>(p.y) + n0 * (p.y_bf16 ? 2 : 4);
    return q;
}

// Tile shapes and the last round.  Time of one round of tiles (every compute unit
// busy), relative to 256x256 tiles on the same K, measured on the prefill shapes:
// 256x128 0.59, 128x128 0.35.  With at least one full round of 256x256 tiles, the
// whole rounds stay 256x256 and the column block left over for a partial last round
// takes the shape that finishes it soonest (a partial round of big tiles leaves
// compute units idle).  Fewer 256x256 tiles than compute units: 128x256 when they give
// every compute unit a tile (FP8 at 2048x4096x4096: 44.6 -> 43.0 us), else 128x128.
template <int F8 = 0>
static hipError_t launch_block(const GemmParams& p, hipStream_t s) {
    const int64_t cus = cu_count();
    const int64_t gm256 = (p.M + 255) / 256, gn256 = (p.N + 255) / 256, t256 = gm256 * gn256;
    if (t256 < cus) {
        // (one round of 256 x 128 tiles on 4 wavefronts measured the same as two of 128 x 128
        // at 2048 x 4096)
        if (((p.M + 127) / 128) * gn256 >= cus) launch_cfg<128, 256, F8>(p, s, cus);
        else launch_cfg<128, 128, F8>(p, s, cus);
        return hipGetLastError();
    }
    const int64_t full_cols = (t256 / cus) * cus / gm256;  // 256-column blocks of whole rounds
    const int64_t n1 = std::min<int64_t>(p.N, full_cols * 256);
    if (n1 >= p.N || t256 % cus == 0) {
        launch_cfg<256, 256, F8>(p, s, cus);
        return hipGetLastError();
    }
    const int64_t rest = p.N - n1;
    auto rounds = [&](int64_t bm, int64_t bn) {
        const int64_t t = ((p.M + bm - 1) / bm) * ((rest + bn - 1) / bn);
        return (double)((t + cus - 1) / cus);
    };
    // cost of the leftover block in 256x256-round units; 256x256 over the whole output
    // costs one more round than the full ones
    const double c256 = rounds(256, 256), c256x128 = 0.59 * rounds(256, 128), c128 = 0.35 * rounds(128, 128);
    if (c256 <= c256x128 && c256 <= c128) {
        launch_cfg<256, 256, F8>(p, s, cus);
        return hipGetLastError();
    }
    launch_cfg<256, 256, F8>(column_block(p, 0, n1), s, cus);
    const GemmParams q = column_block(p, n1, p.N);
    if (c256x128 <= c128) launch_cfg<256, 128, F8>(q, s, cus);
    else launch_cfg<128, 128, F8>(q, s, cus);
    return hipGetLastError();
}

// Byte limit of one launch's A and W ranges (the 32-bit buffer range by default); a
// smaller limit only splits a product into more row blocks, with the same result.
static std::atomic<int64_t> g_split_limit{kMaxBufBytes};

void set_split_limit(int64_t bytes) { g_split_limit.store(bytes > 0 && bytes < kMaxBufBytes ? bytes : kMaxBufBytes); }

template <int F8>
static hipError_t launch_split(const GemmParams& p, hipStream_t s) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    const int64_t lim = g_split_limit.load();
    const int64_t mstep = std::max<int64_t>(256, lim / std::max<int64_t>(p.lda, 1) / 256 * 256);
    const int64_t nstep = std::max<int64_t>(256, lim / std::max<int64_t>(p.ldw, 1) / 256 * 256);
    const size_t ysz = p.y_bf16 ? 2 : 4;
    for (int64_t m0 = 0; m0 < p.M; m0 += mstep) {
        for (int64_t n0 = 0; n0 < p.N; n0 += nstep) {
            GemmParams q = p;
            q.M = std::min(mstep, p.M - m0);
            q.N = std::min(nstep, p.N - n0);
            q.a = reinterpret_cast<const uint8_t*>(p.a) + m0 * p.lda;
            if (p.a_row) q.a_scale = p.a_scale + m0;  // per-token scales of this row block
            q.w = p.w + n0 * p.ldw;
            if (p.w_mode == 1) q.w_scales = reinterpret_cast<const float*>(p.w_scales) + n0;
            q.y = reinterpret_cast<uint8_t*>(p.y) + (m0 * p.ldy + n0) * ysz;
            hipError_t e = launch_block<F8>(q, s);
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

hipError_t launch_w4a4_fp4(const GemmParams& p, hipStream_t s) { return launch_split<0>(p, s); }

// FP8 E4M3 x E4M3 (W8A8): the same kernel, one code per byte
hipError_t launch_w8a8_fp8(const GemmParams& p, hipStream_t s) { return launch_split<1>(p, s); }

// FP8 E5M2 x E5M2 and the mixed FP8 pairs: the same kernel with the MFMA's format codes
hipError_t launch_w8a8_e5m2(const GemmParams& p, hipStream_t s) { return launch_split<4>(p, s); }
hipError_t launch_w8a8_mixed(const GemmParams& p, hipStream_t s) {
    return p.wg.e == 4 ? launch_split<5>(p, s) : launch_split<6>(p, s);
}

// FP6 x FP6 of one format (W6A6), tensor or row weight scales: 128x128 tiles on 4
// wavefronts (a 96-byte step row; larger tiles leave no room in LDS for four stages), one
// launch.
bool w6a6_fits(const GemmParams& p) {
    return p.w_mode != 2 && p.K % 128 == 0 && p.lda % 4 == 0 && p.ldw % 4 == 0 && p.M * p.lda < kMaxBufBytes &&
           p.N * p.ldw < kMaxBufBytes;
}
hipError_t launch_w6a6_fp6(const GemmParams& p, hipStream_t s) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    const int64_t cus = cu_count();
    const int64_t gm = (p.M + 127) / 128, gn = (p.N + 127) / 128, nt = gm * gn;
    const dim3 grid((unsigned)std::min(nt, cus));
    if (p.wg.e == 3) hipLaunchKernelGGL((w4a4_fp4_kernel<128, 128, false, 9, 4>), grid, dim3(256), 0, s, p, (int)gm, (int)nt, GluParams{});
    else hipLaunchKernelGGL((w4a4_fp4_kernel<128, 128, false, 8, 4>), grid, dim3(256), 0, s, p, (int)gm, (int)nt, GluParams{});
    return hipGetLastError();
}

// FP8 E4M3 x E4M3 with f32 or f16 weight scales per row and group of 64 or 128 codes, or
// f32 scales per 256: the same kernel on 128x256 tiles (8 wavefronts; the running sums
// take the registers that 256x256 tiles would need for accumulators), one launch.
bool w8a8_group_fits(const GemmParams& p) {
    if (p.w_mode != 2 || (p.w_group != 64 && p.w_group != 128 && p.w_group != 256) || p.K % p.w_group != 0) return false;
    const int esz = p.w_scale_f16 ? 2 : 4;
    const int64_t grow = p.K / p.w_group * esz;  // scale bytes per output row
    // the scale loads of successive four-step groups start 256 / G scales apart: whole
    // 4-byte words (so not f16 scales with groups of 256), as are the rows
    return grow % 4 == 0 && 256 / p.w_group * esz % 4 == 0 && p.M * p.lda < kMaxBufBytes && p.N * p.ldw < kMaxBufBytes &&
           p.N * grow < kMaxBufBytes;
}
hipError_t launch_w8a8_fp8_group(const GemmParams& p, hipStream_t s) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    const int64_t cus = cu_count();
    const int64_t gm = (p.M + 127) / 128, gn = (p.N + 255) / 256, nt = gm * gn;
    const dim3 grid((unsigned)std::min(nt, cus)), block(64 * kBigTileWaves);
    const bool h = p.w_scale_f16 != 0;
    if (p.w_group == 64) {
        if (h) hipLaunchKernelGGL((w4a4_fp4_kernel<128, 256, false, 13, kBigTileWaves>), grid, block, 0, s, p, (int)gm, (int)nt, GluParams{});
        else hipLaunchKernelGGL((w4a4_fp4_kernel<128, 256, false, 12, kBigTileWaves>), grid, block, 0, s, p, (int)gm, (int)nt, GluParams{});
    } else if (p.w_group == 256) {  // f32 scales only (w8a8_group_fits)
        hipLaunchKernelGGL((w4a4_fp4_kernel<128, 256, false, 14, kBigTileWaves>), grid, block, 0, s, p, (int)gm, (int)nt, GluParams{});
    } else {
        if (h) hipLaunchKernelGGL((w4a4_fp4_kernel<128, 256, false, 3, kBigTileWaves>), grid, block, 0, s, p, (int)gm, (int)nt, GluParams{});
        else hipLaunchKernelGGL((w4a4_fp4_kernel<128, 256, false, 2, kBigTileWaves>), grid, block, 0, s, p, (int)gm, (int)nt, GluParams{});
    }
    return hipGetLastError();
}

// SwiGLU + next-layer quantization: tiles of BM rows x BN/2 output columns (gate and up
// rows of those columns), 256 x 128 when they give every compute unit a tile, else
// 128 x 64; operands past the 32-bit buffer range are split into row blocks.
template <int BM, int BN>
static void launch_glu_cfg(const GemmParams& p, const GluParams& gp, hipStream_t s, int64_t cus) {
    const int64_t gm = (p.M + BM - 1) / BM, gn = (p.N + BN / 2 - 1) / (BN / 2), nt = gm * gn;
    constexpr int NWV = (BM == 256 && BN == 256) ? kBigTileWaves : 4;
    hipLaunchKernelGGL((w4a4_fp4_kernel<BM, BN, true, 0, NWV>), dim3((unsigned)std::min(nt, cus)), dim3(64 * NWV), 0,
                       s, p, (int)gm, (int)nt, gp);
}

hipError_t launch_w4a4_swiglu(const GemmParams& p, const GluParams& gp, hipStream_t s) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    const int64_t cus = cu_count();
    const int64_t lim = g_split_limit.load();
    const int64_t mstep = std::max<int64_t>(256, lim / std::max<int64_t>(p.lda, 1) / 256 * 256);
    const int64_t nstep = std::max<int64_t>(128, lim / std::max<int64_t>(p.ldw, 1) / 128 * 128);
    for (int64_t m0 = 0; m0 < p.M; m0 += mstep) {
        for (int64_t n0 = 0; n0 < p.N; n0 += nstep) {
            GemmParams q = p;
            q.M = std::min(mstep, p.M - m0);
            q.N = std::min(nstep, p.N - n0);
            q.a = reinterpret_cast<const uint8_t*>(p.a) + m0 * p.lda;
            q.w = p.w + n0 * p.ldw;
            q.w_scales = reinterpret_cast<const float*>(p.w_scales) + n0;
            q.y = reinterpret_cast<uint8_t*>(p.y) + m0 * p.ldy + n0 / 2;
            GluParams g = gp;
            g.w_up = gp.w_up + n0 * p.ldw;
            g.s_up = gp.s_up + n0;
            if (gp.out_shift) g.out_shift = gp.out_shift + n0;
            if (((q.M + 255) / 256) * ((q.N + 127) / 128) >= cus) launch_glu_cfg<256, 256>(q, g, s, cus);
            else launch_glu_cfg<128, 128>(q, g, s, cus);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace fp4

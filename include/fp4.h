/*
 * fp4.h -- C ABI of libfp4: low-bit floating-point quantization of LLM weights and
 * activations and the quantized matrix products that consume them, as hand-written
 * HIP kernels for AMD MI355X (gfx950).
 *
 * Method sources (web pages, cited by title and section):
 *   [FP4-LLM]  "首个支持4-bit浮点量化的LLM来了，解决LLaMA、BERT等的部署难题" (811yy.cn), a
 *              summary of the LLM-FP4 paper: FP value formula (sign, exponent field p,
 *              mantissa bits, bias b); "scale and clip", eqs. (2)-(3); bias from the
 *              range, eq. (4); "compare and quantize", eq. (5); scales kept outside the
 *              low-bit product ("efficient matrix multiplication"); search over the
 *              exponent/mantissa split and range; pre-shifted exponent bias.
 *   [Overview] "量化技术详解" (aidocs.cortexgrid.cn): granularities (per tensor / channel /
 *              token), static quantization, NF4.
 *   [W8A8]     intelliparadigm.com LLM-quantization practice, section 2.2: calibrate by
 *              max |x|; quantized matmul = low-bit product times the product of scales;
 *              group size 128.
 *   [Tutorial] "为什么我们需要4-bit浮点量化" (devpress.csdn.net), section 2.2: two 4-bit
 *              values per byte, on-the-fly 4->8-bit decode for the matmul.
 *   [HiFloat4] "HiFloat4格式" (cf-1.com), section 3.2: 128-bit loads of 32 packed values;
 *              section 5 (LLaMA-13B case): activation quantization fused with the
 *              activation function.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless the comment says "host".  The caller owns
 *     all memory; the library allocates nothing and keeps no pointer after returning.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream) and never synchronises.  Results are valid once the stream reaches them.
 *   - Matrices are row-major with a leading dimension (ld, in ELEMENTS for f32/bf16/
 *     f16 and in BYTES for packed 4-bit data).  Linear-layer shapes: W is [N, K]
 *     (out x in, K contiguous), X is [M, K], Y = X * W^T is [M, N].
 *   - Packed 4-bit data: byte j of a row holds element 2j in its low nibble and
 *     element 2j+1 in its high nibble.  Minifloat code = sign<<3 | p<<m | d; lookup-
 *     grid code = index into the 16 sorted grid values.
 *   - Alignment: every pointer 16-byte aligned; see each call for stride rules.
 *   - Inputs must be finite (no inf/NaN); results for non-finite inputs are unspecified.
 *   - Return value: FP4_OK, or an error detected on the host BEFORE anything is
 *     launched (INVALID_ARG, UNSUPPORTED, ALIGNMENT, WORKSPACE), or FP4_ERR_HIP when
 *     a launch failed.  fp4_last_error() gives a message for the calling thread.
 *   - Calls are thread-safe; calls that share output buffers must be ordered by the
 *     caller.
 */
#ifndef FP4_H_
#define FP4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t fp4_status;
#define FP4_OK               0
#define FP4_ERR_INVALID_ARG  1  /* null pointer, bad size, stride or enum value      */
#define FP4_ERR_UNSUPPORTED  2  /* valid request this library does not implement     */
#define FP4_ERR_ALIGNMENT    3  /* pointer or stride breaks the alignment rule       */
#define FP4_ERR_WORKSPACE    4  /* workspace missing or smaller than required        */
#define FP4_ERR_HIP          5  /* a HIP launch failed (message in fp4_last_error)   */

/* element types */
#define FP4_F32     0
#define FP4_BF16    1
#define FP4_F16     2
#define FP4_PACKED  3   /* two 4-bit codes per byte */

/* ---- number grids -------------------------------------------------------------
 * FP4_GRID_MINIFLOAT: FP(e, m) with e + m == 3 and the canonical bias 1 ([FP4-LLM]
 *   FP value formula): magnitude of code p<<m | d is 2^(1-1) * d / 2^m for p == 0
 *   (subnormal) and 2^(p-1) * (1 + d / 2^m) for p >= 1; no code is reserved for
 *   inf/NaN.  E2M1 = {0, .5, 1, 1.5, 2, 3, 4, 6}, E1M2 = {0, .25, ..., 1.75},
 *   E3M0 = {0, 1, 2, 4, ..., 64}.  A real-valued bias b is the same grid times
 *   2^(1-b) ([FP4-LLM] eq. (4)), i.e. it lives entirely in the scale.
 *   With e + m == 7 the grid is an OCP FP8 format ([FP4-LLM] FP8 for key layers):
 *   (4, 3) E4M3 (bias 7, S.1111.111 is NaN, largest 448) or (5, 2) E5M2 (bias 15,
 *   exponent 31 is inf/NaN, largest 57344); one code per byte (sign in bit 7), so
 *   code arrays hold `cols` bytes per row.  With e + m == 5 it is an OCP FP6 format
 *   ([FP4-LLM] progressive 8/6/4 bits): (2, 3) E2M3 (bias 1, largest 7.5) or (3, 2)
 *   E3M2 (bias 3, largest 28), no reserved code; codes form a little-endian bit
 *   stream, code i in bits [6i, 6i+6) of its row (3 cols / 4 bytes; cols a multiple
 *   of 4).  FP8/FP6 take TENSOR, ROW or GROUP scales in quantize/dequantize (cols a
 *   multiple of 8; column shifts allowed) and the W4A16 product (W8A16 / W6A16); codes are the nearest
 *   finite value with ties to the even code, saturating at the largest.
 * FP4_GRID_LUT16: 16 sorted signed values in lut[] (e.g. NF4, [Overview] NF4), each
 *   exactly representable in binary16.
 * FP4_GRID_TWO_MODE: per scale group either E2M1 (mode 0) or E1M2 (mode 1)
 *   ([HiFloat4] section 2.1: a small-value and a large-value bit layout, marked by one
 *   control bit shared by a batch of values).  Only with GROUP granularity.  The
 *   quantizer computes both candidates for each group -- s_m = fl32(amax / Qmax_m)
 *   (Qmax 6 and 1.75; rounded to binary16 for f16 scales), the codes of
 *   y = fl32(x * fl32(1/s_m)) -- and keeps the one whose squared error
 *   sum (|x| - fl32(g(code) * s_m))^2 is smaller (equal: E2M1).  The mode is the sign
 *   bit of the stored group scale (scales are otherwise non-negative): a negative
 *   stored scale -s means E1M2 with scale s.  The comparison sums the per-element
 *   differences of the exact squares in binary64 and double-double: it equals the exact
 *   comparison unless the two errors agree to about 2^-49 of their size without being
 *   equal.  e, m and lut[] are ignored.                                               */
#define FP4_GRID_MINIFLOAT 0
#define FP4_GRID_LUT16     1
#define FP4_GRID_TWO_MODE  2
typedef struct {
    int32_t kind;     /* FP4_GRID_MINIFLOAT, FP4_GRID_LUT16 or FP4_GRID_TWO_MODE */
    int32_t e;        /* minifloat exponent bits (1, 2 or 3)                 */
    int32_t m;        /* minifloat mantissa bits (e + m == 3)                */
    int32_t reserved; /* must be 0                                           */
    float   lut[16];  /* LUT16 values, strictly increasing; ignored otherwise */
} fp4_grid;

/* ---- scale granularity ([Overview] granularities; [W8A8] group size 128) -------
 * TENSOR: one scale; ROW: one scale per row (output channel of a weight, token of an
 * activation); GROUP: one scale per `group` consecutive elements of a row.          */
#define FP4_SCALE_TENSOR 0
#define FP4_SCALE_ROW    1
#define FP4_SCALE_GROUP  2
typedef struct {
    int32_t mode;         /* FP4_SCALE_TENSOR | _ROW | _GROUP                    */
    int32_t group;        /* GROUP: 8, 16, 32, 64, 128, 256 or 512; else 0       */
    int32_t scale_dtype;  /* FP4_F32, or FP4_F16 (ROW and GROUP only)            */
    int32_t reserved;     /* must be 0                                           */
} fp4_gran;

/* ---- calibration reductions ---------------------------------------------------- */
#define FP4_REDUCE_TENSOR    0   /* amax_out[0]                                      */
#define FP4_REDUCE_COLUMN    1   /* amax_out[cols]   (per input channel)             */
#define FP4_REDUCE_ROW_GROUP 2   /* amax_out[rows * cols/group]                      */

/* ---- search record ([FP4-LLM] search over exponent/mantissa split and range) ---- */
typedef struct {
    int32_t e, m;           /* winning format                                       */
    int32_t clip_index;     /* j in [0, nclips): clip = amax * ratio_j               */
    int32_t format_index;   /* index into the caller's format list                  */
    float   clip;           /* fl32(amax * ratio_j)                                 */
    float   scale;          /* s = fl32(clip / Qmax(e, m)), the stored scale         */
    float   amax;           /* max |w| of the tensor                                */
    float   reserved;
    double  bias;           /* real exponent bias equivalent to s: 1 - log2(s)      */
    double  mse;            /* mean of (w - dequant(quant(w)))^2, correctly rounded */
    double  mse_runner_up;  /* smallest MSE among the other candidates              */
} fp4_search_result;

/* ---- quantized GEMM descriptor ------------------------------------------------- */
typedef struct {
    int64_t M, N, K;
    /* activations X [M, K] */
    int32_t a_kind;           /* FP4_F32, FP4_BF16 (W4A16) or FP4_PACKED (W4A4)      */
    int32_t a_scale_mode;     /* PACKED: FP4_SCALE_TENSOR (one a) or FP4_SCALE_ROW    */
    const void* a;            /* device                                             */
    int64_t lda;              /* elements (F32/BF16) or bytes (PACKED)              */
    fp4_grid a_grid;          /* PACKED only: grid of the activation codes          */
    const float* a_scale;     /* PACKED only: device f32, the one scale a, or with
                                 a_scale_mode ROW one scale a_m per row (token) of X
                                 ([Overview] per-token granularity; the products
                                 of two minifloat grids)                            */
    /* weights W [N, K], packed */
    const uint8_t* w;
    int64_t ldw;              /* bytes                                              */
    fp4_grid w_grid;
    fp4_gran w_gran;          /* TENSOR, ROW or GROUP along K                        */
    const void* w_scales;     /* f32 or f16 per w_gran                              */
    /* output Y [M, N] */
    void* y;
    int64_t ldy;              /* elements                                           */
    int32_t y_dtype;          /* FP4_BF16 or FP4_F32                                */
    int32_t reserved1;
} fp4_gemm_desc;

/* Human-readable name of a status code (static storage). */
const char* fp4_status_string(fp4_status s);

/* Message describing the last error returned on the calling thread ("" if none). */
const char* fp4_last_error(void);

/* Calibrate: amax = max |x| ([W8A8] section 2.2 calibrate; [FP4-LLM] pre-shift uses
 * per-channel maxima from a small calibration set; [Overview] static quantization).
 *   x          device, x_dtype FP4_F32 or FP4_BF16, [rows, cols] with leading dim ld
 *   reduce     FP4_REDUCE_TENSOR | _COLUMN | _ROW_GROUP
 *   group      ROW_GROUP: group size (divides cols, one of 8..512 as in fp4_gran)
 *   first_rows only rows [0, first_rows) are reduced (the calibration tokens); <= 0
 *              means all rows
 *   amax_out   device f32: 1, cols, or rows*(cols/group) values
 * The result is exact (max is order-free) and identical for any launch geometry. */
fp4_status fp4_calibrate(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                         int64_t ld, int32_t reduce, int32_t group, int64_t first_rows,
                         float* amax_out, void* stream);

/* Quantize and pack ([FP4-LLM] eqs. (2)-(5): scale and clip, compare and quantize;
 * [Tutorial] section 2.2: two codes per byte).
 *   For every scale unit u (tensor, row or group): s_u = fl32(amax_u / Qmax) (Qmax =
 *   largest grid magnitude; for ROW/GROUP with FP4_F16 scales s_u is rounded to
 *   binary16 and the rounded value is used), r_u = fl32(1 / s_u) (0 if s_u == 0).
 *   Element x: y = fl32(x * r) with r = r_u, or r_u * 2^-k[col] when col_shift is
 *   given (pre-shifted exponent bias, activation side); code = nearest grid point to
 *   y after clipping to +-Qmax, exact ties to the even code; minifloat codes carry
 *   signbit(x).
 *   x            device, FP4_F32 or FP4_BF16, [rows, cols], leading dim ldx elements
 *   cols         even; GROUP: multiple of group
 *   grid, gran   see above (gran.scale_dtype FP4_F16 only for ROW/GROUP)
 *   amax_in      device f32 per scale unit from fp4_calibrate, or NULL = computed here
 *   tensor_scale TENSOR only: device pointer to a fixed f32 scale s (static
 *                activation quantization, e.g. the per-tensor scale a from
 *                fp4_preshift_weights), or NULL
 *   col_shift    device int8 k[cols] (values in [-64, 0]), or NULL
 *   packed       device u8 [rows, cols/2], leading dim ldp bytes
 *   scales_out   device, f32 or f16 per scale unit (1, rows, or rows*cols/group);
 *                may be NULL only when tensor_scale is given                         */
fp4_status fp4_quantize_pack(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                             int64_t ldx, fp4_grid grid, fp4_gran gran,
                             const float* amax_in, const float* tensor_scale,
                             const int8_t* col_shift, uint8_t* packed, int64_t ldp,
                             void* scales_out, void* stream);

/* Dequantize (inverse of the codec, [Tutorial] section 2.2 decode):
 *   out = +-fl32(g(code) * s_u), times 2^k[col] when col_shift is given (exact).
 *   packed [rows, cols/2] (ldp bytes), scales per gran, out f32 [rows, cols] (ldo). */
fp4_status fp4_dequantize(const uint8_t* packed, int64_t rows, int64_t cols, int64_t ldp,
                          fp4_grid grid, fp4_gran gran, const void* scales,
                          const int8_t* col_shift, float* out, int64_t ldo, void* stream);

/* Pre-shifted exponent bias ([FP4-LLM], pre-shifted exponent bias): from per-channel
 * activation maxima c[k] (fp4_calibrate COLUMN over the calibration tokens):
 *   c_max = max_k c[k];  a = fl32(c_max / Qmax(act_grid))           -> act_scale_out
 *   shift k_k = smallest integer j with c_max * 2^j >= c[k] (0 if c[k] == 0, clamped
 *   at -64; always <= 0), computed exactly from the binary exponents  -> shift_out
 *   W'[n, k] = W[n, k] * 2^k_k (exact), then W' is quantized with w_grid / w_gran
 *   (scales from the amax of W') -> w_packed, w_scales.
 * Activations are then quantized with fp4_quantize_pack(gran TENSOR, tensor_scale =
 * act_scale_out, col_shift = shift_out), and X * W^T = (X 2^-k) * (W 2^k)^T exactly.
 * act_grid and w_grid are any minifloat / LUT16 grids or the FP8 / FP6 grids (not the
 * two-mode grid); FP8 / FP6 weights need k a multiple of 8 (FP6: ldp even).
 *   w            device f32 [n, k], leading dim ldw elements
 *   chan_amax    device f32 [k]
 *   w_packed     device u8 [n, k * bits / 8], leading dim ldp bytes                 */
fp4_status fp4_preshift_weights(const float* w, int64_t n, int64_t k, int64_t ldw,
                                const float* chan_amax, fp4_grid act_grid,
                                fp4_grid w_grid, fp4_gran w_gran, int8_t* shift_out,
                                float* act_scale_out, uint8_t* w_packed, int64_t ldp,
                                void* w_scales, void* stream);

/* Workspace bytes that fp4_search_format needs for these sizes. */
size_t fp4_search_workspace_size(int64_t ntensors, int64_t numel, int32_t nformats,
                                 int32_t nclips);

/* Format and clip-range search ([FP4-LLM] search-based FP quantization): for each of
 * ntensors contiguous tensors of numel f32 values, evaluate every format in
 * formats_em (host, nformats pairs (e, m), minifloat with e + m == 3) times nclips
 * clip values c_j = fl32(amax * ratio_j), ratio_j = fl32(lo + (hi - lo) * j /
 * (nclips - 1)) evaluated in binary64; candidate error = mean over the tensor of
 * (w - dequant(quant(w)))^2 with s = fl32(c_j / Qmax), accumulated so that the
 * result is the correctly rounded mean (independent of summation order).  The
 * winner is the smallest MSE; exact ties go to the earliest candidate (formats
 * outer, clips inner).  Each tensor is then packed with its winner (TENSOR scale s).
 *   w        device f32 [ntensors, numel] (numel even)
 *   results  device fp4_search_result [ntensors]
 *   packed   device u8 [ntensors, numel/2]
 *   workspace, ws_bytes  device scratch of at least fp4_search_workspace_size()    */
fp4_status fp4_search_format(const float* w, int64_t ntensors, int64_t numel,
                             const int32_t* formats_em, int32_t nformats, int32_t nclips,
                             float clip_lo, float clip_hi, fp4_search_result* results,
                             uint8_t* packed, void* workspace, size_t ws_bytes,
                             void* stream);

/* fp4_search_format without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments, results and errors
 * as fp4_search_format; the cross-workgroup partial sums live instead in a scratch array
 * of 16 MiB that the library holds on each GPU it runs on until the process ends (one
 * copy per GPU, located on the first call on that GPU).  Sizes whose
 * fp4_search_workspace_size() exceeds 16 MiB return FP4_ERR_WORKSPACE before anything
 * is launched (32 tensors of 4096 x 4096 with 3 formats x 100 clips need about 9.8 MB).
 * Every call on one GPU shares that GPU's scratch and leaves its contents behind (each
 * call clears what it needs zeroed): calls that may overlap on one GPU -- on different
 * streams, or from several threads -- race and must be ordered by the caller. */
fp4_status fp4_search_format_static(const float* w, int64_t ntensors, int64_t numel,
                                    const int32_t* formats_em, int32_t nformats, int32_t nclips,
                                    float clip_lo, float clip_hi, fp4_search_result* results,
                                    uint8_t* packed, void* stream);

/* The same search on activations ([FP4-LLM] search-based FP quantization applied to
 * activations as to weights; [Overview] static quantization from calibration data and
 * per-token granularity):
 *   x          device, x_dtype FP4_F32 or FP4_BF16 (bf16 values are searched exactly as
 *              their binary32 values), [rows, cols], leading dim ldx elements (>= cols,
 *              a multiple of 4); cols a multiple of 16
 *   unit       FP4_SCALE_TENSOR: rows [0, T) form one search unit, T = first_rows (all
 *              rows if first_rows <= 0 or >= rows): the calibration tokens choose one
 *              format and clip for the activation tensor, and EVERY row (those past T
 *              included) is packed with it -- static activation quantization;
 *              FP4_SCALE_ROW: every row (token) is its own unit, searched and packed with
 *              its own winner -- per-token formats and scales.
 *   formats_em, nformats, nclips, clip_lo, clip_hi: as fp4_search_format; each unit's
 *              candidates, error, winner and record are defined as there, with the unit's
 *              values in place of a tensor's.
 *   results    device fp4_search_result [1] (TENSOR) or [rows] (ROW)
 *   packed     device u8 [rows, cols/2], leading dim ldp bytes (>= cols/2, a multiple of 4)
 *   workspace  at least fp4_search_workspace_size(1, T * cols, ...) (TENSOR) or
 *              fp4_search_workspace_size(rows, cols, ...) (ROW) bytes                 */
fp4_status fp4_search_activations(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                                  int32_t unit, int64_t first_rows, const int32_t* formats_em,
                                  int32_t nformats, int32_t nclips, float clip_lo, float clip_hi,
                                  fp4_search_result* results, uint8_t* packed, int64_t ldp,
                                  void* workspace, size_t ws_bytes, void* stream);

/* Quantized GEMM Y = X * W^T with scales factored out of the low-bit inner product
 * ([FP4-LLM] efficient matrix multiplication; [W8A8] section 2.2 quantized_matmul):
 *   W4A16 (a_kind F32/BF16):  Y[m,n] = sum_u s[n,u] * sum_{k in u} x[m,k] * g(c[n,k])
 *                              (u = the scale units of w_gran along K), fp32 accumulate.
 *   W4A4  (a_kind PACKED):    Y[m,n] = a * sum_u s[n,u] * sum_{k in u} A_q[m,k] W_q[n,k]
 *     - E2M1 x E2M1 with TENSOR/ROW weight scales runs on the FP4 matrix cores; the
 *       code product is exact in fp32 and the epilogue is y = fl32(acc * fl32(a * s_n))
 *       (per-token activation scales: y = fl32(acc * fl32(a_m * s_n)));
 *       K <= 116508 (the quarter-integer partial sums stay below 2^22), else
 *       FP4_ERR_UNSUPPORTED.
 *     - E1M2 or E3M0 on either side, the other operand a 4-bit minifloat grid, runs on
 *       the f8f6f4 matrix cores with each E1M2 / E3M0 code rewritten as the E4M3 byte
 *       of the same value on its way into LDS (every E1M2 and E3M0 value is an E4M3
 *       value).  Products of two 4-bit grids, or of a 4-bit grid and E2M3, are
 *       multiples of 2^-5 that the instruction keeps whole, so acc is exact while
 *       |acc| stays below 2^19; y = fl32(acc * fl32(a * s_n)) (per token: a_m) as
 *       above, with f32 TENSOR/ROW weight scales and K a multiple of 32.
 *     - E2M1 activations x LUT16 weights (NF4) with GROUP scales (group a multiple of
 *       64) runs on the f16 matrix cores: each weight is expanded to
 *       w = fl16(G[c] * fl16(s[n,g] * 2^-e_n)), 2^e_n the power of two just above the
 *       largest group scale of row n, the f16 products are summed in fp32 and the
 *       result is y = fl32(acc * fl32(a * 2^e_n)).  Within about 1e-3 (relative, in
 *       norm) of the exact value; groups whose scale is below 2^-14 of their row's
 *       largest lose relative precision to f16 subnormals.
 *   y_dtype FP4_BF16 rounds the f32 result to nearest-even.
 *   4-bit minifloat weights (E2M1, E1M2, E3M0) with BF16 activations run on the bf16
 *   matrix cores (each code decoded exactly to bf16) when K is a multiple of 128, lda a
 *   multiple of 8 and GROUP scales have a group that is a multiple of 128; other W4A16
 *   shapes, and F32 activations, on a VALU kernel.
 *   FP8 / FP6 weights with F32/BF16 activations take the W4A16 path (W8A16 / W6A16):
 *   ldw >= K (FP8) or 3K/4 (FP6) bytes.  With PACKED activations both operands are FP8
 *   (E4M3, E5M2) or FP6 (E2M3, E3M2), in any pairing (W8A8, W6A6, mixed), on the
 *   f8f6f4 matrix cores with f32 TENSOR/ROW weight scales and one activation scale
 *   (or one per row of A with a_scale_mode ROW, y = fl32(acc * fl32(a_m * s_n))):
 *   y = fl32(acc * fl32(a * s_n)), acc summed in fp32 (not exact: within the GEMM
 *   tolerance); lda, ldw >= the code bytes of a row (K or 3K/4), lda a multiple of 16,
 *   K a multiple of 32, rows shorter than 8 MiB.  The same holds when one operand is a
 *   4-bit minifloat grid (E2M1, E1M2, E3M0) and the other FP8 / FP6 (rows of K/2 bytes).
 *   FP8 / FP6 weights with PACKED activations also take GROUP weight scales (f32 or
 *   f16, group G a multiple of 64 dividing K; [W8A8] section 2.2's group of 128):
 *   y = fl32(T * a) (per token: a_m), T = sum over the groups g in K order of
 *   T = fma(P_g, s[n, g], T), P_g the group's fp32 sum; within the GEMM tolerance.  A
 *   group that is not a multiple of 64 (one matrix instruction spans 64 codes of K)
 *   returns FP4_ERR_UNSUPPORTED.
 *   Two-mode weights (FP4_GRID_TWO_MODE, GROUP scales) take the W4A16 path only: each
 *   group's codes are read on its own grid (the sign of its scale) and scaled by |s|.
 * Strides: K a multiple of 32 for the matrix-core paths; packed rows 16-byte aligned. */
fp4_status fp4_gemm(const fp4_gemm_desc* d, void* stream);

/* ---- fused SwiGLU + next-layer activation quantization ---------------------------- */
typedef struct {
    int64_t M, N, K;          /* X [M, K]; W_gate, W_up [N, K]; h [M, N]            */
    const uint8_t* a;         /* packed E2M1 activations [M, K/2], leading dim lda   */
    int64_t lda;              /* bytes, multiple of 16                              */
    const float* a_scale;     /* device: the one f32 activation scale a             */
    const uint8_t* w_gate;    /* packed E2M1 [N, K/2], leading dim ldw              */
    const uint8_t* w_up;      /* packed E2M1 [N, K/2], leading dim ldw              */
    int64_t ldw;              /* bytes, multiple of 16                              */
    const float* s_gate;      /* f32 [N] row scales of W_gate                       */
    const float* s_up;        /* f32 [N] row scales of W_up                         */
    const float* out_scale;   /* device: the consumer's f32 activation scale a'     */
    const int8_t* out_shift;  /* int8 [N]: the consumer's column shifts k', or NULL */
    uint8_t* h_packed;        /* E2M1 codes of h [M, N/2], leading dim ldh          */
    int64_t ldh;              /* bytes, multiple of 16, >= N/2                       */
} fp4_swiglu_desc;

/* The LLaMA MLP's gate and up products of the same E2M1 activations with the SwiGLU
 * activation and the down projection's activation quantization in the epilogue, so that
 * h never exists in high precision in memory ([HiFloat4] section 5: quantization fused
 * with the activation function; [FP4-LLM] pre-shifted exponent bias on the consumer):
 *   y_g = fl32(acc_g[m,n] * fl32(a * s_gate[n])),  y_u likewise with W_up, s_up
 *     (acc = the exact code product, as in fp4_gemm's E2M1 x E2M1 path)
 *   h   = fl32(SiLU(y_g) * y_u),  SiLU(x) = fl32(x / fl32(1 + exp32(-x))), where
 *     exp32 is a fixed binary32 operation sequence: t = fl(x * log2 e), n = rint(t),
 *     f = t - n, 2^f by its degree-7 Taylor polynomial in Horner form (coefficients
 *     (ln 2)^i / i! rounded to binary32, a separate multiply and add per term), times
 *     2^n (n clamped to [-300, 300]); relative error below 1e-5 for |x| <= 88
 *   codes = fp4_quantize_pack(h, E2M1, TENSOR, tensor_scale = out_scale,
 *     col_shift = out_shift): y = fl32(h * fl32(r' * 2^-k'[n])), r' = fl32(1 / a'),
 *     nearest E2M1 value after clipping to +-6, ties to even, sign bit of y.
 * Every step is a fixed binary32 sequence: the codes are bit-reproducible.
 * Requirements: N a multiple of 32; K a multiple of 32 and <= 116508; a, w_gate, w_up,
 * h_packed 16-byte aligned.  Empty M or N returns FP4_OK with nothing launched. */
fp4_status fp4_gemm_swiglu_quant(const fp4_swiglu_desc* d, void* stream);

/* NF4 lookup grid ([Overview], NF4: 16 levels placed at quantiles of the normal
 * distribution).  Fills *out (host) with kind FP4_GRID_LUT16 and
 *   lut[i] = RNE_binary16( Phi^-1((i + 1/2) / 16) / Phi^-1(15.5 / 16) ),  i = 0..15:
 * symmetric, end points -1 and +1, no exact zero; every level is a binary16 value, so
 * levels and the midpoints between neighbours are exact in binary32.  Phi^-1 is found
 * by bisection on Phi(x) = erfc(-x / sqrt 2) / 2 in binary64.  Host only, no launch.
 * Returns FP4_ERR_INVALID_ARG for a null pointer. */
fp4_status fp4_nf4_grid(fp4_grid* out);

/* Launch splitting of the W4A4 / W8A8 matrix-core products (host setting, process-wide).
 * Those kernels address each operand through a 32-bit buffer range, so a product whose A
 * or W spans more than `bytes` is launched as several row blocks of A and W (the per-row
 * scales, per-token scales and Y offset with them); the result is the same bit for bit.
 * The default, and the value set by bytes <= 0 or >= 0x7fff0000, is 0x7fff0000.  A
 * smaller limit lets a test exercise the block split on small shapes.  Takes effect for
 * launches made after it returns; not synchronised with calls running on other threads.
 * Always returns FP4_OK. */
fp4_status fp4_set_split_limit(int64_t bytes);

#ifdef __cplusplus
}
#endif
#endif /* FP4_H_ */

"""CPU oracle for the FP4 quantize / pre-shift / search / quantized-GEMM path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package imports this module; only
``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg use it.
It shares no code with the HIP library.  The brute-force parts (grid enumeration,
nearest-point search, exact error sums) are plain C in ``fp4_oracle.c``; everything
else is numpy, with float64 BLAS for the GEMM contractions.

Sources (web pages, cited by title and section):

* [FP4-LLM]  "首个支持4-bit浮点量化的LLM来了，解决LLaMA、BERT等的部署难题" (811yy.cn),
  summarising the LLM-FP4 paper: the FP value formula (sign, exponent field
  p in [0, 2^e-1], mantissa bits, bias b); "scale and clip" eqs. (2)-(3); bias from
  the chosen range, eq. (4), usable as a real-valued scale; "compare and quantize",
  eq. (5); the scaling factor kept outside the low-bit matrix product ("efficient
  matrix multiplication"); the search over exponent/mantissa split and range; the
  pre-shifted exponent bias (per-channel maxima split into a per-tensor real scale
  times per-channel powers of two that are folded into the weights).
* [Overview] "量化技术详解" (aidocs.cortexgrid.cn): floating-point types (FP16 range),
  granularities, static quantization, section NF4 (grid at normal quantiles).
* [W8A8]     intelliparadigm.com LLM-quantization practice, section 2.2: scale-factored
  integer matmul (low-bit product first, scales multiplied afterwards); group size 128.
* [Tutorial] "为什么我们需要4-bit浮点量化" (devpress.csdn.net), section 2.2: two 4-bit
  values per byte.

Readings where the pages are silent or garbled are stated in the docstrings of the
functions that take them.  Every function that has no independent pin in
``tests/test_oracle_pins.py`` says "parity unpinned" in its docstring (none at
present).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass
from fractions import Fraction

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libfp4_oracle.so")

GCC_CMD = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
           "-shared", "-std=c11", "-o", _LIB_PATH, _SRC, "-lm"]


def build(force: bool = False) -> str:
    """Compile the C part of the oracle (gcc, no FMA contraction, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        subprocess.check_call(GCC_CMD)
    return _LIB_PATH


_lib = None


def _c():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        lib.orc_minifloat_value.restype = ctypes.c_double
        lib.orc_minifloat_value.argtypes = [ctypes.c_int] * 4
        lib.orc_minifloat_grid.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P]
        lib.orc_quantize.argtypes = [P, P, ctypes.c_int64, ctypes.c_int, P, ctypes.c_int, P]
        lib.orc_search_sse.argtypes = [P, ctypes.c_int64, P, ctypes.c_int, ctypes.c_int, P,
                                       ctypes.c_int, P]
        lib.orc_exp_min.restype = ctypes.c_int
        lib.orc_nbucket.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


# ----------------------------------------------------------------------------------
# Grids ([FP4-LLM] FP value formula; [Overview] NF4)
# ----------------------------------------------------------------------------------
E1M2, E2M1, E3M0 = (1, 2), (2, 1), (3, 0)
FORMATS_4BIT = (E1M2, E2M1, E3M0)


def minifloat_grid(e: int, m: int, b: int = 1) -> np.ndarray:
    """All 2^(e+m) magnitudes of the FP(e, m, b) grid, indexed by the magnitude code
    c = p<<m | d.  p == 0 is subnormal (2^(1-b)*d/2^m), p >= 1 normal
    (2^(p-b)*(1+d/2^m)); no code is reserved for inf/NaN."""
    out = np.zeros(1 << (e + m), dtype=np.float64)
    _c().orc_minifloat_grid(e, m, b, _ptr(out))
    return out


def nf4_table() -> np.ndarray:
    """16-point NF4 grid ([Overview], NF4: levels at quantiles of N(0,1)).

    Plainest 16-level reading: G_i = Phi^-1((i + 1/2)/16) normalised so the end points
    are +-1, each rounded to binary16 (so every grid value and every midpoint of two
    neighbours is exact in binary32).  Symmetric, no exact zero."""
    from scipy.special import ndtri
    q = ndtri((np.arange(16) + 0.5) / 16.0)
    g = q / ndtri(15.5 / 16.0)
    return g.astype(np.float16).astype(np.float64)


@dataclass(frozen=True)
class Grid:
    """kind 'minifloat': sign-magnitude code sign<<(e+m) | (p<<m | d), values = the
    magnitudes by magnitude code (4-bit: e + m == 3; 8-bit FP8: e + m == 7).
    kind 'lut': code = index into 16 sorted signed values."""
    kind: str
    e: int = 0
    m: int = 0
    values: tuple = ()

    @property
    def bits(self) -> int:
        """Bits per code: 4, 6 for the FP6 grids, 8 for the FP8 grids."""
        if self.kind == "minifloat" and self.e + self.m in (5, 7):
            return self.e + self.m + 1
        return 4

    @property
    def array(self) -> np.ndarray:
        return np.asarray(self.values, dtype=np.float64)

    @property
    def qmax(self) -> float:
        v = self.array
        return float(v[-1]) if self.kind == "minifloat" else float(max(abs(v[0]), abs(v[-1])))

    def decode(self, codes: np.ndarray) -> np.ndarray:
        """Grid value of each code (float64), without any scale."""
        c = codes.astype(np.int64)
        if self.kind == "minifloat":
            nb = self.e + self.m
            mag = self.array[c & ((1 << nb) - 1)]
            return np.where((c >> nb) & 1, -mag, mag)
        return self.array[c & 15]


def minifloat(e: int, m: int) -> Grid:
    return Grid("minifloat", e, m, tuple(minifloat_grid(e, m, 1)))


def fp6(e: int, m: int) -> Grid:
    """The OCP 6-bit formats (FP6 of the progressive 8/6/4-bit precision, [FP4-LLM]):
    E2M3 with bias 1 (largest 7.5) and E3M2 with bias 3 (largest 28), no code reserved;
    32 magnitudes each by the same FP value formula."""
    if (e, m) == (2, 3):
        g = minifloat_grid(2, 3, 1)
    elif (e, m) == (3, 2):
        g = minifloat_grid(3, 2, 3)
    else:
        raise ValueError((e, m))
    return Grid("minifloat", e, m, tuple(g))


def fp8(e: int, m: int) -> Grid:
    """The OCP 8-bit formats (FP8 for key layers, [FP4-LLM] mixed precision): E4M3 with
    bias 7 whose all-ones code S.1111.111 is NaN (127 magnitudes, largest 448), and E5M2
    with bias 15 whose top exponent holds inf/NaN (124 magnitudes, largest 57344).  The
    magnitude of code p<<m | d follows the same FP value formula as the 4-bit grids."""
    if (e, m) == (4, 3):
        g = minifloat_grid(4, 3, 7)[:127]
    elif (e, m) == (5, 2):
        g = minifloat_grid(5, 2, 15)[:124]
    else:
        raise ValueError((e, m))
    return Grid("minifloat", e, m, tuple(g))


def lut(values) -> Grid:
    v = np.asarray(values, dtype=np.float64)
    assert v.shape == (16,) and np.all(np.diff(v) > 0)
    return Grid("lut", 0, 0, tuple(v))


def nf4() -> Grid:
    return lut(nf4_table())


def qmax(e: int, m: int, b: int = 1) -> float:
    """Largest magnitude of FP(e, m, b): (2 - 2^-m) * 2^(2^e - 1 - b)  ([FP4-LLM] the
    clipping bound +-Qmax of eq. (2))."""
    return float(minifloat_grid(e, m, b)[-1])


def real_bias(s: float) -> float:
    """Real-valued exponent bias equivalent to scale s on the canonical bias-1 grid
    ([FP4-LLM] eq. (4): the bias derived from the range acts as a real scale):
    values 2^(p-b)(1+d/2^m) = s * 2^(p-1)(1+d/2^m)  <=>  b = 1 - log2(s)."""
    return 1.0 - math.log2(float(s)) if s > 0 else math.inf


# ----------------------------------------------------------------------------------
# Rounding helpers (binary16 / bfloat16 storage)
# ----------------------------------------------------------------------------------
def f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32)


def rne_f16(x) -> np.ndarray:
    """Round binary32 to binary16 (numpy's cast is round-to-nearest-even)."""
    return f32(x).astype(np.float16)


def rne_bf16_bits(x) -> np.ndarray:
    """Round finite binary32 values to bfloat16, nearest-even; returns uint16 bits."""
    u = f32(x).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def reciprocal(s) -> np.ndarray:
    """r = fl32(1/s), and 0 where s == 0 (an all-zero block quantizes to +-0)."""
    s = f32(s)
    with np.errstate(divide="ignore", over="ignore"):
        r = np.where(s == 0, np.float32(0), np.float32(1) / np.where(s == 0, np.float32(1), s))
    return r.astype(np.float32)


# ----------------------------------------------------------------------------------
# Quantize ("scale and clip" + "compare and quantize") and pack
# ----------------------------------------------------------------------------------
def quantize(x, r, grid: Grid) -> np.ndarray:
    """codes[i] for y = fl32(x[i] * r[i]); brute-force nearest grid point, exact ties
    to the even code; minifloat codes carry signbit(x) in bit 3 ([FP4-LLM] eqs. (2)-(5)
    read as: scale by the reciprocal of the full-precision scale, clip to +-Qmax,
    round to the nearest representable value)."""
    x = np.ascontiguousarray(f32(x))
    r = np.ascontiguousarray(np.broadcast_to(f32(r), x.shape))
    assert np.all(np.isfinite(x)), "non-finite inputs are not valid"
    out = np.empty(x.shape, dtype=np.uint8)
    g = np.ascontiguousarray(grid.array)
    kind = {4: 0, 6: 3, 8: 2}[grid.bits] if grid.kind == "minifloat" else 1
    _c().orc_quantize(_ptr(x), _ptr(r), x.size, kind, _ptr(g), g.size, _ptr(out))
    return out


def pack_codes(codes: np.ndarray, grid: Grid) -> np.ndarray:
    """Storage of codes: two 4-bit codes per byte; one 8-bit code per byte; 6-bit codes
    as a little-endian bit stream, code i in bits [6 i, 6 i + 6) of its row (four codes
    in three bytes; the matrix cores' FP6 operand layout)."""
    c = np.asarray(codes, dtype=np.uint8)
    if grid.bits == 8:
        return c.copy()
    if grid.bits == 6:
        assert c.shape[-1] % 4 == 0
        q = c.reshape(c.shape[:-1] + (-1, 4)).astype(np.uint32)
        v = q[..., 0] | (q[..., 1] << 6) | (q[..., 2] << 12) | (q[..., 3] << 18)
        b = np.stack([v & 255, (v >> 8) & 255, v >> 16], axis=-1).astype(np.uint8)
        return b.reshape(c.shape[:-1] + (-1,))
    return pack(c)


def unpack_codes(packed: np.ndarray, grid: Grid) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    if grid.bits == 8:
        return p.copy()
    if grid.bits == 6:
        b = p.reshape(p.shape[:-1] + (-1, 3)).astype(np.uint32)
        v = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16)
        q = np.stack([(v >> (6 * i)) & 63 for i in range(4)], axis=-1).astype(np.uint8)
        return q.reshape(p.shape[:-1] + (-1,))
    return unpack(p)


def pack(codes: np.ndarray) -> np.ndarray:
    """Two codes per byte along the last axis: byte j = code[2j] | code[2j+1] << 4
    ([Tutorial] section 2.2, two 4-bit values per byte; the low nibble holding the
    even element is a reading)."""
    c = np.asarray(codes, dtype=np.uint8)
    assert c.shape[-1] % 2 == 0
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


# ----------------------------------------------------------------------------------
# Calibration ([Overview] granularities; [W8A8] section 2.2 calibrate: max |x|)
# ----------------------------------------------------------------------------------
def amax_tensor(x) -> np.float32:
    return np.float32(np.max(np.abs(f32(x)))) if np.size(x) else np.float32(0)


def amax_columns(x, first_rows: int) -> np.ndarray:
    """Per-column max |x| over rows 0 .. first_rows-1 (static calibration tokens)."""
    return np.max(np.abs(f32(x)[:first_rows]), axis=0).astype(np.float32)


def amax_row_groups(x, group: int) -> np.ndarray:
    x = f32(x)
    R, C = x.shape
    return np.max(np.abs(x.reshape(R, C // group, group)), axis=2).astype(np.float32)


def scale_from_amax(amax, grid: Grid) -> np.ndarray:
    """s = fl32(amax / Qmax): the full-precision scale that maps the range onto +-Qmax."""
    return (f32(amax) / np.float32(grid.qmax)).astype(np.float32)


# ----------------------------------------------------------------------------------
# Granular quantize + pack, dequantize
# ----------------------------------------------------------------------------------
def quantize_pack(x, grid: Grid, mode: str, group: int = 0, scale_dtype: str = "f32",
                  tensor_scale=None, col_shift=None, amax=None):
    """mode: 'tensor' | 'row' | 'group' (group columns along each row).
    scale_dtype 'f16' stores binary16 scales; quantization always uses the STORED
    scale (r = fl32(1/stored)).  tensor_scale: fixed per-tensor scale (static
    activation quantization).  col_shift k[cols]: the multiplier of column j becomes
    r * 2^-k[j] (pre-shifted exponent bias).  Returns (packed uint8, scales)."""
    x = f32(x)
    R, C = x.shape
    if mode == "tensor":
        if tensor_scale is not None:
            s = np.float32(tensor_scale)
        else:
            s = scale_from_amax(amax_tensor(x) if amax is None else amax, grid)
        s_st = rne_f16(s).astype(np.float32) if scale_dtype == "f16" else np.float32(s)
        r = np.full((R, C), reciprocal(s_st), dtype=np.float32)
        scales = np.array([s_st], dtype=np.float32)
    elif mode == "row":
        s = scale_from_amax(np.max(np.abs(x), axis=1) if amax is None else amax, grid)
        s_st = rne_f16(s).astype(np.float32) if scale_dtype == "f16" else s
        r = np.repeat(reciprocal(s_st)[:, None], C, axis=1)
        scales = s_st.astype(np.float32)
    elif mode == "group":
        s = scale_from_amax(amax_row_groups(x, group) if amax is None else amax, grid)
        s_st = rne_f16(s).astype(np.float32) if scale_dtype == "f16" else s
        r = np.repeat(reciprocal(s_st), group, axis=1)
        scales = s_st.astype(np.float32)
    else:
        raise ValueError(mode)
    if col_shift is not None:
        k = np.asarray(col_shift, dtype=np.int64)
        r = np.ldexp(r, -k[None, :]).astype(np.float32)
    codes = quantize(x, r, grid)
    if scale_dtype == "f16":
        scales = scales.astype(np.float16)
    return pack_codes(codes, grid), scales


def dequantize(packed, grid: Grid, mode: str, scales, group: int = 0, col_shift=None):
    """v = +-fl32(g(code) * s), times 2^k[j] for a shifted column (exact)."""
    codes = unpack_codes(packed, grid)
    R, C = codes.shape
    s = f32(np.asarray(scales).astype(np.float32))
    if mode == "tensor":
        sf = np.full((R, C), s.reshape(-1)[0], dtype=np.float32)
    elif mode == "row":
        sf = np.repeat(s.reshape(R, 1), C, axis=1)
    else:
        sf = np.repeat(s.reshape(R, C // group), group, axis=1)
    v = (grid.decode(codes).astype(np.float32) * sf).astype(np.float32)
    if col_shift is not None:
        v = np.ldexp(v, np.asarray(col_shift, dtype=np.int64)[None, :]).astype(np.float32)
    return v


# ----------------------------------------------------------------------------------
# Two-mode grid ([HiFloat4] section 2.1: each value group uses either the small-value
# layout sign|2 exponent|1 mantissa (E2M1) or the large-value layout sign|1 exponent|
# 2 mantissa (E1M2), marked by one control bit whose cost is shared by the group)
# ----------------------------------------------------------------------------------
TWO_MODES = (E2M1, E1M2)  # mode 0, mode 1


def two_mode_error(x, codes, s, grid: Grid) -> float:
    """Squared quantization error of one group under one mode, as an exact comparison
    key: the sum over the group of (|x| - fl32(g(code) * s))^2, each difference and
    square exact in binary64 (|x| and the dequantized value are binary32 values within
    a factor of 4 of each other or the latter is 0), summed without rounding
    (math.fsum returns the correctly rounded exact sum)."""
    q = (grid.array[codes & 7].astype(np.float32) * np.float32(s)).astype(np.float32)
    d = np.abs(f32(x)).astype(np.float64) - q.astype(np.float64)
    return math.fsum((d * d).tolist())


def quantize_two_mode(x, group: int, scale_dtype: str = "f32"):
    """Per group of `group` consecutive elements of each row: for each mode m (E2M1,
    E1M2) the scale s_m = fl32(amax / Qmax_m) (stored rounding: binary16 for f16
    scales), r_m = fl32(1/s_m), codes = quantize(x, r_m, grid m), and the squared error
    against fl32(g * s_m).  The mode with the smaller exact error wins (equal errors:
    E2M1); its codes are stored and its scale with the sign bit set for E1M2 (the control
    bit, in the otherwise unused sign of the non-negative scale).  Returns (packed,
    scales [R, C/group], modes [R, C/group])."""
    x = f32(x)
    R, C = x.shape
    G = C // group
    amax = amax_row_groups(x, group)
    codes_m, scales_m = [], []
    for (e, m) in TWO_MODES:
        g = minifloat(e, m)
        sc = scale_from_amax(amax, g)
        st = rne_f16(sc).astype(np.float32) if scale_dtype == "f16" else sc
        codes_m.append(quantize(x, np.repeat(reciprocal(st), group, axis=1), g))
        scales_m.append(st)
    codes = np.empty((R, C), dtype=np.uint8)
    scales = np.empty((R, G), dtype=np.float32)
    modes = np.zeros((R, G), dtype=np.uint8)
    grids = [minifloat(*f) for f in TWO_MODES]
    for r in range(R):
        for gi in range(G):
            sl = slice(gi * group, (gi + 1) * group)
            e0 = two_mode_error(x[r, sl], codes_m[0][r, sl], scales_m[0][r, gi], grids[0])
            e1 = two_mode_error(x[r, sl], codes_m[1][r, sl], scales_m[1][r, gi], grids[1])
            mode = 1 if e1 < e0 else 0
            modes[r, gi] = mode
            codes[r, sl] = codes_m[mode][r, sl]
            scales[r, gi] = -scales_m[1][r, gi] if mode else scales_m[0][r, gi]
    if scale_dtype == "f16":
        scales = scales.astype(np.float16)
    return pack(codes), scales, modes


def two_mode_values(packed, scales, group: int) -> np.ndarray:
    """Dequantized values of a two-mode tensor: v = +-fl32(g_mode(code) * |s|), the mode
    from the sign bit of the group's stored scale."""
    codes = unpack(packed)
    R, C = codes.shape
    s = np.asarray(scales).astype(np.float32).reshape(R, C // group)
    mode = np.signbit(s)
    mag = np.abs(s)
    e2, e1 = minifloat(*TWO_MODES[0]), minifloat(*TWO_MODES[1])
    g = np.where(np.repeat(mode, group, axis=1), e1.array[codes & 7], e2.array[codes & 7]).astype(np.float32)
    v = (g * np.repeat(mag, group, axis=1)).astype(np.float32)
    return np.where((codes >> 3) & 1, -v, v).astype(np.float32)


def gemm_w4a16_two_mode(x, w_packed, w_scales, group: int, absolute: bool = False):
    """r[m, n] = sum_g |s[n, g]| * sum_{k in g} x[m, k] * g_mode(n,g)(c[n, k]) in binary64
    (the W4A16 product with the grid chosen per group by the scale's sign bit);
    absolute=True sums magnitudes instead."""
    X = f32(x).astype(np.float64)
    if absolute:
        X = np.abs(X)
    codes = unpack(w_packed)
    N, K = codes.shape
    s = np.asarray(w_scales).astype(np.float32).reshape(N, K // group)
    mode = np.repeat(np.signbit(s), group, axis=1)
    e2, e1 = minifloat(*TWO_MODES[0]), minifloat(*TWO_MODES[1])
    V = np.where(mode, e1.array[codes & 7], e2.array[codes & 7])
    if not absolute:
        V = np.where((codes >> 3) & 1, -V, V)
    mag = np.abs(s).astype(np.float64)
    out = np.zeros((X.shape[0], N), dtype=np.float64)
    for gi in range(K // group):
        sl = slice(gi * group, (gi + 1) * group)
        out += (X[:, sl] @ V[:, sl].T) * mag[None, :, gi]
    return out

# ----------------------------------------------------------------------------------
# Pre-shifted exponent bias ([FP4-LLM], pre-shifted exponent bias paragraphs)
# ----------------------------------------------------------------------------------
K_MIN = -64


def preshift(chan_amax, act_grid: Grid):
    """Split per-channel activation maxima c_k into a per-tensor real scale and
    per-channel powers of two:  a = fl32(c_max / Qmax),  k_k = the smallest integer j
    with c_max * 2^j >= c_k (so k_k <= 0 and no calibrated value leaves the range),
    k_k = 0 for c_k = 0, clamped at -64.  Exact, from frexp: c = f * 2^E with
    f in [0.5, 1):  k = E_k - E_max + (f_max < f_k)."""
    c = f32(chan_amax)
    cmax = np.float32(np.max(c)) if c.size else np.float32(0)
    a = np.float32(cmax / np.float32(act_grid.qmax))
    fk, ek = np.frexp(c.astype(np.float64))
    fm, em = np.frexp(np.float64(cmax))
    k = (ek - em + (fm < fk).astype(np.int64)).astype(np.int64)
    k = np.where(c == 0, 0, np.maximum(k, K_MIN)).astype(np.int8)
    return k, a


def shift_weights(w, k) -> np.ndarray:
    """W'[n, j] = W[n, j] * 2^k[j]  (exact power-of-two scaling)."""
    return np.ldexp(f32(w), np.asarray(k, dtype=np.int64)[None, :]).astype(np.float32)


def preshift_weights(w, chan_amax, act_grid: Grid, w_grid: Grid, w_mode: str = "row",
                     w_group: int = 0):
    """Fold the per-channel powers of two into W before weight quantization; the
    weight scale is taken per output row (or per group) of the shifted W'."""
    k, a = preshift(chan_amax, act_grid)
    wp = shift_weights(w, k)
    packed, scales = quantize_pack(wp, w_grid, w_mode, w_group)
    return k, a, packed, scales


def quantize_activations(x, act_grid: Grid, a, k):
    """Static activation quantization with the pre-shift: multiplier of column j is
    fl32(1/a) * 2^-k_j; one per-tensor scale a."""
    return quantize_pack(x, act_grid, "tensor", tensor_scale=a, col_shift=k)


# ----------------------------------------------------------------------------------
# Format and clip-range search ([FP4-LLM] search-based FP quantization)
# ----------------------------------------------------------------------------------
def clip_ratios(nclips: int = 100, lo: float = 0.5, hi: float = 1.0) -> np.ndarray:
    """nclips evenly spaced fractions of max|w| from lo to hi inclusive, computed in
    binary64 and rounded once to binary32."""
    j = np.arange(nclips, dtype=np.float64)
    return (lo + (hi - lo) * j / (nclips - 1)).astype(np.float32)


def _buckets_to_float(buckets: np.ndarray, exp_min: int, denom: int) -> float:
    """Correctly rounded binary64 of (sum_j bucket_j * 2^(exp_min + j)) / denom."""
    total = 0
    lo = buckets[0::2]
    hi = buckets[1::2]
    for j in np.nonzero((lo != 0) | (hi != 0))[0]:
        total += (int(lo[j]) | (int(hi[j]) << 64)) << int(j)
    # total = sum_j bucket_j * 2^j; the exact sum is total * 2^exp_min
    return float(Fraction(total, denom) * Fraction(2) ** exp_min)


def candidate_mse(w, formats, clips) -> np.ndarray:
    """mse[f, j] = correctly rounded binary64 of (1/n) * sum_i (w_i - deq_i)^2 for
    format f and clip value clips[j] (see fp4_oracle.c: exact accumulation)."""
    w = np.ascontiguousarray(f32(w).reshape(-1))
    grids = np.ascontiguousarray(np.stack([minifloat_grid(e, m) for (e, m) in formats]))
    clips = np.ascontiguousarray(f32(clips))
    lib = _c()
    nb = lib.orc_nbucket()
    emin = lib.orc_exp_min()
    out = np.zeros(len(formats) * clips.size * nb * 2, dtype=np.uint64)
    lib.orc_search_sse(_ptr(w), w.size, _ptr(grids), len(formats), grids.shape[1],
                       _ptr(clips), clips.size, _ptr(out))
    out = out.reshape(len(formats), clips.size, nb * 2)
    mse = np.empty((len(formats), clips.size), dtype=np.float64)
    for f in range(len(formats)):
        for j in range(clips.size):
            mse[f, j] = _buckets_to_float(out[f, j], emin, w.size)
    return mse


@dataclass
class SearchRecord:
    e: int
    m: int
    clip_index: int
    clip: np.float32
    scale: np.float32
    bias: float
    mse: float
    mse_runner_up: float


def search_tensor(w, formats=FORMATS_4BIT, nclips: int = 100, lo: float = 0.5,
                  hi: float = 1.0):
    """Evaluate every (format, clip) candidate, pick the minimum-MSE one (exact ties:
    earliest in enumeration order, formats outer, clips inner), and pack the tensor
    with the winner.  Returns (SearchRecord, packed codes, mse table)."""
    w = f32(w).reshape(-1)
    amax = amax_tensor(w)
    clips = (np.float32(amax) * clip_ratios(nclips, lo, hi)).astype(np.float32)
    mse = candidate_mse(w, formats, clips)
    flat = mse.reshape(-1)
    best = int(np.argmin(flat))  # argmin returns the first minimum
    runner = float(np.min(np.delete(flat, best))) if flat.size > 1 else math.inf
    f, j = divmod(best, nclips)
    e, m = formats[f]
    g = minifloat(e, m)
    s = np.float32(clips[j] / np.float32(g.qmax))
    packed, _ = quantize_pack(w.reshape(1, -1), g, "tensor", tensor_scale=s)
    rec = SearchRecord(e, m, j, np.float32(clips[j]), s, real_bias(s), float(flat[best]), runner)
    return rec, packed.reshape(-1), mse


def search_activations(x, unit: str, first_rows: int = 0, formats=FORMATS_4BIT, nclips: int = 100,
                       lo: float = 0.5, hi: float = 1.0):
    """The search applied to activations ([FP4-LLM] search-based FP quantization, for
    activations as for weights; [Overview] static quantization from calibration data,
    per-token granularity).  x [rows, cols] (bf16 values taken as their binary32 values).
    unit 'tensor': rows [0, T) (T = first_rows, or every row when first_rows <= 0 or >=
    rows) are one tensor for search_tensor, and every row is packed with its winner
    (quantize_pack, TENSOR scale); unit 'row': search_tensor on each row, each row packed
    with its own winner.  Returns (list of SearchRecord, packed [rows, cols/2])."""
    x = f32(x)
    R, C = x.shape
    if unit == "row":
        recs, rows = [], []
        for r in range(R):
            rec, p, _ = search_tensor(x[r], formats, nclips, lo, hi)
            recs.append(rec)
            rows.append(p)
        return recs, (np.stack(rows) if R else np.zeros((0, C // 2), np.uint8))
    if unit != "tensor":
        raise ValueError(unit)
    T = first_rows if 0 < first_rows < R else R
    rec, _, _ = search_tensor(x[:T], formats, nclips, lo, hi)
    packed, _ = quantize_pack(x, minifloat(rec.e, rec.m), "tensor", tensor_scale=rec.scale)
    return [rec], packed

# ----------------------------------------------------------------------------------
# Quantized GEMMs (scales factored out of the low-bit product: [FP4-LLM] "efficient
# matrix multiplication"; [W8A8] section 2.2 quantized_matmul).  Y = X W^T, W [N, K].
# ----------------------------------------------------------------------------------
def _weight_values(packed, grid: Grid) -> np.ndarray:
    return grid.decode(unpack_codes(packed, grid))


def gemm_w4a16(x, w_packed, w_grid: Grid, mode: str, w_scales, group: int = 0, absolute: bool = False):
    """r[m, n] = sum_g s[n, g] * sum_{k in g} x[m, k] * g(c[n, k])  in binary64.
    x: binary32 values (bf16 activations widened exactly).  absolute=True evaluates the
    same sum over |x|, |g(c)| and |s| (the magnitude that bounds rounding errors)."""
    X = f32(x).astype(np.float64)
    V = _weight_values(w_packed, w_grid)
    N, K = V.shape
    s = np.asarray(w_scales).astype(np.float64)
    if absolute:
        X, V, s = np.abs(X), np.abs(V), np.abs(s)
    if mode == "tensor":
        return (X @ V.T) * s.reshape(-1)[0]
    if mode == "row":
        return (X @ V.T) * s.reshape(1, N)
    G = K // group
    s = s.reshape(N, G)
    out = np.zeros((X.shape[0], N), dtype=np.float64)
    for gi in range(G):
        sl = slice(gi * group, (gi + 1) * group)
        out += (X[:, sl] @ V[:, sl].T) * s[None, :, gi]
    return out


def gemm_w4a4(a_packed, a_grid: Grid, a_scale, w_packed, w_grid: Grid, mode: str,
              w_scales, group: int = 0, absolute: bool = False):
    """Both operands quantized.  Returns (r, acc):
    r = a * sum_(blocks) s[n, b] * sum_{k in b} A_q[m, k] * W_q[n, k]  (binary64);
    acc = the unscaled code product sum_k A_q W_q (exact in binary64 for the 4-bit
    minifloat grids: every product is a multiple of 2^-4 and the sums stay far below
    2^53; for FP8 a binary64 sum)."""
    A = _weight_values(a_packed, a_grid)
    V = _weight_values(w_packed, w_grid)
    if absolute:  # the same sums over magnitudes (bounds rounding errors)
        A, V = np.abs(A), np.abs(V)
    N, K = V.shape
    # one activation scale, or one per row (token) of A ([Overview] per-token granularity)
    a_arr = np.asarray(a_scale, dtype=np.float32).astype(np.float64)
    if absolute:
        a_arr = np.abs(a_arr)
    a = a_arr.reshape(-1, 1) if a_arr.size > 1 else float(a_arr.reshape(-1)[0])
    s = np.asarray(w_scales).astype(np.float64)
    if absolute:
        s = np.abs(s)
    if mode in ("tensor", "row"):
        acc = A @ V.T
        sv = s.reshape(-1)[0] if mode == "tensor" else s.reshape(1, N)
        return acc * sv * a, acc
    G = K // group
    s = s.reshape(N, G)
    out = np.zeros((A.shape[0], N), dtype=np.float64)
    for gi in range(G):
        sl = slice(gi * group, (gi + 1) * group)
        out += (A[:, sl] @ V[:, sl].T) * s[None, :, gi]
    return out * a, None


def w4a4_epilogue_f32(acc, a_scale, s_row) -> np.ndarray:
    """Fixed epilogue of the row-scaled minifloat W4A4 product, used where the result
    is compared bit for bit: y32 = fl32(acc * fl32(a * s_n)); with one activation scale
    per token, y32[m, n] = fl32(acc * fl32(a_m * s_n))."""
    a = f32(a_scale)
    if a.size > 1:
        mult = (a.reshape(-1, 1) * f32(s_row).reshape(1, -1)).astype(np.float32)
        return (f32(acc) * mult).astype(np.float32)
    sn = (np.float32(a.reshape(-1)[0]) * f32(s_row)).astype(np.float32)
    return (f32(acc) * sn[None, :]).astype(np.float32)


# ----------------------------------------------------------------------------------
# Activation quantization fused into the producing GEMM (the pages' fused
# quantize-activation-dequantize idea, [HiFloat4] "Quant-GeLU-Dequant"): the LLaMA MLP
# producer is SwiGLU, h = SiLU(x W_gate^T) * (x W_up^T), and its consumer the W4A4 down
# projection, which takes h as E2M1 codes with its own pre-shift.
# ----------------------------------------------------------------------------------
LOG2E_F32 = np.float32(1.4426950408889634)
# 2^f = e^(f ln 2): Taylor coefficients (ln 2)^i / i!, rounded to binary32, i = 0..7
EXP2_COEF_F32 = [np.float32(math.log(2.0) ** i / math.factorial(i)) for i in range(8)]


def exp_f32(x) -> np.ndarray:
    """e^x as a fixed sequence of binary32 operations, so that any IEEE binary32
    implementation of the same sequence gives the same bits: t = fl(x * log2 e),
    n = rint(t) (ties to even), f = t - n (exact, |f| <= 1/2), p = the degree-7 Taylor
    polynomial of 2^f in Horner form (a multiply and an add per term, no fused
    multiply-add), result fl(p * 2^n).  Relative error below 1e-5 for |x| <= 88 (the
    rounding of t dominates); 2^n over- and underflows like e^x."""
    x = f32(x)
    t = (x * LOG2E_F32).astype(np.float32)
    n = np.rint(t).astype(np.float32)
    fr = (t - n).astype(np.float32)
    p = np.full_like(fr, EXP2_COEF_F32[7])
    for c in reversed(EXP2_COEF_F32[:7]):
        p = ((p * fr).astype(np.float32) + c).astype(np.float32)
    with np.errstate(over="ignore", under="ignore"):
        return np.ldexp(p, np.clip(n, -300, 300).astype(np.int64)).astype(np.float32)


def silu_f32(x) -> np.ndarray:
    """SiLU(x) = x * sigmoid(x) = x / (1 + e^-x), in binary32: fl(x / fl(1 + exp_f32(-x)))
    (the division correctly rounded; e^-x = inf for very negative x gives -0)."""
    x = f32(x)
    with np.errstate(over="ignore"):
        d = (np.float32(1) + exp_f32(-x)).astype(np.float32)
        return (x / d).astype(np.float32)


def w4a4_swiglu_quant(a_packed, a_scale, wg_packed, s_gate, wu_packed, s_up, out_scale, out_shift):
    """Gate and up W4A4 E2M1 products of the same packed activations, each through the
    fixed epilogue y = fl32(acc * fl32(a * s_n)) (binary32, before any bf16 rounding),
    h = fl32(silu_f32(y_gate) * y_up), and h quantized as the next layer's activations:
    quantize_activations(h, E2M1, out_scale, out_shift).  Returns (codes, h)."""
    e2 = minifloat(2, 1)
    _, acc_g = gemm_w4a4(a_packed, e2, a_scale, wg_packed, e2, "row", s_gate)
    _, acc_u = gemm_w4a4(a_packed, e2, a_scale, wu_packed, e2, "row", s_up)
    yg = w4a4_epilogue_f32(acc_g, a_scale, s_gate)
    yu = w4a4_epilogue_f32(acc_u, a_scale, s_up)
    h = (silu_f32(yg) * yu).astype(np.float32)
    codes, _ = quantize_activations(h, e2, out_scale, out_shift)
    return codes, h


def rel_err(y, r) -> float:
    """Normwise max relative error max|y - r| / max|r|."""
    r = np.asarray(r, dtype=np.float64)
    d = np.max(np.abs(np.asarray(y, dtype=np.float64) - r)) if r.size else 0.0
    den = np.max(np.abs(r)) if r.size else 1.0
    return float(d / den) if den > 0 else float(d)


# ----------------------------------------------------------------------------------
# Elementwise error bounds (test tolerances).  A float computation whose additions and
# multiplications are each rounded (relative error <= u = 2^-24 when rounded to nearest)
# and whose products of terms are exact satisfies, for each output,
# |y - r| <= d * u * S + O(u^2), with S the same sum over magnitudes
# (gemm_*(..., absolute=True)) and d the largest number of roundings on the path from one
# product to the output (Higham, Accuracy and Stability of Numerical Algorithms,
# sections 3.1 and 4.2: the error bounds of recursive and tree summation).  The callers
# give each output its bound d * u * S (+ any further term of their arithmetic).
# ----------------------------------------------------------------------------------
U32 = 2.0 ** -24


def elementwise_excess(y32, r, bound) -> float:
    """max over outputs of |y32 - r| / bound; <= 1 means every output is within its
    bound."""
    y = np.asarray(y32, np.float64)
    r = np.asarray(r, np.float64)
    bound = np.broadcast_to(np.asarray(bound, np.float64), r.shape)
    err = np.abs(y - r)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(err == 0, 0.0, err / bound)
    return float(np.max(q)) if q.size else 0.0


def bf16_ulps_from_rounded(yb_bits, r, bound):
    """For the outputs whose binary32 error bound is at most 2^-10 |r| (a quarter of a
    bfloat16 ulp or less), the distance in bfloat16 ulps between the output's bf16 bits
    and RNE_bf16(r).  Returns (largest distance, number of outputs checked)."""
    r = np.asarray(r, np.float64)
    mask = np.broadcast_to(np.asarray(bound, np.float64), r.shape) <= 2.0 ** -10 * np.abs(r)
    if not mask.any():
        return 0, 0
    f, e = np.frexp(r[mask])  # RNE to 8 significant bits straight from binary64
    want = rne_bf16_bits(np.ldexp(np.rint(np.ldexp(f, 8)), e - 8).astype(np.float32)).astype(np.int64)
    got = np.asarray(yb_bits, np.uint16)[mask].astype(np.int64)
    # same sign (the bound keeps y32 on r's side of zero): compare magnitudes
    dist = np.abs((got & 0x7FFF) - (want & 0x7FFF)) + 0x10000 * ((got ^ want) >> 15 & 1)
    return int(dist.max()), int(mask.sum())

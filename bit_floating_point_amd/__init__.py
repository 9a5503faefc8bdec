"""Python binding of libfp4 (include/fp4.h): FP4 quantize / pre-shift / search /
quantized GEMM for AMD MI355X.

Argument marshalling only: every function here allocates its outputs as torch device
tensors (when the caller does not pass them), passes raw device pointers and the
current HIP stream to the C ABI, and raises ``FP4Error`` on a non-OK status.  All
arithmetic runs in the HIP kernels of libfp4.so; there is no CPU path.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib as L
from ._lib import (FP4Error, FP4_BF16, FP4_F16, FP4_F32, FP4_PACKED, FP4_REDUCE_COLUMN,
                   FP4_REDUCE_ROW_GROUP, FP4_REDUCE_TENSOR, FP4_SCALE_GROUP, FP4_SCALE_ROW,
                   FP4_SCALE_TENSOR)

__all__ = ["FP4Error", "grid_minifloat", "grid_lut", "grid_nf4", "grid_two_mode", "nf4_values", "set_split_limit", "gran", "fp4_calibrate", "fp4_quantize_pack",
           "fp4_dequantize", "fp4_preshift_weights", "fp4_search_format", "fp4_search_format_static", "fp4_gemm",
           "fp4_gemm_swiglu_quant", "fp4_search_activations", "search_results_host", "E2M1", "E1M2", "E3M0"]


def grid_minifloat(e: int, m: int) -> L.fp4_grid:
    g = L.fp4_grid()
    g.kind, g.e, g.m, g.reserved = L.FP4_GRID_MINIFLOAT, e, m, 0
    return g


def grid_lut(values) -> L.fp4_grid:
    vals = [float(v) for v in values]
    if len(vals) != 16:
        raise ValueError("a lookup grid has 16 values")
    g = L.fp4_grid()
    g.kind, g.e, g.m, g.reserved = L.FP4_GRID_LUT16, 0, 0, 0
    for i, v in enumerate(vals):
        g.lut[i] = v
    return g


E2M1, E1M2, E3M0 = (2, 1), (1, 2), (3, 0)


def grid_nf4() -> L.fp4_grid:
    """The library's NF4 lookup grid (fp4_nf4_grid: 16 levels at normal quantiles)."""
    g = L.fp4_grid()
    L.check(L.lib().fp4_nf4_grid(ctypes.byref(g)), "fp4_nf4_grid")
    return g


def nf4_values() -> list:
    """The 16 NF4 levels of grid_nf4() as Python floats."""
    return [float(v) for v in grid_nf4().lut]


def set_split_limit(nbytes: int = 0) -> None:
    """fp4_set_split_limit: operand bytes per launch of the W4A4 / W8A8 products (<= 0:
    the default 32-bit buffer range)."""
    L.check(L.lib().fp4_set_split_limit(int(nbytes)), "fp4_set_split_limit")


def grid_two_mode() -> L.fp4_grid:
    """E2M1 or E1M2 per scale group, the mode in the sign bit of the group's scale."""
    g = L.fp4_grid()
    g.kind, g.e, g.m, g.reserved = L.FP4_GRID_TWO_MODE, 0, 0, 0
    return g


def gran(mode: str = "tensor", group: int = 0, scale_dtype: str = "f32") -> L.fp4_gran:
    g = L.fp4_gran()
    g.mode = {"tensor": FP4_SCALE_TENSOR, "row": FP4_SCALE_ROW, "group": FP4_SCALE_GROUP}[mode]
    g.group = group if mode == "group" else 0
    g.scale_dtype = FP4_F16 if scale_dtype == "f16" else FP4_F32
    g.reserved = 0
    return g


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return FP4_F32
    if t.dtype == torch.bfloat16:
        return FP4_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ld(t: torch.Tensor) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D row-major tensor")
    return t.stride(0)


def _units(g: L.fp4_gran, rows: int, cols: int) -> int:
    if g.mode == FP4_SCALE_TENSOR:
        return 1
    if g.mode == FP4_SCALE_ROW:
        return rows
    return rows * (cols // g.group)


def fp4_calibrate(x: torch.Tensor, reduce: str = "tensor", group: int = 0, first_rows: int = 0,
                  out: torch.Tensor | None = None) -> torch.Tensor:
    rows, cols = x.shape
    r = {"tensor": FP4_REDUCE_TENSOR, "column": FP4_REDUCE_COLUMN, "row_group": FP4_REDUCE_ROW_GROUP}[reduce]
    n = 1 if r == FP4_REDUCE_TENSOR else (cols if r == FP4_REDUCE_COLUMN else rows * (cols // max(group, 1)))
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=x.device)
    L.check(L.lib().fp4_calibrate(_ptr(x), _dtype_code(x), rows, cols, _ld(x), r, group, first_rows,
                                  _ptr(out), _stream(x.device)), "fp4_calibrate")
    return out


def code_bits(grid: L.fp4_grid) -> int:
    """Bits per stored code: 8 for the FP8 grids, 6 for the FP6 grids (a bit stream),
    4 otherwise (two codes per byte)."""
    if grid.kind == L.FP4_GRID_MINIFLOAT and grid.e + grid.m in (5, 7):
        return grid.e + grid.m + 1
    return 4


def fp4_quantize_pack(x: torch.Tensor, grid: L.fp4_grid, g: L.fp4_gran, amax_in=None, tensor_scale=None,
                      col_shift=None, packed=None, scales=None):
    rows, cols = x.shape
    if packed is None:
        packed = torch.empty((rows, cols * code_bits(grid) // 8), dtype=torch.uint8, device=x.device)
    if scales is None and tensor_scale is None:
        sd = torch.float16 if g.scale_dtype == FP4_F16 else torch.float32
        scales = torch.empty(_units(g, rows, cols), dtype=sd, device=x.device)
    L.check(L.lib().fp4_quantize_pack(_ptr(x), _dtype_code(x), rows, cols, _ld(x), grid, g, _ptr(amax_in),
                                      _ptr(tensor_scale), _ptr(col_shift), _ptr(packed), _ld(packed),
                                      _ptr(scales), _stream(x.device)), "fp4_quantize_pack")
    return packed, scales


def fp4_dequantize(packed: torch.Tensor, grid: L.fp4_grid, g: L.fp4_gran, scales: torch.Tensor,
                   col_shift=None, out=None) -> torch.Tensor:
    rows, width = packed.shape
    cols = width * 8 // code_bits(grid)
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float32, device=packed.device)
    L.check(L.lib().fp4_dequantize(_ptr(packed), rows, cols, _ld(packed), grid, g, _ptr(scales),
                                   _ptr(col_shift), _ptr(out), _ld(out), _stream(packed.device)),
            "fp4_dequantize")
    return out


def fp4_preshift_weights(w: torch.Tensor, chan_amax: torch.Tensor, act_grid: L.fp4_grid,
                         w_grid: L.fp4_grid, w_gran: L.fp4_gran, shift=None, act_scale=None, packed=None,
                         scales=None):
    n, k = w.shape
    dev = w.device
    if shift is None:
        shift = torch.empty(k, dtype=torch.int8, device=dev)
    if act_scale is None:
        act_scale = torch.empty(1, dtype=torch.float32, device=dev)
    if packed is None:
        packed = torch.empty((n, k * code_bits(w_grid) // 8), dtype=torch.uint8, device=dev)
    if scales is None:
        sd = torch.float16 if w_gran.scale_dtype == FP4_F16 else torch.float32
        scales = torch.empty(_units(w_gran, n, k), dtype=sd, device=dev)
    L.check(L.lib().fp4_preshift_weights(_ptr(w), n, k, _ld(w), _ptr(chan_amax), act_grid, w_grid, w_gran,
                                         _ptr(shift), _ptr(act_scale), _ptr(packed), _ld(packed),
                                         _ptr(scales), _stream(dev)), "fp4_preshift_weights")
    return shift, act_scale, packed, scales


SEARCH_RESULT_BYTES = ctypes.sizeof(L.fp4_search_result)


def fp4_search_format(w: torch.Tensor, formats=(E1M2, E2M1, E3M0), nclips: int = 100, clip_lo: float = 0.5,
                      clip_hi: float = 1.0, workspace: torch.Tensor | None = None):
    """w: [ntensors, numel] float32.  Returns (results as a uint8 device buffer of
    fp4_search_result records, packed [ntensors, numel/2])."""
    T, numel = w.shape
    dev = w.device
    fm = (ctypes.c_int32 * (2 * len(formats)))(*[v for f in formats for v in f])
    need = L.lib().fp4_search_workspace_size(T, numel, len(formats), nclips)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    results = torch.empty(T * SEARCH_RESULT_BYTES, dtype=torch.uint8, device=dev)
    packed = torch.empty((T, numel // 2), dtype=torch.uint8, device=dev)
    L.check(L.lib().fp4_search_format(_ptr(w), T, numel, fm, len(formats), nclips, clip_lo, clip_hi,
                                      _ptr(results), _ptr(packed), _ptr(workspace), workspace.numel(),
                                      _stream(dev)), "fp4_search_format")
    return results, packed



def fp4_search_format_static(w: torch.Tensor, formats=(E1M2, E2M1, E3M0), nclips: int = 100,
                             clip_lo: float = 0.5, clip_hi: float = 1.0, results: torch.Tensor | None = None,
                             packed: torch.Tensor | None = None):
    """fp4_search_format on the library's static scratch (no workspace is allocated;
    calls on one GPU must not overlap).  results / packed may be given to make the call
    allocate nothing at all.  Returns (results buffer, packed [ntensors, numel/2])."""
    T, numel = w.shape
    dev = w.device
    fm = (ctypes.c_int32 * (2 * len(formats)))(*[v for f in formats for v in f])
    if results is None:
        results = torch.empty(T * SEARCH_RESULT_BYTES, dtype=torch.uint8, device=dev)
    if packed is None:
        packed = torch.empty((T, numel // 2), dtype=torch.uint8, device=dev)
    L.check(L.lib().fp4_search_format_static(_ptr(w), T, numel, fm, len(formats), nclips, clip_lo, clip_hi,
                                             _ptr(results), _ptr(packed), _stream(dev)), "fp4_search_format_static")
    return results, packed


def fp4_search_activations(x: torch.Tensor, unit: str = "row", first_rows: int = 0, formats=(E1M2, E2M1, E3M0),
                           nclips: int = 100, clip_lo: float = 0.5, clip_hi: float = 1.0,
                           workspace: torch.Tensor | None = None, packed: torch.Tensor | None = None):
    """x: [rows, cols] float32 or bfloat16.  unit 'row': a search per row (token);
    'tensor': one search over rows [0, first_rows) (all rows if first_rows <= 0), every
    row packed with its winner.  Returns (results buffer, packed [rows, cols/2])."""
    rows, cols = x.shape
    dev = x.device
    per_row = unit == "row"
    units = rows if per_row else 1
    t = 1 if per_row else (first_rows if 0 < first_rows < rows else rows)
    fm = (ctypes.c_int32 * (2 * len(formats)))(*[v for f in formats for v in f])
    need = L.lib().fp4_search_workspace_size(units, t * cols, len(formats), nclips)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    results = torch.empty(max(units, 1) * SEARCH_RESULT_BYTES, dtype=torch.uint8, device=dev)
    if packed is None:
        packed = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    L.check(L.lib().fp4_search_activations(_ptr(x), _dtype_code(x), rows, cols, _ld(x),
                                           FP4_SCALE_ROW if per_row else FP4_SCALE_TENSOR, first_rows, fm,
                                           len(formats), nclips, clip_lo, clip_hi, _ptr(results), _ptr(packed),
                                           _ld(packed), _ptr(workspace), workspace.numel(), _stream(dev)),
            "fp4_search_activations")
    return results, packed

@dataclass
class SearchRecord:
    e: int
    m: int
    clip_index: int
    format_index: int
    clip: float
    scale: float
    amax: float
    bias: float
    mse: float
    mse_runner_up: float


def search_results_host(results: torch.Tensor) -> list:
    raw = results.cpu().numpy().tobytes()
    out = []
    for i in range(len(raw) // SEARCH_RESULT_BYTES):
        r = L.fp4_search_result.from_buffer_copy(raw[i * SEARCH_RESULT_BYTES:(i + 1) * SEARCH_RESULT_BYTES])
        out.append(SearchRecord(r.e, r.m, r.clip_index, r.format_index, r.clip, r.scale, r.amax, r.bias, r.mse,
                                r.mse_runner_up))
    return out


def fp4_gemm(a: torch.Tensor, w_packed: torch.Tensor, w_scales: torch.Tensor, w_grid: L.fp4_grid,
             w_gran: L.fp4_gran, K: int | None = None, a_grid: L.fp4_grid | None = None,
             a_scale: torch.Tensor | None = None, y_dtype: torch.dtype = torch.bfloat16,
             y: torch.Tensor | None = None, a_scale_mode: str | None = None) -> torch.Tensor:
    """Y = X W^T.  a: [M, K] f32/bf16 (W4A16), or packed codes uint8 [M, K * bits / 8]
    (W4A4, W8A8, W6A6, with a_grid and a_scale).  a_scale: float32 on a's device, one
    value ('tensor') or one per row of a ('row'); a_scale_mode defaults to 'row' when
    a_scale holds M > 1 values."""
    M = a.shape[0]
    N = w_packed.shape[0]
    if a_scale is not None:
        if a_scale.dtype != torch.float32 or a_scale.device != a.device or not a_scale.is_contiguous():
            raise ValueError("a_scale must be a contiguous float32 tensor on the activations' device")
        if a_scale_mode is None:
            a_scale_mode = "row" if a_scale.numel() > 1 else "tensor"
        want = M if a_scale_mode == "row" else 1
        if a_scale_mode not in ("tensor", "row") or a_scale.numel() != want:
            raise ValueError(f"a_scale_mode {a_scale_mode!r} needs {want} scale(s), got {a_scale.numel()}")
    if a.dtype == torch.uint8:
        kind = FP4_PACKED
        K = K if K is not None else a.shape[1] * 8 // code_bits(a_grid if a_grid is not None else w_grid)
    else:
        kind = _dtype_code(a)
        K = K if K is not None else a.shape[1]
    if y is None:
        y = torch.empty((M, N), dtype=y_dtype, device=a.device)
    d = L.fp4_gemm_desc()
    d.M, d.N, d.K = M, N, K
    d.a_kind = kind
    d.a = a.data_ptr()
    d.lda = _ld(a)
    if a_grid is not None:
        d.a_grid = a_grid
    d.a_scale = a_scale.data_ptr() if a_scale is not None else None
    d.a_scale_mode = FP4_SCALE_ROW if a_scale_mode == "row" else FP4_SCALE_TENSOR
    d.w = w_packed.data_ptr()
    d.ldw = _ld(w_packed)
    d.w_grid = w_grid
    d.w_gran = w_gran
    d.w_scales = w_scales.data_ptr()
    d.y = y.data_ptr()
    d.ldy = _ld(y)
    d.y_dtype = FP4_BF16 if y.dtype == torch.bfloat16 else FP4_F32
    L.check(L.lib().fp4_gemm(ctypes.byref(d), _stream(a.device)), "fp4_gemm")
    return y


def fp4_gemm_swiglu_quant(a: torch.Tensor, a_scale: torch.Tensor, w_gate: torch.Tensor, s_gate: torch.Tensor,
                          w_up: torch.Tensor, s_up: torch.Tensor, out_scale: torch.Tensor,
                          out_shift: torch.Tensor | None = None, K: int | None = None,
                          h_packed: torch.Tensor | None = None) -> torch.Tensor:
    """E2M1 codes of h = SiLU(X W_gate^T) * (X W_up^T) quantized for the next layer
    (scale out_scale, column shifts out_shift).  a: packed E2M1 [M, K/2]; w_gate, w_up:
    packed E2M1 [N, K/2] with f32 row scales s_gate, s_up.  Returns uint8 [M, N/2]."""
    M = a.shape[0]
    N = w_gate.shape[0]
    K = K if K is not None else 2 * a.shape[1]
    if h_packed is None:
        h_packed = torch.empty((M, N // 2), dtype=torch.uint8, device=a.device)
    d = L.fp4_swiglu_desc()
    d.M, d.N, d.K = M, N, K
    d.a, d.lda, d.a_scale = a.data_ptr(), _ld(a), a_scale.data_ptr()
    d.w_gate, d.w_up, d.ldw = w_gate.data_ptr(), w_up.data_ptr(), _ld(w_gate)
    d.s_gate, d.s_up = s_gate.data_ptr(), s_up.data_ptr()
    d.out_scale = out_scale.data_ptr()
    d.out_shift = out_shift.data_ptr() if out_shift is not None else None
    d.h_packed, d.ldh = h_packed.data_ptr(), _ld(h_packed)
    L.check(L.lib().fp4_gemm_swiglu_quant(ctypes.byref(d), _stream(a.device)), "fp4_gemm_swiglu_quant")
    return h_packed

"""Checkpoint of a quantized tensor as a NumPy .npz archive.

Saving a quantized model keeps the packed codes together with everything needed to
decode and use them ("为什么我们需要4-bit浮点量化？" page, section 3.3, saving and
loading the quantized model): the scales, the grid (minifloat e/m, lookup table or the
two-mode grid), the scale granularity, the pre-shift's column shifts and activation scale
where there are any, and the format / clip search records that chose the grid.

Only plain arrays are stored (no Python objects), and `load_quantized` reads the archive
with `allow_pickle=False`, so loading a file runs no code from it.  Search records are
kept as the raw bytes of `fp4_search_result` (the layout `include/fp4.h` declares) and
decoded with the same ctypes structure on load.
"""
import ctypes

import numpy as np
import torch

from . import _lib as L

FORMAT_VERSION = 1


def _host(t):
    return None if t is None else t.detach().to("cpu").contiguous().numpy()


def save_quantized(path, packed: torch.Tensor, scales: torch.Tensor, grid: L.fp4_grid, gran: L.fp4_gran,
                   shift: torch.Tensor | None = None, act_scale: torch.Tensor | None = None,
                   records: torch.Tensor | None = None) -> None:
    """Write one quantized tensor: packed codes [rows, bytes] (uint8), its scales, grid,
    granularity and the optional pre-shift column shifts (int8), activation scale (f32)
    and search records (the uint8 buffer the search entry points fill)."""
    if packed.dtype != torch.uint8 or packed.dim() != 2:
        raise ValueError("packed must be a 2-D uint8 tensor")
    if scales.dtype not in (torch.float16, torch.float32):
        raise ValueError("scales must be float16 or float32")
    arrays = {
        "format_version": np.array([FORMAT_VERSION], np.int32),
        "codes": _host(packed),
        "scales": _host(scales).reshape(-1),
        "grid": np.array([grid.kind, grid.e, grid.m, grid.reserved], np.int32),
        "grid_lut": np.array(list(grid.lut), np.float32),
        "gran": np.array([gran.mode, gran.group, gran.scale_dtype, gran.reserved], np.int32),
    }
    if shift is not None:
        if shift.dtype != torch.int8:
            raise ValueError("shift must be int8")
        arrays["col_shift"] = _host(shift).reshape(-1)
    if act_scale is not None:
        arrays["act_scale"] = _host(act_scale).astype(np.float32).reshape(-1)
    if records is not None:
        raw = _host(records).view(np.uint8).reshape(-1)
        if raw.size % ctypes.sizeof(L.fp4_search_result):
            raise ValueError("records must hold whole fp4_search_result entries")
        arrays["search_records"] = raw
    np.savez(path, **arrays)


def load_quantized(path, device="cpu") -> dict:
    """Read an archive written by `save_quantized`.  Returns a dict with "packed",
    "scales" (tensors on `device`), "grid" (fp4_grid), "gran" (fp4_gran) and, when
    stored, "shift", "act_scale" (tensors) and "records" (a list of fp4_search_result)."""
    with np.load(path, allow_pickle=False) as z:
        if int(z["format_version"][0]) != FORMAT_VERSION:
            raise ValueError(f"unsupported checkpoint format {int(z['format_version'][0])}")
        g = L.fp4_grid()
        g.kind, g.e, g.m, g.reserved = (int(v) for v in z["grid"])
        for i, v in enumerate(z["grid_lut"]):
            g.lut[i] = float(v)
        gr = L.fp4_gran()
        gr.mode, gr.group, gr.scale_dtype, gr.reserved = (int(v) for v in z["gran"])
        out = {"packed": torch.from_numpy(z["codes"].copy()).to(device),
               "scales": torch.from_numpy(z["scales"].copy()).to(device), "grid": g, "gran": gr}
        if "col_shift" in z:
            out["shift"] = torch.from_numpy(z["col_shift"].copy()).to(device)
        if "act_scale" in z:
            out["act_scale"] = torch.from_numpy(z["act_scale"].copy()).to(device)
        if "search_records" in z:
            raw = z["search_records"].tobytes()
            n = ctypes.sizeof(L.fp4_search_result)
            out["records"] = [L.fp4_search_result.from_buffer_copy(raw[i:i + n]) for i in range(0, len(raw), n)]
    return out

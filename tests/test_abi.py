"""C-ABI checks that need no GPU: the library loads, exports every symbol the header
declares with the struct layouts the header defines, and rejects bad arguments on the
host with the documented status codes before anything is launched."""
import ctypes
import os
import re
import subprocess

import pytest

from bit_floating_point_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp4_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = L.load()
    names = _declared_functions()
    assert len(names) == 14, names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.SIGNATURES)


def test_struct_layouts_match_header(tmp_path):
    src = tmp_path / "sz.c"
    src.write_text('#include "fp4.h"\n#include <stdio.h>\n#include <stddef.h>\n'
                   'int main(void){printf("%zu %zu %zu %zu %zu %zu %zu\\n", sizeof(fp4_grid), sizeof(fp4_gran),'
                   ' sizeof(fp4_search_result), sizeof(fp4_gemm_desc), offsetof(fp4_gemm_desc, a_scale),'
                   ' offsetof(fp4_gemm_desc, w_gran), offsetof(fp4_gemm_desc, y_dtype));'
                   ' printf("%zu %zu %zu\\n", sizeof(fp4_swiglu_desc), offsetof(fp4_swiglu_desc, out_shift),'
                   ' offsetof(fp4_swiglu_desc, ldh)); return 0;}\n')
    exe = tmp_path / "sz"
    subprocess.check_call(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    got = [int(v) for v in subprocess.check_output([str(exe)]).split()]
    want = [ctypes.sizeof(L.fp4_grid), ctypes.sizeof(L.fp4_gran), ctypes.sizeof(L.fp4_search_result),
            ctypes.sizeof(L.fp4_gemm_desc), L.fp4_gemm_desc.a_scale.offset, L.fp4_gemm_desc.w_gran.offset,
            L.fp4_gemm_desc.y_dtype.offset, ctypes.sizeof(L.fp4_swiglu_desc), L.fp4_swiglu_desc.out_shift.offset,
            L.fp4_swiglu_desc.ldh.offset]
    assert got == want


def test_nf4_grid_matches_oracle_table():
    """The library's host NF4 table (bisection on erfc, manual binary16 rounding) equals
    the oracle's (scipy's ndtri, numpy's binary16 cast): two independent computations of
    the same closed form."""
    import numpy as np
    import oracle as O
    lib = L.load()
    g = L.fp4_grid()
    assert lib.fp4_nf4_grid(ctypes.byref(g)) == L.FP4_OK
    assert g.kind == L.FP4_GRID_LUT16 and g.e == 0 and g.m == 0 and g.reserved == 0
    got = np.array(list(g.lut), dtype=np.float64)
    assert np.array_equal(got, O.nf4_table())
    assert got[0] == -1.0 and got[-1] == 1.0 and np.array_equal(got, -got[::-1])
    assert lib.fp4_nf4_grid(None) == L.FP4_ERR_INVALID_ARG


def test_search_static_rejects_before_launch():
    lib = L.load()
    fm = (ctypes.c_int32 * 6)(1, 2, 2, 1, 3, 0)
    # 64 tensors of 2^24 values need more than the 16 MiB static scratch
    st = lib.fp4_search_format_static(FAKE, 64, 1 << 24, fm, 3, 100, 0.5, 1.0, FAKE, FAKE, None)
    assert st == L.FP4_ERR_WORKSPACE and b"16777216" in lib.fp4_last_error()
    assert lib.fp4_search_format_static(None, 1, 1024, fm, 3, 100, 0.5, 1.0, FAKE, FAKE, None) == L.FP4_ERR_INVALID_ARG
    assert lib.fp4_search_format_static(FAKE, 1, 1000, fm, 3, 100, 0.5, 1.0, FAKE, FAKE, None) == L.FP4_ERR_INVALID_ARG
    assert lib.fp4_search_format_static(ODD, 1, 1024, fm, 3, 100, 0.5, 1.0, FAKE, FAKE, None) == L.FP4_ERR_ALIGNMENT


def test_split_limit_hook_accepts_any_value():
    lib = L.load()
    for v in (0, -5, 4096, 1 << 40):
        assert lib.fp4_set_split_limit(v) == L.FP4_OK
    assert lib.fp4_set_split_limit(0) == L.FP4_OK


def test_status_strings():
    lib = L.load()
    assert lib.fp4_status_string(0) == b"FP4_OK"
    assert lib.fp4_status_string(4) == b"FP4_ERR_WORKSPACE"


# ---- host-side validation (no launch happens for any of these) ----
FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: every call below is rejected first
ODD = ctypes.c_void_p(0x10004)


def _grid(kind=0, e=2, m=1):
    g = L.fp4_grid()
    g.kind, g.e, g.m = kind, e, m
    return g


def _gran(mode=0, group=0, sd=0):
    g = L.fp4_gran()
    g.mode, g.group, g.scale_dtype = mode, group, sd
    return g


def test_quantize_validation():
    lib = L.load()
    q = lib.fp4_quantize_pack
    N = ctypes.c_void_p(0)
    assert q(N, 0, 4, 8, 8, _grid(), _gran(), N, N, N, FAKE, 4, FAKE, N) == L.FP4_ERR_INVALID_ARG
    assert b"null" in lib.fp4_last_error()
    assert q(FAKE, 0, 4, 7, 8, _grid(), _gran(), N, N, N, FAKE, 4, FAKE, N) == L.FP4_ERR_INVALID_ARG  # odd cols
    assert q(FAKE, 0, 4, 8, 8, _grid(0, 2, 2), _gran(), N, N, N, FAKE, 4, FAKE, N) == L.FP4_ERR_UNSUPPORTED
    assert q(FAKE, 0, 4, 8, 8, _grid(0, 0, 3), _gran(), N, N, N, FAKE, 4, FAKE, N) == L.FP4_ERR_UNSUPPORTED
    assert q(FAKE, 0, 4, 8, 8, _grid(7), _gran(), N, N, N, FAKE, 4, FAKE, N) == L.FP4_ERR_INVALID_ARG
    assert q(FAKE, 0, 4, 96, 96, _grid(), _gran(2, 64), N, N, N, FAKE, 48, FAKE, N) == L.FP4_ERR_INVALID_ARG
    assert q(FAKE, 0, 4, 96, 96, _grid(), _gran(2, 24), N, N, N, FAKE, 48, FAKE, N) == L.FP4_ERR_UNSUPPORTED
    assert q(FAKE, 0, 4, 8, 8, _grid(), _gran(0, 0, 2), N, N, N, FAKE, 4, FAKE, N) == L.FP4_ERR_UNSUPPORTED
    assert q(ODD, 0, 4, 8, 8, _grid(), _gran(), N, N, N, FAKE, 4, FAKE, N) == L.FP4_ERR_ALIGNMENT
    assert q(FAKE, 0, 4, 8, 8, _grid(), _gran(), N, N, N, FAKE, 4, N, N) == L.FP4_ERR_INVALID_ARG
    assert q(FAKE, 5, 4, 8, 8, _grid(), _gran(), N, N, N, FAKE, 4, FAKE, N) == L.FP4_ERR_INVALID_ARG
    lut = _grid(1)
    for i in range(16):
        lut.lut[i] = i * 0.1  # not binary16-exact
    assert q(FAKE, 0, 4, 8, 8, lut, _gran(), N, N, N, FAKE, 4, FAKE, N) == L.FP4_ERR_INVALID_ARG


def test_calibrate_validation():
    lib = L.load()
    c = lib.fp4_calibrate
    N = ctypes.c_void_p(0)
    assert c(N, 0, 4, 8, 8, 0, 0, 0, FAKE, N) == L.FP4_ERR_INVALID_ARG
    assert c(FAKE, 0, 4, 8, 4, 0, 0, 0, FAKE, N) == L.FP4_ERR_INVALID_ARG  # ld < cols
    assert c(FAKE, 0, 4, 8, 8, 9, 0, 0, FAKE, N) == L.FP4_ERR_INVALID_ARG
    assert c(FAKE, 0, 4, 8, 8, 2, 6, 0, FAKE, N) == L.FP4_ERR_UNSUPPORTED
    assert c(ODD, 0, 4, 8, 8, 0, 0, 0, FAKE, N) == L.FP4_ERR_ALIGNMENT


def test_search_validation():
    lib = L.load()
    s = lib.fp4_search_format
    N = ctypes.c_void_p(0)
    fm = (ctypes.c_int32 * 6)(1, 2, 2, 1, 3, 0)
    need = lib.fp4_search_workspace_size(2, 1024, 3, 100)
    assert need > 0
    assert s(FAKE, 2, 1024, fm, 3, 100, 0.5, 1.0, FAKE, FAKE, FAKE, need - 1, N) == L.FP4_ERR_WORKSPACE
    assert s(FAKE, 2, 1024, fm, 3, 100, 0.5, 1.0, FAKE, FAKE, N, need, N) == L.FP4_ERR_WORKSPACE
    assert s(FAKE, 2, 1000, fm, 3, 100, 0.5, 1.0, FAKE, FAKE, FAKE, need, N) == L.FP4_ERR_INVALID_ARG
    assert s(FAKE, 2, 1024, fm, 3, 1, 0.5, 1.0, FAKE, FAKE, FAKE, need, N) == L.FP4_ERR_UNSUPPORTED
    assert s(FAKE, 2, 1024, fm, 3, 200, 0.5, 1.0, FAKE, FAKE, FAKE, need, N) == L.FP4_ERR_UNSUPPORTED
    assert s(FAKE, 2, 1024, fm, 3, 100, 0.0, 1.0, FAKE, FAKE, FAKE, need, N) == L.FP4_ERR_INVALID_ARG
    bad = (ctypes.c_int32 * 2)(2, 2)
    assert s(FAKE, 2, 1024, bad, 1, 100, 0.5, 1.0, FAKE, FAKE, FAKE, need, N) == L.FP4_ERR_UNSUPPORTED


def test_search_activations_validation():
    lib = L.load()
    f = lib.fp4_search_activations
    N = ctypes.c_void_p(0)
    fm = (ctypes.c_int32 * 6)(1, 2, 2, 1, 3, 0)
    need = lib.fp4_search_workspace_size(64, 1024, 3, 100)
    ok = dict(x=FAKE, dt=L.FP4_BF16, rows=64, cols=1024, ldx=1024, unit=L.FP4_SCALE_ROW, first=0, fm=fm, nf=3,
              nc=100, lo=0.5, hi=1.0, res=FAKE, packed=FAKE, ldp=512, ws=FAKE, wsb=need)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["dt"], a["rows"], a["cols"], a["ldx"], a["unit"], a["first"], a["fm"], a["nf"], a["nc"],
                 a["lo"], a["hi"], a["res"], a["packed"], a["ldp"], a["ws"], a["wsb"], N)

    assert call(x=N) == L.FP4_ERR_INVALID_ARG
    assert call(dt=L.FP4_F16) == L.FP4_ERR_INVALID_ARG
    assert call(cols=1000, ldx=1000, ldp=512) == L.FP4_ERR_INVALID_ARG     # cols % 16
    assert call(ldx=1026) == L.FP4_ERR_ALIGNMENT
    assert call(ldp=514) == L.FP4_ERR_ALIGNMENT
    assert call(ldp=256) == L.FP4_ERR_ALIGNMENT                            # ldp < cols/2
    assert call(unit=L.FP4_SCALE_GROUP) == L.FP4_ERR_INVALID_ARG
    assert call(nc=1) == L.FP4_ERR_UNSUPPORTED
    assert call(x=ODD) == L.FP4_ERR_ALIGNMENT
    assert call(wsb=need - 1) == L.FP4_ERR_WORKSPACE
    # TENSOR over the first 16 rows needs the workspace of one unit of 16 x 1024 values
    need_t = lib.fp4_search_workspace_size(1, 16 * 1024, 3, 100)
    assert call(unit=L.FP4_SCALE_TENSOR, first=16, wsb=need_t - 1) == L.FP4_ERR_WORKSPACE
    assert call(rows=0) == L.FP4_OK  # empty: nothing launched


def test_gemm_validation():
    lib = L.load()
    N = ctypes.c_void_p(0)
    assert lib.fp4_gemm(None, N) == L.FP4_ERR_INVALID_ARG
    d = L.fp4_gemm_desc()
    d.M, d.N, d.K = 16, 32, 256
    d.a_kind = L.FP4_PACKED
    d.a, d.lda, d.w, d.ldw, d.w_scales, d.y, d.ldy = 0x10000, 128, 0x20000, 128, 0x30000, 0x40000, 32
    d.a_grid, d.w_grid = _grid(), _grid()
    d.w_gran = _gran(1)
    d.y_dtype = L.FP4_BF16
    assert lib.fp4_gemm(ctypes.byref(d), N) == L.FP4_ERR_INVALID_ARG  # no a_scale
    d.a_scale = 0x50000
    d.a_grid = _grid(0, 1, 2)
    d.w_gran = _gran(2, 64)
    assert lib.fp4_gemm(ctypes.byref(d), N) == L.FP4_ERR_UNSUPPORTED  # E1M2 activations, group weight scales
    d.w_gran = _gran(1)
    d.a_grid = _grid()
    d.w_gran = _gran(2, 64)
    assert lib.fp4_gemm(ctypes.byref(d), N) == L.FP4_ERR_UNSUPPORTED  # E2M1 x E2M1 with group scales
    d.w_gran = _gran(1)
    d.ldw = 100
    assert lib.fp4_gemm(ctypes.byref(d), N) == L.FP4_ERR_INVALID_ARG  # ldw < K/2
    d.ldw = 136
    assert lib.fp4_gemm(ctypes.byref(d), N) == L.FP4_ERR_ALIGNMENT
    d.ldw = 128
    d.y_dtype = 7
    assert lib.fp4_gemm(ctypes.byref(d), N) == L.FP4_ERR_INVALID_ARG
    d.y_dtype = L.FP4_BF16
    d.a_scale_mode = 5
    assert lib.fp4_gemm(ctypes.byref(d), N) == L.FP4_ERR_INVALID_ARG
    d.a_scale_mode = L.FP4_SCALE_ROW  # per-token activation scales: minifloat weights only
    d.w_grid, d.w_gran = _grid(1), _gran(2, 64)
    for i in range(16):
        d.w_grid.lut[i] = (i - 7.5) / 8
    assert lib.fp4_gemm(ctypes.byref(d), N) == L.FP4_ERR_UNSUPPORTED


def test_swiglu_validation():
    lib = L.load()
    N = ctypes.c_void_p(0)
    assert lib.fp4_gemm_swiglu_quant(None, N) == L.FP4_ERR_INVALID_ARG
    d = L.fp4_swiglu_desc()
    d.M, d.N, d.K = 16, 64, 256
    d.a, d.lda, d.a_scale = 0x10000, 128, 0x18000
    d.w_gate, d.w_up, d.ldw = 0x20000, 0x28000, 128
    d.s_gate, d.s_up, d.out_scale = 0x30000, 0x38000, 0x40000
    d.h_packed, d.ldh = 0x50000, 32
    d.N = 48
    assert lib.fp4_gemm_swiglu_quant(ctypes.byref(d), N) == L.FP4_ERR_UNSUPPORTED  # N % 32
    d.N, d.K = 64, 240
    assert lib.fp4_gemm_swiglu_quant(ctypes.byref(d), N) == L.FP4_ERR_UNSUPPORTED  # K % 32
    d.K = 116512
    assert lib.fp4_gemm_swiglu_quant(ctypes.byref(d), N) == L.FP4_ERR_UNSUPPORTED  # K too large for exact sums
    d.K = 256
    d.s_up = None
    assert lib.fp4_gemm_swiglu_quant(ctypes.byref(d), N) == L.FP4_ERR_INVALID_ARG
    d.s_up = 0x38000
    d.ldh = 16
    assert lib.fp4_gemm_swiglu_quant(ctypes.byref(d), N) == L.FP4_ERR_INVALID_ARG  # ldh < N/2
    d.ldh = 40
    assert lib.fp4_gemm_swiglu_quant(ctypes.byref(d), N) == L.FP4_ERR_ALIGNMENT
    d.ldh = 32
    d.w_up = 0x28004
    assert lib.fp4_gemm_swiglu_quant(ctypes.byref(d), N) == L.FP4_ERR_ALIGNMENT
    d.w_up = 0x28000
    d.M = 0
    assert lib.fp4_gemm_swiglu_quant(ctypes.byref(d), N) == L.FP4_OK  # empty: nothing launched


def test_two_mode_validation():
    lib = L.load()
    N = ctypes.c_void_p(0)
    tm = _grid(2)
    q = lib.fp4_quantize_pack
    assert q(FAKE, 0, 4, 256, 256, tm, _gran(1), N, N, N, FAKE, 128, FAKE, N) == L.FP4_ERR_UNSUPPORTED  # ROW
    assert q(FAKE, 0, 4, 256, 256, tm, _gran(2, 32), N, N, FAKE, FAKE, 128, FAKE, N) == L.FP4_ERR_UNSUPPORTED  # shifts
    assert lib.fp4_dequantize(FAKE, 4, 256, 128, tm, _gran(0), FAKE, N, FAKE, 256, N) == L.FP4_ERR_UNSUPPORTED
    f = lib.fp4_preshift_weights
    assert f(FAKE, 8, 256, 256, FAKE, _grid(), tm, _gran(2, 32), FAKE, FAKE, FAKE, 128, FAKE, N) == L.FP4_ERR_UNSUPPORTED
    d = L.fp4_gemm_desc()
    d.M, d.N, d.K = 16, 32, 256
    d.a_kind = L.FP4_PACKED
    d.a, d.lda, d.w, d.ldw, d.w_scales, d.y, d.ldy = 0x10000, 128, 0x20000, 128, 0x30000, 0x40000, 32
    d.a_scale = 0x50000
    d.a_grid, d.w_grid = _grid(), tm
    d.w_gran = _gran(2, 128)
    d.y_dtype = L.FP4_BF16
    assert lib.fp4_gemm(ctypes.byref(d), N) == L.FP4_ERR_UNSUPPORTED  # W4A4 with two-mode weights
    d.a_kind, d.lda = L.FP4_BF16, 256
    d.w_gran = _gran(1)
    assert lib.fp4_gemm(ctypes.byref(d), N) == L.FP4_ERR_UNSUPPORTED  # two-mode needs GROUP scales


def test_fp8_validation():
    lib = L.load()
    N = ctypes.c_void_p(0)
    g8 = _grid(0, 4, 3)
    q = lib.fp4_quantize_pack
    g6 = _grid(0, 2, 3)
    assert q(FAKE, 0, 4, 256, 256, g6, _gran(1), N, N, N, FAKE, 193, FAKE, N) == L.FP4_ERR_UNSUPPORTED  # FP6: odd ldp
    assert q(FAKE, 0, 4, 256, 256, g6, _gran(1), N, N, N, FAKE, 190, FAKE, N) == L.FP4_ERR_INVALID_ARG  # ldp < 192
    f = lib.fp4_preshift_weights  # FP8 weights: ldp below a row's 256 code bytes, then k % 8
    assert f(FAKE, 8, 256, 256, FAKE, g8, g8, _gran(1), FAKE, FAKE, FAKE, 128, FAKE, N) == L.FP4_ERR_INVALID_ARG
    assert f(FAKE, 8, 252, 256, FAKE, g8, g8, _gran(1), FAKE, FAKE, FAKE, 256, FAKE, N) == L.FP4_ERR_UNSUPPORTED
    assert q(FAKE, 0, 4, 252, 256, g8, _gran(1), N, N, N, FAKE, 256, FAKE, N) == L.FP4_ERR_UNSUPPORTED  # cols % 8
    assert q(FAKE, 0, 4, 256, 256, g8, _gran(2, 32), N, N, N, FAKE, 128, FAKE, N) == L.FP4_ERR_INVALID_ARG  # ldp
    assert q(FAKE, 0, 4, 256, 256, _grid(0, 3, 4), _gran(2, 32), N, N, N, FAKE, 256, FAKE, N) == L.FP4_ERR_UNSUPPORTED
    d = L.fp4_gemm_desc()
    d.M, d.N, d.K = 16, 32, 256
    d.a_kind = L.FP4_PACKED
    d.a, d.lda, d.w, d.ldw, d.w_scales, d.y, d.ldy = 0x10000, 128, 0x20000, 256, 0x30000, 0x40000, 32
    d.a_scale = 0x50000
    d.a_grid, d.w_grid = _grid(0, 1, 2), g8
    d.w_gran = _gran(1)
    d.y_dtype = L.FP4_BF16
    d.lda = 120
    assert lib.fp4_gemm(ctypes.byref(d), N) == L.FP4_ERR_ALIGNMENT  # E1M2 activation rows below K/2 bytes
    d.lda = 128
    # W6A6 (FP6 E2M3 x FP6 E2M3): rows of 256 codes are 192 bytes
    g6 = _grid(0, 2, 3)
    d.a_grid, d.w_grid, d.lda, d.ldw = g6, g6, 192, 192
    d.K = 240
    assert lib.fp4_gemm(ctypes.byref(d), N) == L.FP4_ERR_UNSUPPORTED  # K not a multiple of 32
    d.K, d.lda = 256, 176
    assert lib.fp4_gemm(ctypes.byref(d), N) == L.FP4_ERR_ALIGNMENT  # lda below a row's code bytes
    d.lda, d.w_gran = 192, _gran(2, 32)
    assert lib.fp4_gemm(ctypes.byref(d), N) == L.FP4_ERR_UNSUPPORTED  # GROUP of 32: below one instruction's 64 codes
    d.K, d.lda, d.ldw, d.w_gran = 320, 240, 240, _gran(2, 128)
    assert lib.fp4_gemm(ctypes.byref(d), N) == L.FP4_ERR_INVALID_ARG  # a group of 128 does not divide K = 320
    d.K, d.lda, d.ldw = 256, 192, 192
    d.w_gran, d.a_scale = _gran(1), 0
    assert lib.fp4_gemm(ctypes.byref(d), N) == L.FP4_ERR_INVALID_ARG  # no activation scale
    d.a_scale, d.a_grid = 0x50000, _grid(0, 3, 4)
    assert lib.fp4_gemm(ctypes.byref(d), N) == L.FP4_ERR_UNSUPPORTED  # E3M4 is no grid
    d.a_grid, d.w_grid, d.lda, d.ldw = g6, g8, 192, 256
    d.a_kind, d.lda, d.ldw = L.FP4_BF16, 256, 128
    assert lib.fp4_gemm(ctypes.byref(d), N) == L.FP4_ERR_INVALID_ARG  # ldw < K


def test_preshift_validation():
    lib = L.load()
    N = ctypes.c_void_p(0)
    f = lib.fp4_preshift_weights
    assert f(FAKE, 8, 16, 16, FAKE, _grid(), _grid(), _gran(0), FAKE, FAKE, FAKE, 8, FAKE, N) == L.FP4_ERR_UNSUPPORTED
    assert f(FAKE, 8, 16, 16, N, _grid(), _grid(), _gran(1), FAKE, FAKE, FAKE, 8, FAKE, N) == L.FP4_ERR_INVALID_ARG
    assert f(ODD, 8, 16, 16, FAKE, _grid(), _grid(), _gran(1), FAKE, FAKE, FAKE, 8, FAKE, N) == L.FP4_ERR_ALIGNMENT


def test_binding_refuses_missing_library(tmp_path):
    with pytest.raises(ImportError):
        L.load(str(tmp_path / "missing.so"))

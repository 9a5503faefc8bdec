"""Parity of the HIP library (through its C ABI) against the CPU oracle.

Bar: codes, packed bytes, scales, shifts and search records bit-exact; W4A4 E2M1
outputs bit-exact (fp32 accumulation of FP4 products is exact); other GEMM outputs
(_check_gemm) within normwise max relative error 1e-3 of the binary64 oracle AND every
output element within its derived rounding bound |y32 - r| <= d * 2^-24 * S (S = the
same product over magnitudes, d = the number of binary32 roundings on the path from a
product to the output; the NF4 product adds the binary16 rounding of its expanded
weights), with the bf16 output equal to the round-to-nearest-even of the fp32 output and
within one bf16 ulp of RNE_bf16(r) wherever the fp32 bound is below a quarter ulp.
Sizes span several tiles with ragged tails; full workload sizes are checked on sampled
rows.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth

pytestmark = pytest.mark.gpu

F = pytest.importorskip("bit_floating_point_amd")
DEV = "cuda"
TOL = 1e-3


def dev(x, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(dtype)


def host(t):
    return t.detach().cpu().numpy()


def grids(fmt):
    if fmt == "nf4":
        return O.nf4(), F.grid_nf4()
    return O.minifloat(*fmt), F.grid_minifloat(*fmt)


def say(*a):
    print(*a, flush=True)


def _bf16_bits(t):
    return host(t.view(torch.int16)).view(np.uint16)


# Rounding depth d (see oracle.U32 and the module docstring) of each product family.
def depth_w4a16(K, unit):
    """W4A16 / W8A16 / W6A16 (exact products of a bf16 or binary32 activation and a
    4/6/8-bit grid value): at most unit - 1 additions inside a scale unit (the matrix-
    core chain, or a fused multiply-add chain), one rounding where a unit's partial sum is
    scaled and added (fused), at most K / unit of those, at most 8 additions combining
    the partial sums of K ranges and one final scaling; unit = the group, or K."""
    return unit + K // unit + 9


def depth_packed(K):
    """Two packed operands on the f8f6f4 / f16 matrix cores: at most K additions of
    partial sums, whether rounded to nearest or truncated (2 u each), and the roundings
    of fl32(a * s_n) and of the final product."""
    return 2 * K + 4


# The f8f6f4 matrix instruction sums each group of 8 consecutive products of a K block
# on a fixed-point grid whose least bit is 2^-13 of the group's largest product (2^E,
# E its binary exponent), dropping product bits below it (toward zero); measured with
# one-hot FP8 operands: 1 + 2^-13 is kept and 1 + 2^-14 is not, 448^2 + 16 is kept and
# 448^2 + 4 is not, 1 - 2^-14 gives 1, and 1 + 63 * 2^-k (k >= 14) gives 1 + 56 * 2^-k
# (the 7 small products sharing the group of the 1 are lost, the other 56 are not).
# A group of 8 then loses less than 7 * 2^(E - 13) <= 7 * 2^-13 * (its magnitude sum).
# Products that are multiples of 2^(E - 13) lose nothing: every E2M1 x E2M1, E2M3 x
# E2M3 and E2M3 x E2M1 product (multiples of 2^-6 at most 56.25 in magnitude), so those
# pairs are exact.  E1M2 values are multiples of 2^-2 below 2, E3M0 values powers of two
# from 1 to 64: their products with each other, with E2M1 and with E2M3 are multiples of
# 2^-5 no larger than 480 (2^-5 >= 2^(8 - 13)), exact too.  FP8 and E3M2 operands span
# more binades and can lose bits.
WINDOW_LOSS = 7 * 2.0 ** -13


def packed_window_term(af, wf, S):
    """The extra bound of the matrix instruction's product window (zero for the pairs
    whose products it keeps exactly)."""
    exact = {(2, 1), (2, 3), (1, 2), (3, 0)}
    return 0.0 if (tuple(af) in exact and tuple(wf) in exact) else WINDOW_LOSS * np.asarray(S, np.float64)


def _check_gemm(y32, r, S, d, yb=None, extra=0.0):
    """Normwise 1e-3, the elementwise bound d * u * S + extra, and the bf16 output rules."""
    bound = d * O.U32 * np.asarray(S, np.float64) + extra
    err = O.rel_err(y32, r)
    ex = O.elementwise_excess(y32, r, bound)
    say(f"  rel err {err:.3e}, elementwise bound used {ex:.3f} (d = {d})")
    assert err <= TOL
    assert ex <= 1.0
    if yb is not None:
        bits = yb if isinstance(yb, np.ndarray) else _bf16_bits(yb)
        assert np.array_equal(bits, O.rne_bf16_bits(y32))
        ulps, n = O.bf16_ulps_from_rounded(bits, r, bound)
        say(f"  bf16 within {ulps} ulp of RNE(r) on {n} of {np.size(r)} outputs")
        assert ulps <= 1


def _nf4_extra(ap, a, wscales, S, group):
    """The NF4 product's additional bound: each expanded weight carries two binary16
    roundings (2^-10 + 2^-22 relative) and, where it is subnormal in binary16, an absolute
    error below 2^-22 times its row's largest group scale."""
    e2 = O.minifloat(2, 1)
    A = np.abs(e2.decode(O.unpack(ap))).sum(axis=1).astype(np.float64) * abs(float(np.float32(a)))
    smax = np.abs(np.asarray(wscales, np.float32).astype(np.float64)).reshape(S.shape[1], -1).max(axis=1)
    return (2.0 ** -10 + 2.0 ** -22) * S + 2.0 ** -22 * A[:, None] * smax[None, :]


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    F._lib.lib()
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------- calibrate -------
@pytest.mark.parametrize("bf16", [True, False])
def test_calibrate(bf16):
    say("calibrate", bf16)
    x = synth.activations(3, 5, 300, 520, outlier_frac=0.01, bf16=bf16)
    xt = dev(x, torch.bfloat16 if bf16 else torch.float32)
    assert host(F.fp4_calibrate(xt, "tensor"))[0] == O.amax_tensor(x)
    assert np.array_equal(host(F.fp4_calibrate(xt, "column", first_rows=128)), O.amax_columns(x, 128))
    assert np.array_equal(host(F.fp4_calibrate(xt, "row_group", group=8)), O.amax_row_groups(x, 8).reshape(-1))
    x2 = x[:, :512]
    xt2 = dev(x2, torch.bfloat16 if bf16 else torch.float32)
    assert np.array_equal(host(F.fp4_calibrate(xt2, "row_group", group=64)), O.amax_row_groups(x2, 64).reshape(-1))


# ---------------------------------------------------------------- quantize --------
FMTS = [(2, 1), (1, 2), (3, 0), "nf4"]
MODES = [("tensor", 0, "f32"), ("row", 0, "f32"), ("row", 0, "f16"), ("group", 128, "f16"),
         ("group", 128, "f32"), ("group", 64, "f32"), ("group", 8, "f32"), ("group", 512, "f32")]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("mode,group,sd", MODES)
@pytest.mark.parametrize("bf16", [False, True])
def test_quantize_pack_dequantize(fmt, mode, group, sd, bf16):
    say("quantize", fmt, mode, group, sd, bf16)
    # group: 3072 = one whole 2048-column chunk and a partial one; 1030: ragged
    # 8-element tail, scalar path
    cols = 3072 if mode == "group" else 1030
    x = synth.heavy_tail_weight(2, 7, 37, cols)
    if bf16:
        x = synth.to_bf16_values(x)
    x[3, :] = 0.0  # an all-zero row / group
    og, fg = grids(fmt)
    packed, scales = O.quantize_pack(x, og, mode, group, sd)
    g = F.gran(mode, group, sd)
    gp, gs = F.fp4_quantize_pack(dev(x, torch.bfloat16 if bf16 else torch.float32), fg, g)
    assert np.array_equal(host(gp), packed)
    assert np.array_equal(host(gs).view(np.uint16 if sd == "f16" else np.uint32),
                          scales.reshape(-1).view(np.uint16 if sd == "f16" else np.uint32))
    deq = O.dequantize(packed, og, mode, scales, group)
    gd = F.fp4_dequantize(gp, fg, g, gs)
    assert np.array_equal(host(gd).view(np.uint32), deq.view(np.uint32))


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_bit_pattern_sweep(fmt):
    """2^22 binary32 bit patterns spread over the whole encoding space (finite values
    only), quantized at scale 1: every code must match the brute-force oracle."""
    say("sweep", fmt)
    u = (np.arange(1 << 22, dtype=np.uint64) * 1021 + 12345) % (1 << 32)
    x = u.astype(np.uint32).view(np.float32)
    x = x[np.isfinite(x)]
    x = x[: (x.size // 1024) * 1024].reshape(-1, 1024)
    og, fg = grids(fmt)
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    gp, _ = F.fp4_quantize_pack(dev(x), fg, F.gran("tensor"), tensor_scale=one)
    want = O.pack(O.quantize(x, np.float32(1), og))
    assert np.array_equal(host(gp), want)


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_full_sweep(fmt):
    """Every finite binary32 bit pattern (2^32 - 2^24 of them: all but exponent 255),
    quantized at scale 1 by the library and by the brute-force oracle, in 128 chunks of
    2^25 consecutive patterns: every packed byte equal."""
    say("full sweep", fmt)
    og, fg = grids(fmt)
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    CH = 1 << 25
    done = 0
    for c in range(128):
        u = np.arange(c * CH, (c + 1) * CH, dtype=np.uint64).astype(np.uint32)
        if c % 64 == 63:
            u = u[:3 << 23]  # the last chunk of each sign holds exponents 252..255: drop 255
        x = u.view(np.float32).reshape(-1, 1024)
        gp, _ = F.fp4_quantize_pack(torch.from_numpy(x).to(DEV), fg, F.gran("tensor"), tensor_scale=one)
        want = O.pack(O.quantize(x, np.float32(1), og))
        got = host(gp)
        if not np.array_equal(got, want):
            i = np.argwhere(got != want)[0]
            raise AssertionError(f"chunk {c}: first difference at pattern "
                                 f"{int(u[i[0] * 1024 + 2 * i[1]]):#010x}: {got[tuple(i)]:#04x} vs {want[tuple(i)]:#04x}")
        done += u.size
        if c % 32 == 31:
            say(f"  {done} patterns")
    assert done == (1 << 32) - (1 << 24)


def test_quantize_edge_cases():
    og, fg = grids((2, 1))
    z = torch.zeros((0, 64), device=DEV)
    p, s = F.fp4_quantize_pack(z, fg, F.gran("row"))
    assert p.shape == (0, 32)
    x = np.zeros((4, 64), dtype=np.float32)
    x[1] = -0.0
    gp, gs = F.fp4_quantize_pack(dev(x), fg, F.gran("tensor"))
    assert np.array_equal(host(gp), O.quantize_pack(x, og, "tensor")[0]) and host(gs)[0] == 0
    tiny = np.full((2, 16), 1e-40, dtype=np.float32)
    tiny[1] *= -1
    gp, gs = F.fp4_quantize_pack(dev(tiny), fg, F.gran("row"))
    p, s = O.quantize_pack(tiny, og, "row")
    assert np.array_equal(host(gp), p) and np.array_equal(host(gs), s)


# ---------------------------------------------------------------- W4A16 -----------
def test_tiny_round_trip():
    """4-bit FP round trip on a 256x256 N(0, 0.02) matrix with one per-tensor scale,
    then an 8x256 fp32-activation GEMM."""
    w, x = synth.tiny()
    og, fg = grids((2, 1))
    packed, scales = O.quantize_pack(w, og, "tensor")
    assert packed.shape == (256, 128)
    gp, gs = F.fp4_quantize_pack(dev(w), fg, F.gran("tensor"))
    assert np.array_equal(host(gp), packed) and host(gs)[0] == scales[0]
    gd = F.fp4_dequantize(gp, fg, F.gran("tensor"), gs)
    assert np.array_equal(host(gd), O.dequantize(packed, og, "tensor", scales))
    r = O.gemm_w4a16(x, packed, og, "tensor", scales)
    S = O.gemm_w4a16(x, packed, og, "tensor", scales, absolute=True)
    y32 = F.fp4_gemm(dev(x), gp, gs, fg, F.gran("tensor"), y_dtype=torch.float32)
    yb = F.fp4_gemm(dev(x), gp, gs, fg, F.gran("tensor"), y_dtype=torch.bfloat16)
    _check_gemm(host(y32), r, S, depth_w4a16(256, 256), yb)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_w4a16_decode_full(M):
    """LLaMA-7B MLP linear 11008x4096, E2M1 with fp16 scales per 128 along K, bf16
    activations: full-size weight codes bit-exact, every output within tolerance."""
    say("w4a16", M)
    w = _decode_weight()
    og, fg = grids((2, 1))
    packed, scales = _decode_packed()
    g = F.gran("group", 128, "f16")
    gp, gs = F.fp4_quantize_pack(dev(w), fg, g)
    assert np.array_equal(host(gp), packed)
    assert np.array_equal(host(gs).view(np.uint16), scales.reshape(-1).view(np.uint16))
    x = synth.decode_activations(M)
    r = O.gemm_w4a16(x, packed, og, "group", scales, group=128)
    S = O.gemm_w4a16(x, packed, og, "group", scales, group=128, absolute=True)
    xt = dev(x, torch.bfloat16)
    y32 = F.fp4_gemm(xt, gp, gs, fg, g, y_dtype=torch.float32)
    yb = F.fp4_gemm(xt, gp, gs, fg, g, y_dtype=torch.bfloat16)
    _check_gemm(host(y32), r, S, depth_w4a16(4096, 128), yb)


_cache = {}


def _decode_weight():
    if "w" not in _cache:
        _cache["w"] = synth.decode_weight()
    return _cache["w"]


def _decode_packed():
    if "p" not in _cache:
        _cache["p"] = O.quantize_pack(_decode_weight(), O.minifloat(2, 1), "group", 128, "f16")
    return _cache["p"]


@pytest.mark.parametrize("M,N,K,mode,group,fmt,bf16", [
    (5, 100, 384, "group", 128, (2, 1), True),     # MFMA path, ragged N and M
    (19, 70, 512, "group", 256, (2, 1), True),     # two chunks per group, M > 16
    (3, 48, 640, "row", 0, (2, 1), True),          # per-row scales
    (7, 33, 96, "group", 32, (2, 1), True),        # VALU path (group < 128)
    (4, 40, 256, "group", 64, "nf4", True),        # lookup grid, VALU path
    (6, 20, 128, "group", 64, (3, 0), False),      # f32 activations
])
def test_w4a16_shapes(M, N, K, mode, group, fmt, bf16):
    say("w4a16 shape", M, N, K, mode, group, fmt, bf16)
    w = synth.weight(2, 11, N, K)
    x = synth.activations(2, 12, M, K, bf16=bf16)
    og, fg = grids(fmt)
    sd = "f16" if mode == "group" and group == 128 else "f32"
    packed, scales = O.quantize_pack(w, og, mode, group, sd)
    g = F.gran(mode, group, sd)
    gp, gs = F.fp4_quantize_pack(dev(w), fg, g)
    assert np.array_equal(host(gp), packed)
    r = O.gemm_w4a16(x, packed, og, mode, scales, group=group)
    S = O.gemm_w4a16(x, packed, og, mode, scales, group=group, absolute=True)
    xt = dev(x, torch.bfloat16 if bf16 else torch.float32)
    y32 = F.fp4_gemm(xt, gp, gs, fg, g, y_dtype=torch.float32)
    yb = F.fp4_gemm(xt, gp, gs, fg, g, y_dtype=torch.bfloat16)
    _check_gemm(host(y32), r, S, depth_w4a16(K, group or K), yb)


@pytest.mark.parametrize("M,N,K,mode,sd", [
    (1, 100, 128, "group", "f16"),     # one K chunk: seven of eight wavefronts own no K
    (9, 61, 2176, "group", "f16"),     # 17 chunks: per-chunk scale loads, three tiles, ragged N
    (16, 100, 4096, "group", "f32"),   # f32 group scales as vector loads, M = 16
    (2, 50, 1024, "tensor", "f32"),    # one scale for the tensor
    (12, 70, 768, "row", "f32"),       # per-row scales, three tiles
    (8, 40, 8192, "group", "f16"),     # 128 KiB of staged activations
    (16, 40, 8192, "group", "f16"),    # too large to stage: the two-tile kernel
    (4, 1000, 4096, "group", "f16"),   # decode shape, many workgroups
    (1, 13000, 3072, "group", "f16"),  # three chunks per wavefront, ragged N
    (3, 700, 1024, "group", "f16"),    # one chunk per wavefront
    (2, 2000, 4096, "group", "f32"),   # f32 scales
    (4, 40, 2048, "group", "f16"),     # fewer workgroups than compute units
])
def test_w4a16_small_batch(M, N, K, mode, sd):
    """Decode / small-batch W4A16 (M <= 16, bf16 activations, E2M1): the staged-
    activation kernel across its geometry cases, within tolerance of the oracle, bf16
    output the rounding of the fp32 output."""
    say("w4a16 small", M, N, K, mode, sd)
    w = synth.weight(2, 13, N, K)
    x = synth.activations(2, 14, M, K, bf16=True)
    og, fg = grids((2, 1))
    group = 128 if mode == "group" else 0
    packed, scales = O.quantize_pack(w, og, mode, group, sd)
    g = F.gran(mode, group, sd)
    gp, gs = F.fp4_quantize_pack(dev(w), fg, g)
    assert np.array_equal(host(gp), packed)
    r = O.gemm_w4a16(x, packed, og, mode, scales, group=group)
    S = O.gemm_w4a16(x, packed, og, mode, scales, group=group, absolute=True)
    xt = dev(x, torch.bfloat16)
    y32 = F.fp4_gemm(xt, gp, gs, fg, g, y_dtype=torch.float32)
    yb = F.fp4_gemm(xt, gp, gs, fg, g, y_dtype=torch.bfloat16)
    _check_gemm(host(y32), r, S, depth_w4a16(K, group or K), yb)
    # a second call gives the same bits (no state carried between launches)
    y32b = F.fp4_gemm(xt, gp, gs, fg, g, y_dtype=torch.float32)
    assert np.array_equal(host(y32b).view(np.uint32), host(y32).view(np.uint32))


# ---------------------------------------------------------------- pre-shift + W4A4 --
def _preshift_chain(x, w, w_fmt="e2m1", group=64):
    """Oracle and GPU through calibrate -> pre-shift -> quantize -> GEMM; compares
    every intermediate bit for bit and returns (oracle pieces, gpu pieces)."""
    e2 = O.minifloat(2, 1)
    fe2 = F.grid_minifloat(2, 1)
    chan = O.amax_columns(x, 128)
    if w_fmt == "e2m1":
        k, a, wp, ws = O.preshift_weights(w, chan, e2, e2, "row")
        fw, fgran = fe2, F.gran("row")
    else:
        k, a, wp, ws = O.preshift_weights(w, chan, e2, O.nf4(), "group", group)
        fw, fgran = F.grid_nf4(), F.gran("group", group)
    ap, _ = O.quantize_activations(x, e2, a, k)
    xt = dev(x, torch.bfloat16)
    gchan = F.fp4_calibrate(xt, "column", first_rows=128)
    assert np.array_equal(host(gchan), chan)
    gk, ga, gwp, gws = F.fp4_preshift_weights(dev(w), gchan, fe2, fw, fgran)
    assert np.array_equal(host(gk), k)
    assert host(ga)[0] == a
    assert np.array_equal(host(gwp), wp)
    assert np.array_equal(host(gws), ws.reshape(-1))
    gap, _ = F.fp4_quantize_pack(xt, fe2, F.gran("tensor"), tensor_scale=ga, col_shift=gk)
    assert np.array_equal(host(gap), ap)
    return (k, a, wp, ws, ap), (gk, ga, gwp, gws, gap, fw, fgran)


@pytest.mark.parametrize("M,N,K,mode,group,sd,fmt", [
    (1, 100, 128, "group", 128, "f16", (1, 2)),    # staged-activation kernel, one K chunk
    (9, 61, 2176, "group", 128, "f16", (3, 0)),    # 17 chunks, ragged N
    (16, 100, 4096, "group", 128, "f32", (1, 2)),  # f32 group scales as vector loads
    (12, 70, 768, "row", 0, "f32", (3, 0)),        # per-row scales
    (4, 1000, 4096, "group", 128, "f16", (3, 0)),  # decode shape, many workgroups
    (19, 70, 512, "group", 256, "f32", (1, 2)),    # M > 16: the 16-row tile kernel, two chunks per group
    (40, 200, 1024, "tensor", 0, "f32", (3, 0)),   # M > 16, one scale
])
def test_w4a16_e1m2_e3m0_matrix_cores(M, N, K, mode, group, sd, fmt):
    """E1M2 / E3M0 weights with bf16 activations on the bf16 matrix-core kernels (each
    code decoded exactly to bf16 through the FP8 convert): codes bit-exact, the product
    within the bound of the binary64 oracle, bf16 output the rounding of the fp32 one."""
    say("w4a16 e1m2/e3m0", M, N, K, mode, group, sd, fmt)
    w = synth.weight(3, 15, N, K)
    x = synth.activations(3, 16, M, K, bf16=True)
    og, fg = grids(fmt)
    packed, scales = O.quantize_pack(w, og, mode, group, sd)
    g = F.gran(mode, group, sd)
    gp, gs = F.fp4_quantize_pack(dev(w), fg, g)
    assert np.array_equal(host(gp), packed)
    r = O.gemm_w4a16(x, packed, og, mode, scales, group=group)
    S = O.gemm_w4a16(x, packed, og, mode, scales, group=group, absolute=True)
    xt = dev(x, torch.bfloat16)
    y32 = F.fp4_gemm(xt, gp, gs, fg, g, y_dtype=torch.float32)
    yb = F.fp4_gemm(xt, gp, gs, fg, g, y_dtype=torch.bfloat16)
    _check_gemm(host(y32), r, S, depth_w4a16(K, group or K), yb)


@pytest.mark.parametrize("M,N,K", [(256, 384, 512), (200, 300, 544), (64, 96, 4096), (520, 1100, 1024)])
def test_preshift_w4a4_e2m1(M, N, K):
    say("w4a4", M, N, K)
    x = synth.activations(3, M, M, K, outlier_frac=0.01)
    w = synth.weight(3, N, N, K)
    (k, a, wp, ws, ap), (gk, ga, gwp, gws, gap, fw, fgran) = _preshift_chain(x, w)
    e2 = O.minifloat(2, 1)
    r, acc = O.gemm_w4a4(ap, e2, a, wp, e2, "row", ws)
    y_pin = O.w4a4_epilogue_f32(acc, a, ws)
    fe2 = F.grid_minifloat(2, 1)
    y32 = F.fp4_gemm(gap, gwp, gws, fw, fgran, K=K, a_grid=fe2, a_scale=ga, y_dtype=torch.float32)
    assert np.array_equal(host(y32).view(np.uint32), y_pin.view(np.uint32))
    assert O.rel_err(host(y32), r) <= TOL
    yb = F.fp4_gemm(gap, gwp, gws, fw, fgran, K=K, a_grid=fe2, a_scale=ga, y_dtype=torch.bfloat16)
    assert np.array_equal(host(yb.view(torch.int16)).view(np.uint16), O.rne_bf16_bits(y_pin))


def test_preshift_w4a4_full_2048x4096x4096():
    """Calibration + pre-shift + W4A4 at the full 2048-token, 4096x4096 size: every
    code bit-exact; the GEMM output bit-exact on 64 sampled rows."""
    say("w4a4 full c3")
    x, w = synth.preshift_inputs()
    (k, a, wp, ws, ap), (gk, ga, gwp, gws, gap, fw, fgran) = _preshift_chain(x, w)
    fe2 = F.grid_minifloat(2, 1)
    y32 = host(F.fp4_gemm(gap, gwp, gws, fw, fgran, K=4096, a_grid=fe2, a_scale=ga, y_dtype=torch.float32))
    rows = np.random.default_rng(0).choice(2048, 64, replace=False)
    e2 = O.minifloat(2, 1)
    r, acc = O.gemm_w4a4(ap[rows], e2, a, wp, e2, "row", ws)
    assert np.array_equal(y32[rows].view(np.uint32), O.w4a4_epilogue_f32(acc, a, ws).view(np.uint32))


@pytest.mark.parametrize("M,N,K,mode,ldy_pad", [
    (2100, 2200, 544, "row", 0),     # 17 x 18 tiles of 128: more tiles than workgroups, ragged
    (4100, 6000, 288, "row", 0),     # 17 x 24 tiles of 256, ragged M, N and K tail
    (4100, 6000, 256, "tensor", 0),
    (1500, 3000, 384, "row", 3),     # output rows not 16-byte aligned: element stores
    (4096, 5200, 256, "row", 0),     # one round of 256x256 tiles, the rest as 256x128
    (4096, 5120, 512, "tensor", 0),  # one round of 256x256 tiles, the rest as 128x128
    (2048, 4096, 256, "row", 0),     # one round of 128x256 tiles on 8 wavefronts
    (2000, 4000, 288, "row", 0),     # 128x256 tiles, ragged M, N and K tail
])
def test_w4a4_e2m1_many_tiles(M, N, K, mode, ldy_pad):
    """W4A4 E2M1 GEMM on random codes where each workgroup computes several tiles in
    turn (edge tiles included): fp32 and bf16 outputs bit-exact."""
    say("w4a4 tiles", M, N, K, mode, ldy_pad)
    rng = np.random.default_rng(M + N + K)
    e2 = O.minifloat(2, 1)
    ap = rng.integers(0, 256, (M, max(K // 2, 16)), dtype=np.uint8)[:, :K // 2]
    wp = rng.integers(0, 256, (N, max(K // 2, 16)), dtype=np.uint8)[:, :K // 2]
    a = np.float32(rng.uniform(0.5, 2.0))
    ws = (rng.uniform(0.5, 2.0, N if mode == "row" else 1)).astype(np.float32)
    _, acc = O.gemm_w4a4(ap, e2, a, wp, e2, mode, ws)
    y_pin = O.w4a4_epilogue_f32(acc, a, np.broadcast_to(ws, (N,)))
    # packed operands with 16-byte aligned rows (lda, ldw multiples of 16)
    lda = max((K // 2 + 15) // 16 * 16, 16)
    gap = torch.zeros((M, lda), dtype=torch.uint8, device=DEV)
    gwp = torch.zeros((N, lda), dtype=torch.uint8, device=DEV)
    gap[:, :K // 2] = torch.from_numpy(ap).to(DEV)
    gwp[:, :K // 2] = torch.from_numpy(wp).to(DEV)
    fe2 = F.grid_minifloat(2, 1)
    ga = dev(np.array([a], np.float32))
    gws = dev(ws)
    for dt, bits in ((torch.float32, lambda y: y.view(np.uint32)), (torch.bfloat16, None)):
        ybuf = torch.full((M, N + ldy_pad), -7.0, dtype=dt, device=DEV)
        y = ybuf[:, :N]
        F.fp4_gemm(gap, gwp, gws, fe2, F.gran(mode), K=K, a_grid=fe2, a_scale=ga, y=y)
        if dt == torch.float32:
            assert np.array_equal(host(y).view(np.uint32), y_pin.view(np.uint32))
        else:
            assert np.array_equal(host(y.view(torch.int16)).view(np.uint16), O.rne_bf16_bits(y_pin))
        if ldy_pad:
            assert bool((ybuf[:, N:] == -7.0).all())
    with pytest.raises(F._lib.FP4Error):  # K = 0 is rejected, not computed
        F.fp4_gemm(gap, gwp, gws, fe2, F.gran(mode), K=0, a_grid=fe2, a_scale=ga)


def _swiglu_case(rng, M, N, K):
    """Random E2M1 codes for X, W_gate, W_up (16-byte aligned rows), scales that put
    y_gate and y_up around +-4, the consumer's scale a' at the 99th percentile of |h| / 6
    (so some values clip) and shifts k' in [-3, 0] or none."""
    e2 = O.minifloat(2, 1)
    ap = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    wg = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    wu = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    a = np.float32(rng.uniform(0.5, 2.0) / np.sqrt(K) / 4)
    sg = rng.uniform(0.5, 2.0, N).astype(np.float32)
    su = rng.uniform(0.5, 2.0, N).astype(np.float32)
    return e2, ap, wg, wu, a, sg, su


def _swiglu_dev(ap, wg, wu, a, sg, su, out_scale, out_shift, M, N, K, pad=16):
    lda = (K // 2 + 15) // 16 * 16
    gap = torch.zeros((M, lda), dtype=torch.uint8, device=DEV)
    gwg = torch.zeros((N, lda), dtype=torch.uint8, device=DEV)
    gwu = torch.zeros((N, lda), dtype=torch.uint8, device=DEV)
    gap[:, :K // 2] = torch.from_numpy(ap).to(DEV)
    gwg[:, :K // 2] = torch.from_numpy(wg).to(DEV)
    gwu[:, :K // 2] = torch.from_numpy(wu).to(DEV)
    hbuf = torch.full((M, N // 2 + pad), 0xAB, dtype=torch.uint8, device=DEV)
    gk = dev(out_shift, torch.int8) if out_shift is not None else None
    F.fp4_gemm_swiglu_quant(gap, dev(np.array([a], np.float32)), gwg, dev(sg), gwu, dev(su),
                            dev(np.array([out_scale], np.float32)), gk, K=K, h_packed=hbuf[:, :N // 2])
    return host(hbuf)


@pytest.mark.parametrize("M,N,K,shifts", [
    (300, 320, 544, True),     # 128x128 tiles (64 output columns each), ragged M, K tail
    (300, 320, 544, False),    # no consumer shifts
    (2100, 4128, 288, True),   # 256x256 tiles (128 output columns), ragged M; last tile 32 columns
    (40, 96, 32, True),        # one K step of 32 codes, a single partial tile
])
def test_swiglu_quant(M, N, K, shifts):
    """Gate/up W4A4 with SwiGLU and the consumer's E2M1 quantization in the epilogue:
    every code bit-exact against the oracle; bytes past N/2 in each row untouched."""
    say("swiglu", M, N, K, shifts)
    rng = np.random.default_rng(M * 7 + N + K)
    e2, ap, wg, wu, a, sg, su = _swiglu_case(rng, M, N, K)
    k = rng.integers(-3, 1, N).astype(np.int8) if shifts else None
    _, h = O.w4a4_swiglu_quant(ap, a, wg, sg, wu, su, np.float32(1.0), None)
    out_scale = np.float32(np.percentile(np.abs(h), 99) / 6.0)
    codes, _ = O.w4a4_swiglu_quant(ap, a, wg, sg, wu, su, out_scale, k)
    got = _swiglu_dev(ap, wg, wu, a, sg, su, out_scale, k, M, N, K)
    assert np.array_equal(got[:, :N // 2], codes)
    assert bool((got[:, N // 2:] == 0xAB).all())
    # the codes are not degenerate: several magnitudes and both signs occur
    u = O.unpack(codes)
    assert len(np.unique(u & 7)) == 8 and (u >= 8).any()


def test_swiglu_quant_full_4096x13824x5120():
    """The LLaMA-13B MLP gate/up shape (4096 tokens, 5120 -> 2 x 13824): codes of 24
    sampled rows bit-exact against the oracle."""
    M, N, K = 4096, 13824, 5120
    say("swiglu full", M, N, K)
    rng = np.random.default_rng(13824)
    e2, ap, wg, wu, a, sg, su = _swiglu_case(rng, M, N, K)
    k = rng.integers(-3, 1, N).astype(np.int8)
    rows = np.sort(rng.choice(M, 24, replace=False))
    _, h = O.w4a4_swiglu_quant(ap[rows], a, wg, sg, wu, su, np.float32(1.0), None)
    out_scale = np.float32(np.percentile(np.abs(h), 99) / 6.0)
    codes, _ = O.w4a4_swiglu_quant(ap[rows], a, wg, sg, wu, su, out_scale, k)
    got = _swiglu_dev(ap, wg, wu, a, sg, su, out_scale, k, M, N, K, pad=0)
    assert np.array_equal(got[rows], codes)


@pytest.mark.parametrize("M,N,K", [(300, 520, 544), (2100, 2200, 1024), (4096, 5120, 512), (2048, 4096, 256)])
def test_w4a4_per_token_scales(M, N, K):
    """Dynamic per-token activation quantization (E2M1, one scale per token) into the
    W4A4 product with per-token scales: fp32 and bf16 outputs bit-exact."""
    say("w4a4 per-token", M, N, K)
    e2 = O.minifloat(2, 1)
    x = synth.activations(16, M, M, K, outlier_frac=0.01, bf16=True)
    w = synth.weight(16, N, N, K)
    ap, asc = O.quantize_pack(x, e2, "row")
    wp, ws = O.quantize_pack(w, e2, "row")
    _, acc = O.gemm_w4a4(ap, e2, asc, wp, e2, "row", ws)
    y_pin = O.w4a4_epilogue_f32(acc, asc, ws)
    fe2 = F.grid_minifloat(2, 1)
    # the activation codes and scales come from the library's own per-token quantizer
    gap, gas = F.fp4_quantize_pack(dev(x, torch.bfloat16), fe2, F.gran("row"))
    assert np.array_equal(host(gap), ap) and np.array_equal(host(gas), asc)
    gwp, gws = torch.from_numpy(wp).to(DEV), dev(ws)
    y32 = F.fp4_gemm(gap, gwp, gws, fe2, F.gran("row"), K=K, a_grid=fe2, a_scale=gas, y_dtype=torch.float32)
    assert np.array_equal(host(y32).view(np.uint32), y_pin.view(np.uint32))
    yb = F.fp4_gemm(gap, gwp, gws, fe2, F.gran("row"), K=K, a_grid=fe2, a_scale=gas, y_dtype=torch.bfloat16)
    assert np.array_equal(host(yb.view(torch.int16)).view(np.uint16), O.rne_bf16_bits(y_pin))


@pytest.mark.parametrize("fmt", [(2, 1), (4, 3)])
def test_per_token_scales_across_row_blocks(fmt):
    """The W4A4 / W8A8 launch splits A and W into row blocks when they pass the 32-bit
    buffer range; a lowered split limit makes a small product span three row blocks of A
    and two of W, and each block must use its own tokens' scales: E2M1 bit-exact, FP8
    within its bound, both equal to the unsplit launch."""
    M, N, K = 700, 600, 512
    say("per-token split", fmt)
    g = O.minifloat(2, 1) if fmt == (2, 1) else O.fp8(4, 3)
    fg = F.grid_minifloat(*fmt)
    x = synth.activations(20, M, M, K, outlier_frac=0.01, bf16=True)
    w = synth.weight(20, N, N, K)
    ap, asc = O.quantize_pack(x, g, "row")
    wp, ws = O.quantize_pack(w, g, "row")
    gap, gas = F.fp4_quantize_pack(dev(x, torch.bfloat16), fg, F.gran("row"))
    gwp, gws = F.fp4_quantize_pack(dev(w), fg, F.gran("row"))
    assert np.array_equal(host(gap), ap) and np.array_equal(host(gas), asc)
    whole = host(F.fp4_gemm(gap, gwp, gws, fg, F.gran("row"), K=K, a_grid=fg, a_scale=gas, y_dtype=torch.float32))
    row_bytes = ap.shape[1]
    try:
        F.set_split_limit(256 * row_bytes)  # 256-row blocks of A and of W
        split = host(F.fp4_gemm(gap, gwp, gws, fg, F.gran("row"), K=K, a_grid=fg, a_scale=gas,
                                y_dtype=torch.float32))
    finally:
        F.set_split_limit(0)
    assert np.array_equal(split.view(np.uint32), whole.view(np.uint32))
    r, acc = O.gemm_w4a4(ap, g, asc, wp, g, "row", ws)
    if fmt == (2, 1):
        assert np.array_equal(split.view(np.uint32), O.w4a4_epilogue_f32(acc, asc, ws).view(np.uint32))
    else:
        S, _ = O.gemm_w4a4(ap, g, asc, wp, g, "row", ws, absolute=True)
        _check_gemm(split, r, S, depth_packed(K), None, packed_window_term(fmt, fmt, S))


@pytest.mark.parametrize("M,N,K", [(256, 384, 512), (130, 200, 640)])
def test_preshift_nf4(M, N, K):
    say("nf4", M, N, K)
    x = synth.activations(5, M, M, K, outlier_frac=0.01)
    w = synth.weight(5, N, N, K)
    (k, a, wp, ws, ap), (gk, ga, gwp, gws, gap, fw, fgran) = _preshift_chain(x, w, "nf4", 64)
    r, _ = O.gemm_w4a4(ap, O.minifloat(2, 1), a, wp, O.nf4(), "group", ws, group=64)
    S, _ = O.gemm_w4a4(ap, O.minifloat(2, 1), a, wp, O.nf4(), "group", ws, group=64, absolute=True)
    fe2 = F.grid_minifloat(2, 1)
    y32 = F.fp4_gemm(gap, gwp, gws, fw, fgran, K=K, a_grid=fe2, a_scale=ga, y_dtype=torch.float32)
    yb = F.fp4_gemm(gap, gwp, gws, fw, fgran, K=K, a_grid=fe2, a_scale=ga, y_dtype=torch.bfloat16)
    _check_gemm(host(y32), r, S, depth_packed(K), yb, _nf4_extra(ap, a, ws, S, 64))


@pytest.mark.parametrize("M,N,K,group,sd,spread", [
    (130, 200, 640, 64, "f16", False),     # fp16 group scales, ragged M and N
    (96, 136, 1024, 128, "f32", False),    # two K steps per scale group
    (256, 384, 512, 64, "f32", True),      # rows whose group scales span 2^-12 .. 1
])
def test_nf4_gemm_scales(M, N, K, group, sd, spread):
    """NF4 weights x E2M1 activations with directly quantized operands: fp16 or fp32
    group scales, groups of 64 or 128, and weight rows whose groups differ by many
    powers of two (the expansion scales each row relative to its largest group)."""
    say("nf4 scales", M, N, K, group, sd, spread)
    x = synth.activations(6, M, M, K)
    w = synth.weight(6, N, N, K)
    if spread:
        # group g of every row scaled by 2^(-12 g / (K/group - 1))
        ng = K // group
        f = np.repeat(np.float32(2.0) ** (-12.0 * np.arange(ng, dtype=np.float32) / (ng - 1)), group)
        w = (w * f[None, :]).astype(np.float32)
    e2, fe2 = O.minifloat(2, 1), F.grid_minifloat(2, 1)
    wp, ws = O.quantize_pack(w, O.nf4(), "group", group, sd)
    ap, asc = O.quantize_pack(x, e2, "tensor")
    gwp, gws = F.fp4_quantize_pack(dev(w), F.grid_nf4(), F.gran("group", group, sd))
    gap, gasc = F.fp4_quantize_pack(dev(x, torch.bfloat16), fe2, F.gran("tensor"))
    assert np.array_equal(host(gwp), wp) and np.array_equal(host(gap), ap)
    r, _ = O.gemm_w4a4(ap, e2, asc[0], wp, O.nf4(), "group", ws.astype(np.float32), group=group)
    S, _ = O.gemm_w4a4(ap, e2, asc[0], wp, O.nf4(), "group", ws.astype(np.float32), group=group, absolute=True)
    y32 = F.fp4_gemm(gap, gwp, gws, F.grid_nf4(), F.gran("group", group, sd), K=K, a_grid=fe2, a_scale=gasc,
                     y_dtype=torch.float32)
    yb = F.fp4_gemm(gap, gwp, gws, F.grid_nf4(), F.gran("group", group, sd), K=K, a_grid=fe2, a_scale=gasc,
                    y_dtype=torch.bfloat16)
    _check_gemm(host(y32), r, S, depth_packed(K), yb,
                _nf4_extra(ap, asc[0], ws.astype(np.float32), S, group))


# ---------------------------------------------------------------- search ----------
def test_search_small():
    say("search small")
    T, rows, cols = 5, 32, 1040  # numel 33280: several passes and a ragged tail
    ws = np.stack([synth.search_tensor(100 + t, rows, cols).reshape(-1) for t in range(T)])
    res, packed = F.fp4_search_format(dev(ws))
    recs = F.search_results_host(res)
    gp = host(packed)
    for t in range(T):
        rec, p, mse = O.search_tensor(ws[t])
        g = recs[t]
        assert (g.e, g.m, g.clip_index) == (rec.e, rec.m, rec.clip_index), (t, g, rec)
        assert np.float32(g.clip) == rec.clip and np.float32(g.scale) == rec.scale
        assert g.mse == rec.mse and g.mse_runner_up == rec.mse_runner_up
        assert abs(g.bias - rec.bias) <= 1e-14 * abs(rec.bias)
        assert np.array_equal(gp[t], p)


@pytest.mark.parametrize("fmt", [(1, 2), (2, 1), (3, 0)])
def test_search_planted(fmt):
    g = O.minifloat(*fmt)
    rng = np.random.default_rng(3)
    codes = np.concatenate([np.arange(8), rng.integers(0, 8, 4096 - 8)])
    w = (g.array[codes] * 2.0 ** -6).astype(np.float32) * np.where(rng.random(4096) < 0.5, -1, 1).astype(np.float32)
    res, packed = F.fp4_search_format(dev(w.reshape(1, -1)))
    r = F.search_results_host(res)[0]
    assert (r.e, r.m, r.clip_index, r.mse) == (fmt[0], fmt[1], 99, 0.0)


def test_search_full_32_tensors():
    """The format / clip search as the 32-tensor workload runs it: 32 heavy-tailed
    4096x4096 tensors in one call (the launch geometry and workspace layout of that
    size); two sampled tensors' records and packed codes bit-exact against the oracle
    over all 300 candidates, and every record a valid candidate of its tensor."""
    from concurrent.futures import ThreadPoolExecutor
    say("search 32 tensors")
    with ThreadPoolExecutor(8) as ex:
        ws = list(ex.map(lambda t: synth.search_tensor(t).reshape(-1), range(32)))
    w = torch.empty((32, 4096 * 4096), dtype=torch.float32, device=DEV)
    for t in range(32):
        w[t] = torch.from_numpy(ws[t]).to(DEV)
    res, packed = F.fp4_search_format(w)
    recs = F.search_results_host(res)
    del w
    for t in (0, 21):
        say("  oracle on tensor", t)
        rec, p, _ = O.search_tensor(ws[t])
        _check_records(res[t * F.SEARCH_RESULT_BYTES:(t + 1) * F.SEARCH_RESULT_BYTES], [rec])
        assert np.array_equal(host(packed[t]), p)
    for t, g in enumerate(recs):
        amax = np.float32(np.max(np.abs(ws[t])))
        assert np.float32(g.amax) == amax
        assert (g.e, g.m) in ((1, 2), (2, 1), (3, 0)) and 0 <= g.clip_index < 100
        assert np.float32(g.clip) == np.float32(amax * O.clip_ratios()[g.clip_index])
        assert g.mse <= g.mse_runner_up


def _check_records(gres, orecs):
    for g, rec in zip(F.search_results_host(gres), orecs):
        assert (g.e, g.m, g.clip_index) == (rec.e, rec.m, rec.clip_index), (g, rec)
        assert np.float32(g.clip) == rec.clip and np.float32(g.scale) == rec.scale
        assert g.mse == rec.mse and g.mse_runner_up == rec.mse_runner_up
        assert abs(g.bias - rec.bias) <= 1e-14 * abs(rec.bias)


@pytest.mark.parametrize("rows,cols,bf16,pad", [
    (37, 1040, True, 8),     # 1040 per row: 8 values per lane, a ragged last pass
    (20, 5120, True, 0),     # 24 values per lane
    (9, 4096, False, 4),     # f32 rows, 16 values per lane
    (3, 40000, False, 0),    # several passes per row
])
def test_search_activations_per_token(rows, cols, bf16, pad):
    """Per-token search on activations with outlier channels: every record and every
    packed row bit-exact; packed bytes past cols/2 untouched."""
    say("search act row", rows, cols, bf16, pad)
    x = synth.activations(7, rows, rows, cols, outlier_frac=0.01, bf16=bf16)
    xbuf = torch.zeros((rows, cols + pad), dtype=torch.bfloat16 if bf16 else torch.float32, device=DEV)
    xbuf[:, :cols] = dev(x, xbuf.dtype)
    pbuf = torch.full((rows, cols // 2 + 16), 0xAB, dtype=torch.uint8, device=DEV)
    res, _ = F.fp4_search_activations(xbuf[:, :cols], "row", packed=pbuf[:, :cols // 2])
    recs, packed = O.search_activations(x, "row")
    _check_records(res, recs)
    gp = host(pbuf)
    assert np.array_equal(gp[:, :cols // 2], packed)
    assert bool((gp[:, cols // 2:] == 0xAB).all())


@pytest.mark.parametrize("rows,first,cols,bf16", [(300, 128, 2048, True), (50, 0, 1040, False), (7, 64, 4096, True)])
def test_search_activations_calibration(rows, first, cols, bf16):
    """One search over the calibration tokens (the first rows), every row packed with the
    winner: the record and all packed rows bit-exact."""
    say("search act tensor", rows, first, cols, bf16)
    x = synth.activations(8, rows, rows, cols, outlier_frac=0.01, bf16=bf16)
    xt = dev(x, torch.bfloat16 if bf16 else torch.float32)
    res, gp = F.fp4_search_activations(xt, "tensor", first_rows=first)
    recs, packed = O.search_activations(x, "tensor", first_rows=first)
    _check_records(res, recs)
    assert np.array_equal(host(gp), packed)


def test_search_activations_full_4096x5120_sampled():
    """Per-token search at the LLaMA-13B prefill activation shape (4096 tokens x 5120
    bf16): 12 sampled rows' records and codes bit-exact."""
    rows, cols = 4096, 5120
    say("search act full", rows, cols)
    x = synth.activations(9, rows, rows, cols, outlier_frac=0.01, bf16=True)
    res, gp = F.fp4_search_activations(dev(x, torch.bfloat16), "row")
    pick = np.sort(np.random.default_rng(5).choice(rows, 12, replace=False))
    recs, packed = O.search_activations(x[pick], "row")
    allrec = F.search_results_host(res)
    for k, r in enumerate(pick):
        g, rec = allrec[r], recs[k]
        assert (g.e, g.m, g.clip_index, g.mse, g.mse_runner_up) == (rec.e, rec.m, rec.clip_index, rec.mse,
                                                                     rec.mse_runner_up)
        assert np.float32(g.scale) == rec.scale
    assert np.array_equal(host(gp)[pick], packed)


# ---------------------------------------------------------------- two-mode grid ---
def _f16_or_f32_bits(a):
    a = np.asarray(a)
    return a.view(np.uint16) if a.dtype == np.float16 else a.astype(np.float32).view(np.uint32)


@pytest.mark.parametrize("rows,cols,group,sd,bf16", [
    (37, 1040, 8, "f32", False),     # one lane per group, a ragged chunk
    (64, 4096, 32, "f16", True),
    (30, 6144, 128, "f16", False),   # the W4A16 group size
    (9, 2048, 512, "f32", True),     # a whole wavefront per group
])
def test_two_mode_quantize_dequantize(rows, cols, group, sd, bf16):
    """Two-mode quantize: every code, scale and mode (the scale's sign) bit-exact; the
    dequantized values bit-exact; both modes occur."""
    say("two-mode", rows, cols, group, sd, bf16)
    x = synth.weight(11, rows, rows, cols) if not bf16 else synth.activations(11, rows, rows, cols, outlier_frac=0.01,
                                                                             bf16=True)
    xt = dev(x, torch.bfloat16 if bf16 else torch.float32)
    g = F.gran("group", group, sd)
    packed, scales = F.fp4_quantize_pack(xt, F.grid_two_mode(), g)
    op, osc, modes = O.quantize_two_mode(x, group, sd)
    assert np.array_equal(host(packed), op)
    gs = host(scales).reshape(osc.shape)
    assert np.array_equal(_f16_or_f32_bits(gs), _f16_or_f32_bits(osc))
    assert 0 < modes.mean() < 1
    deq = host(F.fp4_dequantize(packed, F.grid_two_mode(), g, scales))
    assert np.array_equal(deq.view(np.uint32), O.two_mode_values(op, osc, group).view(np.uint32))


_TWO_MODE_W = {}


def _two_mode_weight(N, K, sd):
    """The oracle's two-mode quantization of a synthetic weight, shared by the cases."""
    if (N, K, sd) not in _TWO_MODE_W:
        _TWO_MODE_W[(N, K, sd)] = O.quantize_two_mode(synth.weight(12, N, N, K), 128, sd)
    return _TWO_MODE_W[(N, K, sd)]


@pytest.mark.parametrize("M,N,K,sd,adt", [
    (1, 11008, 4096, "f16", "bf16"),   # decode GEMV shape: the small matrix-core kernel
    (4, 11008, 4096, "f16", "bf16"),
    (16, 11008, 4096, "f32", "bf16"),
    (40, 1000, 1024, "f16", "bf16"),   # larger M: the VALU kernel
    (3, 520, 512, "f32", "f32"),       # f32 activations: the VALU kernel
])
def test_two_mode_w4a16_gemm(M, N, K, sd, adt):
    """W4A16 with two-mode weights: within the GEMM tolerance of the binary64 oracle,
    bf16 output the nearest-even rounding of the fp32 output."""
    say("two-mode gemm", M, N, K, sd, adt)
    op, osc, modes = _two_mode_weight(N, K, sd)
    gp = torch.from_numpy(op).to(DEV)
    gs = torch.from_numpy(np.ascontiguousarray(osc)).to(DEV)
    x = synth.activations(12, M, M, K, outlier_frac=0.01, bf16=adt == "bf16")
    xt = dev(x, torch.bfloat16 if adt == "bf16" else torch.float32)
    g = F.gran("group", 128, sd)
    y32 = host(F.fp4_gemm(xt, gp, gs, F.grid_two_mode(), g, y_dtype=torch.float32))
    r = O.gemm_w4a16_two_mode(x, op, osc, 128)
    S = O.gemm_w4a16_two_mode(x, op, osc, 128, absolute=True)
    say("  modes", modes.mean())
    yb = F.fp4_gemm(xt, gp, gs, F.grid_two_mode(), g, y_dtype=torch.bfloat16)
    _check_gemm(y32, r, S, depth_w4a16(K, 128), yb)


# ---------------------------------------------------------------- FP8 / FP6 grids -
def _wide(fmt):
    return O.fp8(*fmt) if sum(fmt) == 7 else (O.fp6(*fmt) if sum(fmt) == 5 else O.minifloat(*fmt))


@pytest.mark.parametrize("fmt", [(4, 3), (5, 2), (2, 3), (3, 2)])
@pytest.mark.parametrize("rows,cols,mode,group,sd,bf16", [
    (33, 5120, "group", 128, "f16", False),  # f32 group-128 kernel: a partial second 4096-column unit
    (7, 256, "group", 128, "f32", False),
    (37, 1040, "group", 8, "f32", False),
    (64, 4096, "group", 128, "f16", True),
    (30, 2056, "tensor", 0, "f32", False),   # a ragged last chunk, amax computed here
    (9, 2048, "group", 512, "f32", True),
    (40, 2056, "row", 0, "f32", False),      # one scale per row, a ragged last chunk
    (33, 4096, "row", 0, "f16", True),
])
def test_fp8_quantize_dequantize(fmt, rows, cols, mode, group, sd, bf16):
    """OCP FP8 (one code per byte) and FP6 (four codes in three bytes) quantize: every
    code byte and scale bit-exact; dequantized values bit-exact."""
    say("fp8/fp6", fmt, rows, cols, mode, group, sd, bf16)
    x = synth.weight(13, rows, rows, cols) if not bf16 else synth.activations(13, rows, rows, cols,
                                                                             outlier_frac=0.01, bf16=True)
    xt = dev(x, torch.bfloat16 if bf16 else torch.float32)
    og, fg = _wide(fmt), F.grid_minifloat(*fmt)
    g = F.gran(mode, group, sd)
    packed, scales = F.fp4_quantize_pack(xt, fg, g)
    op, osc = O.quantize_pack(x, og, mode, group=group, scale_dtype=sd)
    assert packed.shape == (rows, cols * og.bits // 8) and np.array_equal(host(packed), op)
    assert np.array_equal(_f16_or_f32_bits(host(scales).reshape(np.asarray(osc).shape)), _f16_or_f32_bits(osc))
    deq = host(F.fp4_dequantize(packed, fg, g, scales))
    assert np.array_equal(deq.view(np.uint32), O.dequantize(op, og, mode, osc, group=group).view(np.uint32))


@pytest.mark.parametrize("fmt", [(4, 3), (5, 2), (2, 3), (3, 2)])
@pytest.mark.parametrize("M,N,K,mode,adt", [
    (1, 11008, 4096, "group", "bf16"),   # decode GEMV shape: the small matrix-core kernel
    (16, 11008, 4096, "group", "bf16"),
    (8, 1000, 1024, "tensor", "bf16"),
    (3, 520, 512, "group", "f32"),       # f32 activations: the VALU kernel
])
def test_fp8_w8a16_gemm(fmt, M, N, K, mode, adt):
    """W8A16 / W6A16 with FP8 / FP6 weights: within the GEMM tolerance of the binary64
    oracle, bf16 output the nearest-even rounding of the fp32 output."""
    say("w8a16/w6a16", fmt, M, N, K, mode, adt)
    og, fg = _wide(fmt), F.grid_minifloat(*fmt)
    w = synth.weight(14, N, N, K)
    gr = 128 if mode == "group" else 0
    op, osc = O.quantize_pack(w, og, mode, group=gr, scale_dtype="f16" if mode == "group" else "f32")
    x = synth.activations(14, M, M, K, outlier_frac=0.01, bf16=adt == "bf16")
    xt = dev(x, torch.bfloat16 if adt == "bf16" else torch.float32)
    gp = torch.from_numpy(op).to(DEV)
    gs = torch.from_numpy(np.ascontiguousarray(osc)).to(DEV)
    g = F.gran(mode, gr, "f16" if mode == "group" else "f32")
    y32 = host(F.fp4_gemm(xt, gp, gs, fg, g, y_dtype=torch.float32))
    r = O.gemm_w4a16(x, op, og, mode, osc, group=gr)
    S = O.gemm_w4a16(x, op, og, mode, osc, group=gr, absolute=True)
    yb = F.fp4_gemm(xt, gp, gs, fg, g, y_dtype=torch.bfloat16)
    _check_gemm(y32, r, S, depth_w4a16(K, gr or K), yb)


@pytest.mark.parametrize("M,N,K,mode", [
    (300, 520, 544, "row"),      # ragged tiles, a K tail of half a step
    (2100, 2200, 1024, "row"),   # several tiles per workgroup
    (4096, 5120, 4096, "tensor"),
    (2048, 4096, 320, "row"),    # one round of 128x256 tiles, a K tail of one step
])
def test_fp8_w8a8_gemm(M, N, K, mode):
    """W8A8: FP8 E4M3 activations (per-tensor scale) x FP8 E4M3 weights on the FP8 matrix
    cores, within the GEMM tolerance of the binary64 oracle; bf16 output the nearest-even
    rounding of the fp32 output."""
    say("w8a8", M, N, K, mode)
    g8 = O.fp8(4, 3)
    x = synth.activations(15, M, M, K, outlier_frac=0.01)
    w = synth.weight(15, N, N, K)
    ap, asc = O.quantize_pack(x, g8, "tensor")
    wp, wsc = O.quantize_pack(w, g8, mode)
    r, _ = O.gemm_w4a4(ap, g8, asc[0], wp, g8, mode, wsc)
    fg = F.grid_minifloat(4, 3)
    gap, gwp = torch.from_numpy(ap).to(DEV), torch.from_numpy(wp).to(DEV)
    ga, gws = dev(np.asarray(asc, np.float32)), dev(np.asarray(wsc, np.float32))
    S, _ = O.gemm_w4a4(ap, g8, asc[0], wp, g8, mode, wsc, absolute=True)
    y32 = host(F.fp4_gemm(gap, gwp, gws, fg, F.gran(mode), K=K, a_grid=fg, a_scale=ga, y_dtype=torch.float32))
    yb = F.fp4_gemm(gap, gwp, gws, fg, F.gran(mode), K=K, a_grid=fg, a_scale=ga, y_dtype=torch.bfloat16)
    _check_gemm(y32, r, S, depth_packed(K), yb, packed_window_term((4, 3), (4, 3), S))


@pytest.mark.parametrize("M,N,K", [(256, 384, 512), (520, 1100, 1024)])
@pytest.mark.parametrize("af,wf", [((4, 3), (4, 3)), ((2, 3), (2, 3)), ((4, 3), (2, 3))])
def test_preshift_fp8_fp6(M, N, K, af, wf):
    """The pre-shifted exponent bias with FP8 / FP6 grids: channel maxima, shifts, the
    activation scale, the shifted weights' codes and row scales and the shifted
    activations' codes bit-exact; the W8A8 / W6A6 / mixed product from them within the
    GEMM tolerance of the binary64 oracle."""
    say("preshift fp8/fp6", M, N, K, af, wf)
    x = synth.activations(18, M, M, K, outlier_frac=0.01, bf16=True)
    w = synth.weight(18, N, N, K)
    og_a, og_w = _wide(af), _wide(wf)
    chan = O.amax_columns(x, 128)
    k, a, wp, ws = O.preshift_weights(w, chan, og_a, og_w, "row")
    ap, _ = O.quantize_activations(x, og_a, a, k)
    fa, fw = F.grid_minifloat(*af), F.grid_minifloat(*wf)
    xt = dev(x, torch.bfloat16)
    gchan = F.fp4_calibrate(xt, "column", first_rows=128)
    assert np.array_equal(host(gchan), chan)
    gk, ga, gwp, gws = F.fp4_preshift_weights(dev(w), gchan, fa, fw, F.gran("row"))
    assert np.array_equal(host(gk), k) and host(ga)[0] == a
    assert np.array_equal(host(gwp), wp) and np.array_equal(host(gws), np.asarray(ws).reshape(-1))
    gap, _ = F.fp4_quantize_pack(xt, fa, F.gran("tensor"), tensor_scale=ga, col_shift=gk)
    assert np.array_equal(host(gap), ap)
    r, _ = O.gemm_w4a4(ap, og_a, a, wp, og_w, "row", ws)
    S, _ = O.gemm_w4a4(ap, og_a, a, wp, og_w, "row", ws, absolute=True)
    y32 = host(F.fp4_gemm(gap, gwp, gws, fw, F.gran("row"), K=K, a_grid=fa, a_scale=ga, y_dtype=torch.float32))
    _check_gemm(y32, r, S, depth_packed(K), None, packed_window_term(af, wf, S))


@pytest.mark.parametrize("af,wf", [((4, 3), (4, 3)), ((2, 3), (2, 3)), ((5, 2), (2, 3)), ((2, 1), (4, 3)),
                                   ((4, 3), (2, 1))])
def test_f8f6_per_token_scales(af, wf):
    """FP8 / FP6 activations quantized per token (one scale per row, on the GPU) and
    their product with row-scaled FP8 / FP6 weights (y = fl32(acc * fl32(a_m * s_n))):
    codes and scales bit-exact, the product within the GEMM tolerance."""
    M, N, K = 300, 520, 512
    say("f8f6 per-token", af, wf)
    x = synth.activations(19, M, M, K, outlier_frac=0.01, bf16=True)
    w = synth.weight(19, N, N, K)
    og_a, og_w = _wide(af), _wide(wf)
    ap, asc = O.quantize_pack(x, og_a, "row")
    wp, wsc = O.quantize_pack(w, og_w, "row")
    fa, fw = F.grid_minifloat(*af), F.grid_minifloat(*wf)
    gap, gas = F.fp4_quantize_pack(dev(x, torch.bfloat16), fa, F.gran("row"))
    gwp, gws = F.fp4_quantize_pack(dev(w), fw, F.gran("row"))
    assert np.array_equal(host(gap), ap) and np.array_equal(host(gas), np.asarray(asc, np.float32))
    assert np.array_equal(host(gwp), wp) and np.array_equal(host(gws), np.asarray(wsc, np.float32))
    r, _ = O.gemm_w4a4(ap, og_a, asc, wp, og_w, "row", wsc)
    S, _ = O.gemm_w4a4(ap, og_a, asc, wp, og_w, "row", wsc, absolute=True)
    y32 = host(F.fp4_gemm(gap, gwp, gws, fw, F.gran("row"), K=K, a_grid=fa, a_scale=gas, y_dtype=torch.float32))
    _check_gemm(y32, r, S, depth_packed(K), None, packed_window_term(af, wf, S))


def depth_packed_group(K, G):
    """Group-scaled FP8 / FP6 weights with packed activations: each group's partial sum
    as in depth_packed, one fused multiply-add per group folding it into the running sum,
    and the final scaling by the activation scale."""
    return 2 * K + K // G + 4


@pytest.mark.parametrize("M,N,K,wf,af,G,sdt,per_token", [
    (300, 520, 640, (4, 3), (4, 3), 128, "f16", False),    # E4M3 x E4M3, [W8A8] group 128
    (300, 520, 640, (2, 3), (2, 3), 64, "f32", False),     # W6A6, two groups per 128-code step
    (130, 270, 1024, (5, 2), (4, 3), 256, "f16", False),   # a group spans two steps
    (257, 300, 512, (3, 2), (2, 1), 512, "f32", False),    # one group per row; E2M1 activations
    (300, 520, 640, (4, 3), (2, 3), 128, "f16", True),     # per-token activation scales
    (2100, 2200, 1024, (2, 3), (2, 3), 128, "f16", False), # several tile rows and columns
    # E4M3 x E4M3, group 128, whole 4-byte scale rows: the persistent kernel's 128x256 tiles
    (300, 520, 1024, (4, 3), (4, 3), 128, "f16", False),   # ragged tiles
    (300, 520, 1152, (4, 3), (4, 3), 128, "f32", False),   # K steps past the last group
    (4100, 2200, 1280, (4, 3), (4, 3), 128, "f32", True),  # several tiles per workgroup, per-token
    (130, 300, 128, (4, 3), (4, 3), 128, "f32", False),    # one group per row (a single four-step group)
    (64, 260, 256, (4, 3), (4, 3), 128, "f16", True),      # two groups, one partial tile row
    (300, 520, 1024, (4, 3), (4, 3), 64, "f32", False),    # groups of 64: a fold after every step
    (300, 520, 1024, (4, 3), (4, 3), 256, "f16", True),    # groups of 256: a fold every four steps
    (130, 270, 1280, (4, 3), (4, 3), 256, "f32", False),   # five groups of 256
])
def test_f8f6_group_scaled_weights(M, N, K, wf, af, G, sdt, per_token):
    """FP8 / FP6 weights with one scale per row and group of G codes along K ([W8A8]
    section 2.2), quantized on the GPU (codes and scales bit-exact against the oracle), and
    their product with packed activations: within the GEMM tolerance of the binary64
    oracle's a * sum_g s[n, g] * sum_{k in g} A_q W_q, elementwise; bf16 the nearest-even
    rounding of the fp32 output."""
    say("f8f6 group", M, N, K, wf, af, G, sdt, per_token)
    x = synth.activations(21, M, M, K, outlier_frac=0.01)
    w = synth.weight(21, N, N, K)
    og_a, og_w = _wide(af), _wide(wf)
    amode = "row" if per_token else "tensor"
    ap, asc = O.quantize_pack(x, og_a, amode)
    wp, wsc = O.quantize_pack(w, og_w, "group", G, sdt)
    fa, fw = F.grid_minifloat(*af), F.grid_minifloat(*wf)
    wg = F.gran("group", G, sdt)
    gwp, gws = F.fp4_quantize_pack(dev(w), fw, wg)
    assert np.array_equal(host(gwp), wp)
    assert np.array_equal(host(gws.float()), np.asarray(wsc, np.float32).reshape(-1))
    gap = _padded_rows(ap)
    ga = dev(np.asarray(asc, np.float32).reshape(-1))
    r, _ = O.gemm_w4a4(ap, og_a, asc, wp, og_w, "group", wsc, group=G)
    S, _ = O.gemm_w4a4(ap, og_a, asc, wp, og_w, "group", wsc, group=G, absolute=True)
    y32 = host(F.fp4_gemm(gap, gwp, gws, fw, wg, K=K, a_grid=fa, a_scale=ga, y_dtype=torch.float32))
    yb = F.fp4_gemm(gap, gwp, gws, fw, wg, K=K, a_grid=fa, a_scale=ga, y_dtype=torch.bfloat16)
    _check_gemm(y32, r, S, depth_packed_group(K, G), yb, packed_window_term(af, wf, S))


def _padded_rows(packed, align=16):
    """uint8 rows copied into a device buffer whose row stride is a multiple of `align`
    bytes (the packed products need 16-byte aligned rows), returned as the [:, :bytes] view."""
    R, B = packed.shape
    ld = (B + align - 1) // align * align
    buf = torch.zeros((R, ld), dtype=torch.uint8, device=DEV)
    buf[:, :B] = torch.from_numpy(np.ascontiguousarray(packed)).to(DEV)
    return buf[:, :B]


@pytest.mark.parametrize("M,N,K,wf,af,mode", [
    (300, 520, 544, (2, 3), (2, 3), "row"),     # W6A6 E2M3: ragged tiles, a half-filled last FP6 piece
    (2100, 2200, 1024, (3, 2), (3, 2), "row"),  # W6A6 E3M2, several tile rows and columns
    (300, 520, 640, (2, 3), (2, 3), "row"),     # W6A6 on the persistent kernel: ragged 128x128 tiles
    (4096, 5120, 4096, (2, 3), (2, 3), "tensor"),
    (256, 384, 512, (5, 2), (5, 2), "row"),     # W8A8 with E5M2
    (2100, 2200, 1024, (5, 2), (5, 2), "row"),  # E5M2 x E5M2 on the persistent kernel: 128x128 tiles, ragged
    (4100, 6000, 256, (5, 2), (5, 2), "tensor"),  # E5M2 x E5M2: rounds of 256x256 tiles and a leftover block
    (300, 520, 544, (4, 3), (5, 2), "row"),     # mixed FP8: E4M3 weights, E5M2 activations
    (4100, 6000, 256, (5, 2), (4, 3), "tensor"),  # mixed FP8: E5M2 weights, E4M3 activations, 256x256 tiles
    (300, 520, 544, (4, 3), (2, 3), "row"),     # mixed: FP8 E4M3 weights, FP6 E2M3 activations
    (130, 270, 96, (2, 3), (5, 2), "tensor"),   # mixed: FP6 weights, FP8 E5M2 activations; K below one step
    (300, 520, 544, (4, 3), (2, 1), "row"),     # FP8 weights, FP4 E2M1 activations
    (300, 520, 544, (2, 1), (2, 3), "row"),     # FP4 E2M1 weights, FP6 activations
    (130, 270, 1024, (3, 2), (2, 1), "tensor"),
    (300, 520, 544, (2, 1), (4, 3), "row"),     # FP4 E2M1 weights, FP8 E4M3 activations
    (130, 270, 1024, (2, 1), (5, 2), "tensor"), # FP4 E2M1 weights, FP8 E5M2 activations
])
def test_f8f6_gemm(M, N, K, wf, af, mode):
    """Both operands FP8 / FP6, or one of them FP4 E2M1 (every pair other than E4M3 x
    E4M3, which the W8A8 test covers) on the f8f6f4 matrix cores: within the GEMM tolerance of the binary64
    oracle; bf16 output the nearest-even rounding of the fp32 output."""
    say("f8f6", M, N, K, wf, af, mode)
    og_w, og_a = _wide(wf), _wide(af)
    x = synth.activations(16, M, M, K, outlier_frac=0.01)
    w = synth.weight(16, N, N, K)
    ap, asc = O.quantize_pack(x, og_a, "tensor")
    wp, wsc = O.quantize_pack(w, og_w, mode)
    r, _ = O.gemm_w4a4(ap, og_a, asc[0], wp, og_w, mode, wsc)
    fw, fa = F.grid_minifloat(*wf), F.grid_minifloat(*af)
    gap, gwp = _padded_rows(ap), _padded_rows(wp)
    ga, gws = dev(np.asarray(asc, np.float32)), dev(np.asarray(wsc, np.float32))
    S, _ = O.gemm_w4a4(ap, og_a, asc[0], wp, og_w, mode, wsc, absolute=True)
    y32 = host(F.fp4_gemm(gap, gwp, gws, fw, F.gran(mode), K=K, a_grid=fa, a_scale=ga, y_dtype=torch.float32))
    yb = F.fp4_gemm(gap, gwp, gws, fw, F.gran(mode), K=K, a_grid=fa, a_scale=ga, y_dtype=torch.bfloat16)
    _check_gemm(y32, r, S, depth_packed(K), yb, packed_window_term(af, wf, S))


@pytest.mark.parametrize("M,N,K,wf,af,mode", [
    (300, 520, 544, (1, 2), (1, 2), "row"),      # E1M2 x E1M2, ragged tiles and K tail
    (2100, 2200, 1024, (3, 0), (3, 0), "row"),   # E3M0 x E3M0, several tile rows and columns
    (300, 520, 544, (2, 1), (1, 2), "tensor"),   # E2M1 weights, E1M2 activations
    (300, 520, 544, (1, 2), (2, 1), "row"),      # E1M2 weights, E2M1 activations
    (130, 270, 96, (3, 0), (2, 1), "row"),       # K below one step
    (300, 520, 544, (2, 1), (3, 0), "row"),
    (300, 520, 544, (3, 0), (1, 2), "tensor"),
])
def test_w4a4_e1m2_e3m0_exact(M, N, K, wf, af, mode):
    """W4A4 with E1M2 or E3M0 on either side (codes expanded to E4M3 on their way into
    LDS, every value of both grids being an E4M3 value): all their products with a 4-bit
    grid are multiples of 2^-4 that the matrix instruction keeps whole, and the fp32 sums
    stay exact, so the fp32 output is fl32(acc * fl32(a * s_n)) bit for bit and the bf16
    output its nearest-even rounding."""
    say("w4a4 e1m2/e3m0", M, N, K, wf, af, mode)
    rng = np.random.default_rng(M + K + 7 * sum(wf) + af[0])
    og_w, og_a = _wide(wf), _wide(af)
    ap = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    wp = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    a = np.float32(rng.uniform(0.5, 2.0))
    ws = rng.uniform(0.5, 2.0, N if mode == "row" else 1).astype(np.float32)
    _, acc = O.gemm_w4a4(ap, og_a, a, wp, og_w, mode, ws)
    assert np.array_equal(acc, acc.astype(np.float32).astype(np.float64))  # exact in binary32
    y_pin = O.w4a4_epilogue_f32(acc, a, np.broadcast_to(ws, (N,)))
    fw, fa = F.grid_minifloat(*wf), F.grid_minifloat(*af)
    gap, gwp = _padded_rows(ap), _padded_rows(wp)
    ga, gws = dev(np.array([a], np.float32)), dev(ws)
    y32 = host(F.fp4_gemm(gap, gwp, gws, fw, F.gran(mode), K=K, a_grid=fa, a_scale=ga, y_dtype=torch.float32))
    assert np.array_equal(y32.view(np.uint32), y_pin.view(np.uint32))
    yb = F.fp4_gemm(gap, gwp, gws, fw, F.gran(mode), K=K, a_grid=fa, a_scale=ga, y_dtype=torch.bfloat16)
    assert np.array_equal(_bf16_bits(yb), O.rne_bf16_bits(y_pin))


@pytest.mark.parametrize("wf,af", [((4, 3), (1, 2)), ((1, 2), (4, 3)), ((3, 0), (2, 3)), ((2, 3), (1, 2)),
                                   ((3, 0), (5, 2))])
def test_w4a4_e1m2_e3m0_with_wide_grids(wf, af):
    """E1M2 / E3M0 paired with an FP8 or FP6 grid, per-token activation scales: within
    the GEMM tolerance of the binary64 oracle (with the product-window term where a
    pair can lose product bits)."""
    M, N, K = 300, 520, 512
    say("w4a4 e1m2/e3m0 wide", wf, af)
    x = synth.activations(21, M, M, K, outlier_frac=0.01, bf16=True)
    w = synth.weight(21, N, N, K)
    og_a, og_w = _wide(af), _wide(wf)
    ap, asc = O.quantize_pack(x, og_a, "row")
    wp, wsc = O.quantize_pack(w, og_w, "row")
    fa, fw = F.grid_minifloat(*af), F.grid_minifloat(*wf)
    gap, gas = F.fp4_quantize_pack(dev(x, torch.bfloat16), fa, F.gran("row"))
    gwp, gws = F.fp4_quantize_pack(dev(w), fw, F.gran("row"))
    assert np.array_equal(host(gap), ap) and np.array_equal(host(gwp), wp)
    r, _ = O.gemm_w4a4(ap, og_a, asc, wp, og_w, "row", wsc)
    S, _ = O.gemm_w4a4(ap, og_a, asc, wp, og_w, "row", wsc, absolute=True)
    y32 = host(F.fp4_gemm(gap, gwp, gws, fw, F.gran("row"), K=K, a_grid=fa, a_scale=gas, y_dtype=torch.float32))
    yb = F.fp4_gemm(gap, gwp, gws, fw, F.gran("row"), K=K, a_grid=fa, a_scale=gas, y_dtype=torch.bfloat16)
    _check_gemm(y32, r, S, depth_packed(K), yb, packed_window_term(af, wf, S))


def _one_row_product(fmt, a_vals, w_vals, K=128):
    """y[0, 0] of a product whose first rows hold the given values (codes from the
    oracle's quantizer at scale 1, every value exactly on the grid)."""
    g = _wide(fmt)
    a = np.zeros((256, K), np.float32)
    w = np.zeros((256, K), np.float32)
    for i, v in a_vals.items():
        a[0, i] = v
    for i, v in w_vals.items():
        w[0, i] = v
    ap = O.pack_codes(O.quantize(a, np.float32(1), g), g)
    wp = O.pack_codes(O.quantize(w, np.float32(1), g), g)
    assert np.array_equal(g.decode(O.unpack_codes(ap, g)), a)  # the values are grid points
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    fg = F.grid_minifloat(*fmt)
    y = F.fp4_gemm(_padded_rows(ap), _padded_rows(wp), one, fg, F.gran("tensor"), K=K, a_grid=fg, a_scale=one,
                   y_dtype=torch.float32)
    return float(host(y)[0, 0])


def test_matrix_instruction_product_window():
    """The facts the packed products' tolerances rest on: within a group of 8 products
    the f8f6f4 instruction keeps bits down to 2^-13 of the largest product (FP8: 1 + 2^-13
    kept, 1 + 2^-14 dropped, across groups nothing dropped), and the E2M1 and E2M3 grids'
    extreme products (36 with 0.25; 56.25 with 2^-6) add exactly in one group."""
    assert _one_row_product((4, 3), {0: 1.0, 5: 2.0 ** -9}, {0: 1.0, 5: 2.0 ** -4}) == 1 + 2.0 ** -13
    assert _one_row_product((4, 3), {0: 1.0, 5: 2.0 ** -9}, {0: 1.0, 5: 2.0 ** -5}) == 1.0
    assert _one_row_product((4, 3), {0: 1.0, 9: 2.0 ** -9}, {0: 1.0, 9: 2.0 ** -5}) == 1 + 2.0 ** -14
    assert _one_row_product((2, 1), {0: 6.0, 1: 0.5, 2: -0.5}, {0: 6.0, 1: 0.5, 2: 0.5}) == 36.0
    assert _one_row_product((2, 1), {0: 6.0, 1: 0.5}, {0: 6.0, 1: 0.5}) == 36.25
    assert _one_row_product((2, 3), {0: 7.5, 1: 0.125}, {0: 7.5, 1: 0.125}) == 56.25 + 2.0 ** -6


# ---------------------------------------------------------------- determinism -----
def test_graph_replays_match_eager():
    """The library's calls captured in one HIP graph (calibrate, pre-shift, quantize,
    W4A4, W4A16, the activation search with its zero-filled workspace) and replayed
    several times with eager work in between: every replay equals the eager results."""
    fe2 = F.grid_minifloat(2, 1)
    x = dev(synth.activations(17, 1, 300, 1024, outlier_frac=0.01), torch.bfloat16)
    w = dev(synth.weight(17, 1, 512, 1024))
    ws = torch.empty(F._lib.lib().fp4_search_workspace_size(300, 1024, 3, 100), dtype=torch.uint8, device=DEV)
    gpk = torch.empty((300, 512), dtype=torch.uint8, device=DEV)

    def run():
        c = F.fp4_calibrate(x, "column", first_rows=128)
        k, a, wp, wsc = F.fp4_preshift_weights(w, c, fe2, fe2, F.gran("row"))
        ap, _ = F.fp4_quantize_pack(x, fe2, F.gran("tensor"), tensor_scale=a, col_shift=k)
        y = F.fp4_gemm(ap, wp, wsc, fe2, F.gran("row"), K=1024, a_grid=fe2, a_scale=a, y_dtype=torch.float32)
        p16, s16 = F.fp4_quantize_pack(w, fe2, F.gran("group", 128, "f16"))
        y16 = F.fp4_gemm(x[:4], p16, s16, fe2, F.gran("group", 128, "f16"), y_dtype=torch.float32)
        res, _ = F.fp4_search_activations(x, "row", workspace=ws, packed=gpk)
        return [y, y16, res, gpk]

    eager = [t.clone() for t in run()]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = run()
    for rep in range(4):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, eager):
            assert torch.equal(got, want), rep
        run()  # eager work between replays
        torch.cuda.synchronize()


def test_repeat_runs_identical():
    x = synth.activations(3, 1, 256, 1024, outlier_frac=0.01)
    w = synth.weight(3, 1, 512, 1024)
    fe2 = F.grid_minifloat(2, 1)
    xt, wt = dev(x, torch.bfloat16), dev(w)
    outs = []
    for _ in range(2):
        c = F.fp4_calibrate(xt, "column", first_rows=128)
        k, a, wp, ws = F.fp4_preshift_weights(wt, c, fe2, fe2, F.gran("row"))
        ap, _ = F.fp4_quantize_pack(xt, fe2, F.gran("tensor"), tensor_scale=a, col_shift=k)
        y = F.fp4_gemm(ap, wp, ws, fe2, F.gran("row"), K=1024, a_grid=fe2, a_scale=a)
        outs.append([host(t).tobytes() for t in (c, k, a, wp, ws, ap, y.view(torch.int16))])
    assert outs[0] == outs[1]


@pytest.mark.parametrize("K", [9000, 17000, 13824])
def test_preshift_long_rows(K):
    """Per-row weight scales on long rows (register-resident and two-pass kernels)."""
    say("preshift long rows", K)
    x = synth.activations(5, K, 160, K, outlier_frac=0.01)
    w = synth.weight(5, K, 40, K)
    _preshift_chain(x, w)


def test_prefill_full_sampled():
    """LLaMA-13B prefill layer at full size: QKV, up, gate (K = 5120, shared activations
    and shift) and down (K = 13824): every code bit-exact, GEMM outputs bit-exact on
    sampled rows; the NF4 repeat of all four within tolerance on sampled rows."""
    e2 = O.minifloat(2, 1)
    fe2 = F.grid_minifloat(2, 1)
    rows = np.random.default_rng(1).choice(4096, 24, replace=False)
    for which, names in ((1, ("qkv", "up", "gate")), (2, ("down",))):
        x = synth.prefill_activations(which)
        for name in names:
            say("prefill", name)
            w = synth.prefill_weight(name)
            (k, a, wp, ws, ap), (gk, ga, gwp, gws, gap, fw, fgran) = _preshift_chain(x, w)
            K = w.shape[1]
            y32 = host(F.fp4_gemm(gap, gwp, gws, fw, fgran, K=K, a_grid=fe2, a_scale=ga, y_dtype=torch.float32))
            _, acc = O.gemm_w4a4(ap[rows], e2, a, wp, e2, "row", ws)
            pin = O.w4a4_epilogue_f32(acc, a, ws)
            assert np.array_equal(y32[rows].view(np.uint32), pin.view(np.uint32))
            # bf16 output (the LDS-staged epilogue): sampled rows against the oracle, the
            # whole tensor against the rounding of the fp32 output, and a second run
            # identical bit for bit (a stage overwritten while still being read would
            # show up as run-to-run differences in a few tiles)
            yb = host(F.fp4_gemm(gap, gwp, gws, fw, fgran, K=K, a_grid=fe2, a_scale=ga,
                                 y_dtype=torch.bfloat16).view(torch.int16)).view(np.uint16)
            assert np.array_equal(yb[rows], O.rne_bf16_bits(pin))
            assert np.array_equal(yb, O.rne_bf16_bits(y32))
            yb2 = host(F.fp4_gemm(gap, gwp, gws, fw, fgran, K=K, a_grid=fe2, a_scale=ga,
                                  y_dtype=torch.bfloat16).view(torch.int16)).view(np.uint16)
            assert np.array_equal(yb2, yb)
            del yb, yb2
            # the NF4 repeat of every projection
            (k, a, wp, ws, ap), (gk, ga, gwp, gws, gap, fw, fgran) = _preshift_chain(x, w, "nf4", 64)
            y32 = host(F.fp4_gemm(gap, gwp, gws, fw, fgran, K=K, a_grid=fe2, a_scale=ga, y_dtype=torch.float32))
            r, _ = O.gemm_w4a4(ap[rows], e2, a, wp, O.nf4(), "group", ws, group=64)
            S, _ = O.gemm_w4a4(ap[rows], e2, a, wp, O.nf4(), "group", ws, group=64, absolute=True)
            _check_gemm(y32[rows], r, S, depth_packed(K), None, _nf4_extra(ap[rows], a, ws, S, 64))
            del w, wp, gwp

"""Pins of the CPU oracle against facts fixed outside it (no GPU needed).

Each test checks the oracle against something other than itself: values printed on
the pages or fixed by published formats (tests/golden/), textbook rounding routines
(numpy round-half-even, frexp), exact rational arithmetic, brute-force searches with
a different structure, and invariants of the method.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows


# ---------------------------------------------------------------- grids ---------
def test_e2m1_grid_matches_published_element_type():
    want = [float(r.split()[1]) for r in _read_golden("e2m1_grid.txt")]
    assert O.minifloat_grid(2, 1).tolist() == want
    assert O.qmax(2, 1) == 6.0


def test_generic_formula_reproduces_fp16_range():
    rows = {r.split()[0]: float(r.split()[2]) for r in _read_golden("fp16_range.txt")}
    # smallest normal: p = 1, d = 0 with e=5, m=10, b=15
    assert O._c().orc_minifloat_value(5, 10, 15, 1 << 10) == rows["min_normal"]
    # IEEE reserves p = 31; its largest finite value is p = 30, d = 1023
    assert O._c().orc_minifloat_value(5, 10, 15, (30 << 10) | 1023) == rows["max_finite"]
    # the smallest subnormal is 2^-24
    assert O._c().orc_minifloat_value(5, 10, 15, 1) == 2.0 ** -24


def test_other_4bit_grids_by_hand():
    assert O.minifloat_grid(1, 2).tolist() == [0, .25, .5, .75, 1, 1.25, 1.5, 1.75]
    assert O.minifloat_grid(3, 0).tolist() == [0, 1, 2, 4, 8, 16, 32, 64]
    for e, m in O.FORMATS_4BIT:
        g = O.minifloat_grid(e, m)
        assert np.all(np.diff(g) > 0)
        assert O.qmax(e, m) == (2 - 2.0 ** -m) * 2.0 ** (2 ** e - 2)
        # E1M2 with bias 1 is a uniform 8-level grid: 0..7 steps of 1/4
    assert np.array_equal(O.minifloat_grid(1, 2) * 4, np.arange(8))


def test_bias_shifts_grid_by_power_of_two():
    # a real bias b is the canonical bias-1 grid scaled by 2^(1-b)
    for e, m in O.FORMATS_4BIT:
        for b in (-2, 0, 1, 3, 7):
            assert np.array_equal(O.minifloat_grid(e, m, b), O.minifloat_grid(e, m, 1) * 2.0 ** (1 - b))
    assert O.real_bias(1.0) == 1.0
    assert O.real_bias(0.25) == 3.0


# ----------------------------------------------------- rounding (textbook) ------
def _textbook_e2m1(y):
    """Round |y| to 1 fraction bit (normal) / step 1/2 (subnormal), ties to even,
    saturate at 6 -- IEEE-style rounding written with numpy's round-half-even."""
    y = np.abs(y.astype(np.float64))
    f, E = np.frexp(y)  # y = f * 2^E, f in [0.5, 1)
    normal = np.ldexp(np.round(f * 4) / 4, E)
    sub = np.round(y * 2) / 2
    q = np.where(y < 1.0, sub, normal)
    q = np.minimum(q, 6.0)
    return np.searchsorted(O.minifloat_grid(2, 1), q)


def _textbook_e1m2(y):
    return np.minimum(np.round(np.abs(y.astype(np.float64)) * 4), 7).astype(np.int64)


def _textbook_e3m0(y):
    """Nearest power of two (or zero), an exact midpoint going to the even code."""
    y = np.abs(y.astype(np.float64))
    out = np.zeros(y.shape, dtype=np.int64)
    # code c >= 1 has value 2^(c-1); midpoints 0.5, 1.5, 3, 6, 12, 24, 48
    mids = [0.5] + [1.5 * 2.0 ** (c - 1) for c in range(1, 7)]
    for c, t in enumerate(mids, start=1):
        out = np.where((y > t) | ((y == t) & (c % 2 == 0)), c, out)
    return out


def _interesting_values(lim, rng):
    g = np.concatenate([O.minifloat_grid(e, m) for e, m in O.FORMATS_4BIT])
    mids = np.concatenate([(O.minifloat_grid(e, m)[1:] + O.minifloat_grid(e, m)[:-1]) / 2
                           for e, m in O.FORMATS_4BIT])
    pts = np.concatenate([g, mids])
    near = np.concatenate([np.nextafter(pts.astype(np.float32), np.float32(np.inf)),
                           np.nextafter(pts.astype(np.float32), np.float32(-np.inf))])
    rnd = rng.uniform(0, lim, 20000).astype(np.float32)
    tiny = np.array([0.0, 1e-45, 1e-38, 1e-20], dtype=np.float32)
    big = np.array([1e10, 3e38, np.finfo(np.float32).max], dtype=np.float32)
    v = np.concatenate([pts.astype(np.float32), near, rnd, tiny, big]).astype(np.float32)
    v = v[v >= 0]
    return np.concatenate([v, -v])


@pytest.mark.parametrize("fmt,ref", [((2, 1), _textbook_e2m1), ((1, 2), _textbook_e1m2),
                                     ((3, 0), _textbook_e3m0)])
def test_quantize_matches_textbook_rounding(fmt, ref):
    v = _interesting_values(80.0, np.random.default_rng(7))
    codes = O.quantize(v, np.float32(1), O.minifloat(*fmt))
    assert np.array_equal(codes & 7, ref(v))
    assert np.array_equal(codes >> 3, np.signbit(v).astype(np.uint8))


def test_e2m1_tie_table():
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    got = O.minifloat_grid(2, 1)[O.quantize(ties, 1, O.minifloat(2, 1)) & 7]
    assert got.tolist() == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]


def test_golden_tiny_example():
    rows = _read_golden("e2m1_tiny.txt")
    X, C, P = [], [], []
    for r in rows:
        a, b, c = r.split("|")
        X.append([float(t) for t in a.split()])
        C.append([int(t) for t in b.split()])
        P.append([int(t, 16) for t in c.split()])
    X = np.array(X, dtype=np.float32)
    X[1, 0] = -0.0
    packed, scales = O.quantize_pack(X, O.minifloat(2, 1), "tensor")
    assert scales.tolist() == [1.0]
    assert np.array_equal(O.unpack(packed), np.array(C))
    assert np.array_equal(packed, np.array(P, dtype=np.uint8))


def test_idempotence_dequant_quant():
    rng = np.random.default_rng(3)
    scales = np.concatenate([[1.0, 0.5, 3.0], rng.uniform(1e-6, 1e3, 40)]).astype(np.float32)
    codes = np.arange(16, dtype=np.uint8)
    for e, m in O.FORMATS_4BIT:
        g = O.minifloat(e, m)
        for s in scales:
            v = (g.decode(codes).astype(np.float32) * s).astype(np.float32)
            c2 = O.quantize(v, O.reciprocal(s), g)
            assert np.array_equal(c2, codes), (e, m, s)
    g = O.nf4()
    for s in scales:
        v = (g.decode(codes).astype(np.float32) * s).astype(np.float32)
        assert np.array_equal(O.quantize(v, O.reciprocal(s), g), codes)


def test_exhaustive_tiny_tensors_bruteforce():
    """Every sign x 16 codes x random scales: quantize(+-g*s*(1+-eps)) stays on g."""
    rng = np.random.default_rng(11)
    for e, m in O.FORMATS_4BIT:
        g = O.minifloat(e, m)
        mags = g.array
        for s in rng.uniform(0.01, 10, 20).astype(np.float32):
            for sign in (1.0, -1.0):
                v = (sign * mags * s * (1 + rng.uniform(-1e-3, 1e-3, mags.size))).astype(np.float32)
                c = O.quantize(v, O.reciprocal(s), g)
                assert np.array_equal(c & 7, np.arange(8))


def test_zero_scale_gives_signed_zero_codes():
    x = np.array([[0.0, -0.0, 0.0, -0.0]], dtype=np.float32)
    packed, s = O.quantize_pack(x, O.minifloat(2, 1), "tensor")
    assert s.tolist() == [0.0]
    assert O.unpack(packed).tolist() == [[0, 8, 0, 8]]


# ---------------------------------------------------------------- pack ----------
def test_pack_layout_and_shape():
    assert O.pack(np.array([[1, 2, 15, 0]], dtype=np.uint8)).tolist() == [[0x21, 0x0F]]
    w, _ = __import__("synth").tiny()
    packed, s = O.quantize_pack(w, O.minifloat(2, 1), "tensor")
    assert packed.shape == (256, 128) and packed.dtype == np.uint8
    c = np.random.default_rng(0).integers(0, 16, (5, 12)).astype(np.uint8)
    assert np.array_equal(O.unpack(O.pack(c)), c)


# ---------------------------------------------------------------- NF4 -----------
def _inv_normal_bisect(p):
    lo, hi = -10.0, 10.0
    for _ in range(200):
        mid = (lo + hi) / 2
        if 0.5 * math.erfc(-mid / math.sqrt(2)) < p:
            lo = mid
        else:
            hi = mid
    return (lo + hi) / 2


def test_nf4_table_construction():
    G = O.nf4_table()
    assert G.shape == (16,)
    assert G[0] == -1.0 and G[-1] == 1.0
    assert np.all(np.diff(G) > 0)
    assert np.array_equal(G, -G[::-1])
    assert np.array_equal(G.astype(np.float16).astype(np.float64), G)
    z = _inv_normal_bisect(15.5 / 16)
    for i in range(16):
        q = _inv_normal_bisect((i + 0.5) / 16) / z
        assert abs(q - G[i]) <= 2.0 ** -11 * max(abs(q), 2.0 ** -14), (i, q, G[i])


def test_nf4_quantize_matches_searchsorted():
    G = O.nf4_table()
    mids = ((G[1:] + G[:-1]) / 2).astype(np.float32)
    rng = np.random.default_rng(5)
    tiny = np.array([1e-45, 5e-44, 1e-40, 1e-30, 1e-10], dtype=np.float32)  # at the zero midpoint
    y = np.concatenate([rng.uniform(-1.3, 1.3, 50000), mids, -mids, tiny, -tiny, [0.0, -0.0]]).astype(np.float32)
    got = O.quantize(y, 1, O.nf4())
    idx = np.searchsorted(mids.astype(np.float64), y.astype(np.float64), side="left")
    at_mid = np.isin(y, mids) | (y == 0)
    # at an exact midpoint between i and i+1 the even index wins
    idx = np.where(at_mid & (idx % 2 == 1), idx + 1, idx)
    assert np.array_equal(got, idx)
    # the level on the value's own side of zero wins for any tiny nonzero value
    assert O.quantize(-tiny, 1, O.nf4()).tolist() == [7] * tiny.size
    assert O.quantize(tiny, 1, O.nf4()).tolist() == [8] * tiny.size


# ---------------------------------------------------------------- bf16 / f16 ----
def test_bf16_rounding_matches_torch():
    import torch
    rng = np.random.default_rng(1)
    v = rng.standard_normal(100000).astype(np.float32) * 100
    ties = (np.arange(1, 200, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    v = np.concatenate([v, ties, -ties, [0.0, -0.0, 1e-40, 3e38]]).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.rne_bf16_bits(v), want)


# ---------------------------------------------------------------- calibration ---
def test_calibration_planted_maxima():
    rng = np.random.default_rng(2)
    x = rng.uniform(-1, 1, (300, 64)).astype(np.float32)
    x[17, 5] = -9.5
    assert O.amax_tensor(x) == np.float32(9.5)
    cols = O.amax_columns(x, 128)
    assert cols[5] == np.float32(9.5)
    x2 = x.copy()
    x2[200, 6] = 50.0  # outside the calibration rows
    assert O.amax_columns(x2, 128)[6] == cols[6] < 1
    rg = O.amax_row_groups(x, 16)
    assert rg.shape == (300, 4) and rg[17, 0] == np.float32(9.5)
    for i in range(0, 300, 37):
        for j in range(4):
            assert rg[i, j] == max(abs(float(t)) for t in x[i, 16 * j:16 * j + 16])


# ---------------------------------------------------------------- pre-shift -----
def _k_bruteforce(c, cmax):
    out = []
    for ck in c:
        if ck == 0:
            out.append(0)
            continue
        j = 1
        while math.ldexp(float(cmax), j - 1) >= float(ck):
            j -= 1
        out.append(max(j, O.K_MIN))
    return np.array(out)


def test_preshift_k_bruteforce_and_range():
    x = __import__("synth").activations(3, 9, 256, 512, outlier_frac=0.01)
    c = O.amax_columns(x, 128)
    c[3] = 0.0
    c[4] = np.float32(c.max() / 2 ** 70)
    k, a = O.preshift(c, O.minifloat(2, 1))
    assert np.array_equal(k.astype(np.int64), _k_bruteforce(c, c.max()))
    assert a == np.float32(c.max() / np.float32(6.0))
    assert np.all(k <= 0) and k[4] == O.K_MIN
    cmax = float(c.max())
    for j in range(c.size):
        if c[j] > 0 and k[j] > O.K_MIN:
            assert math.ldexp(cmax, int(k[j])) >= c[j] > math.ldexp(cmax, int(k[j]) - 1)
    # no calibrated value leaves the range after the shift
    keep = np.ones(c.size, bool)
    keep[[3, 4]] = False  # their maxima were overwritten above
    shifted = np.ldexp(np.abs(x[:128]).astype(np.float64), -k.astype(np.int64)[None, :])
    assert shifted[:, keep].max() <= cmax


def test_preshift_invariance_bitwise():
    x = __import__("synth").activations(3, 8, 64, 96, outlier_frac=0.05)
    w = __import__("synth").weight(3, 8, 40, 96)
    k, _ = O.preshift(O.amax_columns(x, 64), O.minifloat(2, 1))
    xs = np.ldexp(x, -k.astype(np.int64)[None, :]).astype(np.float32)
    ws = O.shift_weights(w, k)
    lhs = (x[:, None, :] * w[None, :, :]).sum(axis=-1, dtype=np.float32)
    rhs = (xs[:, None, :] * ws[None, :, :]).sum(axis=-1, dtype=np.float32)
    assert np.array_equal(lhs, rhs)
    assert (k != 0).any()


def test_preshift_all_zero_k_reduces_to_per_tensor():
    rng = np.random.default_rng(4)
    x = rng.uniform(-1, 1, (64, 32)).astype(np.float32)
    x[0, :] = np.linspace(0.6, 1.0, 32, dtype=np.float32)  # every channel max in (1/2, 1]
    c = O.amax_columns(x, 64)
    k, a = O.preshift(c, O.minifloat(2, 1))
    assert not k.any()
    p1, _ = O.quantize_activations(x, O.minifloat(2, 1), a, k)
    p2, _ = O.quantize_pack(x, O.minifloat(2, 1), "tensor")
    assert np.array_equal(p1, p2)


# ---------------------------------------------------------------- search --------
def test_clip_grid():
    r = O.clip_ratios()
    assert r.size == 100 and r[0] == np.float32(0.5) and r[-1] == np.float32(1.0)
    assert np.all(np.diff(r) > 0)


@pytest.mark.parametrize("fmt", O.FORMATS_4BIT)
def test_search_planted_format(fmt):
    """A tensor lying exactly on one format's grid (all magnitudes used, max at the
    top grid point) is found with MSE 0 at clip ratio 1."""
    g = O.minifloat(*fmt)
    rng = np.random.default_rng(hash(fmt) % 1000)
    s = np.float32(2.0 ** -6)  # a power of two, so amax / Qmax recovers s exactly
    codes = np.concatenate([np.arange(8), rng.integers(0, 8, 500)])
    w = (g.array[codes].astype(np.float32) * s).astype(np.float32)
    w *= np.where(rng.random(w.size) < 0.5, -1, 1).astype(np.float32)
    rec, packed, mse = O.search_tensor(w)
    assert (rec.e, rec.m) == fmt and rec.clip_index == 99 and rec.mse == 0.0
    assert rec.mse_runner_up > 0
    assert np.array_equal(O.unpack(packed.reshape(1, -1)).reshape(-1) & 7, codes)


def test_search_mse_exact_rational():
    """Each candidate's MSE equals the exact rational mean of squared errors (rounded
    once), with dequantized values from the textbook rounding routines."""
    w = __import__("synth").heavy_tail_weight(4, 99, 3, 40)
    w = w.reshape(-1)
    amax = O.amax_tensor(w)
    clips = (amax * O.clip_ratios(7)).astype(np.float32)
    mse = O.candidate_mse(w, O.FORMATS_4BIT, clips)
    refs = {(2, 1): _textbook_e2m1, (1, 2): _textbook_e1m2, (3, 0): _textbook_e3m0}
    for f, fmt in enumerate(O.FORMATS_4BIT):
        grid = O.minifloat_grid(*fmt)
        for j, c in enumerate(clips):
            s = np.float32(c / np.float32(grid[-1]))
            r = np.float32(1) / s
            y = (np.abs(w) * r).astype(np.float32)
            deq = (grid[refs[fmt](y)].astype(np.float32) * s).astype(np.float32)
            exact = sum((Fraction(float(abs(a))) - Fraction(float(d))) ** 2 for a, d in zip(w, deq))
            assert mse[f, j] == float(exact / w.size), (fmt, j)


def test_search_picks_minimum_earliest():
    w = __import__("synth").heavy_tail_weight(4, 98, 16, 64)
    rec, packed, mse = O.search_tensor(w)
    flat = mse.reshape(-1)
    best = min(range(flat.size), key=lambda i: (flat[i], i))
    assert (O.FORMATS_4BIT.index((rec.e, rec.m)), rec.clip_index) == divmod(best, 100)
    assert rec.mse == flat[best] and rec.mse_runner_up == np.sort(flat)[1]
    g = O.minifloat(rec.e, rec.m)
    assert rec.scale == np.float32(rec.clip / np.float32(g.qmax))
    assert rec.bias == 1 - math.log2(float(rec.scale))


# ---------------------------------------------------------------- GEMMs ---------
def _exact_gemm_grouped(X, V, S, group):
    M, K = X.shape
    N = V.shape[0]
    out = np.zeros((M, N))
    for i in range(M):
        for n in range(N):
            tot = Fraction(0)
            for g0 in range(0, K, group):
                part = sum(Fraction(float(X[i, k])) * Fraction(float(V[n, k]))
                           for k in range(g0, g0 + group))
                tot += Fraction(float(S[n, g0 // group])) * part
            out[i, n] = float(tot)
    return out


def test_w4a16_group_gemm_exact_rational():
    rng = np.random.default_rng(9)
    w = rng.normal(0, 0.02, (5, 16)).astype(np.float32)
    x = __import__("synth").to_bf16_values(rng.normal(0, 1, (3, 16)).astype(np.float32))
    g = O.minifloat(2, 1)
    packed, s16 = O.quantize_pack(w, g, "group", group=8, scale_dtype="f16")
    r = O.gemm_w4a16(x, packed, g, "group", s16, group=8)
    V = g.decode(O.unpack(packed))
    ref = _exact_gemm_grouped(x, V, s16.astype(np.float64), 8)
    assert np.max(np.abs(r - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_w4a4_factoring_identity_integer():
    """W4A4 E2M1 = (integer code product) x scales, exactly: twice every E2M1 value is
    an integer, so the code GEMM is an int64 matmul divided by 4."""
    rng = np.random.default_rng(10)
    g = O.minifloat(2, 1)
    A = rng.integers(0, 16, (7, 64)).astype(np.uint8)
    W = rng.integers(0, 16, (9, 64)).astype(np.uint8)
    s = rng.uniform(0.001, 0.01, 9).astype(np.float32)
    a = np.float32(0.37)
    r, acc = O.gemm_w4a4(O.pack(A), g, a, O.pack(W), g, "row", s)
    Ai = (g.decode(A) * 2).astype(np.int64)
    Wi = (g.decode(W) * 2).astype(np.int64)
    assert np.array_equal(acc * 4, (Ai @ Wi.T).astype(np.float64))
    y = O.w4a4_epilogue_f32(acc, a, s)
    for i in range(7):
        for n in range(9):
            assert y[i, n] == np.float32(np.float32(acc[i, n]) * np.float32(a * s[n]))


def test_nf4_gemm_exact_rational():
    rng = np.random.default_rng(12)
    g4 = O.nf4()
    ge = O.minifloat(2, 1)
    A = rng.integers(0, 16, (2, 16)).astype(np.uint8)
    W = rng.normal(0, 0.02, (3, 16)).astype(np.float32)
    pw, sw = O.quantize_pack(W, g4, "group", group=8)
    a = np.float32(0.11)
    r, _ = O.gemm_w4a4(O.pack(A), ge, a, pw, g4, "group", sw, group=8)
    ref = _exact_gemm_grouped(ge.decode(A), g4.decode(O.unpack(pw)), sw.astype(np.float64), 8)
    assert np.max(np.abs(r - ref * float(a))) <= 1e-12 * np.max(np.abs(ref))


def test_rel_err_definition():
    assert O.rel_err(np.array([1.0, 2.0]), np.array([1.0, 2.002])) == pytest.approx(0.002 / 2.002)


# ---------------------------------------------------- SwiGLU + fused quantization -----
def test_exp_f32_against_math_exp():
    """exp_f32 is e^x to the stated accuracy (the rounding of x * log2 e dominates), exact
    at 0, and its Horner coefficients are the Taylor coefficients of 2^f."""
    assert O.exp_f32(np.float32(0.0)) == np.float32(1.0)
    assert O.EXP2_COEF_F32[0] == np.float32(1.0) and abs(float(O.EXP2_COEF_F32[1]) - math.log(2)) < 1e-7
    x = np.linspace(-87.0, 88.0, 100001).astype(np.float32)
    r = np.array([math.exp(float(v)) for v in x[::97]])
    assert np.max(np.abs(O.exp_f32(x[::97]).astype(np.float64) - r) / r) < 5e-6
    xs = np.linspace(-10.0, 10.0, 20001).astype(np.float32)
    rs = np.exp(xs.astype(np.float64))
    assert np.max(np.abs(O.exp_f32(xs).astype(np.float64) - rs) / rs) < 1e-6
    # e^x e^-x = 1 and e^1 = e, to binary32 accuracy
    assert np.max(np.abs(O.exp_f32(xs).astype(np.float64) * O.exp_f32(-xs) - 1.0)) < 2e-6
    assert abs(float(O.exp_f32(np.float32(1.0))) - math.e) < 4e-7


def test_silu_f32_closed_forms():
    """SiLU(0) = +-0, SiLU(x) - SiLU(-x) = x, SiLU -> x for large x and -> -0 for very
    negative x, and x / (1 + e^-x) in binary64 to 1e-6 relative."""
    z = O.silu_f32(np.array([0.0, -0.0], np.float32))
    assert z[0] == 0 and z[1] == 0 and not np.signbit(z[0]) and np.signbit(z[1])
    x = np.linspace(-12.0, 12.0, 4801).astype(np.float32)
    d = O.silu_f32(x).astype(np.float64) - O.silu_f32(-x)
    assert np.max(np.abs(d - x)) <= 2e-6 * np.max(np.abs(x))
    big = O.silu_f32(np.array([100.0, 1000.0, -200.0, -1e30], np.float32))
    assert big[0] == 100.0 and big[1] == 1000.0 and big[2] == 0 and big[3] == 0 and np.signbit(big[3])
    r = x.astype(np.float64) / (1.0 + np.exp(-x.astype(np.float64)))
    m = np.abs(r) > 1e-20
    assert np.max(np.abs(O.silu_f32(x)[m] - r[m]) / np.abs(r[m])) < 1e-6


def test_swiglu_quant_composition_by_hand():
    """A 3x4 output with K = 32 from hand-made codes: gate and up computed directly from
    the grid values in binary64, h = SiLU(gate) * up, then the next layer's activation
    codes: matches w4a4_swiglu_quant except where h lies within 1e-5 of a rounding
    midpoint (none here); swapping gate and up, or applying SiLU to up, changes codes."""
    rng = np.random.default_rng(7)
    e2 = O.minifloat(2, 1)
    M, N, K = 3, 4, 32
    a_codes = rng.integers(0, 16, (M, K)).astype(np.uint8)
    g_codes = rng.integers(0, 16, (N, K)).astype(np.uint8)
    u_codes = rng.integers(0, 16, (N, K)).astype(np.uint8)
    pk = lambda c: (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    a = np.float32(0.0625)
    sg = np.array([0.5, 0.25, 1.0, 0.125], np.float32)
    su = np.array([0.25, 0.5, 0.125, 1.0], np.float32)
    out_a = np.float32(0.5)
    k = np.array([0, -1, 0, -2], np.int8)
    codes, h = O.w4a4_swiglu_quant(pk(a_codes), a, pk(g_codes), sg, pk(u_codes), su, out_a, k)
    val = lambda c: e2.decode(c).astype(np.float64)
    yg = (val(a_codes) @ val(g_codes).T) * (float(a) * sg.astype(np.float64))
    yu = (val(a_codes) @ val(u_codes).T) * (float(a) * su.astype(np.float64))
    h64 = yg / (1.0 + np.exp(-yg)) * yu
    assert np.max(np.abs(h - h64)) <= 1e-5 * np.max(np.abs(h64))
    want, _ = O.quantize_activations(h64.astype(np.float32), e2, out_a, k)
    assert np.array_equal(codes, want)
    swapped, _ = O.w4a4_swiglu_quant(pk(a_codes), a, pk(u_codes), su, pk(g_codes), sg, out_a, k)
    assert not np.array_equal(swapped, codes)


# ---- the search on activations: per-token units and calibration-token units ----------
def _planted_row(rng, fmt, cols, scale_exp):
    """A row of exact grid values of one format times 2^scale_exp, every magnitude code
    present and the largest attained: the clip-1.0 candidate of that format reproduces
    it with zero error, and no other format's grid holds all its ratios."""
    g = O.minifloat(*fmt)
    codes = np.concatenate([np.arange(8), rng.integers(0, 8, cols - 8)])
    rng.shuffle(codes)
    sign = np.where(rng.random(cols) < 0.5, -1.0, 1.0)
    return (g.array[codes] * sign * 2.0 ** scale_exp).astype(np.float32), codes


def test_search_activations_per_row_recovers_each_rows_format():
    rng = np.random.default_rng(21)
    fmts = [(1, 2), (2, 1), (3, 0), (2, 1), (1, 2)]
    rows = [_planted_row(rng, f, 64, -3 - i) for i, f in enumerate(fmts)]
    x = np.stack([r for r, _ in rows])
    recs, packed = O.search_activations(x, "row", nclips=8)
    assert packed.shape == (5, 32)
    for i, (f, rec) in enumerate(zip(fmts, recs)):
        assert (rec.e, rec.m, rec.clip_index, rec.mse) == (f[0], f[1], 7, 0.0)
        assert rec.scale == np.float32(2.0 ** (-3 - i))  # largest grid value x 2^e / Qmax
        mag = O.unpack(packed[i]) & 7
        assert np.array_equal(mag, rows[i][1])


def test_search_activations_calibration_rows_decide_every_row():
    """Unit 'tensor' with T calibration rows: the winner comes from rows [0, T) only
    (E3M0 at scale 2^-5), and every row -- the ones past T included -- is packed with it:
    a row of E1M2 values k 2^-5 (k = 0..7) maps to the E3M0 values 0, 1, 2, 2, 4, 4, 8, 8
    (3 and 6 are ties, each to the even code), values beyond the clip saturate at code 7."""
    rng = np.random.default_rng(22)
    calib = np.stack([_planted_row(rng, (3, 0), 48, -5)[0] for _ in range(3)])
    later, later_codes = _planted_row(rng, (1, 2), 48, -3)
    big = np.full(48, 1000.0, np.float32)
    big[::2] = -1000.0
    x = np.concatenate([calib, later[None], big[None]])
    recs, packed = O.search_activations(x, "tensor", first_rows=3, nclips=4)
    assert len(recs) == 1
    rec = recs[0]
    assert (rec.e, rec.m, rec.clip_index, rec.mse) == (3, 0, 3, 0.0)
    assert rec.scale == np.float32(2.0 ** -5)
    codes = O.unpack(packed)
    e3m0 = O.minifloat(3, 0).array
    assert np.array_equal(e3m0[codes[3] & 7], np.array([0, 1, 2, 2, 4, 4, 8, 8], np.float32)[later_codes])
    assert np.array_equal(codes[3] >> 3, np.signbit(later).astype(np.uint8))  # -0 keeps its sign
    assert np.all(codes[4] & 7 == 7) and np.array_equal(codes[4] >> 3, (np.arange(48) % 2 == 0).astype(np.uint8))
    # taking the E1M2 row into the calibration set makes E3M0 at that scale inexact
    recs_all, _ = O.search_activations(x[:4], "tensor", nclips=4)
    assert recs_all[0].mse > 0.0


# ---- two-mode grid: E2M1 or E1M2 per group, the mode in the scale's sign bit ----------
def test_two_mode_planted_groups():
    """A group of exact E1M2 multiples (every magnitude present) has zero error only in
    E1M2; a group of exact E2M1 multiples only in E2M1; an all-zero group ties and keeps
    E2M1 with scale +0.  Codes, scales and dequantized values follow exactly."""
    rng = np.random.default_rng(31)
    e1m2 = _planted_row(rng, (1, 2), 32, -4)
    e2m1 = _planted_row(rng, (2, 1), 32, 2)
    x = np.stack([np.concatenate([e1m2[0], e2m1[0], np.zeros(32, np.float32)])])
    packed, scales, modes = O.quantize_two_mode(x, 32)
    assert modes.tolist() == [[1, 0, 0]]
    assert scales[0, 0] == np.float32(-(1.75 * 2.0 ** -4) / np.float32(1.75))
    assert scales[0, 0] == np.float32(-(2.0 ** -4)) and scales[0, 1] == np.float32(4.0)
    assert scales[0, 2] == 0.0 and not np.signbit(scales[0, 2])
    codes = O.unpack(packed)[0]
    assert np.array_equal(codes[:32] & 7, e1m2[1]) and np.array_equal(codes[32:64] & 7, e2m1[1])
    assert np.array_equal(O.two_mode_values(packed, scales, 32), x)


def test_two_mode_choice_by_hand():
    """Group [1.0, 0.3]: E2M1 (s = 1/6) stores 0.3 as 2/6 (error about 1.1e-3), E1M2
    (s = 1/1.75) as 0.5/1.75 (error about 2.0e-4): E1M2 wins.  Group [1.0, 0.38]: E2M1
    gives 2/6 (error 2.2e-3), E1M2 0.75/1.75 (error 2.5e-3): E2M1 wins."""
    x = np.array([[1.0, 0.3, 1.0, 0.38]], np.float32)
    packed, scales, modes = O.quantize_two_mode(x, 2)
    assert modes.tolist() == [[1, 0]]
    v = O.two_mode_values(packed, scales, 2)[0]
    assert abs(v[1] - 0.5 / 1.75) < 1e-7 and abs(v[3] - 2.0 / 6.0) < 1e-7
    e2 = O.two_mode_error(x[0, :2], np.array([7, 4]), np.float32(1) / np.float32(6), O.minifloat(2, 1))
    e1 = O.two_mode_error(x[0, :2], np.array([7, 2]), np.float32(1) / np.float32(1.75), O.minifloat(1, 2))
    assert abs(e2 - (0.3 - 1 / 3) ** 2) < 1e-8 and abs(e1 - (0.3 - 0.5 / 1.75) ** 2) < 1e-8 and e1 < e2


def test_two_mode_f16_scales_and_gemm_special_cases():
    """f16 scales store the rounded scale with the mode in its sign; when every group takes
    one mode the two-mode product equals the plain W4A16 product on that grid."""
    rng = np.random.default_rng(32)
    w = np.stack([_planted_row(rng, (2, 1), 64, -3)[0] for _ in range(3)])
    packed, scales, modes = O.quantize_two_mode(w, 32, "f16")
    assert scales.dtype == np.float16 and not modes.any()
    x = rng.normal(size=(4, 64)).astype(np.float32)
    r2 = O.gemm_w4a16_two_mode(x, packed, scales, 32)
    r = O.gemm_w4a16(x, packed, O.minifloat(2, 1), "group", np.abs(scales.astype(np.float32)), 32)
    assert np.array_equal(r2, r)
    w1 = np.stack([_planted_row(rng, (1, 2), 64, -6)[0] for _ in range(3)])
    p1, s1, m1 = O.quantize_two_mode(w1, 32, "f16")
    assert m1.all() and np.all(np.signbit(s1))
    r1 = O.gemm_w4a16_two_mode(x, p1, s1, 32)
    assert np.array_equal(r1, O.gemm_w4a16(x, p1, O.minifloat(1, 2), "group", np.abs(s1.astype(np.float32)), 32))


# ---- FP8 grids (OCP E4M3 / E5M2) ---------------------------------------------------
def test_fp8_grids_match_the_ocp_definition():
    """Facts of the OCP 8-bit formats: E4M3 has 127 magnitudes from the subnormal 2^-9 to
    448 (min normal 2^-6); E5M2 124 from 2^-16 to 57344 (min normal 2^-14)."""
    g4, g5 = O.fp8(4, 3), O.fp8(5, 2)
    a4, a5 = g4.array, g5.array
    assert len(a4) == 127 and a4[0] == 0 and a4[1] == 2.0 ** -9 and a4[8] == 2.0 ** -6 and a4[-1] == 448.0
    assert len(a5) == 124 and a5[1] == 2.0 ** -16 and a5[4] == 2.0 ** -14 and a5[-1] == 57344.0
    assert np.all(np.diff(a4) > 0) and np.all(np.diff(a5) > 0)
    assert g4.bits == 8 and O.minifloat(2, 1).bits == 4


@pytest.mark.parametrize("fmt,vals,codes", [
    ((4, 3), [1.0, 0.1, 1.0625, 1.1875, 500.0, -0.0, -3.0, 2.0 ** -10, 3 * 2.0 ** -10],
     [0x38, 0x1D, 0x38, 0x3A, 0x7E, 0x80, 0xC4, 0x00, 0x02]),
    ((5, 2), [1.0, 1.125, 60000.0, -2.0 ** -17, 3 * 2.0 ** -17, 0.75],
     [0x3C, 0x3C, 0x7B, 0x80, 0x02, 0x3A]),
])
def test_fp8_codes_by_hand(fmt, vals, codes):
    """Nearest value with exact ties to the even code (1.0625 and 1.1875 in E4M3, 1.125
    in E5M2, the subnormal midpoints), saturation at the largest finite value, sign of -0."""
    g = O.fp8(*fmt)
    got = O.quantize(np.array(vals, np.float32), np.ones(len(vals), np.float32), g)
    assert [int(c) for c in got] == codes


def test_fp8_fp6_round_trip_and_product():
    """Grid values times a power-of-two scale quantize to themselves (dequantize is exact),
    and the W8A16 / W6A16 product of such a weight is the dense product."""
    rng = np.random.default_rng(41)
    for g in (O.fp8(4, 3), O.fp8(5, 2), O.fp6(2, 3), O.fp6(3, 2)):
        idx = rng.integers(0, len(g.values), (6, 64))
        idx[:, ::32] = len(g.values) - 1  # every group's largest magnitude is the grid's
        w = (g.array[idx] * np.where(rng.random((6, 64)) < 0.5, -1, 1) * 2.0 ** -10).astype(np.float32)
        packed, sc = O.quantize_pack(w, g, "group", group=32)
        assert packed.shape == (6, 64 * g.bits // 8) and np.array_equal(sc, np.full((6, 2), 2.0 ** -10, np.float32))
        assert np.array_equal(O.dequantize(packed, g, "group", sc, group=32), w)
        x = rng.normal(size=(3, 64)).astype(np.float32)
        r = O.gemm_w4a16(x, packed, g, "group", sc, group=32)
        assert np.allclose(r, x.astype(np.float64) @ w.astype(np.float64).T, rtol=0, atol=1e-12)


# ---- FP6 grids (OCP E2M3 / E3M2), packed four codes in three bytes -------------------
def test_fp6_grids_and_packing():
    """E2M3: 32 magnitudes in steps of 1/8 below 1, largest 7.5; E3M2: smallest subnormal
    1/16, largest 28.  Codes by hand (ties to even, saturation, sign in bit 5) and the
    bit-stream packing of four codes into three bytes."""
    g23, g32 = O.fp6(2, 3), O.fp6(3, 2)
    assert len(g23.values) == 32 and g23.array[1] == 0.125 and g23.array[8] == 1.0 and g23.array[-1] == 7.5
    assert len(g32.values) == 32 and g32.array[1] == 0.0625 and g32.array[4] == 0.25 and g32.array[-1] == 28.0
    assert g23.bits == 6 and g32.bits == 6
    vals = np.array([1.0, 1.0625, 1.1875, 9.0, -0.0, -0.1875, 0.0625, 3.3], np.float32)
    c = O.quantize(vals, np.ones(8, np.float32), g23)
    # 1.0625 ties 1.0/1.125 -> 1.0 (even code 8); 1.1875 ties 1.125/1.25 -> 1.25 (code 10);
    # -0.1875 ties 0.125/0.25 -> 0.25 (code 2); 0.0625 ties 0/0.125 -> 0; 3.3 -> 3.25
    assert [int(v) for v in c] == [8, 8, 10, 31, 32, 32 | 2, 0, 21]
    codes = np.array([[1, 2, 3, 4, 63, 0, 32, 5]], np.uint8)
    packed = O.pack_codes(codes, g23)
    v = 1 | 2 << 6 | 3 << 12 | 4 << 18
    assert packed[0, :3].tolist() == [v & 255, (v >> 8) & 255, v >> 16]
    v = 63 | 0 << 6 | 32 << 12 | 5 << 18
    assert packed[0, 3:].tolist() == [v & 255, (v >> 8) & 255, v >> 16]
    assert np.array_equal(O.unpack_codes(packed, g23), codes)


# ---- per-token activation scales in the W4A4 product ---------------------------------
def test_w4a4_per_token_scales():
    """With one scale per token the product is the per-tensor one row by row: equal
    scales reproduce the per-tensor result bit for bit, and power-of-two scales scale
    each output row exactly."""
    rng = np.random.default_rng(51)
    e2 = O.minifloat(2, 1)
    ap = rng.integers(0, 256, (6, 64), dtype=np.uint8)
    wp = rng.integers(0, 256, (5, 64), dtype=np.uint8)
    ws = rng.uniform(0.5, 2.0, 5).astype(np.float32)
    r1, acc = O.gemm_w4a4(ap, e2, np.float32(0.75), wp, e2, "row", ws)
    rr, _ = O.gemm_w4a4(ap, e2, np.full(6, 0.75, np.float32), wp, e2, "row", ws)
    assert np.array_equal(r1, rr)
    y1 = O.w4a4_epilogue_f32(acc, np.float32(0.75), ws)
    assert np.array_equal(O.w4a4_epilogue_f32(acc, np.full(6, 0.75, np.float32), ws), y1)
    p2 = (2.0 ** np.arange(-3, 3)).astype(np.float32)
    rp, _ = O.gemm_w4a4(ap, e2, p2, wp, e2, "row", ws)
    r_unit, _ = O.gemm_w4a4(ap, e2, np.float32(1.0), wp, e2, "row", ws)
    assert np.array_equal(rp, r_unit * p2[:, None].astype(np.float64))
    yp = O.w4a4_epilogue_f32(acc, p2, ws)
    yu = O.w4a4_epilogue_f32(acc, np.float32(1.0), ws)
    assert np.array_equal(yp, (yu * p2[:, None]).astype(np.float32))


# ------------------------------------- ROW / GROUP quantize, binary16, dequantize --------
def _hexf32(tok):
    return np.uint32(int(tok, 16)).view(np.float32)


def _group_golden():
    X, C, P, S = [], [], [], []
    for r in _read_golden("quantize_group_f16.txt"):
        a, b, c, d = r.split("|")
        X.append([np.float32(t) if t != "-0.0" else np.float32(-0.0) for t in a.split()])
        C.append([int(t) for t in b.split()])
        P.append([int(t, 16) for t in c.split()])
        S.append([int(t, 16) for t in d.split()])
    return (np.array(X, np.float32), np.array(C, np.uint8), np.array(P, np.uint8), np.array(S, np.uint16))


def _row_golden():
    X, C, P, S = [], [], [], []
    for r in _read_golden("quantize_row_f32.txt"):
        a, b, c, d = r.split("|")
        X.append([np.float32(t) for t in a.split()])
        C.append([int(t) for t in b.split()])
        P.append([int(t, 16) for t in c.split()])
        S.append(int(d.strip(), 16))
    return (np.array(X, np.float32), np.array(C, np.uint8), np.array(P, np.uint8), np.array(S, np.uint32))


def _matches_group_golden(quantize_pack):
    x, codes, packed, sbits = _group_golden()
    p, s = quantize_pack(x, O.minifloat(2, 1), "group", 8, "f16")
    return (np.array_equal(p, packed) and np.array_equal(O.unpack(p), codes)
            and np.array_equal(np.asarray(s).view(np.uint16).reshape(sbits.shape), sbits))


def test_group_f16_quantize_golden():
    """GROUP quantization with stored binary16 scales against a hand-worked 2x16 case."""
    assert _matches_group_golden(O.quantize_pack)


def test_row_quantize_golden():
    x, codes, packed, sbits = _row_golden()
    p, s = O.quantize_pack(x, O.minifloat(2, 1), "row")
    assert np.array_equal(O.unpack(p), codes)
    assert np.array_equal(p, packed)
    assert np.array_equal(np.asarray(s, np.float32).view(np.uint32), sbits)


def test_rne_f16_golden():
    rows = [r.split("|") for r in _read_golden("rne_f16.txt")]
    src = np.array([int(a, 16) for a, _, _ in rows], dtype=np.uint32).view(np.float32)
    want = np.array([int(b, 16) for _, b, _ in rows], dtype=np.uint16)
    with np.errstate(over="ignore"):
        got = O.rne_f16(src).view(np.uint16)
    assert np.array_equal(got, want), [(hex(a), hex(b)) for a, b in zip(got, want) if a != b]


def _dequant_golden():
    out = []
    for r in _read_golden("dequantize_e2m1.txt"):
        mode, sc, cs, vs = [t.strip() for t in r.split("|")]
        codes = np.array([int(t) for t in cs.split()], np.uint8).reshape(1, -1)
        vals = np.array([int(t, 16) for t in vs.split()], np.uint32)
        out.append((mode, sc.split(), codes, vals))
    return out


def test_dequantize_golden():
    for mode, sc, codes, vals in _dequant_golden():
        packed = O.pack(codes)
        if mode == "tensor":
            v = O.dequantize(packed, O.minifloat(2, 1), "tensor", np.array([_hexf32(sc[0])], np.float32))
        else:
            s16 = np.array([int(t, 16) for t in sc], np.uint16).view(np.float16).reshape(1, -1)
            v = O.dequantize(packed, O.minifloat(2, 1), "group", s16, group=8)
        assert np.array_equal(np.asarray(v, np.float32).reshape(-1).view(np.uint32), vals), mode


class _NumpyTiledScales:
    """numpy, except that repeat along axis 1 tiles instead (scales laid out
    [s0, s1, s0, s1, ...] instead of [s0 x group, s1 x group]): a planted mistake."""

    def __getattr__(self, k):
        return getattr(np, k)

    @staticmethod
    def repeat(a, n, axis=None):
        if axis == 1:
            return np.tile(np.asarray(a), (1, n))
        return np.repeat(a, n, axis=axis)


def test_planted_oracle_mistakes_fail_the_pins(monkeypatch):
    """Each plausible mistake in the ROW/GROUP quantizer and the dequantizer, planted in the
    oracle on the CPU, fails a golden pin above."""
    # 1. group scales tiled instead of repeated along the row
    with monkeypatch.context() as m:
        m.setattr(O, "np", _NumpyTiledScales())
        assert not _matches_group_golden(O.quantize_pack)
    # 2. quantizing with the unrounded fp32 scale instead of the stored binary16 one
    with monkeypatch.context() as m:
        m.setattr(O, "rne_f16", lambda v: np.asarray(v, np.float32))
        x, codes, _, _ = _group_golden()
        p, _ = O.quantize_pack(x, O.minifloat(2, 1), "group", 8, "f16")
        assert not np.array_equal(O.unpack(p), codes)
    # 3. x / s in place of x * fl32(1/s) changes no code of these cases, but dropping the
    #    sign of zero does: codes of -0.0 and of negatives rounding to 0 must be 8
    x, codes, _, _ = _row_golden()
    c = O.quantize(np.abs(x), 1, O.minifloat(2, 1))
    assert not np.array_equal(c, codes)
    # 4. dequantize with tiled scales, or with the sign bit ignored
    (_, _, c_t, v_t), (_, sc_g, c_g, v_g) = _dequant_golden()
    s16 = np.array([int(t, 16) for t in sc_g], np.uint16).view(np.float16).reshape(1, -1)
    with monkeypatch.context() as m:
        m.setattr(O, "np", _NumpyTiledScales())
        v = O.dequantize(O.pack(c_g), O.minifloat(2, 1), "group", s16, group=8)
        assert not np.array_equal(np.asarray(v, np.float32).reshape(-1).view(np.uint32), v_g)
    v = O.dequantize(O.pack(c_t & 7), O.minifloat(2, 1), "tensor", np.array([_hexf32("3e4ccccd")], np.float32))
    assert not np.array_equal(np.asarray(v, np.float32).reshape(-1).view(np.uint32), v_t)
    # 5. a double rounding binary64 -> binary32 -> binary16 is caught by the tie rows
    assert O.rne_f16(np.float32(1 + 2.0 ** -11)).view(np.uint16) == 0x3C00


# ------------------------------------------------ elementwise GEMM error bounds ---------
def test_absolute_gemm_is_the_sum_of_magnitudes():
    rng = np.random.default_rng(4)
    e2 = O.minifloat(2, 1)
    w = rng.normal(0, 1, (6, 64)).astype(np.float32)
    x = rng.normal(0, 1, (3, 64)).astype(np.float32)
    p, s = O.quantize_pack(w, e2, "group", 32)
    V = e2.decode(O.unpack(p)) * np.repeat(s.astype(np.float64), 32, axis=1)
    want = np.abs(x.astype(np.float64)) @ np.abs(V).T
    assert np.allclose(O.gemm_w4a16(x, p, e2, "group", s, 32, absolute=True), want, rtol=1e-15, atol=0)
    # with non-negative operands the two agree; otherwise |r| <= S
    r = O.gemm_w4a16(x, p, e2, "group", s, 32)
    assert np.all(np.abs(r) <= want * (1 + 1e-15))
    pa = O.pack(O.unpack(p) & 7)
    assert np.array_equal(O.gemm_w4a16(np.abs(x), pa, e2, "group", s, 32),
                          O.gemm_w4a16(np.abs(x), pa, e2, "group", s, 32, absolute=True))
    ap, asc = O.quantize_pack(x, e2, "tensor")
    ra, _ = O.gemm_w4a4(ap, e2, asc[0], p, e2, "group", s, group=32, absolute=True)
    A = e2.decode(O.unpack(ap)) * float(asc[0])
    assert np.allclose(ra, np.abs(A) @ np.abs(V).T, rtol=1e-15, atol=0)


def test_elementwise_bound_holds_for_binary32_summation_and_catches_an_error():
    """Recursive binary32 summation of K exact products stays within d = K of the bound;
    one output perturbed by 1e-3 of a small value's magnitude sum is flagged."""
    rng = np.random.default_rng(5)
    K = 4096
    x = rng.normal(0, 1, (8, K)).astype(np.float32)
    w = rng.normal(0, 1, (16, K)).astype(np.float32)
    xb = O.bf16_bits_to_f32(O.rne_bf16_bits(x))
    wq = (np.round(w * 2) / 2).astype(np.float32)  # products of bf16 and half-integers: exact
    r = xb.astype(np.float64) @ wq.astype(np.float64).T
    S = np.abs(xb).astype(np.float64) @ np.abs(wq).astype(np.float64).T
    y = np.zeros(r.shape, np.float32)
    for k in range(K):  # one rounding per addition
        y = (y + (xb[:, k:k + 1] * wq[None, :, k]).reshape(8, 16)).astype(np.float32)
    assert O.elementwise_excess(y, r, K * O.U32 * S) <= 1.0
    y2 = y.copy()
    y2[3, 5] += np.float32(1e-3 * S[3, 5])
    assert O.elementwise_excess(y2, r, K * O.U32 * S) > 1.0


def test_bf16_ulp_distance():
    r = np.array([1.0, 1.0 + 2.0 ** -9, 3.0, -2.5], np.float64)  # 1 + 2^-9: tie -> 1.0
    S = np.abs(r)
    bits = O.rne_bf16_bits(np.array([1.0, 1.0, 3.0 + 2 ** -6, -2.5], np.float32))
    # 3 + 2^-6 is one bf16 ulp (2^-6 at 2..4) above 3.0
    assert O.bf16_ulps_from_rounded(bits, r, 0 * S) == (1, 4)
    far = O.rne_bf16_bits(np.array([1.0, 1.0, 3.0, -2.5 - 2 ** -5], np.float32))
    assert O.bf16_ulps_from_rounded(far, r, 0 * S) == (2, 4)
    # outputs whose binary32 bound exceeds a quarter ulp are not checked
    assert O.bf16_ulps_from_rounded(far, r, S * 1e-2)[1] == 0

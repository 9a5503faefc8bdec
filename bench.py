#!/usr/bin/env python3
"""Benchmark of the FP4 quantize + quantized-GEMM hot path on one MI355X.

Headline line: the LLaMA-7B decode workload -- weight 11008x4096 (N(0, 0.02) fp32)
quantized to E2M1 with fp16 scales per 128 along K (calibration fused), then the W4A16
decode GEMV at M = 1, 4 and 16 (bf16 activations, bf16 output).  One step = one weight
quantize + the three GEMVs; value = algorithmic HBM bytes of the step / step time.
Inputs are resident in HBM before the timed region; weight copies rotate (2 fp32
copies, 16 packed copies) so no step reads data the 256 MB Infinity Cache still holds
from the previous step.  The K timed steps run as one captured HIP graph (launch
overhead excluded; the graph's outputs are checked against an eager run).

Also measured in the same run, each against its own roofline (the "kernels" list):
the 2048x4096x4096 calibration + pre-shift + W4A4 GEMM, the LLaMA-13B prefill layer
(QKV / up / gate / down W4A4 GEMMs with pre-shifted E2M1, and the NF4 repeat), and the
format/clip search over 32 heavy-tailed 4096x4096 tensors.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--main-only]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP4 quantize GB/s + W4A16/W4A4 GEMM TFLOP/s, % of MI355X roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP4_PEAK_TFLOPS = 10100.0      # dense FP4 MFMA
F16_PEAK_TFLOPS = 2500.0       # dense f16/bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0       # dense FP8 MFMA
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12  # lane-instructions/s: 256 CU x 4 SIMD x 16 lanes x 2.4 GHz


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--main-only", action="store_true", help="only the headline decode workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", choices=["decode", "quantize", "all"], default=None,
                    help="short run for rocprofv3: a few eager launches, no JSON line")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"), default=None,
                    help="turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) of "
                         "'bench.py --profile all' into profiles/traffic.json (no GPU needed)")
    return ap.parse_args()


# ----------------------------------------------------------------------------- timing
def graph_time(torch, fn, iters: int, reps: int = 3) -> float:
    """Seconds per iteration of fn(i), i < iters, captured into one HIP graph and
    replayed; events are recorded on the stream the kernels run on."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(iters):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        st = torch.cuda.current_stream()
        e0.record(st)
        g.replay()
        e1.record(st)
        e1.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e-3 / iters)
    return best


ROTATE_BYTES = 512 * 1024 * 1024  # rotated working set: twice the 256 MB Infinity Cache


def rotations(nbytes: int, least: int = 2) -> int:
    """Distinct input copies to rotate so that the copies together pass ROTATE_BYTES (no
    launch reads data the Infinity Cache still holds from an earlier one)."""
    return max(least, -(-ROTATE_BYTES // max(int(nbytes), 1)))


def clones(t, n):
    return [t] + [t.clone() for _ in range(n - 1)]


_BENCH_LIB = None


def stream_read_ceiling(torch, nbytes: int):
    """Seconds per launch of a plain streaming read of nbytes (whole-line nontemporal 16-byte
    loads, libfp4_bench.so) over rotating buffers, in the graph harness of the kernels:
    the attainable HBM rate for a kernel that moves that many bytes."""
    import ctypes
    global _BENCH_LIB
    if _BENCH_LIB is None:
        _BENCH_LIB = ctypes.CDLL(os.path.join(ROOT, "bit_floating_point_amd", "libfp4_bench.so"))
        _BENCH_LIB.fp4bench_stream_read.restype = ctypes.c_int
        _BENCH_LIB.fp4bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    n = rotations(nbytes)
    bufs = [torch.full((nbytes,), 1, dtype=torch.uint8, device="cuda") for _ in range(n)]
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")

    def fn(i):
        st = torch.cuda.current_stream().cuda_stream
        rc = _BENCH_LIB.fp4bench_stream_read(bufs[i % n].data_ptr(), nbytes, sink.data_ptr(), st)
        assert rc == 0, rc
    t = graph_time(torch, fn, 64)
    del bufs
    return t


def roofline_entry(name, bound, achieved, peak, unit, seconds, work, work_unit, traffic=None, **extra):
    d = {"kernel": name, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4), "us_per_launch": round(seconds * 1e6, 3), "work_per_launch": work,
         "work_unit": work_unit, "traffic": traffic}
    d.update(extra)
    return d


# ----------------------------------------------------------------------------- inputs
def gen_normal(torch, shape, std, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32) * std


def gen_activations(torch, rows, cols, seed, outlier_frac=0.01, gain=50.0):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn((rows, cols), generator=g, device="cuda", dtype=torch.float32)
    n_out = int(round(outlier_frac * cols))
    if n_out:
        idx = torch.randperm(cols, generator=g, device="cuda")[:n_out]
        x[:, idx] *= gain
    return x.to(torch.bfloat16)


def gen_heavy_tail(torch, shape, seed, std=0.02, p_tail=0.05):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    z = torch.randn(shape, generator=g, device="cuda")
    chi = sum(torch.randn(shape, generator=g, device="cuda") ** 2 for _ in range(4))
    t4 = torch.randn(shape, generator=g, device="cuda") / torch.sqrt(chi / 4)
    sel = torch.rand(shape, generator=g, device="cuda") < p_tail
    return torch.where(sel, t4, z) * std


# ----------------------------------------------------------------------------- traffic
def traffic_for(kernel_file: str, key: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if the kernel source
    is unchanged since they were taken (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(key)
    if not rec:
        return None
    src = os.path.join(ROOT, "bit_floating_point_amd", "csrc", kernel_file)
    h = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if rec.get("source_sha256") != h:
        return None
    return rec.get("bytes_per_launch")


# Dispatches of `bench.py --profile all`, in launch order: (key, kernel file, kernel-name
# fragment, index range among the dispatches whose name has that fragment).
TRAFFIC_KERNELS = [
    ("quantize_decode", "quant.hip", "quantize_e2m1_g128_f32_kernel<512, 1>", (0, 3)),
    ("gemv_m1", "gemm_w4a16.hip", "w4a16_small_kernel<2, true, true, 1, false, 0, 2>", (0, 3)),
    ("gemv_m4", "gemm_w4a16.hip", "w4a16_small_kernel<2, true, true, 1, false, 0, 2>", (3, 6)),
    ("gemv_m16", "gemm_w4a16.hip", "w4a16_small_kernel<2, true, true, 3, false, 0, 2>", (0, 3)),
    ("quantize_act", "quant.hip", "quantize_e2m1_tensor_bf16_kernel<true, 4>", (0, 3)),
    ("w4a4_c3", "gemm_w4a4.hip", "w4a4_fp4_kernel<128, 256, false, 0, 8>", (0, 3)),
    ("w4a4_qkv", "gemm_w4a4.hip", "w4a4_fp4_kernel<256, 256, false, 0, 8>", (0, 3)),
    ("nf4_qkv", "gemm_lut.hip", "w4a4_lut_kernel<256, 256, false>", (0, 3)),
    ("swiglu", "gemm_w4a4.hip", "w4a4_fp4_kernel<256, 256, true, 0, 8>", (0, 3)),
]
COPY_BYTES = 256 * 1024 * 1024  # the reference device copy of profile_run


def write_traffic(fetch_csv: str, write_csv: str):
    """HBM bytes per launch: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of each kernel,
    each scaled by bytes / counter of the 256 MiB reference copy in the same run."""
    import csv
    import statistics

    def read(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        return [(r["Kernel_Name"], float(r["Counter_Value"]) * 1024.0) for r in rows]

    out = {}
    data = {c: read(p, c) for c, p in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv))}
    factor = {}
    for c, rows in data.items():
        copies = [v for n, v in rows if "copyBuffer" in n]
        factor[c] = COPY_BYTES / max(copies)
    for key, src, frag, (i0, i1) in TRAFFIC_KERNELS:
        per = {}
        for c, rows in data.items():
            vals = [v for n, v in rows if frag in n][i0:i1]
            if not vals:
                break
            per[c] = statistics.median(vals) * factor[c]
        if len(per) != 2:
            continue
        h = hashlib.sha256(open(os.path.join(ROOT, "bit_floating_point_amd", "csrc", src), "rb").read()).hexdigest()
        out[key] = {"bytes_per_launch": round(per["FETCH_SIZE"] + per["WRITE_SIZE"]),
                    "fetch_bytes": round(per["FETCH_SIZE"]), "write_bytes": round(per["WRITE_SIZE"]),
                    "source_sha256": h, "kernel": frag}
    out["_scale"] = {"fetch": factor["FETCH_SIZE"], "write": factor["WRITE_SIZE"],
                     "reference": "256 MiB device-to-device copy (rocclr copyBuffer) in the same run"}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    json.dump(out, open(path, "w"), indent=1)
    print(f"wrote {path}: {', '.join(k for k in out if not k.startswith('_'))}")


# ----------------------------------------------------------------------------- decode
DEC_N, DEC_K, DEC_G = 11008, 4096, 128
DEC_MS = (1, 4, 16)


def decode_bytes():
    q = DEC_N * DEC_K * 4 + DEC_N * DEC_K // 2 + DEC_N * (DEC_K // DEC_G) * 2
    gemv = {m: DEC_N * DEC_K // 2 + DEC_N * (DEC_K // DEC_G) * 2 + m * DEC_K * 2 + m * DEC_N * 2 for m in DEC_MS}
    return q, gemv


def bench_decode(torch, F, steps, warmup):
    fe2 = F.grid_minifloat(2, 1)
    g = F.gran("group", DEC_G, "f16")
    NW, NP = 2, 16
    W = [gen_normal(torch, (DEC_N, DEC_K), 0.02, 100 + i) for i in range(NW)]
    P = [torch.empty((DEC_N, DEC_K // 2), dtype=torch.uint8, device="cuda") for _ in range(NP)]
    S = [torch.empty(DEC_N * (DEC_K // DEC_G), dtype=torch.float16, device="cuda") for _ in range(NP)]
    for i in range(NP):
        F.fp4_quantize_pack(W[i % NW], fe2, g, packed=P[i], scales=S[i])
    X = {m: gen_activations(torch, m, DEC_K, 200 + m, outlier_frac=0.0) for m in DEC_MS}
    Y = {m: torch.empty((m, DEC_N), dtype=torch.bfloat16, device="cuda") for m in DEC_MS}

    def step(i):
        F.fp4_quantize_pack(W[i % NW], fe2, g, packed=P[i % NP], scales=S[i % NP])
        j = (i + NP // 2) % NP
        for m in DEC_MS:
            F.fp4_gemm(X[m], P[j], S[j], fe2, g, y=Y[m])

    qb, gb = decode_bytes()
    step_bytes = qb + sum(gb.values())
    # `warmup` untimed steps, then exactly `steps` steps replayed as one captured graph
    # between two synchronisations; events on the stream the kernels run on
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(warmup):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            step(i)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    graph.replay()
    e1.record(st)
    torch.cuda.synchronize()
    t_step = e0.elapsed_time(e1) * 1e-3 / steps
    # graph outputs equal an eager call on the same inputs
    j = (steps - 1 + NP // 2) % NP
    for m in DEC_MS:
        ref = F.fp4_gemm(X[m], P[j], S[j], fe2, g)
        assert torch.equal(ref, Y[m]), "graph replay differs from eager run"
    # per-kernel launch durations
    t_q = graph_time(torch, lambda i: F.fp4_quantize_pack(W[i % NW], fe2, g, packed=P[i % NP], scales=S[i % NP]), 32)
    t_g = {m: graph_time(torch, lambda i, m=m: F.fp4_gemm(X[m], P[i % NP], S[i % NP], fe2, g, y=Y[m]), 64)
           for m in DEC_MS}
    kernels = [roofline_entry("quantize_pack f32->E2M1 g128 (11008x4096)", "hbm", qb / t_q / 1e9, HBM_PEAK_GBS,
                              "GB/s", t_q, qb, "bytes", traffic_for("quant.hip", "quantize_decode"))]
    for m in DEC_MS:
        flops = 2 * m * DEC_N * DEC_K
        t_c = stream_read_ceiling(torch, gb[m])
        kernels.append(roofline_entry(f"w4a16 gemv M={m} (11008x4096, g128)", "hbm", gb[m] / t_g[m] / 1e9,
                                      HBM_PEAK_GBS, "GB/s", t_g[m], gb[m], "bytes",
                                      traffic_for("gemm_w4a16.hip", f"gemv_m{m}"),
                                      tflops=round(flops / t_g[m] / 1e12, 3),
                                      read_ceiling_gbs=round(gb[m] / t_c / 1e9, 1),
                                      read_ceiling_us=round(t_c * 1e6, 3),
                                      frac_of_read_ceiling=round(t_c / t_g[m], 4)))
    del W, P, S
    torch.cuda.empty_cache()
    return t_step, step_bytes, kernels


# ----------------------------------------------------------------------------- extras
def bench_preshift_w4a4(torch, F):
    M, N, K = 2048, 4096, 4096
    fe2 = F.grid_minifloat(2, 1)
    NX = rotations(M * K * 2)
    Xs = clones(gen_activations(torch, M, K, 300), NX)
    NWc = rotations(N * K * 4)
    Ws = clones(gen_normal(torch, (N, K), 0.02, 400), NWc)
    chan = F.fp4_calibrate(Xs[0], "column", first_rows=128)
    k, a, wp, ws = F.fp4_preshift_weights(Ws[0], chan, fe2, fe2, F.gran("row"))
    ap, _ = F.fp4_quantize_pack(Xs[0], fe2, F.gran("tensor"), tensor_scale=a, col_shift=k)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    out = []
    t = graph_time(torch, lambda i: F.fp4_calibrate(Xs[i % NX], "column", first_rows=128, out=chan), 32)
    b = 128 * K * 2 + K * 4
    out.append(roofline_entry("calibrate column amax (128 of 2048 tokens x 4096, bf16)", "hbm", b / t / 1e9,
                              HBM_PEAK_GBS, "GB/s", t, b, "bytes"))
    packs = [torch.empty_like(wp) for _ in range(NWc)]
    scs = [torch.empty_like(ws) for _ in range(NWc)]
    ks = [torch.empty_like(k) for _ in range(NWc)]
    As = [torch.empty_like(a) for _ in range(NWc)]

    def pre(i):
        j = i % NWc
        F.fp4_preshift_weights(Ws[j], chan, fe2, fe2, F.gran("row"), shift=ks[j], act_scale=As[j], packed=packs[j],
                               scales=scs[j])
    t = graph_time(torch, pre, 16)
    b = N * K * 4 + N * K // 2 + N * 4 + K * 4 + K + 4
    out.append(roofline_entry("preshift + weight quantize E2M1 per-row (4096x4096 f32)", "hbm", b / t / 1e9,
                              HBM_PEAK_GBS, "GB/s", t, b, "bytes"))
    aps = [torch.empty_like(ap) for _ in range(NX)]
    t = graph_time(torch, lambda i: F.fp4_quantize_pack(Xs[i % NX], fe2, F.gran("tensor"), tensor_scale=a,
                                                        col_shift=k, packed=aps[i % NX]), 32)
    b = M * K * 2 + M * K // 2 + K
    out.append(roofline_entry("activation quantize E2M1 + pre-shift (2048x4096 bf16)", "hbm", b / t / 1e9,
                              HBM_PEAK_GBS, "GB/s", t, b, "bytes", traffic_for("quant.hip", "quantize_act")))
    t = graph_time(torch, lambda i: F.fp4_gemm(ap, wp, ws, fe2, F.gran("row"), K=K, a_grid=fe2, a_scale=a, y=y), 20)
    fl = 2 * M * N * K
    out.append(roofline_entry("w4a4 E2M1 GEMM 2048x4096x4096", "mfma", fl / t / 1e12, FP4_PEAK_TFLOPS, "TFLOP/s",
                              t, fl, "flop", traffic_for("gemm_w4a4.hip", "w4a4_c3")))
    del Xs, Ws
    torch.cuda.empty_cache()
    return out


PREFILL = {"qkv": (15360, 5120), "up": (13824, 5120), "gate": (13824, 5120), "down": (5120, 13824)}


def bench_prefill(torch, F):
    T = 4096
    fe2, fnf4 = F.grid_minifloat(2, 1), F.grid_nf4()
    X1 = gen_activations(torch, T, 5120, 500)
    X2 = gen_activations(torch, T, 13824, 501)
    c1 = F.fp4_calibrate(X1, "column", first_rows=128)
    c2 = F.fp4_calibrate(X2, "column", first_rows=128)
    out = []
    tot_fl, tot_t, tot_t_nf4 = 0, 0.0, 0.0
    qa = {}
    for name, (n, k) in PREFILL.items():
        w = gen_normal(torch, (n, k), 0.02, 600 + len(qa))
        chan = c2 if name == "down" else c1
        X = X2 if name == "down" else X1
        kk, a, wp, ws = F.fp4_preshift_weights(w, chan, fe2, fe2, F.gran("row"))
        ap, _ = F.fp4_quantize_pack(X, fe2, F.gran("tensor"), tensor_scale=a, col_shift=kk)
        y = torch.empty((T, n), dtype=torch.bfloat16, device="cuda")
        t = graph_time(torch, lambda i: F.fp4_gemm(ap, wp, ws, fe2, F.gran("row"), K=k, a_grid=fe2, a_scale=a, y=y), 5)
        fl = 2 * T * n * k
        tot_fl += fl
        tot_t += t
        out.append(roofline_entry(f"w4a4 E2M1 GEMM {name} {T}x{n}x{k}", "mfma", fl / t / 1e12, FP4_PEAK_TFLOPS,
                                  "TFLOP/s", t, fl, "flop",
                                  traffic_for("gemm_w4a4.hip", "w4a4_qkv") if name == "qkv" else None))
        kn, an, wpn, wsn = F.fp4_preshift_weights(w, chan, fe2, fnf4, F.gran("group", 64))
        apn, _ = F.fp4_quantize_pack(X, fe2, F.gran("tensor"), tensor_scale=an, col_shift=kn)
        t = graph_time(torch, lambda i: F.fp4_gemm(apn, wpn, wsn, fnf4, F.gran("group", 64), K=k, a_grid=fe2,
                                                   a_scale=an, y=y), 3)
        tot_t_nf4 += t
        out.append(roofline_entry(f"nf4 x E2M1 GEMM (f16 MFMA) {name} {T}x{n}x{k}", "mfma", fl / t / 1e12,
                                  F16_PEAK_TFLOPS, "TFLOP/s", t, fl, "flop",
                                  traffic_for("gemm_lut.hip", "nf4_qkv") if name == "qkv" else None))
        if name in ("qkv", "down"):
            xb = T * k * 2 + T * k // 2 + k
            nx = rotations(T * k * 2)
            Xr = clones(X, nx)
            apr = [torch.empty_like(ap) for _ in range(nx)]
            t = graph_time(torch, lambda i: F.fp4_quantize_pack(Xr[i % nx], fe2, F.gran("tensor"), tensor_scale=a,
                                                                col_shift=kk, packed=apr[i % nx]), 2 * nx)
            out.append(roofline_entry(f"activation quantize E2M1 + pre-shift ({T}x{k} bf16)", "hbm",
                                      xb / t / 1e9, HBM_PEAK_GBS, "GB/s", t, xb, "bytes", rotated_copies=nx))
            del Xr, apr
            wb = n * k * 4 + n * k // 2 + n * 4 + k * 5 + 4
            nw = rotations(n * k * 4)
            wr = clones(w, nw)
            wpr = [torch.empty_like(wp) for _ in range(nw)]
            wsr = [torch.empty_like(ws) for _ in range(nw)]
            t = graph_time(torch, lambda i: F.fp4_preshift_weights(wr[i % nw], chan, fe2, fe2, F.gran("row"),
                                                                   shift=kk, act_scale=a, packed=wpr[i % nw],
                                                                   scales=wsr[i % nw]), 2 * nw)
            out.append(roofline_entry(f"preshift + weight quantize E2M1 per-row ({n}x{k} f32)", "hbm",
                                      wb / t / 1e9, HBM_PEAK_GBS, "GB/s", t, wb, "bytes", rotated_copies=nw))
            del wr, wpr, wsr
        qa[name] = True
        del w, wp, wpn, y
        torch.cuda.empty_cache()
    # dynamic per-token activation quantization (E2M1, one scale per token) into the QKV
    # product with per-token scales
    n, k = PREFILL["qkv"]
    w = gen_normal(torch, (n, k), 0.02, 600)
    wp, ws = F.fp4_quantize_pack(w, fe2, F.gran("row"))
    del w
    apt, ast = F.fp4_quantize_pack(X1, fe2, F.gran("row"))
    xb = T * k * 2 + T * k // 2 + T * 4
    nx = rotations(T * k * 2)
    Xr = clones(X1, nx)
    aptr = [torch.empty_like(apt) for _ in range(nx)]
    astr = [torch.empty_like(ast) for _ in range(nx)]
    t = graph_time(torch, lambda i: F.fp4_quantize_pack(Xr[i % nx], fe2, F.gran("row"), packed=aptr[i % nx],
                                                        scales=astr[i % nx]), 2 * nx)
    out.append(roofline_entry(f"activation quantize E2M1 per-token ({T}x{k} bf16)", "hbm", xb / t / 1e9,
                              HBM_PEAK_GBS, "GB/s", t, xb, "bytes", rotated_copies=nx))
    del Xr, aptr, astr
    y = torch.empty((T, n), dtype=torch.bfloat16, device="cuda")
    t = graph_time(torch, lambda i: F.fp4_gemm(apt, wp, ws, fe2, F.gran("row"), K=k, a_grid=fe2, a_scale=ast, y=y), 5)
    fl = 2 * T * n * k
    out.append(roofline_entry(f"w4a4 E2M1 GEMM qkv {T}x{n}x{k}, per-token activation scales", "mfma",
                              fl / t / 1e12, FP4_PEAK_TFLOPS, "TFLOP/s", t, fl, "flop"))
    del wp, y
    torch.cuda.empty_cache()
    out.append(roofline_entry("prefill layer: 4 W4A4 E2M1 GEMMs (QKV, up, gate, down)", "mfma",
                              tot_fl / tot_t / 1e12, FP4_PEAK_TFLOPS, "TFLOP/s", tot_t, tot_fl, "flop"))
    out.append(roofline_entry("prefill layer: 4 NF4 GEMMs (QKV, up, gate, down)", "mfma",
                              tot_fl / tot_t_nf4 / 1e12, F16_PEAK_TFLOPS, "TFLOP/s", tot_t_nf4, tot_fl, "flop"))
    return out


def bench_swiglu(torch, F):
    """The LLaMA-13B MLP producer: gate and up W4A4 products of the same 4096 tokens with
    SwiGLU and the down projection's E2M1 quantization (its scale a' and shifts k' from
    pre-shifting the down weights) in one kernel, against the separate launches it
    replaces: the gate and up GEMMs to bf16 and the activation quantization of h (the
    SwiGLU elementwise pass between them is not counted, so the separate figure is a
    lower bound)."""
    T, (n, k) = 4096, PREFILL["up"]
    fe2 = F.grid_minifloat(2, 1)
    X1 = gen_activations(torch, T, k, 500)
    X2 = gen_activations(torch, T, n, 501)
    c1 = F.fp4_calibrate(X1, "column", first_rows=128)
    c2 = F.fp4_calibrate(X2, "column", first_rows=128)
    wd = gen_normal(torch, PREFILL["down"], 0.02, 603)
    kd, ad, _, _ = F.fp4_preshift_weights(wd, c2, fe2, fe2, F.gran("row"))
    del wd
    wg = gen_normal(torch, (n, k), 0.02, 601)
    wu = gen_normal(torch, (n, k), 0.02, 602)
    kk, a, wgp, wgs = F.fp4_preshift_weights(wg, c1, fe2, fe2, F.gran("row"))
    _, _, wup, wus = F.fp4_preshift_weights(wu, c1, fe2, fe2, F.gran("row"), shift=kk, act_scale=a)
    del wg, wu
    ap, _ = F.fp4_quantize_pack(X1, fe2, F.gran("tensor"), tensor_scale=a, col_shift=kk)
    h = torch.empty((T, n // 2), dtype=torch.uint8, device="cuda")
    t_f = graph_time(torch, lambda i: F.fp4_gemm_swiglu_quant(ap, a, wgp, wgs, wup, wus, ad, kd, K=k, h_packed=h), 5)
    yg = torch.empty((T, n), dtype=torch.bfloat16, device="cuda")
    yu = torch.empty_like(yg)
    t_g = graph_time(torch, lambda i: F.fp4_gemm(ap, wgp, wgs, fe2, F.gran("row"), K=k, a_grid=fe2, a_scale=a,
                                                 y=yg), 5)
    t_u = graph_time(torch, lambda i: F.fp4_gemm(ap, wup, wus, fe2, F.gran("row"), K=k, a_grid=fe2, a_scale=a,
                                                 y=yu), 5)
    nx = rotations(T * n * 2)
    X2r = clones(X2, nx)
    t_q = graph_time(torch, lambda i: F.fp4_quantize_pack(X2r[i % nx], fe2, F.gran("tensor"), tensor_scale=ad,
                                                          col_shift=kd, packed=h), 2 * nx)
    del X2r
    fl = 2 * T * 2 * n * k
    sep = t_g + t_u + t_q
    out = [roofline_entry(f"w4a4 gate+up GEMM with SwiGLU + E2M1 quantize epilogue {T}x(2x{n})x{k}", "mfma",
                          fl / t_f / 1e12, FP4_PEAK_TFLOPS, "TFLOP/s", t_f, fl, "flop", traffic_for("gemm_w4a4.hip", "swiglu"),
                          separate_us=round(sep * 1e6, 2), separate_gemm_us=round((t_g + t_u) * 1e6, 2),
                          separate_quantize_us=round(t_q * 1e6, 2), speedup_vs_separate=round(sep / t_f, 3))]
    del X1, X2, ap, wgp, wup, h, yg, yu
    torch.cuda.empty_cache()
    return out


def bench_two_mode(torch, F):
    """The decode workload with two-mode weights (E2M1 or E1M2 per 128-group, the mode in
    the fp16 scale's sign): the weight quantize (both candidates and the exact error
    comparison per group) and the W4A16 GEMV at M = 1, 4, 16.  Same bytes as the E2M1
    decode step."""
    tm = F.grid_two_mode()
    g = F.gran("group", DEC_G, "f16")
    NP = 16
    W = gen_normal(torch, (DEC_N, DEC_K), 0.02, 100)
    P = [torch.empty((DEC_N, DEC_K // 2), dtype=torch.uint8, device="cuda") for _ in range(NP)]
    S = [torch.empty(DEC_N * (DEC_K // DEC_G), dtype=torch.float16, device="cuda") for _ in range(NP)]
    for i in range(NP):
        F.fp4_quantize_pack(W, tm, g, packed=P[i], scales=S[i])
    qb, gb = decode_bytes()
    nw = rotations(DEC_N * DEC_K * 4)
    Wr = clones(W, nw)
    t_q = graph_time(torch, lambda i: F.fp4_quantize_pack(Wr[i % nw], tm, g, packed=P[i % NP], scales=S[i % NP]), 32)
    del Wr
    out = [roofline_entry("quantize_pack f32->two-mode E2M1/E1M2 g128 (11008x4096)", "hbm", qb / t_q / 1e9,
                          HBM_PEAK_GBS, "GB/s", t_q, qb, "bytes")]
    for m in DEC_MS:
        X = gen_activations(torch, m, DEC_K, 200 + m, outlier_frac=0.0)
        Y = torch.empty((m, DEC_N), dtype=torch.bfloat16, device="cuda")
        t = graph_time(torch, lambda i: F.fp4_gemm(X, P[i % NP], S[i % NP], tm, g, y=Y), 64)
        out.append(roofline_entry(f"w4a16 gemv two-mode M={m} (11008x4096, g128)", "hbm", gb[m] / t / 1e9,
                                  HBM_PEAK_GBS, "GB/s", t, gb[m], "bytes"))
    del W, P, S
    torch.cuda.empty_cache()
    return out


def bench_fp8(torch, F):
    """The decode workload with OCP FP8 E4M3 weights (one byte per code) and FP6 E2M3
    weights (four codes in three bytes), fp16 scales per 128: the weight quantize and the
    W8A16 / W6A16 GEMV at M = 1, 4, 16."""
    g = F.gran("group", DEC_G, "f16")
    NP = 8
    W = gen_normal(torch, (DEC_N, DEC_K), 0.02, 100)
    sb = DEC_N * (DEC_K // DEC_G) * 2
    out = []
    for (e, m), name, tag in (((4, 3), "FP8 E4M3", "w8a16"), ((2, 3), "FP6 E2M3", "w6a16")):
        fg = F.grid_minifloat(e, m)
        cb = DEC_N * DEC_K * (e + m + 1) // 8  # code bytes
        P = [torch.empty((DEC_N, DEC_K * (e + m + 1) // 8), dtype=torch.uint8, device="cuda") for _ in range(NP)]
        S = [torch.empty(DEC_N * (DEC_K // DEC_G), dtype=torch.float16, device="cuda") for _ in range(NP)]
        for i in range(NP):
            F.fp4_quantize_pack(W, fg, g, packed=P[i], scales=S[i])
        qb = DEC_N * DEC_K * 4 + cb + sb
        nw = rotations(DEC_N * DEC_K * 4)
        Wr = clones(W, nw)
        t_q = graph_time(torch, lambda i: F.fp4_quantize_pack(Wr[i % nw], fg, g, packed=P[i % NP], scales=S[i % NP]),
                         32)
        del Wr
        out.append(roofline_entry(f"quantize_pack f32->{name} g128 (11008x4096)", "hbm", qb / t_q / 1e9,
                                  HBM_PEAK_GBS, "GB/s", t_q, qb, "bytes"))
        for mm in DEC_MS:
            X = gen_activations(torch, mm, DEC_K, 200 + mm, outlier_frac=0.0)
            Y = torch.empty((mm, DEC_N), dtype=torch.bfloat16, device="cuda")
            b = cb + sb + mm * DEC_K * 2 + mm * DEC_N * 2
            t = graph_time(torch, lambda i: F.fp4_gemm(X, P[i % NP], S[i % NP], fg, g, y=Y), 64)
            out.append(roofline_entry(f"{tag} gemv {name} M={mm} (11008x4096, g128)", "hbm", b / t / 1e9,
                                      HBM_PEAK_GBS, "GB/s", t, b, "bytes"))
        del P, S
    del W
    torch.cuda.empty_cache()
    return out


def bench_w8a8(torch, F):
    """FP8 E4M3 x E4M3 (W8A8, key layers in FP8): activations per-tensor, weights per-row
    (quantized on the GPU with one scale per output row),
    on the 2048x4096x4096 shape and the LLaMA-13B QKV projection 4096x15360x5120."""
    f8 = F.grid_minifloat(4, 3)
    out = []
    for (M, N, K, name) in ((2048, 4096, 4096, "2048x4096x4096"), (4096, 15360, 5120, "qkv 4096x15360x5120")):
        X = gen_activations(torch, M, K, 500)
        W = gen_normal(torch, (N, K), 0.02, 600)
        ap, asc = F.fp4_quantize_pack(X, f8, F.gran("tensor"))
        wp, ws = F.fp4_quantize_pack(W, f8, F.gran("row"))  # one scale per output row
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        t = graph_time(torch, lambda i: F.fp4_gemm(ap, wp, ws, f8, F.gran("row"), K=K, a_grid=f8, a_scale=asc, y=y), 5)
        fl = 2 * M * N * K
        out.append(roofline_entry(f"w8a8 FP8 E4M3 GEMM {name}", "mfma", fl / t / 1e12, FP8_PEAK_TFLOPS, "TFLOP/s", t,
                                  fl, "flop"))
        del X, W, ap, wp, y
        torch.cuda.empty_cache()
    # group-scaled FP8 weights (one f16 scale per row and 128 codes of K) on the tiled kernel
    M, N, K = 4096, 15360, 5120
    X = gen_activations(torch, M, K, 500)
    W = gen_normal(torch, (N, K), 0.02, 600)
    g128 = F.gran("group", 128, "f16")
    ap, asc = F.fp4_quantize_pack(X, f8, F.gran("tensor"))
    wp, ws = F.fp4_quantize_pack(W, f8, g128)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    t = graph_time(torch, lambda i: F.fp4_gemm(ap, wp, ws, f8, g128, K=K, a_grid=f8, a_scale=asc, y=y), 5)
    fl = 2 * M * N * K
    out.append(roofline_entry("w8a8 FP8 E4M3 GEMM qkv 4096x15360x5120, group-128 weight scales", "mfma", fl / t / 1e12,
                              FP8_PEAK_TFLOPS, "TFLOP/s", t, fl, "flop"))
    del X, W, ap, wp, y
    torch.cuda.empty_cache()
    # W6A6 (FP6 E2M3 x E2M3, whose matrix-core rate is the FP4 one) and W8A8 with E5M2
    # operands, on the tiled FP8/FP6 kernel; FP6 rows padded to 16-byte multiples
    for (wf, peak, shapes) in (((2, 3), FP4_PEAK_TFLOPS, ((2048, 4096, 4096, "2048x4096x4096"),
                                                           (4096, 15360, 5120, "qkv 4096x15360x5120"))),
                               ((5, 2), FP8_PEAK_TFLOPS, ((2048, 4096, 4096, "2048x4096x4096"),))):
        g = F.grid_minifloat(*wf)
        label = "w6a6 FP6 E2M3" if wf == (2, 3) else "w8a8 FP8 E5M2"
        for (M, N, K, name) in shapes:
            X = gen_activations(torch, M, K, 500)
            W = gen_normal(torch, (N, K), 0.02, 600)
            row = K * (8 if sum(wf) == 7 else 6) // 8
            ap = torch.empty((M, row), dtype=torch.uint8, device="cuda")
            wp = torch.empty((N, row), dtype=torch.uint8, device="cuda")
            _, asc = F.fp4_quantize_pack(X, g, F.gran("tensor"), packed=ap)
            _, ws = F.fp4_quantize_pack(W, g, F.gran("row"), packed=wp)
            y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            t = graph_time(torch, lambda i: F.fp4_gemm(ap, wp, ws, g, F.gran("row"), K=K, a_grid=g, a_scale=asc, y=y),
                           5)
            fl = 2 * M * N * K
            out.append(roofline_entry(f"{label} GEMM {name}", "mfma", fl / t / 1e12, peak, "TFLOP/s", t, fl, "flop"))
            del X, W, ap, wp, y
            torch.cuda.empty_cache()
    return out


# Operations per (element, candidate) fixed by the definition of the search ("首个支持4-bit
# 浮点量化的LLM来了" page, the format/range search: quantize every weight with every
# candidate and sum the squared error): the multiply y = w * r, the clip to Qmax, the
# rounding to the nearest grid point, the dequantizing multiply g * s, the difference
# from w, its square and its addition to the sum: 7.  Each is one lane operation (binary32
# or binary64, not fused), whose peak rate is 256 CU x 4 SIMD x 16 lanes x 2.4 GHz.
SEARCH_DEF_OPS_PER_EVAL = 7
# VALU instructions the kernel issues per (element, candidate), counted from the gfx950
# assembly of search_eval_kernel: E1M2 14.8, E2M1 12.3, E3M0 17.8 per element, plus 2.4 per
# element for the per-candidate wavefront reduction, averaged over the formats (the
# exact, order-independent MSE costs a double-double TwoSum per term)
SEARCH_VALU_PER_EVAL = 17.4


def search_entry(name, t, evals):
    """The search against the ALU roofline of the operations its definition needs, with the
    kernel's VALU issue utilisation beside it."""
    return roofline_entry(name, "alu", evals * SEARCH_DEF_OPS_PER_EVAL / t / 1e12, VALU_PEAK_TOPS, "TOP/s", t,
                          evals, "element-candidate evaluations", evals_per_s=evals / t,
                          ops_per_eval_definition=SEARCH_DEF_OPS_PER_EVAL,
                          valu_instructions_per_eval=SEARCH_VALU_PER_EVAL,
                          valu_issue_frac=round(evals * SEARCH_VALU_PER_EVAL / t / 1e12 / VALU_PEAK_TOPS, 4))


def bench_search(torch, F):
    T, numel = 32, 4096 * 4096
    w = torch.empty((T, numel), dtype=torch.float32, device="cuda")
    for t in range(T):
        w[t] = gen_heavy_tail(torch, (numel,), 700 + t)
    res, packed = F.fp4_search_format(w)
    torch.cuda.synchronize()
    reps = 2
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        F.fp4_search_format(w)
    e1.record()
    e1.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / reps
    evals = T * numel * 3 * 100
    del w, packed
    torch.cuda.empty_cache()
    out = [search_entry("format/clip search 32 x 4096x4096 (3 formats x 100 clips)", t, evals)]
    # the same search on activations: per token over the LLaMA-13B prefill input (4096 x
    # 5120 bf16), and once over its 128 calibration tokens with every token packed
    X = gen_activations(torch, 4096, 5120, 500)
    ws = torch.empty(F._lib.lib().fp4_search_workspace_size(4096, 5120, 3, 100), dtype=torch.uint8, device="cuda")
    packed = torch.empty((4096, 2560), dtype=torch.uint8, device="cuda")
    for unit, first, name in (("row", 0, "per-token"), ("tensor", 128, "128 calibration tokens")):
        fn = (lambda i, unit=unit, first=first:
              F.fp4_search_activations(X, unit, first_rows=first, workspace=ws, packed=packed))
        t = graph_time(torch, fn, 3)
        evals = (4096 if unit == "row" else 128) * 5120 * 3 * 100
        out.append(search_entry(f"activation format/clip search, {name}, 4096x5120 bf16 (3 formats x 100 clips)",
                                t, evals))
    del X, ws, packed
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------- CPU oracle
def cpu_baseline(target_s=12.0):
    """The CPU oracle (as it is) on a bounded sample of the decode step: the first R
    weight rows quantized (E2M1, fp16 group scales) and the three GEMVs on them."""
    import numpy as np
    import oracle as O
    import synth
    O.build()
    e2 = O.minifloat(2, 1)

    def run(rows):
        w = synth.weight(2, 0, rows, DEC_K)
        xs = {m: synth.activations(2, m, m, DEC_K) for m in DEC_MS}
        t0 = time.perf_counter()
        p, s = O.quantize_pack(w, e2, "group", DEC_G, "f16")
        for m in DEC_MS:
            O.gemm_w4a16(xs[m], p, e2, "group", s, group=DEC_G)
        dt = time.perf_counter() - t0
        b = rows * DEC_K * 4 + rows * DEC_K // 2 + rows * (DEC_K // DEC_G) * 2
        b += sum(rows * DEC_K // 2 + rows * (DEC_K // DEC_G) * 2 + m * DEC_K * 2 + m * rows * 2 for m in DEC_MS)
        return dt, b

    dt, _ = run(128)
    rows = int(min(DEC_N, max(128, 128 * target_s / max(dt, 1e-3))))
    # the whole step when it fits; repeated until about target_s seconds of CPU work
    total_t, total_b, reps = 0.0, 0, 0
    while total_t < target_s and reps < 64:
        dt, b = run(rows)
        total_t += dt
        total_b += b
        reps += 1
    cores = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
    return {"value": round(total_b / total_t / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"decode step on the first {rows} of 11008 weight rows (quantize E2M1 g128 + GEMV "
                      f"M=1,4,16), {reps} repetition(s), {total_t:.1f} s"}


# ----------------------------------------------------------------------------- main
def main():
    args = parse()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path is per-GPU and shards "
              "without collectives", file=sys.stderr)
        sys.exit(2)
    import torch
    import bit_floating_point_amd as F
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.init()
    if args.profile:
        profile_run(torch, F, args.profile)
        return
    log("decode workload ...")
    t_step, step_bytes, kernels = bench_decode(torch, F, args.steps, args.warmup)
    if not args.main_only:
        log("pre-shift + W4A4 2048x4096x4096 ...")
        kernels += bench_preshift_w4a4(torch, F)
        log("LLaMA-13B prefill layer ...")
        kernels += bench_prefill(torch, F)
        log("FP8 / FP6 grids ...")
        kernels += bench_fp8(torch, F)
        kernels += bench_w8a8(torch, F)
        log("two-mode grid ...")
        kernels += bench_two_mode(torch, F)
        log("fused SwiGLU + quantize ...")
        kernels += bench_swiglu(torch, F)
        log("format search ...")
        kernels += bench_search(torch, F)
    dominant = max(kernels[:4], key=lambda d: d["us_per_launch"])
    cpu = None if args.no_cpu_baseline else cpu_baseline()
    line = {
        "metric": METRIC,
        "value": round(step_bytes / t_step / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4-e2m1 weights x bf16 activations, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": "LLaMA-7B MLP linear 11008x4096: E2M1 g128 fp16-scale weight quantize + "
                               "W4A16 decode GEMV at M=1,4,16 (bf16)",
                   "N": DEC_N, "K": DEC_K, "group": DEC_G, "M": list(DEC_MS), "step_bytes": step_bytes},
        "roofline": {k: dominant[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")},
        "cpu_baseline": cpu,
        "kernels": kernels,
    }
    line["roofline"]["kernel"] = dominant["kernel"]
    for k in kernels:  # the metric's W4A4 half, on the LLaMA-13B prefill layer and the 2048-token GEMM
        if k["kernel"].startswith("prefill layer: 4 W4A4"):
            line["w4a4_prefill"] = {"workload": "LLaMA-13B prefill layer, 4096 tokens: QKV 15360x5120, up and gate "
                                                "13824x5120, down 5120x13824, W4A4 E2M1 pre-shifted, bf16 out",
                                    "value": k["achieved"], "unit": "TFLOP/s", "peak": k["peak"], "frac": k["frac"],
                                    "us": k["us_per_launch"]}
        if k["kernel"] == "w4a4 E2M1 GEMM 2048x4096x4096":
            line["w4a4_2048x4096x4096"] = {"value": k["achieved"], "unit": "TFLOP/s", "peak": k["peak"],
                                           "frac": k["frac"], "us": k["us_per_launch"]}
    print(json.dumps(line), flush=True)


def profile_run(torch, F, what):
    """A few eager launches of the chosen kernels plus a plain 256 MiB device copy (the
    reference for scaling HBM byte counters)."""
    fe2 = F.grid_minifloat(2, 1)
    src = torch.empty(64 * 1024 * 1024, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    if what in ("quantize", "decode", "all"):
        W = gen_normal(torch, (DEC_N, DEC_K), 0.02, 100)
        g = F.gran("group", DEC_G, "f16")
        for _ in range(3):
            p, s = F.fp4_quantize_pack(W, fe2, g)
        if what in ("decode", "all"):
            for m in DEC_MS:
                x = gen_activations(torch, m, DEC_K, 200 + m, outlier_frac=0.0)
                for _ in range(3):
                    F.fp4_gemm(x, p, s, fe2, g)
    if what == "all":
        M, N, K = 2048, 4096, 4096
        X = gen_activations(torch, M, K, 300)
        Wt = gen_normal(torch, (N, K), 0.02, 400)
        chan = F.fp4_calibrate(X, "column", first_rows=128)
        k, a, wp, ws = F.fp4_preshift_weights(Wt, chan, fe2, fe2, F.gran("row"))
        for _ in range(3):
            ap, _ = F.fp4_quantize_pack(X, fe2, F.gran("tensor"), tensor_scale=a, col_shift=k)
        for _ in range(3):
            F.fp4_gemm(ap, wp, ws, fe2, F.gran("row"), K=K, a_grid=fe2, a_scale=a)
        # the prefill QKV projection, W4A4 E2M1 and NF4 x E2M1
        T, (n, k) = 4096, PREFILL["qkv"]
        X = gen_activations(torch, T, k, 500)
        chan = F.fp4_calibrate(X, "column", first_rows=128)
        w = gen_normal(torch, (n, k), 0.02, 600)
        y = torch.empty((T, n), dtype=torch.bfloat16, device="cuda")
        kk, a, wp, ws = F.fp4_preshift_weights(w, chan, fe2, fe2, F.gran("row"))
        ap, _ = F.fp4_quantize_pack(X, fe2, F.gran("tensor"), tensor_scale=a, col_shift=kk)
        for _ in range(3):
            F.fp4_gemm(ap, wp, ws, fe2, F.gran("row"), K=k, a_grid=fe2, a_scale=a, y=y)
        fnf4 = F.grid_nf4()
        kn, an, wpn, wsn = F.fp4_preshift_weights(w, chan, fe2, fnf4, F.gran("group", 64))
        apn, _ = F.fp4_quantize_pack(X, fe2, F.gran("tensor"), tensor_scale=an, col_shift=kn)
        for _ in range(3):
            F.fp4_gemm(apn, wpn, wsn, fnf4, F.gran("group", 64), K=k, a_grid=fe2, a_scale=an, y=y)
        # the MLP gate/up pair with SwiGLU and the down projection's quantization fused
        n, k = PREFILL["up"]
        X = gen_activations(torch, T, k, 500)
        chan = F.fp4_calibrate(X, "column", first_rows=128)
        wg = gen_normal(torch, (n, k), 0.02, 601)
        kk, a, wgp, wgs = F.fp4_preshift_weights(wg, chan, fe2, fe2, F.gran("row"))
        ap, _ = F.fp4_quantize_pack(X, fe2, F.gran("tensor"), tensor_scale=a, col_shift=kk)
        h = torch.empty((T, n // 2), dtype=torch.uint8, device="cuda")
        kd = torch.zeros(n, dtype=torch.int8, device="cuda")
        for _ in range(3):
            F.fp4_gemm_swiglu_quant(ap, a, wgp, wgs, wgp, wgs, a, kd, K=k, h_packed=h)
    torch.cuda.synchronize()
    log("profile run done")


if __name__ == "__main__":
    main()

"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module holds no quantization arithmetic: it only draws random tensors with the
shapes and value distributions of the workloads below and rounds activations to
bfloat16 storage.  Every draw uses ``numpy.random.default_rng([config, tensor,
stream])``; streams: 0 = weights, 1 = activations, 2 = outlier-channel choice,
3 = heavy-tail mixture selector, 4 = heavy-tail values.  "N(0, 0.02)" means a normal
distribution with standard deviation 0.02.

Workloads (LLaMA-shaped stand-ins; no model weights or datasets are used):

1. tiny round trip: W 256x256 N(0,0.02), X 8x256 fp32 N(0,1)
2. W4A16 decode on a LLaMA-7B MLP linear: W 11008x4096 N(0,0.02); X M x 4096 bf16 N(0,1)
   for M in {1, 4, 16}
3. calibration + pre-shift + W4A4: X 2048x4096 bf16 N(0,1) with 1% of the channels
   (41) scaled x50; W 4096x4096 N(0,0.02)
4. format/clip search: 32 tensors 4096x4096, per element 0.02 * N(0,1), or with
   probability 0.05 0.02 * Student-t(4)
5. LLaMA-13B prefill layer: X1 4096x5120 and X2 4096x13824 bf16 N(0,1) with 1%
   outlier channels x50; W_qkv 15360x5120, W_up/W_gate 13824x5120, W_down 5120x13824
   N(0,0.02)
"""
from __future__ import annotations

import numpy as np

TINY, DECODE, PRESHIFT, SEARCH, PREFILL = 1, 2, 3, 4, 5


def rng(config: int, tensor: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([config, tensor, stream])


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Round float32 data to bfloat16 storage (nearest-even) and return it widened
    back to float32 (exactly), so host code can keep float32 arrays."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def weight(config: int, tensor: int, rows: int, cols: int, std: float = 0.02) -> np.ndarray:
    return (rng(config, tensor, 0).standard_normal((rows, cols), dtype=np.float32)
            * np.float32(std)).astype(np.float32)


def heavy_tail_weight(config: int, tensor: int, rows: int, cols: int, std: float = 0.02,
                      p_tail: float = 0.05, dof: float = 4.0) -> np.ndarray:
    z = rng(config, tensor, 0).standard_normal((rows, cols), dtype=np.float32)
    sel = rng(config, tensor, 3).random((rows, cols), dtype=np.float32) < p_tail
    t = rng(config, tensor, 4).standard_t(dof, size=(rows, cols)).astype(np.float32)
    return (np.where(sel, t, z) * np.float32(std)).astype(np.float32)


def outlier_channels(config: int, tensor: int, cols: int, frac: float = 0.01) -> np.ndarray:
    n = int(round(frac * cols))
    return np.sort(rng(config, tensor, 2).choice(cols, size=n, replace=False))


def activations(config: int, tensor: int, rows: int, cols: int, outlier_frac: float = 0.0,
                outlier_gain: float = 50.0, bf16: bool = True) -> np.ndarray:
    x = rng(config, tensor, 1).standard_normal((rows, cols), dtype=np.float32)
    if outlier_frac > 0:
        x[:, outlier_channels(config, tensor, cols, outlier_frac)] *= np.float32(outlier_gain)
    return to_bf16_values(x) if bf16 else x


# ---- the five workloads at their full sizes (and scaled-down parity variants) ----
def tiny():
    return weight(TINY, 0, 256, 256), activations(TINY, 0, 8, 256, bf16=False)


def decode_weight(n: int = 11008, k: int = 4096) -> np.ndarray:
    return weight(DECODE, 0, n, k)


def decode_activations(m: int, k: int = 4096) -> np.ndarray:
    return activations(DECODE, m, m, k)


def preshift_inputs(m: int = 2048, n: int = 4096, k: int = 4096):
    return activations(PRESHIFT, 0, m, k, outlier_frac=0.01), weight(PRESHIFT, 0, n, k)


def search_tensor(t: int, rows: int = 4096, cols: int = 4096) -> np.ndarray:
    return heavy_tail_weight(SEARCH, t, rows, cols)


PREFILL_SHAPES = {"qkv": (15360, 5120), "up": (13824, 5120), "gate": (13824, 5120),
                  "down": (5120, 13824)}
PREFILL_TENSOR_ID = {"qkv": 0, "up": 1, "gate": 2, "down": 3}


def prefill_weight(name: str, scale_down: int = 1) -> np.ndarray:
    n, k = PREFILL_SHAPES[name]
    return weight(PREFILL, PREFILL_TENSOR_ID[name], n // scale_down, k // scale_down)


def prefill_activations(which: int, tokens: int = 4096, scale_down: int = 1) -> np.ndarray:
    k = (5120 if which == 1 else 13824) // scale_down
    return activations(PREFILL, which, tokens, k, outlier_frac=0.01)

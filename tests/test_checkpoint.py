"""The .npz checkpoint of a quantized tensor: a round trip keeps every array and
structure bit for bit, and loading refuses archives that would need unpickling."""
import ctypes

import numpy as np
import pytest
import torch

import bit_floating_point_amd as F
from bit_floating_point_amd import _lib as L
from bit_floating_point_amd.checkpoint import load_quantized, save_quantized


def _records(n):
    out = bytearray()
    for i in range(n):
        r = L.fp4_search_result()
        r.e, r.m, r.clip_index, r.format_index = 2, 1, 40 + i, 1
        r.clip, r.scale, r.amax, r.bias, r.mse, r.mse_runner_up = 0.8, 0.125, 6.0 + i, 1.0, 1e-3 * (i + 1), 2e-3
        out += bytes(r)
    return torch.frombuffer(out, dtype=torch.uint8).clone()


def test_round_trip_keeps_everything(tmp_path):
    g = torch.Generator().manual_seed(3)
    packed = torch.randint(0, 256, (48, 64), dtype=torch.uint8, generator=g)
    scales = torch.rand(48 * 1, generator=g).to(torch.float16)
    shift = torch.randint(-3, 2, (128,), dtype=torch.int8, generator=g)
    act = torch.tensor([0.0625], dtype=torch.float32)
    recs = _records(3)
    path = tmp_path / "w.npz"
    save_quantized(path, packed, scales, F.grid_minifloat(2, 1), F.gran("row", 0, "f16"), shift=shift, act_scale=act,
                   records=recs)
    back = load_quantized(path)
    assert torch.equal(back["packed"], packed)
    assert torch.equal(back["scales"].view(torch.int16), scales.view(torch.int16))
    assert torch.equal(back["shift"], shift) and torch.equal(back["act_scale"], act)
    assert bytes(back["grid"]) == bytes(F.grid_minifloat(2, 1))
    assert bytes(back["gran"]) == bytes(F.gran("row", 0, "f16"))
    assert [bytes(r) for r in back["records"]] == [bytes(recs[i * ctypes.sizeof(L.fp4_search_result):
                                                               (i + 1) * ctypes.sizeof(L.fp4_search_result)].numpy())
                                                   for i in range(3)]
    assert back["records"][2].amax == 8.0 and back["records"][0].clip_index == 40


def test_lookup_grid_round_trip(tmp_path):
    vals = [(i - 7.5) / 8 for i in range(16)]
    path = tmp_path / "lut.npz"
    save_quantized(path, torch.zeros((2, 8), dtype=torch.uint8), torch.ones(4, dtype=torch.float32), F.grid_lut(vals),
                   F.gran("group", 64))
    back = load_quantized(path)
    assert list(back["grid"].lut) == pytest.approx(vals, abs=0) and "shift" not in back and "records" not in back


def test_load_refuses_object_arrays(tmp_path):
    path = tmp_path / "bad.npz"
    np.savez(path, format_version=np.array([1], np.int32), codes=np.array([object()], dtype=object),
             scales=np.ones(1, np.float32), grid=np.array([0, 2, 1, 0], np.int32), grid_lut=np.zeros(16, np.float32),
             gran=np.zeros(4, np.int32))
    with pytest.raises(ValueError):
        load_quantized(path)


def test_save_rejects_wrong_types(tmp_path):
    with pytest.raises(ValueError):
        save_quantized(tmp_path / "x.npz", torch.zeros(4, dtype=torch.uint8), torch.ones(1), F.grid_minifloat(2, 1),
                       F.gran())
    with pytest.raises(ValueError):
        save_quantized(tmp_path / "x.npz", torch.zeros((1, 4), dtype=torch.uint8), torch.ones(1, dtype=torch.int32),
                       F.grid_minifloat(2, 1), F.gran())

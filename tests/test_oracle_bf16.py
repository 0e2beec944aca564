"""Pins for the oracle's bf16 helpers (CPU): IEEE-fixed values and torch's cast."""

import json
import os

import numpy as np
import torch

from oracle import bf16_to_f32, f32_to_bf16_rne, bf16_ulp_distance


def _u32(h):
    return np.array([int(h, 16)], dtype=np.uint32)


def test_golden_values(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "bf16_values.json")))
    for c in g["cases"]:
        f = _u32(c["f32"]).view(np.float32)
        got = int(f32_to_bf16_rne(f)[0])
        assert got == int(c["bf16"], 16), c["why"]


def test_widen_is_exact():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = bf16_to_f32(bits)
    assert np.array_equal(f.view(np.uint32) >> 16, bits.astype(np.uint32))
    assert np.all(f.view(np.uint32) & 0xFFFF == 0)
    # Round-tripping every bf16 pattern is the identity (NaNs stay NaN).
    back = f32_to_bf16_rne(f)
    nan = np.isnan(f)
    assert np.array_equal(back[~nan], bits[~nan])
    assert np.all(np.isnan(bf16_to_f32(back[nan])))


def test_matches_torch_cast():
    # torch's CPU float32 -> bfloat16 cast rounds to nearest even.
    rng = np.random.default_rng(1)
    f = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 200000),
        rng.integers(0, 1 << 32, 200000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ]).astype(np.float32)
    finite = np.isfinite(f)
    ref = torch.from_numpy(f[finite]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_rne(f[finite]), ref)


def test_nan_is_quiet():
    f = _u32("0x7f800001").view(np.float32)   # signalling NaN
    out = f32_to_bf16_rne(f)
    assert np.isnan(bf16_to_f32(out))[0] and int(out[0]) & 0x0040
    neg = _u32("0xffc00000").view(np.float32)
    assert int(f32_to_bf16_rne(neg)[0]) == 0xFFC0


def test_ulp_distance():
    a = np.array([0x3F80, 0x3F80, 0x0000, 0x8000, 0x0001, 0x7F7F], dtype=np.uint16)
    b = np.array([0x3F81, 0x3F80, 0x8000, 0x0001, 0x8001, 0x7F80], dtype=np.uint16)
    assert bf16_ulp_distance(a, b).tolist() == [1, 0, 0, 1, 2, 1]

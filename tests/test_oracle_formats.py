"""Pins of the oracle's number formats against library routines and hand-worked
values (no GPU)."""

import json
import os

import numpy as np
import torch

from oracle import formats

HERE = os.path.dirname(os.path.abspath(__file__))


def test_e4m3fn_all_codes_match_torch_cast():
    codes = np.arange(256, dtype=np.uint8)
    ours = formats.e4m3fn_to_f32(codes)
    lib = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    nan_ours = np.isnan(ours)
    assert np.array_equal(nan_ours, np.isnan(lib))
    assert nan_ours.sum() == 2
    assert np.array_equal(ours[~nan_ours].view(np.uint32), lib[~nan_ours].view(np.uint32))


def test_e4m3fn_hand_worked_codes():
    with open(os.path.join(HERE, "golden", "fp8_e4m3fn_codes.json")) as f:
        g = json.load(f)
    for code, val in g["codes"].items():
        assert formats.e4m3fn_to_f32(np.array([int(code, 16)], np.uint8))[0] == np.float32(val), code
    nz = formats.e4m3fn_to_f32(np.array([int(g["negative_zero"], 16)], np.uint8))[0]
    assert nz == 0.0 and np.signbit(nz)
    for c in g["nan"]:
        assert np.isnan(formats.e4m3fn_to_f32(np.array([int(c, 16)], np.uint8))[0])
    finite = formats.e4m3fn_to_f32(np.arange(256, dtype=np.uint8))
    finite = finite[~np.isnan(finite)]
    assert finite.size == 254 and np.abs(finite).max() == 448.0


def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    # constructed ties: exactly half an ulp above even and odd bf16 values
    base = rng.integers(0, 0xFFFF, 5000).astype(np.uint32) << 16
    base &= ~np.uint32(0x7F800000) | np.uint32(0x3F800000)      # keep finite
    ties = (base | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.array([0.0, -0.0, 1.0, 3.0e38], np.float32)])
    ours = formats.f32_to_bf16_bits(x)
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, lib)


def test_bf16_hand_worked_ties():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to the even value 1.0
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 (odd) and 1 + 2^-6: goes up.
    vals = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8)], np.float32)
    out = formats.bf16_bits_to_f32(formats.f32_to_bf16_bits(vals))
    assert out.tolist() == [1.0, 1 + 2.0 ** -6, -1.0]


def test_bf16_widen_is_exact_inverse_on_bf16_values():
    bits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    f = formats.bf16_bits_to_f32(bits)
    keep = ~np.isnan(f)
    assert np.array_equal(formats.f32_to_bf16_bits(f[keep]), bits[keep])

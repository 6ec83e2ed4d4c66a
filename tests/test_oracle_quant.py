"""Pins of the oracle's quantisers (no GPU).

What pins them, besides themselves:
  * hand-worked tie cases (golden/quant_ties.json) fix the rounding mode and
    the scale definition;
  * exact rational arithmetic (fractions) fixes the correctly rounded fp32
    divisions of the scale and of the quotient;
  * the quantise/dequantise round-trip bound |x - q s| <= s/2 (1 + 2^-16);
  * identities between the schemes (token == group when K == 128; the
    channel-wise weight quantiser is the token quantiser on W);
  * the FP8 -> BF16 -> INT8 conversion is exactly equivariant to power-of-two
    scale_inv, and with scale_inv = 1 its bf16 step is exact.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import formats, quant

HERE = os.path.dirname(os.path.abspath(__file__))


def _round_to_f32(fr):
    """Round a Fraction to the nearest float32, ties to even (exact search)."""
    f = np.float32(float(fr))            # within an ulp or so of the answer
    cands = [f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - fr),
                                     int(np.array(c, np.float32).view(np.uint32)) & 1))
    return np.float32(best)


def _bf16_tensor_bits(x):
    return synth.to_numpy(x)


def test_golden_ties():
    with open(os.path.join(HERE, "golden", "quant_ties.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        vals = np.zeros(case["pad_to"], np.float32)
        vals[: len(case["values"])] = case["values"]
        bits = formats.f32_to_bf16_bits(vals)
        assert np.array_equal(formats.bf16_bits_to_f32(bits), vals)     # exact in bf16
        for fn in (quant.quant_act_group, quant.quant_act_token):
            q, s = fn(bits[None, :])
            assert np.float32(s.reshape(-1)[0]) == np.float32(case["scale"]), case["name"]
            assert q[0, : len(case["q"])].tolist() == case["q"], case["name"]
            assert np.all(q[0, len(case["q"]):] == 0)


def test_scale_and_quotient_are_correctly_rounded_fp32_divisions():
    rng = np.random.default_rng(1)
    x = synth.to_numpy(synth.activations(4, 1024, seed=7, outlier_frac=0.01, outlier_factor=20.0))
    q, s = quant.quant_act_group(x)
    x32 = formats.bf16_bits_to_f32(x)
    g = x32.reshape(4, 8, 128)
    for (m, kb) in [(0, 0), (1, 3), (2, 7), (3, 5)]:
        amax = Fraction(float(np.abs(g[m, kb]).max()))
        s_exact = _round_to_f32(amax / 127)
        assert s[m, kb] == s_exact
        for j in rng.integers(0, 128, 24):
            quo = _round_to_f32(Fraction(float(g[m, kb, j])) / Fraction(float(s_exact)))
            want = int(np.rint(np.float64(quo)))
            assert q[m, kb * 128 + j] == max(-127, min(127, want))


def test_round_trip_bound_and_amax_maps_to_127():
    x = synth.to_numpy(synth.activations(64, 2048, seed=3))
    x32 = formats.bf16_bits_to_f32(x).astype(np.float64)
    for fn, shape in ((quant.quant_act_group, (64, 16)), (quant.quant_act_token, (64,))):
        q, s = fn(x)
        assert s.shape == shape and q.dtype == np.int8
        assert q.min() >= -127 and q.max() <= 127
        se = np.repeat(s, 128, axis=1) if s.ndim == 2 else s[:, None]
        err = np.abs(x32 - q.astype(np.float64) * se.astype(np.float64))
        assert np.all(err <= se * 0.5 * (1 + 2.0 ** -16))
        # the element of largest magnitude of each group lands on +-127
        if s.ndim == 2:
            g = x32.reshape(64, 16, 128)
            idx = np.abs(g).argmax(axis=2)
            qq = q.reshape(64, 16, 128)
            picked = np.take_along_axis(qq, idx[:, :, None], axis=2)[..., 0]
        else:
            idx = np.abs(x32).argmax(axis=1)
            picked = q[np.arange(64), idx]
        assert np.all(np.abs(picked.astype(int)) == 127)


def test_zero_group_gives_zero_codes_and_eps_scale():
    x = np.zeros((2, 256), np.uint16)
    x[1, 128:] = formats.f32_to_bf16_bits(np.full(128, 0.5, np.float32))
    q, s = quant.quant_act_group(x)
    eps_scale = _round_to_f32(Fraction(float(np.float32(1e-10))) / 127)
    assert s[0, 0] == eps_scale and s[0, 1] == eps_scale and s[1, 0] == eps_scale
    assert np.all(q[0] == 0) and np.all(q[1, :128] == 0) and np.all(q[1, 128:] == 127)


def test_group_equals_token_when_k_is_one_block():
    x = synth.to_numpy(synth.activations(32, 128, seed=5))
    qg, sg = quant.quant_act_group(x)
    qt, st = quant.quant_act_token(x)
    assert np.array_equal(qg, qt) and np.array_equal(sg[:, 0], st)


def test_tile_quantiser_against_groupwise_definition():
    """A 128x128 tile is one quantisation group: quantising the flattened tile
    as one token row must give the same codes and scale."""
    w = synth.to_numpy(synth.weights(200, 384, seed=9))            # ragged last tile (72 rows)
    q, s = quant.quant_weight_block(w)
    assert s.shape == (2, 3)
    for nb in range(2):
        r0, r1 = nb * 128, min(200, nb * 128 + 128)
        for kb in range(3):
            tile = w[r0:r1, kb * 128:(kb + 1) * 128]
            qt, st = quant.quant_act_token(tile.reshape(1, -1))
            assert st[0] == s[nb, kb]
            assert np.array_equal(qt.reshape(tile.shape), q[r0:r1, kb * 128:(kb + 1) * 128])


def test_requant_power_of_two_equivariance():
    codes, _ = synth.fp8_weights(192, 256, seed=11)
    codes = codes.numpy()
    base = np.full((2, 2), 1.0, np.float32)
    q0, s0, w0 = quant.requant_fp8_to_int8_block(codes, base)
    # scale_inv = 1: every E4M3 value is exact in bf16, so the bf16 step is exact
    assert np.array_equal(formats.bf16_bits_to_f32(w0), formats.e4m3fn_to_f32(codes))
    for e in (-20, -7, 3, 9):
        q1, s1, _ = quant.requant_fp8_to_int8_block(codes, base * np.float32(2.0 ** e))
        assert np.array_equal(q1, q0)
        assert np.array_equal(s1, (s0 * np.float32(2.0 ** e)).astype(np.float32))


def test_requant_uses_each_tiles_scale_inv():
    """A tile-wise scale_inv that differs per tile must act only on its tile:
    with per-tile powers of two, each tile's codes match the unit-scale codes
    and its scale is multiplied by that tile's power of two."""
    codes, _ = synth.fp8_weights(256, 384, seed=12)
    codes = codes.numpy()
    exps = np.array([[-3, 0, 5], [7, -9, 2]])
    si = (2.0 ** exps).astype(np.float32)
    q0, s0, _ = quant.requant_fp8_to_int8_block(codes, np.ones((2, 3), np.float32))
    q1, s1, _ = quant.requant_fp8_to_int8_block(codes, si)
    assert np.array_equal(q0, q1)
    assert np.array_equal(s1, (s0 * si).astype(np.float32))


def test_requant_matches_library_cast_route():
    """FP8 -> BF16 via torch's own casts (fp8 -> fp32, multiply, -> bf16) then
    tile quantisation gives the same result as the oracle's requant."""
    codes, si = synth.fp8_weights(200, 256, seed=13)
    f = codes.view(torch.float8_e4m3fn).to(torch.float32)
    rows = torch.arange(200) // 128
    cols = torch.arange(256) // 128
    wb = (f * si[rows][:, cols]).to(torch.bfloat16)
    q_ref, s_ref = quant.quant_weight_block(synth.to_numpy(wb))
    q, s, wbits = quant.requant_fp8_to_int8_block(codes.numpy(), si.numpy())
    assert np.array_equal(wbits, synth.to_numpy(wb))
    assert np.array_equal(q, q_ref) and np.array_equal(s, s_ref)


def test_channel_wise_is_more_exposed_to_outliers():
    """Page 1 section 2.3: per-channel/per-token groups meet outliers more often
    than small groups, so their quantisation error is larger.  Statistical
    property on the outlier-laden activations (not a parity check)."""
    x = synth.to_numpy(synth.activations(64, 7168, seed=1))
    x32 = formats.bf16_bits_to_f32(x).astype(np.float64)
    qg, sg = quant.quant_act_group(x)
    qt, st = quant.quant_act_token(x)
    eg = np.abs(x32 - qg * np.repeat(sg, 128, axis=1)).mean()
    et = np.abs(x32 - qt * st[:, None]).mean()
    assert et > 2 * eg


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_fp16_and_bf16_inputs_give_the_same_codes_for_common_values(dtype):
    # values exactly representable in both formats quantise identically
    rng = np.random.default_rng(2)
    v = (rng.integers(-255, 256, (4, 256)) / 64.0).astype(np.float32)
    x = v.astype(np.float16) if dtype == "fp16" else formats.f32_to_bf16_bits(v)
    q, s = quant.quant_act_group(x)
    q2, s2 = quant.quant_act_group(v)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_requant_channel_hand_worked():
    """FP8 -> BF16 -> per-output-channel INT8 (page 1 section 2.3, channel-wise
    paragraph), worked by hand on two 128-row tile rows and two K blocks with a
    different scale_inv per tile, so that each row's amax spans both K blocks:

      rows 0..127:  codes 0x30 (0.5) x 5    = 2.5   in K block 0,
                    codes 0x38 (1.0) x 127  = 127   in K block 1
                    -> amax 127, s = 1 exactly, q = rne(2.5) = 2 and 127;
      rows 128,129: codes 0x38 (1.0) x 15.875 = 15.875 in K block 0,
                    codes 0x34 (0.75) x 0.25 = 0.1875 and 0xB4 -> -0.1875
                    in K block 1
                    -> amax 15.875, s = 0.125 exactly, q = 127 and
                    rne(+-1.5) = +-2.

    Every product above is exact in fp32 and bf16.  Indexing scale_inv by the K
    block alone, taking a 128 x 128 tile's amax instead of the row's, or
    rounding half away from zero each changes some code or scale."""
    N, K = 130, 256
    codes = np.zeros((N, K), np.uint8)
    codes[:128, :128] = 0x30
    codes[:128, 128:] = 0x38
    codes[128:, :128] = 0x38
    codes[128:, 128:] = 0x34
    codes[129, 128:] = 0xB4
    si = np.array([[5.0, 127.0], [15.875, 0.25]], np.float32)
    q, s, wb = quant.requant_fp8_to_int8_channel(codes, si)
    assert s.shape == (N,)
    assert np.all(s[:128] == np.float32(1.0)) and np.all(s[128:] == np.float32(0.125))
    assert np.all(q[:128, :128] == 2) and np.all(q[:128, 128:] == 127)
    assert np.all(q[128:, :128] == 127)
    assert np.all(q[128, 128:] == 2) and np.all(q[129, 128:] == -2)
    w = formats.bf16_bits_to_f32(wb)
    assert np.all(w[:128, :128] == 2.5) and np.all(w[129, 128:] == np.float32(-0.1875))


def test_requant_channel_matches_library_cast_route_and_rational_scales():
    """torch's own casts give the bf16 weights (fp8 -> fp32, times the tile's
    scale_inv, -> bf16); each row's scale is the correctly rounded
    fp32(amax / 127) of the row's largest magnitude (checked with fractions),
    and sampled codes are rne of the correctly rounded quotient."""
    N, K = 200, 384
    codes, si = synth.fp8_weights(N, K, seed=14)
    f = codes.view(torch.float8_e4m3fn).to(torch.float32)
    rows = torch.arange(N) // 128
    cols = torch.arange(K) // 128
    wb = (f * si[rows][:, cols]).to(torch.bfloat16)
    q, s, wbits = quant.requant_fp8_to_int8_channel(codes.numpy(), si.numpy())
    assert np.array_equal(wbits, synth.to_numpy(wb))
    w = wb.to(torch.float32).numpy()
    rng = np.random.default_rng(3)
    for n in list(rng.choice(N, 12, replace=False)) + [0, 127, 128, N - 1]:
        amax = Fraction(float(np.abs(w[n]).max()))
        assert s[n] == _round_to_f32(amax / 127), n
        for k in rng.choice(K, 16, replace=False):
            quo = _round_to_f32(Fraction(float(w[n, k])) / Fraction(float(s[n])))
            assert q[n, k] == int(np.rint(quo)), (n, k)


def test_requant_channel_power_of_two_equivariance_per_tile_row():
    """scale_inv = 2^e[nb] constant along a tile row: every row n keeps its
    codes and its scale is multiplied by 2^e[n // 128] exactly (a scale_inv
    looked up by the K block, or by the wrong tile row, breaks it)."""
    N, K = 300, 384
    codes, _ = synth.fp8_weights(N, K, seed=15)
    codes = codes.numpy()
    q0, s0, _ = quant.requant_fp8_to_int8_channel(codes, np.ones((3, 3), np.float32))
    exps = np.array([-6.0, 4.0, 11.0])
    si = np.repeat((2.0 ** exps)[:, None], 3, axis=1).astype(np.float32)
    q1, s1, _ = quant.requant_fp8_to_int8_channel(codes, si)
    assert np.array_equal(q0, q1)
    assert np.array_equal(s1, (s0 * (2.0 ** exps)[np.arange(N) // 128]).astype(np.float32))

"""Pins of the asymmetric per-tensor quantiser and its GEMM (no GPU).

What pins them, besides themselves:
  * a hand-worked example (range [-1, 3] over 255 codes) and constructed
    exact ties (golden/asym_ties.json: rounding mode, division rather than a
    reciprocal multiply);
  * exact rational arithmetic (fractions) for the fp32 scale, zero point and
    every quotient;
  * the range ends map to codes 0 and 255, a constant tensor to all zeros
    with the floored scale, and the round-trip bound |s (q - z) - x| <= s/2
    up to the fp32 rounding of z;
  * a pure-Python loop for the integer sums, the dequantise-then-multiply
    route in fp64 for the GEMM, and its distance to the unquantised product.
"""

import json
import os
from fractions import Fraction

import numpy as np

import synth
from oracle import asym, formats


HERE = os.path.dirname(os.path.abspath(__file__))


def _round_to_f32(fr):
    """Round a Fraction to the nearest float32, ties to even (exact search)."""
    f = np.float32(float(fr))
    cands = [f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - fr),
                                     int(np.array(c, np.float32).view(np.uint32)) & 1))
    return np.float32(best)


def _bf16(vals):
    return formats.f32_to_bf16_bits(np.asarray(vals, np.float32))


def test_hand_worked_example():
    # x = [-1, 0, 0.5, 3]: mn = -1, range 4, s = fp32(4/255) = 0.015686275,
    # z = fp32(1/s) = 63.75, codes rne((x + 1)/s) = [0, 63.75 -> 64,
    # 95.625 -> 96, 255]
    q, s, z = asym.quant_act_asym(_bf16([[-1.0, 0.0, 0.5, 3.0]]))
    assert s == _round_to_f32(Fraction(4, 255))
    assert abs(float(z) - 63.75) < 1e-4
    assert q.tolist() == [[0, 64, 96, 255]]


def test_golden_ties():
    """Exact half-integer quotients (golden/asym_ties.json): round half to
    even on an exact fp32 division."""
    g = json.load(open(os.path.join(HERE, "golden", "asym_ties.json")))
    xs = [c[0] for c in g["cases"]]
    q, s, z = asym.quant_act_asym(_bf16([xs]))
    assert float(s) == g["scale"]
    assert z == _round_to_f32(Fraction(1, 8) / Fraction(7, 8))
    assert q[0].tolist() == [c[1] for c in g["cases"]]


def test_scale_zero_point_and_codes_are_correctly_rounded_fp32():
    x = synth.to_numpy(synth.activations(6, 256, seed=3))
    q, s, z = asym.quant_act_asym(x)
    v = formats.bf16_bits_to_f32(x)
    mn, mx = Fraction(float(v.min())), Fraction(float(v.max()))
    rng = _round_to_f32(mx - mn)
    s_exact = _round_to_f32(Fraction(float(rng)) / 255)
    assert s == s_exact
    assert z == _round_to_f32(-mn / Fraction(float(s_exact)))
    rs = np.random.default_rng(0)
    for idx in rs.choice(v.size, 300, replace=False):
        xv = Fraction(float(v.flat[idx]))
        d = _round_to_f32(xv - mn)
        quo = _round_to_f32(Fraction(float(d)) / Fraction(float(s_exact)))
        want = min(255, max(0, int(np.rint(np.float64(quo)))))
        assert q.flat[idx] == want


def test_range_ends_constant_tensor_and_round_trip():
    x = synth.to_numpy(synth.activations(16, 512, seed=5))
    q, s, z = asym.quant_act_asym(x)
    v = formats.bf16_bits_to_f32(x)
    assert q.flat[np.argmin(v)] == 0 and q.flat[np.argmax(v)] == 255
    err = np.abs(asym.dequant_asym(q, s, z) - v.astype(np.float64))
    # s/2 from the rounding of the code, plus the fp32 rounding of z (and of
    # the fp32 quotient) scaled by s
    bound = float(s) * (0.5 + (abs(float(z)) + 256.0) * 2.0 ** -23)
    assert err.max() <= bound
    # codes are monotone in x
    order = np.argsort(v.ravel(), kind="stable")
    assert np.all(np.diff(q.ravel()[order].astype(int)) >= 0)
    # constant tensors: every code 0, scale fp32(1e-10 / 255), x^ = x
    for c in (0.0, 2.5, -7.0):
        qc, sc, zc = asym.quant_act_asym(_bf16(np.full((3, 128), c)))
        assert not qc.any()
        assert sc == _round_to_f32(Fraction(float(np.float32(1e-10))) / 255)
        assert abs(float(asym.dequant_asym(qc, sc, zc)[0, 0]) - c) <= abs(c) * 1e-6


def test_all_positive_and_all_negative_tensors():
    for sign in (1.0, -1.0):
        v = sign * (1.0 + np.abs(np.random.default_rng(7).standard_normal((4, 128))))
        q, s, z = asym.quant_act_asym(_bf16(v))
        # z is the code of 0, which lies below (above) the range
        assert (z < 0) if sign > 0 else (z > 255)
        assert q.min() == 0 and q.max() == 255


def test_gemm_integer_sums_by_loop():
    rs = np.random.default_rng(11)
    q = rs.integers(0, 256, (3, 128)).astype(np.uint8)
    Wq = rs.integers(-127, 128, (5, 128)).astype(np.int8)
    ACC, WS, _, _ = asym.gemm_asym(q, np.float32(0.01), np.float32(100.25), Wq, np.ones(5, np.float32))
    for m in range(3):
        for n in range(5):
            assert ACC[m, n] == sum(int(q[m, k]) * int(Wq[n, k]) for k in range(128))
    for n in range(5):
        assert WS[n] == sum(int(Wq[n, k]) for k in range(128))


def test_gemm_equals_dequantised_route_and_approximates_the_product():
    x = synth.to_numpy(synth.activations(24, 384, seed=13))
    w = synth.to_numpy(synth.weights(40, 384, seed=14))
    q, s, z = asym.quant_act_asym(x)
    w32 = formats.bf16_bits_to_f32(w)
    sw = (np.abs(w32).max(axis=1) / np.float32(127)).astype(np.float32)
    Wq = np.clip(np.rint((w32 / sw[:, None]).astype(np.float32)), -127, 127).astype(np.int8)
    _, _, y64, y32 = asym.gemm_asym(q, s, z, Wq, sw)
    xhat = asym.dequant_asym(q, s, z)
    what = sw.astype(np.float64)[:, None] * Wq.astype(np.float64)
    route = xhat @ what.T
    assert np.abs(y64 - route).max() <= 1e-12 * np.abs(route).max()
    # a sign slip on z (adding z WS) or a dropped z term moves it far
    ACC = q.astype(np.float64) @ Wq.astype(np.float64).T
    WS = Wq.astype(np.float64).sum(axis=1)
    wrong = float(s) * sw.astype(np.float64)[None, :] * (ACC + float(z) * WS[None, :])
    assert np.abs(wrong - route).max() > 1e3 * np.abs(y64 - route).max()
    # the fp32 evaluation stays close to the fp64 one
    assert np.abs(y32 - y64).max() <= 1e-5 * np.abs(y64).max()
    # and the whole thing approximates the unquantised product
    exact = formats.bf16_bits_to_f32(x).astype(np.float64) @ w32.astype(np.float64).T
    assert np.abs(y64 - exact).max() <= 0.05 * np.abs(exact).max()

"""Pins of the oracle's INT4 weights and W4A16 GEMM (no GPU).

The reading pinned (page 3 section 3.3 reports INT4 by measurement only): the
page-5 group-wise weight scheme with qmax = 7, codes in offset binary two per
byte.  What pins it, besides itself:
  * the byte layout, worked by hand from that definition, and every one of
    the 256 byte values unpacked by integer division instead of masks;
  * exact rational arithmetic for the correctly rounded fp32 scale and
    quotient;
  * tie cases on a group whose scale is exactly 1 (rounding half to even);
  * the round-trip bound |x - q s| <= s/2, -8 never produced, amax -> +-7;
  * the GEMM against an exact rational sum on a tiny brute-force case.
"""

from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import formats, gemm, int4


def _round_to_f32(fr):
    """Round a Fraction to the nearest float32, ties to even (exact search)."""
    f = np.float32(float(fr))
    cands = [f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - fr),
                                     int(np.array(c, np.float32).view(np.uint32)) & 1))
    return np.float32(best)


def test_pack_layout_hand_worked():
    # q = -7, 7, 0, 1, -1, 3 -> u = q + 8 = 1, 15, 8, 9, 7, 11;
    # byte j = u[2j] | u[2j+1] << 4 -> 0xF1, 0x98, 0xB7
    q = np.array([[-7, 7, 0, 1, -1, 3]], np.int8)
    p = int4.pack_int4(q)
    assert p.dtype == np.uint8 and p.tolist() == [[0xF1, 0x98, 0xB7]]
    assert np.array_equal(int4.unpack_int4(p), q)


def test_unpack_every_byte():
    b = np.arange(256, dtype=np.uint8)[None, :]
    q = int4.unpack_int4(b)
    for v in range(256):
        hi, lo = divmod(v, 16)
        assert (int(q[0, 2 * v]), int(q[0, 2 * v + 1])) == (lo - 8, hi - 8)


def test_pack_round_trip_all_code_pairs():
    c = np.arange(-7, 8, dtype=np.int8)
    a, b = np.meshgrid(c, c, indexing="ij")
    q = np.stack([a.ravel(), b.ravel()], axis=1).reshape(1, -1)
    assert np.array_equal(int4.unpack_int4(int4.pack_int4(q)), q)


def test_scale_and_quotient_are_correctly_rounded_fp32_divisions():
    w = synth.to_numpy(synth.weights(6, 512, seed=41))
    q, s = int4.quant_weight_int4_group(w)
    g = formats.bf16_bits_to_f32(w).reshape(6, 4, 128)
    rng = np.random.default_rng(5)
    for (n, kb) in [(0, 0), (1, 3), (3, 2), (5, 1)]:
        amax = Fraction(float(np.abs(g[n, kb]).max()))
        s_exact = _round_to_f32(amax / 7)
        assert s[n, kb] == s_exact
        for j in rng.integers(0, 128, 32):
            quo = _round_to_f32(Fraction(float(g[n, kb, j])) / Fraction(float(s_exact)))
            want = int(np.rint(np.float64(quo)))
            assert q[n, kb * 128 + j] == max(-7, min(7, want))


def test_ties_round_half_to_even():
    # a group with amax 7 has scale exactly 1, so x / s = x
    vals = np.zeros(128, np.float32)
    vals[:9] = [7.0, 0.5, 1.5, 2.5, -2.5, 3.5, -0.5, 6.5, -7.0]
    q, s = int4.quant_weight_int4_group(vals[None, :])
    assert s[0, 0] == np.float32(1.0)
    assert q[0, :9].tolist() == [7, 0, 2, 2, -2, 4, 0, 6, -7]
    assert np.all(q[0, 9:] == 0)


def test_zero_group_and_range():
    w = np.zeros((2, 256), np.float32)
    w[1, 128:] = np.linspace(-3, 3, 128, dtype=np.float32)
    q, s = int4.quant_weight_int4_group(w)
    assert np.all(q[0] == 0) and np.all(q[1, :128] == 0)
    assert s[0, 0] == np.float32(np.float32(1e-10) / np.float32(7))
    assert q[1, 128] == -7 and q[1, 255] == 7


def test_round_trip_bound_and_no_minus_eight():
    w = synth.to_numpy(synth.weights(64, 1024, seed=42))
    q, s = int4.quant_weight_int4_group(w)
    assert q.min() >= -7 and q.max() <= 7
    x = formats.bf16_bits_to_f32(w).astype(np.float64)
    se = np.repeat(s.astype(np.float64), 128, axis=1)
    err = np.abs(x - q.astype(np.float64) * se)
    assert np.all(err <= se * 0.5 * (1 + 2.0 ** -16))
    # every group reaches +-7 at its amax
    amax_code = np.abs(q.reshape(64, 8, 128)).max(axis=2)
    assert np.all(amax_code == 7)


def test_w4a16_gemm_brute_force():
    rng = np.random.default_rng(9)
    M, N, K = 3, 5, 256
    x = (rng.standard_normal((M, K)) * 2).astype(np.float16)
    q = rng.integers(-7, 8, (N, K)).astype(np.int8)
    s = rng.uniform(1e-3, 1e-1, (N, K // 128)).astype(np.float32)
    y64, y32 = int4.gemm_w4a16_group(x, int4.pack_int4(q), s)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(float(s[n, k // 128])) * Fraction(float(x[m, k])) * int(q[n, k])
                        for k in range(K))
            assert abs(Fraction(float(y64[m, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 60)
            # fp32 with products exact: at most ~K roundings of 2^-24 relative
            bound = sum(abs(Fraction(float(s[n, k // 128])) * Fraction(float(x[m, k])) * int(q[n, k]))
                        for k in range(K)) * Fraction(K + 8, 2 ** 24)
            assert abs(Fraction(float(y32[m, n])) - exact) <= bound


def test_w4a16_on_codes_is_the_w8a16_formula():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((4, 384)).astype(np.float16)
    q = rng.integers(-7, 8, (6, 384)).astype(np.int8)
    s = rng.uniform(1e-3, 1e-1, (6, 3)).astype(np.float32)
    a64, a32 = int4.gemm_w4a16_group(x, int4.pack_int4(q), s)
    b64, b32 = gemm.gemm_w8a16_group(x, q, s)
    assert np.array_equal(a64, b64) and np.array_equal(a32.view(np.uint32), b32.view(np.uint32))

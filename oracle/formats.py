"""Number formats used on the path, written from their definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* bf16: the top 16 bits of an IEEE binary32 value.  Widening is exact; the
  narrowing used by the offline conversion (FP8 -> BF16 before the INT8
  quantisation, page 1 section 2.3) rounds to nearest, ties to even.
* fp16: IEEE binary16 (numpy's float16), used by the W8A16 variant of the
  release note on page 5 ("DeepSeek-R1-0528-Qwen3-8B Int8 W8A16").
* FP8: the DeepSeek checkpoints are FP8 (page 1 sections 1 and 2.2); page 4
  section 2.1 names the layout E4M3 (4 exponent bits, 3 mantissa bits).  The
  encoding decoded here is the OCP "E4M3FN" variant: exponent bias 7, no
  infinities, S.1111.111 is NaN, largest finite value 448.  (Page 4's printed
  dynamic range for E4M3 is not the range of this format; the layout is what
  is taken from it.)
"""

import numpy as np

F32 = np.float32


def bf16_bits_to_f32(bits):
    """Widen bf16 bit patterns (uint16) to float32; exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def f32_to_bf16_bits(x):
    """Round float32 values to bf16, nearest-even; returns uint16 bit patterns.

    The 16 low bits of the binary32 pattern are dropped.  If they exceed half
    of one bf16 unit in the last place the kept part is incremented; if they
    equal exactly half, it is incremented only when the kept part is odd.
    Inputs are finite (NaN is outside the path's contract).
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    hi = u >> np.uint64(16)
    lo = u & np.uint64(0xFFFF)
    half = np.uint64(0x8000)
    up = (lo > half) | ((lo == half) & ((hi & np.uint64(1)) == np.uint64(1)))
    return (hi + up.astype(np.uint64)).astype(np.uint16)


def e4m3fn_to_f32(codes):
    """Decode OCP FP8-E4M3FN byte codes to float32 (exact).

    exponent field e (4 bits), mantissa field m (3 bits), sign s:
      e == 0          : (-1)^s * m * 2^-9            (zero and subnormals)
      e == 15, m == 7 : NaN
      otherwise       : (-1)^s * (1 + m/8) * 2^(e-7)
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = c >> 7
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0,
                   np.ldexp(m.astype(np.float64), -9),
                   np.ldexp(1.0 + m.astype(np.float64) / 8.0, (e - 7).astype(np.int64)))
    val = np.where(s == 1, -mag, mag)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return val.astype(np.float32)

"""Asymmetric per-tensor UINT8 activations with symmetric per-channel INT8
weights: the "dynamic range-aware" variant.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: page 2, "Meituan open-sources a lossless INT8 DeepSeek R1: technical
breakthroughs and practice guide" (xfz.ruibaoantu.com), part two, item 1
"dynamic range-aware quantisation" and its pseudocode.  For one activation
tensor (one layer's input) the page takes the tensor's minimum and maximum,
spreads that range over the 256 codes of an unsigned byte, and records the
zero point as the (unrounded) code of 0:

    mn, mx = min(x), max(x)
    s  = (mx - mn) / 255
    z  = -mn / s
    q  = clamp(round((x - mn) / s), 0, 255)

Dequantisation is x^ = s (q - z).  The page's main scheme (page 1) is
symmetric; this variant is an alternative the library offers beside it.

Readings taken where the page is silent:
  * every step is an fp32 IEEE operation (subtraction, division) on the
    fp32 values of the bf16 / fp16 inputs; round() is half-to-even, as in
    the symmetric quantiser;
  * a constant tensor (mx == mn) would divide by zero: the range is floored
    at eps = fp32(1e-10), as the symmetric quantiser floors its amax, so
    every code is 0 and s = fp32(1e-10 / 255);
  * z is kept as the fp32 quotient, not rounded to an integer (the
    pseudocode does not round it);
  * the weights stay symmetric per output channel (page 1, channel-wise
    scheme): w^[n, k] = w_scale[n] Wq[n, k].

The GEMM of the two:

    Y[m, n] = sum_k x^[m, k] w^[n, k] = s w_scale[n] (ACC[m, n] - z WS[n])
    ACC[m, n] = sum_k q[m, k] Wq[n, k]      (exact integer)
    WS[n]     = sum_k Wq[n, k]               (exact integer)

y64 evaluates it in fp64 from the stored fp32 s, z and w_scale; y32 in fp32 in
the fixed order fp32(fp32(s * w_scale[n]) * fp32(fp32(ACC) - fp32(z * fp32(WS)))).
"""

import numpy as np

from .quant import widen

F32 = np.float32
F64 = np.float64
EPS = np.float32(1e-10)
UMAX = np.float32(255.0)


def quant_act_asym(x):
    """Per-tensor asymmetric quantisation of x [M, K] (bf16 bits, fp16, fp32).

    Returns q uint8 [M, K] and the fp32 scalars s (scale) and z (zero point).
    """
    x32 = widen(x)
    mn = x32.min() if x32.size else F32(0)
    mx = x32.max() if x32.size else F32(0)
    rng = np.maximum(F32(mx - mn), EPS)
    s = F32(rng / UMAX)
    z = F32(-mn / s)
    d = (x32 - mn).astype(F32)
    q = np.clip(np.rint((d / s).astype(F32)), 0, 255).astype(np.uint8)
    return q, s, z


def dequant_asym(q, s, z):
    """x^ = s (q - z) in fp64 from the stored fp32 s and z."""
    return F64(s) * (np.asarray(q, F64) - F64(z))


def weight_row_sums(Wq):
    """WS[n] = sum_k Wq[n, k] (exact)."""
    return np.asarray(Wq, np.int64).sum(axis=1)


def gemm_asym(q, s, z, Wq, w_scale):
    """Asymmetric UINT8 activations times symmetric per-channel INT8 weights.

    q uint8 [M, K], s and z fp32 scalars, Wq int8 [N, K], w_scale fp32 [N].
    Returns (ACC int64, WS int64, y64, y32).
    """
    ACC = q.astype(F64) @ np.asarray(Wq, F64).T          # |sums| < 2^53: exact
    ACC = ACC.astype(np.int64)
    WS = weight_row_sums(Wq)
    sw = np.asarray(w_scale, F32)
    y64 = F64(s) * sw.astype(F64)[None, :] * (ACC.astype(F64) - F64(z) * WS.astype(F64)[None, :])
    c32 = (F32(s) * sw).astype(F32)
    zw32 = (F32(z) * WS.astype(F32)).astype(F32)
    y32 = (c32[None, :] * (ACC.astype(F32) - zw32[None, :]).astype(F32)).astype(F32)
    return ACC, WS, y64, y32

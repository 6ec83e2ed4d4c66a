"""INT4 group-wise weights and the W4A16 GEMM.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The page "DeepSeek-R1-Distill-Llama-8B quantisation practice" (page 3),
section 3.3, compares INT4 with INT8 by measurement only (memory, speed,
accuracy) and states no scheme.  The reading taken here, and by the library:
the group-wise weight scheme of the W8A16 release note (page 5: symmetric
group-wise weights, groups of 128 along K, fp16 activations) with a 4-bit code
range, so that the quantiser of page 4 (section 3.2.1, int8 branch) becomes

    s = fp32(max(amax, eps) / 7)
    q = clamp(round_half_even(fp32(x / s)), -7, 7)

(the symmetric range leaves -8 unused, as INT8 leaves -128), and the codes are
stored two per byte in offset binary, u = q + 8 in [1, 15], the even k in the
low nibble and the odd k in the high nibble.  The 4-bit width is what the
page's memory figure implies: about half a byte per weight for an 8B model.

The GEMM is the group-wise formula of the W8A16 variant applied to these
codes:

    Y[m, n] = sum_g s[n, g] * sum_{k in group g} x[m, k] * q[n, k]
"""

import numpy as np

from .quant import widen, EPS
from .gemm import gemm_w8a16_group

F32 = np.float32
QMAX4 = np.float32(7.0)
GROUP = 128


def quant_weight_int4_group(w):
    """Group-wise INT4 weight quantisation, groups of 1 x 128 along K.

    w: [N, K] bf16 bits (uint16), fp16 or fp32.  Returns (q int8 [N, K] in
    [-7, 7], s fp32 [N, K / 128]).
    """
    x32 = widen(w)
    N, K = x32.shape
    g = x32.reshape(N, K // GROUP, GROUP)
    amax = np.abs(g).max(axis=2)
    s = (np.maximum(amax, EPS) / QMAX4).astype(F32)
    y = (g / s[:, :, None]).astype(F32)
    q = np.clip(np.rint(y), -7, 7).astype(np.int8)
    return q.reshape(N, K), s


def pack_int4(q):
    """int8 codes [N, K] in [-8, 7] -> uint8 [N, K / 2]: byte j holds q[:, 2j] + 8
    in its low nibble and q[:, 2j + 1] + 8 in its high nibble."""
    q = np.asarray(q)
    u = (q.astype(np.int16) + 8).astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def unpack_int4(p):
    """uint8 [N, K / 2] -> int8 codes [N, K] (nibble value minus 8)."""
    p = np.asarray(p, np.uint8)
    N, H = p.shape
    q = np.empty((N, 2 * H), np.int8)
    q[:, 0::2] = (p & 0x0F).astype(np.int8) - 8
    q[:, 1::2] = (p >> 4).astype(np.int8) - 8
    return q


def gemm_w4a16_group(x, W4, w_scale):
    """W4A16 group-wise GEMM: x fp16 [M, K], W4 packed uint8 [N, K / 2], w_scale
    fp32 [N, K / 128].  Returns (y64, y32) with the evaluation orders of
    gemm.gemm_w8a16_group on the unpacked codes."""
    return gemm_w8a16_group(x, unpack_int4(W4), w_scale)

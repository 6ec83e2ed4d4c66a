"""The symmetric INT8 quantisers and the offline FP8 -> BF16 -> INT8 conversion.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The quantiser (page 4, "FP8 vs INT8 quantisation for DeepSeek", section 3.2.1,
int8 branch of the QAT example; page 1 section 2.1 "basic principle": compute
a scaling factor, then quantise and dequantise) is, for one group of values:

    s = max(amax, eps) / 127          (fp32, IEEE division)
    q = clamp(round_half_even(x / s), -127, 127)   (x / s in fp32, IEEE)

Readings taken where the pages are silent:
  * round() is half-to-even (the PyTorch ``round`` used on page 4);
  * the quotient x / s is the correctly rounded fp32 division, as written;
  * a group whose amax is 0 would give 0/0: amax is clamped to eps = fp32(1e-10),
    so such a group quantises to all zeros with a tiny finite scale;
  * the symmetric range is [-127, 127]; -128 is never produced.

Groups (page 1 section 2.3):
  * token-group (block-wise scheme): 1 x 128 along K of each activation row;
  * token (channel-wise scheme): a whole activation row;
  * 128 x 128 weight tiles (block-wise scheme), clipped at the N edge;
  * one output channel (channel-wise weights) is a whole row of W[N, K], i.e.
    the token quantiser applied to W.
"""

import numpy as np

from .formats import bf16_bits_to_f32, f32_to_bf16_bits, e4m3fn_to_f32

F32 = np.float32
EPS = np.float32(1e-10)
QMAX = np.float32(127.0)
GROUP = 128


def widen(x):
    """bf16 bit patterns (uint16), fp16 or fp32 -> float32 (exact)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x)
    if x.dtype == np.float16:
        return x.astype(np.float32)
    if x.dtype == np.float32:
        return x
    raise TypeError(f"unsupported input dtype {x.dtype}")


def scale_from_amax(amax):
    """s = fp32(max(amax, eps) / 127)."""
    a = np.maximum(np.asarray(amax, dtype=np.float32), EPS)
    return (a / QMAX).astype(np.float32)


def quantise_values(x32, s):
    """q = clamp(rint(fp32(x / s)), -127, 127) with s broadcast over x."""
    y = (x32 / s).astype(np.float32)
    return np.clip(np.rint(y), -127, 127).astype(np.int8)


def quant_act_group(x):
    """Per-token-group quantisation, groups of 1 x 128 along K.

    x: [M, K] (bf16 bits, fp16 or fp32), K % 128 == 0.
    Returns q int8 [M, K] and a_scale fp32 [M, K/128].
    """
    x32 = widen(x)
    M, K = x32.shape
    assert K % GROUP == 0
    g = x32.reshape(M, K // GROUP, GROUP)
    amax = np.abs(g).max(axis=2) if M > 0 else np.zeros((0, K // GROUP), F32)
    s = scale_from_amax(amax)
    q = quantise_values(g, s[:, :, None]).reshape(M, K)
    return q, s


def quant_act_token(x):
    """Per-token quantisation: one group per row.

    x: [M, K].  Returns q int8 [M, K] and a_scale fp32 [M].
    Applied to a weight W[N, K] this is the channel-wise weight quantiser
    (one scale per output channel).
    """
    x32 = widen(x)
    M, K = x32.shape
    amax = np.abs(x32).max(axis=1) if K > 0 else np.zeros(M, F32)
    s = scale_from_amax(amax)
    q = quantise_values(x32, s[:, None])
    return q, s


def quant_weight_block(w):
    """Block-wise weight quantisation in 128 x 128 tiles.

    w: [N, K] (bf16 bits or fp32), K % 128 == 0; the last tile row may hold
    fewer than 128 rows (amax over the rows that exist).
    Returns q int8 [N, K] and w_scale fp32 [ceil(N/128), K/128].
    """
    w32 = widen(w)
    N, K = w32.shape
    assert K % GROUP == 0
    KB = K // GROUP
    NB = (N + GROUP - 1) // GROUP
    q = np.empty((N, K), np.int8)
    s = np.empty((NB, KB), np.float32)
    for nb in range(NB):
        r0, r1 = nb * GROUP, min(N, (nb + 1) * GROUP)
        t = w32[r0:r1].reshape(r1 - r0, KB, GROUP)
        amax = np.abs(t).max(axis=(0, 2))
        s[nb] = scale_from_amax(amax)
        q[r0:r1] = quantise_values(t, s[nb][None, :, None]).reshape(r1 - r0, K)
    return q, s


def dequant_fp8_to_bf16(codes, scale_inv):
    """FP8-E4M3FN [N, K] with per-128x128 scale_inv -> bf16 bits [N, K].

    w = bf16_rne(fp32(decode(code) * scale_inv[n // 128, k // 128])).
    The dequantised value is multiplied by scale_inv (the DeepSeek checkpoint
    stores the inverse of the quantisation scale under that name).
    """
    f8 = e4m3fn_to_f32(codes)
    N, K = f8.shape
    si = np.asarray(scale_inv, dtype=np.float32)
    rows = np.arange(N) // GROUP
    cols = np.arange(K) // GROUP
    prod = (f8 * si[rows][:, cols]).astype(np.float32)
    return f32_to_bf16_bits(prod)


def requant_fp8_to_int8_block(codes, scale_inv):
    """Offline conversion of page 1 section 2.3: FP8 -> BF16 -> INT8 128x128 tiles.

    Returns (q int8 [N, K], w_scale fp32 [NB, KB], w_bf16 bits [N, K]).
    """
    wb = dequant_fp8_to_bf16(codes, scale_inv)
    q, s = quant_weight_block(wb)
    return q, s, wb


def requant_fp8_to_int8_channel(codes, scale_inv):
    """Channel-wise variant of the same conversion (page 1 section 2.3,
    channel-wise paragraph): FP8 -> BF16, then one scale per output channel."""
    wb = dequant_fp8_to_bf16(codes, scale_inv)
    q, s = quant_act_token(wb)
    return q, s, wb

"""The INT8 GEMMs of the two schemes, the W8A16 variant and the grouped MoE GEMM.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Layouts (nn.Linear convention; the pages print none): activations A[M, K],
weights W[N, K], output Y[M, N] = A . W^T, all row-major.  KB = K / 128 and
NB = ceil(N / 128).

Block-wise scheme (page 1 section 2.3, block-wise paragraph and Figure 3):
because every 128 x 128 weight tile and every 1 x 128 activation group has its
own scale, the INT8 matmul is dequantised once per 128-wide K block:

    P[kb, m, n] = sum_{k in block kb} Aq[m, k] * Wq[n, k]          (exact int32)
    Y[m, n]     = sum_kb a_scale[m, kb] * w_scale[n // 128, kb] * P[kb, m, n]

Channel-wise scheme (page 1 section 2.3, channel-wise paragraph): one
dequantisation after the INT8 matmul:

    ACC[m, n] = sum_k Aq[m, k] * Wq[n, k]                          (exact int32)
    Y[m, n]   = a_scale[m] * w_scale[n] * ACC[m, n]

Two float evaluations are returned:
  y64 - every product and sum in fp64 (the accuracy reference);
  y32 - fp32 in a fixed order: for the block scheme
        acc = fp32(acc + fp32(fp32(sa * sw) * fp32(P))) over kb = 0, 1, ...;
        for the channel scheme fp32(fp32(ACC) * fp32(sa * sw)).

The integer products use a float64 matrix product (a library routine): every
partial sum is an integer of magnitude below 2^53, so the result is exact.
"""

import numpy as np

from .quant import widen

F32 = np.float32
F64 = np.float64
GROUP = 128


def _int_matmul(a_i8, w_i8):
    """Exact int64 A . W^T of int8 matrices (fp64 product; |sums| << 2^53)."""
    r = a_i8.astype(F64) @ w_i8.astype(F64).T
    return r.astype(np.int64)


def block_partials(Aq, Wq):
    """P[kb, m, n] int32: the exact int8 dot product over each 128-wide K block."""
    M, K = Aq.shape
    N = Wq.shape[0]
    assert Wq.shape[1] == K and K % GROUP == 0
    KB = K // GROUP
    P = np.empty((KB, M, N), np.int32)
    for kb in range(KB):
        ks = slice(kb * GROUP, (kb + 1) * GROUP)
        P[kb] = _int_matmul(Aq[:, ks], Wq[:, ks])
    return P


def gemm_block(Aq, a_scale, Wq, w_scale, P=None):
    """Block-wise W8A8 GEMM.  Returns (P, y64, y32)."""
    if P is None:
        P = block_partials(Aq, Wq)
    KB, M, N = P.shape
    sa = np.asarray(a_scale, F32).reshape(M, KB)
    swn = np.asarray(w_scale, F32)[np.arange(N) // GROUP]          # [N, KB]
    y64 = np.zeros((M, N), F64)
    acc = np.zeros((M, N), F32)
    for kb in range(KB):
        y64 += sa[:, kb].astype(F64)[:, None] * swn[:, kb].astype(F64)[None, :] * P[kb].astype(F64)
        s32 = (sa[:, kb][:, None] * swn[:, kb][None, :]).astype(F32)
        acc = (acc + (s32 * P[kb].astype(F32)).astype(F32)).astype(F32)
    return P, y64, acc


def gemm_channel(Aq, a_scale, Wq, w_scale):
    """Channel-wise W8A8 GEMM.  Returns (ACC int32, y64, y32)."""
    acc64 = _int_matmul(Aq, Wq)
    assert np.all(np.abs(acc64) < 2 ** 31)
    ACC = acc64.astype(np.int32)
    sa = np.asarray(a_scale, F32)
    sw = np.asarray(w_scale, F32)
    y64 = sa.astype(F64)[:, None] * sw.astype(F64)[None, :] * acc64.astype(F64)
    s32 = (sa[:, None] * sw[None, :]).astype(F32)
    y32 = (ACC.astype(F32) * s32).astype(F32)
    return ACC, y64, y32


def gemm_w8a16_group(x, Wq, w_scale):
    """W8A16 group-wise GEMM (page 5, symmetric group-wise INT8 weights with
    fp16 activations), groups of 128 along K.

        Y[m, n] = sum_g w_scale[n, g] * sum_{k in g} x[m, k] * Wq[n, k]

    x: fp16 [M, K]; Wq int8 [N, K]; w_scale fp32 [N, K/128].
    Returns (y64, y32).  y32 is evaluated in fp32 in a fixed order: inside
    each group the dot product runs k = 128 g, 128 g + 1, ... with
    partial = fp32(partial + fp32(x * q)) (every product of an fp16 value and
    an int8 code is exact in fp32, so only the sums round), then across
    groups acc = fp32(acc + fp32(s * partial)) for g = 0, 1, ...
    """
    x32 = widen(x)
    M, K = x32.shape
    N = Wq.shape[0]
    KB = K // GROUP
    s = np.asarray(w_scale, F32).reshape(N, KB)
    wq32 = np.asarray(Wq).astype(F32)
    y64 = np.zeros((M, N), F64)
    acc = np.zeros((M, N), F32)
    for g in range(KB):
        ks = slice(g * GROUP, (g + 1) * GROUP)
        y64 += (x32[:, ks].astype(F64) @ wq32[:, ks].astype(F64).T) * s[:, g].astype(F64)[None, :]
        part = np.zeros((M, N), F32)
        for k in range(g * GROUP, (g + 1) * GROUP):
            part = (part + x32[:, k][:, None] * wq32[:, k][None, :]).astype(F32)
        acc = (acc + (s[:, g][None, :] * part).astype(F32)).astype(F32)
    return y64, acc


def gemm_block_grouped(Aq, a_scale, Wq, w_scale, offsets):
    """Grouped block-wise GEMM for MoE: rows offsets[e]:offsets[e+1] of the
    expert-sorted activations use expert e's weights Wq[e], w_scale[e].
    Returns (y64, y32) of shape [P, N]."""
    P_rows, K = Aq.shape
    E, N, _ = Wq.shape
    y64 = np.zeros((P_rows, N), F64)
    y32 = np.zeros((P_rows, N), F32)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 <= r0:
            continue
        _, a, b = gemm_block(Aq[r0:r1], a_scale[r0:r1], Wq[e], w_scale[e])
        y64[r0:r1] = a
        y32[r0:r1] = b
    return y64, y32


def normwise_rel_err(y, ref):
    """||y - ref||_inf / ||ref||_inf over the whole tensor."""
    y = np.asarray(y, F64)
    ref = np.asarray(ref, F64)
    den = np.abs(ref).max() if ref.size else 0.0
    if den == 0.0:
        return float(np.abs(y - ref).max()) if ref.size else 0.0
    return float(np.abs(y - ref).max() / den)

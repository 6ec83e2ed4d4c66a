"""GPU parity of the one-call linear layers (online activation quantisation,
then the INT8 GEMM; page "DeepSeek R1 INT8 quantisation in SGLang",
section 2.3).

linear_w8a8_block / linear_w8a8_channel against the oracle's quantiser
followed by its GEMM: the output within the GEMM bars of test_gpu_gemm
(channel-wise fp32 bit-exact, block-wise fp32 within 1e-5 normwise of the
oracle's fp32 path, both within 1e-2 of its fp64 path), and bit-identical to
the quantiser and GEMM entry points called one after the other; the int8
codes and fp32 scales left in the workspace bit-exact to the oracle's
quantiser.  One workspace serves two calls in a row, the second on a smaller
input.
"""

import numpy as np
import pytest
import torch

import synth
import w8a8_int8_quantized_amd as w8
from oracle import formats, gemm, quant

pytestmark = pytest.mark.gpu
DEV = "cuda"

# (M, N, K): decode rows (weight-streaming kernels), a split-K tile grid and
# ragged 128/256-row tiles; N ragged against the 128-column weight blocks.
CASES = [(1, 300, 256), (37, 700, 1024), (130, 513, 640), (300, 1100, 384)]
# decode rows on output widths that spread evenly over the CUs (the
# shared-activation weight-streaming kernel), odd numbers of K blocks
WIDE = [(1, 36864, 640), (5, 12288, 384), (16, 36864, 1152), (11, 12288, 128), (17, 12288, 384)]


def _np(t):
    return t.detach().cpu().numpy()


def _workspace_parts(ws, scheme, M, K):
    off = (M * K + 255) // 256 * 256
    ns = M * (K // 128) if scheme == w8.W8_SCHEME_BLOCK else M
    q = _np(ws[:M * K]).view(np.int8).reshape(M, K)
    s = _np(ws[off:off + 4 * ns]).view(np.float32)
    return q, s


def _inputs(M, N, K, seed, fp16):
    dt = torch.float16 if fp16 else torch.bfloat16
    x = synth.activations(M, K, seed=seed, dtype=dt)
    w = synth.to_numpy(synth.weights(N, K, seed=seed + 1))
    return x, (x.numpy() if fp16 else synth.to_numpy(x)), w


@pytest.mark.parametrize("fp16", [False, True])
@pytest.mark.parametrize("M,N,K", CASES + WIDE)
def test_linear_block(M, N, K, fp16):
    print(f"linear block M={M} N={N} K={K} fp16={fp16}", flush=True)
    x, xo, w = _inputs(M, N, K, seed=M + 11, fp16=fp16)
    qa, sa = quant.quant_act_group(xo)
    qw, sw = quant.quant_weight_block(w)
    _, y64, y32 = gemm.gemm_block(qa, sa, qw, sw)
    X = x.to(DEV)
    W, SW = (torch.from_numpy(a).to(DEV) for a in (qw, sw))
    ws = torch.empty(w8.linear_workspace_bytes(w8.W8_SCHEME_BLOCK, M, K), dtype=torch.uint8, device=DEV)
    y = w8.linear_w8a8_block(X, W, SW, out_dtype=torch.float32, workspace=ws)
    gq, gs = _workspace_parts(ws, w8.W8_SCHEME_BLOCK, M, K)
    assert np.array_equal(gq, qa)
    assert np.array_equal(gs.view(np.uint32), sa.reshape(-1).view(np.uint32))
    got = _np(y)
    e32, e64 = gemm.normwise_rel_err(got, y32), gemm.normwise_rel_err(got, y64)
    assert e32 <= 1e-5 and e64 <= 1e-2, (e32, e64)
    q2, s2 = w8.quant_act_group(X)
    ref = _np(w8.gemm_w8a8_block(q2, s2, W, SW, out_dtype=torch.float32))
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    yb = w8.linear_w8a8_block(X, W, SW, workspace=ws)
    assert np.array_equal(_np(yb.view(torch.int16)).view(np.uint16), formats.f32_to_bf16_bits(got))


@pytest.mark.parametrize("fp16", [False, True])
@pytest.mark.parametrize("M,N,K", CASES + WIDE)
def test_linear_channel(M, N, K, fp16):
    print(f"linear channel M={M} N={N} K={K} fp16={fp16}", flush=True)
    x, xo, w = _inputs(M, N, K, seed=M + 21, fp16=fp16)
    qa, sa = quant.quant_act_token(xo)
    qw, sw = quant.quant_act_token(w)
    _, y64, y32 = gemm.gemm_channel(qa, sa, qw, sw)
    X = x.to(DEV)
    W, SW = (torch.from_numpy(a).to(DEV) for a in (qw, sw))
    ws = torch.empty(w8.linear_workspace_bytes(w8.W8_SCHEME_CHANNEL, M, K), dtype=torch.uint8, device=DEV)
    y = w8.linear_w8a8_channel(X, W, SW, out_dtype=torch.float32, workspace=ws)
    gq, gs = _workspace_parts(ws, w8.W8_SCHEME_CHANNEL, M, K)
    assert np.array_equal(gq, qa)
    assert np.array_equal(gs.view(np.uint32), sa.view(np.uint32))
    got = _np(y)
    assert np.array_equal(got.view(np.uint32), y32.view(np.uint32))
    assert gemm.normwise_rel_err(got, y64) <= 1e-2
    yb = w8.linear_w8a8_channel(X, W, SW, workspace=ws)
    assert np.array_equal(_np(yb.view(torch.int16)).view(np.uint16), formats.f32_to_bf16_bits(y32))


@pytest.mark.parametrize("fp16", [False, True])
def test_linear_block_zero_and_extreme_groups(fp16):
    """Zero rows and groups (the 1e-10 floor), a group whose amax sits at
    both signs, and values of very different magnitude in one row (8 rows,
    N = 12288), bit-identical to the quantiser and GEMM called one after
    the other."""
    M, N, K = 8, 12288, 512
    x, _, w = _inputs(M, N, K, seed=77, fp16=fp16)
    x[3] = 0
    x[5, 128:256] = 0
    x[6, 0:128] = torch.linspace(-3.0, 3.0, 128).to(x.dtype)
    x[7, 256:384] *= 1000
    xo = x.numpy() if fp16 else synth.to_numpy(x)
    qa, sa = quant.quant_act_group(xo)
    qw, sw = quant.quant_weight_block(w)
    _, y64, y32 = gemm.gemm_block(qa, sa, qw, sw)
    X = x.to(DEV)
    W, SW = (torch.from_numpy(a).to(DEV) for a in (qw, sw))
    got = _np(w8.linear_w8a8_block(X, W, SW, out_dtype=torch.float32))
    q2, s2 = w8.quant_act_group(X)
    ref = _np(w8.gemm_w8a8_block(q2, s2, W, SW, out_dtype=torch.float32))
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert not got[3].any() and np.isfinite(got).all()
    e32 = gemm.normwise_rel_err(got, y32)
    assert e32 <= 1e-5, e32


def test_linear_workspace_reused_smaller():
    """One workspace, two calls in a row; the second input is smaller."""
    K, N = 512, 12288
    ws = torch.empty(w8.linear_workspace_bytes(w8.W8_SCHEME_BLOCK, 200, K), dtype=torch.uint8, device=DEV)
    for M in (200, 9):
        print(f"linear reuse M={M}", flush=True)
        x, xo, w = _inputs(M, N, K, seed=M + 31, fp16=False)
        qa, sa = quant.quant_act_group(xo)
        qw, sw = quant.quant_weight_block(w)
        _, y64, y32 = gemm.gemm_block(qa, sa, qw, sw)
        W, SW = (torch.from_numpy(a).to(DEV) for a in (qw, sw))
        got = _np(w8.linear_w8a8_block(x.to(DEV), W, SW, out_dtype=torch.float32, workspace=ws))
        e32, e64 = gemm.normwise_rel_err(got, y32), gemm.normwise_rel_err(got, y64)
        assert e32 <= 1e-5 and e64 <= 1e-2, (M, e32, e64)


def test_linear_rejects_short_workspace():
    x = torch.zeros(4, 128, dtype=torch.bfloat16, device=DEV)
    W = torch.zeros(8, 128, dtype=torch.int8, device=DEV)
    sw = torch.ones(1, 1, dtype=torch.float32, device=DEV)
    ws = torch.empty(w8.linear_workspace_bytes(w8.W8_SCHEME_BLOCK, 4, 128) - 4, dtype=torch.uint8, device=DEV)
    with pytest.raises(w8.W8Error, match="workspace"):
        w8.linear_w8a8_block(x, W, sw, workspace=ws)

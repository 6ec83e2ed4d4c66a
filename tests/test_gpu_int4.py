"""GPU parity of the INT4 weight quantiser and the W4A16 GEMM against the
CPU oracle (oracle/int4.py).

Bars:
  * packed INT4 codes and their fp32 scales: bit-exact (bf16 and fp16
    weights, hand-made tie groups, an all-zero group, ragged row counts);
  * W4A16 fp16 output: bit-identical to the W8A16 kernel run on the same
    codes unpacked to int8 (same fp16 operands, same fp32 order), and
    normwise relative error <= 1e-3 against the oracle's fp32 path and
    <= 1e-2 against its fp64 path, at the decode-kernel, staged-activation,
    shared-activation and split-K shapes and at the Qwen3-8B decode rows
    (sampled columns, as the benchmark runs them).
"""

import numpy as np
import pytest
import torch

import synth
import w8a8_int8_quantized_amd as w8
from oracle import formats, gemm, int4

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _np(t):
    return t.detach().cpu().numpy()


def _tie_weights(N, K, seed, dtype):
    w = synth.weights(N, K, seed=seed, dtype=torch.float32)
    # group (0, 0): scale exactly 1 with every half-integer tie; group (1, 0)
    # all zero (when present)
    w[0, :128] = 0.0
    w[0, :10] = torch.tensor([7.0, 0.5, 1.5, 2.5, -2.5, 3.5, -0.5, 6.5, -7.0, 5.5])
    if N > 1:
        w[1, :128] = 0.0
    return w.to(dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("N,K", [(3, 128), (100, 640), (257, 1024)])
def test_int4_quantiser_bit_exact(N, K, dtype):
    w = _tie_weights(N, K, seed=N + K, dtype=dtype)
    wn = synth.to_numpy(w) if dtype == torch.bfloat16 else w.numpy()
    q, s = int4.quant_weight_int4_group(wn)
    p = int4.pack_int4(q)
    P, S = w8.quant_weight_int4_group(w.to(DEV))
    assert P.shape == (N, K // 2) and P.dtype == torch.uint8
    assert np.array_equal(_np(P), p)
    assert np.array_equal(_np(S).view(np.uint32), s.view(np.uint32))
    assert _np(P)[0, :5].tolist() == [int4.pack_int4(np.array([[7, 0, 2, 2, -2, 4, 0, 6, -7, 6]], np.int8))[0, i]
                                     for i in range(5)]


SHAPES = [(1, 256, 512), (3, 4096, 12288), (8, 1000, 4096), (12, 12288, 4096), (32, 512, 1024),
          (64, 384, 12288), (100, 256, 256)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_w4a16_group(M, N, K):
    x = synth.activations(M, K, seed=M + 5, dtype=torch.float16)
    w = synth.weights(N, K, seed=N + 5, dtype=torch.float16)
    q, s = int4.quant_weight_int4_group(w.numpy())
    p = int4.pack_int4(q)
    y64, y32 = int4.gemm_w4a16_group(x.numpy(), p, s)
    X = x.to(DEV)
    P, Q, S = (torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (p, q, s))
    y = w8.gemm_w4a16_group(X, P, S)
    yn = _np(y).astype(np.float32)
    e32, e64 = gemm.normwise_rel_err(yn, y32), gemm.normwise_rel_err(yn, y64)
    assert e32 <= 1e-3 and e64 <= 1e-2, (e32, e64)
    # the same kernels on int8 codes give the same bits
    y8 = w8.gemm_w8a16_group(X, Q, S)
    assert torch.equal(y.view(torch.int16), y8.view(torch.int16))


def test_w4a16_after_gpu_quantiser_and_repeat():
    M, N, K = 8, 4096, 4096
    x = synth.activations(M, K, seed=81, dtype=torch.float16)
    w = synth.weights(N, K, seed=82, dtype=torch.float16)
    P, S = w8.quant_weight_int4_group(w.to(DEV))
    q, s = int4.quant_weight_int4_group(w.numpy())
    assert np.array_equal(_np(P), int4.pack_int4(q))
    y64, y32 = int4.gemm_w4a16_group(x.numpy(), int4.pack_int4(q), s)
    X = x.to(DEV)
    a = w8.gemm_w4a16_group(X, P, S)
    b = w8.gemm_w4a16_group(X, P, S)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    e32 = gemm.normwise_rel_err(_np(a).astype(np.float32), y32)
    assert e32 <= 1e-3, e32


def test_w4a16_empty_and_argument_errors():
    X = torch.zeros(0, 256, dtype=torch.float16, device=DEV)
    P = torch.zeros(64, 128, dtype=torch.uint8, device=DEV)
    S = torch.ones(64, 2, dtype=torch.float32, device=DEV)
    assert w8.gemm_w4a16_group(X, P, S).shape == (0, 64)
    with pytest.raises(w8.W8Error):
        w8.gemm_w4a16_group(torch.zeros(2, 256, dtype=torch.float16, device=DEV), P[:, :100].contiguous(), S)


# The benchmark's Qwen3-8B decode rows with INT4 weights: qkv K = 4096 ->
# N = 12288 and down K = 12288 -> N = 4096, M = 1, 8, 32, 64; three 128-column
# blocks (first, last, one inside) are checked against the oracle.
@pytest.mark.parametrize("name,K,N", [("qkv", 4096, 12288), ("down", 12288, 4096)])
def test_w4a16_full_size_sampled(name, K, N):
    w = synth.weights(N, K, seed=64, dtype=torch.float16)
    q, s = int4.quant_weight_int4_group(w.numpy())
    p = int4.pack_int4(q)
    P, S = (torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (p, s))
    rng = np.random.default_rng(65)
    NB = N // 128
    blocks = sorted({0, NB - 1, int(rng.integers(1, NB - 1))})
    cols = np.concatenate([np.arange(b * 128, (b + 1) * 128) for b in blocks])
    C = torch.from_numpy(cols).to(DEV)
    for M in (1, 8, 32, 64):
        print(f"w4a16 {name}: M={M} K={K} N={N}", flush=True)
        x = synth.activations(M, K, seed=66 + M, dtype=torch.float16).numpy()
        y64, y32 = int4.gemm_w4a16_group(x, p[cols], s[cols])
        got = _np(w8.gemm_w4a16_group(torch.from_numpy(x).to(DEV), P, S).index_select(1, C)).astype(np.float32)
        e32, e64 = gemm.normwise_rel_err(got, y32), gemm.normwise_rel_err(got, y64)
        assert e32 <= 1e-3 and e64 <= 1e-2, (M, e32, e64)

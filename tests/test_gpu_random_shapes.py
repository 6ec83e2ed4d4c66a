"""GPU parity of the GEMM entry points on seeded random shapes.

Beside the fixed shape lists of test_gpu_gemm, every GEMM entry point runs
on shapes drawn from a seeded generator: M from 1 to 700 (so every routing
decision is taken: decode kernels up to 64 rows, channel-wise decode to 128
rows, 128- and 256-row tiles, split over K or not, last tiles ragged inside
an 8-row load group), N from 1 to 1500 (ragged weight blocks and waves), K a
multiple of 128 up to 3072.  Bars as in test_gpu_gemm: channel-wise int32
and fp32 bit-exact, block-wise and grouped fp32 within 1e-5 normwise of the
oracle's fp32 path, W8A16 within 1e-3, bf16 the nearest-even rounding of
the fp32 result, and everything within 1e-2 of the oracle's fp64 path.
"""

import numpy as np
import pytest
import torch

import synth
import w8a8_int8_quantized_amd as w8
from oracle import formats, gemm, quant, routing

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _np(t):
    return t.detach().cpu().numpy()


def _dev(*arrs):
    return [torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in arrs]


def _shapes(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.choice([rng.integers(1, 65), rng.integers(65, 129), rng.integers(129, 701)]))
        N = int(rng.integers(1, 1501))
        K = 128 * int(rng.integers(1, 25))
        out.append((M, N, K))
    return out


@pytest.mark.parametrize("M,N,K", _shapes(101, 8))
def test_channel_random_shapes(M, N, K):
    print(f"channel M={M} N={N} K={K}", flush=True)
    qa, sa = quant.quant_act_token(synth.to_numpy(synth.activations(M, K, seed=M + 1)))
    qw, sw = quant.quant_act_token(synth.to_numpy(synth.weights(N, K, seed=N + 2)))
    ACC, y64, y32 = gemm.gemm_channel(qa, sa, qw, sw)
    A, SA, W, SW = _dev(qa, sa, qw, sw)
    assert np.array_equal(_np(w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=torch.int32)), ACC)
    yf = w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=torch.float32)
    assert np.array_equal(_np(yf).view(np.uint32), y32.view(np.uint32))
    yb = w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=torch.bfloat16)
    assert np.array_equal(_np(yb.view(torch.int16)).view(np.uint16), formats.f32_to_bf16_bits(y32))


@pytest.mark.parametrize("M,N,K", _shapes(202, 8))
def test_block_random_shapes(M, N, K):
    print(f"block M={M} N={N} K={K}", flush=True)
    qa, sa = quant.quant_act_group(synth.to_numpy(synth.activations(M, K, seed=M + 3)))
    qw, sw = quant.quant_weight_block(synth.to_numpy(synth.weights(N, K, seed=N + 4)))
    _, y64, y32 = gemm.gemm_block(qa, sa, qw, sw)
    A, SA, W, SW = _dev(qa, sa, qw, sw)
    yf = _np(w8.gemm_w8a8_block(A, SA, W, SW, out_dtype=torch.float32))
    e32, e64 = gemm.normwise_rel_err(yf, y32), gemm.normwise_rel_err(yf, y64)
    assert e32 <= 1e-5 and e64 <= 1e-2, (e32, e64)
    yb = w8.gemm_w8a8_block(A, SA, W, SW, out_dtype=torch.bfloat16)
    assert np.array_equal(_np(yb.view(torch.int16)).view(np.uint16), formats.f32_to_bf16_bits(yf))


@pytest.mark.parametrize("M,N,K", _shapes(303, 4))
def test_block_partials_random_shapes(M, N, K):
    qa, _ = quant.quant_act_group(synth.to_numpy(synth.activations(M, K, seed=M + 5)))
    qw, _ = quant.quant_weight_block(synth.to_numpy(synth.weights(N, K, seed=N + 6)))
    A, W = _dev(qa, qw)
    assert np.array_equal(_np(w8.gemm_w8a8_block_partials(A, W)), gemm.block_partials(qa, qw))


@pytest.mark.parametrize("M,N,K", [(m, n, k) for (m, n, k) in _shapes(404, 6)])
def test_w8a16_random_shapes(M, N, K):
    print(f"w8a16 M={M} N={N} K={K}", flush=True)
    x = synth.activations(M, K, seed=M + 7, dtype=torch.float16).numpy()
    qw, sw = quant.quant_act_group(synth.weights(N, K, seed=N + 8, dtype=torch.float16).numpy())
    y64, y32 = gemm.gemm_w8a16_group(x, qw, sw)
    X, W, SW = _dev(x, qw, sw)
    y = _np(w8.gemm_w8a16_group(X, W, SW)).astype(np.float32)
    e32, e64 = gemm.normwise_rel_err(y, y32), gemm.normwise_rel_err(y, y64)
    assert e32 <= 1e-3 and e64 <= 1e-2, (e32, e64)


@pytest.mark.parametrize("seed", [505, 606, 707, 808])
def test_grouped_random_shapes(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(1, 40))
    T = int(rng.integers(1, 1200))
    topk = int(rng.integers(1, min(E, 8) + 1))
    K = 128 * int(rng.integers(1, 13))
    N = int(rng.integers(1, 700))
    print(f"grouped E={E} T={T} topk={topk} K={K} N={N}", flush=True)
    rows, _, offs = routing.topk_route(synth.router_logits(T, E, seed=seed).numpy(), topk)
    x = synth.to_numpy(synth.activations(T, K, seed=seed + 1))
    qa, sa = quant.quant_act_group(x[rows])
    NB = (N + 127) // 128
    qw = np.empty((E, N, K), np.int8)
    sw = np.empty((E, NB, K // 128), np.float32)
    for e in range(E):
        qw[e], sw[e] = quant.quant_weight_block(synth.to_numpy(synth.weights(N, K, seed=seed + 10 + e)))
    y64, y32 = gemm.gemm_block_grouped(qa, sa, qw, sw, offs)
    A, SA, W, SW = _dev(qa, sa, qw, sw)
    OFF = torch.from_numpy(offs.astype(np.int32)).to(DEV)
    y = _np(w8.gemm_w8a8_block_grouped(A, SA, W, SW, OFF, out_dtype=torch.float32))
    for e in range(E):
        r0, r1 = offs[e], offs[e + 1]
        if r1 > r0:
            e32 = gemm.normwise_rel_err(y[r0:r1], y32[r0:r1])
            e64 = gemm.normwise_rel_err(y[r0:r1], y64[r0:r1])
            assert e32 <= 1e-5 and e64 <= 1e-2, (e, e32, e64)
    yb = w8.gemm_w8a8_block_grouped(A, SA, W, SW, OFF, out_dtype=torch.bfloat16)
    assert np.array_equal(_np(yb.view(torch.int16)).view(np.uint16), formats.f32_to_bf16_bits(y))

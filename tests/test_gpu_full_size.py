"""GPU parity of the large-M GEMMs at the benchmark's full sizes, on samples.

The DeepSeek-V3 dense MLP at 4096 tokens: gate_up (K = 7168 -> N = 36864)
and down (K = 18432 -> N = 7168), channel-wise (the headline step) and
block-wise (bf16 weights quantised per 128 x 128 block by the oracle; the
benchmark's block rows reach INT8 codes of the same shapes through the FP8
requantisation, whose plain oracle decode is too slow at this size for a
GPU test).  The GPU runs the whole GEMM through
the same entry points and output types as the benchmark, so the same kernels
and launch configuration; the oracle recomputes a sample: every output
depends only on its row of A (with that row's scales) and its row of W (with
its scales), so the oracle's GEMM over 64 sampled rows (the first and last
among them) times three whole 128-column weight blocks (the first, the last
and one drawn at random) equals that part of the full product.

Bars as in test_gpu_gemm: channel-wise int32 accumulator and fp32 output
bit-exact; block-wise fp32 within 1e-5 normwise of the oracle's fp32 path
(1e-2 of its fp64 path); bf16 outputs the round-to-nearest-even of the
oracle's (channel) or the kernel's own (block) fp32 values.
"""

import numpy as np
import pytest
import torch

import synth
import w8a8_int8_quantized_amd as w8
from oracle import formats, gemm, quant

pytestmark = pytest.mark.gpu
DEV = "cuda"
M = 4096
SHAPES = {"gate_up": (7168, 36864), "down": (18432, 7168)}


def _np(t):
    return t.detach().cpu().numpy()


def _sample(N, seed):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(np.arange(1, M - 1), 62, replace=False)]))
    NB = (N + 127) // 128
    blocks = np.array(sorted({0, NB - 1, int(rng.integers(1, NB - 1))}))
    cols = np.concatenate([np.arange(b * 128, min((b + 1) * 128, N)) for b in blocks])
    return rows, blocks, cols


def _pick(t, rows, cols):
    """The sampled submatrix of a device result, gathered on the device."""
    r = torch.from_numpy(rows).to(DEV)
    c = torch.from_numpy(cols).to(DEV)
    return _np(t.index_select(0, r).index_select(1, c))


@pytest.mark.parametrize("name", ["gate_up", "down"])
def test_channel_full_size_sampled(name):
    K, N = SHAPES[name]
    print(f"channel {name}: M={M} K={K} N={N}", flush=True)
    qa, sa = quant.quant_act_token(synth.to_numpy(synth.activations(M, K, seed=31)))
    qw, sw = quant.quant_act_token(synth.to_numpy(synth.weights(N, K, seed=32)))
    rows, _, cols = _sample(N, seed=33)
    ACC, y64, y32 = gemm.gemm_channel(qa[rows], sa[rows], qw[cols], sw[cols])
    A, SA, W, SW = (torch.from_numpy(a).to(DEV) for a in (qa, sa, qw, sw))
    del qw
    acc = w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=torch.int32)
    assert np.array_equal(_pick(acc, rows, cols), ACC)
    del acc
    yf = w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=torch.float32)
    assert np.array_equal(_pick(yf, rows, cols).view(np.uint32), y32.view(np.uint32))
    del yf
    yb = w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=torch.bfloat16)
    got = _pick(yb.view(torch.int16), rows, cols).view(np.uint16)
    assert np.array_equal(got, formats.f32_to_bf16_bits(y32))
    assert gemm.normwise_rel_err(formats.bf16_bits_to_f32(got).astype(np.float64), y64) <= 1e-2


@pytest.mark.parametrize("name", ["gate_up", "down"])
def test_block_full_size_sampled(name):
    K, N = SHAPES[name]
    print(f"block {name}: M={M} K={K} N={N}", flush=True)
    qa, sa = quant.quant_act_group(synth.to_numpy(synth.activations(M, K, seed=41)))
    qw, sw = quant.quant_weight_block(synth.to_numpy(synth.weights(N, K, seed=42)))
    rows, blocks, cols = _sample(N, seed=43)
    _, y64, y32 = gemm.gemm_block(qa[rows], sa[rows], qw[cols], sw[blocks])
    A, SA, W, SW = (torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (qa, sa, qw, sw))
    del qw
    yf = w8.gemm_w8a8_block(A, SA, W, SW, out_dtype=torch.float32)
    got32 = _pick(yf, rows, cols)
    del yf
    e32 = gemm.normwise_rel_err(got32, y32)
    e64 = gemm.normwise_rel_err(got32, y64)
    assert e32 <= 1e-5 and e64 <= 1e-2, (e32, e64)
    yb = w8.gemm_w8a8_block(A, SA, W, SW, out_dtype=torch.bfloat16)
    gotb = _pick(yb.view(torch.int16), rows, cols).view(np.uint16)
    assert np.array_equal(gotb, formats.f32_to_bf16_bits(got32))
    assert gemm.normwise_rel_err(formats.bf16_bits_to_f32(gotb).astype(np.float64), y64) <= 1e-2

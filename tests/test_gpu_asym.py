"""GPU parity of the asymmetric per-tensor path (page 2, dynamic range-aware
quantisation) against oracle/asym.py.

Bars: codes (stored as q - 128), the scale and the weight row sums
bit-exact; the zero point equal in value; the GEMM's fp32 output bit-exact
to the oracle's fixed-order fp32 evaluation, bf16 its nearest-even rounding,
both within 1e-2 of the fp64 evaluation.  Shapes cover one to many
workgroups of the two-pass range reduction, the decode (weight-streaming)
and tile GEMM routes with ragged N, and the benchmark's gate_up shape at
4096 rows (outputs sampled as in test_gpu_full_size).
"""

import json
import os

import numpy as np
import pytest
import torch

import synth
import w8a8_int8_quantized_amd as w8
from oracle import asym, formats, quant

pytestmark = pytest.mark.gpu
DEV = "cuda"
HERE = os.path.dirname(os.path.abspath(__file__))


def _np(t):
    return t.detach().cpu().numpy()


def _check_quant(x_cpu, fp16):
    xo = x_cpu.numpy() if fp16 else synth.to_numpy(x_cpu)
    q, s, z = asym.quant_act_asym(xo)
    codes, prm = w8.quant_act_asym(x_cpu.to(DEV))
    assert np.array_equal(_np(codes).view(np.uint8) ^ 0x80, q)
    p = _np(prm)
    assert p[0].view(np.uint32) == np.float32(s).view(np.uint32)
    assert p[1] == np.float32(z)
    return q, s, z


@pytest.mark.parametrize("fp16", [False, True])
@pytest.mark.parametrize("M,K", [(1, 128), (7, 384), (300, 1024), (2000, 7168)])
def test_quant_act_asym(M, K, fp16):
    print(f"asym quant M={M} K={K} fp16={fp16}", flush=True)
    x = synth.activations(M, K, seed=M + 3, dtype=torch.float16 if fp16 else torch.bfloat16)
    _check_quant(x, fp16)


def test_quant_act_asym_edges():
    g = json.load(open(os.path.join(HERE, "golden", "asym_ties.json")))
    vals = [c[0] for c in g["cases"]]
    row = torch.tensor([vals[i % len(vals)] for i in range(256)], dtype=torch.float32)
    q, s, _ = _check_quant(row.reshape(2, 128).to(torch.bfloat16), False)
    assert float(s) == g["scale"]
    for c in (0.0, 2.5, -7.0):
        q, _, _ = _check_quant(torch.full((3, 256), c, dtype=torch.bfloat16), False)
        assert not q.any()
    neg = -(1.0 + synth.activations(5, 128, seed=9).float().abs())
    _check_quant(neg.to(torch.bfloat16), False)
    codes = torch.empty(0, 128, dtype=torch.int8, device=DEV)
    prm = torch.full((2,), 7.0, device=DEV)
    w8.quant_act_asym(torch.empty(0, 128, dtype=torch.bfloat16, device=DEV), out=(codes, prm))
    assert _np(prm).tolist() == [7.0, 7.0]


@pytest.mark.parametrize("N,K", [(1, 128), (300, 256), (513, 7168)])
def test_weight_row_sums(N, K):
    qw, _ = quant.quant_act_token(synth.to_numpy(synth.weights(N, K, seed=N)))
    got = _np(w8.weight_row_sums(torch.from_numpy(qw).to(DEV)))
    assert np.array_equal(got.astype(np.int64), asym.weight_row_sums(qw))


def _gemm_inputs(M, N, K, seed):
    q, s, z = asym.quant_act_asym(synth.to_numpy(synth.activations(M, K, seed=seed)))
    qw, sw = quant.quant_act_token(synth.to_numpy(synth.weights(N, K, seed=seed + 1)))
    A = torch.from_numpy((q ^ 0x80).view(np.int8)).to(DEV)
    prm = torch.tensor([s, z], dtype=torch.float32, device=DEV)
    W, SW = (torch.from_numpy(a).to(DEV) for a in (qw, sw))
    WS = torch.from_numpy(asym.weight_row_sums(qw).astype(np.int32)).to(DEV)
    return (q, s, z, qw, sw), (A, prm, W, SW, WS)


# decode kernels (M <= 128), split-K tiles, and unsplit tile grids whose
# epilogue runs inside the tile kernel (1024 x 36864, 520 x 9000: ragged)
@pytest.mark.parametrize("M,N,K", [(1, 300, 256), (37, 700, 1024), (64, 36864, 256), (100, 12288, 384),
                                   (130, 513, 640), (300, 1100, 384), (1024, 36864, 256), (520, 9000, 384)])
def test_gemm_asym(M, N, K):
    print(f"asym gemm M={M} N={N} K={K}", flush=True)
    (q, s, z, qw, sw), (A, prm, W, SW, WS) = _gemm_inputs(M, N, K, seed=M + N)
    _, _, y64, y32 = asym.gemm_asym(q, s, z, qw, sw)
    yf = _np(w8.gemm_w8a8_asym(A, prm, W, SW, WS, out_dtype=torch.float32))
    assert np.array_equal(yf.view(np.uint32), y32.view(np.uint32))
    yb = w8.gemm_w8a8_asym(A, prm, W, SW, WS)
    gb = _np(yb.view(torch.int16)).view(np.uint16)
    assert np.array_equal(gb, formats.f32_to_bf16_bits(y32))
    err = np.abs(formats.bf16_bits_to_f32(gb).astype(np.float64) - y64).max() / np.abs(y64).max()
    assert err <= 1e-2


def test_gemm_asym_full_size_sampled():
    """gate_up at 4096 rows (K = 7168 -> N = 36864): the whole quantiser and
    GEMM on the GPU, the oracle on 64 sampled rows x 3 column blocks."""
    M, K, N = 4096, 7168, 36864
    x = synth.activations(M, K, seed=81)
    q, s, z = asym.quant_act_asym(synth.to_numpy(x))
    codes, prm = w8.quant_act_asym(x.to(DEV))
    assert np.array_equal(_np(codes).view(np.uint8) ^ 0x80, q)
    qw, sw = quant.quant_act_token(synth.to_numpy(synth.weights(N, K, seed=82)))
    W, SW = (torch.from_numpy(a).to(DEV) for a in (qw, sw))
    WS = w8.weight_row_sums(W)
    y = w8.gemm_w8a8_asym(codes, prm, W, SW, WS, out_dtype=torch.float32)
    rng = np.random.default_rng(83)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(np.arange(1, M - 1), 62, replace=False)]))
    blocks = [0, int(rng.integers(1, N // 128 - 1)), N // 128 - 1]
    cols = np.concatenate([np.arange(b * 128, (b + 1) * 128) for b in blocks])
    _, _, y64, y32 = asym.gemm_asym(q[rows], s, z, qw[cols], sw[cols])
    got = _np(y.index_select(0, torch.from_numpy(rows).to(DEV)).index_select(1, torch.from_numpy(cols).to(DEV)))
    assert np.array_equal(got.view(np.uint32), y32.view(np.uint32))


def test_gemm_asym_max_k_extreme_codes():
    """K = 2^16, the limit: every code 255 but one 0 per row and every weight
    code 127, so ACC = 255 * 127 * (K - 1) = 2.12e9 sits just inside int32
    (and the stored codes' sum 127 * 127 * (K - 1) plus 128 WS as well)."""
    M, N, K = 2, 3, 1 << 16
    x = torch.ones(M, K, dtype=torch.bfloat16)
    x[:, 0] = -1.0
    q, s, z = asym.quant_act_asym(synth.to_numpy(x))
    assert q[:, 1:].min() == 255 and q[:, 0].max() == 0
    qw, sw = quant.quant_act_token(synth.to_numpy(torch.full((N, K), 0.02, dtype=torch.bfloat16)))
    assert (qw == 127).all()
    ACC, _, y64, y32 = asym.gemm_asym(q, s, z, qw, sw)
    assert ACC.max() == 255 * 127 * (K - 1) < 2 ** 31
    codes, prm = w8.quant_act_asym(x.to(DEV))
    assert np.array_equal(_np(codes).view(np.uint8) ^ 0x80, q)
    W, SW = (torch.from_numpy(a).to(DEV) for a in (qw, sw))
    got = _np(w8.gemm_w8a8_asym(codes, prm, W, SW, w8.weight_row_sums(W), out_dtype=torch.float32))
    assert np.array_equal(got.view(np.uint32), y32.view(np.uint32))

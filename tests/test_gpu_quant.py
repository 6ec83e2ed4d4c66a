"""GPU parity of the quantisation kernels against the CPU oracle: int8 codes
and fp32 scales must be bit-exact (same inputs, seeded)."""

import json
import os

import numpy as np
import pytest
import torch

import synth
import w8a8_int8_quantized_amd as w8
from oracle import formats, quant

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))
DEV = "cuda"


def _eq(gpu, ref, what):
    g = gpu.detach().cpu().numpy()
    if g.dtype == np.float32:
        ok = np.array_equal(g.view(np.uint32), np.asarray(ref, np.float32).view(np.uint32))
    else:
        ok = np.array_equal(g, ref)
    if not ok:
        diff = np.argwhere(g != ref)
        raise AssertionError(f"{what}: {len(diff)} mismatches, first at {diff[:5].tolist()}")


@pytest.mark.parametrize("M,K", [(16, 256), (1, 128), (300, 7168), (37, 18432)])
def test_quant_act_group_bf16(M, K):
    x = synth.activations(M, K, seed=M + K, outlier_frac=0.005, outlier_factor=30.0)
    q, s = w8.quant_act_group(x.to(DEV))
    rq, rs = quant.quant_act_group(synth.to_numpy(x))
    _eq(q, rq, "q")
    _eq(s, rs, "scale")


@pytest.mark.parametrize("M,K", [(64, 4096), (5, 12288)])
def test_quant_act_group_fp16(M, K):
    x = synth.activations(M, K, seed=3, dtype=torch.float16)
    q, s = w8.quant_act_group(x.to(DEV))
    rq, rs = quant.quant_act_group(x.numpy())
    _eq(q, rq, "q")
    _eq(s, rs, "scale")


def test_quant_ties_zero_groups_and_extremes():
    with open(os.path.join(HERE, "golden", "quant_ties.json")) as f:
        g = json.load(f)
    rows = []
    for case in g["cases"]:
        v = np.zeros(128, np.float32)
        v[: len(case["values"])] = case["values"]
        rows.append(v)
    rows.append(np.zeros(128, np.float32))                              # all-zero group
    rows.append(np.full(128, 3.0e38, np.float32))                       # largest magnitudes
    rows.append(np.full(128, 1e-38, np.float32))                        # tiny values (below eps)
    v = np.zeros(128, np.float32)
    v[::2] = -2.5
    rows.append(v)
    x = formats.f32_to_bf16_bits(np.stack(rows))
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(DEV)
    for fn, ofn in ((w8.quant_act_group, quant.quant_act_group), (w8.quant_act_token, quant.quant_act_token)):
        q, s = fn(xt)
        rq, rs = ofn(x)
        _eq(q, rq, "q")
        _eq(s, rs, "scale")
    q, _ = w8.quant_act_group(xt)
    for i, case in enumerate(g["cases"]):
        assert q[i, : len(case["q"])].cpu().tolist() == case["q"]


@pytest.mark.parametrize("M,K", [(4, 128), (33, 7168), (7, 18432), (3, 131072)])
def test_quant_act_token_bf16(M, K):
    x = synth.activations(M, K, seed=K, outlier_frac=0.005, outlier_factor=30.0)
    q, s = w8.quant_act_token(x.to(DEV))
    rq, rs = quant.quant_act_token(synth.to_numpy(x))
    _eq(q, rq, "q")
    _eq(s, rs, "scale")


def test_quant_act_token_fp16_and_channel_weights():
    x = synth.activations(9, 4096, seed=4, dtype=torch.float16)
    q, s = w8.quant_act_token(x.to(DEV))
    rq, rs = quant.quant_act_token(x.numpy())
    _eq(q, rq, "q")
    _eq(s, rs, "scale")
    w = synth.weights(1000, 1024, seed=5)
    q, s = w8.quant_weight_channel(w.to(DEV))
    rq, rs = quant.quant_act_token(synth.to_numpy(w))
    _eq(q, rq, "q")
    _eq(s, rs, "scale")


@pytest.mark.parametrize("N,K", [(256, 256), (576, 1024), (200, 384), (1, 128)])
def test_quant_weight_block(N, K):
    w = synth.weights(N, K, seed=N)
    q, s = w8.quant_weight_block(w.to(DEV))
    rq, rs = quant.quant_weight_block(synth.to_numpy(w))
    _eq(q, rq, "q")
    _eq(s, rs, "scale")


def test_requant_all_fp8_codes():
    codes = np.arange(256, dtype=np.uint8)
    finite = codes[~np.isnan(formats.e4m3fn_to_f32(codes))]             # NaN codes are out of contract
    rng = np.random.default_rng(0)
    N, K = 256, 512
    w = finite[rng.integers(0, finite.size, (N, K))]
    w[0, :254] = finite                                                   # every finite code once in tile (0, 0)
    si = np.exp(rng.uniform(np.log(1e-4), np.log(1e-2), (2, 4))).astype(np.float32)
    si[1, 3] = 1.0
    wt = torch.from_numpy(w).to(DEV)
    st = torch.from_numpy(si).to(DEV)
    q, s, wb = w8.requant_fp8_to_int8_block(wt, st, return_bf16=True)
    rq, rs, rwb = quant.requant_fp8_to_int8_block(w, si)
    _eq(wb.view(torch.int16), rwb.view(np.int16), "bf16")
    _eq(q, rq, "q")
    _eq(s, rs, "scale")


@pytest.mark.parametrize("N,K", [(576, 7168), (300, 256)])
def test_requant_synthetic_fp8_weights(N, K):
    codes, si = synth.fp8_weights(N, K, seed=2)
    q, s = w8.requant_fp8_to_int8_block(codes.to(DEV), si.to(DEV))
    rq, rs, _ = quant.requant_fp8_to_int8_block(codes.numpy(), si.numpy())
    _eq(q, rq, "q")
    _eq(s, rs, "scale")
    qc, sc = w8.requant_fp8_to_int8_channel(codes.to(DEV), si.to(DEV))
    rqc, rsc, _ = quant.requant_fp8_to_int8_channel(codes.numpy(), si.numpy())
    _eq(qc, rqc, "q channel")
    _eq(sc, rsc, "scale channel")


def test_quantisers_are_deterministic():
    x = synth.activations(128, 7168, seed=11).to(DEV)
    a = w8.quant_act_group(x)
    b = w8.quant_act_group(x)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_empty_inputs_are_noops():
    x = torch.empty(0, 256, dtype=torch.bfloat16, device=DEV)
    q, s = w8.quant_act_group(x)
    assert q.shape == (0, 256) and s.shape == (0, 2)
    q, s = w8.quant_act_token(x)
    assert q.shape == (0, 256) and s.shape == (0,)

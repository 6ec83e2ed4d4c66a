"""GPU parity of the GEMMs at the benchmark's full sizes, on samples.

The DeepSeek-V3 dense MLP at 4096 tokens: gate_up (K = 7168 -> N = 36864)
and down (K = 18432 -> N = 7168), channel-wise (the headline step) and
block-wise (bf16 weights quantised per 128 x 128 block by the oracle; the
benchmark's block rows reach INT8 codes of the same shapes through the FP8
requantisation, checked below on sampled 128 x 128 tiles of the full-size
conversion: every tile depends only on its own codes and scale_inv).  The
GPU runs the whole GEMM through
the same entry points and output types as the benchmark, so the same kernels
and launch configuration; the oracle recomputes a sample: every output
depends only on its row of A (with that row's scales) and its row of W (with
its scales), so the oracle's GEMM over 64 sampled rows (the first and last
among them) times three whole 128-column weight blocks (the first, the last
and one drawn at random) equals that part of the full product.

The decode, W8A16 and MoE rows follow below with the same sampling.

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
from oracle import formats, gemm, quant, routing

pytestmark = pytest.mark.gpu
DEV = "cuda"
M = 4096
SHAPES = {"gate_up": (7168, 36864), "down": (18432, 7168)}


def _np(t):
    return t.detach().cpu().numpy()


def _sample(N, seed, M=M):
    rng = np.random.default_rng(seed)
    if M <= 64:
        rows = np.arange(M)
    else:
        rows = np.unique(np.concatenate([[0, M - 1], rng.choice(np.arange(1, M - 1), 62, replace=False)]))
    NB = (N + 127) // 128
    blocks = np.array(sorted({0, NB - 1, int(rng.integers(1, NB - 1))}))
    cols = np.concatenate([np.arange(b * 128, min((b + 1) * 128, N)) for b in blocks])
    return rows, blocks, cols


_CHANNEL_CACHE = {}


def _channel_operands(name):
    """Oracle-quantised channel-wise operands of one DeepSeek-V3 MLP shape
    (activations for all 4096 tokens; smaller M use the leading rows)."""
    if name not in _CHANNEL_CACHE:
        K, N = SHAPES[name]
        qa, sa = quant.quant_act_token(synth.to_numpy(synth.activations(M, K, seed=31)))
        qw, sw = quant.quant_act_token(synth.to_numpy(synth.weights(N, K, seed=32)))
        _CHANNEL_CACHE.clear()
        _CHANNEL_CACHE[name] = (qa, sa, qw, sw)
    return _CHANNEL_CACHE[name]


def _pick(t, rows, cols):
    """The sampled submatrix of a device result, gathered on the device."""
    r = torch.from_numpy(rows).to(DEV)
    c = torch.from_numpy(cols).to(DEV)
    return _np(t.index_select(0, r).index_select(1, c))


# The channel-wise rows of the benchmark: 128 tokens (the weight-streaming
# decode kernel for gate_up, K split over tiles for down), 1024 and 4096
# tokens (the tile kernel, split over K where the grid is small).
@pytest.mark.parametrize("Mr", [128, 1024, 4096])
@pytest.mark.parametrize("name", ["gate_up", "down"])
def test_channel_full_size_sampled(name, Mr):
    K, N = SHAPES[name]
    print(f"channel {name}: M={Mr} K={K} N={N}", flush=True)
    qa, sa, qw, sw = _channel_operands(name)
    qa, sa = np.ascontiguousarray(qa[:Mr]), np.ascontiguousarray(sa[:Mr])
    rows, _, cols = _sample(N, seed=33 + Mr, M=Mr)
    ACC, y64, y32 = gemm.gemm_channel(qa[rows], sa[rows], qw[cols], sw[cols])
    A, SA, W, SW = (torch.from_numpy(a).to(DEV) for a in (qa, sa, qw, sw))
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


# The attention projections of the block-wise configuration at 4096 tokens:
# q_a (K = 7168 -> N = 1536), q_b (1536 -> 24576) and kv_a (7168 -> 576, whose
# last 128-row weight tile holds 64 rows), with the weights taken as the
# benchmark takes them: FP8-E4M3FN codes and per-tile scale_inv drawn on the
# GPU, requantised to INT8 tiles by the library.  The oracle requantises the
# sampled column blocks' weight rows from the same codes (bit-exact against
# the library's codes and scales) and computes the sampled outputs from them.
@pytest.mark.parametrize("name", ["q_a", "q_b", "kv_a"])
def test_block_attention_full_size_sampled(name):
    K, N = synth.SHAPES[name]
    print(f"block {name}: M={M} K={K} N={N} (FP8 weights requantised)", flush=True)
    codes, si = synth.fp8_weights(N, K, seed=synth.SEEDS["block"], device=DEV)
    wq, ws = w8.requant_fp8_to_int8_block(codes, si)
    rows, blocks, cols = _sample(N, seed=44 + N)
    oq, osc, _ = quant.requant_fp8_to_int8_block(_np(codes[torch.from_numpy(cols).to(DEV)]),
                                                 _np(si[torch.from_numpy(blocks).to(DEV)]))
    del codes
    assert np.array_equal(_np(wq[torch.from_numpy(cols).to(DEV)]), oq)
    assert np.array_equal(_np(ws[torch.from_numpy(blocks).to(DEV)]).view(np.uint32), osc.view(np.uint32))
    qa, sa = quant.quant_act_group(synth.to_numpy(synth.activations(M, K, seed=45)))
    _, y64, y32 = gemm.gemm_block(qa[rows], sa[rows], oq, osc)
    A, SA = (torch.from_numpy(a).to(DEV) for a in (qa, sa))
    yf = w8.gemm_w8a8_block(A, SA, wq, ws, out_dtype=torch.float32)
    got32 = _pick(yf, rows, cols)
    del yf
    e32, e64 = gemm.normwise_rel_err(got32, y32), gemm.normwise_rel_err(got32, y64)
    assert e32 <= 1e-5 and e64 <= 1e-2, (e32, e64)
    yb = w8.gemm_w8a8_block(A, SA, wq, ws, out_dtype=torch.bfloat16)
    gotb = _pick(yb.view(torch.int16), rows, cols).view(np.uint16)
    assert np.array_equal(gotb, formats.f32_to_bf16_bits(got32))


# FP8 -> BF16 -> INT8 conversion of the whole gate_up weight (36864 x 7168,
# the benchmark's requantisation row, inputs drawn on the GPU as the
# benchmark draws them); the oracle converts four sampled tiles (the first,
# the last and two at random) from the same codes and scale_inv.
def test_requant_fp8_full_size_sampled():
    K, N = SHAPES["gate_up"]
    NB, KB = N // 128, K // 128
    print(f"requant fp8: N={N} K={K}", flush=True)
    codes, si = synth.fp8_weights(N, K, seed=synth.SEEDS["block"], device=DEV)
    q, sc, wb = w8.requant_fp8_to_int8_block(codes, si, return_bf16=True)
    rng = np.random.default_rng(91)
    tiles = sorted({(0, 0), (NB - 1, KB - 1), (int(rng.integers(NB)), int(rng.integers(KB))),
                    (int(rng.integers(NB)), int(rng.integers(KB)))})
    for nb, kb in tiles:
        r, c = slice(nb * 128, (nb + 1) * 128), slice(kb * 128, (kb + 1) * 128)
        oq, osc, owb = quant.requant_fp8_to_int8_block(_np(codes[r, c]), _np(si[nb:nb + 1, kb:kb + 1]))
        assert np.array_equal(_np(q[r, c]), oq), (nb, kb)
        assert _np(sc[nb:nb + 1, kb:kb + 1]).view(np.uint32)[0, 0] == osc.view(np.uint32)[0, 0], (nb, kb)
        assert np.array_equal(_np(wb[r, c].contiguous().view(torch.int16)).view(np.uint16), owb), (nb, kb)


# ------------------------------------------------------------ decode shapes
# Block-wise decode at the benchmark's decode rows (K = 7168 -> N = 36864,
# M in {1, 8, 32, 64}: one weight-streaming launch per M), every row checked
# on three whole 128-column blocks.
def test_block_decode_full_size_sampled():
    K, N = SHAPES["gate_up"]
    qw, sw = quant.quant_weight_block(synth.to_numpy(synth.weights(N, K, seed=52)))
    _, blocks, cols = _sample(N, seed=53)
    W, SW = (torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (qw, sw))
    qwc, swb = qw[cols], sw[blocks]
    del qw
    for M in (1, 8, 32, 64):
        print(f"block decode: M={M} K={K} N={N}", flush=True)
        qa, sa = quant.quant_act_group(synth.to_numpy(synth.activations(M, K, seed=50 + M)))
        _, y64, y32 = gemm.gemm_block(qa, sa, qwc, swb)
        A, SA = (torch.from_numpy(a).to(DEV) for a in (qa, sa))
        rows = np.arange(M)
        got32 = _pick(w8.gemm_w8a8_block(A, SA, W, SW, out_dtype=torch.float32), rows, cols)
        e32, e64 = gemm.normwise_rel_err(got32, y32), gemm.normwise_rel_err(got32, y64)
        assert e32 <= 1e-5 and e64 <= 1e-2, (M, e32, e64)
        gotb = _pick(w8.gemm_w8a8_block(A, SA, W, SW, out_dtype=torch.bfloat16).view(torch.int16), rows, cols)
        assert np.array_equal(gotb.view(np.uint16), formats.f32_to_bf16_bits(got32))


# W8A16 at the benchmark's Qwen3-8B-shaped rows (qkv K = 4096 -> N = 12288,
# down K = 12288 -> N = 4096; fp16 activations, group-wise INT8 weights).
@pytest.mark.parametrize("name,K,N", [("qkv", 4096, 12288), ("down", 12288, 4096)])
def test_w8a16_full_size_sampled(name, K, N):
    qw, sw = quant.quant_act_group(synth.weights(N, K, seed=62, dtype=torch.float16).numpy())
    _, _, cols = _sample(N, seed=63)
    W, SW = (torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (qw, sw))
    qwc, swc = qw[cols], sw[cols]
    for M in (1, 8, 32, 64):
        print(f"w8a16 {name}: M={M} K={K} N={N}", flush=True)
        x = synth.activations(M, K, seed=60 + M, dtype=torch.float16).numpy()
        y64, y32 = gemm.gemm_w8a16_group(x, qwc, swc)
        got = _pick(w8.gemm_w8a16_group(torch.from_numpy(x).to(DEV), W, SW), np.arange(M), cols).astype(np.float32)
        e32, e64 = gemm.normwise_rel_err(got, y32), gemm.normwise_rel_err(got, y64)
        assert e32 <= 1e-3 and e64 <= 1e-2, (M, e32, e64)


# ---------------------------------------------------------------------- MoE
# The benchmark's MoE gate_up: 256 experts, top-8 routing of 4096 tokens
# (32768 expert-sorted rows, 128 per expert on average), K = 7168 -> N = 4096
# per expert, 7.5 GB of expert weights.  Four experts are checked (the first,
# the last, the one with the most rows and the one with the fewest non-zero
# rows), on three whole 128-column blocks: their weights and every
# activation row come from the oracle's quantisers; the other experts'
# weights are arbitrary INT8 codes (torch's generator), which no checked
# output depends on.
def test_moe_full_size_sampled():
    E, T, TOPK = 256, 4096, 8
    K, N = 7168, 4096
    NB, KB = N // 128, K // 128
    rows, _, offs = routing.topk_route(synth.router_logits(T, E, seed=4).numpy(), TOPK)
    P = rows.size
    x = synth.to_numpy(synth.activations(T, K, seed=71))
    qa, sa = quant.quant_act_group(x[rows])
    del x
    cnt = np.diff(offs)
    nz = np.nonzero(cnt)[0]
    experts = sorted({0, E - 1, int(np.argmax(cnt)), int(nz[np.argmin(cnt[nz])])})
    print(f"moe: E={E} P={P} K={K} N={N} experts {experts} rows {[int(cnt[e]) for e in experts]}", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(72)
    Wq = torch.empty(E, N, K, dtype=torch.int8, device=DEV)
    for e0 in range(0, E, 16):
        Wq[e0:e0 + 16] = torch.randint(-127, 128, (16, N, K), generator=g, dtype=torch.int8, device=DEV)
    Ws = torch.rand(E, NB, KB, generator=g, device=DEV) * 1e-3 + 1e-4
    ref = {}
    for e in experts:
        qw, sw = quant.quant_weight_block(synth.to_numpy(synth.weights(N, K, seed=200 + e)))
        Wq[e] = torch.from_numpy(qw).to(DEV)
        Ws[e] = torch.from_numpy(sw).to(DEV)
        ref[e] = (qw, sw)
    _, blocks, cols = _sample(N, seed=73)
    A, SA = (torch.from_numpy(a).to(DEV) for a in (qa, sa))
    OFF = torch.from_numpy(offs.astype(np.int32)).to(DEV)
    y = w8.gemm_w8a8_block_grouped(A, SA, Wq, Ws, OFF, out_dtype=torch.float32)
    yb = w8.gemm_w8a8_block_grouped(A, SA, Wq, Ws, OFF, out_dtype=torch.bfloat16)
    for e in experts:
        r = np.arange(offs[e], offs[e + 1])
        qw, sw = ref[e]
        _, y64, y32 = gemm.gemm_block(qa[r], sa[r], qw[cols], sw[blocks])
        got32 = _pick(y, r, cols)
        e32, e64 = gemm.normwise_rel_err(got32, y32), gemm.normwise_rel_err(got32, y64)
        assert e32 <= 1e-5 and e64 <= 1e-2, (e, e32, e64)
        assert np.array_equal(_pick(yb.view(torch.int16), r, cols).view(np.uint16), formats.f32_to_bf16_bits(got32))


# The benchmark's MoE down projection: K = 2048 -> N = 7168 per expert over
# the same 32768 routed rows (synthetic inputs in place of the SiLU-and-
# multiply output), the rows of four experts on three whole column blocks.
def test_moe_down_full_size_sampled():
    E, T, TOPK = 256, 4096, 8
    K, N = 2048, 7168
    NB, KB = N // 128, K // 128
    _, _, offs = routing.topk_route(synth.router_logits(T, E, seed=4).numpy(), TOPK)
    P = int(offs[-1])
    qa, sa = quant.quant_act_group(synth.to_numpy(synth.activations(P, K, seed=81)))
    cnt = np.diff(offs)
    nz = np.nonzero(cnt)[0]
    experts = sorted({0, E - 1, int(np.argmax(cnt)), int(nz[np.argmin(cnt[nz])])})
    print(f"moe down: E={E} P={P} K={K} N={N} experts {experts} rows {[int(cnt[e]) for e in experts]}", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(82)
    Wq = torch.empty(E, N, K, dtype=torch.int8, device=DEV)
    for e0 in range(0, E, 32):
        Wq[e0:e0 + 32] = torch.randint(-127, 128, (32, N, K), generator=g, dtype=torch.int8, device=DEV)
    Ws = torch.rand(E, NB, KB, generator=g, device=DEV) * 1e-3 + 1e-4
    ref = {}
    for e in experts:
        qw, sw = quant.quant_weight_block(synth.to_numpy(synth.weights(N, K, seed=300 + e)))
        Wq[e] = torch.from_numpy(qw).to(DEV)
        Ws[e] = torch.from_numpy(sw).to(DEV)
        ref[e] = (qw, sw)
    _, blocks, cols = _sample(N, seed=83)
    A, SA = (torch.from_numpy(a).to(DEV) for a in (qa, sa))
    OFF = torch.from_numpy(offs.astype(np.int32)).to(DEV)
    y = w8.gemm_w8a8_block_grouped(A, SA, Wq, Ws, OFF, out_dtype=torch.float32)
    yb = w8.gemm_w8a8_block_grouped(A, SA, Wq, Ws, OFF, out_dtype=torch.bfloat16)
    for e in experts:
        r = np.arange(offs[e], offs[e + 1])
        qw, sw = ref[e]
        _, y64, y32 = gemm.gemm_block(qa[r], sa[r], qw[cols], sw[blocks])
        got32 = _pick(y, r, cols)
        e32, e64 = gemm.normwise_rel_err(got32, y32), gemm.normwise_rel_err(got32, y64)
        assert e32 <= 1e-5 and e64 <= 1e-2, (e, e32, e64)
        assert np.array_equal(_pick(yb.view(torch.int16), r, cols).view(np.uint16), formats.f32_to_bf16_bits(got32))

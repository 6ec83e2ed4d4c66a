"""GPU parity of the block-wise GEMMs with the next layer's group quantiser
fused into the epilogue (gemm_w8a8_block_quant, gemm_w8a8_block_grouped_quant).

Page 1 section 2.3 quantises activations online per 1 x 128 token-group
before every block-wise INT8 matmul; the fused calls quantise a GEMM's bf16
output where it is produced.  Their definition is the composition
quant_act_group(bf16 GEMM output), so:
  * codes and scales are bit-identical to gemm_w8a8_block (bf16) followed by
    quant_act_group on the GPU, over the whole output;
  * they equal the oracle's quant_act_group applied to that bf16 output
    (bit-exact), and the bf16 output itself is within the block GEMM's bars
    of the oracle;
  * the paths covered: the unsplit 256-row and 128-row tile epilogues, the
    split-K reduction, decode-sized M (tile kernels), the grouped MoE
    epilogue (128- and 256-row expert tiles, empty experts).
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


def _block_operands(M, N, K, seed):
    qa, sa = quant.quant_act_group(synth.to_numpy(synth.activations(M, K, seed=seed)))
    qw, sw = quant.quant_weight_block(synth.to_numpy(synth.weights(N, K, seed=seed + 1)))
    return qa, sa, qw, sw


def _check_against_composition(q, s, ybf16, rows=None):
    """Fused (q, s) == quant_act_group of the bf16 GEMM output, on the GPU and
    by the oracle (on `rows` when given)."""
    q2, s2 = w8.quant_act_group(ybf16)
    assert torch.equal(q, q2)
    assert torch.equal(s.view(torch.int32), s2.view(torch.int32))
    ybits = _np(ybf16.view(torch.int16)).view(np.uint16)
    qn, sn = _np(q), _np(s)
    if rows is not None:
        ybits, qn, sn = ybits[rows], qn[rows], sn[rows]
    oq, os_ = quant.quant_act_group(ybits)
    assert np.array_equal(qn, oq)
    assert np.array_equal(sn.view(np.uint32), os_.view(np.uint32))


# (M, N, K): a 2048 x 8192 grid of 256-row tiles runs unsplit; 1500 x 5120
# takes 128 x 256 tiles unsplit (the quantising epilogue) and 513 x 384 split
# over K (slices quantised in the sum); 300 x 1024 is where gemm_w8a8_block
# takes the K-parity 128 x 192 tiles, split over K, whose fp32 slices the
# quantising call sums; 1, 24 and 64 rows are decode-sized.
@pytest.mark.parametrize("M,N,K", [(2048, 8192, 1024), (1500, 5120, 256), (300, 1024, 1024), (24, 1536, 2048),
                                   (1, 4096, 1024), (64, 12288, 4096), (513, 384, 640)])
def test_block_quant_equals_gemm_then_group_quant(M, N, K):
    qa, sa, qw, sw = _block_operands(M, N, K, seed=M + N)
    A, SA, W, SW = (torch.from_numpy(a).to(DEV) for a in (qa, sa, qw, sw))
    q, s = w8.gemm_w8a8_block_quant(A, SA, W, SW)
    y = w8.gemm_w8a8_block(A, SA, W, SW, out_dtype=torch.bfloat16)
    rows = None if M * N <= 4 * 1024 * 1024 else np.unique(np.r_[0, M - 1, np.arange(1, M - 1, 61)])
    _check_against_composition(q, s, y, rows)
    # the bf16 output behind the codes is within the block GEMM's bar
    if M * N <= 4 * 1024 * 1024:
        _, y64, _ = gemm.gemm_block(qa, sa, qw, sw)
        got = formats.bf16_bits_to_f32(_np(y.view(torch.int16)).view(np.uint16)).astype(np.float64)
        assert gemm.normwise_rel_err(got, y64) <= 1e-2
        # and the codes dequantise to it within half a scale step
        deq = _np(q).astype(np.float64) * np.repeat(_np(s).astype(np.float64), 128, axis=1)
        assert np.all(np.abs(deq - got) <= np.repeat(_np(s).astype(np.float64), 128, axis=1) * 0.5 * (1 + 2.0 ** -16))


def test_block_quant_full_size_gate_up():
    """The DeepSeek-V3 gate_up projection at 4096 tokens (K = 7168 ->
    N = 36864): fused codes and scales equal the composition over the whole
    output; the oracle checks 64 sampled rows."""
    M, K, N = 4096, 7168, 36864
    print(f"fused block quant gate_up M={M} K={K} N={N}", flush=True)
    A, SA = w8.quant_act_group(synth.activations(M, K, seed=41, device=DEV))
    W, SW = w8.quant_weight_block(synth.weights(N, K, seed=42, device=DEV))
    q, s = w8.gemm_w8a8_block_quant(A, SA, W, SW)
    y = w8.gemm_w8a8_block(A, SA, W, SW, out_dtype=torch.bfloat16)
    rng = np.random.default_rng(5)
    rows = np.unique(np.r_[0, M - 1, rng.choice(np.arange(1, M - 1), 62, replace=False)])
    q2, s2 = w8.quant_act_group(y)
    assert torch.equal(q, q2) and torch.equal(s.view(torch.int32), s2.view(torch.int32))
    r = torch.from_numpy(rows).to(DEV)
    oq, os_ = quant.quant_act_group(_np(y.index_select(0, r).view(torch.int16)).view(np.uint16))
    assert np.array_equal(_np(q.index_select(0, r)), oq)
    assert np.array_equal(_np(s.index_select(0, r)).view(np.uint32), os_.view(np.uint32))


@pytest.mark.parametrize("E,T,topk,N,K", [(8, 300, 2, 512, 640), (16, 1024, 8, 1024, 512)])
def test_grouped_quant_equals_grouped_gemm_then_group_quant(E, T, topk, N, K):
    logits = synth.router_logits(T, E, seed=E + T).numpy()
    rows, _, offs = routing.topk_route(logits, topk)
    P = rows.size
    qa, sa = quant.quant_act_group(synth.to_numpy(synth.activations(P, K, seed=E)))
    ws = [quant.quant_weight_block(synth.to_numpy(synth.weights(N, K, seed=100 + e))) for e in range(E)]
    Wq = np.stack([w for w, _ in ws])
    Ws = np.stack([s for _, s in ws])
    A, SA, W, SW = (torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (qa, sa, Wq, Ws))
    OFF = torch.from_numpy(offs.astype(np.int32)).to(DEV)
    q, s = w8.gemm_w8a8_block_grouped_quant(A, SA, W, SW, OFF)
    y = w8.gemm_w8a8_block_grouped(A, SA, W, SW, OFF, out_dtype=torch.bfloat16)
    _check_against_composition(q, s, y)


def test_grouped_quant_moe_gate_up_full_size():
    """The benchmark's MoE gate_up (256 experts, top-8 of 4096 tokens, K = 7168
    -> N = 4096 per expert): fused codes and scales equal the composition
    over all 32768 routed rows."""
    E, T, TOPK, K, N = 256, 4096, 8, 7168, 4096
    _, _, offs = routing.topk_route(synth.router_logits(T, E, seed=4).numpy(), TOPK)
    P = int(offs[-1])
    print(f"fused grouped quant E={E} P={P} K={K} N={N}", flush=True)
    A, SA = w8.quant_act_group(synth.activations(P, K, seed=91, device=DEV))
    g = torch.Generator(device=DEV)
    g.manual_seed(92)
    W = torch.empty(E, N, K, dtype=torch.int8, device=DEV)
    for e0 in range(0, E, 32):
        W[e0:e0 + 32] = torch.randint(-127, 128, (32, N, K), generator=g, dtype=torch.int8, device=DEV)
    SW = torch.rand(E, N // 128, K // 128, generator=g, device=DEV) * 1e-3 + 1e-4
    OFF = torch.from_numpy(offs.astype(np.int32)).to(DEV)
    q, s = w8.gemm_w8a8_block_grouped_quant(A, SA, W, SW, OFF)
    y = w8.gemm_w8a8_block_grouped(A, SA, W, SW, OFF, out_dtype=torch.bfloat16)
    q2, s2 = w8.quant_act_group(y)
    assert torch.equal(q, q2) and torch.equal(s.view(torch.int32), s2.view(torch.int32))


def test_block_quant_rejects_partial_groups_and_allows_empty():
    A = torch.zeros(4, 128, dtype=torch.int8, device=DEV)
    SA = torch.ones(4, 1, dtype=torch.float32, device=DEV)
    W = torch.zeros(200, 128, dtype=torch.int8, device=DEV)
    SW = torch.ones(2, 1, dtype=torch.float32, device=DEV)
    with pytest.raises(w8.W8Error):
        w8.gemm_w8a8_block_quant(A, SA, W, SW, out=(torch.empty(4, 200, dtype=torch.int8, device=DEV),
                                                     torch.empty(4, 2, dtype=torch.float32, device=DEV)))
    q, s = w8.gemm_w8a8_block_quant(A[:0], SA[:0], W[:128], SW[:1])
    assert q.shape == (0, 128)

"""GPU parity of the GEMM kernels against the CPU oracle.

Bars (same seeded inputs on both sides):
  * int32 block partials P and the channel-wise raw accumulator: bit-exact;
  * channel-wise fp32 output: bit-exact with the oracle's fp32 path (the kernel
    evaluates fp32(fp32(ACC) * fp32(sa * sw)) exactly as the oracle does);
  * block-wise / W8A16 / grouped fp32 outputs: normwise relative error
    <= 1e-3 against the oracle's fp32 path and <= 1e-2 against its fp64 path;
  * bf16 outputs: the round-to-nearest-even of the same kernel's fp32 output
    (and <= 1e-2 against fp64).
Shapes cover several tiles plus ragged tails in M, N (576 = 4.5 N blocks) and
the decode (M <= 64) and tile (M > 64) code paths.
"""

import numpy as np
import pytest
import torch

import synth
import w8a8_int8_quantized_amd as w8
from oracle import formats, gemm, int4, quant, routing

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL32, TOL64 = 1e-3, 1e-2


def _np(t):
    return t.detach().cpu().numpy()


def _bf16_of(y32_gpu):
    return formats.f32_to_bf16_bits(_np(y32_gpu))


def _inputs(M, N, K, seed, scheme):
    x = synth.activations(M, K, seed=seed)
    w = synth.weights(N, K, seed=seed + 1)
    xn, wn = synth.to_numpy(x), synth.to_numpy(w)
    if scheme == "block":
        qa, sa = quant.quant_act_group(xn)
        qw, sw = quant.quant_weight_block(wn)
    else:
        qa, sa = quant.quant_act_token(xn)
        qw, sw = quant.quant_act_token(wn)
    return qa, sa, qw, sw


def _dev(*arrs):
    return [torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in arrs]


SHAPES = [(1, 256, 256), (8, 576, 1024), (16, 256, 256), (32, 1000, 512), (64, 576, 768),
          (65, 256, 256), (128, 512, 1024), (300, 576, 512), (513, 384, 384)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_channel_gemm_bit_exact(M, N, K):
    qa, sa, qw, sw = _inputs(M, N, K, seed=M * 7 + N, scheme="channel")
    A, SA, W, SW = _dev(qa, sa, qw, sw)
    ACC, y64, y32 = gemm.gemm_channel(qa, sa, qw, sw)
    acc = w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=torch.int32)
    assert np.array_equal(_np(acc), ACC)
    yf = w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=torch.float32)
    assert np.array_equal(_np(yf).view(np.uint32), y32.view(np.uint32))
    yb = w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=torch.bfloat16)
    assert np.array_equal(_np(yb.view(torch.int16)).view(np.uint16), _bf16_of(yf))
    assert gemm.normwise_rel_err(_np(yb.float()), y64) <= TOL64


# The largest K the channel-wise entry point accepts (2^17) with codes at
# +-127: |ACC| reaches 2^17 * 127^2 = 2,114,060,288 (row 0 of A and of W are
# all +127), just inside int32.  M = 2 runs the decode kernel, M = 300 the
# tile kernel split over K (int32 slice sums).
@pytest.mark.parametrize("M,N", [(2, 256), (300, 256)])
def test_channel_gemm_max_k_extreme_codes(M, N):
    K = 1 << 17
    rng = np.random.default_rng(M + N)
    qa = (rng.integers(0, 2, (M, K), dtype=np.int8) * 2 - 1) * np.int8(127)
    qw = (rng.integers(0, 2, (N, K), dtype=np.int8) * 2 - 1) * np.int8(127)
    qa[0, :] = 127
    qw[0, :] = 127
    sa = rng.uniform(1e-3, 2e-2, M).astype(np.float32)
    sw = rng.uniform(1e-4, 1e-3, N).astype(np.float32)
    ACC, y64, y32 = gemm.gemm_channel(qa, sa, qw, sw)
    assert ACC[0, 0] == K * 127 * 127
    A, SA, W, SW = _dev(qa, sa, qw, sw)
    assert np.array_equal(_np(w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=torch.int32)), ACC)
    yf = w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=torch.float32)
    assert np.array_equal(_np(yf).view(np.uint32), y32.view(np.uint32))
    yb = w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=torch.bfloat16)
    assert np.array_equal(_np(yb.view(torch.int16)).view(np.uint16), _bf16_of(yf))


# Shapes whose unsplit tile grid takes the narrower channel tiles: 224 columns
# (300 x 27990: 250 tiles in one round) and 192 columns (1000 x 12200: 256
# tiles; 520 x 30000: 471 tiles in two rounds), each with a ragged last tile
# in both M and N.
@pytest.mark.parametrize("M,N,K", [(300, 27990, 256), (1000, 12200, 256), (520, 30000, 256)])
def test_channel_gemm_narrow_tiles_bit_exact(M, N, K):
    qa, sa, qw, sw = _inputs(M, N, K, seed=M + N, scheme="channel")
    A, SA, W, SW = _dev(qa, sa, qw, sw)
    ACC, y64, y32 = gemm.gemm_channel(qa, sa, qw, sw)
    acc = w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=torch.int32)
    assert np.array_equal(_np(acc), ACC)
    yf = w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=torch.float32)
    assert np.array_equal(_np(yf).view(np.uint32), y32.view(np.uint32))
    yb = w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=torch.bfloat16)
    assert np.array_equal(_np(yb.view(torch.int16)).view(np.uint16), _bf16_of(yf))
    assert gemm.normwise_rel_err(_np(yb.float()), y64) <= TOL64


@pytest.mark.parametrize("M,N,K", [(16, 256, 256), (300, 576, 512), (129, 640, 1024)])
def test_block_partials_bit_exact(M, N, K):
    qa, _, qw, _ = _inputs(M, N, K, seed=M + 3, scheme="block")
    A, W = _dev(qa, qw)
    P = w8.gemm_w8a8_block_partials(A, W)
    assert np.array_equal(_np(P), gemm.block_partials(qa, qw))


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_block_gemm(M, N, K):
    qa, sa, qw, sw = _inputs(M, N, K, seed=M * 5 + K, scheme="block")
    A, SA, W, SW = _dev(qa, sa, qw, sw)
    _, y64, y32 = gemm.gemm_block(qa, sa, qw, sw)
    yf = w8.gemm_w8a8_block(A, SA, W, SW, out_dtype=torch.float32)
    e32 = gemm.normwise_rel_err(_np(yf), y32)
    e64 = gemm.normwise_rel_err(_np(yf), y64)
    assert e32 <= TOL32 and e64 <= TOL64, (e32, e64)
    assert e32 <= 1e-5          # in practice the fp32 orders differ by a few ulps
    yb = w8.gemm_w8a8_block(A, SA, W, SW, out_dtype=torch.bfloat16)
    assert np.array_equal(_np(yb.view(torch.int16)).view(np.uint16), _bf16_of(yf))
    assert gemm.normwise_rel_err(_np(yb.float()), y64) <= TOL64


# The 128-row tile widths of the block-wise GEMM, picked by the launch model:
# 128 x 192 tiles (four waves, a weight scale per 32-column chain since a
# wave's 96 columns can straddle two 128-column scale blocks) where the tiles
# do not fill the CUs, unsplit (300 x 1000) and split over K (3 and 10
# slices); 128 x 256 tiles on eight waves where they take more than one
# round, unsplit (1500 x 5000) and split (200 x 9000, 3 slices).  M and N
# are ragged in every case.
@pytest.mark.parametrize("M,N,K", [(300, 1000, 512), (1000, 1500, 3072), (257, 700, 4096), (1500, 5000, 256),
                                   (200, 9000, 4096)])
def test_block_gemm_tile_widths(M, N, K):
    qa, sa, qw, sw = _inputs(M, N, K, seed=M + N, scheme="block")
    A, SA, W, SW = _dev(qa, sa, qw, sw)
    _, y64, y32 = gemm.gemm_block(qa, sa, qw, sw)
    yf = w8.gemm_w8a8_block(A, SA, W, SW, out_dtype=torch.float32)
    e32, e64 = gemm.normwise_rel_err(_np(yf), y32), gemm.normwise_rel_err(_np(yf), y64)
    assert e32 <= 1e-5 and e64 <= TOL64, (e32, e64)
    yb = w8.gemm_w8a8_block(A, SA, W, SW, out_dtype=torch.bfloat16)
    assert np.array_equal(_np(yb.view(torch.int16)).view(np.uint16), _bf16_of(yf))


# 256-row tiles (a grid of at least 256 of them, unsplit) with one, two and
# three K blocks: the block loop's barrier before the last chain row, the
# stage loads past the last block, and the next block's fragments read from
# the other stage in the last block; M and N ragged.
@pytest.mark.parametrize("K", [128, 256, 384])
def test_block_gemm_256_row_tiles_short_k(K):
    M, N = 2000, 8000
    qa, sa, qw, sw = _inputs(M, N, K, seed=K + 11, scheme="block")
    A, SA, W, SW = _dev(qa, sa, qw, sw)
    _, y64, y32 = gemm.gemm_block(qa, sa, qw, sw)
    yf = w8.gemm_w8a8_block(A, SA, W, SW, out_dtype=torch.float32)
    e32, e64 = gemm.normwise_rel_err(_np(yf), y32), gemm.normwise_rel_err(_np(yf), y64)
    assert e32 <= 1e-5 and e64 <= TOL64, (e32, e64)
    yb = w8.gemm_w8a8_block(A, SA, W, SW, out_dtype=torch.bfloat16)
    assert np.array_equal(_np(yb.view(torch.int16)).view(np.uint16), _bf16_of(yf))


def test_block_equals_channel_when_k_is_one_block():
    M, N, K = 70, 256, 128
    qa, sa, qw, sw = _inputs(M, N, K, seed=1, scheme="block")
    A, SA, W, SW = _dev(qa, sa, qw, sw)
    sw_ch = torch.from_numpy(sw[np.arange(N) // 128, 0].copy()).to(DEV)
    yb = w8.gemm_w8a8_block(A, SA, W, SW, out_dtype=torch.float32)
    yc = w8.gemm_w8a8_channel(A, SA.reshape(-1).contiguous(), W, sw_ch, out_dtype=torch.float32)
    _, _, yb32 = gemm.gemm_block(qa, sa, qw, sw)
    assert gemm.normwise_rel_err(_np(yb), yb32) <= 1e-6
    assert gemm.normwise_rel_err(_np(yc), yb32) <= 1e-6


# (3, 4096, 12288): the Qwen3-8B down projection at 3 rows, whose 72 KB of
# activations are staged in LDS by the decode kernel; (12, 12288, 4096): the
# qkv projection at 12 rows, on the shared-activation kernel split over K.
@pytest.mark.parametrize("M,N,K", [(1, 256, 512), (3, 4096, 12288), (8, 1000, 4096), (12, 12288, 4096),
                                   (32, 512, 1024), (64, 384, 12288), (100, 256, 256)])
def test_w8a16_group(M, N, K):
    x = synth.activations(M, K, seed=M, dtype=torch.float16)
    w = synth.weights(N, K, seed=N, dtype=torch.float16)
    qw, sw = quant.quant_act_group(w.numpy())
    y64, y32 = gemm.gemm_w8a16_group(x.numpy(), qw, sw)
    X, W, SW = _dev(x.numpy(), qw, sw)
    y = w8.gemm_w8a16_group(X, W, SW)
    yn = _np(y).astype(np.float32)
    e32, e64 = gemm.normwise_rel_err(yn, y32), gemm.normwise_rel_err(yn, y64)
    assert e32 <= TOL32 and e64 <= TOL64, (e32, e64)


# Decode shapes wide enough for the workgroup-shared activation kernels: each
# N makes a different workgroup width (3, 4, 6, 8 and 9 waves of 16 columns)
# the one whose grid splits evenly over the CUs, and is 8 columns short of a
# whole number of workgroups, so the last wave is ragged.  K = 640 is five K
# blocks: two full staging groups of two blocks and a half-empty third.
DECODE_WIDE_N = [12280, 16376, 24568, 32760, 36856]


@pytest.mark.parametrize("N", DECODE_WIDE_N)
@pytest.mark.parametrize("M", [1, 24, 64])
def test_decode_wide_block_and_channel(M, N):
    K = 640
    qa, sa, qw, sw = _inputs(M, N, K, seed=M + N, scheme="block")
    A, SA, W, SW = _dev(qa, sa, qw, sw)
    _, y64, y32 = gemm.gemm_block(qa, sa, qw, sw)
    yf = w8.gemm_w8a8_block(A, SA, W, SW, out_dtype=torch.float32)
    e32 = gemm.normwise_rel_err(_np(yf), y32)
    assert e32 <= 1e-5 and gemm.normwise_rel_err(_np(yf), y64) <= TOL64, e32
    yb = w8.gemm_w8a8_block(A, SA, W, SW, out_dtype=torch.bfloat16)
    assert np.array_equal(_np(yb.view(torch.int16)).view(np.uint16), _bf16_of(yf))

    qa, sa, qw, sw = _inputs(M, N, K, seed=M + N + 7, scheme="channel")
    A, SA, W, SW = _dev(qa, sa, qw, sw)
    ACC, _, y32 = gemm.gemm_channel(qa, sa, qw, sw)
    assert np.array_equal(_np(w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=torch.int32)), ACC)
    yf = w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=torch.float32)
    assert np.array_equal(_np(yf).view(np.uint32), y32.view(np.uint32))
    yb = w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=torch.bfloat16)
    assert np.array_equal(_np(yb.view(torch.int16)).view(np.uint16), _bf16_of(yf))


# Five K blocks (an odd count, so the two-block activation stage of the decode
# kernels runs one block past the row) and an infinite block scale at the
# start of row 3: rows are independent in the block-wise definition, so every
# other row stays finite and matches the oracle.  N = 12288 takes the
# workgroup-shared decode kernel for M <= 64, N = 512 the split-K one, M = 200
# the tile kernel.
@pytest.mark.parametrize("M,N", [(8, 12288), (24, 12288), (64, 12288), (24, 512), (200, 512)])
def test_block_rows_independent_of_next_row_scale(M, N):
    K = 640
    qa, sa, qw, sw = _inputs(M, N, K, seed=M + N + 5, scheme="block")
    sa = sa.copy()
    sa[3, 0] = np.float32(np.inf)
    A, SA, W, SW = _dev(qa, sa, qw, sw)
    yf = _np(w8.gemm_w8a8_block(A, SA, W, SW, out_dtype=torch.float32))
    good = [m for m in range(M) if m != 3]
    _, y64, y32 = gemm.gemm_block(qa[good], sa[good], qw, sw)
    assert np.isfinite(yf[good]).all()
    e32 = gemm.normwise_rel_err(yf[good], y32)
    assert e32 <= 1e-5 and gemm.normwise_rel_err(yf[good], y64) <= TOL64, e32


# The workgroup-shared block-wise decode kernel stages a tile's activation
# scales in LDS (16 MF rows of K/128 | 1 floats, at most 64 KB): at 64 rows
# K = 32640 (255 K blocks, an odd row stride with no padding) is the longest
# staged, and K = 32768 (256 blocks) runs the split-K decode kernel instead.
# K = 7296 (57 blocks) and 7424 (58, a padded row) exercise the blocks past
# the last of an odd and an even count.  Checked on three sampled 128-column
# weight blocks; an infinite scale at the start of row 4 must reach no other
# row (past the end of row 3's staged scales lies row 4's).
@pytest.mark.parametrize("M,K", [(64, 32640), (64, 32768), (40, 7296), (40, 7424)])
def test_block_decode_staged_scales(M, K):
    N = 12288
    rng = np.random.default_rng(K)
    NB = N // 128
    blocks = np.array(sorted({0, NB - 1, int(rng.integers(1, NB - 1))}))
    cols = np.concatenate([np.arange(b * 128, (b + 1) * 128) for b in blocks])
    qw, sw = quant.quant_weight_block(synth.to_numpy(synth.weights(N, K, seed=K + 1)))
    qa, sa = quant.quant_act_group(synth.to_numpy(synth.activations(M, K, seed=K + 2)))
    sa = sa.copy()
    sa[4, 0] = np.float32(np.inf)
    A, SA, W, SW = _dev(qa, sa, qw, sw)
    qwc, swb = qw[cols], sw[blocks]
    del qw
    yf = _np(w8.gemm_w8a8_block(A, SA, W, SW, out_dtype=torch.float32))[:, cols]
    good = [m for m in range(M) if m != 4]
    _, y64, y32 = gemm.gemm_block(qa[good], sa[good], qwc, swb)
    assert np.isfinite(yf[good]).all()
    e32 = gemm.normwise_rel_err(yf[good], y32)
    assert e32 <= 1e-5 and gemm.normwise_rel_err(yf[good], y64) <= TOL64, e32


# N = 1000 is not a multiple of the 64-column workgroup: the last workgroup's
# fourth wave owns no columns, and K is split over 8 workgroups (slices past
# the first start their descriptors mid-row).  Regression case for such a wave
# reading past its (empty) range.
@pytest.mark.parametrize("M", [24, 32, 64])
def test_w8a16_split_k_ragged_workgroup(M):
    N, K = 1000, 4096
    x = synth.activations(M, K, seed=M + 11, dtype=torch.float16)
    w = synth.weights(N, K, seed=N + M + 1, dtype=torch.float16)
    qw, sw = quant.quant_act_group(w.numpy())
    y64, y32 = gemm.gemm_w8a16_group(x.numpy(), qw, sw)
    X, W, SW = _dev(x.numpy(), qw, sw)
    yn = _np(w8.gemm_w8a16_group(X, W, SW)).astype(np.float32)
    e32, e64 = gemm.normwise_rel_err(yn, y32), gemm.normwise_rel_err(yn, y64)
    assert e32 <= TOL32 and e64 <= TOL64, (e32, e64)


# Five and nine K blocks: the activation stage holds two K blocks, so the
# last stage of a K slice has a block past the slice's end, and in the last
# slice those bytes start the next row.  Non-finite values there must not
# reach the row above (0 * inf); rows are independent in the definition.
@pytest.mark.parametrize("M,N,K", [(4, 512, 640), (8, 512, 640), (24, 512, 640), (32, 512, 1152), (64, 384, 1152)])
def test_w8a16_rows_independent_of_next_row(M, N, K):
    x = synth.activations(M, K, seed=M + K, dtype=torch.float16).numpy().copy()
    w = synth.weights(N, K, seed=N + 7, dtype=torch.float16)
    qw, sw = quant.quant_act_group(w.numpy())
    bad = [3, M - 1]
    x[3, :128] = np.float16(np.inf)
    x[M - 1, :64] = np.float16(np.nan)
    X, W, SW = _dev(x, qw, sw)
    yn = _np(w8.gemm_w8a16_group(X, W, SW)).astype(np.float32)
    good = [m for m in range(M) if m not in bad]
    xg = np.ascontiguousarray(x[good])
    y64, y32 = gemm.gemm_w8a16_group(xg, qw, sw)
    assert np.isfinite(yn[good]).all()
    e32 = gemm.normwise_rel_err(yn[good], y32)
    e64 = gemm.normwise_rel_err(yn[good], y64)
    assert e32 <= TOL32 and e64 <= TOL64, (e32, e64)


# K split over workgroups, each slice writing fp32 partials that a second
# kernel (k_w16_slices_sum) sums in slice order: N not a multiple of 4 (the
# reduction's scalar tail), and repeated calls on one stream sharing the
# stream's workspace.
def _w8a16_case(M, N, K, seed):
    x = synth.activations(M, K, seed=seed, dtype=torch.float16)
    w = synth.weights(N, K, seed=seed + 1, dtype=torch.float16)
    qw, sw = quant.quant_act_group(w.numpy())
    return x.numpy(), qw, sw


def test_w8a16_split_k_odd_n():
    x, qw, sw = _w8a16_case(24, 998, 4096, seed=5)
    y64, y32 = gemm.gemm_w8a16_group(x, qw, sw)
    X, W, SW = _dev(x, qw, sw)
    yn = _np(w8.gemm_w8a16_group(X, W, SW)).astype(np.float32)
    e32, e64 = gemm.normwise_rel_err(yn, y32), gemm.normwise_rel_err(yn, y64)
    assert e32 <= TOL32 and e64 <= TOL64, (e32, e64)


# From 17 rows the shared-activation kernel runs twice its waves, the second
# half on the odd K blocks: an odd number of K blocks per slice (K = 1152 in
# two slices of 4 and 5 blocks at 20 and 24 rows on the balanced 12288
# columns; unsplit K = 1920 at 40 rows), INT8 and INT4 weights.
@pytest.mark.parametrize("M,K", [(20, 1152), (24, 1152), (40, 1920)])
def test_w8a16_k_parity_odd_blocks(M, K):
    N = 12288
    x, qw, sw = _w8a16_case(M, N, K, seed=M + K)
    y64, y32 = gemm.gemm_w8a16_group(x, qw, sw)
    X, W, SW = _dev(x, qw, sw)
    yn = _np(w8.gemm_w8a16_group(X, W, SW)).astype(np.float32)
    e32, e64 = gemm.normwise_rel_err(yn, y32), gemm.normwise_rel_err(yn, y64)
    assert e32 <= TOL32 and e64 <= TOL64, (e32, e64)
    w = synth.weights(N, K, seed=M + K + 1, dtype=torch.float16)
    q4, s4 = w8.quant_weight_int4_group(w.to(DEV))
    y4 = _np(w8.gemm_w4a16_group(X, q4, s4)).astype(np.float32)
    y4r = _np(w8.gemm_w8a16_group(X, torch.from_numpy(int4.unpack_int4(_np(q4))).to(DEV), s4)).astype(np.float32)
    assert np.array_equal(y4, y4r)


def test_w8a16_split_k_repeated_calls():
    N, K = 12288, 4096
    qw, sw = _w8a16_case(12, N, K, seed=9)[1:]
    W, SW = _dev(qw, sw)
    outs = []
    for seed in (21, 22, 21):
        x = synth.activations(12, K, seed=seed, dtype=torch.float16).numpy()
        y64, y32 = gemm.gemm_w8a16_group(x, qw, sw)
        (X,) = _dev(x)
        yn = _np(w8.gemm_w8a16_group(X, W, SW))
        e32 = gemm.normwise_rel_err(yn.astype(np.float32), y32)
        assert e32 <= TOL32, (seed, e32)
        outs.append(yn)
    assert np.array_equal(outs[0].view(np.uint16), outs[2].view(np.uint16))


@pytest.mark.parametrize("M", [1, 24, 64, 80])
def test_w8a16_wide(M):
    N, K = 12280, 640
    x = synth.activations(M, K, seed=M + 3, dtype=torch.float16)
    w = synth.weights(N, K, seed=N + M, dtype=torch.float16)
    qw, sw = quant.quant_act_group(w.numpy())
    y64, y32 = gemm.gemm_w8a16_group(x.numpy(), qw, sw)
    X, W, SW = _dev(x.numpy(), qw, sw)
    yn = _np(w8.gemm_w8a16_group(X, W, SW)).astype(np.float32)
    e32, e64 = gemm.normwise_rel_err(yn, y32), gemm.normwise_rel_err(yn, y64)
    assert e32 <= TOL32 and e64 <= TOL64, (e32, e64)


# 2048 x 8192 is 256 output tiles of 256 x 256: enough to fill the CUs, so
# the tile kernels run unsplit over K (the small shapes above, with a handful
# of tiles, run split over K with a reduction of the slices).
def test_tile_gemms_full_grid_unsplit():
    M, N, K = 2048, 8192, 768
    qa, sa, qw, sw = _inputs(M, N, K, seed=11, scheme="block")
    A, SA, W, SW = _dev(qa, sa, qw, sw)
    _, y64, y32 = gemm.gemm_block(qa, sa, qw, sw)
    yf = w8.gemm_w8a8_block(A, SA, W, SW, out_dtype=torch.float32)
    assert gemm.normwise_rel_err(_np(yf), y32) <= 1e-5
    yb = w8.gemm_w8a8_block(A, SA, W, SW, out_dtype=torch.bfloat16)
    assert np.array_equal(_np(yb.view(torch.int16)).view(np.uint16), _bf16_of(yf))
    qa, sa, qw, sw = _inputs(M, N, K, seed=12, scheme="channel")
    A, SA, W, SW = _dev(qa, sa, qw, sw)
    ACC, _, y32 = gemm.gemm_channel(qa, sa, qw, sw)
    assert np.array_equal(_np(w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=torch.int32)), ACC)
    yf = w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=torch.float32)
    assert np.array_equal(_np(yf).view(np.uint32), y32.view(np.uint32))
    yb = w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=torch.bfloat16)
    assert np.array_equal(_np(yb.view(torch.int16)).view(np.uint16), _bf16_of(yf))


# Grouped (MoE) cases: (experts, tokens, top-k, K, N, experts given no
# tokens, expert made hot).  Expert row ranges are cut into 128-row tiles
# below 96 rows per expert on average and 256-row tiles from there; the hot
# expert spans several tiles, 300 experts is more than the tile lookup's 64
# lanes x 4, and 256-row tiles of experts with fewer rows leave whole waves
# idle.  N = 400 and N = 300 leave a ragged last weight block.
GROUPED_CASES = [
    (12, 200, 2, 512, 384, (5, 7), None),
    (40, 1024, 4, 640, 400, (), 3),
    (300, 256, 8, 256, 256, (0, 299), None),
    (8, 1024, 3, 384, 300, (2,), 5),
    (4, 1024, 2, 512, 400, (), None),
]


@pytest.mark.parametrize("E,T,topk,K,N,empty,hot", GROUPED_CASES)
def test_grouped_moe_gemm(E, T, topk, K, N, empty, hot):
    lg = synth.router_logits(T, E, seed=4).numpy()
    for e in empty:
        lg[:, e] = -100.0
    if hot is not None:
        lg[:, hot] += 3.0
    rows, exps, offs = routing.topk_route(lg, topk)
    for e in empty:
        assert offs[e + 1] == offs[e]
    x = synth.to_numpy(synth.activations(T, K, seed=8))
    qa, sa = quant.quant_act_group(x[rows])
    NB = (N + 127) // 128
    qw = np.empty((E, N, K), np.int8)
    sw = np.empty((E, NB, K // 128), np.float32)
    for e in range(E):
        qw[e], sw[e] = quant.quant_weight_block(synth.to_numpy(synth.weights(N, K, seed=100 + e)))
    y64, y32 = gemm.gemm_block_grouped(qa, sa, qw, sw, offs)
    A, SA, W, SW = _dev(qa, sa, qw, sw)
    OFF = torch.from_numpy(offs.astype(np.int32)).to(DEV)
    y = w8.gemm_w8a8_block_grouped(A, SA, W, SW, OFF, out_dtype=torch.float32)
    yn = _np(y)
    for e in range(E):
        r0, r1 = offs[e], offs[e + 1]
        if r1 > r0:
            assert gemm.normwise_rel_err(yn[r0:r1], y32[r0:r1]) <= TOL32
            assert gemm.normwise_rel_err(yn[r0:r1], y64[r0:r1]) <= TOL64
    yb = w8.gemm_w8a8_block_grouped(A, SA, W, SW, OFF, out_dtype=torch.bfloat16)
    assert np.array_equal(_np(yb.view(torch.int16)).view(np.uint16), _bf16_of(y))


# From 96 rows per expert on average, experts with at most 128 rows run on
# 128-row tiles and the others on 256-row tiles, in two launches.  Row counts
# on both sides of the boundary (128 / 129), an empty expert, a one-row
# expert, exactly one 256-row tile and two tiles (300 rows).
def test_grouped_light_and_heavy_experts():
    counts = [128, 129, 0, 1, 256, 300]
    E, K, N = len(counts), 512, 384
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    P = int(offs[-1])
    assert P >= 96 * E
    x = synth.to_numpy(synth.activations(P, K, seed=21))
    qa, sa = quant.quant_act_group(x)
    NB = (N + 127) // 128
    qw = np.empty((E, N, K), np.int8)
    sw = np.empty((E, NB, K // 128), np.float32)
    for e in range(E):
        qw[e], sw[e] = quant.quant_weight_block(synth.to_numpy(synth.weights(N, K, seed=200 + e)))
    y64, y32 = gemm.gemm_block_grouped(qa, sa, qw, sw, offs)
    A, SA, W, SW = _dev(qa, sa, qw, sw)
    OFF = torch.from_numpy(offs.astype(np.int32)).to(DEV)
    y = _np(w8.gemm_w8a8_block_grouped(A, SA, W, SW, OFF, out_dtype=torch.float32))
    for e in range(E):
        r0, r1 = offs[e], offs[e + 1]
        if r1 > r0:
            assert gemm.normwise_rel_err(y[r0:r1], y32[r0:r1]) <= 1e-5, e
            assert gemm.normwise_rel_err(y[r0:r1], y64[r0:r1]) <= TOL64, e
    yb = w8.gemm_w8a8_block_grouped(A, SA, W, SW, OFF, out_dtype=torch.bfloat16)
    assert np.array_equal(_np(yb.view(torch.int16)).view(np.uint16), _bf16_of(torch.from_numpy(y)))


# 65..128 rows on N that balances over the CUs: the workgroup-shared decode
# kernel with eight 16-row fragments per wave; its int32, fp32 and bf16
# epilogues.
@pytest.mark.parametrize("N", [12280, 36856])
@pytest.mark.parametrize("M", [80, 100, 128])
def test_channel_up_to_128_rows_wide(M, N):
    K = 640
    qa, sa, qw, sw = _inputs(M, N, K, seed=M + N + 7, scheme="channel")
    A, SA, W, SW = _dev(qa, sa, qw, sw)
    ACC, _, y32 = gemm.gemm_channel(qa, sa, qw, sw)
    assert np.array_equal(_np(w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=torch.int32)), ACC)
    yf = w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=torch.float32)
    assert np.array_equal(_np(yf).view(np.uint32), y32.view(np.uint32))
    yb = w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=torch.bfloat16)
    assert np.array_equal(_np(yb.view(torch.int16)).view(np.uint16), _bf16_of(yf))


# Up to 128 rows where N does not balance the decode kernel: the tile kernel
# split over K with the upper half of its row tile idle (waves 4..7 only
# load), int32 slice sums, ragged N and one-block slices (K = 2048, 16 slices).
@pytest.mark.parametrize("M,N,K", [(72, 1000, 4096), (128, 2000, 2048), (100, 520, 2048)])
def test_channel_split_k_up_to_128_rows(M, N, K):
    qa, sa, qw, sw = _inputs(M, N, K, seed=M + N + 11, scheme="channel")
    A, SA, W, SW = _dev(qa, sa, qw, sw)
    ACC, y64, y32 = gemm.gemm_channel(qa, sa, qw, sw)
    assert np.array_equal(_np(w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=torch.int32)), ACC)
    yf = w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=torch.float32)
    assert np.array_equal(_np(yf).view(np.uint32), y32.view(np.uint32))
    yb = w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=torch.bfloat16)
    assert np.array_equal(_np(yb.view(torch.int16)).view(np.uint16), _bf16_of(yf))


def test_gemms_are_deterministic():
    qa, sa, qw, sw = _inputs(300, 576, 1024, seed=2, scheme="block")
    A, SA, W, SW = _dev(qa, sa, qw, sw)
    a = w8.gemm_w8a8_block(A, SA, W, SW, out_dtype=torch.float32)
    b = w8.gemm_w8a8_block(A, SA, W, SW, out_dtype=torch.float32)
    assert torch.equal(a, b)
    a = w8.gemm_w8a8_block(A[:8].contiguous(), SA[:8].contiguous(), W, SW, out_dtype=torch.float32)
    b = w8.gemm_w8a8_block(A[:8].contiguous(), SA[:8].contiguous(), W, SW, out_dtype=torch.float32)
    assert torch.equal(a, b)


def test_empty_gemms_are_noops():
    A = torch.empty(0, 256, dtype=torch.int8, device=DEV)
    SA = torch.empty(0, 2, dtype=torch.float32, device=DEV)
    W = torch.zeros(128, 256, dtype=torch.int8, device=DEV)
    SW = torch.ones(1, 2, dtype=torch.float32, device=DEV)
    assert w8.gemm_w8a8_block(A, SA, W, SW).shape == (0, 128)


def test_split_workspaces_are_per_stream():
    """Split-K GEMMs (partials in the library's per-stream workspace) and the
    asymmetric decode GEMM (int32 accumulators in the second workspace) on
    two streams at once give the same bits as on one stream."""
    M, N, K = 512, 1536, 7168          # few tiles: the block and channel GEMMs split K
    outs = {}
    inputs = []
    for i in range(2):
        qa, sa = quant.quant_act_group(synth.to_numpy(synth.activations(M, K, seed=140 + i)))
        qw, sw = quant.quant_weight_block(synth.to_numpy(synth.weights(N, K, seed=150 + i)))
        qt, st = quant.quant_act_token(synth.to_numpy(synth.activations(M, K, seed=160 + i)))
        qc, sc = quant.quant_act_token(synth.to_numpy(synth.weights(N, K, seed=170 + i)))
        inputs.append([torch.from_numpy(a).to(DEV) for a in (qa, sa, qw, sw, qt, st, qc, sc)])

    def run(t):
        A, SA, W, SW, AT, ST, WC, SC = t
        yb = w8.gemm_w8a8_block(A, SA, W, SW, out_dtype=torch.float32)
        yc = w8.gemm_w8a8_channel(AT, ST, WC, SC, out_dtype=torch.float32)
        prm = torch.tensor([0.01, 3.5], device=DEV)
        ya = w8.gemm_w8a8_asym(AT[:8].contiguous(), prm, WC, SC, w8.weight_row_sums(WC), out_dtype=torch.float32)
        return yb, yc, ya

    ref = [run(t) for t in inputs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for i, s in enumerate(streams):
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                outs[i] = run(inputs[i])
        torch.cuda.synchronize()
        for i in range(2):
            for got, want in zip(outs[i], ref[i]):
                assert torch.equal(got.view(torch.int32), want.view(torch.int32)), (rep, i)


def test_graph_capture_replays_match_eager():
    """The GEMM paths launch no memsets and allocate nothing once a stream's
    workspace has grown, so a captured HIP graph (split-K block-wise GEMM,
    one-call linear layer, split-K channel-wise GEMM) replays to the eager
    bits; eager overwrites and synchronisations run between the replays."""
    M, N, K = 512, 1536, 7168
    qa, sa = quant.quant_act_group(synth.to_numpy(synth.activations(M, K, seed=180)))
    qw, sw = quant.quant_weight_block(synth.to_numpy(synth.weights(N, K, seed=181)))
    qt, st = quant.quant_act_token(synth.to_numpy(synth.activations(M, K, seed=182)))
    qc, sc = quant.quant_act_token(synth.to_numpy(synth.weights(N, K, seed=183)))
    A, SA, W, SW, AT, ST, WC, SC = (torch.from_numpy(a).to(DEV) for a in (qa, sa, qw, sw, qt, st, qc, sc))
    x = synth.activations(8, 4096, seed=184).to(DEV)
    qd, sd = quant.quant_weight_block(synth.to_numpy(synth.weights(12288, 4096, seed=185)))
    WD, SWD = torch.from_numpy(qd).to(DEV), torch.from_numpy(sd).to(DEV)
    ws = torch.empty(w8.linear_workspace_bytes(w8.W8_SCHEME_BLOCK, 8, 4096), dtype=torch.uint8, device=DEV)

    def step():
        return (w8.gemm_w8a8_block(A, SA, W, SW, out_dtype=torch.float32),
                w8.linear_w8a8_block(x, WD, SWD, out_dtype=torch.float32, workspace=ws),
                w8.gemm_w8a8_channel(AT, ST, WC, SC, out_dtype=torch.float32))

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ref = [t.clone() for t in step()]          # grows this stream's workspaces
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        outs = step()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o.view(torch.int32), r.view(torch.int32)), rep


def test_split_k_under_capture_without_workspace_is_refused():
    """A stream being captured gets no allocation: a split-K call whose
    stream has no workspace yet returns W8_ERR_CAPTURE with nothing enqueued
    (the capture stays valid and records nothing); after one eager call on
    that stream the same call captures and replays to the eager bits."""
    M, N, K = 300, 1000, 4096        # small tile grid: K is split
    qt, st = quant.quant_act_token(synth.to_numpy(synth.activations(M, K, seed=190)))
    qc, sc = quant.quant_act_token(synth.to_numpy(synth.weights(N, K, seed=191)))
    AT, ST, WC, SC = (torch.from_numpy(a).to(DEV) for a in (qt, st, qc, sc))
    y = torch.empty(M, N, dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with pytest.raises(w8.W8Error) as ei:
        with torch.cuda.graph(g, stream=s):
            w8.gemm_w8a8_channel(AT, ST, WC, SC, out=y)
    assert ei.value.status == w8.W8_ERR_CAPTURE
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        ref = w8.gemm_w8a8_channel(AT, ST, WC, SC, out_dtype=torch.float32)
    torch.cuda.synchronize()
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2, stream=s):
        w8.gemm_w8a8_channel(AT, ST, WC, SC, out=y)
    for rep in range(2):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g2.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), ref.view(torch.int32)), rep

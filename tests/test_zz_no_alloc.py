"""The allocation-free entry point gemm_w8a8_channel_noalloc against
gemm_w8a8_channel (GPU).

Two calls in a row on split-K shapes (so the fixed scratch array is used),
the second smaller than the first, each bit-identical to
gemm_w8a8_channel's output in int32, fp32 and bf16; then a shape whose
partials exceed the 64 MiB array is refused with W8_ERR_WORKSPACE and
nothing is written.
"""

import numpy as np
import pytest
import torch

import synth
import w8a8_int8_quantized_amd as w8
from oracle import quant

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _operands(M, N, K, seed):
    qa, sa = quant.quant_act_token(synth.to_numpy(synth.activations(M, K, seed=seed)))
    qw, sw = quant.quant_act_token(synth.to_numpy(synth.weights(N, K, seed=seed + 1)))
    return tuple(torch.from_numpy(a).to(DEV) for a in (qa, sa, qw, sw))


@pytest.mark.parametrize("shapes", [[(1024, 7168, 18432), (300, 1000, 4096)]])
def test_noalloc_matches_allocating_entry_point(shapes):
    for M, N, K in shapes:                      # the second call is the smaller one
        print(f"noalloc channel GEMM M={M} N={N} K={K}", flush=True)
        A, SA, W, SW = _operands(M, N, K, seed=M + N)
        for dt in (torch.int32, torch.float32, torch.bfloat16):
            want = w8.gemm_w8a8_channel(A, SA, W, SW, out_dtype=dt)
            got = torch.full_like(want, 7) if dt != torch.bfloat16 else torch.zeros_like(want)
            w8.gemm_w8a8_channel_noalloc(A, SA, W, SW, out=got)
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                               want.view(torch.int16 if dt == torch.bfloat16 else torch.int32)), (M, N, K, dt)


def test_noalloc_refuses_shapes_beyond_its_scratch():
    # 1280 x 5120 output (100 tiles of 256 x 256) over K = 65536: the slice
    # rule splits K five ways, 5 x 1280 x 5120 x 4 bytes > 64 MiB
    M, N, K = 1280, 5120, 65536
    print(f"noalloc refusal M={M} N={N} K={K}", flush=True)
    A = torch.zeros(M, K, dtype=torch.int8, device=DEV)
    W = torch.zeros(N, K, dtype=torch.int8, device=DEV)
    SA = torch.ones(M, dtype=torch.float32, device=DEV)
    SW = torch.ones(N, dtype=torch.float32, device=DEV)
    y = torch.full((M, N), 3.0, dtype=torch.float32, device=DEV)
    with pytest.raises(w8.W8Error) as ei:
        w8.gemm_w8a8_channel_noalloc(A, SA, W, SW, out=y)
    assert ei.value.status == w8.W8_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())                # nothing was enqueued

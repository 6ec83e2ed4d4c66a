"""Seeded synthetic inputs for the W8A8 INT8 linear-layer path.

This module only draws random inputs and lays them out; it holds none of the
method's arithmetic (no quantisation, no scaling, no GEMM).  Both the HIP path
(through the tests and the benchmark) and the CPU oracle take their inputs
from here.  Tensors are created with a seeded ``torch.Generator`` on the
requested device; the same (seed, device type) always gives the same values.

Workloads (shapes of DeepSeek-V3/R1 linears and of a Qwen3-8B-shaped W8A16
decode, all from the build's configuration list):

  tiny     M=16, K=256, N=256; activations N(0,1) with 1% of entries x20;
           weights N(0, 0.02); block-wise scheme.
  channel  DeepSeek-V3 dense MLP: gate_up K=7168 -> N=36864, down K=18432 ->
           N=7168; M in {128, 1024, 4096}; activations N(0,1) with 0.5% x30.
  block    same MLP shapes plus q_a (7168 -> 1536), q_b (1536 -> 24576) and
           kv_a (7168 -> 576) at M=4096; weights drawn as FP8-E4M3 codes with
           a per-128x128 scale_inv ~ LogUniform(1e-4, 1e-2).
  decode   M in {1, 8, 32, 64}: block-wise at K=7168, N=36864, and W8A16
           (fp16 activations, group-wise int8 weights) at K=4096 -> N=12288
           and K=12288 -> N=4096.
  moe      256 experts, top-8 routing of 4096 tokens (logits N(0,1)); gate_up
           K=7168 -> N=4096 and down K=2048 -> N=7168 per expert.

Outliers: exactly round(p * M * K) distinct positions, uniform without
replacement, multiplied by the factor (sign kept) before the bf16 rounding.
"""

import math

import torch

GROUP = 128

SHAPES = {
    "gate_up": (7168, 36864),   # (K, N)
    "down": (18432, 7168),
    "q_a": (7168, 1536),
    "q_b": (1536, 24576),
    "kv_a": (7168, 576),
    "w8a16_qkv": (4096, 12288),
    "w8a16_down": (12288, 4096),
    "moe_gate_up": (7168, 4096),
    "moe_down": (2048, 7168),
}

SEEDS = {"tiny": 0, "channel": 1, "block": 2, "decode": 3, "moe": 4}


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def activations(M, K, seed, device="cpu", outlier_frac=0.005, outlier_factor=30.0,
                dtype=torch.bfloat16):
    """N(0,1) activations [M, K] with exactly round(p*M*K) outliers x factor."""
    g = _gen(seed, device)
    x = torch.randn(M, K, generator=g, device=device, dtype=torch.float32)
    n_out = int(round(outlier_frac * M * K))
    if n_out > 0:
        pos = torch.randperm(M * K, generator=g, device=device)[:n_out]
        flat = x.view(-1)
        flat[pos] = flat[pos] * outlier_factor
    return x.to(dtype)


def weights(N, K, seed, device="cpu", std=0.02, dtype=torch.bfloat16):
    """N(0, std) weights [N, K] (nn.Linear layout)."""
    g = _gen(seed, device)
    w = torch.randn(N, K, generator=g, device=device, dtype=torch.float32) * std
    return w.to(dtype)


def fp8_weights(N, K, seed, device="cpu"):
    """FP8-E4M3FN weight codes [N, K] (uint8) and scale_inv [ceil(N/128), K/128].

    Per 128x128 tile: z ~ N(0,1) scaled so that the tile's largest |z| maps to
    448 (the largest E4M3FN value), then encoded to E4M3FN by torch's cast;
    scale_inv = exp(U(ln 1e-4, ln 1e-2)) independently per tile, in fp32.
    """
    assert K % GROUP == 0
    g = _gen(seed, device)
    NB, KB = (N + GROUP - 1) // GROUP, K // GROUP
    z = torch.randn(N, K, generator=g, device=device, dtype=torch.float32)
    pad = NB * GROUP - N
    zt = torch.nn.functional.pad(z, (0, 0, 0, pad)) if pad else z
    tmax = zt.abs().view(NB, GROUP, KB, GROUP).amax(dim=(1, 3))        # [NB, KB]
    tmax = torch.clamp(tmax, min=1e-30)
    rows = torch.arange(N, device=device) // GROUP
    cols = torch.arange(K, device=device) // GROUP
    scaled = z * (448.0 / tmax)[rows][:, cols]
    scaled = torch.clamp(scaled, -448.0, 448.0)
    codes = scaled.to(torch.float8_e4m3fn).view(torch.uint8)
    u = torch.rand(NB, KB, generator=g, device=device, dtype=torch.float64)
    scale_inv = torch.exp(math.log(1e-4) + u * (math.log(1e-2) - math.log(1e-4))).to(torch.float32)
    return codes.contiguous(), scale_inv.contiguous()


def router_logits(T, E, seed, device="cpu"):
    g = _gen(seed, device)
    return torch.randn(T, E, generator=g, device=device, dtype=torch.float32)


def route_topk(logits, k):
    """Data layout for the grouped GEMM: top-k experts per token by raw logit
    (ties to the lower expert index), pairs ordered by (expert, token).

    Returns (rows [T*k] int64 token of each sorted pair, experts [T*k] int64,
    offsets [E+1] int32 exclusive prefix sum of the per-expert counts).
    """
    T, E = logits.shape
    order = torch.sort(logits, dim=1, descending=True, stable=True).indices[:, :k]
    tok = torch.arange(T, device=logits.device).repeat_interleave(k)
    exp = order.reshape(-1)
    key = exp * T + tok
    perm = torch.sort(key, stable=True).indices
    counts = torch.bincount(exp, minlength=E)
    offsets = torch.zeros(E + 1, dtype=torch.int64, device=logits.device)
    offsets[1:] = torch.cumsum(counts, 0)
    return tok[perm], exp[perm], offsets.to(torch.int32)


def to_numpy(t):
    """CPU numpy view for the oracle: bf16 -> uint16 bit patterns, fp8 codes
    stay uint8, other dtypes unchanged."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()

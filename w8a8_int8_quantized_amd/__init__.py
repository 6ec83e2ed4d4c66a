"""MI355X (gfx950) W8A8 INT8 linear layers: thin Python binding of libw8a8.so.

Every function here only checks tensors, allocates outputs with torch (device
memory only) and calls the C ABI declared in include/w8a8.h on torch's current
HIP stream.  All arithmetic runs in the library's HIP kernels; there is no
fallback: if libw8a8.so is missing, importing this package raises.

    q, s  = quant_act_group(x)                 # block-wise activations, 1x128 groups
    q, s  = quant_act_token(x)                 # channel-wise activations, one scale per row
    wq, ws = quant_weight_block(w_bf16)        # 128x128 weight tiles
    wq, ws = requant_fp8_to_int8_block(w_fp8, scale_inv)
    y = gemm_w8a8_block(q, s, wq, ws)          # bf16 (or fp32) output
    y = gemm_w8a8_channel(q, s, wq, ws)
    y = linear_w8a8_block(x, wq, ws)           # quant_act_group + gemm_w8a8_block in one call
    qa, prm = quant_act_asym(x)                # asymmetric per-tensor uint8 (stored as q - 128)
    y = gemm_w8a8_asym(qa, prm, wq, ws, weight_row_sums(wq))   # per-channel weights
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw8a8.so")

W8_BF16, W8_FP16, W8_FP32, W8_I32 = 0, 1, 2, 3
W8_SCHEME_BLOCK, W8_SCHEME_CHANNEL = 0, 1
GROUP = 128

_FUNCS = {
    "w8_abi_version": (ctypes.c_int, []),
    "w8_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "quant_act_group": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "quant_act_token": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "quant_weight_block": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "requant_fp8_to_int8_block": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_void_p]),
    "requant_fp8_to_int8_channel": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                                   ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                                   ctypes.c_void_p]),
    "gemm_w8a8_block": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_void_p]),
    "gemm_w8a8_channel": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_void_p]),
    "gemm_w8a8_channel_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                                 ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]),
    "gemm_w8a8_block_quant": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_int64, ctypes.c_void_p]),
    "gemm_w8a8_block_grouped_quant": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                     ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                                     ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]),
    "gemm_w8a8_block_partials": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]),
    "gemm_w8a16_group": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]),
    "quant_weight_int4_group": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "gemm_w4a16_group": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]),
    "gemm_w8a8_block_grouped": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                               ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                               ctypes.c_void_p]),
    "linear_workspace_bytes": (ctypes.c_int64, [ctypes.c_int, ctypes.c_int64, ctypes.c_int64]),
    "quant_act_asym": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "weight_row_sums": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                       ctypes.c_void_p]),
    "gemm_w8a8_asym": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]),
    "linear_w8a8_block": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]),
    "linear_w8a8_channel": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                           ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python w8a8_int8_quantized_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _FUNCS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


W8_ERR_WORKSPACE, W8_ERR_CAPTURE = -6, -7


class W8Error(RuntimeError):
    def __init__(self, msg, status=None):
        super().__init__(msg)
        self.status = status


def _check(rc, what):
    if rc != 0:
        raise W8Error(f"{what}: {lib.w8_status_string(rc).decode()} (status {rc})", rc)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise W8Error("tensors must be on the GPU")
            if not t.is_contiguous():
                raise W8Error("tensors must be contiguous")


def _act_dtype(x):
    if x.dtype == torch.bfloat16:
        return W8_BF16
    if x.dtype == torch.float16:
        return W8_FP16
    raise W8Error(f"activations must be bf16 or fp16, got {x.dtype}")


def _out_code(dt):
    return {torch.bfloat16: W8_BF16, torch.float32: W8_FP32, torch.int32: W8_I32}[dt]


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


# ----------------------------------------------------------------- quantisers
def quant_act_group(x, out=None):
    """Per-token-group (1x128) quantisation of x [M, K] (bf16 or fp16)."""
    _dev(x)
    M, K = x.shape
    q, s = out if out is not None else (_empty((M, K), torch.int8, x), _empty((M, K // GROUP), torch.float32, x))
    _check(lib.quant_act_group(_p(x), _act_dtype(x), M, K, _p(q), _p(s), _stream()), "quant_act_group")
    return q, s


def quant_act_token(x, out=None):
    """Per-token quantisation of x [M, K] (bf16 or fp16): one scale per row."""
    _dev(x)
    M, K = x.shape
    q, s = out if out is not None else (_empty((M, K), torch.int8, x), _empty((M,), torch.float32, x))
    _check(lib.quant_act_token(_p(x), _act_dtype(x), M, K, _p(q), _p(s), _stream()), "quant_act_token")
    return q, s


def quant_weight_block(w, out=None):
    """128x128 tile quantisation of bf16 weights w [N, K]."""
    _dev(w)
    if w.dtype != torch.bfloat16:
        raise W8Error("quant_weight_block takes bf16 weights")
    N, K = w.shape
    NB = (N + GROUP - 1) // GROUP
    q, s = out if out is not None else (_empty((N, K), torch.int8, w), _empty((NB, K // GROUP), torch.float32, w))
    _check(lib.quant_weight_block(_p(w), N, K, _p(q), _p(s), _stream()), "quant_weight_block")
    return q, s


def quant_weight_channel(w):
    """Channel-wise weight quantisation: one scale per output channel (row)."""
    return quant_act_token(w)


def requant_fp8_to_int8_block(w_fp8, scale_inv, return_bf16=False, out=None):
    """FP8-E4M3FN codes [N, K] (uint8) with scale_inv [NB, KB] -> BF16 -> INT8 128x128 tiles
    (out: an optional (codes, scales) pair to write into)."""
    _dev(w_fp8, scale_inv)
    if w_fp8.dtype == torch.float8_e4m3fn:
        w_fp8 = w_fp8.view(torch.uint8)
    N, K = w_fp8.shape
    NB = (N + GROUP - 1) // GROUP
    q, s = out if out is not None else (_empty((N, K), torch.int8, w_fp8), _empty((NB, K // GROUP), torch.float32,
                                                                                 w_fp8))
    _dev(q, s)
    wb = _empty((N, K), torch.bfloat16, w_fp8) if return_bf16 else None
    _check(lib.requant_fp8_to_int8_block(_p(w_fp8), _p(scale_inv), N, K, _p(q), _p(s), _p(wb), _stream()),
           "requant_fp8_to_int8_block")
    return (q, s, wb) if return_bf16 else (q, s)


def requant_fp8_to_int8_channel(w_fp8, scale_inv):
    """FP8-E4M3FN codes [N, K] with scale_inv [NB, KB] -> BF16 -> per-channel INT8."""
    _dev(w_fp8, scale_inv)
    if w_fp8.dtype == torch.float8_e4m3fn:
        w_fp8 = w_fp8.view(torch.uint8)
    N, K = w_fp8.shape
    q = _empty((N, K), torch.int8, w_fp8)
    s = _empty((N,), torch.float32, w_fp8)
    _check(lib.requant_fp8_to_int8_channel(_p(w_fp8), _p(scale_inv), N, K, _p(q), _p(s), _stream()),
           "requant_fp8_to_int8_channel")
    return q, s


# ---------------------------------------------------------------------- GEMMs
def gemm_w8a8_block(A, a_scale, W, w_scale, out_dtype=torch.bfloat16, out=None):
    """Block-wise W8A8 GEMM: Y[M, N] = sum_kb sa[m,kb] sw[n/128,kb] P[kb,m,n]."""
    _dev(A, a_scale, W, w_scale)
    M, K = A.shape
    N = W.shape[0]
    y = out if out is not None else _empty((M, N), out_dtype, A)
    _check(lib.gemm_w8a8_block(_p(A), _p(a_scale), _p(W), _p(w_scale), _p(y), _out_code(y.dtype), M, N, K,
                               _stream()), "gemm_w8a8_block")
    return y


def gemm_w8a8_channel(A, a_scale, W, w_scale, out_dtype=torch.bfloat16, out=None):
    """Channel-wise W8A8 GEMM: Y = (A . W^T) * sa[m] * sw[n]; int32 output = raw accumulator."""
    _dev(A, W, a_scale, w_scale)
    M, K = A.shape
    N = W.shape[0]
    y = out if out is not None else _empty((M, N), out_dtype, A)
    _check(lib.gemm_w8a8_channel(_p(A), _p(a_scale), _p(W), _p(w_scale), _p(y), _out_code(y.dtype), M, N, K,
                                 _stream()), "gemm_w8a8_channel")
    return y


def gemm_w8a8_block_quant(A, a_scale, W, w_scale, out=None):
    """Block-wise GEMM whose bf16 output is quantised per 1 x 128 group in the
    epilogue (the next layer's activations): returns (q int8 [M, N], scales
    fp32 [M, N/128]), equal to quant_act_group(gemm_w8a8_block(...))."""
    _dev(A, W, a_scale, w_scale)
    M, K = A.shape
    N = W.shape[0]
    q, s = out if out is not None else (_empty((M, N), torch.int8, A), _empty((M, N // GROUP), torch.float32, A))
    _dev(q, s)
    _check(lib.gemm_w8a8_block_quant(_p(A), _p(a_scale), _p(W), _p(w_scale), _p(q), _p(s), M, N, K, _stream()),
           "gemm_w8a8_block_quant")
    return q, s


def gemm_w8a8_block_grouped_quant(A, a_scale, W, w_scale, offsets, out=None):
    """Grouped (MoE) block-wise GEMM with the output group quantisation fused:
    returns (q int8 [P, N], scales fp32 [P, N/128])."""
    _dev(A, W, a_scale, w_scale, offsets)
    P, K = A.shape
    E, N, _ = W.shape
    q, s = out if out is not None else (_empty((P, N), torch.int8, A), _empty((P, N // GROUP), torch.float32, A))
    _dev(q, s)
    _check(lib.gemm_w8a8_block_grouped_quant(_p(A), _p(a_scale), _p(W), _p(w_scale), _p(offsets), _p(q), _p(s), E,
                                             P, N, K, _stream()), "gemm_w8a8_block_grouped_quant")
    return q, s


def gemm_w8a8_channel_noalloc(A, a_scale, W, w_scale, out_dtype=torch.bfloat16, out=None):
    """gemm_w8a8_channel with its split-K partials in the library's fixed
    64 MiB scratch array instead of an allocated workspace (for callers that
    cannot allocate); pass `out` to allocate nothing here either."""
    _dev(A, W, a_scale, w_scale)
    M, K = A.shape
    N = W.shape[0]
    y = out if out is not None else _empty((M, N), out_dtype, A)
    _check(lib.gemm_w8a8_channel_noalloc(_p(A), _p(a_scale), _p(W), _p(w_scale), _p(y), _out_code(y.dtype), M, N,
                                         K, _stream()), "gemm_w8a8_channel_noalloc")
    return y


def gemm_w8a8_block_partials(A, W):
    """The exact int32 partial sums P[kb, m, n] of the block-wise GEMM."""
    _dev(A, W)
    M, K = A.shape
    N = W.shape[0]
    P = _empty((K // GROUP, M, N), torch.int32, A)
    _check(lib.gemm_w8a8_block_partials(_p(A), _p(W), _p(P), M, N, K, _stream()), "gemm_w8a8_block_partials")
    return P


def gemm_w8a16_group(x, W, w_scale, out=None):
    """W8A16: fp16 x [M, K], int8 W [N, K], group scales [N, K/128] -> fp16 Y [M, N]."""
    _dev(x, W, w_scale)
    if x.dtype != torch.float16:
        raise W8Error("gemm_w8a16_group takes fp16 activations")
    M, K = x.shape
    N = W.shape[0]
    y = out if out is not None else _empty((M, N), torch.float16, x)
    _check(lib.gemm_w8a16_group(_p(x), _p(W), _p(w_scale), _p(y), M, N, K, _stream()), "gemm_w8a16_group")
    return y


def quant_weight_int4_group(w, out=None):
    """Group-wise (1x128) INT4 quantisation of weights w [N, K] (bf16 or fp16):
    packed codes uint8 [N, K/2] (two offset-binary nibbles per byte) and
    scales fp32 [N, K/128]."""
    _dev(w)
    N, K = w.shape
    q, s = out if out is not None else (_empty((N, K // 2), torch.uint8, w), _empty((N, K // GROUP), torch.float32, w))
    _check(lib.quant_weight_int4_group(_p(w), _act_dtype(w), N, K, _p(q), _p(s), _stream()),
           "quant_weight_int4_group")
    return q, s


def gemm_w4a16_group(x, W4, w_scale, out=None):
    """W4A16: fp16 x [M, K], packed INT4 W4 [N, K/2], group scales [N, K/128] -> fp16 Y [M, N]."""
    _dev(x, W4, w_scale)
    if x.dtype != torch.float16:
        raise W8Error("gemm_w4a16_group takes fp16 activations")
    if W4.dtype != torch.uint8:
        raise W8Error("gemm_w4a16_group takes packed uint8 weights")
    M, K = x.shape
    N = W4.shape[0]
    if W4.shape[1] * 2 != K:
        raise W8Error("gemm_w4a16_group: W4 must be [N, K/2]")
    y = out if out is not None else _empty((M, N), torch.float16, x)
    _check(lib.gemm_w4a16_group(_p(x), _p(W4), _p(w_scale), _p(y), M, N, K, _stream()), "gemm_w4a16_group")
    return y


def gemm_w8a8_block_grouped(A, a_scale, W, w_scale, expert_offsets, out_dtype=torch.bfloat16, out=None):
    """Grouped block-wise GEMM over expert-sorted rows; W [E, N, K], offsets int32 [E+1] on the GPU."""
    _dev(A, a_scale, W, w_scale, expert_offsets)
    if expert_offsets.dtype != torch.int32:
        raise W8Error("expert_offsets must be int32")
    P, K = A.shape
    E, N, _ = W.shape
    y = out if out is not None else _empty((P, N), out_dtype, A)
    _check(lib.gemm_w8a8_block_grouped(_p(A), _p(a_scale), _p(W), _p(w_scale), _p(expert_offsets), _p(y),
                                       _out_code(y.dtype), E, P, N, K, _stream()), "gemm_w8a8_block_grouped")
    return y


# ------------------------------------------------------------- linear layers
def linear_workspace_bytes(scheme, M, K):
    """Bytes of workspace linear_w8a8_block (W8_SCHEME_BLOCK) or linear_w8a8_channel needs."""
    n = lib.linear_workspace_bytes(scheme, M, K)
    _check(min(n, 0), "linear_workspace_bytes")
    return n


def _linear(fn, scheme, x, W, w_scale, out_dtype, out, workspace):
    _dev(x, W, w_scale, out, workspace)
    M, K = x.shape
    N = W.shape[0]
    need = linear_workspace_bytes(scheme, M, K)
    ws = workspace if workspace is not None else _empty((max(need, 1),), torch.uint8, x)
    y = out if out is not None else _empty((M, N), out_dtype, x)
    _check(fn(_p(x), _act_dtype(x), _p(W), _p(w_scale), _p(y), _out_code(y.dtype), M, N, K, _p(ws),
              ws.numel() * ws.element_size(), _stream()), fn.__name__)
    return y


def linear_w8a8_block(x, W, w_scale, out_dtype=torch.bfloat16, out=None, workspace=None):
    """quant_act_group(x) then the block-wise GEMM, in one call; x [M, K] bf16/fp16."""
    return _linear(lib.linear_w8a8_block, W8_SCHEME_BLOCK, x, W, w_scale, out_dtype, out, workspace)


def linear_w8a8_channel(x, W, w_scale, out_dtype=torch.bfloat16, out=None, workspace=None):
    """quant_act_token(x) then the channel-wise GEMM, in one call; x [M, K] bf16/fp16."""
    return _linear(lib.linear_w8a8_channel, W8_SCHEME_CHANNEL, x, W, w_scale, out_dtype, out, workspace)


# ------------------------------------------------- asymmetric (per tensor)
def quant_act_asym(x, out=None):
    """Per-tensor asymmetric quantisation of x [M, K] (bf16 or fp16).

    Returns (codes, params): int8 codes holding q - 128 for the uint8 code q,
    and a device fp32 tensor [2] = (scale, zero point).
    """
    _dev(x)
    M, K = x.shape
    q, prm = out if out is not None else (_empty((M, K), torch.int8, x), _empty((2,), torch.float32, x))
    _check(lib.quant_act_asym(_p(x), _act_dtype(x), M, K, _p(q), _p(prm), _stream()), "quant_act_asym")
    return q, prm


def weight_row_sums(W):
    """int32 [N]: the sum of each row of the int8 weights W [N, K]."""
    _dev(W)
    N, K = W.shape
    ws = _empty((N,), torch.int32, W)
    _check(lib.weight_row_sums(_p(W), N, K, _p(ws), _stream()), "weight_row_sums")
    return ws


def gemm_w8a8_asym(A, a_params, W, w_scale, w_sum, out_dtype=torch.bfloat16, out=None):
    """Asymmetric activations (quant_act_asym) times per-channel int8 weights."""
    _dev(A, a_params, W, w_scale, w_sum)
    M, K = A.shape
    N = W.shape[0]
    y = out if out is not None else _empty((M, N), out_dtype, A)
    _check(lib.gemm_w8a8_asym(_p(A), _p(a_params), _p(W), _p(w_scale), _p(w_sum), _p(y), _out_code(y.dtype),
                              M, N, K, _stream()), "gemm_w8a8_asym")
    return y

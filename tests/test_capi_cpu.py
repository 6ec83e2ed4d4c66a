"""The C ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before anything reaches a GPU (no GPU needed: every
call below fails its argument checks or is a no-op, so no kernel launches)."""

import ctypes
import os
import re

import pytest

import w8a8_int8_quantized_amd as w8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w8a8.h")

OK, ENULL, ESHAPE, EALIGN, EDTYPE, EWS, ECAP = 0, -1, -2, -3, -4, -6, -7
P16 = ctypes.c_void_p(1 << 20)        # a 16-byte aligned fake address (never dereferenced)
P4 = ctypes.c_void_p((1 << 20) + 4)   # 4-byte but not 16-byte aligned
NUL = ctypes.c_void_p(0)


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^(?:int|int64_t|const char\s*\*)\s*(\w+)\s*\(", text, flags=re.M))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 12
    cdll = ctypes.CDLL(w8.LIB_PATH)
    for n in names:
        assert hasattr(cdll, n), n
    assert names == set(w8._FUNCS), names ^ set(w8._FUNCS)


def test_version_and_status_strings():
    assert w8.lib.w8_abi_version() == 3
    for rc in (OK, ENULL, ESHAPE, EALIGN, EDTYPE, -5, EWS, ECAP):
        assert len(w8.lib.w8_status_string(rc)) > 0
    assert w8.lib.w8_status_string(99) == b"unknown status"


def test_quant_argument_checks():
    L = w8.lib
    for fn in (L.quant_act_group, L.quant_act_token):
        assert fn(P16, 0, 4, 100, P16, P16, NUL) == ESHAPE          # K % 128 != 0
        assert fn(P16, 0, -1, 128, P16, P16, NUL) == ESHAPE         # negative M
        assert fn(P16, 0, 4, 1 << 21, P16, P16, NUL) == ESHAPE      # K beyond 2^20
        assert fn(P16, 7, 4, 128, P16, P16, NUL) == EDTYPE          # unknown dtype
        assert fn(P16, w8.W8_FP32, 4, 128, P16, P16, NUL) == EDTYPE
        assert fn(NUL, 0, 4, 128, P16, P16, NUL) == ENULL
        assert fn(P16, 0, 4, 128, NUL, P16, NUL) == ENULL
        assert fn(P16, 0, 4, 128, P16, NUL, NUL) == ENULL
        assert fn(P4, 0, 4, 128, P16, P16, NUL) == EALIGN
        assert fn(P16, 0, 4, 128, P4, P16, NUL) == EALIGN
        assert fn(P16, 0, 0, 128, NUL, NUL, NUL) == OK              # M == 0: no-op
    assert L.quant_weight_block(P16, 4, 130, P16, P16, NUL) == ESHAPE
    assert L.quant_weight_block(P16, 4, 128, NUL, P16, NUL) == ENULL
    assert L.quant_weight_block(P16, 0, 128, NUL, NUL, NUL) == OK
    assert L.requant_fp8_to_int8_block(P16, P16, 4, 128, P16, P16, P4, NUL) == EALIGN
    assert L.requant_fp8_to_int8_block(P16, NUL, 4, 128, P16, P16, NUL, NUL) == ENULL
    assert L.requant_fp8_to_int8_block(P16, P16, 4, 64, P16, P16, NUL, NUL) == ESHAPE
    assert L.requant_fp8_to_int8_channel(P16, P16, -3, 128, P16, P16, NUL) == ESHAPE
    assert L.requant_fp8_to_int8_channel(P16, P16, 0, 128, P16, P16, NUL) == OK


def test_gemm_argument_checks():
    L = w8.lib
    assert L.gemm_w8a8_block(P16, P16, P16, P16, P16, w8.W8_I32, 4, 4, 128, NUL) == EDTYPE
    assert L.gemm_w8a8_block(P16, P16, P16, P16, P16, w8.W8_FP16, 4, 4, 128, NUL) == EDTYPE
    assert L.gemm_w8a8_block(P16, P16, P16, P16, P16, w8.W8_BF16, 4, 4, 100, NUL) == ESHAPE
    assert L.gemm_w8a8_block(P16, P16, P16, P16, P16, w8.W8_BF16, 4, 4, 0, NUL) == ESHAPE
    assert L.gemm_w8a8_block(P16, NUL, P16, P16, P16, w8.W8_BF16, 4, 4, 128, NUL) == ENULL
    assert L.gemm_w8a8_block(P16, P16, P4, P16, P16, w8.W8_BF16, 4, 4, 128, NUL) == EALIGN
    assert L.gemm_w8a8_block(NUL, NUL, NUL, NUL, NUL, w8.W8_BF16, 0, 4, 128, NUL) == OK
    assert L.gemm_w8a8_channel(P16, P16, P16, P16, P16, 9, 4, 4, 128, NUL) == EDTYPE
    assert L.gemm_w8a8_channel(P16, P16, P16, P16, P16, w8.W8_I32, 4, 4, 1 << 18, NUL) == ESHAPE
    assert L.gemm_w8a8_channel(P16, NUL, P16, P16, P16, w8.W8_FP32, 4, 4, 128, NUL) == ENULL
    assert L.gemm_w8a8_channel(P16, P16, P16, P16, NUL, w8.W8_FP32, 4, 4, 128, NUL) == ENULL
    assert L.gemm_w8a8_channel(NUL, NUL, NUL, NUL, NUL, w8.W8_FP32, 4, 0, 128, NUL) == OK
    # the allocation-free variant checks its arguments the same way
    fn = L.gemm_w8a8_channel_noalloc
    assert fn(P16, P16, P16, P16, P16, 9, 4, 4, 128, NUL) == EDTYPE
    assert fn(P16, P16, P16, P16, P16, w8.W8_I32, 4, 4, 1 << 18, NUL) == ESHAPE
    assert fn(P16, P16, P16, P16, P16, w8.W8_I32, 4, 4, 200, NUL) == ESHAPE
    assert fn(P16, NUL, P16, P16, P16, w8.W8_FP32, 4, 4, 128, NUL) == ENULL
    assert fn(P16, P16, P16, P16, NUL, w8.W8_FP32, 4, 4, 128, NUL) == ENULL
    assert fn(P4, P16, P16, P16, P16, w8.W8_I32, 4, 4, 128, NUL) == EALIGN
    assert fn(NUL, NUL, NUL, NUL, NUL, w8.W8_FP32, 0, 4, 128, NUL) == OK
    assert L.gemm_w8a8_block_partials(P16, P16, NUL, 4, 4, 128, NUL) == ENULL
    assert L.gemm_w8a8_block_partials(P16, P16, P16, 4, -4, 128, NUL) == ESHAPE
    assert L.gemm_w8a16_group(P16, P16, P16, P16, 4, 4, 96, NUL) == ESHAPE
    assert L.gemm_w8a16_group(P16, P16, P4, P4, 4, 4, 128, NUL) == EALIGN
    assert L.gemm_w8a16_group(P16, NUL, P16, P16, 4, 4, 128, NUL) == ENULL
    assert L.gemm_w8a8_block_grouped(P16, P16, P16, P16, P16, P16, w8.W8_BF16, 5000, 4, 4, 128, NUL) == ESHAPE
    assert L.gemm_w8a8_block_grouped(P16, P16, P16, P16, NUL, P16, w8.W8_BF16, 8, 4, 4, 128, NUL) == ENULL
    assert L.gemm_w8a8_block_grouped(P16, P16, P16, P16, P16, P16, w8.W8_I32, 8, 4, 4, 128, NUL) == EDTYPE
    assert L.gemm_w8a8_block_grouped(NUL, NUL, NUL, NUL, NUL, NUL, w8.W8_BF16, 8, 0, 4, 128, NUL) == OK
    # fused output quantisation: N must be whole 128-column groups
    assert L.gemm_w8a8_block_quant(P16, P16, P16, P16, P16, P16, 4, 100, 128, NUL) == ESHAPE
    assert L.gemm_w8a8_block_quant(P16, P16, P16, P16, P16, P16, 4, 128, 100, NUL) == ESHAPE
    assert L.gemm_w8a8_block_quant(P16, P16, P16, P16, P16, NUL, 4, 128, 128, NUL) == ENULL
    assert L.gemm_w8a8_block_quant(P16, P16, P16, P16, P4, P16, 4, 128, 128, NUL) == EALIGN
    assert L.gemm_w8a8_block_quant(NUL, NUL, NUL, NUL, NUL, NUL, 0, 128, 128, NUL) == OK
    assert L.gemm_w8a8_block_grouped_quant(P16, P16, P16, P16, P16, P16, P16, 8, 4, 200, 128, NUL) == ESHAPE
    assert L.gemm_w8a8_block_grouped_quant(P16, P16, P16, P16, P16, P16, P16, 5000, 4, 128, 128, NUL) == ESHAPE
    assert L.gemm_w8a8_block_grouped_quant(P16, P16, P16, P16, NUL, P16, P16, 8, 4, 128, 128, NUL) == ENULL
    assert L.gemm_w8a8_block_grouped_quant(NUL, NUL, NUL, NUL, NUL, NUL, NUL, 8, 0, 128, 128, NUL) == OK


def test_int4_argument_checks():
    L = w8.lib
    fn = L.quant_weight_int4_group
    assert fn(P16, 0, 4, 100, P16, P16, NUL) == ESHAPE          # K % 128 != 0
    assert fn(P16, 0, -1, 128, P16, P16, NUL) == ESHAPE
    assert fn(P16, w8.W8_FP32, 4, 128, P16, P16, NUL) == EDTYPE
    assert fn(NUL, 0, 4, 128, P16, P16, NUL) == ENULL
    assert fn(P16, 0, 4, 128, NUL, P16, NUL) == ENULL
    assert fn(P16, 0, 4, 128, P4, P16, NUL) == EALIGN
    assert fn(P16, 0, 0, 128, NUL, NUL, NUL) == OK              # N == 0: no-op
    g = L.gemm_w4a16_group
    assert g(P16, P16, P16, P16, 4, 4, 96, NUL) == ESHAPE
    assert g(P16, P16, P16, P16, 4, 4, 0, NUL) == ESHAPE
    assert g(P16, P4, P16, P16, 4, 4, 128, NUL) == EALIGN
    assert g(P16, P16, P4, P4, 4, 4, 128, NUL) == EALIGN
    assert g(P16, NUL, P16, P16, 4, 4, 128, NUL) == ENULL
    assert g(NUL, NUL, NUL, NUL, 0, 4, 128, NUL) == OK


def test_linear_workspace_bytes():
    L = w8.lib
    B, C = w8.W8_SCHEME_BLOCK, w8.W8_SCHEME_CHANNEL
    # int8 codes rounded up to 256 bytes, then fp32 scales: M x K/128 (block) or M (channel)
    assert L.linear_workspace_bytes(B, 3, 256) == 768 + 3 * 2 * 4
    assert L.linear_workspace_bytes(C, 3, 256) == 768 + 3 * 4
    assert L.linear_workspace_bytes(B, 1, 128) == 256 + 4
    assert L.linear_workspace_bytes(C, 5, 128) == 768 + 5 * 4
    assert L.linear_workspace_bytes(B, 4096, 7168) == 4096 * 7168 + 4096 * 56 * 4
    assert L.linear_workspace_bytes(B, 0, 128) == 0
    assert L.linear_workspace_bytes(2, 4, 128) == EDTYPE
    assert L.linear_workspace_bytes(B, 4, 100) == ESHAPE
    assert L.linear_workspace_bytes(C, -1, 128) == ESHAPE


def test_linear_argument_checks():
    L = w8.lib
    big = 1 << 30
    P256 = ctypes.c_void_p(1 << 20)
    P16o = ctypes.c_void_p((1 << 20) + 16)   # 16-byte but not 256-byte aligned
    for fn in (L.linear_w8a8_block, L.linear_w8a8_channel):
        assert fn(P16, w8.W8_FP32, P16, P16, P16, w8.W8_BF16, 4, 4, 128, P256, big, NUL) == EDTYPE
        assert fn(P16, 0, P16, P16, P16, w8.W8_I32, 4, 4, 128, P256, big, NUL) == EDTYPE
        assert fn(P16, 0, P16, P16, P16, w8.W8_BF16, 4, 4, 100, P256, big, NUL) == ESHAPE
        assert fn(P16, 0, P16, P16, P16, w8.W8_BF16, 4, 4, 0, P256, big, NUL) == ESHAPE
        assert fn(NUL, 0, P16, P16, P16, w8.W8_BF16, 4, 4, 128, P256, big, NUL) == ENULL
        assert fn(P16, 0, P16, NUL, P16, w8.W8_BF16, 4, 4, 128, P256, big, NUL) == ENULL
        assert fn(P16, 0, P16, P16, P16, w8.W8_BF16, 4, 4, 128, NUL, big, NUL) == ENULL
        assert fn(P4, 0, P16, P16, P16, w8.W8_BF16, 4, 4, 128, P256, big, NUL) == EALIGN
        assert fn(P16, 0, P16, P16, P16, w8.W8_BF16, 4, 4, 128, P16o, big, NUL) == EALIGN
        assert fn(P16, 0, P16, P16, P16, w8.W8_BF16, 4, 4, 128, P256, 256, NUL) == EWS
        assert fn(NUL, 0, NUL, NUL, NUL, w8.W8_BF16, 0, 4, 128, NUL, 0, NUL) == OK     # M == 0: no-op
        assert fn(NUL, 0, NUL, NUL, NUL, w8.W8_BF16, 4, 0, 128, NUL, 0, NUL) == OK     # N == 0: no-op
    # the channel-wise GEMM's K limit
    assert L.linear_w8a8_channel(P16, 0, P16, P16, P16, w8.W8_BF16, 4, 4, 1 << 18, P256, 1 << 40, NUL) == ESHAPE
    # one byte short of the required size
    need = L.linear_workspace_bytes(w8.W8_SCHEME_BLOCK, 4, 128)
    assert need == 512 + 16
    assert L.linear_w8a8_block(P16, 0, P16, P16, P16, w8.W8_BF16, 4, 4, 128, P256, need - 1, NUL) == EWS


def test_asym_argument_checks():
    L = w8.lib
    assert L.quant_act_asym(P16, w8.W8_FP32, 4, 128, P16, P16, NUL) == EDTYPE
    assert L.quant_act_asym(P16, 0, 4, 100, P16, P16, NUL) == ESHAPE
    assert L.quant_act_asym(P16, 0, 4, 128, P16, NUL, NUL) == ENULL
    assert L.quant_act_asym(P4, 0, 4, 128, P16, P16, NUL) == EALIGN
    assert L.quant_act_asym(NUL, 0, 0, 128, NUL, NUL, NUL) == OK
    assert L.weight_row_sums(P16, 4, 1 << 17, P16, NUL) == ESHAPE          # K beyond 2^16
    assert L.weight_row_sums(P16, 4, 0, P16, NUL) == ESHAPE
    assert L.weight_row_sums(P16, 4, 128, NUL, NUL) == ENULL
    assert L.weight_row_sums(NUL, 0, 128, NUL, NUL) == OK
    assert L.gemm_w8a8_asym(P16, P16, P16, P16, P16, P16, w8.W8_I32, 4, 4, 128, NUL) == EDTYPE
    assert L.gemm_w8a8_asym(P16, P16, P16, P16, P16, P16, w8.W8_BF16, 4, 4, 1 << 17, NUL) == ESHAPE
    assert L.gemm_w8a8_asym(P16, NUL, P16, P16, P16, P16, w8.W8_BF16, 4, 4, 128, NUL) == ENULL
    assert L.gemm_w8a8_asym(P16, P16, P16, P16, NUL, P16, w8.W8_BF16, 4, 4, 128, NUL) == ENULL
    assert L.gemm_w8a8_asym(P4, P16, P16, P16, P16, P16, w8.W8_FP32, 4, 4, 128, NUL) == EALIGN   # misaligned A
    assert L.gemm_w8a8_asym(NUL, NUL, NUL, NUL, NUL, NUL, w8.W8_BF16, 0, 4, 128, NUL) == OK


def test_python_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(4, 128, dtype=torch.bfloat16)
    with pytest.raises(w8.W8Error):
        w8.quant_act_group(x)

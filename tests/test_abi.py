"""The C-ABI library loads, exports every symbol include/cubic.h declares, and
rejects invalid arguments on the host before any GPU call (runs without a GPU)."""
import ctypes
import os
import re

import pytest

import dequant_gemm_amd as cq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cubic.h")

OK, ERR_NULL, ERR_SHAPE, ERR_BITS, ERR_GROUP, ERR_ALIGN, ERR_RANGE, ERR_WS, ERR_HIP = (
    0, -1, -2, -3, -4, -5, -6, -7, -8)


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_matches_binding_list():
    assert _declared() == sorted(cq.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = cq.load_library()
    for name in _declared():
        assert hasattr(lib, name), name


def test_size_helpers_match_storage_formula():
    # B + 64/G bits per weight (CubicQuant article, storage section)
    assert cq.cubic_code_bytes(6144, 7168, 2) == 11_010_048
    assert cq.cubic_storage_bytes(6144, 7168, 2, 512) == 11_010_048 + 8 * 6144 * 14
    assert cq.cubic_storage_bytes(1, 512, 3, 512) / 512 == 0.390625
    assert cq.cubic_code_bytes(3, 5, 3) == 0          # not a whole number of bytes
    assert cq.cubic_code_bytes(4, 64, 9) == 0
    assert cq.cubic_storage_bytes(4, 300, 2, 128) == 0


def test_workspace_sizes():
    assert cq.cubic_gemm_a16_workspace_bytes(1, 7168) == 0
    assert cq.cubic_gemm_a16_workspace_bytes(4, 7168) == 0
    assert cq.cubic_gemm_a16_workspace_bytes(8, 7168) >= 8 * 7168 * 2 + 8 * 4
    # one 32-byte record per expert and the grouped pair ids; no activation copy
    assert cq.cubic_moe_workspace_bytes(64, 16, 896) >= 32 * 896 + 4 * 1024
    # 256-byte aligned parts: header, 896 records of 32 bytes, 1024 pair ids
    assert cq.cubic_moe_workspace_bytes(64, 16, 896) == 256 + 28672 + 4096
    assert cq.cubic_moe_workspace_bytes(64, 0, 896) == 0
    lib = cq.load_library()
    assert lib.cubic_status_string(ERR_WS) == b"workspace missing or too small"
    assert lib.cubic_version().startswith(b"cubic")


def test_linear_mode_rule_and_workspace():
    # Dynamic A8 for 2- and 3-bit codes from 256 rows on (the measured crossover), A16 otherwise
    A16, A8 = cq.MODE_A16, cq.MODE_A8
    assert cq.cubic_linear_mode(1, 6144, 7168, 2, 512) == A16
    assert cq.cubic_linear_mode(127, 6144, 7168, 2, 512) == A16
    assert cq.cubic_linear_mode(128, 6144, 7168, 2, 512) == A8
    assert cq.cubic_linear_mode(4096, 6144, 7168, 3, 256) == A8
    assert cq.cubic_linear_mode(4096, 6144, 7168, 4, 128) == A16
    assert cq.cubic_linear_mode(256, 7168, 3072, 5, 128) == A16
    assert cq.cubic_linear_mode(4096, 256, 4096, 2, 2048) == A16     # group beyond the A8 kernel
    assert cq.cubic_linear_mode(0, 6144, 7168, 2, 512) == A16
    # the small-batch window: 8..16 rows of long rows (K >= 4096), 2- and 3-bit codes
    assert cq.cubic_linear_mode(8, 6144, 7168, 2, 512) == A8
    assert cq.cubic_linear_mode(16, 6144, 7168, 3, 256) == A8
    assert cq.cubic_linear_mode(7, 6144, 7168, 2, 512) == A16
    assert cq.cubic_linear_mode(17, 6144, 7168, 2, 512) == A16
    assert cq.cubic_linear_mode(12, 7168, 3072, 2, 512) == A16
    assert cq.cubic_linear_mode(12, 6144, 7168, 4, 128) == A16
    # the larger of the A16 workspace and the A8 staging (xq, then x_scale, 256-aligned)
    assert cq.cubic_linear_workspace_bytes(1, 7168) == 7168 + 256
    assert cq.cubic_linear_workspace_bytes(4096, 7168) == max(
        cq.cubic_gemm_a16_workspace_bytes(4096, 7168), 4096 * 7168 + 4096 * 4)
    assert cq.cubic_linear_workspace_bytes(0, 7168) == 0


def test_linear_validation_before_launch():
    lib = cq.load_library()
    p16, p8 = ctypes.c_void_p(16), ctypes.c_void_p(8)
    w8 = _w(N=256, K=512, bits=3, group=128)           # M = 256 takes the A8 route
    need = lib.cubic_linear_workspace_bytes(256, 512)
    a8_need = 256 * 512 + 256 * 4                      # the A8 staging this route checks
    assert lib.cubic_linear(p16, 256, ctypes.byref(w8), p16, p16, a8_need - 1, None) == ERR_WS
    assert lib.cubic_linear(p16, 256, ctypes.byref(w8), p16, None, 0, None) == ERR_WS
    assert lib.cubic_linear(None, 256, ctypes.byref(w8), p16, p16, need, None) == ERR_NULL
    assert lib.cubic_linear(p8, 256, ctypes.byref(w8), p16, p16, need, None) == ERR_ALIGN
    assert lib.cubic_linear(p16, 256, ctypes.byref(w8), p16, p8, need, None) == ERR_ALIGN
    assert lib.cubic_linear(p16, -1, ctypes.byref(w8), p16, p16, need, None) == ERR_SHAPE
    assert lib.cubic_linear(p16, 256, ctypes.byref(_w(bits=1)), p16, p16, need, None) == ERR_BITS
    assert lib.cubic_linear(p16, 0, ctypes.byref(w8), p16, None, 0, None) == OK   # no-op
    # the A16 route validates as cubic_gemm_a16 does
    assert lib.cubic_linear(p16, 8, ctypes.byref(w8), p16, None, 0, None) == ERR_WS


def test_encode_validation_before_launch():
    lib = cq.load_library()
    p16, p8 = ctypes.c_void_p(16), ctypes.c_void_p(8)
    assert lib.cubic_encode(p16, 4, 512, 1, 128, p16, p16, p16, None) == ERR_BITS
    assert lib.cubic_encode(p16, 4, 512, 3, 64, p16, p16, p16, None) == ERR_GROUP
    assert lib.cubic_encode(p16, 4, 384, 3, 256, p16, p16, p16, None) == ERR_GROUP
    assert lib.cubic_encode(p16, -1, 512, 3, 128, p16, p16, p16, None) == ERR_SHAPE
    assert lib.cubic_encode(None, 4, 512, 3, 128, p16, p16, p16, None) == ERR_NULL
    assert lib.cubic_encode(p16, 4, 512, 3, 128, p16, p16, None, None) == ERR_NULL
    assert lib.cubic_encode(p8, 4, 512, 3, 128, p16, p16, p16, None) == ERR_ALIGN
    assert lib.cubic_encode(p16, 0, 512, 3, 128, None, None, None, None) == OK    # no-op


def test_fit_validation_before_launch():
    lib = cq.load_library()
    p16, p8 = ctypes.c_void_p(16), ctypes.c_void_p(8)
    assert lib.cubic_fit(p16, 4, 512, 9, 128, p16, p16, p16, None, None) == ERR_BITS
    assert lib.cubic_fit(p16, 4, 512, 3, 64, p16, p16, p16, None, None) == ERR_GROUP
    assert lib.cubic_fit(p16, 4, 4096, 3, 4096, p16, p16, p16, None, None) == ERR_GROUP   # above 2048
    assert lib.cubic_fit(p16, 4, 384, 3, 256, p16, p16, p16, None, None) == ERR_GROUP
    assert lib.cubic_fit(p16, -1, 512, 3, 128, p16, p16, p16, None, None) == ERR_SHAPE
    assert lib.cubic_fit(None, 4, 512, 3, 128, p16, p16, p16, None, None) == ERR_NULL
    assert lib.cubic_fit(p16, 4, 512, 3, 128, p16, None, p16, None, None) == ERR_NULL
    assert lib.cubic_fit(p8, 4, 512, 3, 128, p16, p16, p16, None, None) == ERR_ALIGN
    assert lib.cubic_fit(p16, 4, 512, 3, 128, p16, p16, p16, ctypes.c_void_p(18), None) == ERR_ALIGN
    assert lib.cubic_fit(p16, 0, 512, 3, 128, None, None, None, None, None) == OK        # no-op


def test_moe_mlp_validation_before_launch():
    lib = cq.load_library()
    p16, p8 = ctypes.c_void_p(16), ctypes.c_void_p(8)
    gu = _w(N=1024, K=512, bits=2, group=256)         # H = 512, I = 512
    dn = _w(N=512, K=512, bits=2, group=256)
    need = lib.cubic_moe_mlp_workspace_bytes(4, 2, 8, 512, 512)
    assert need >= 4 * 2 * (1024 * 4 + 512 * 2 + 512 * 4)
    assert lib.cubic_moe_mlp(p16, 4, p16, p16, 2, ctypes.byref(gu), ctypes.byref(dn), 8, p16, p16, need - 1,
                             None) == ERR_WS
    bad = _w(N=500, K=512, bits=2, group=256)         # gate_up rows != 2 x down K
    assert lib.cubic_moe_mlp(p16, 4, p16, p16, 2, ctypes.byref(bad), ctypes.byref(dn), 8, p16, p16, need,
                             None) == ERR_SHAPE
    assert lib.cubic_moe_mlp(p16, 4, None, p16, 2, ctypes.byref(gu), ctypes.byref(dn), 8, p16, p16, need,
                             None) == ERR_NULL
    assert lib.cubic_moe_mlp(p16, 4, p16, p8, 2, ctypes.byref(gu), ctypes.byref(dn), 8, p16, p16, need,
                             None) == ERR_ALIGN
    assert lib.cubic_moe_mlp(p16, 0, p16, p16, 2, ctypes.byref(gu), ctypes.byref(dn), 8, p16, p16, need,
                             None) == OK                                       # no-op


def _w(N=256, K=512, bits=3, group=128, codes=16, scales=16, shapes=16):
    return cq._CWeight(codes, scales, shapes, N, K, bits, group)


@pytest.mark.parametrize("kw,status", [
    (dict(bits=1), ERR_BITS), (dict(bits=9), ERR_BITS),
    (dict(group=64), ERR_GROUP), (dict(group=256, K=384), ERR_GROUP), (dict(group=0), ERR_GROUP),
    (dict(N=-1), ERR_SHAPE), (dict(codes=0), ERR_NULL), (dict(scales=8), ERR_ALIGN),
])
def test_weight_validation_before_launch(kw, status):
    lib = cq.load_library()
    w = _w(**kw)
    p16 = ctypes.c_void_p(16)
    assert lib.cubic_gemm_a16(p16, 4, ctypes.byref(w), p16, None, 0, None) == status
    assert lib.cubic_dequant(ctypes.byref(w), p16, None) == status
    assert lib.cubic_gemm_a8(p16, p16, 4, ctypes.byref(w), p16, None) == status


def test_call_argument_validation_before_launch():
    lib = cq.load_library()
    w = _w()
    p16, p8 = ctypes.c_void_p(16), ctypes.c_void_p(8)
    assert lib.cubic_gemm_a16(None, 4, ctypes.byref(w), p16, None, 0, None) == ERR_NULL
    assert lib.cubic_gemm_a16(p8, 4, ctypes.byref(w), p16, None, 0, None) == ERR_ALIGN
    assert lib.cubic_gemm_a16(p16, -1, ctypes.byref(w), p16, None, 0, None) == ERR_SHAPE
    assert lib.cubic_gemm_a16(p16, 0, ctypes.byref(w), p16, None, 0, None) == OK   # no-op
    assert lib.cubic_gemm_a16(p16, 8, ctypes.byref(w), p16, None, 0, None) == ERR_WS
    assert lib.cubic_gemm_a16(p16, 8, ctypes.byref(w), p16, p16, 10, None) == ERR_WS
    assert lib.cubic_gemm_a16(None, 4, None, p16, None, 0, None) == ERR_NULL
    w_big_group = _w(group=2048, K=4096)
    assert lib.cubic_gemm_a8(p16, p16, 4, ctypes.byref(w_big_group), p16, None) == ERR_GROUP
    assert lib.act_quant_int8_per_token(p16, 4, 100, p16, p16, None) == ERR_SHAPE
    assert lib.act_quant_int8_per_token(None, 4, 128, p16, p16, None) == ERR_NULL
    assert lib.act_quant_int8_per_token(p16, 0, 128, p16, p16, None) == OK
    assert lib.cubic_pack(p16, 4, 48, 3, p16, None) == ERR_SHAPE
    assert lib.cubic_pack(p16, 4, 64, 9, p16, None) == ERR_BITS
    assert lib.cubic_unpack(None, 4, 64, 3, p16, None) == ERR_NULL
    assert lib.cubic_unpack(p16, 4, 64, 3, p8, None) == ERR_ALIGN
    need = lib.cubic_moe_workspace_bytes(4, 2, 8)
    assert lib.cubic_moe_grouped_gemm(p16, 4, p16, 2, ctypes.byref(w), 8, p16, p16, need - 1, None) == ERR_WS
    assert lib.cubic_moe_grouped_gemm(p16, 4, p16, 0, ctypes.byref(w), 8, p16, p16, need, None) == ERR_SHAPE
    assert lib.cubic_moe_grouped_gemm(p16, 4, None, 2, ctypes.byref(w), 8, p16, p16, need, None) == ERR_NULL


def test_dtype_codes_rejected_before_launch():
    """Element-type codes: inputs bf16 (1) or fp16 (2), outputs fp32 (0) or bf16 (1)."""
    lib = cq.load_library()
    w = _w()
    p16 = ctypes.c_void_p(16)
    ERR_DTYPE = -9
    for xd, yd in ((0, 0), (3, 0), (1, 2), (1, -1), (-1, 1)):
        assert lib.cubic_gemm_a16_ex(p16, xd, 4, ctypes.byref(w), p16, yd, None, 0, None) == ERR_DTYPE
        assert lib.cubic_moe_grouped_gemm_ex(p16, xd, 4, p16, 2, ctypes.byref(w), 8, p16, yd, p16, 1 << 20,
                                             None) == ERR_DTYPE
    for xd in (0, 3):
        assert lib.act_quant_int8_per_token_ex(p16, xd, 4, 128, p16, p16, None) == ERR_DTYPE
    for yd in (2, 5):
        assert lib.cubic_gemm_a8_ex(p16, p16, 4, ctypes.byref(w), p16, yd, None) == ERR_DTYPE
    assert lib.cubic_gemm_a16_ex(p16, 2, 0, ctypes.byref(w), p16, 1, None, 0, None) == OK   # no-op
    assert "type" in lib.cubic_status_string(ERR_DTYPE).decode()


def test_moe_a8_validation_before_launch():
    lib = cq.load_library()
    p16 = ctypes.c_void_p(16)
    need = lib.cubic_moe_workspace_bytes(4, 2, 8)
    w = _w()
    call = lambda w, T=4, topk=2, yd=0, ws=need, ids=p16: lib.cubic_moe_grouped_gemm_a8(
        p16, p16, T, ids, topk, ctypes.byref(w), 8, p16, yd, p16, ws, None)
    assert call(w, yd=2) == -9                       # fp16 output: unsupported type
    assert call(_w(group=2048, K=4096)) == ERR_GROUP
    assert call(w, ws=need - 1) == ERR_WS
    assert call(w, topk=0) == ERR_SHAPE
    assert call(w, T=-1) == ERR_SHAPE
    assert call(w, T=0) == OK                         # no-op
    assert call(w, ids=None) == ERR_NULL
    assert call(_w(bits=9)) == ERR_BITS
    assert lib.cubic_moe_grouped_gemm_a8(ctypes.c_void_p(8), p16, 4, p16, 2, ctypes.byref(w), 8, p16, 0, p16,
                                         need, None) == ERR_ALIGN


def test_moe_mlp_a8_validation_and_workspace():
    lib = cq.load_library()
    p16 = ctypes.c_void_p(16)
    T, topk, E, H, I = 3, 2, 4, 256, 128
    need = lib.cubic_moe_mlp_a8_workspace_bytes(T, topk, E, H, I)
    up = lambda n: -(-n // 256) * 256
    P = T * topk
    assert need == (lib.cubic_moe_workspace_bytes(T, topk, E) + up(T * H) + up(T * 4) + up(P * 2 * I * 4)
                    + up(P * I * 2) + up(P * I) + up(P * 4) + up(P * H * 4))
    gu, dn = _w(N=2 * I, K=H), _w(N=H, K=I)
    call = lambda gu, dn, ws=need: lib.cubic_moe_mlp_a8(p16, T, p16, p16, topk, ctypes.byref(gu), ctypes.byref(dn),
                                                        E, p16, p16, ws, None)
    assert call(gu, dn, ws=need - 1) == ERR_WS
    assert call(gu, _w(N=H + 1, K=I)) == ERR_SHAPE
    assert call(_w(N=2 * I, K=2048, group=2048), _w(N=2048, K=I)) == ERR_GROUP


def test_product_path_has_no_oracle_dependency():
    """The package never imports the oracle; the library is the only compute."""
    pkg = os.path.join(ROOT, "dequant_gemm_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "import oracle" not in text and "from oracle" not in text, f

"""Thin Python binding of libcubic.so (the CubicQuant dequant-GEMM for gfx950).

Argument marshalling only: every function takes torch tensors, checks their
dtype, device and contiguity, allocates outputs (and workspaces) with torch, and
calls the C function of the same name on torch's current HIP stream. All the
arithmetic runs in the library's HIP kernels; there is no CPU fallback, and a
missing library raises immediately.

Weight layout (see include/cubic.h): ``codes`` uint8 [N][K*bits/8] bit stream,
``scales`` float32 [N][K/group], ``shapes`` int16 [N][K/group][2] holding the
fp16 bit patterns of (a, b).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

__all__ = [
    "CubicError", "CubicWeight", "library_path", "load_library",
    "cubic_code_bytes", "cubic_storage_bytes", "cubic_pack", "cubic_unpack",
    "cubic_dequant", "cubic_encode", "cubic_fit", "cubic_gemm_a16", "cubic_gemm_a16_workspace_bytes",
    "act_quant_int8_per_token", "cubic_gemm_a8", "cubic_linear_mode", "cubic_linear_workspace_bytes",
    "cubic_linear", "MODE_A16", "MODE_A8", "cubic_moe_workspace_bytes", "cubic_moe_grouped_gemm",
    "cubic_moe_grouped_gemm_static_max_bytes", "cubic_moe_grouped_gemm_static",
    "cubic_moe_mlp_workspace_bytes", "cubic_moe_mlp", "EXPORTED_SYMBOLS", "cubic_moe_grouped_gemm_a8",
    "cubic_moe_mlp_a8_workspace_bytes", "cubic_moe_mlp_a8",
    "DTYPE_F32", "DTYPE_BF16", "DTYPE_F16",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
EXPORTED_SYMBOLS = [
    "cubic_code_bytes", "cubic_storage_bytes", "cubic_status_string", "cubic_version",
    "cubic_pack", "cubic_unpack", "cubic_dequant", "cubic_encode", "cubic_fit", "cubic_gemm_a16_workspace_bytes",
    "cubic_gemm_a16", "act_quant_int8_per_token", "cubic_gemm_a8", "cubic_linear_mode",
    "cubic_linear_workspace_bytes", "cubic_linear", "cubic_moe_workspace_bytes",
    "cubic_moe_grouped_gemm", "cubic_moe_grouped_gemm_static_max_bytes", "cubic_moe_grouped_gemm_static",
    "cubic_moe_mlp_workspace_bytes", "cubic_moe_mlp",
    "cubic_gemm_a16_ex", "act_quant_int8_per_token_ex", "cubic_gemm_a8_ex", "cubic_moe_grouped_gemm_ex",
    "cubic_moe_grouped_gemm_a8", "cubic_moe_mlp_a8_workspace_bytes", "cubic_moe_mlp_a8",
]
MODE_A16, MODE_A8 = 0, 1          # cubic_linear_mode results


class CubicError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {_status_string(status)} ({status})")
        self.status = status


class _CWeight(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("shapes", ctypes.c_void_p), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("bits", ctypes.c_int32), ("group", ctypes.c_int32)]


def library_path() -> str:
    return os.environ.get("CUBIC_LIBRARY", os.path.join(_PKG, "lib", "libcubic.so"))


_lib = None


def load_library():
    """Load libcubic.so (built by dequant_gemm_amd.build); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"libcubic.so not found at {path}; run `python -m dequant_gemm_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    wp = ctypes.POINTER(_CWeight)
    sigs = {
        "cubic_code_bytes": (sz, [i64, i64, i32]),
        "cubic_storage_bytes": (sz, [i64, i64, i32, i32]),
        "cubic_status_string": (ctypes.c_char_p, [i32]),
        "cubic_version": (ctypes.c_char_p, []),
        "cubic_pack": (i32, [vp, i64, i64, i32, vp, vp]),
        "cubic_unpack": (i32, [vp, i64, i64, i32, vp, vp]),
        "cubic_dequant": (i32, [wp, vp, vp]),
        "cubic_encode": (i32, [vp, i64, i64, i32, i32, vp, vp, vp, vp]),
        "cubic_fit": (i32, [vp, i64, i64, i32, i32, vp, vp, vp, vp, vp]),
        "cubic_gemm_a16_workspace_bytes": (sz, [i64, i64]),
        "cubic_gemm_a16": (i32, [vp, i64, wp, vp, vp, sz, vp]),
        "act_quant_int8_per_token": (i32, [vp, i64, i64, vp, vp, vp]),
        "cubic_gemm_a8": (i32, [vp, vp, i64, wp, vp, vp]),
        "cubic_linear_mode": (i32, [i64, i64, i64, i32, i32]),
        "cubic_linear_workspace_bytes": (sz, [i64, i64]),
        "cubic_linear": (i32, [vp, i64, wp, vp, vp, sz, vp]),
        "cubic_moe_workspace_bytes": (sz, [i64, i32, i32]),
        "cubic_moe_grouped_gemm": (i32, [vp, i64, vp, i32, wp, i32, vp, vp, sz, vp]),
        "cubic_moe_grouped_gemm_static_max_bytes": (sz, []),
        "cubic_gemm_a16_ex": (i32, [vp, i32, i64, wp, vp, i32, vp, sz, vp]),
        "act_quant_int8_per_token_ex": (i32, [vp, i32, i64, i64, vp, vp, vp]),
        "cubic_gemm_a8_ex": (i32, [vp, vp, i64, wp, vp, i32, vp]),
        "cubic_moe_grouped_gemm_ex": (i32, [vp, i32, i64, vp, i32, wp, i32, vp, i32, vp, sz, vp]),
        "cubic_moe_grouped_gemm_static": (i32, [vp, i64, vp, i32, wp, i32, vp, vp]),
        "cubic_moe_grouped_gemm_a8": (i32, [vp, vp, i64, vp, i32, wp, i32, vp, i32, vp, sz, vp]),
        "cubic_moe_mlp_workspace_bytes": (sz, [i64, i32, i32, i64, i64]),
        "cubic_moe_mlp": (i32, [vp, i64, vp, vp, i32, wp, wp, i32, vp, vp, sz, vp]),
        "cubic_moe_mlp_a8_workspace_bytes": (sz, [i64, i32, i32, i64, i64]),
        "cubic_moe_mlp_a8": (i32, [vp, i64, vp, vp, i32, wp, wp, i32, vp, vp, sz, vp]),
    }
    for name, (res, args) in sigs.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _status_string(status: int) -> str:
    try:
        return load_library().cubic_status_string(status).decode()
    except Exception:  # pragma: no cover
        return "status"


def _check(status: int, what: str):
    if status != 0:
        raise CubicError(status, what)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t: torch.Tensor, dtype, name: str):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


@dataclass
class CubicWeight:
    """Device buffers of one Cubic weight (or of E experts back to back)."""
    codes: torch.Tensor     # uint8, N*K*bits/8 bytes per matrix
    scales: torch.Tensor    # float32, N*K/group per matrix
    shapes: torch.Tensor    # int16 (fp16 bit patterns), 2*N*K/group per matrix
    N: int
    K: int
    bits: int
    group: int

    def c_struct(self) -> _CWeight:
        _need(self.codes, torch.uint8, "codes")
        _need(self.scales, torch.float32, "scales")
        _need(self.shapes, torch.int16, "shapes")
        return _CWeight(self.codes.data_ptr(), self.scales.data_ptr(), self.shapes.data_ptr(),
                        self.N, self.K, self.bits, self.group)


def cubic_code_bytes(N: int, K: int, bits: int) -> int:
    return int(load_library().cubic_code_bytes(N, K, bits))


def cubic_storage_bytes(N: int, K: int, bits: int, group: int) -> int:
    return int(load_library().cubic_storage_bytes(N, K, bits, group))


def cubic_pack(codes: torch.Tensor, bits: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """int8 codes [N][K] -> uint8 bit stream [N][K*bits/8]."""
    _need(codes, torch.int8, "codes")
    N, K = codes.shape
    if out is None:
        out = torch.empty((N, K * bits // 8), dtype=torch.uint8, device=codes.device)
    _check(load_library().cubic_pack(_ptr(codes), N, K, bits, _ptr(out), _stream(codes)), "cubic_pack")
    return out


def cubic_unpack(packed: torch.Tensor, N: int, K: int, bits: int,
                 out: torch.Tensor | None = None) -> torch.Tensor:
    _need(packed, torch.uint8, "packed")
    if out is None:
        out = torch.empty((N, K), dtype=torch.int8, device=packed.device)
    _check(load_library().cubic_unpack(_ptr(packed), N, K, bits, _ptr(out), _stream(packed)),
           "cubic_unpack")
    return out


def cubic_dequant(w: CubicWeight, out: torch.Tensor | None = None) -> torch.Tensor:
    cw = w.c_struct()
    if out is None:
        out = torch.empty((w.N, w.K), dtype=torch.float32, device=w.codes.device)
    _check(load_library().cubic_dequant(ctypes.byref(cw), _ptr(out), _stream(w.codes)),
           "cubic_dequant")
    return out


def cubic_encode(w: torch.Tensor, scales: torch.Tensor, shapes: torch.Tensor, bits: int, group: int,
                 out: torch.Tensor | None = None) -> torch.Tensor:
    """fp32 weights [N][K] -> int8 codes [N][K] of the nearest levels (pack with cubic_pack)."""
    _need(w, torch.float32, "w")
    N, K = w.shape
    if out is None:
        out = torch.empty((N, K), dtype=torch.int8, device=w.device)
    _check(load_library().cubic_encode(_ptr(w), N, K, bits, group, _ptr(scales), _ptr(shapes), _ptr(out),
                                        _stream(w)), "cubic_encode")
    return out


def cubic_fit(w: torch.Tensor, bits: int, group: int, with_loss: bool = False):
    """Fit every group of fp32 weights w [N][K]: returns (codes int8 [N][K], scales
    fp32 [N][K/group], shapes int16 [N][K/group][2] holding fp16 a, b bits), plus the
    per-group loss (fp32) when with_loss."""
    _need(w, torch.float32, "w")
    N, K = w.shape
    G = K // group if group > 0 else 0
    codes = torch.empty((N, K), dtype=torch.int8, device=w.device)
    scales = torch.empty((N, G), dtype=torch.float32, device=w.device)
    shapes = torch.empty((N, G, 2), dtype=torch.int16, device=w.device)
    loss = torch.empty((N, G), dtype=torch.float32, device=w.device) if with_loss else None
    _check(load_library().cubic_fit(_ptr(w), N, K, bits, group, _ptr(codes), _ptr(scales), _ptr(shapes),
                                    _ptr(loss) if loss is not None else None, _stream(w)), "cubic_fit")
    return (codes, scales, shapes, loss) if with_loss else (codes, scales, shapes)


def cubic_gemm_a16_workspace_bytes(M: int, K: int) -> int:
    return int(load_library().cubic_gemm_a16_workspace_bytes(M, K))


DTYPE_F32, DTYPE_BF16, DTYPE_F16 = 0, 1, 2          # element types of the _ex entry points
_DT_IN = {torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_F16}
_DT_OUT = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}


def _in_dtype(x: torch.Tensor, name: str) -> int:
    if x.dtype not in _DT_IN:
        raise TypeError(f"{name}: expected bfloat16 or float16, got {x.dtype}")
    _need(x, x.dtype, name)
    return _DT_IN[x.dtype]


def _out_dtype(out_dtype) -> int:
    if out_dtype not in _DT_OUT:
        raise TypeError(f"out_dtype: expected float32 or bfloat16, got {out_dtype}")
    return _DT_OUT[out_dtype]


def cubic_gemm_a16(x: torch.Tensor, w: CubicWeight, out: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None, out_dtype=torch.float32) -> torch.Tensor:
    """y[M][N] = x[M][K] * W^T; x bf16 (cubic_gemm_a16) or fp16, y fp32 or bf16
    (cubic_gemm_a16_ex)."""
    xd, yd = _in_dtype(x, "x"), _out_dtype(out_dtype)
    M = x.shape[0]
    cw = w.c_struct()
    if out is None:
        out = torch.empty((M, w.N), dtype=out_dtype, device=x.device)
    elif out.dtype != out_dtype:
        raise TypeError(f"out: expected {out_dtype}, got {out.dtype}")
    need = cubic_gemm_a16_workspace_bytes(M, w.K)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = workspace.numel() if workspace is not None else 0
    lib = load_library()
    if xd == DTYPE_BF16 and yd == DTYPE_F32:
        st = lib.cubic_gemm_a16(_ptr(x), M, ctypes.byref(cw), _ptr(out), _ptr(workspace), ws_bytes, _stream(x))
    else:
        st = lib.cubic_gemm_a16_ex(_ptr(x), xd, M, ctypes.byref(cw), _ptr(out), yd, _ptr(workspace), ws_bytes,
                                   _stream(x))
    _check(st, "cubic_gemm_a16")
    return out


def act_quant_int8_per_token(x: torch.Tensor, xq: torch.Tensor | None = None,
                             x_scale: torch.Tensor | None = None):
    """bf16 or fp16 [M][K] -> (int8 [M][K], fp32 [M])."""
    xd = _in_dtype(x, "x")
    M, K = x.shape
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if x_scale is None:
        x_scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    lib = load_library()
    if xd == DTYPE_BF16:
        st = lib.act_quant_int8_per_token(_ptr(x), M, K, _ptr(xq), _ptr(x_scale), _stream(x))
    else:
        st = lib.act_quant_int8_per_token_ex(_ptr(x), xd, M, K, _ptr(xq), _ptr(x_scale), _stream(x))
    _check(st, "act_quant_int8_per_token")
    return xq, x_scale


def cubic_gemm_a8(xq: torch.Tensor, x_scale: torch.Tensor, w: CubicWeight,
                  out: torch.Tensor | None = None, out_dtype=torch.float32) -> torch.Tensor:
    _need(xq, torch.int8, "xq")
    _need(x_scale, torch.float32, "x_scale")
    yd = _out_dtype(out_dtype)
    M = xq.shape[0]
    cw = w.c_struct()
    if out is None:
        out = torch.empty((M, w.N), dtype=out_dtype, device=xq.device)
    elif out.dtype != out_dtype:
        raise TypeError(f"out: expected {out_dtype}, got {out.dtype}")
    lib = load_library()
    if yd == DTYPE_F32:
        st = lib.cubic_gemm_a8(_ptr(xq), _ptr(x_scale), M, ctypes.byref(cw), _ptr(out), _stream(xq))
    else:
        st = lib.cubic_gemm_a8_ex(_ptr(xq), _ptr(x_scale), M, ctypes.byref(cw), _ptr(out), yd, _stream(xq))
    _check(st, "cubic_gemm_a8")
    return out


def cubic_linear_mode(M: int, N: int, K: int, bits: int, group: int) -> int:
    """MODE_A16 or MODE_A8: the activation mode cubic_linear takes for this shape."""
    return int(load_library().cubic_linear_mode(M, N, K, bits, group))


def cubic_linear_workspace_bytes(M: int, K: int) -> int:
    return int(load_library().cubic_linear_workspace_bytes(M, K))


def cubic_linear(x: torch.Tensor, w: CubicWeight, out: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y[M][N] (fp32) from bf16 x[M][K] in the mode of cubic_linear_mode (A16, or
    the per-token INT8 quantiser followed by the A8 product)."""
    _need(x, torch.bfloat16, "x")
    M = x.shape[0]
    cw = w.c_struct()
    if out is None:
        out = torch.empty((M, w.N), dtype=torch.float32, device=x.device)
    need = cubic_linear_workspace_bytes(M, w.K)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = workspace.numel() if workspace is not None else 0
    _check(load_library().cubic_linear(_ptr(x), M, ctypes.byref(cw), _ptr(out), _ptr(workspace),
                                        ws_bytes, _stream(x)), "cubic_linear")
    return out


def cubic_moe_workspace_bytes(T: int, topk: int, E: int) -> int:
    return int(load_library().cubic_moe_workspace_bytes(T, topk, E))


def cubic_moe_grouped_gemm(x: torch.Tensor, topk_ids: torch.Tensor, experts: CubicWeight, E: int,
                           out: torch.Tensor | None = None,
                           workspace: torch.Tensor | None = None, out_dtype=torch.float32) -> torch.Tensor:
    """y[T][topk][N]: each (token, slot) pair times its expert's weights; x bf16 or
    fp16, y fp32 or bf16."""
    xd, yd = _in_dtype(x, "x"), _out_dtype(out_dtype)
    _need(topk_ids, torch.int32, "topk_ids")
    T, topk = topk_ids.shape
    cw = experts.c_struct()
    if out is None:
        out = torch.empty((T, topk, experts.N), dtype=out_dtype, device=x.device)
    elif out.dtype != out_dtype:
        raise TypeError(f"out: expected {out_dtype}, got {out.dtype}")
    need = cubic_moe_workspace_bytes(T, topk, E)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    lib = load_library()
    if xd == DTYPE_BF16 and yd == DTYPE_F32:
        st = lib.cubic_moe_grouped_gemm(_ptr(x), T, _ptr(topk_ids), topk, ctypes.byref(cw), E, _ptr(out),
                                        _ptr(workspace), workspace.numel(), _stream(x))
    else:
        st = lib.cubic_moe_grouped_gemm_ex(_ptr(x), xd, T, _ptr(topk_ids), topk, ctypes.byref(cw), E, _ptr(out),
                                           yd, _ptr(workspace), workspace.numel(), _stream(x))
    _check(st, "cubic_moe_grouped_gemm")
    return out


def cubic_moe_grouped_gemm_a8(xq: torch.Tensor, x_scale: torch.Tensor, topk_ids: torch.Tensor,
                              experts: CubicWeight, E: int, out: torch.Tensor | None = None,
                              workspace: torch.Tensor | None = None, out_dtype=torch.float32) -> torch.Tensor:
    """y[T][topk][N]: each (token, slot) pair's Dynamic A8 product with its expert;
    xq int8 [T][K] and x_scale fp32 [T] from act_quant_int8_per_token."""
    _need(xq, torch.int8, "xq")
    _need(x_scale, torch.float32, "x_scale")
    _need(topk_ids, torch.int32, "topk_ids")
    yd = _out_dtype(out_dtype)
    T, topk = topk_ids.shape
    cw = experts.c_struct()
    if out is None:
        out = torch.empty((T, topk, experts.N), dtype=out_dtype, device=xq.device)
    elif out.dtype != out_dtype:
        raise TypeError(f"out: expected {out_dtype}, got {out.dtype}")
    if workspace is None:
        workspace = torch.empty(cubic_moe_workspace_bytes(T, topk, E), dtype=torch.uint8, device=xq.device)
    _check(load_library().cubic_moe_grouped_gemm_a8(_ptr(xq), _ptr(x_scale), T, _ptr(topk_ids), topk,
                                                    ctypes.byref(cw), E, _ptr(out), yd, _ptr(workspace),
                                                    workspace.numel(), _stream(xq)),
           "cubic_moe_grouped_gemm_a8")
    return out


def cubic_moe_grouped_gemm_static_max_bytes() -> int:
    return int(load_library().cubic_moe_grouped_gemm_static_max_bytes())


def cubic_moe_grouped_gemm_static(x: torch.Tensor, topk_ids: torch.Tensor, experts: CubicWeight, E: int,
                                  out: torch.Tensor | None = None) -> torch.Tensor:
    """cubic_moe_grouped_gemm with the library's per-device routing scratch (no workspace)."""
    _need(x, torch.bfloat16, "x")
    _need(topk_ids, torch.int32, "topk_ids")
    T, topk = topk_ids.shape
    cw = experts.c_struct()
    if out is None:
        out = torch.empty((T, topk, experts.N), dtype=torch.float32, device=x.device)
    _check(load_library().cubic_moe_grouped_gemm_static(_ptr(x), T, _ptr(topk_ids), topk, ctypes.byref(cw),
                                                        E, _ptr(out), _stream(x)),
           "cubic_moe_grouped_gemm_static")
    return out


def cubic_moe_mlp_workspace_bytes(T: int, topk: int, E: int, H: int, I: int) -> int:
    return int(load_library().cubic_moe_mlp_workspace_bytes(T, topk, E, H, I))


def cubic_moe_mlp(x: torch.Tensor, topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                  gate_up: CubicWeight, down: CubicWeight, E: int, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y[T][H] (fp32): sum_j w[t][j] * (bf16(SiLU(gate) * up) of token t through expert
    topk_ids[t][j]'s gate_up) through that expert's down projection."""
    _need(x, torch.bfloat16, "x")
    _need(topk_ids, torch.int32, "topk_ids")
    _need(topk_weights, torch.float32, "topk_weights")
    T, topk = topk_ids.shape
    if out is None:
        out = torch.empty((T, down.N), dtype=torch.float32, device=x.device)
    need = cubic_moe_mlp_workspace_bytes(T, topk, E, gate_up.K, down.K)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    gu, dn = gate_up.c_struct(), down.c_struct()
    _check(load_library().cubic_moe_mlp(_ptr(x), T, _ptr(topk_ids), _ptr(topk_weights), topk,
                                        ctypes.byref(gu), ctypes.byref(dn), E, _ptr(out), _ptr(workspace),
                                        workspace.numel(), _stream(x)), "cubic_moe_mlp")
    return out


def cubic_moe_mlp_a8_workspace_bytes(T: int, topk: int, E: int, H: int, I: int) -> int:
    return int(load_library().cubic_moe_mlp_a8_workspace_bytes(T, topk, E, H, I))


def cubic_moe_mlp_a8(x: torch.Tensor, topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                     gate_up: CubicWeight, down: CubicWeight, E: int, out: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None) -> torch.Tensor:
    """cubic_moe_mlp in the Dynamic A8 mode: the token rows and the intermediate h
    rows are quantised per row to int8 before their grouped products."""
    _need(x, torch.bfloat16, "x")
    _need(topk_ids, torch.int32, "topk_ids")
    _need(topk_weights, torch.float32, "topk_weights")
    T, topk = topk_ids.shape
    if out is None:
        out = torch.empty((T, down.N), dtype=torch.float32, device=x.device)
    need = cubic_moe_mlp_a8_workspace_bytes(T, topk, E, gate_up.K, down.K)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    gu, dn = gate_up.c_struct(), down.c_struct()
    _check(load_library().cubic_moe_mlp_a8(_ptr(x), T, _ptr(topk_ids), _ptr(topk_weights), topk,
                                           ctypes.byref(gu), ctypes.byref(dn), E, _ptr(out), _ptr(workspace),
                                           workspace.numel(), _stream(x)), "cubic_moe_mlp_a8")
    return out

"""Helpers of the GPU parity tests: upload synthetic weights through the HIP
library (cubic_pack), convert tensors for the oracle, and the acceptance metric."""
from __future__ import annotations

import sys

import numpy as np
import torch

import dequant_gemm_amd as cq
import synth

DEV = torch.device("cuda:0")


def say(msg: str):
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def np_weight(w: synth.Weight):
    return (w.codes.cpu().numpy(), w.scales.cpu().numpy(),
            w.shapes.cpu().numpy().view(np.uint16))


def x_bits(x: torch.Tensor) -> np.ndarray:
    return x.cpu().view(torch.int16).numpy().view(np.uint16)


def upload(w: synth.Weight) -> cq.CubicWeight:
    codes = w.codes.to(DEV)
    packed = cq.cubic_pack(codes, w.bits)
    return cq.CubicWeight(packed.reshape(-1), w.scales.to(DEV).contiguous(),
                          w.shapes.to(DEV).contiguous(), w.N, w.K, w.bits, w.group)


def row_rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of max_n |y - ref| / max_n |ref|; an all-zero reference row
    must come back exactly zero (then it contributes 0, else inf)."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max(axis=1)
    num = np.abs(y - ref).max(axis=1)
    out = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num == 0, 0.0, np.inf))
    return float(out.max()) if out.size else 0.0


def ulp32(v: np.ndarray) -> np.ndarray:
    """ulp of fp32 at |v| (2^-149 in the subnormal range)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    return np.where(a > 0, np.exp2(e - 23), 2.0 ** -149)


def pack_fields(codes: np.ndarray, bits: int) -> np.ndarray:
    """Packs any two's-complement field values, including -2^(bits-1), which the
    format's packer rejects: LSB-first over the row-major [N][K] codes. Lets
    tests plant codes outside [-Kmax, Kmax]; checked against oracle.pack and
    oracle.unpack in the CPU tests."""
    codes = np.asarray(codes)
    if bits in (2, 4, 8):                           # whole fields per byte: shift and add
        per = 8 // bits
        u = (codes.astype(np.int64) & ((1 << bits) - 1)).reshape(-1, per)
        out = np.zeros(u.shape[0], dtype=np.int64)
        for i in range(per):
            out |= u[:, i] << (bits * i)
        return out.astype(np.uint8).reshape(codes.shape[0], -1)
    u = (codes.astype(np.int64) & ((1 << bits) - 1)).reshape(-1)
    pos0 = np.arange(u.size, dtype=np.int64) * bits
    out = np.zeros(u.size * bits // 8, dtype=np.int64)
    for b in range(bits):
        pos = pos0 + b
        np.add.at(out, pos // 8, ((u >> b) & 1) << (pos % 8))
    return out.astype(np.uint8).reshape(codes.shape[0], -1)

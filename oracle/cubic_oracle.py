"""CPU oracle for the CubicQuant weight-only dequant-GEMM, in numpy float64.

TEST INFRASTRUCTURE. This module is the plain, slow definition that the HIP
library is checked against. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The product path never
imports, links or calls it, and the two share no code, tables or helpers.

Source pages (cited by title and section, never quoted):

* CubicQuant article on ModelScope, "CubicQuant：用三次曲线重塑低比特量化，Kimi K3
  2.5Bit 模型首发实践" (below: *the CubicQuant article*).
  - section "CubicQuant 核心：把直线网格掰弯" (*Core*): the positive-side maximum
    code, the normalised magnitude t of a code, the cubic q(t) with c = 1 - a - b,
    the reconstructed weight, and the three properties (q(0) = 0, q(1) = 1,
    q'(t) > 0; a = 1, b = 0 is symmetric uniform INT). The display equations of
    this section did not survive text extraction; the readings used here are
    listed under "Readings" below.
  - section "存储开销是透明的：B+64/G bit" (*Storage*): per group of G weights the
    format holds G B-bit integer codes, one FP32 scale and two FP16 shape
    parameters, so B + 64/G bits per weight; first table (bits per weight for
    G = 128, 256, 512) and second table (bytes per weight and ratio to BF16 at
    G512).
  - section "一份 checkpoint，同时服务 A16 与 Dynamic A8" (*A16/A8*): A16 consumes
    the continuous levels with FP16/BF16 activations; Dynamic A8 quantises each
    activation row to INT8 at run time, maps the weight levels to a deterministic
    INT8 carrier, takes integer dot products and scales per group in FP32. The
    carrier equation did not survive extraction.
  - section "Kimi-K3-Cubic-2.5Bit 是怎样得到 2.4986 bit 的？" (*Mix*): the per-layer
    format plan and the payload / metadata arithmetic.
* msModelSlim article on ai6s.net (Kimi K3 INT quantisation), section
  "具体量化策略", sub-section on routed experts (W4A8): activations are quantised
  dynamically per token.

Readings (where the pages are silent or their equations were stripped):

* Kmax = 2^(B-1) - 1; t = |k| / Kmax; q(t) = a t + b t^2 + (1 - a - b) t^3;
  w = s * sign(k) * q(t). Supported widths B in [2, 8].
* Codes are B-bit two's complement fields in one LSB-first bitstream over the
  row-major [N][K] matrix (little-endian bytes).
* Groups are G consecutive weights along K within a row; scales are a float32
  array [N][K/G]; shapes are float16 bit patterns [N][K/G][2] (a, then b).
* The code -2^(B-1) (outside the symmetric range) decodes by the same formula
  (t > 1); the carrier clamps it.
* A8 carrier: C_j = clamp(RNE(127 * q_j), -127, 127) and the group scale is
  s / 127. Activation scale: sx = fp32(amax / 127), xq = clamp(RNE(fp32(x / sx)),
  -127, 127); an all-zero row gives sx = 0 and xq = 0.

Exactness: a and b are fp16, hence integer multiples of 2^-24. For |a|, |b| <= 16
every term of Q_j = a j K^2 + b j^2 K + c j^3 (with K = Kmax) is a multiple of
2^-24 below 2^28, so Q_j is exact in float64 (at most 52 significant bits);
q_j = Q_j / K^3 and s * q_j each round once in float64.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

__all__ = [
    "kmax", "bits_per_weight", "code_bytes", "storage_bytes",
    "pack", "unpack", "f16_bits_to_f64", "bf16_bits_to_f64",
    "level_numerators", "levels", "dequant", "gemm_a16",
    "act_quant", "carrier_table", "carrier_codes", "gemm_a8", "moe_a16", "moe_a8",
    "format_levels", "dequant_f32", "encode", "bf16_rne", "silu_mul", "moe_mlp_hidden", "moe_mlp", "moe_mlp_a8",
    "FIT_CLIP_STEPS", "fit_is_monotone", "fit_shape_candidates", "f64_to_f16_bits", "fit_group_sse", "fit",
]

# Domain in which the float64 evaluation of Q_j is exact (see module docstring).
_SHAPE_ABS_MAX = 16.0


def kmax(bits: int) -> int:
    """Positive-side maximum code, 2^(B-1) - 1 (CubicQuant article, Core)."""
    if not 2 <= bits <= 8:
        raise ValueError(f"bits must be in [2, 8], got {bits}")
    return (1 << (bits - 1)) - 1


# ----------------------------------------------------------------------------
# Storage (CubicQuant article, Storage section and its two tables)
# ----------------------------------------------------------------------------
def bits_per_weight(bits: int, group: int) -> Fraction:
    """B payload bits plus 32 (fp32 scale) + 2 * 16 (fp16 a, b) bits per group."""
    return Fraction(bits) + Fraction(32 + 2 * 16, group)


def code_bytes(N: int, K: int, bits: int) -> int:
    """Bytes of the packed code stream of an N x K matrix."""
    total_bits = N * K * bits
    if total_bits % 8:
        raise ValueError("N*K*bits must be a multiple of 8")
    return total_bits // 8


def storage_bytes(N: int, K: int, bits: int, group: int) -> int:
    """Code stream plus 8 bytes of metadata per group."""
    if K % group:
        raise ValueError("K must be a multiple of group")
    return code_bytes(N, K, bits) + 8 * N * (K // group)


# ----------------------------------------------------------------------------
# Code stream (reading: B-bit two's complement, LSB-first, row-major [N][K])
# ----------------------------------------------------------------------------
def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    """int codes [N][K] -> packed uint8 [N][K*bits/8]. Rejects |k| > Kmax."""
    codes = np.asarray(codes)
    N, K = codes.shape
    km = kmax(bits)
    if codes.size and (codes.min() < -km or codes.max() > km):
        raise ValueError("code outside [-Kmax, Kmax]")
    if (K * bits) % 8:
        raise ValueError("K*bits must be a multiple of 8")
    field = codes.astype(np.int64) & ((1 << bits) - 1)          # two's complement
    bitplanes = (field[..., None] >> np.arange(bits)) & 1        # [N][K][bits], LSB first
    stream = bitplanes.reshape(N, K * bits).astype(np.uint8)
    return np.packbits(stream, axis=1, bitorder="little")


def unpack(packed: np.ndarray, N: int, K: int, bits: int) -> np.ndarray:
    """packed uint8 [N][K*bits/8] (or flat) -> int8 codes [N][K]."""
    packed = np.asarray(packed, dtype=np.uint8).reshape(N, (K * bits) // 8)
    stream = np.unpackbits(packed, axis=1, bitorder="little").astype(np.int64)
    bitplanes = stream.reshape(N, K, bits)
    field = (bitplanes << np.arange(bits)).sum(axis=2)
    signed = np.where(field >= (1 << (bits - 1)), field - (1 << bits), field)
    return signed.astype(np.int8)


# ----------------------------------------------------------------------------
# Scalar decodings of the stored floating-point formats
# ----------------------------------------------------------------------------
def f16_bits_to_f64(u16: np.ndarray) -> np.ndarray:
    return np.asarray(u16, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_bits_to_f64(u16: np.ndarray) -> np.ndarray:
    u32 = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16
    return u32.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# Levels (CubicQuant article, Core)
# ----------------------------------------------------------------------------
def level_numerators(a: np.ndarray, b: np.ndarray, bits: int) -> np.ndarray:
    """Q_j = Kmax^3 * q(j / Kmax) for j = 0 .. 2^(B-1), exact in float64.

    a, b: float64 arrays (values of fp16 numbers), any shape S. Returns S + (2^(B-1)+1,).
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size and (np.abs(a).max() > _SHAPE_ABS_MAX or np.abs(b).max() > _SHAPE_ABS_MAX):
        raise ValueError("shape parameters outside the exactly evaluated domain |a|,|b| <= 16")
    km = float(kmax(bits))
    j = np.arange((1 << (bits - 1)) + 1, dtype=np.float64)
    c = 1.0 - a - b
    return (a[..., None] * (j * km * km)
            + b[..., None] * (j * j * km)
            + c[..., None] * (j * j * j))


def levels(a: np.ndarray, b: np.ndarray, bits: int) -> np.ndarray:
    """q_j = q(j / Kmax) for j = 0 .. 2^(B-1) (j = 2^(B-1) is the extra negative code)."""
    km = float(kmax(bits))
    return level_numerators(a, b, bits) / (km * km * km)


def _group_params(scales, shapes, N, K, group):
    G = K // group
    s = np.asarray(scales, dtype=np.float32).reshape(N, G).astype(np.float64)
    ab = np.asarray(shapes, dtype=np.uint16).reshape(N, G, 2)
    return s, f16_bits_to_f64(ab[..., 0]), f16_bits_to_f64(ab[..., 1])


def dequant(codes: np.ndarray, scales: np.ndarray, shapes: np.ndarray,
            bits: int, group: int) -> np.ndarray:
    """W[n,k] = s * sign(k) * q(|k| / Kmax) in float64; code 0 gives +0.0."""
    codes = np.asarray(codes)
    N, K = codes.shape
    if K % group:
        raise ValueError("K must be a multiple of group")
    s, a, b = _group_params(scales, shapes, N, K, group)
    w_level = s[..., None] * levels(a, b, bits)                  # [N][G][2^(B-1)+1]
    mag = np.abs(codes.astype(np.int64)).reshape(N, K // group, group)
    w = np.take_along_axis(w_level, mag, axis=2).reshape(N, K)
    sign = np.sign(codes.astype(np.int64))
    return np.where(codes == 0, 0.0, sign * w)


# ----------------------------------------------------------------------------
# A16 (CubicQuant article, A16/A8 section): activations consume continuous levels
# ----------------------------------------------------------------------------
def _act_values(x_bits: np.ndarray, fmt: str) -> np.ndarray:
    """Exact values of 16-bit activations: bf16 or fp16 bit patterns."""
    if fmt == "bf16":
        return bf16_bits_to_f64(x_bits)
    if fmt == "f16":
        return f16_bits_to_f64(x_bits)
    raise ValueError(f"activation format {fmt!r}")


def gemm_a16(x_bits: np.ndarray, W: np.ndarray, fmt: str = "bf16") -> np.ndarray:
    """Y[m,n] = sum_k x[m,k] * W[n,k] in float64 (x given as bf16, or with
    fmt="f16" fp16, bit patterns: the article's A16 takes FP16 or BF16)."""
    X = _act_values(x_bits, fmt)
    return X @ np.asarray(W, dtype=np.float64).T


# ----------------------------------------------------------------------------
# Dynamic A8 (CubicQuant article, A16/A8 section; msModelSlim article, per-token
# dynamic activation quantisation)
# ----------------------------------------------------------------------------
def act_quant(x_bf16: np.ndarray, fmt: str = "bf16"):
    """Per-row INT8 quantisation: returns (xq int8 [M][K], sx float32 [M]); x as
    bf16 (or, with fmt="f16", fp16) bit patterns.

    sx = fp32(amax / 127); xq = clamp(RNE(fp32(x / sx)), -127, 127). Each fp32
    division is a float64 division rounded to float32, which equals the IEEE
    fp32 quotient (53 >= 2*24 + 2, so the double rounding is innocuous).
    """
    X = _act_values(x_bf16, fmt)
    M = X.shape[0]
    amax = np.abs(X).max(axis=1) if X.shape[1] else np.zeros(M)
    sx = (amax / 127.0).astype(np.float32)
    xq = np.zeros(X.shape, dtype=np.int8)
    nz = sx != 0
    if nz.any():
        r = (X[nz] / sx[nz].astype(np.float64)[:, None]).astype(np.float32)
        xq[nz] = np.clip(np.rint(r.astype(np.float64)), -127, 127).astype(np.int8)
    return xq, sx


def _rne_div(num: np.ndarray, den: int) -> np.ndarray:
    """Round-to-nearest-even of num / den for int64 num and a positive int den."""
    q = np.floor_divide(num, den)
    r = num - q * den                       # 0 <= r < den
    up = (2 * r > den) | ((2 * r == den) & (q % 2 != 0))
    return q + up.astype(np.int64)


def carrier_table(a: np.ndarray, b: np.ndarray, bits: int) -> np.ndarray:
    """C_j = clamp(RNE(127 * q_j), -127, 127) for j = 0 .. 2^(B-1), exactly.

    Uses integers: with A = a * 2^24 (exact for fp16), Q_j * 2^24 is an integer,
    so 127 * q_j = 127 * (Q_j * 2^24) / (Kmax^3 * 2^24) is a ratio of int64s.
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size and (np.abs(a).max() > _SHAPE_ABS_MAX or np.abs(b).max() > _SHAPE_ABS_MAX):
        raise ValueError("shape parameters outside the exactly evaluated domain |a|,|b| <= 16")
    km = kmax(bits)
    A = (a * 2.0 ** 24).astype(np.int64)
    B = (b * 2.0 ** 24).astype(np.int64)
    C = (1 << 24) - A - B
    j = np.arange((1 << (bits - 1)) + 1, dtype=np.int64)
    Q = A[..., None] * (j * km * km) + B[..., None] * (j * j * km) + C[..., None] * (j * j * j)
    return np.clip(_rne_div(127 * Q, km ** 3 << 24), -127, 127)


def carrier_codes(codes: np.ndarray, shapes: np.ndarray, bits: int, group: int) -> np.ndarray:
    """Per-weight INT8 carrier sign(k) * C_|k| as int64 [N][K]."""
    codes = np.asarray(codes)
    N, K = codes.shape
    ab = np.asarray(shapes, dtype=np.uint16).reshape(N, K // group, 2)
    tab = carrier_table(f16_bits_to_f64(ab[..., 0]), f16_bits_to_f64(ab[..., 1]), bits)
    mag = np.abs(codes.astype(np.int64)).reshape(N, K // group, group)
    c = np.take_along_axis(tab, mag, axis=2).reshape(N, K)
    return np.sign(codes.astype(np.int64)) * c


def gemm_a8(xq: np.ndarray, sx: np.ndarray, codes: np.ndarray, scales: np.ndarray,
            shapes: np.ndarray, bits: int, group: int) -> np.ndarray:
    """Y[m,n] = sx_m * sum_g (s_{n,g} / 127) * I[m,n,g], I = exact integer group dot."""
    codes = np.asarray(codes)
    N, K = codes.shape
    G = K // group
    Cw = carrier_codes(codes, shapes, bits, group).astype(np.float64)
    Xq = np.asarray(xq, dtype=np.float64)
    s = np.asarray(scales, dtype=np.float32).reshape(N, G).astype(np.float64)
    Y = np.zeros((Xq.shape[0], N), dtype=np.float64)
    for g in range(G):
        sl = slice(g * group, (g + 1) * group)
        I = Xq[:, sl] @ Cw[:, sl].T        # integers below 2^53: exact in float64
        Y += I * (s[:, g] / 127.0)[None, :]
    return np.asarray(sx, dtype=np.float32).astype(np.float64)[:, None] * Y


# ----------------------------------------------------------------------------
# Routed experts: each (token, slot) pair is an A16 product with its expert
# ----------------------------------------------------------------------------
def moe_a16(x_bf16: np.ndarray, topk_ids: np.ndarray, num_experts: int, N: int,
            expert_weight, fmt: str = "bf16") -> np.ndarray:
    """Y[t, j, :] = W_e @ x[t] with e = topk_ids[t, j]; ids outside [0, E) give zeros.

    expert_weight(e) -> float64 W_e [N][K] (the caller dequantises its experts);
    x as bf16 (or, with fmt="f16", fp16) bit patterns.
    """
    ids = np.asarray(topk_ids)
    T, topk = ids.shape
    X = _act_values(x_bf16, fmt)
    Y = np.zeros((T, topk, N), dtype=np.float64)
    cache = {}
    for t in range(T):
        for j in range(topk):
            e = int(ids[t, j])
            if not 0 <= e < num_experts:
                continue
            if e not in cache:
                cache[e] = np.asarray(expert_weight(e), dtype=np.float64)
            Y[t, j] = cache[e] @ X[t]
    return Y


def moe_a8(xq: np.ndarray, sx: np.ndarray, topk_ids: np.ndarray, num_experts: int, N: int,
           expert_codes, bits: int, group: int) -> np.ndarray:
    """Dynamic A8 on the routed experts: Y[t, j, :] = gemm_a8 of row t of (xq, sx)
    with expert e = topk_ids[t, j]; ids outside [0, E) give zeros.

    expert_codes(e) -> (codes [N][K], scales [N][K/G], shapes [N][K/G][2] as fp16 bits).
    """
    ids = np.asarray(topk_ids)
    T, topk = ids.shape
    Y = np.zeros((T, topk, N), dtype=np.float64)
    cache = {}
    for t in range(T):
        for j in range(topk):
            e = int(ids[t, j])
            if not 0 <= e < num_experts:
                continue
            if e not in cache:
                cache[e] = expert_codes(e)
            codes, scales, shapes = cache[e]
            Y[t, j] = gemm_a8(xq[t:t + 1], sx[t:t + 1], codes, scales, shapes, bits, group)[0]
    return Y


# ----------------------------------------------------------------------------
# The format's fp32 levels. A stored group reconstructs each weight as the real
# number s * sign(k) * q(|k| / Kmax) (CubicQuant article, Core); written out in
# fp32 (the storage section keeps s in fp32) it is that number rounded once to
# the nearest fp32 value, ties to even. An exact zero is +0.0; a nonzero value
# too small for fp32 rounds to a zero of its own sign, and one beyond the fp32
# range to an infinity.
# ----------------------------------------------------------------------------
def _rn32_rational(v: Fraction) -> np.float32:
    """Nearest fp32 value of an exact rational (ties to even)."""
    if v == 0:
        return np.float32(0.0)
    m = abs(v)
    e = m.numerator.bit_length() - m.denominator.bit_length()   # floor(log2 m) is e or e - 1
    if m < Fraction(2) ** e:
        e -= 1
    e = max(e, -126)                                            # subnormals share the smallest spacing
    ulp = Fraction(2) ** (e - 23)
    n = round(m / ulp)                                          # Fraction rounding: half to even
    mag = np.float32(np.inf) if n * ulp >= 2 ** 128 else np.float32(float(n * ulp))
    return -mag if v < 0 else mag


def _level_exact(s: float, a: float, b: float, j: int, bits: int) -> Fraction:
    """s * q(j / Kmax) as an exact rational from the stored fp32 s and fp16 a, b."""
    km = kmax(bits)
    a, b = Fraction(a), Fraction(b)
    t = Fraction(j, km)
    return Fraction(float(s)) * (a * t + b * t * t + (1 - a - b) * t * t * t)


def format_levels(scales: np.ndarray, a: np.ndarray, b: np.ndarray, bits: int) -> np.ndarray:
    """fp32 levels RN32(s * q_j) for j = 0 .. 2^(B-1) (float32, shape S + (2^(B-1)+1,)).

    scales float32, a and b float64 values of fp16 numbers, all of one shape S.
    The float64 product y = s * q_j (q_j from `levels`) carries two roundings, so
    it lies within 2^-52 |V| of the exact value V; wherever y is further than
    2^-51 |y| from every fp32 rounding boundary, V rounds like y. The remaining
    entries, shapes outside the exactly evaluated domain, and non-finite scales
    are computed with exact rationals instead."""
    s32 = np.asarray(scales, dtype=np.float32)
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    L = (1 << (bits - 1)) + 1
    out = np.zeros(s32.shape + (L,), dtype=np.float32)
    inside = (np.abs(a) <= _SHAPE_ABS_MAX) & (np.abs(b) <= _SHAPE_ABS_MAX)
    y = np.zeros(out.shape, dtype=np.float64)
    if inside.any():
        y[inside] = s32[inside].astype(np.float64)[..., None] * levels(a[inside], b[inside], bits)
    with np.errstate(over="ignore", invalid="ignore"):
        v = y.astype(np.float32)
        mag = np.abs(v)
        down = np.nextafter(mag, np.float32(0)).astype(np.float64)
        down = np.where(mag > 0, down, -(2.0 ** -149))
        up = np.nextafter(mag, np.float32(np.inf)).astype(np.float64)
        lo = (mag.astype(np.float64) + down) / 2
        hi = (mag.astype(np.float64) + up) / 2
        ay = np.abs(y)
        tol = ay * 2.0 ** -51
        safe = (ay - tol > lo) & (ay + tol < hi) & np.isfinite(mag) & (mag < np.float32(3.4028235e38))
    safe &= inside[..., None] & np.isfinite(s32)[..., None]
    # exact zeros (s = 0 or Q_j = 0) are +0.0, whatever the other factor is
    q_zero = level_numerators(np.where(inside, a, 0), np.where(inside, b, 0), bits) == 0
    zero = inside[..., None] & ((s32[..., None] == 0) | q_zero)
    out[safe] = v[safe]
    out[zero] = np.float32(0.0)
    for idx in zip(*np.nonzero(~(safe | zero))):
        g, j = idx[:-1], int(idx[-1])
        s = float(s32[g])
        exact = _level_exact(1.0, float(a[g]), float(b[g]), j, bits)      # q_j
        if s == 0 or exact == 0:
            out[idx] = np.float32(0.0)
        elif not np.isfinite(s):
            out[idx] = np.float32(s * float(exact))                         # +-inf or NaN
        else:
            out[idx] = _rn32_rational(Fraction(s) * exact)
    return out


def dequant_f32(codes: np.ndarray, scales: np.ndarray, shapes: np.ndarray,
                bits: int, group: int) -> np.ndarray:
    """W[n,k] in fp32 as the format stores it: RN32(s * sign(k) * q(|k| / Kmax))."""
    codes = np.asarray(codes)
    N, K = codes.shape
    if K % group:
        raise ValueError("K must be a multiple of group")
    G = K // group
    s = np.asarray(scales, dtype=np.float32).reshape(N, G)
    ab = np.asarray(shapes, dtype=np.uint16).reshape(N, G, 2)
    lv = format_levels(s, f16_bits_to_f64(ab[..., 0]), f16_bits_to_f64(ab[..., 1]), bits)
    mag = np.abs(codes.astype(np.int64)).reshape(N, G, group)
    w = np.take_along_axis(lv, mag, axis=2).reshape(N, K)
    out = np.where(codes < 0, -w, w)
    return np.where(out == 0, np.float32(0.0), out).astype(np.float32)


# ----------------------------------------------------------------------------
# Nearest-level encoding (CubicQuant article, Core: each weight takes the code of
# its group's nearest reconstruction level, given the group's s, a, b). The
# levels are the format's fp32 values L_k = RN32(s * sign(k) * q(|k| / Kmax)) for
# k in [-Kmax, Kmax] (the extra code -2^(B-1) is never chosen), and distances
# are exact. With v_j = RN32(s q_j), L_{+-j} = +-v_j, so |w - L_k| is smallest
# over the two signs at | |w| - |v_j| |: the code is j* sign(w) sign(v_j*) for
# the first j (smallest |k|) of smallest exact | |w| - |v_j| |. A weight of
# either zero sign takes code 0, and so does a NaN weight (no distance is smaller
# than another's).
# ----------------------------------------------------------------------------
def _nearest_j(aw: np.ndarray, av: np.ndarray):
    """First index j of the smallest exact | aw - av[j] | for non-negative float32
    aw [...][n] against av [...][L]: int64 [...][n]. A NaN distance counts as
    larger than every other, so NaN levels never win and a NaN weight takes 0.

    The difference of two non-negative fp32 values x >= y is exact in float64
    when y = 0 or x < 2^28 y (it then spans at most 53 bits); weights with a
    level outside that ratio are decided with exact rationals."""
    x = aw.astype(np.float64)
    y = av.astype(np.float64)
    best = np.full(x.shape, np.inf)
    bj = np.zeros(x.shape, dtype=np.int64)
    for j in range(y.shape[-1]):                     # the first strictly smaller distance wins
        with np.errstate(invalid="ignore"):
            dj = np.abs(x - y[..., j:j + 1])
            better = dj < best                       # False for NaN
        best = np.where(better, dj, best)
        bj[better] = j
    # the largest and the smallest positive finite level of each set decide the ratio test
    fin = np.isfinite(y)
    ymax = np.where(fin, y, 0.0).max(axis=-1)[..., None]
    ymin = np.where(fin & (y > 0), y, np.inf).min(axis=-1)[..., None]
    with np.errstate(over="ignore", invalid="ignore"):
        loose = (x > 0) & np.isfinite(x) & ((x >= ymin * 2.0 ** 28) | (ymax >= x * 2.0 ** 28))
    for idx in zip(*np.nonzero(loose)):
        xv = Fraction(float(x[idx]))
        best_f, jj = None, 0
        for j in range(y.shape[-1]):
            yv = float(y[idx[:-1]][j])
            if not np.isfinite(yv):
                continue
            dj = abs(xv - Fraction(yv))
            if best_f is None or dj < best_f:
                best_f, jj = dj, j
        bj[idx] = jj
    return bj


def encode(w: np.ndarray, scales: np.ndarray, shapes: np.ndarray, bits: int,
           group: int) -> np.ndarray:
    """int8 codes [N][K] of float32 weights w [N][K] by the nearest-level rule above."""
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    if K % group:
        raise ValueError("K must be a multiple of group")
    G = K // group
    km = kmax(bits)
    s = np.asarray(scales, dtype=np.float32).reshape(N, G)
    ab = np.asarray(shapes, dtype=np.uint16).reshape(N, G, 2)
    v = format_levels(s, f16_bits_to_f64(ab[..., 0]), f16_bits_to_f64(ab[..., 1]), bits)[..., :km + 1]
    wg = w.reshape(N, G, group)
    out = np.empty((N, G, group), dtype=np.int64)
    for n in range(N):                                     # one row at a time bounds the memory
        j = _nearest_j(np.abs(wg[n]), np.abs(v[n]))        # [G][group]
        vj = np.take_along_axis(v[n], j, axis=1)
        flip = np.signbit(wg[n]) != np.signbit(vj)
        out[n] = np.where(flip, -j, j)
    return out.reshape(N, K).astype(np.int8)


# ----------------------------------------------------------------------------
# Data-free group fitting (CubicQuant article, the section on data-free in-group
# fitting: per group, search monotone (a, b) candidates, choose the scale together
# with a soft-clip threshold, give every weight its nearest level, store a, b as
# fp16 and s as fp32). The pages fix neither the search grid nor the loss; this
# library's reading: the loss is the group's sum of squared weight errors, a and b
# run over multiples of 1/8 (a in [0, 3], b in [-3, 3], exact in fp16, so the fp16
# step changes nothing), and the clip threshold is the scale itself,
# s = fl32(rho * max|w|) with rho = 1 - r/32, r = 0 .. 15: weights beyond s take
# the top level. Codes follow the nearest-level rule of `encode`.
# ----------------------------------------------------------------------------
FIT_CLIP_STEPS = 16


def fit_is_monotone(a: Fraction, b: Fraction) -> bool:
    """True when q(t) = a t + b t^2 + (1-a-b) t^3 is non-decreasing on [0, 1]:
    q'(t) = a + 2 b t + 3 c t^2 >= 0 at both ends and at an interior stationary point."""
    c = 1 - a - b

    def dq(t):
        return a + 2 * b * t + 3 * c * t * t

    if dq(Fraction(0)) < 0 or dq(Fraction(1)) < 0:
        return False
    if c != 0:
        t = -b / (3 * c)
        if 0 < t < 1 and dq(t) < 0:
            return False
    return True


def fit_shape_candidates() -> np.ndarray:
    """(a, b) pairs of the search in search order, float64 [n][2]: a = i/8 for
    i = 0 .. 24 (outer), b = j/8 for j = -24 .. 24 (inner), monotone pairs only."""
    out = []
    for i in range(0, 25):
        for j in range(-24, 25):
            a, b = Fraction(i, 8), Fraction(j, 8)
            if fit_is_monotone(a, b):
                out.append((float(a), float(b)))
    return np.array(out, dtype=np.float64)


def f64_to_f16_bits(v: np.ndarray) -> np.ndarray:
    """Exact fp16 bit patterns of float64 values that fp16 represents."""
    h = np.asarray(v, dtype=np.float64).astype(np.float16)
    if not np.array_equal(h.astype(np.float64), np.asarray(v, dtype=np.float64)):
        raise ValueError("value not representable in fp16")
    return h.view(np.uint16)


def fit_group_sse(wg: np.ndarray, bits: int, ab: np.ndarray):
    """Losses of every candidate for one group of float32 weights wg [G]:
    float64 [n_ab][FIT_CLIP_STEPS], the sum over the group of the squared
    distance from each |w| to its nearest fp32 level of the candidate (the
    format's levels RN32(s q_j), the nearest by exact distance, as `encode`
    chooses), each distance exact and squared and summed in float64."""
    wg = np.asarray(wg, dtype=np.float32)
    aw = np.abs(wg)
    amax = aw.max() if aw.size else np.float32(0.0)
    km = kmax(bits)
    rho = (np.float32(1.0) - np.arange(FIT_CLIP_STEPS, dtype=np.float32) / np.float32(32.0)).astype(np.float32)
    s = (rho * amax).astype(np.float32)                         # [R], one fp32 rounding each
    out = np.empty((len(ab), FIT_CLIP_STEPS), dtype=np.float64)
    step = max(1, (1 << 22) // (FIT_CLIP_STEPS * (km + 1) * max(1, aw.size)))
    R = FIT_CLIP_STEPS
    for c0 in range(0, len(ab), step):                         # chunks of pairs bound the memory
        abc = ab[c0:c0 + step]
        n = len(abc)
        sc = np.broadcast_to(s[None, :], (n, R))
        a = np.broadcast_to(abc[:, 0:1], (n, R))
        b = np.broadcast_to(abc[:, 1:2], (n, R))
        v = np.abs(format_levels(sc, a, b, bits)[..., :km + 1])          # [n][R][L] fp32
        j = _nearest_j(np.broadcast_to(aw, (n, R, aw.size)), v)         # [n][R][G]
        vj = np.take_along_axis(v, j, axis=2).astype(np.float64)
        e = aw.astype(np.float64)[None, None, :] - vj
        out[c0:c0 + step] = (e * e).sum(axis=2)
    return out, s


def fit(w: np.ndarray, bits: int, group: int):
    """Fit every group of float32 weights w [N][K]: returns (codes int8 [N][K],
    scales float32 [N][K/group], shapes fp16 bits [N][K/group][2], loss float64
    [N][K/group], candidate index int64 [N][K/group] = shape index * 16 + r).
    The first candidate of smallest loss wins."""
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    if K % group:
        raise ValueError("K must be a multiple of group")
    G = K // group
    ab = fit_shape_candidates()
    scales = np.zeros((N, G), dtype=np.float32)
    shapes = np.zeros((N, G, 2), dtype=np.uint16)
    loss = np.zeros((N, G), dtype=np.float64)
    index = np.zeros((N, G), dtype=np.int64)
    for n in range(N):
        for g in range(G):
            sse, s = fit_group_sse(w[n, g * group:(g + 1) * group], bits, ab)
            k = int(np.argmin(sse.reshape(-1)))
            i, r = divmod(k, FIT_CLIP_STEPS)
            scales[n, g] = s[r]
            shapes[n, g] = f64_to_f16_bits(ab[i])
            loss[n, g] = sse.reshape(-1)[k]
            index[n, g] = k
    codes = encode(w, scales, shapes, bits, group)
    return codes, scales, shapes, loss, index


# ----------------------------------------------------------------------------
# Routed-expert MLP step (Kimi K3 guide, model card: routed experts with a fused
# gate_up and a down projection). The pages give the expert layout, not the
# arithmetic between the products; this library's reading: h = SiLU(gate) * up
# rounded to bf16 (the down projection's activations), outputs weighted by the
# router's weights and summed over the token's slots.
# ----------------------------------------------------------------------------
def bf16_rne(v: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 value (ties to even), as float64, by exact rational
    steps: the bf16 spacing around v is a power of two, so v / spacing is rounded
    to an even integer on ties with np.rint and scaled back. Finite inputs."""
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros_like(v)
    nz = v != 0
    e = np.floor(np.log2(np.abs(v[nz])))
    # fix the exponent where log2 rounded across a power of two
    e = np.where(np.abs(v[nz]) >= 2.0 ** (e + 1), e + 1, e)
    e = np.where(np.abs(v[nz]) < 2.0 ** e, e - 1, e)
    e = np.maximum(e, -126.0)                          # bf16 subnormals share the smallest spacing
    spacing = 2.0 ** (e - 7)                           # 8 significant bits
    out[nz] = np.rint(v[nz] / spacing) * spacing
    return out


def silu_mul(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """SiLU(g) * u = g / (1 + exp(-g)) * u in float64 (before the bf16 rounding of h)."""
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g)) * np.asarray(u, dtype=np.float64)


def moe_mlp_hidden(x_bf16: np.ndarray, topk_ids: np.ndarray, num_experts: int, gate_up_weight):
    """The MLP step's intermediate per pair: (v, h) float64 [T][topk][I] with
    v = SiLU(g) * u and h = bf16(v), [g | u] = GU_e @ x[t]; zeros for invalid ids."""
    ids = np.asarray(topk_ids)
    T, topk = ids.shape
    X = bf16_bits_to_f64(x_bf16)
    v_out = None
    cache = {}
    for t in range(T):
        for j in range(topk):
            e = int(ids[t, j])
            if not 0 <= e < num_experts:
                continue
            if e not in cache:
                cache[e] = np.asarray(gate_up_weight(e), dtype=np.float64)
            gu = cache[e] @ X[t]
            I = gu.shape[0] // 2
            if v_out is None:
                v_out = np.zeros((T, topk, I), dtype=np.float64)
            v_out[t, j] = silu_mul(gu[:I], gu[I:])
    if v_out is None:
        return None, None
    return v_out, bf16_rne(v_out)


def moe_mlp(x_bf16: np.ndarray, topk_ids: np.ndarray, topk_w: np.ndarray, num_experts: int,
            gate_up_weight, down_weight) -> np.ndarray:
    """y[t] = sum_j w[t, j] * D_e @ bf16(SiLU(g) * u), [g | u] = GU_e @ x[t], e = ids[t, j]
    (float64; ids outside [0, E) add nothing). gate_up_weight(e): [2I][H]; down_weight(e): [H][I]."""
    ids = np.asarray(topk_ids)
    T, topk = ids.shape
    X = bf16_bits_to_f64(x_bf16)
    Y = np.zeros((T, X.shape[1]), dtype=np.float64)      # H = K of gate_up = N of down
    cache = {}
    for t in range(T):
        for j in range(topk):
            e = int(ids[t, j])
            if not 0 <= e < num_experts:
                continue
            if e not in cache:
                cache[e] = (np.asarray(gate_up_weight(e), dtype=np.float64),
                            np.asarray(down_weight(e), dtype=np.float64))
            GU, D = cache[e]
            I = D.shape[1]
            gu = GU @ X[t]
            g, u = gu[:I], gu[I:]
            h = bf16_rne(g / (1.0 + np.exp(-g)) * u)
            Y[t] += float(topk_w[t, j]) * (D @ h)
    return Y


def _bf16_bits_of(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of values that are bf16 numbers already (exact)."""
    return (np.asarray(h, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def moe_mlp_a8(x_bf16: np.ndarray, topk_ids: np.ndarray, topk_w: np.ndarray, num_experts: int,
               gate_up_codes, down_codes, up_bits: int, up_group: int, dn_bits: int, dn_group: int):
    """The MLP step with both products in the Dynamic A8 mode (float64 apart from
    the steps the mode fixes). Per token t: (xq, sx) = act_quant(x[t]); per pair
    (t, j), e = ids[t, j] in [0, E): [g | u] = gemm_a8(xq, sx, GU_e);
    h = bf16(SiLU(g) * u); (hq, hs) = act_quant(h); o = gemm_a8(hq, hs, D_e);
    y[t] += w[t, j] * o. gate_up_codes(e) / down_codes(e) -> (codes, scales, shapes).
    Returns (y [T][H], v [T][topk][I], h [T][topk][I]); v and h are zero for
    invalid ids."""
    ids = np.asarray(topk_ids)
    T, topk = ids.shape
    xq, sx = act_quant(x_bf16)
    y = np.zeros((T, np.asarray(x_bf16).shape[1]))     # H = K of gate_up = N of down
    v_all = h_all = None
    cache = {}
    for t in range(T):
        for j in range(topk):
            e = int(ids[t, j])
            if not 0 <= e < num_experts:
                continue
            if e not in cache:
                cache[e] = (gate_up_codes(e), down_codes(e))
            (gc, gs, gsh), (dc, ds, dsh) = cache[e]
            gu = gemm_a8(xq[t:t + 1], sx[t:t + 1], gc, gs, gsh, up_bits, up_group)[0]
            I = gu.shape[0] // 2
            v = silu_mul(gu[:I], gu[I:])
            h = bf16_rne(v)
            hq, hs = act_quant(_bf16_bits_of(h)[None, :])
            o = gemm_a8(hq, hs, dc, ds, dsh, dn_bits, dn_group)[0]
            if v_all is None:
                v_all = np.zeros((T, topk, I))
                h_all = np.zeros((T, topk, I))
            v_all[t, j], h_all[t, j] = v, h
            y[t] += float(topk_w[t, j]) * o
    return y, v_all, h_all

"""GPU parity of the code stream and of the fp32 dequant against the oracle.

Bars: pack / unpack bit-exact; dequant bit-exact against the correctly rounded
fp32 levels of the oracle (and within 1 fp32 ulp of its float64 values),
exact for code 0 (+0.0), codes +-Kmax (+-s) and the uniform-INT case a=1, b=0."""
import numpy as np
import pytest
import torch

import dequant_gemm_amd as cq
import oracle
import synth
from tests._gpu import DEV, np_weight, say, ulp32

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("bits", range(2, 9))
@pytest.mark.parametrize("N,K", [(1, 32), (7, 96), (33, 512), (300, 1024)])
def test_pack_unpack_bit_exact(bits, N, K):
    say(f"pack/unpack bits={bits} N={N} K={K}")
    km = (1 << (bits - 1)) - 1
    g = torch.Generator().manual_seed(1000 * bits + N + K)
    codes = torch.randint(-km, km + 1, (N, K), generator=g).to(torch.int8)
    packed = cq.cubic_pack(codes.to(DEV), bits)
    ref = oracle.pack(codes.numpy(), bits)
    assert np.array_equal(packed.cpu().numpy(), ref)
    # unpack of an arbitrary stream, including the extra field value -2^(B-1)
    raw = torch.randint(0, 256, (N * K * bits // 8,), generator=g).to(torch.uint8)
    out = cq.cubic_unpack(raw.to(DEV), N, K, bits)
    assert np.array_equal(out.cpu().numpy(), oracle.unpack(raw.numpy(), N, K, bits))


def test_pack_range_error_reported():
    say("pack range error")
    codes = torch.zeros((4, 64), dtype=torch.int8)
    codes[2, 5] = -2                                  # outside [-1, 1] for 2 bits
    with pytest.raises(cq.CubicError) as e:
        cq.cubic_pack(codes.to(DEV), 2)
    assert e.value.status == -6
    # the next valid call is clean again
    cq.cubic_pack(torch.zeros((4, 64), dtype=torch.int8, device=DEV), 2)


def test_pack_full_decode_weight():
    say("pack decode gate_up 6144x7168 W2")
    (w, _), _ = synth.decode_config(seed=2, device=DEV)
    packed = cq.cubic_pack(w.codes, 2)
    ref = oracle.pack(w.codes.cpu().numpy(), 2)
    assert np.array_equal(packed.cpu().numpy(), ref)


def _dequant_check(w: synth.Weight):
    codes, scales, shapes = np_weight(w)
    packed = cq.cubic_pack(w.codes.to(DEV), w.bits)
    cw = cq.CubicWeight(packed.reshape(-1), w.scales.to(DEV), w.shapes.to(DEV), w.N, w.K, w.bits, w.group)
    got32 = cq.cubic_dequant(cw).cpu().numpy()
    exact = oracle.dequant_f32(codes, scales, shapes, w.bits, w.group)
    assert np.array_equal(got32.view(np.uint32), exact.view(np.uint32))
    got = got32.astype(np.float64)
    ref = oracle.dequant(codes, scales, shapes, w.bits, w.group)
    assert np.all(np.abs(got - ref) <= ulp32(ref)), float((np.abs(got - ref) / ulp32(ref)).max())
    z = codes == 0
    assert np.all(got[z] == 0.0) and not np.signbit(got[z]).any()
    km = (1 << (w.bits - 1)) - 1
    s_full = np.repeat(scales, w.group, axis=1).astype(np.float64)
    ext = np.abs(codes.astype(np.int64)) == km
    assert np.array_equal(np.abs(got[ext]), s_full[ext])
    return got, ref


@pytest.mark.parametrize("bits", range(2, 9))
def test_dequant_within_one_ulp(bits):
    say(f"dequant bits={bits}")
    g = synth.make_generator(50 + bits)
    w = synth.make_weight(g, 40, 1024, bits, 256 if bits % 2 else 128, "uniform", 0.02)
    _dequant_check(w)


def test_dequant_uniform_int_bit_exact():
    say("dequant a=1 b=0")
    for bits in (2, 3, 4, 8):
        g = synth.make_generator(70 + bits)
        w = synth.make_weight(g, 16, 512, bits, 128, "uniform", 0.02)
        w.shapes[..., 0] = int(np.float16(1.0).view(np.int16))
        w.shapes[..., 1] = 0
        got, _ = _dequant_check(w)
        km = (1 << (bits - 1)) - 1
        codes, scales, _ = np_weight(w)
        s_full = np.repeat(scales, w.group, axis=1).astype(np.float64)
        want = (s_full * codes / km).astype(np.float32)       # RN32 of s*k/Kmax (see oracle pins)
        assert np.array_equal(got.astype(np.float32), want)


def test_dequant_single_workload_and_extra_code():
    say("dequant single workload W3 G128")
    w, _ = synth.single_config(seed=1)
    _dequant_check(w)


def test_dequant_extra_negative_code():
    say("dequant extra code -2^(B-1)")
    for bits in (2, 3, 4):
        g = torch.Generator().manual_seed(bits)
        N, K, G = 8, 256, 128
        raw = torch.randint(0, 256, (N * K * bits // 8,), generator=g).to(torch.uint8)
        codes = oracle.unpack(raw.numpy(), N, K, bits)
        sg = synth.make_generator(bits)
        scales = synth.lognormal_scales(sg, N * K // G, 0.02).reshape(N, K // G)
        shapes = synth.sample_shapes(sg, N * K // G).reshape(N, K // G, 2)
        cw = cq.CubicWeight(raw.to(DEV), scales.to(DEV), shapes.to(DEV), N, K, bits, G)
        got32 = cq.cubic_dequant(cw).cpu().numpy()
        exact = oracle.dequant_f32(codes, scales.numpy(), shapes.numpy().view(np.uint16), bits, G)
        assert np.array_equal(got32.view(np.uint32), exact.view(np.uint32))
        got = got32.astype(np.float64)
        ref = oracle.dequant(codes, scales.numpy(), shapes.numpy().view(np.uint16), bits, G)
        assert np.all(np.abs(got - ref) <= ulp32(ref))


def _midpoint_groups(bits, n, seed):
    """(s, a, b) for n groups, each with a level s * q_j that lies exactly on the
    midpoint between two neighbouring fp32 numbers, so that only the tie rule
    decides its rounding. With s = Kmax^3 * m * 2^e (m odd) the level is the dyadic
    number m * R_j * 2^(e - 24), R_j = Kmax^3 * q_j * 2^24 an integer; it is a
    midpoint when that product has exactly 25 significant bits."""
    rng = np.random.default_rng(seed)
    km = oracle.kmax(bits)
    D = km ** 3
    mmax = (1 << 24) // D                            # s = D * m stays exact in fp32
    s = np.empty(n, np.float32)
    ab = np.empty((n, 2), np.float16)
    i = 0
    while i < n:
        a, b = np.float16(rng.uniform(0, 4)), np.float16(rng.uniform(-6.5, 3))
        j = int(rng.integers(1, km))
        A, B = int(float(a) * 2 ** 24), int(float(b) * 2 ** 24)
        R = abs(A * j * km * km + B * j * j * km + ((1 << 24) - A - B) * j ** 3)
        if R == 0:
            continue
        Rodd = R >> ((R & -R).bit_length() - 1)
        want = 25 - Rodd.bit_length()                # bits of m for a 25-bit product
        if want < 1 or (1 << (want - 1)) > mmax:
            continue
        for _ in range(64):
            m = int(rng.integers(1 << (want - 1), min(1 << want, mmax + 1))) | 1
            if (m * Rodd).bit_length() == 25:
                break
        else:
            continue
        s[i] = np.float32(D * m * 2.0 ** int(rng.integers(-50, -20)))
        ab[i] = [a, b]
        i += 1
    return s, ab


@pytest.mark.parametrize("bits", [3, 4, 5, 8])
def test_dequant_exact_rounding_near_fp32_midpoints(bits):
    """Scales that put levels on or next to fp32 rounding midpoints, and shape
    values outside the monotone box (|a|, |b| up to the fp16 range), subnormal
    and huge scales: every value equals the correctly rounded level."""
    say(f"dequant rounding edge cases bits={bits}")
    km = oracle.kmax(bits)
    N, G = 16, 128
    K = G * 8
    s, ab = _midpoint_groups(bits, N * 8, 500 + bits)
    rng = np.random.default_rng(600 + bits)
    ab[:8] = rng.uniform(-3e4, 3e4, (8, 2)).astype(np.float16)          # wide shapes: the integer path
    s[8:12] = np.array([1e-45, 3e-42, 2.5e-39, 1.2e-38], np.float32)    # subnormal and tiny scales
    s[12:14] = np.array([3.0e38, -2.0e38], np.float32)                   # levels beyond fp32 overflow
    codes = rng.integers(-km, km + 1, (N, K)).astype(np.int8)
    scales = s.reshape(N, 8)
    shapes = ab.view(np.uint16).reshape(N, 8, 2)
    cw = cq.CubicWeight(cq.cubic_pack(torch.from_numpy(codes).to(DEV), bits).reshape(-1),
                        torch.from_numpy(scales).to(DEV), torch.from_numpy(shapes.view(np.int16)).to(DEV),
                        N, K, bits, G)
    got = cq.cubic_dequant(cw).cpu().numpy()
    exact = oracle.dequant_f32(codes, scales, shapes, bits, G)
    assert np.array_equal(got.view(np.uint32), exact.view(np.uint32))

"""GPU parity of cubic_encode: the device encoder gives the oracle's codes bit
for bit. Both choose the nearest of the format's fp32 levels (the values
cubic_dequant returns) by exact distance, the smaller |k| on ties, so the codes
are unique whatever the arithmetic order."""
import numpy as np
import pytest
import torch

import dequant_gemm_amd as cq
import oracle
import synth
from tests._gpu import DEV, np_weight, say

pytestmark = pytest.mark.gpu


def _params(N, K, bits, group, seed):
    g = synth.make_generator(seed)
    w = synth.make_weight(g, N, K, bits, group, "uniform", 0.02)
    return w.scales, w.shapes


def _encode_both(x, scales, shapes, bits, group):
    codes = cq.cubic_encode(x.to(DEV), scales.to(DEV), shapes.to(DEV), bits, group).cpu().numpy()
    ref = oracle.encode(x.numpy(), scales.numpy(), shapes.numpy().view(np.uint16), bits, group)
    return codes, ref


@pytest.mark.parametrize("bits,group", [(2, 512), (3, 128), (3, 256), (4, 128), (5, 256), (6, 128), (8, 128)])
def test_encode_matches_oracle(bits, group):
    say(f"encode bits={bits} G={group}")
    N, K = 203, 1024
    scales, shapes = _params(N, K, bits, group, 9000 + bits)
    g = torch.Generator().manual_seed(bits)
    x = torch.randn((N, K), generator=g) * 0.03
    x[:, ::97] *= 20.0                               # outliers beyond the largest level
    x[0, :64] = 0.0
    x[1, :64] = -0.0
    codes, ref = _encode_both(x, scales, shapes, bits, group)
    assert np.array_equal(codes, ref)


def test_encode_ties_signs_and_degenerate_scales():
    say("encode ties, signs, degenerate scales")
    bits, group, N, K = 3, 128, 4, 256
    scales, shapes = _params(N, K, bits, group, 9100)
    scales[1] = -scales[1]                            # negative scales flip the codes
    scales[2, 0] = 0.0                                # all levels zero
    ab = shapes.numpy().view(np.uint16)
    v = oracle.format_levels(scales.numpy()[0, 0], oracle.f16_bits_to_f64(ab[0, 0, 0]),
                             oracle.f16_bits_to_f64(ab[0, 0, 1]), bits)
    x = torch.randn((N, K), generator=torch.Generator().manual_seed(7)) * 0.03
    for j in range(1, oracle.kmax(bits) + 1):           # exact midpoints 0|1 and the levels themselves
        x[0, 2 * j] = float(v[j])
        x[0, 2 * j + 1] = -float(v[j])
    x[0, 0] = float(v[1] / np.float32(2))
    x[0, 1] = -float(v[1] / np.float32(2))
    x[3, 5] = float("nan")                            # a NaN weight takes code 0
    codes, ref = _encode_both(x, scales, shapes, bits, group)
    assert np.array_equal(codes, ref)
    assert codes[0, 0] == 0 and codes[0, 1] == 0 and codes[3, 5] == 0
    assert not codes[2, :group].any()


def _neighbours(v):
    """fp32 values just below and above v, and the exact midpoint between the
    levels u < v when it is an fp32 number."""
    v = np.float32(v)
    return [np.nextafter(v, np.float32(-np.inf)), v, np.nextafter(v, np.float32(np.inf))]


@pytest.mark.parametrize("bits", [3, 4, 8])
def test_encode_exact_distances_at_level_midpoints(bits):
    """Weights on, next to and exactly between neighbouring levels (the exact
    midpoint of two fp32 levels is a tie: the smaller |k| wins), levels that sit
    on fp32 rounding midpoints, and weights 2^30 and more above tiny levels (where
    a float64 difference would round): codes bit for bit the oracle's."""
    say(f"encode level midpoints bits={bits}")
    km = oracle.kmax(bits)
    group, G = 128, 6
    N, K = 8, 128 * G
    rng = np.random.default_rng(9400 + bits)
    s = np.exp(np.log(0.02) + 0.3 * rng.standard_normal((N, G))).astype(np.float32)
    ab = np.stack([rng.uniform(0.2, 3, (N, G)), rng.uniform(-1, 1.5, (N, G))], -1).astype(np.float16)
    s[0, 0] = np.float32(2.0 ** -100)                  # tiny levels against O(1) weights
    s[1, 0] = np.float32(1e-40)                        # subnormal scale
    lv = oracle.format_levels(s, ab[..., 0].astype(np.float64), ab[..., 1].astype(np.float64), bits)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    for n in range(N):
        for g in range(G):
            base = g * group
            cands = []
            for j in range(1, km + 1):
                u, v = np.float64(lv[n, g, j - 1]), np.float64(lv[n, g, j])
                mid = (u + v) / 2
                cands += _neighbours(v)
                if np.float64(np.float32(mid)) == mid:
                    cands += _neighbours(mid)
            cands = cands[:group]
            w[n, base:base + len(cands)] = np.array(cands, np.float32) * np.where(rng.random(len(cands)) < .5, 1, -1)
    w[0, :8] = np.array([1.0, -3.0, 0.5, 2.0 ** 40, -7.0, 1e-30, 2.0 ** -90, 3e38], np.float32)
    scales, shapes = torch.from_numpy(s), torch.from_numpy(ab.view(np.int16))
    codes, ref = _encode_both(torch.from_numpy(w), scales, shapes, bits, group)
    assert np.array_equal(codes, ref)


@pytest.mark.parametrize("bits,group", [(2, 512), (4, 128), (8, 256)])
def test_encode_round_trip_through_device_dequant(bits, group):
    say(f"encode round trip bits={bits}")
    N, K = 96, 1536
    g = synth.make_generator(9200 + bits)
    w = synth.make_weight(g, N, K, bits, group, "ternary" if bits == 2 else "uniform", 0.02)
    cw = cq.CubicWeight(cq.cubic_pack(w.codes.to(DEV), bits).reshape(-1), w.scales.to(DEV), w.shapes.to(DEV),
                        N, K, bits, group)
    W = cq.cubic_dequant(cw)
    codes = cq.cubic_encode(W, w.scales.to(DEV), w.shapes.to(DEV), bits, group)
    assert torch.equal(codes.cpu(), w.codes)


def test_encode_full_shape_sampled_rows():
    """gate_up 6144 x 7168, W4 G128 (the small-batch weight shape)."""
    say("encode 6144x7168 W4 G128 (sampled rows)")
    N, K, bits, group = 6144, 7168, 4, 128
    scales, shapes = _params(N, K, bits, group, 9300)
    x = torch.randn((N, K), generator=torch.Generator().manual_seed(3)) * 0.03
    codes = cq.cubic_encode(x.to(DEV), scales.to(DEV), shapes.to(DEV), bits, group).cpu().numpy()
    rows = np.array([0, 1, 2047, 4096, 6143])
    ref = oracle.encode(x.numpy()[rows], scales.numpy()[rows], shapes.numpy().view(np.uint16)[rows], bits, group)
    assert np.array_equal(codes[rows], ref)

"""GPU parity of the prefill-sized A16 product (M >= 256, 2- and 3-bit codes),
which runs on the 256 x 256 tile kernel, against the float64 oracle.

Bar: per-row infinity-norm relative error <= 2e-3. Shapes span several tiles in
both directions with ragged tails (N not a multiple of 4 exercises the scalar
epilogue), and the format's edge cases: extra negative codes, group scales far
outside fp16's range, activation rows far outside it."""
import numpy as np
import pytest
import torch

import dequant_gemm_amd as cq
import oracle
import synth
from tests._gpu import DEV, np_weight, row_rel_err, say, upload, x_bits

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _ref(w, x):
    codes, scales, shapes = np_weight(w)
    return oracle.gemm_a16(x_bits(x), oracle.dequant(codes, scales, shapes, w.bits, w.group))


@pytest.mark.parametrize("bits,group", [(2, 512), (2, 128), (3, 128), (3, 256)])
@pytest.mark.parametrize("M,N", [(256, 256), (300, 203), (520, 516)])
def test_prefill_tiles_ragged(bits, group, M, N):
    say(f"prefill ragged bits={bits} G={group} M={M} N={N}")
    g = synth.make_generator(3000 + 10 * bits + M + N)
    kind = "ternary" if bits == 2 else "uniform"
    K = 1536
    w = synth.make_weight(g, N, K, bits, group, kind, 0.02)
    x = synth.activations(g, M, K, 0.005, 30.0)
    cw = upload(w)
    y = cq.cubic_gemm_a16(x.to(DEV), cw)
    assert torch.equal(y, cq.cubic_gemm_a16(x.to(DEV), cw))
    assert row_rel_err(y.cpu().numpy(), _ref(w, x)) <= TOL


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("K", [1664, 1920])
def test_prefill_step_tails(bits, K):
    """K / 64 steps not a multiple of the 4-step unroll (groups are multiples
    of 128, so two steps are left over)."""
    say(f"prefill tails bits={bits} K={K}")
    g = synth.make_generator(3500 + 10 * bits + K)
    kind = "ternary" if bits == 2 else "uniform"
    w = synth.make_weight(g, 203, K, bits, 128, kind, 0.02)
    x = synth.activations(g, 300, K, 0.005, 30.0)
    cw = upload(w)
    y = cq.cubic_gemm_a16(x.to(DEV), cw)
    assert row_rel_err(y.cpu().numpy(), _ref(w, x)) <= TOL


def _raw_weight(bits, G, N, K, seed):
    gen = torch.Generator().manual_seed(seed)
    raw = torch.randint(0, 256, (N * K * bits // 8,), generator=gen).to(torch.uint8)
    sg = synth.make_generator(seed + 10)
    scales = synth.lognormal_scales(sg, N * K // G, 0.02).reshape(N, K // G)
    shapes = synth.sample_shapes(sg, N * K // G).reshape(N, K // G, 2)
    return raw, oracle.unpack(raw.numpy(), N, K, bits), scales, shapes, sg


@pytest.mark.parametrize("factor", [1.0, 5e7, 5e-7])
@pytest.mark.parametrize("bits,G", [(2, 256), (3, 128)])
def test_prefill_extra_codes_and_scale_range(bits, G, factor):
    """Every field value including -2^(B-1), with all group scales multiplied by
    factor: 5e7 puts s*q far above fp16's largest value, 5e-7 far below its
    smallest normal; the per-row power of two must keep the levels in range."""
    say(f"prefill extra codes bits={bits} scale x{factor}")
    N, K, M = 260, 1024, 272
    raw, codes, scales, shapes, sg = _raw_weight(bits, G, N, K, bits + 20)
    scales *= factor
    cw = cq.CubicWeight(raw.to(DEV), scales.to(DEV), shapes.to(DEV), N, K, bits, G)
    x = synth.activations(sg, M, K)
    y = cq.cubic_gemm_a16(x.to(DEV), cw).cpu().numpy()
    W = oracle.dequant(codes, scales.numpy(), shapes.numpy().view(np.uint16), bits, G)
    assert row_rel_err(y, oracle.gemm_a16(x_bits(x), W)) <= TOL


def test_prefill_rows_with_different_scale_ranges():
    """Weight rows 1e7x and 1e-7x apart in one tile, and a row with one huge
    group. With such columns the per-row metric measures cancellation in the one
    dominant column, so each column is checked against its own largest value."""
    say("prefill mixed scale ranges per column")
    bits, G, N, K, M = 3, 128, 260, 1024, 272
    raw, codes, scales, shapes, sg = _raw_weight(bits, G, N, K, 40)
    scales[0] *= 5e7
    scales[1] *= 5e-7
    scales[2, 0] *= 1e5
    cw = cq.CubicWeight(raw.to(DEV), scales.to(DEV), shapes.to(DEV), N, K, bits, G)
    x = synth.activations(sg, M, K)
    y = cq.cubic_gemm_a16(x.to(DEV), cw).cpu().numpy()
    W = oracle.dequant(codes, scales.numpy(), shapes.numpy().view(np.uint16), bits, G)
    ref = oracle.gemm_a16(x_bits(x), W)
    col_err = np.abs(y - ref).max(0) / np.abs(ref).max(0)
    assert col_err.max() <= TOL, col_err.max()


def test_prefill_activation_extremes_and_zero_rows():
    say("prefill activation range extremes")
    g = synth.make_generator(91)
    w = synth.make_weight(g, 300, 1024, 3, 256, "uniform", 0.02)
    x = torch.randn((300, 1024), generator=g).float()
    x[0] *= 1e6
    x[1] *= 1e-30
    x[2] = 0.0
    x[257] *= 3e4
    xb = x.to(torch.bfloat16)
    y = cq.cubic_gemm_a16(xb.to(DEV), upload(w)).cpu().numpy()
    assert np.all(y[2] == 0.0)
    assert row_rel_err(y, _ref(w, xb)) <= TOL


def test_prefill_uniform_int_special_case():
    """a = 1, b = 0: the product is a symmetric-INT matmul with per-group scales."""
    say("prefill a=1 b=0 vs integer matmul")
    g = synth.make_generator(78)
    N, K, M, G = 264, 1024, 288, 128
    w = synth.make_weight(g, N, K, 3, G, "uniform", 0.02)
    w.shapes[..., 0] = int(np.float16(1.0).view(np.int16))
    w.shapes[..., 1] = 0
    x = synth.activations(g, M, K)
    y = cq.cubic_gemm_a16(x.to(DEV), upload(w)).cpu().numpy()
    codes, scales, _ = np_weight(w)
    X = oracle.bf16_bits_to_f64(x_bits(x))
    ref = np.zeros((M, N))
    for gi in range(K // G):
        sl = slice(gi * G, (gi + 1) * G)
        ref += (X[:, sl] @ codes[:, sl].T.astype(np.float64)) * (scales[:, gi] / 3.0)[None, :]
    assert row_rel_err(y, ref) <= TOL


def test_prefill_full_shape_tile_edges():
    """6144 x 7168 W3 G256 at M = 4096: rows on both sides of every 256-row tile
    edge of two tiles, all columns."""
    say("prefill W3 G256 6144x7168 M=4096 tile-edge rows")
    w, x = synth.prefill_config(seed=5, device=DEV)
    cw = upload(w)
    y = cq.cubic_gemm_a16(x, cw).cpu().numpy()
    rows = np.array([255, 256, 511, 512, 3839, 3840, 4094])
    codes, scales, shapes = np_weight(w)
    ref = oracle.gemm_a16(x_bits(x)[rows], oracle.dequant(codes, scales, shapes, 3, 256))
    assert row_rel_err(y[rows], ref) <= TOL


def test_prefill_half_tiles_of_the_last_round():
    """4352 x 4096 makes 272 tiles of 256 x 256: on a 256-CU part the last 16
    run as 32 half tiles of 128 activation rows. Rows on both sides of every
    half-tile edge of that region, all columns."""
    say("prefill half tiles 4352x4096 W2 G256 K=512")
    g = synth.make_generator(4242)
    M, N, K = 4352, 4096, 512
    w = synth.make_weight(g, N, K, 2, 256, "ternary", 0.02)
    x = synth.activations(g, M, K, 0.005, 30.0)
    cw = upload(w)
    y = cq.cubic_gemm_a16(x.to(DEV), cw).cpu().numpy()
    rows = np.array([0, 4095, 4096, 4223, 4224, 4300, 4351])
    codes, scales, shapes = np_weight(w)
    ref = oracle.gemm_a16(x_bits(x)[rows], oracle.dequant(codes, scales, shapes, 2, 256))
    assert row_rel_err(y[rows], ref) <= TOL

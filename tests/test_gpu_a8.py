"""GPU parity of the Dynamic A8 path: act_quant_int8_per_token bit-exact against
the oracle, cubic_gemm_a8 within 2e-3 (per-row infinity norm)."""
import numpy as np
import pytest
import torch

import dequant_gemm_amd as cq
import oracle
import synth
from tests._gpu import DEV, np_weight, row_rel_err, say, upload, x_bits

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _bf16(t):
    return t.to(torch.bfloat16)


def test_act_quant_golden_row_and_ties():
    say("act_quant golden row")
    row = torch.tensor([[2.0, -1.0, 0.5, 0.0, 1.5, 0.0, 0.0, 0.0]])
    xq, sx = cq.act_quant_int8_per_token(_bf16(row).to(DEV))
    assert xq.cpu().tolist()[0][:5] == [127, -64, 32, 0, 95]
    assert format(int(sx.cpu().view(torch.int32)[0]) & 0xFFFFFFFF, "08x") == "3c810204"


@pytest.mark.parametrize("M,K", [(1, 8), (5, 520), (64, 7168), (4096, 7168)])
def test_act_quant_bit_exact(M, K):
    say(f"act_quant M={M} K={K}")
    g = torch.Generator().manual_seed(M + K)
    x = torch.randn((M, K), generator=g) * torch.exp(torch.randn((M, 1), generator=g) * 3)
    if M > 3:
        x[1] = 0.0
        x[2, : K // 2] *= 1e30
        x[3] *= 1e-35
    xb = _bf16(x)
    xq, sx = cq.act_quant_int8_per_token(xb.to(DEV))
    xq_ref, sx_ref = oracle.act_quant(x_bits(xb))
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), sx_ref.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), xq_ref)


def _quant_rows(K, seed):
    """Rows that exercise each rounding path of the quantiser: exact ties (scale
    1), near-ties at a random scale, scales below 2^-100, above 2^100 and
    denormal, a zero row and a single nonzero element."""
    g = torch.Generator().manual_seed(seed)
    rows = torch.zeros((8, K), dtype=torch.float64)
    rows[0] = torch.randn(K, generator=g, dtype=torch.float64)
    k = torch.arange(K, dtype=torch.float64) % 127
    sign = torch.where(torch.arange(K) % 2 == 0, 1.0, -1.0).to(torch.float64)
    rows[1] = sign * (k + 0.5)
    rows[1, 0] = 127.0
    s = float(torch.exp(torch.randn(1, generator=g, dtype=torch.float64)))
    delta = (torch.rand(K, generator=g, dtype=torch.float64) - 0.5) * 2e-3
    rows[2] = sign * (k + 0.5 + delta) * s
    rows[2, 0] = 127.0 * s
    rows[3] = torch.randn(K, generator=g, dtype=torch.float64) * 1e-32
    rows[4] = torch.randn(K, generator=g, dtype=torch.float64) * 1e33
    rows[5] = torch.randn(K, generator=g, dtype=torch.float64) * 1e-38
    rows[7, K // 3] = -3.0
    return rows.to(torch.bfloat16)


@pytest.mark.parametrize("K", [8, 2048, 2056, 7168, 16384, 16392])
def test_act_quant_rounding_paths(K):
    # K spans one to eight 16-byte vectors per thread and the two-pass fallback
    say(f"act_quant rounding paths K={K}")
    xb = _quant_rows(K, seed=K)
    xq, sx = cq.act_quant_int8_per_token(xb.to(DEV))
    xq_ref, sx_ref = oracle.act_quant(x_bits(xb))
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), sx_ref.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), xq_ref)


def _check_a8(w, x, rows=None):
    cw = upload(w)
    xq, sx = cq.act_quant_int8_per_token(x.to(DEV))
    y = cq.cubic_gemm_a8(xq, sx, cw)
    y2 = cq.cubic_gemm_a8(xq, sx, cw)
    assert torch.equal(y, y2)
    codes, scales, shapes = np_weight(w)
    xb = x_bits(x)
    yn = y.cpu().numpy()
    if rows is not None:
        xb, yn = xb[rows], yn[rows]
    xq_ref, sx_ref = oracle.act_quant(xb)
    if rows is not None:
        assert np.array_equal(xq.cpu().numpy()[rows], xq_ref)
    ref = oracle.gemm_a8(xq_ref, sx_ref, codes, scales, shapes, w.bits, w.group)
    err = row_rel_err(yn, ref)
    assert err <= TOL, err


def test_prefill_a8_full_sampled_rows():
    say("A8 prefill W3 G256 6144x7168 M=4096 (sampled rows)")
    w, x = synth.prefill_config(seed=5, device=DEV)
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([[0, 4095], rng.choice(4096, 46, replace=False)]))
    _check_a8(w, x, rows=rows)


def test_single_workload_a8():
    say("A8 single W3 G128")
    w, x = synth.single_config(seed=1)
    _check_a8(w, x)


@pytest.mark.parametrize("bits,group", [(2, 512), (3, 256), (5, 128), (8, 1024)])
@pytest.mark.parametrize("M", [5, 16, 40])
def test_a8_small_batch_long_rows(bits, group, M):
    """K = 16384: sixteen activation rows of a K quarter no longer fit the LDS, so
    the small-batch A8 kernel falls back to four-row passes; N = 75 leaves a
    ragged last tile."""
    say(f"A8 small batch long rows bits={bits} G={group} M={M}")
    g = synth.make_generator(2600 + 10 * bits + M)
    kind = "ternary" if bits == 2 else "uniform"
    w = synth.make_weight(g, 75, 16384, bits, group, kind, 0.02)
    x = synth.activations(g, M, 16384, 0.005, 30.0)
    _check_a8(w, x)


@pytest.mark.parametrize("bits,group,kind", [(2, 512, "ternary"), (4, 128, "uniform"), (8, 128, "uniform")])
@pytest.mark.parametrize("M", [1, 5, 16])
def test_a8_small_batch_full_shape(bits, group, kind, M):
    """The small-batch A8 product at the gate_up expert shape (6144 x 7168), in
    every launch configuration it takes there (one, four and sixteen rows a
    pass): all rows against the oracle on the first and last 256 weight rows
    and 64 spread ones."""
    say(f"A8 small batch W{bits} G{group} gate_up 6144x7168 M={M}")
    g = synth.make_generator(1700 + bits + M, DEV)
    w = synth.make_weight(g, 6144, 7168, bits, group, kind, 0.02, DEV)
    x = synth.activations(g, M, 7168, 0.005, 30.0, DEV)
    cw = upload(w)
    xq, sx = cq.act_quant_int8_per_token(x)
    y = cq.cubic_gemm_a8(xq, sx, cw).cpu().numpy()
    cols = np.unique(np.r_[0:256, 6144 - 256:6144, np.random.default_rng(M).integers(0, 6144, 64)])
    codes, scales, shapes = np_weight(w)
    xq_ref, sx_ref = oracle.act_quant(x_bits(x.cpu()))
    assert np.array_equal(xq.cpu().numpy(), xq_ref)
    ref = oracle.gemm_a8(xq_ref, sx_ref, codes[cols], scales[cols], shapes[cols], bits, group)
    err = row_rel_err(y[:, cols], ref)
    assert err <= TOL, err


@pytest.mark.parametrize("bits,group", [(2, 128), (2, 256), (2, 512), (3, 128), (3, 256), (3, 512),
                                        (3, 1024), (4, 128), (5, 128), (6, 256), (7, 128), (8, 1024)])
@pytest.mark.parametrize("M", [1, 4, 7, 16, 40, 130, 300])
def test_a8_ragged(bits, group, M):
    say(f"A8 ragged bits={bits} G={group} M={M}")
    g = synth.make_generator(2000 + 10 * bits + M)
    kind = "ternary" if bits == 2 else "uniform"
    w = synth.make_weight(g, 203, 2048, bits, group, kind, 0.02)
    x = synth.activations(g, M, 2048, 0.005, 30.0)
    _check_a8(w, x)


def test_a8_carrier_ties_both_directions():
    """a=2, b=-1.75 (W3): q(1/3) = 1/2 gives carrier 64 (a tie); a=3.625, b=-1.5:
    code -4 has q(4/3) = -1/2, carrier -(-64) = 64. Half-up rounding would move
    either by one unit (1.6 %), far beyond the 2e-3 bar."""
    for a, b, kset in ((2.0, -1.75, (-1, 1)), (3.625, -1.5, (-4,))):
        say(f"A8 carrier tie a={a} b={b}")
        N, K, G = 32, 256, 128
        g = torch.Generator().manual_seed(3)
        codes = torch.tensor(kset, dtype=torch.int64)[torch.randint(0, len(kset), (N, K), generator=g)]
        field = (codes & 7).numpy().astype(np.int64)
        stream = np.zeros(N * K * 3 // 8, dtype=np.uint8)
        bitpos = np.arange(N * K) * 3
        for i in range(3):
            bit = (field.reshape(-1) >> i) & 1
            p = bitpos + i
            np.add.at(stream, p // 8, (bit << (p % 8)).astype(np.uint8))
        shapes = torch.zeros((N, K // G, 2), dtype=torch.int16)
        shapes[..., 0] = int(np.float16(a).view(np.int16))
        shapes[..., 1] = int(np.float16(b).view(np.int16))
        scales = torch.full((N, K // G), 0.02, dtype=torch.float32)
        cw = cq.CubicWeight(torch.from_numpy(stream).to(DEV), scales.to(DEV), shapes.to(DEV), N, K, 3, G)
        x = synth.activations(synth.make_generator(4), 4, K)
        xq, sx = cq.act_quant_int8_per_token(x.to(DEV))
        y = cq.cubic_gemm_a8(xq, sx, cw).cpu().numpy()
        cn = oracle.unpack(stream, N, K, 3)
        xq_ref, sx_ref = oracle.act_quant(x_bits(x))
        ref = oracle.gemm_a8(xq_ref, sx_ref, cn, scales.numpy(), shapes.numpy().view(np.uint16), 3, G)
        assert row_rel_err(y, ref) <= 1e-5


# fp16 shapes on which a carrier is an exact tie (127 q_j = n + 1/2), found by an
# exact rational search: (a, b) for 3-, 5-, 7- and 8-bit codes
TIE_SHAPES = {3: [(2.0, -1.75)], 5: [(1.900390625, 3.97265625)], 7: [(0.57421875, 3.953125)],
              8: [(1.955078125, 3.26171875), (2.802734375, -1.05859375)]}


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_a8_carriers_exact_through_identity_rows(bits):
    """Every carrier the device uses, read back exactly: xq = the K x K identity
    (x_scale 1) gives y[k][n] = fp32(s / 127) * C(n, k), so C is recovered by one
    division and must equal the oracle's carrier (exact integer rounding, ties to
    even, clamps, the extra code -2^(B-1)) for every weight. Rows carry planted
    tie shapes; codes cover every field value."""
    say(f"A8 carriers exact via identity rows bits={bits}")
    N, K, G = 48, 256, 128
    rng = np.random.default_rng(4000 + bits)
    lo = -(1 << (bits - 1))
    codes = rng.integers(lo, -lo, size=(N, K)).astype(np.int8)
    sg = synth.make_generator(4100 + bits)
    scales = synth.lognormal_scales(sg, N * (K // G), 0.02).reshape(N, K // G)
    shapes = synth.sample_shapes(sg, N * (K // G)).reshape(N, K // G, 2).numpy().view(np.uint16).copy()
    for i, (a, b) in enumerate(TIE_SHAPES.get(bits, [])):
        shapes[4 * i:4 * i + 4, :, 0] = np.float16(a).view(np.uint16)
        shapes[4 * i:4 * i + 4, :, 1] = np.float16(b).view(np.uint16)
    from tests._gpu import pack_fields
    cw = cq.CubicWeight(torch.from_numpy(pack_fields(codes, bits).reshape(-1)).to(DEV), scales.to(DEV),
                        torch.from_numpy(shapes.view(np.int16)).to(DEV), N, K, bits, G)
    xq = torch.eye(K, dtype=torch.int8, device=DEV)
    sx = torch.ones(K, dtype=torch.float32, device=DEV)
    y = cq.cubic_gemm_a8(xq, sx, cw).cpu().numpy().astype(np.float64)      # [K][N]
    sc = (scales.numpy() / np.float32(127.0)).astype(np.float32).astype(np.float64)   # fp32(s / 127)
    unit = np.repeat(sc, G, axis=1).T                                       # [K][N]
    C = y / unit
    Ci = np.rint(C)
    assert np.abs(C - Ci).max() < 1e-3
    want = oracle.carrier_codes(codes, shapes, bits, G).T
    assert np.array_equal(Ci.astype(np.int64), want)
    # the same read-back through the small-batch kernel: 16 identity rows a call
    for k0 in range(0, K, 16):
        ys = cq.cubic_gemm_a8(xq[k0:k0 + 16].contiguous(), sx[:16].contiguous(), cw).cpu().numpy()
        Cs = ys.astype(np.float64) / unit[k0:k0 + 16]
        assert np.abs(Cs - np.rint(Cs)).max() < 1e-3
        assert np.array_equal(np.rint(Cs).astype(np.int64), want[k0:k0 + 16]), k0

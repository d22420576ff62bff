"""GPU parity of the A16 product (cubic_gemm_a16) against the float64 oracle.

Bar: per-row infinity-norm relative error <= 2e-3 (an all-zero reference row must
come back exactly zero), on every workload at full size, on small shapes that
span several tiles with ragged tails, and on the edge cases of the format."""
import numpy as np
import pytest
import torch

import dequant_gemm_amd as cq
import oracle
import synth
from tests._gpu import DEV, np_weight, pack_fields, row_rel_err, say, upload, x_bits

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _check(w: synth.Weight, x: torch.Tensor, rows=None, tol=TOL):
    cw = upload(w)
    y = cq.cubic_gemm_a16(x.to(DEV), cw)
    y2 = cq.cubic_gemm_a16(x.to(DEV), cw)
    assert torch.equal(y, y2), "repeat call not bitwise identical"
    yn = y.cpu().numpy()
    codes, scales, shapes = np_weight(w)
    xb = x_bits(x)
    if rows is not None:
        xb, yn = xb[rows], yn[rows]
    ref = oracle.gemm_a16(xb, oracle.dequant(codes, scales, shapes, w.bits, w.group))
    err = row_rel_err(yn, ref)
    assert err <= tol, err
    return err


def test_single_workload_w3g128():
    say("A16 single W3 G128 256x512 M=4")
    w, x = synth.single_config(seed=1)
    _check(w, x)


def test_decode_workload_full():
    for (w, x), name in zip(synth.decode_config(seed=2, device=DEV), ("gate_up", "down")):
        say(f"A16 decode W2 G512 {name} {w.N}x{w.K} M=1")
        _check(w, x)


@pytest.mark.parametrize("M", [8, 64])
def test_smallm_workload_full(M):
    for (w, x), name in zip(synth.smallm_config(M, seed=3, device=DEV), ("gate_up", "down")):
        say(f"A16 small-M W4 G128 {name} {w.N}x{w.K} M={M}")
        _check(w, x)


def test_prefill_workload_full_sampled_rows():
    say("A16 prefill W3 G256 6144x7168 M=4096 (sampled rows)")
    w, x = synth.prefill_config(seed=5, device=DEV)
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, 1, 4095], rng.choice(4096, 45, replace=False)]))
    _check(w, x, rows=rows)


@pytest.mark.parametrize("bits,group", [(2, 512), (2, 128), (3, 128), (3, 256), (4, 128),
                                        (5, 256), (6, 128), (7, 128), (8, 256)])
@pytest.mark.parametrize("M", [1, 3, 4, 5, 8, 9, 16, 17, 65, 100, 256])
def test_small_shapes_ragged(bits, group, M):
    # N not a multiple of 16 or of 128, K spanning several groups and waves
    say(f"A16 ragged bits={bits} G={group} M={M}")
    g = synth.make_generator(1000 + 10 * bits + M)
    kind = "ternary" if bits == 2 else "uniform"
    w = synth.make_weight(g, 203, 1536, bits, group, kind, 0.02)
    x = synth.activations(g, M, 1536, 0.01, 50.0)
    _check(w, x)


@pytest.mark.parametrize("bits,group", [(5, 128), (6, 256), (7, 128), (8, 128), (8, 1024)])
@pytest.mark.parametrize("M", [17, 32, 33, 64, 130])
def test_small_batch_wide_codes(bits, group, M):
    # 5- to 8-bit codes at 17..64 rows (the small-batch kernel: level tables up to
    # 6 bits, levels computed per code for 7 and 8 bits; one or two 32-row blocks);
    # N not a multiple of the 32-row tile, K over several groups and waves
    say(f"A16 small batch wide codes bits={bits} G={group} M={M}")
    g = synth.make_generator(1500 + 10 * bits + M)
    w = synth.make_weight(g, 203, 4096, bits, group, "uniform", 0.02)
    x = synth.activations(g, M, 4096, 0.01, 50.0)
    _check(w, x)


def test_small_batch_wide_codes_full_shape():
    # 130 rows: three passes of the small-batch kernel (64, 64, 2 rows)
    for bits in (5, 8):
        for M in (24, 64, 130):
            say(f"A16 small batch W{bits} G128 gate_up 6144x7168 M={M}")
            g = synth.make_generator(1600 + bits + M, DEV)
            w = synth.make_weight(g, 6144, 7168, bits, 128, "uniform", 0.02, DEV)
            x = synth.activations(g, M, 7168, 0.01, 50.0, DEV)
            rows = np.unique(np.r_[0:3, 63, 64, 127:M, np.random.default_rng(M).integers(0, M, 4)])
            rows = rows[rows < M]
            _check_rows_cols(w, x, rows)


def _check_rows_cols(w, x, rows, cols=None):
    """Sampled outputs of a large product: rows `rows` against the oracle on
    weight rows `cols` (default: the first and last 256 and 64 spread rows)."""
    cw = upload(w)
    y = cq.cubic_gemm_a16(x.to(DEV), cw).cpu().numpy()
    N = w.N
    if cols is None:
        cols = np.unique(np.r_[0:256, N - 256:N, np.random.default_rng(7).integers(0, N, 64)])
    codes, scales, shapes = np_weight(w)
    W = oracle.dequant(codes[cols], scales[cols], shapes[cols], w.bits, w.group)
    ref = oracle.gemm_a16(x_bits(x)[rows], W)
    err = row_rel_err(y[rows][:, cols], ref)
    assert err <= TOL, err


def test_extra_negative_code_w2_w4_w8():
    # codes -2^(B-1) decode by the formula (t > 1); W2 exercises the slow path,
    # W8 the levels computed per code
    for bits in (2, 4, 8):
        say(f"A16 extra code bits={bits}")
        g = torch.Generator().manual_seed(bits)
        N, K, G = 64, 1024, 512 if bits == 2 else 128
        raw = torch.randint(0, 256, (N * K * bits // 8,), generator=g).to(torch.uint8)
        codes = oracle.unpack(raw.numpy(), N, K, bits)
        sg = synth.make_generator(bits + 10)
        scales = synth.lognormal_scales(sg, N * K // G, 0.02).reshape(N, K // G)
        shapes = synth.sample_shapes(sg, N * K // G).reshape(N, K // G, 2)
        cw = cq.CubicWeight(raw.to(DEV), scales.to(DEV), shapes.to(DEV), N, K, bits, G)
        for M in (1, 8, 40):
            x = synth.activations(sg, M, K)
            y = cq.cubic_gemm_a16(x.to(DEV), cw).cpu().numpy()
            W = oracle.dequant(codes, scales.numpy(), shapes.numpy().view(np.uint16), bits, G)
            assert row_rel_err(y, oracle.gemm_a16(x_bits(x), W)) <= TOL


def test_uniform_int_special_case_matches_integer_matmul():
    say("A16 a=1 b=0 vs integer matmul")
    g = synth.make_generator(77)
    w = synth.make_weight(g, 130, 1024, 3, 128, "uniform", 0.02)
    w.shapes[..., 0] = int(np.float16(1.0).view(np.int16))
    w.shapes[..., 1] = 0
    x = synth.activations(g, 3, 1024)
    y = cq.cubic_gemm_a16(x.to(DEV), upload(w)).cpu().numpy()
    codes, scales, _ = np_weight(w)
    X = oracle.bf16_bits_to_f64(x_bits(x))
    ref = np.zeros((3, 130))
    for gi in range(1024 // 128):
        sl = slice(gi * 128, (gi + 1) * 128)
        ref += (X[:, sl] @ codes[:, sl].T.astype(np.float64)) * (scales[:, gi] / 3.0)[None, :]
    assert row_rel_err(y, ref) <= TOL


@pytest.mark.parametrize("bits,group", [(2, 512), (4, 128)])
def test_activation_range_extremes_and_zero_rows(bits, group):
    # rows far outside the fp16 range, tiny rows, an all-zero row (M = 12 takes
    # the raw-bf16 GEMV for 4-bit codes)
    say(f"A16 activation range extremes bits={bits}")
    g = synth.make_generator(88)
    w = synth.make_weight(g, 96, 1024, bits, group, "ternary" if bits == 2 else "uniform", 0.015)
    cw = upload(w)
    for M in (4, 12, 130):
        x = torch.randn((M, 1024), generator=g).float()
        x[0] *= 1e6
        x[1] *= 1e-30
        x[2] = 0.0
        xb = x.to(torch.bfloat16)
        y = cq.cubic_gemm_a16(xb.to(DEV), cw).cpu().numpy()
        codes, scales, shapes = np_weight(w)
        ref = oracle.gemm_a16(x_bits(xb), oracle.dequant(codes, scales, shapes, bits, group))
        assert np.all(y[2] == 0.0)
        assert row_rel_err(y, ref) <= TOL


def test_empty_and_degenerate():
    say("A16 M=0 and N=1")
    g = synth.make_generator(99)
    w = synth.make_weight(g, 1, 512, 3, 128, "uniform", 0.02)
    cw = upload(w)
    y = cq.cubic_gemm_a16(torch.zeros((0, 512), dtype=torch.bfloat16, device=DEV), cw)
    assert y.shape == (0, 1)
    x = synth.activations(g, 2, 512)
    y = cq.cubic_gemm_a16(x.to(DEV), cw).cpu().numpy()
    codes, scales, shapes = np_weight(w)
    assert row_rel_err(y, oracle.gemm_a16(x_bits(x), oracle.dequant(codes, scales, shapes, 3, 128))) <= TOL


def test_workspace_too_small_is_rejected():
    say("A16 workspace check")
    g = synth.make_generator(5)
    w = synth.make_weight(g, 64, 512, 3, 128, "uniform", 0.02)
    cw = upload(w)
    x = synth.activations(g, 20, 512).to(DEV)
    with pytest.raises(cq.CubicError) as e:
        cq.cubic_gemm_a16(x, cw, workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    assert e.value.status == -7


@pytest.mark.parametrize("bits,group", [(2, 512), (3, 128)])
@pytest.mark.parametrize("M", [1, 3, 8])
def test_small_m_rows_per_workgroup_ragged(bits, group, M):
    """N = 4100 gives 257 tiles of 16 rows; on 256 CUs the small-M product then
    uses 9-row workgroups (456 of them, the last holding 5 rows)."""
    say(f"A16 small-M N=4100 bits={bits} G={group} M={M}")
    g = synth.make_generator(5000 + 10 * bits + M)
    kind = "ternary" if bits == 2 else "uniform"
    w = synth.make_weight(g, 4100, 1024, bits, group, kind, 0.02)
    x = synth.activations(g, M, 1024, 0.01, 50.0)
    _check(w, x)


@pytest.mark.parametrize("bits,group", [(2, 128), (2, 512), (3, 128), (3, 512), (4, 128), (4, 256)])
@pytest.mark.parametrize("M,N,K", [(17, 203, 512), (31, 64, 1536), (32, 4100, 1024), (33, 203, 1536),
                                   (64, 230, 3072)])
def test_small_batch_mfma_shapes(bits, group, M, N, K):
    """The small-batch MFMA kernel (2- to 4-bit codes, 17..64 rows): one and two
    32-row activation blocks, ragged N, few steps per wave."""
    say(f"A16 small batch bits={bits} G={group} M={M} N={N} K={K}")
    g = synth.make_generator(6000 + 10 * bits + M + N)
    w = synth.make_weight(g, N, K, bits, group, "uniform", 0.02)
    x = synth.activations(g, M, K, 0.01, 50.0)
    _check(w, x)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("K", [1664, 1920])
def test_small_batch_mfma_uneven_waves(bits, K):
    """K / 64 steps not divisible by the four waves (26 and 30 steps)."""
    say(f"A16 small batch uneven waves bits={bits} K={K}")
    g = synth.make_generator(6100 + 10 * bits + K)
    w = synth.make_weight(g, 96, K, bits, 128, "uniform", 0.02)
    x = synth.activations(g, 40, K, 0.01, 50.0)
    _check(w, x)


@pytest.mark.parametrize("factor", [5e7, 5e-7])
def test_small_batch_mfma_scale_range(factor):
    """Group scales far from 1: the tables hold normalised levels and the scale
    is applied in fp32, so the fp16 range does not matter."""
    say(f"A16 small batch scale x{factor}")
    g = synth.make_generator(6200)
    w = synth.make_weight(g, 203, 1024, 4, 128, "uniform", 0.02)
    w.scales = w.scales * factor
    x = synth.activations(g, 24, 1024, 0.01, 50.0)
    _check(w, x)


@pytest.mark.parametrize("M", [1, 8])
def test_sparse_extra_codes_w2(M):
    """Ternary 2-bit weights with a few codes -2 planted at scattered positions:
    most 128-code steps have none, some have one in only one of their halves."""
    say(f"A16 W2 sparse extra codes M={M}")
    g = synth.make_generator(321)
    N, K, G = 200, 2048, 512
    w = synth.make_weight(g, N, K, 2, G, "ternary", 0.02)
    codes = w.codes.cpu().numpy().copy()
    rng = np.random.default_rng(5)
    for n, k in zip(rng.integers(0, N, 40), rng.integers(0, K, 40)):
        codes[n, k] = -2
    codes[7, 0] = codes[7, 255] = codes[7, 256] = codes[7, K - 1] = -2
    raw = torch.from_numpy(pack_fields(codes, 2).reshape(-1))
    scales, shapes = w.scales.cpu().numpy(), w.shapes.cpu().numpy().view(np.uint16)
    cw = cq.CubicWeight(raw.to(DEV), w.scales.to(DEV), w.shapes.to(DEV), N, K, 2, G)
    x = synth.activations(g, M, K)
    y = cq.cubic_gemm_a16(x.to(DEV), cw).cpu().numpy()
    ref = oracle.gemm_a16(x_bits(x), oracle.dequant(codes, scales, shapes, 2, G))
    assert row_rel_err(y, ref) <= TOL

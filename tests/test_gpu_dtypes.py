"""GPU parity of the other activation and output types (CubicQuant article,
activation modes: A16 takes FP16 or BF16 activations; outputs in BF16).

- fp16 activations: every A16 kernel (in-kernel GEMV, prepared GEMV, small-batch,
  prefill, tiled) and the routed-expert product against the float64 oracle on
  the exact fp16 values, same per-row bar as bf16 (2e-3); the fp16 quantiser
  bit-exact against the oracle's rule.
- bf16 outputs: each kernel computes the fp32 result and rounds it once (nearest
  even), so a bf16 output must equal, bit for bit, the fp32 output of the same
  call rounded to bf16."""
import numpy as np
import pytest
import torch

import dequant_gemm_amd as cq
import oracle
import synth
from tests._gpu import DEV, np_weight, row_rel_err, say, upload, x_bits

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _f16_rows(M, K, seed):
    """fp16 activations of the bf16 workloads' distribution, rows of different
    magnitude up to near the fp16 limit, and an all-zero row."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((M, K), generator=g)
    mag = torch.tensor([1.0, 3e3, 0.02, 30.0, 1e-3])
    x *= mag[torch.arange(M) % 5][:, None]
    if M > 7:
        x[7] = 0.0
    if M > 2:
        x[2, ::97] = 6e4 / 8                       # a few large columns in one row
    return x.to(torch.float16)


def _dense(w):
    codes, scales, shapes = np_weight(w)
    return oracle.dequant(codes, scales, shapes, w.bits, w.group)


def _bf16_of(y32):
    return y32.to(torch.bfloat16)


# M picks the kernel: 1 and 4 the in-kernel GEMV, 8 and 16 the prepared GEMV (8 with
# 2-bit codes the reordered rows), 33 and 64 the small-batch kernel (2- to 4-bit),
# 300 the tiled kernel (or prefill where it applies), 17 with 5-bit codes the tiled.
@pytest.mark.parametrize("bits,group", [(2, 512), (2, 128), (3, 128), (4, 128), (5, 256), (8, 128)])
@pytest.mark.parametrize("M", [1, 4, 8, 16, 17, 33, 64, 100, 300])
def test_a16_fp16_activations(bits, group, M):
    say(f"A16 fp16 x bits={bits} G={group} M={M}")
    g = synth.make_generator(3000 + 10 * bits + M)
    w = synth.make_weight(g, 203, 1536, bits, group, "ternary" if bits == 2 else "uniform", 0.02)
    cw = upload(w)
    x = _f16_rows(M, 1536, 3100 + M)
    xd = x.to(DEV)
    y = cq.cubic_gemm_a16(xd, cw)
    assert torch.equal(y, cq.cubic_gemm_a16(xd, cw))
    ref = oracle.gemm_a16(x.view(torch.int16).numpy().view(np.uint16), _dense(w), fmt="f16")
    assert row_rel_err(y.cpu().numpy(), ref) <= TOL
    yb = cq.cubic_gemm_a16(xd, cw, out_dtype=torch.bfloat16)
    assert torch.equal(yb, _bf16_of(y))


@pytest.mark.parametrize("bits,group", [(2, 256), (3, 128)])
@pytest.mark.parametrize("M,N", [(256, 256), (520, 516)])
def test_prefill_fp16_activations(bits, group, M, N):
    say(f"A16 prefill fp16 x bits={bits} G={group} M={M} N={N}")
    g = synth.make_generator(3300 + bits + M)
    w = synth.make_weight(g, N, 2048, bits, group, "ternary" if bits == 2 else "uniform", 0.02)
    x = _f16_rows(M, 2048, 3400 + M)
    y = cq.cubic_gemm_a16(x.to(DEV), upload(w))
    ref = oracle.gemm_a16(x.view(torch.int16).numpy().view(np.uint16), _dense(w), fmt="f16")
    assert row_rel_err(y.cpu().numpy(), ref) <= TOL


@pytest.mark.parametrize("bits,group", [(2, 512), (3, 128), (4, 128), (6, 128)])
@pytest.mark.parametrize("M", [1, 3, 8, 16, 40, 100, 300])
def test_a16_bf16_outputs(bits, group, M):
    say(f"A16 bf16 out bits={bits} G={group} M={M}")
    g = synth.make_generator(3500 + 10 * bits + M)
    w = synth.make_weight(g, 203, 1536, bits, group, "ternary" if bits == 2 else "uniform", 0.02)
    cw = upload(w)
    x = synth.activations(g, M, 1536, 0.01, 50.0).to(DEV)
    y = cq.cubic_gemm_a16(x, cw)
    yb = cq.cubic_gemm_a16(x, cw, out_dtype=torch.bfloat16)
    assert yb.dtype == torch.bfloat16
    assert torch.equal(yb, _bf16_of(y))
    ref = oracle.gemm_a16(x_bits(x), _dense(w))
    assert row_rel_err(yb.float().cpu().numpy(), ref) <= TOL + 2.0 ** -8


def test_prefill_workload_bf16_output_full():
    say("A16 prefill W3 G256 6144x7168 M=4096 bf16 out")
    w, x = synth.prefill_config(seed=5, device=DEV)
    cw = upload(w)
    y = cq.cubic_gemm_a16(x, cw)
    yb = cq.cubic_gemm_a16(x, cw, out_dtype=torch.bfloat16)
    assert torch.equal(yb, _bf16_of(y))


@pytest.mark.parametrize("M,K", [(1, 8), (5, 520), (64, 7168)])
def test_act_quant_fp16_bit_exact(M, K):
    say(f"act_quant fp16 M={M} K={K}")
    x = _f16_rows(M, K, 3600 + M)
    if M > 3:
        x[3] = (torch.arange(K) % 7 - 3).to(torch.float16) * 2.0 ** -20     # fp16 subnormals
    xq, sx = cq.act_quant_int8_per_token(x.to(DEV))
    xq_ref, sx_ref = oracle.act_quant(x.view(torch.int16).numpy().view(np.uint16), fmt="f16")
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), sx_ref.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), xq_ref)


@pytest.mark.parametrize("bits,group", [(2, 512), (3, 128), (3, 256)])
@pytest.mark.parametrize("M", [1, 7, 40, 300])
def test_a8_bf16_outputs(bits, group, M):
    say(f"A8 bf16 out bits={bits} G={group} M={M}")
    g = synth.make_generator(3700 + 10 * bits + M)
    w = synth.make_weight(g, 203, 2048, bits, group, "ternary" if bits == 2 else "uniform", 0.02)
    cw = upload(w)
    x = synth.activations(g, M, 2048, 0.005, 30.0).to(DEV)
    xq, sx = cq.act_quant_int8_per_token(x)
    y = cq.cubic_gemm_a8(xq, sx, cw)
    yb = cq.cubic_gemm_a8(xq, sx, cw, out_dtype=torch.bfloat16)
    if M <= 32:
        assert torch.equal(yb, _bf16_of(y))
    else:
        # the tile kernel's fp32 result at these sizes adds two K halves (two
        # workgroups per tile), the bf16 result rounds the unsplit sum: they
        # may differ by the fp32 order, so one bf16 unit at most
        yr = _bf16_of(y).float()
        bound = torch.maximum(yb.float().abs(), yr.abs()) * 2.0 ** -7     # one bf16 unit
        assert bool(((yb.float() - yr).abs() <= bound).all())
        codes, scales, shapes = np_weight(w)
        xq_ref, sx_ref = oracle.act_quant(x_bits(x))
        ref = oracle.gemm_a8(xq_ref, sx_ref, codes, scales, shapes, bits, group)
        assert row_rel_err(yb.float().cpu().numpy(), ref) <= TOL + 2.0 ** -8   # bf16 rounding on top


def test_prefill_a8_workload_bf16_output_full():
    say("A8 prefill W3 G256 6144x7168 M=4096 bf16 out")
    w, x = synth.prefill_config(seed=5, device=DEV)
    cw = upload(w)
    xq, sx = cq.act_quant_int8_per_token(x)
    y = cq.cubic_gemm_a8(xq, sx, cw)
    assert torch.equal(cq.cubic_gemm_a8(xq, sx, cw, out_dtype=torch.bfloat16), _bf16_of(y))


def _pool(E, N, K, bits, group, seed):
    cb = N * K * bits // 8
    codes = torch.empty(E * cb, dtype=torch.uint8, device=DEV)
    scales = torch.empty((E, N, K // group), dtype=torch.float32, device=DEV)
    shapes = torch.empty((E, N, K // group, 2), dtype=torch.int16, device=DEV)
    dense = []
    for e in range(E):
        w = synth.moe_expert(e, seed=seed, N=N, K=K, bits=bits, group=group, device=DEV)
        cq.cubic_pack(w.codes, bits, out=codes[e * cb:(e + 1) * cb].view(N, K * bits // 8))
        scales[e] = w.scales
        shapes[e] = w.shapes
        dense.append(_dense(w))
    return cq.CubicWeight(codes, scales.reshape(-1), shapes.reshape(-1), N, K, bits, group), dense


@pytest.mark.parametrize("bits,group", [(2, 512), (3, 128), (5, 128)])
@pytest.mark.parametrize("T", [1, 24])
def test_moe_fp16_activations_and_bf16_outputs(bits, group, T):
    say(f"MoE fp16 x / bf16 out bits={bits} G={group} T={T}")
    E, topk, N, K = 8, 2, 256, 1024
    pool, dense = _pool(E, N, K, bits, group, seed=60 + bits)
    _, ids = synth.moe_routing(seed=61, T=T, E=E, topk=topk, K=K, device=DEV)
    ids[0, 1] = E + 3                                       # an invalid id: a zero row
    x = _f16_rows(T, K, 3800 + T)
    xd = x.to(DEV)
    y = cq.cubic_moe_grouped_gemm(xd, ids, pool, E)
    ref = oracle.moe_a16(x.view(torch.int16).numpy().view(np.uint16), ids.cpu().numpy(), E, N,
                         lambda e: dense[e], fmt="f16")
    assert row_rel_err(y.cpu().numpy().reshape(T * topk, N), ref.reshape(T * topk, N)) <= TOL
    yb = cq.cubic_moe_grouped_gemm(xd, ids, pool, E, out_dtype=torch.bfloat16)
    assert torch.equal(yb, _bf16_of(y))
    xb = synth.activations(synth.make_generator(62), T, K).to(DEV)
    y32 = cq.cubic_moe_grouped_gemm(xb, ids, pool, E)
    assert torch.equal(cq.cubic_moe_grouped_gemm(xb, ids, pool, E, out_dtype=torch.bfloat16), _bf16_of(y32))


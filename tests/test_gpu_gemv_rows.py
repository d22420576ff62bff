"""GPU parity of the whole-row GEMV (one activation row, 2-bit codes, groups of
256 or 512, at most 16 groups per row), against the float64 oracle at the
products' bar (per-row 2e-3). The cases cover every number of rows per wave
load (R = 16 / (K / G) from 1 to 16), one to four wave loads per wave (8- and
12-wave workgroups, staggered second and later wave loads), ragged N (rows past N in the last
wave load), raw random code bytes (every field value, so the code -2 path runs in
many wave loads), fp16 activations and bf16 outputs (the fp32 sums rounded),
and activation rows far outside the fp16 range."""
import numpy as np
import pytest
import torch

import dequant_gemm_amd as cq
import oracle
import synth
from tests._gpu import DEV, np_weight, row_rel_err, say, upload, x_bits

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _raw_weight(N, K, G, seed):
    """Codes from random bytes (field 10, the code -2, included), with the
    workloads' scales and (a, b)."""
    g = torch.Generator().manual_seed(seed)
    raw = torch.randint(0, 256, (N * K // 4,), generator=g).to(torch.uint8)
    codes = oracle.unpack(raw.numpy(), N, K, 2)
    sg = synth.make_generator(seed + 1)
    scales = synth.lognormal_scales(sg, N * K // G, 0.015).reshape(N, K // G)
    shapes = synth.sample_shapes(sg, N * K // G).reshape(N, K // G, 2)
    cw = cq.CubicWeight(raw.to(DEV), scales.to(DEV), shapes.to(DEV), N, K, 2, G)
    W = oracle.dequant(codes, scales.numpy(), shapes.numpy().view(np.uint16), 2, G)
    return cw, W


@pytest.mark.parametrize("N,K,G", [(203, 7168, 512), (130, 3072, 512), (77, 8192, 512), (33, 512, 512),
                                   (203, 4096, 256), (97, 768, 256), (64, 2048, 256), (1, 1024, 256),
                                   (10001, 4096, 256), (2001, 3072, 512), (13001, 4096, 256)])
def test_rows_random_codes(N, K, G):
    say(f"GEMV rows N={N} K={K} G={G} (random code bytes)")
    cw, W = _raw_weight(N, K, G, seed=N + K + G)
    x = synth.activations(synth.make_generator(K + 7), 1, K, 0.01, 50.0)
    y = cq.cubic_gemm_a16(x.to(DEV), cw)
    assert torch.equal(y, cq.cubic_gemm_a16(x.to(DEV), cw))
    assert row_rel_err(y.cpu().numpy(), oracle.gemm_a16(x_bits(x), W)) <= TOL
    # bf16 outputs round the same fp32 sums
    yb = cq.cubic_gemm_a16(x.to(DEV), cw, out_dtype=torch.bfloat16)
    assert torch.equal(yb.float(), y.to(torch.bfloat16).float())


@pytest.mark.parametrize("N,K,G", [(203, 7168, 512), (97, 768, 256), (6144, 7168, 512)])
def test_rows_fp16_activations(N, K, G):
    say(f"GEMV rows fp16 x N={N} K={K} G={G}")
    cw, W = _raw_weight(N, K, G, seed=3 * N + K)
    x = torch.randn((1, K), generator=torch.Generator().manual_seed(K)).to(torch.float16)
    y = cq.cubic_gemm_a16(x.to(DEV), cw).cpu().numpy()
    X = x.float().numpy().astype(np.float64)
    assert row_rel_err(y, X @ W.T) <= TOL


def test_rows_workload_shapes_and_activation_extremes():
    """The K3 expert shapes at W2 G512 (gate_up: one row a wave load; down: two)
    with a row scaled by 1e6 and by 1e-30 (no prescale on this path: bf16
    products are exact), and an all-zero row giving exact zeros."""
    for (w, x), name in zip(synth.decode_config(seed=12, device=DEV), ("gate_up", "down")):
        say(f"GEMV rows {name} {w.N}x{w.K}, scaled and zero activations")
        cw = upload(w)
        codes, scales, shapes = np_weight(w)
        W = oracle.dequant(codes, scales, shapes, 2, 512)
        for f in (1e6, 1e-30, 0.0):
            xs = (x.float() * f).to(torch.bfloat16)
            y = cq.cubic_gemm_a16(xs.to(DEV), cw).cpu().numpy()
            if f == 0.0:
                assert not y.any()
            else:
                assert row_rel_err(y, oracle.gemm_a16(x_bits(xs.cpu()), W)) <= TOL

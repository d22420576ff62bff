"""GPU checks of cubic_linear, the shape dispatcher between A16 and Dynamic A8:
its result equals the chosen path's result bit for bit, and the A8 route stays
within the products' bar (2e-3, per-row infinity norm) of the oracle."""
import numpy as np
import pytest
import torch

import dequant_gemm_amd as cq
import oracle
import synth
from tests._gpu import DEV, np_weight, row_rel_err, say, upload, x_bits

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.mark.parametrize("bits,group,M", [(3, 128, 100), (2, 512, 127), (4, 128, 300), (5, 128, 16)])
def test_a16_route_equals_gemm_a16(bits, group, M):
    say(f"linear A16 route bits={bits} G={group} M={M}")
    N, K = 203, 1024
    assert cq.cubic_linear_mode(M, N, K, bits, group) == cq.MODE_A16
    g = synth.make_generator(8100 + bits + M)
    w = synth.make_weight(g, N, K, bits, group, "ternary" if bits == 2 else "uniform", 0.02)
    x = synth.activations(g, M, K, 0.01, 50.0).to(DEV)
    cw = upload(w)
    assert torch.equal(cq.cubic_linear(x, cw), cq.cubic_gemm_a16(x, cw))


@pytest.mark.parametrize("bits,group,M,K", [(3, 256, 300, 1024), (2, 512, 128, 1024), (3, 128, 513, 1024),
                                            (2, 512, 12, 4096), (3, 256, 8, 4608)])
def test_a8_route_equals_quantiser_and_gemm_a8(bits, group, M, K):
    say(f"linear A8 route bits={bits} G={group} M={M} K={K}")
    N = 203
    assert cq.cubic_linear_mode(M, N, K, bits, group) == cq.MODE_A8
    g = synth.make_generator(8200 + bits + M)
    w = synth.make_weight(g, N, K, bits, group, "ternary" if bits == 2 else "uniform", 0.02)
    x = synth.activations(g, M, K, 0.005, 30.0).to(DEV)
    cw = upload(w)
    y = cq.cubic_linear(x, cw)
    xq, sx = cq.act_quant_int8_per_token(x)
    assert torch.equal(y, cq.cubic_gemm_a8(xq, sx, cw))
    codes, scales, shapes = np_weight(w)
    xq_ref, sx_ref = oracle.act_quant(x_bits(x))
    ref = oracle.gemm_a8(xq_ref, sx_ref, codes, scales, shapes, bits, group)
    assert row_rel_err(y.cpu().numpy(), ref) <= TOL

"""GPU parity of the one-token routed-expert products, which skip the routing
kernel: every workgroup reads its pair's expert id itself (2-bit A16 codes on
the streaming kernel, and every A8 width). Checked against the oracle as the
routed calls are (per-row bar 2e-3): invalid ids give zero rows and are counted
in the workspace's first int32, a repeated expert is computed once per pair,
bf16 outputs round the same sums, and the library-scratch entry point returns
the same bits as the workspace call."""
import numpy as np
import pytest
import torch

import dequant_gemm_amd as cq
import oracle
import synth
from tests._gpu import DEV, row_rel_err, say, x_bits
from tests.test_gpu_moe import _expert_dense, _expert_rows, _pool
from tests.test_gpu_moe_a8 import _pool as _pool_a8
from tests.test_gpu_moe_a8 import _mlp_case, _quant, _ref, _run

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _ids(E, topk, seed, bad=()):
    ids = torch.from_numpy(np.random.default_rng(seed).choice(E, topk, replace=False).astype(np.int32))
    ids = ids.reshape(1, topk)
    ids[0, 1] = ids[0, 0]                 # a repeated expert: two pairs, two rows
    for j, v in bad:
        ids[0, j] = v
    return ids.to(DEV)


@pytest.mark.parametrize("K,group,N", [(7168, 512, 200), (3072, 512, 130), (1024, 256, 96), (2048, 256, 16)])
def test_one_token_a16_invalid_and_repeated_ids(K, group, N):
    say(f"MoE one token A16 W2 G{group} K={K} N={N}")
    E, topk, bits = 20, 16, 2
    pool = _pool(E, N, K, bits, group, seed=300 + K % 7)
    x, _ = synth.moe_routing(seed=301, T=1, E=E, topk=topk, K=K, device=DEV)
    ids = _ids(E, topk, 302, bad=((3, -1), (9, E), (15, 1 << 30)))
    ws = torch.full((cq.cubic_moe_workspace_bytes(1, topk, E),), 0x5A, dtype=torch.uint8, device=DEV)
    y = cq.cubic_moe_grouped_gemm(x, ids, pool, E, workspace=ws)
    assert int(ws[:4].view(torch.int32).item()) == 3
    yn = y.cpu().numpy()
    for j in (3, 9, 15):
        assert not yn[0, j].any() and not np.signbit(yn[0, j]).any()
    ref = oracle.moe_a16(x_bits(x), ids.cpu().numpy(), E, N,
                         lambda e: _expert_dense(e, N, K, bits, group, 300 + K % 7))
    assert row_rel_err(yn.reshape(topk, N), ref.reshape(topk, N)) <= TOL
    # bf16 outputs: the fp32 sums rounded to nearest even
    yb = cq.cubic_moe_grouped_gemm(x, ids, pool, E, out_dtype=torch.bfloat16)
    assert torch.equal(yb.float(), y.to(torch.bfloat16).float())
    # repeated calls and the library-scratch entry point give the same bits
    assert torch.equal(cq.cubic_moe_grouped_gemm(x, ids, pool, E), y)
    assert torch.equal(cq.cubic_moe_grouped_gemm_static(x, ids, pool, E), y)


def test_one_token_a16_full_expert_shape():
    """16 of 24 experts of gate_up 6144 x 7168 W2 G512, one token (the decode step's
    launch): every pair checked on 512 of the 6144 rows (both ends of the tile grid)."""
    say("MoE one token A16 gate_up 6144x7168 W2 G512, 16 of 24 experts")
    E, topk, N, K, bits, group = 24, 16, 6144, 7168, 2, 512
    pool = _pool(E, N, K, bits, group, seed=310)
    x, ids = synth.moe_routing(seed=311, T=1, E=E, topk=topk, K=K, device=DEV)
    y = cq.cubic_moe_grouped_gemm(x, ids, pool, E).cpu().numpy()
    rows = np.r_[0:256, N - 256:N]
    X = oracle.bf16_bits_to_f64(x_bits(x))[0]
    for j, e in enumerate(ids.cpu().numpy()[0]):
        ref = _expert_rows(int(e), rows, N, K, bits, group, 310) @ X
        assert row_rel_err(y[0, j][rows][None, :], ref[None, :]) <= TOL, (j, e)


@pytest.mark.parametrize("bits,group,K", [(2, 512, 7168), (2, 128, 1024), (3, 128, 1024), (4, 256, 2048),
                                          (8, 128, 1024)])
def test_one_token_a8_invalid_and_repeated_ids(bits, group, K):
    say(f"MoE one token A8 bits={bits} G={group} K={K}")
    E, topk, N = 20, 16, 96
    pool, host = _pool_a8(E, N, K, bits, group, seed=320 + bits)
    xq, sx = _quant(1, K, seed=321)
    ids = _ids(E, topk, 322, bad=((2, -5), (11, E)))
    ws = torch.full((cq.cubic_moe_workspace_bytes(1, topk, E),), 0x5A, dtype=torch.uint8, device=DEV)
    y = _run(xq, sx, ids, pool, E, ws=ws)
    assert int(ws[:4].view(torch.int32).item()) == 2
    yn = y.cpu().numpy()
    for j in (2, 11):
        assert not yn[0, j].any() and not np.signbit(yn[0, j]).any()
    ref = _ref(xq, sx, ids, E, N, host, bits, group)
    assert row_rel_err(yn.reshape(topk, N), ref.reshape(topk, N)) <= TOL
    yb = _run(xq, sx, ids, pool, E, out_dtype=torch.bfloat16)
    assert torch.equal(yb.float(), y.to(torch.bfloat16).float())
    assert torch.equal(_run(xq, sx, ids, pool, E), y)


def test_one_token_mlp_a16_with_invalid_ids():
    """The A16 MLP step of one token with invalid ids (they add nothing): both
    products read the ids themselves."""
    say("MoE MLP step one token, invalid ids, A16")
    E, T, topk, H, I, bits, group = 10, 1, 6, 1024, 512, 2, 512
    gu = _pool(E, 2 * I, H, bits, group, seed=330)
    dn = _pool(E, H, I, bits, group, seed=331)
    x, ids = synth.moe_routing(seed=332, T=T, E=E, topk=topk, K=H, device=DEV)
    ids[0, 2] = -1
    ids[0, 4] = E
    w = torch.rand((T, topk), generator=torch.Generator().manual_seed(333)).to(DEV)
    ref = oracle.moe_mlp(x_bits(x), ids.cpu().numpy(), w.cpu().numpy(), E,
                         lambda e: _expert_dense(e, 2 * I, H, bits, group, 330),
                         lambda e: _expert_dense(e, H, I, bits, group, 331))
    y = cq.cubic_moe_mlp(x, ids, w, gu, dn, E)
    assert torch.equal(y, cq.cubic_moe_mlp(x, ids, w, gu, dn, E))
    assert row_rel_err(y.cpu().numpy(), ref) <= 5e-3


@pytest.mark.parametrize("bits,group", [(2, 512), (3, 128)])
def test_one_token_mlp_a8_with_invalid_ids(bits, group):
    """The A8 MLP step of one token with invalid ids, h checked element by element."""
    say(f"MoE MLP A8 step one token, invalid ids, bits={bits} G={group}")

    def bad(ids):
        ids[0, 1] = -3
        ids[0, 5] = 12

    _mlp_case(12, 1, 8, 1024, 512, bits, group, seed=340 + bits, mod_ids=bad)

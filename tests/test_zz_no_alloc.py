"""GPU test of cubic_moe_grouped_gemm_static, the grouped routed-expert product
for callers that cannot allocate: its routing scratch is the library's per-device
buffer instead of a workspace. It runs the same kernels as
cubic_moe_grouped_gemm, so its output must equal that call's bit for bit, also
on a second, smaller call right after the first (the buffer keeps the last
call's contents and the routing rewrites what the product reads)."""
import ctypes

import numpy as np
import pytest
import torch

import dequant_gemm_amd as cq
import synth
from tests._gpu import DEV, say

pytestmark = pytest.mark.gpu


def _pool(E, N, K, bits, group, seed):
    cb = N * K * bits // 8
    codes = torch.empty(E * cb, dtype=torch.uint8, device=DEV)
    scales = torch.empty((E, N, K // group), dtype=torch.float32, device=DEV)
    shapes = torch.empty((E, N, K // group, 2), dtype=torch.int16, device=DEV)
    for e in range(E):
        w = synth.moe_expert(e, seed=seed, N=N, K=K, bits=bits, group=group, device=DEV)
        cq.cubic_pack(w.codes, bits, out=codes[e * cb:(e + 1) * cb].view(N, K * bits // 8))
        scales[e] = w.scales
        shapes[e] = w.shapes
    return cq.CubicWeight(codes, scales.reshape(-1), shapes.reshape(-1), N, K, bits, group)


@pytest.mark.parametrize("bits,group,K", [(2, 512, 1024), (4, 128, 512)])
def test_static_scratch_equals_workspace_call(bits, group, K):
    E, N = 12, 200
    pool = _pool(E, N, K, bits, group, seed=90 + bits)
    for T, topk, seed in ((24, 4, 91), (5, 2, 92)):          # the second call is smaller
        say(f"moe static scratch bits={bits} T={T} topk={topk}")
        x, ids = synth.moe_routing(seed=seed, T=T, E=E, topk=topk, K=K, device=DEV)
        if T > 8:
            ids[3, 0] = -1                                    # an invalid id: a zero row
            ids[:9, 1] = 7                                    # an expert picked by more than four tokens
        ref = cq.cubic_moe_grouped_gemm(x, ids, pool, E)
        got = torch.full_like(ref, float("nan"))
        cq.cubic_moe_grouped_gemm_static(x, ids, pool, E, out=got)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), (bits, T)
        if T > 8:
            assert not got[3, 0].any()


def test_static_scratch_rejects_oversized_routing():
    say("moe static scratch: oversized routing is refused")
    lib = cq.load_library()
    cap = cq.cubic_moe_grouped_gemm_static_max_bytes()
    assert cap == 2 << 20
    E, T, topk = 8, 1 << 17, 8                                # 4 MiB of pair ids
    assert cq.cubic_moe_workspace_bytes(T, topk, E) > cap
    x = torch.zeros((16, 512), dtype=torch.bfloat16, device=DEV)
    w = cq.CubicWeight(torch.zeros(16, dtype=torch.uint8, device=DEV), torch.zeros(4, device=DEV),
                       torch.zeros(8, dtype=torch.int16, device=DEV), 8, 512, 2, 512)
    cw = w.c_struct()
    p = ctypes.c_void_p(x.data_ptr())
    st = lib.cubic_moe_grouped_gemm_static(p, T, p, topk, ctypes.byref(cw), E, p, None)
    assert st == -7                                           # CUBIC_ERR_WORKSPACE, nothing enqueued

"""GPU parity of the routed-expert Dynamic A8 product (cubic_moe_grouped_gemm_a8).

Each (token, slot) pair must equal the oracle's A8 product of that token's int8
row with its expert (oracle.gemm_a8: exact integer group dots, fp32(s / 127)
per group, the token's scale last); per-row bar 2e-3, as for cubic_gemm_a8. The
activations are quantised by the oracle (act_quant) and uploaded, so no input
comes from the device path. The experts are drawn from raw random bytes, so
every field value occurs, the extra code -2^(B-1) (t > 1, clamped carriers)
included."""
import numpy as np
import pytest
import torch

import dequant_gemm_amd as cq
import oracle
import synth
from tests._gpu import DEV, pack_fields, row_rel_err, say, x_bits

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _pool(E, N, K, bits, group, seed, shapes_fn=None):
    """E experts back to back: codes from random bytes (any field value), scales
    and (a, b) as the workloads draw them. Returns the device weight and the
    host arrays the oracle reads."""
    rng = np.random.default_rng(seed)
    lo = -(1 << (bits - 1))
    codes = rng.integers(lo, -lo, size=(E, N, K)).astype(np.int8)
    sg = synth.make_generator(seed + 1)
    scales = synth.lognormal_scales(sg, E * N * (K // group), 0.02).reshape(E, N, K // group)
    shapes = synth.sample_shapes(sg, E * N * (K // group)).reshape(E, N, K // group, 2)
    if shapes_fn is not None:
        shapes = shapes_fn(shapes)
    packed = np.concatenate([pack_fields(codes[e], bits).reshape(-1) for e in range(E)])
    w = cq.CubicWeight(torch.from_numpy(packed).to(DEV), scales.reshape(-1).to(DEV).contiguous(),
                       shapes.reshape(-1).to(DEV).contiguous(), N, K, bits, group)
    host = (codes, scales.numpy(), shapes.numpy().view(np.uint16))
    return w, host


def _quant(T, K, seed, outliers=True):
    x = synth.activations(synth.make_generator(seed), T, K, 0.01 if outliers else 0.0, 40.0)
    xq, sx = oracle.act_quant(x_bits(x))
    return xq, sx


def _run(xq, sx, ids, pool, E, out_dtype=torch.float32, ws=None):
    return cq.cubic_moe_grouped_gemm_a8(torch.from_numpy(xq).to(DEV), torch.from_numpy(sx).to(DEV),
                                        ids.to(DEV), pool, E, out_dtype=out_dtype, workspace=ws)


def _ref(xq, sx, ids, E, N, host, bits, group):
    codes, scales, shapes = host
    return oracle.moe_a8(xq, sx, ids.cpu().numpy(), E, N, lambda e: (codes[e], scales[e], shapes[e]),
                         bits, group)


@pytest.mark.parametrize("bits,group", [(2, 512), (2, 128), (3, 128), (3, 256), (4, 128), (4, 512),
                                        (5, 128), (6, 256), (8, 128)])
def test_mini_all_pairs(bits, group):
    """8 experts of 130 x 1024, 24 tokens x top-2 (several passes per expert, a
    ragged 16-row tile), one invalid id."""
    say(f"MoE A8 mini bits={bits} G={group}")
    E, T, topk, N, K = 8, 24, 2, 130, 1024
    pool, host = _pool(E, N, K, bits, group, seed=100 + bits)
    xq, sx = _quant(T, K, seed=101)
    _, ids = synth.moe_routing(seed=102, T=T, E=E, topk=topk, K=K)
    ids[5, 1] = E + 2
    ws = torch.empty(cq.cubic_moe_workspace_bytes(T, topk, E), dtype=torch.uint8, device=DEV)
    y = _run(xq, sx, ids, pool, E, ws=ws)
    assert torch.equal(y, _run(xq, sx, ids, pool, E))
    assert int(ws[:4].view(torch.int32).item()) == 1
    y = y.cpu().numpy()
    assert not y[5, 1].any()
    ref = _ref(xq, sx, ids, E, N, host, bits, group)
    assert row_rel_err(y.reshape(T * topk, N), ref.reshape(T * topk, N)) <= TOL


@pytest.mark.parametrize("bits,group,K", [(2, 512, 7168), (2, 256, 9216), (3, 128, 7168), (4, 256, 3072),
                                          (8, 1024, 4096)])
def test_decode_one_token(bits, group, K):
    """One token, 16 experts of a pool of 20 (one pass each): the decode shape;
    K = 9216 has more steps per wave than the load slots of 2-bit codes."""
    say(f"MoE A8 decode T=1 bits={bits} G={group} K={K}")
    E, T, topk, N = 20, 1, 16, 96
    pool, host = _pool(E, N, K, bits, group, seed=110 + bits)
    xq, sx = _quant(T, K, seed=111)
    _, ids = synth.moe_routing(seed=112, T=T, E=E, topk=topk, K=K)
    y = _run(xq, sx, ids, pool, E).cpu().numpy()
    ref = _ref(xq, sx, ids, E, N, host, bits, group)
    assert row_rel_err(y.reshape(T * topk, N), ref.reshape(T * topk, N)) <= TOL


@pytest.mark.parametrize("K", [128, 256, 640])
def test_short_rows(K):
    """K of one to five steps: waves without steps, and rows shorter than a tile of 16."""
    say(f"MoE A8 short rows K={K}")
    E, T, topk, N, bits, group = 3, 5, 3, 7, 3, 128
    pool, host = _pool(E, N, K, bits, group, seed=120)
    xq, sx = _quant(T, K, seed=121)
    ids = torch.tensor([[0, 1, 2], [2, 2, 1], [0, 0, 0], [1, -1, 2], [2, 1, 0]], dtype=torch.int32)
    y = _run(xq, sx, ids, pool, E).cpu().numpy()
    ref = _ref(xq, sx, ids, E, N, host, bits, group)
    assert row_rel_err(y.reshape(T * topk, N), ref.reshape(T * topk, N)) <= TOL


def test_skewed_routing_and_bf16_output():
    """40 tokens on one expert (ten passes of four rows), zero activation rows,
    and the bf16 output equal to the rounded fp32 output."""
    say("MoE A8 skewed routing, bf16 out")
    E, T, topk, N, K, bits, group = 5, 40, 2, 64, 2048, 2, 512
    pool, host = _pool(E, N, K, bits, group, seed=130)
    xq, sx = _quant(T, K, seed=131)
    xq[3] = 0
    sx[3] = 0
    ids = torch.full((T, topk), 4, dtype=torch.int32)
    ids[:, 1] = torch.arange(T) % 4
    y = _run(xq, sx, ids, pool, E)
    yb = _run(xq, sx, ids, pool, E, out_dtype=torch.bfloat16)
    assert torch.equal(yb, y.to(torch.bfloat16))
    y = y.cpu().numpy()
    assert not y[3].any()
    ref = _ref(xq, sx, ids, E, N, host, bits, group)
    assert row_rel_err(y.reshape(T * topk, N), ref.reshape(T * topk, N)) <= TOL


def test_carrier_ties_and_clamps():
    """W3 shapes with exact carrier ties: a = 2, b = -1.75 gives q(1/3) = 1/2
    (carrier 63.5, to even 64); a = 3.625, b = -1.5 gives q(4/3) = -1/2 for the
    extra code -4. Half-up rounding would miss by one unit (1.6 %)."""
    say("MoE A8 carrier ties W3")
    E, T, topk, N, K, bits, group = 4, 6, 2, 48, 512, 3, 128

    def tie_shapes(sh):
        sh = sh.clone()
        a1, b1 = np.float16(2.0).view(np.int16), np.float16(-1.75).view(np.int16)
        a2, b2 = np.float16(3.625).view(np.int16), np.float16(-1.5).view(np.int16)
        sh[..., 0::2, 0], sh[..., 0::2, 1] = int(a1), int(b1)
        sh[..., 1::2, 0], sh[..., 1::2, 1] = int(a2), int(b2)
        return sh

    pool, host = _pool(E, N, K, bits, group, seed=140, shapes_fn=tie_shapes)
    tab = oracle.carrier_table(np.array([2.0, 3.625]), np.array([-1.75, -1.5]), bits)
    assert tab[0, 1] == 64 and tab[1, 4] == -64
    xq, sx = _quant(T, K, seed=141, outliers=False)
    _, ids = synth.moe_routing(seed=142, T=T, E=E, topk=topk, K=K)
    y = _run(xq, sx, ids, pool, E).cpu().numpy()
    ref = _ref(xq, sx, ids, E, N, host, bits, group)
    assert row_rel_err(y.reshape(T * topk, N), ref.reshape(T * topk, N)) <= TOL


# ---------------------------------------------------------------------------
# The MLP step in the A8 mode (cubic_moe_mlp_a8)
# ---------------------------------------------------------------------------
TOL_MLP = 5e-3


def _hidden_of(ws, T, topk, E, H, I):
    """Device h [T][topk][I] from the A8 MLP workspace: routing part, xq [T][H],
    sx [T], gate_up outputs [P][2I] fp32, then h [P][I] bf16 (256-byte aligned)."""
    P = T * topk
    up = lambda n: -(-n // 256) * 256
    off = cq.cubic_moe_workspace_bytes(T, topk, E) + up(T * H) + up(T * 4) + up(P * 2 * I * 4)
    hb = ws[off:off + P * I * 2].view(torch.int16).cpu().numpy().view(np.uint16)
    return oracle.bf16_bits_to_f64(hb).reshape(T, topk, I)


def _check_hidden_a8(h_dev, v, h_ref, xq, sx, ids_np, up_codes, E, bits, group):
    """h_dev equals the oracle's h, or lies between bf16(v - dv) and bf16(v + dv):
    dv bounds the device's error in v. The group dots are exact integers on both
    sides; the device rounds fp32(s / 127), each group's scaled sum, the sum of the
    four waves' partials and the token scale: fewer than n = K/G + 8 roundings of
    2^-23 (any rounding mode) of mag = sx * sum_g |s / 127| |I_g|; SiLU and the
    product in fp32 add 2^-20 |v|."""
    T, topk, I = h_ref.shape
    flips = 0
    for t in range(T):
        for j in range(topk):
            e = int(ids_np[t, j])
            if not 0 <= e < E:
                continue
            codes, scales, shapes = up_codes(e)
            C = oracle.carrier_codes(codes, shapes, bits, group).astype(np.float64)
            N, K = C.shape
            Ig = (C.reshape(N, K // group, group) * xq[t].astype(np.float64).reshape(1, K // group, group)).sum(2)
            mag = float(sx[t]) * (np.abs(Ig) * (scales.astype(np.float64) / 127.0)).sum(1)
            g = float(sx[t]) * (Ig * (scales.astype(np.float64) / 127.0)).sum(1)
            n = K // group + 8
            gamma = n * 2.0 ** -23 / (1 - n * 2.0 ** -23)
            gg, uu = g[:I], g[I:]
            sig = 1.0 / (1.0 + np.exp(-gg))
            dsilu = np.abs(sig * (1.0 + gg * (1.0 - sig)))
            dv = dsilu * np.abs(uu) * gamma * mag[:I] + np.abs(gg * sig) * gamma * mag[I:] + 2.0 ** -20 * np.abs(v[t, j])
            same = h_dev[t, j] == h_ref[t, j]
            lo, hi = oracle.bf16_rne(v[t, j] - dv), oracle.bf16_rne(v[t, j] + dv)
            ok = same | ((h_dev[t, j] >= lo) & (h_dev[t, j] <= hi))
            bad = np.nonzero(~ok)[0]
            assert ok.all(), (t, j, [(int(i), v[t, j, i], h_ref[t, j, i], h_dev[t, j, i], dv[i]) for i in bad[:4]])
            flips += int((~same).sum())
    return flips


def _mlp_case(E, T, topk, H, I, bits, group, seed, mod_ids=None):
    gu, gu_host = _pool(E, 2 * I, H, bits, group, seed=seed)
    dn, dn_host = _pool(E, H, I, bits, group, seed=seed + 1)
    x, ids = synth.moe_routing(seed=seed + 2, T=T, E=E, topk=topk, K=H)
    if mod_ids is not None:
        mod_ids(ids)
    w = torch.softmax(torch.rand((T, topk), generator=torch.Generator().manual_seed(seed + 3)), dim=1)
    ws = torch.empty(cq.cubic_moe_mlp_a8_workspace_bytes(T, topk, E, H, I), dtype=torch.uint8, device=DEV)
    xd, idd, wd = x.to(DEV), ids.to(DEV), w.to(DEV)
    y = cq.cubic_moe_mlp_a8(xd, idd, wd, gu, dn, E, workspace=ws)
    h_dev = _hidden_of(ws, T, topk, E, H, I)
    assert torch.equal(y, cq.cubic_moe_mlp_a8(xd, idd, wd, gu, dn, E))
    ids_np = ids.numpy()
    up_codes = lambda e: tuple(a[e] for a in gu_host)
    dn_codes = lambda e: tuple(a[e] for a in dn_host)
    ref, v, h_ref = oracle.moe_mlp_a8(x_bits(x), ids_np, w.numpy(), E, up_codes, dn_codes, bits, group,
                                      bits, group)
    xq, sx = oracle.act_quant(x_bits(x))
    flips = _check_hidden_a8(h_dev, v, h_ref, xq, sx, ids_np, up_codes, E, bits, group)
    assert flips <= 0.002 * h_ref.size, flips
    assert row_rel_err(y.cpu().numpy(), ref) <= TOL_MLP


@pytest.mark.parametrize("bits,group", [(2, 256), (3, 128), (4, 128)])
def test_mlp_a8_step(bits, group):
    """gate_up and down in A8, h checked element by element, invalid ids add nothing."""
    say(f"MoE MLP A8 step bits={bits} G={group}")

    def bad(ids):
        ids[3, 1] = -1
        ids[5, 0] = 6

    _mlp_case(6, 20, 2, 1024, 512, bits, group, seed=150 + bits, mod_ids=bad)


def test_mlp_a8_k3_dims_one_token():
    """Kimi K3 expert dims (hidden 7168, intermediate 3072), W2 G512, one token
    over 16 experts: the decode shape of the A8 step."""
    say("MoE MLP A8 K3 dims, one token top-16 of 16")
    _mlp_case(16, 1, 16, 7168, 3072, 2, 512, seed=160)

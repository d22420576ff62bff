"""GPU parity of the routed-expert grouped product (cubic_moe_grouped_gemm).

Each (token, slot) pair must equal the oracle's product of that token with its
expert's weights (per-row bar 2e-3); invalid ids give zero rows and are counted.
The full 896-expert pool is checked on sampled pairs."""
import numpy as np
import pytest
import torch

import dequant_gemm_amd as cq
import oracle
import synth
from tests._gpu import DEV, np_weight, pack_fields, row_rel_err, say, x_bits

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _pool(E, N, K, bits, group, seed, device=DEV):
    """Experts back to back on the device, each drawn from its own seed."""
    cb = N * K * bits // 8
    codes = torch.empty(E * cb, dtype=torch.uint8, device=device)
    scales = torch.empty((E, N, K // group), dtype=torch.float32, device=device)
    shapes = torch.empty((E, N, K // group, 2), dtype=torch.int16, device=device)
    for e in range(E):
        w = synth.moe_expert(e, seed=seed, N=N, K=K, bits=bits, group=group, device=device)
        cq.cubic_pack(w.codes, bits, out=codes[e * cb:(e + 1) * cb].view(N, K * bits // 8))
        scales[e] = w.scales
        shapes[e] = w.shapes
    return cq.CubicWeight(codes, scales.reshape(-1), shapes.reshape(-1), N, K, bits, group)


def _expert_dense(e, N, K, bits, group, seed):
    w = synth.moe_expert(e, seed=seed, N=N, K=K, bits=bits, group=group, device=DEV)
    codes, scales, shapes = np_weight(w)
    return oracle.dequant(codes, scales, shapes, bits, group)


@pytest.mark.parametrize("bits,group", [(2, 512), (3, 128), (4, 256), (7, 128), (8, 256)])
def test_mini_k3_all_pairs(bits, group):
    # K3 mini shapes (hidden 512, expert intermediate 256, 8 experts, top-2)
    say(f"MoE mini bits={bits}")
    E, T, topk, N, K = 8, 24, 2, 256, 512
    pool = _pool(E, N, K, bits, group, seed=40 + bits)
    x, ids = synth.moe_routing(seed=41, T=T, E=E, topk=topk, K=K, device=DEV)
    ids[0, 0] = ids[0, 1]              # a token may repeat an expert; the pair is still computed
    y = cq.cubic_moe_grouped_gemm(x, ids, pool, E).cpu().numpy()
    ref = oracle.moe_a16(x_bits(x), ids.cpu().numpy(), E, N,
                         lambda e: _expert_dense(e, N, K, bits, group, 40 + bits))
    assert row_rel_err(y.reshape(T * topk, N), ref.reshape(T * topk, N)) <= TOL


def test_skewed_routing_and_invalid_ids():
    # 40 tokens all on expert 3 (more than one 16-row activation tile), invalid ids
    say("MoE skewed + invalid ids")
    E, T, topk, N, K, bits, group = 6, 40, 2, 130, 512, 2, 512
    pool = _pool(E, N, K, bits, group, seed=50)
    x, _ = synth.moe_routing(seed=51, T=T, E=E, topk=topk, K=K, device=DEV)
    ids = torch.full((T, topk), 3, dtype=torch.int32)
    ids[:, 1] = torch.arange(T) % E
    ids[5, 1] = -1
    ids[7, 0] = E
    ids = ids.to(DEV)
    ws = torch.empty(cq.cubic_moe_workspace_bytes(T, topk, E), dtype=torch.uint8, device=DEV)
    y = cq.cubic_moe_grouped_gemm(x, ids, pool, E, workspace=ws).cpu().numpy()
    assert int(ws[:4].view(torch.int32).item()) == 2
    ref = oracle.moe_a16(x_bits(x), ids.cpu().numpy(), E, N,
                         lambda e: _expert_dense(e, N, K, bits, group, 50))
    assert not y[5, 1].any() and not y[7, 0].any()
    assert row_rel_err(y.reshape(T * topk, N), ref.reshape(T * topk, N)) <= TOL


@pytest.mark.parametrize("K", [1024, 7168])
def test_pass_remainders(K):
    # expert e is picked by e + 1 pairs (1..9): every remainder of the passes
    # that take an expert's pairs several rows at a time, ragged N
    say(f"MoE pass remainders W2 G512 K={K}")
    E, N, bits, group = 9, 130, 2, 512
    T = E * (E + 1) // 2
    pool = _pool(E, N, K, bits, group, seed=55)
    x, _ = synth.moe_routing(seed=56, T=T, E=E, topk=1, K=K, device=DEV)
    ids = torch.tensor([e for e in range(E) for _ in range(e + 1)], dtype=torch.int32)
    ids = ids[torch.randperm(T, generator=torch.Generator().manual_seed(57))].reshape(T, 1).to(DEV)
    y = cq.cubic_moe_grouped_gemm(x, ids, pool, E).cpu().numpy()
    ref = oracle.moe_a16(x_bits(x), ids.cpu().numpy(), E, N,
                         lambda e: _expert_dense(e, N, K, bits, group, 55))
    assert row_rel_err(y.reshape(T, N), ref.reshape(T, N)) <= TOL


def _expert_rows(e, rows, N, K, bits, group, seed):
    """Float64 rows `rows` of expert e (drawn on the device, dequantised by the oracle)."""
    w = synth.moe_expert(e, seed=seed, N=N, K=K, bits=bits, group=group, device=DEV)
    codes, scales, shapes = np_weight(w)
    return oracle.dequant(codes[rows], scales[rows], shapes[rows], bits, group)


def test_full_pool_sampled_pairs():
    """896 experts of gate_up 6144 x 7168 W2 G512, 64 tokens x top-16. Checked:
    64 pairs on 1024 of the 6144 output rows each (the first and last 512, so both
    ends of the tile grid). Forced into the routing: the last expert (its codes
    start 9.9 GB into the pool, past 4 GiB), expert 391 (the first whose codes
    start past 4 GiB), and expert 895 picked by 6 tokens (more than the four
    activation rows of one pass)."""
    say("MoE full pool 896 x 6144x7168 W2 G512, T=64 top-16 (64 sampled pairs)")
    E, T, topk, N, K, bits, group = 896, 64, 16, 6144, 7168, 2, 512
    assert 391 * N * K * bits // 8 >= 1 << 32 > 390 * N * K * bits // 8
    pool = _pool(E, N, K, bits, group, seed=4)
    x, ids = synth.moe_routing(seed=4, T=T, E=E, topk=topk, K=K, device=DEV)
    ids_np = ids.cpu().numpy()
    for t in range(6):                                   # expert 895: six tokens, slot 0
        if 895 in ids_np[t]:
            ids_np[t, list(ids_np[t]).index(895)] = ids_np[t, 0]
        ids_np[t, 0] = 895
    for t in (10, 11):                                   # expert 391: two tokens, slot 1
        if 391 in ids_np[t]:
            ids_np[t, list(ids_np[t]).index(391)] = ids_np[t, 1]
        ids_np[t, 1] = 391
    assert all(len(set(r)) == topk for r in ids_np)
    ids = torch.from_numpy(ids_np).to(DEV)
    y = cq.cubic_moe_grouped_gemm(x, ids, pool, E)
    y2 = cq.cubic_moe_grouped_gemm(x, ids, pool, E)
    assert torch.equal(y, y2)
    y = y.cpu().numpy()
    X = x_bits(x)
    rows = np.r_[0:512, N - 512:N]
    pairs = [(t, 0) for t in range(6)] + [(10, 1), (11, 1)]
    rng = np.random.default_rng(4)
    while len(pairs) < 64:
        t, j = int(rng.integers(T)), int(rng.integers(topk))
        if (t, j) not in pairs:
            pairs.append((t, j))
    dense = {}
    for t, j in pairs:
        e = int(ids_np[t, j])
        if e not in dense:
            dense[e] = _expert_rows(e, rows, N, K, bits, group, 4)
        ref = oracle.gemm_a16(X[t:t + 1], dense[e])
        assert row_rel_err(y[t, j][rows][None, :], ref) <= TOL, (t, j, e)
    assert {895, 391} <= set(dense)


@pytest.mark.parametrize("bits,group,K", [(2, 512, 1024), (3, 128, 1024), (4, 128, 9216), (2, 128, 9216)])
@pytest.mark.parametrize("T", [1, 3])
def test_decode_routing_and_long_slices(bits, group, K, T):
    """Decode-sized routing (one activation row per pass for T = 1, two for T = 3,
    an odd count that leaves a one-row pass), and K = 9216, whose per-wave
    activation slices are longer than the part staged through registers."""
    say(f"MoE decode T={T} bits={bits} G={group} K={K}")
    E, topk, N = 20, 16, 200
    pool = _pool(E, N, K, bits, group, seed=60 + bits)
    x, ids = synth.moe_routing(seed=61 + T, T=T, E=E, topk=topk, K=K, device=DEV)
    if T == 3:
        ids[1, :3] = ids[0, :3]        # experts picked by several tokens
        ids[2, :3] = ids[0, :3]
    y = cq.cubic_moe_grouped_gemm(x, ids, pool, E).cpu().numpy()
    ref = oracle.moe_a16(x_bits(x), ids.cpu().numpy(), E, N,
                         lambda e: _expert_dense(e, N, K, bits, group, 60 + bits))
    assert row_rel_err(y.reshape(T * topk, N), ref.reshape(T * topk, N)) <= TOL


def test_routing_over_expert_chunks_and_long_pair_lists():
    """2500 experts (two LDS chunks of the routing kernel) and 300 x 16 = 4800
    pairs (more than the routing kernel keeps in registers), with invalid ids."""
    say("MoE routing: 2500 experts, 4800 pairs")
    E, T, topk, N, K, bits, group = 2500, 300, 16, 16, 128, 2, 128
    pool = _pool(E, N, K, bits, group, seed=70)
    x, ids = synth.moe_routing(seed=71, T=T, E=E, topk=topk, K=K, device=DEV)
    ids[3, 5] = -7
    ids[299, 15] = E + 3
    ids[:40, 0] = 2499                  # one expert with many tokens, in the second chunk
    ws = torch.empty(cq.cubic_moe_workspace_bytes(T, topk, E), dtype=torch.uint8, device=DEV)
    y = cq.cubic_moe_grouped_gemm(x, ids, pool, E, workspace=ws).cpu().numpy()
    assert int(ws[:4].view(torch.int32).item()) == 2
    ids_np = ids.cpu().numpy()
    dense = {}

    def w_of(e):
        if e not in dense:
            dense[e] = _expert_dense(e, N, K, bits, group, 70)
        return dense[e]

    ref = oracle.moe_a16(x_bits(x), ids_np, E, N, w_of)
    assert not y[3, 5].any() and not y[299, 15].any()
    assert row_rel_err(y.reshape(T * topk, N), ref.reshape(T * topk, N)) <= TOL


@pytest.mark.parametrize("T", [1, 3])
def test_sparse_extra_codes_routed(T):
    """Routed 2-bit experts with a few codes -2 planted (the rare decode path
    inside the persistent kernel), decode-sized routing."""
    say(f"MoE W2 sparse extra codes T={T}")
    E, topk, N, K, bits, group = 12, 6, 144, 1024, 2, 512
    cb = N * K * bits // 8
    rng = np.random.default_rng(9)
    codes_all, dense = [], []
    packed = torch.empty(E * cb, dtype=torch.uint8)
    scales = torch.empty((E, N, K // group), dtype=torch.float32)
    shapes = torch.empty((E, N, K // group, 2), dtype=torch.int16)
    for e in range(E):
        w = synth.moe_expert(e, seed=90, N=N, K=K, bits=bits, group=group)
        c = w.codes.numpy().copy()
        for n, k in zip(rng.integers(0, N, 6), rng.integers(0, K, 6)):
            c[n, k] = -2
        packed[e * cb:(e + 1) * cb] = torch.from_numpy(pack_fields(c, bits).reshape(-1))
        scales[e], shapes[e] = w.scales, w.shapes
        dense.append(oracle.dequant(c, w.scales.numpy(), w.shapes.numpy().view(np.uint16), bits, group))
    pool = cq.CubicWeight(packed.to(DEV), scales.reshape(-1).to(DEV), shapes.reshape(-1).to(DEV),
                          N, K, bits, group)
    x, ids = synth.moe_routing(seed=91, T=T, E=E, topk=topk, K=K, device=DEV)
    y = cq.cubic_moe_grouped_gemm(x, ids, pool, E).cpu().numpy()
    ref = oracle.moe_a16(x_bits(x), ids.cpu().numpy(), E, N, lambda e: dense[e])
    assert row_rel_err(y.reshape(T * topk, N), ref.reshape(T * topk, N)) <= TOL


# The MLP step composes two products through h = bf16(SiLU(g) * u). The device's
# h is checked element by element below: it equals the oracle's bf16(v) except
# where v lies within the gate_up error of a bf16 rounding boundary (then it is
# the rounding of a value within that error: a neighbour, or several ulps of a
# near-zero v whose g or u cancelled). Such elements are a small fraction (checked
# below), so the step's output differs from the oracle's by the down product's
# own error (the products' bar, 2e-3 per row) plus those few moves of h carried
# through the down weights; the bar below is 2.5 times the products' bar.
# Swapped halves, a wrong router weight or a lost term give errors of order one.
TOL_MLP = 5e-3


def _mlp_hidden_of(ws, T, topk, E, I):
    """(v-free) device h [T][topk][I] as float64, read from the MLP workspace:
    routing part, then [P][2I] fp32, then h [P][I] bf16 (256-byte aligned parts)."""
    P = T * topk
    off = cq.cubic_moe_workspace_bytes(T, topk, E)
    off += -(-(P * 2 * I * 4) // 256) * 256
    hb = ws[off:off + P * I * 2].view(torch.int16).cpu().numpy().view(np.uint16)
    return oracle.bf16_bits_to_f64(hb).reshape(T, topk, I)


def _check_hidden(h_dev, v, h_ref, x_bits_rows, ids_np, gate_up_dense, H, K_up, E):
    """h_dev equals h_ref, or lies between bf16(v - dv) and bf16(v + dv) where dv
    bounds the device's error in v from its gate_up outputs. The gate_up bound: fp32
    accumulation of K exact products (2-bit codes: +-s exactly) over any order,
    gamma = n u / (1 - n u), n = K + 64 operations, u = 2^-23 (an error of up to
    one ulp per operation, so any rounding mode of the matrix cores is covered), times
    sum |x| |w| per output; SiLU and the product in fp32 add 2^-20 |v|."""
    X = oracle.bf16_bits_to_f64(x_bits_rows)
    T, topk, I = h_ref.shape
    n = K_up + 64
    gamma = n * 2.0 ** -23 / (1 - n * 2.0 ** -23)
    flips = 0
    for t in range(T):
        for j in range(topk):
            e = int(ids_np[t, j])
            if not 0 <= e < E:
                continue
            W = gate_up_dense(e)
            mag = np.abs(W) @ np.abs(X[t])
            g = W[:I] @ X[t]
            u = W[I:] @ X[t]
            sig = 1.0 / (1.0 + np.exp(-g))
            dsilu = np.abs(sig * (1.0 + g * (1.0 - sig)))
            dv = dsilu * np.abs(u) * gamma * mag[:I] + np.abs(g * sig) * gamma * mag[I:] + 2.0 ** -20 * np.abs(v[t, j])
            same = h_dev[t, j] == h_ref[t, j]
            # bf16 rounding is monotone: h_dev must lie between the roundings of
            # v - dv and v + dv (h_ref itself, or a neighbour when v is within dv
            # of a rounding boundary)
            lo = oracle.bf16_rne(v[t, j] - dv)
            hi = oracle.bf16_rne(v[t, j] + dv)
            ok = same | ((h_dev[t, j] >= lo) & (h_dev[t, j] <= hi))
            bad = np.nonzero(~ok)[0]
            assert ok.all(), (t, j, [(int(i), v[t, j, i], h_ref[t, j, i], h_dev[t, j, i], dv[i]) for i in bad[:4]])
            flips += int((~same).sum())
    return flips


@pytest.mark.parametrize("bits,group,T,topk,E", [(2, 256, 20, 2, 6), (4, 128, 20, 2, 6), (2, 512, 1, 4, 16)])
def test_moe_mlp_step(bits, group, T, topk, E):
    """cubic_moe_mlp: gate_up and down experts, SiLU * up in bf16, router-weighted sum."""
    say(f"MoE MLP step bits={bits} G={group} T={T} topk={topk} E={E}")
    H, I = 1024, 512
    gu = _pool(E, 2 * I, H, bits, group, seed=80 + bits)
    dn = _pool(E, H, I, bits, group, seed=90 + bits)
    x, ids = synth.moe_routing(seed=81, T=T, E=E, topk=topk, K=H, device=DEV)
    if T > 1:
        ids[3, 1] = -1                                   # invalid ids add nothing
        ids[5, 0] = E
    w = torch.rand((T, topk), generator=torch.Generator().manual_seed(82)).to(DEV)
    y = cq.cubic_moe_mlp(x, ids, w, gu, dn, E)
    y2 = cq.cubic_moe_mlp(x, ids, w, gu, dn, E)
    assert torch.equal(y, y2)
    ref = oracle.moe_mlp(x_bits(x), ids.cpu().numpy(), w.cpu().numpy(), E,
                         lambda e: _expert_dense(e, 2 * I, H, bits, group, 80 + bits),
                         lambda e: _expert_dense(e, H, I, bits, group, 90 + bits))
    assert row_rel_err(y.cpu().numpy(), ref) <= TOL_MLP


def test_moe_mlp_k3_dims_few_tokens():
    """Kimi K3 expert dims (hidden 7168, intermediate 3072), W2 G512, 2 tokens x top-2."""
    say("MoE MLP step K3 dims, 2 tokens x top-2 of 4 experts")
    E, T, topk, H, I, bits, group = 4, 2, 2, 7168, 3072, 2, 512
    gu = _pool(E, 2 * I, H, bits, group, seed=84)
    dn = _pool(E, H, I, bits, group, seed=85)
    x, ids = synth.moe_routing(seed=86, T=T, E=E, topk=topk, K=H, device=DEV)
    w = torch.tensor([[0.6, 0.4], [0.3, 0.7]], dtype=torch.float32, device=DEV)
    y = cq.cubic_moe_mlp(x, ids, w, gu, dn, E).cpu().numpy()
    ref = oracle.moe_mlp(x_bits(x), ids.cpu().numpy(), w.cpu().numpy(), E,
                         lambda e: _expert_dense(e, 2 * I, H, bits, group, 84),
                         lambda e: _expert_dense(e, H, I, bits, group, 85))
    assert row_rel_err(y, ref) <= TOL_MLP


@pytest.mark.parametrize("E,T", [(64, 1), (896, 64)])
def test_moe_mlp_full_size_sampled_tokens(E, T):
    """The MLP step at hidden 7168 / intermediate 3072, W2 G512, top-16, in the two
    launch configurations the bench times (one token over 64 experts; 64 tokens over
    896), with softmax router weights. Checked against the oracle: the bf16
    intermediate h of every pair of the checked tokens, element by element, and
    their outputs on 1024 of the 7168 rows. For T = 64, tokens 0..7 share their
    16 experts (so 8 tokens are checked on 16 experts, each picked by more than
    four tokens: several passes per expert)."""
    say(f"MoE MLP step full size E={E} T={T} top-16 (sampled tokens, intermediate h)")
    H, I, topk, bits, group = 7168, 3072, 16, 2, 512
    gu = _pool(E, 2 * I, H, bits, group, seed=4)
    dn = _pool(E, H, I, bits, group, seed=6)
    x, ids = synth.moe_routing(seed=4, T=T, E=E, topk=topk, K=H, device=DEV)
    if T > 1:
        ids[1:8] = ids[0]
    w = torch.softmax(torch.rand((T, topk), generator=torch.Generator().manual_seed(8)), dim=1).to(DEV)
    ws = torch.empty(cq.cubic_moe_mlp_workspace_bytes(T, topk, E, H, I), dtype=torch.uint8, device=DEV)
    y = cq.cubic_moe_mlp(x, ids, w, gu, dn, E, workspace=ws)
    h_dev = _mlp_hidden_of(ws, T, topk, E, I)
    assert torch.equal(y, cq.cubic_moe_mlp(x, ids, w, gu, dn, E))
    y = y.cpu().numpy()
    X, ids_np, w_np = x_bits(x), ids.cpu().numpy(), w.cpu().numpy()
    toks = [0] if T == 1 else list(range(8))
    rows = np.r_[0:512, H - 512:H]
    gu_dense, dn_rows = {}, {}

    def gu_of(e):
        if e not in gu_dense:
            gu_dense[e] = _expert_dense(e, 2 * I, H, bits, group, 4)
        return gu_dense[e]

    def dn_of(e):
        if e not in dn_rows:
            dn_rows[e] = _expert_rows(e, rows, H, I, bits, group, 6)
        return dn_rows[e]

    tk = np.array(toks)
    v, h_ref = oracle.moe_mlp_hidden(X[tk], ids_np[tk], E, gu_of)
    flips = _check_hidden(h_dev[tk], v, h_ref, X[tk], ids_np[tk], gu_of, H, H, E)
    assert flips <= 0.002 * h_ref.size, flips
    for i, t in enumerate(toks):
        # the step's output on the sampled rows, from the oracle's h
        ref = np.zeros(len(rows))
        for j in range(topk):
            ref += float(w_np[t, j]) * (dn_of(int(ids_np[t, j])) @ h_ref[i, j])
        assert row_rel_err(y[t:t + 1, rows], ref[None, :]) <= TOL_MLP, t

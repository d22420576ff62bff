"""Seeded generators (torch; CPU or GPU device) for the five workloads.

Workloads (shapes of the Kimi K3 routed experts: hidden 7168, expert
intermediate 3072, fused gate_up 6144 x 7168, down 7168 x 3072; 896 experts,
top-16 routing, from the Kimi K3 guide's model-card table):

* ``single``   W3 G128, weight 256 x 512, M = 4, codes uniform on [-3, 3],
                scale LogNormal(ln 0.02, 0.3), group 0 of row 0 forced to a=1, b=0.
* ``decode``   W2 G512, gate_up 6144 x 7168 and down 7168 x 3072, M = 1,
                P(0) = 1/2, P(+-1) = 1/4, scale LogNormal(ln 0.015, 0.3).
* ``smallm``   W4 G128, same two shapes, M in {8, 64}, codes
                round(7 * clip(Laplace(0, 0.25), -1, 1)), scale LogNormal(ln 0.02, 0.3),
                1 % of activation columns scaled by 50.
* ``moe``      896 experts of gate_up at the ``decode`` distributions; 64 tokens,
                each routed to 16 distinct experts uniformly.
* ``prefill``  W3 G256, 6144 x 7168, M = 4096, codes uniform on [-3, 3],
                0.5 % of activation columns scaled by 30.

Shape parameters (a, b) are drawn uniformly from the box [0, 4] x [-6.5, 3],
rounded to fp16, and kept only where q'(t) = a + 2bt + 3(1-a-b)t^2 stays above
1e-9 on [0, 1] (the region in which the cubic is increasing).

Tensors returned: codes int8 [N][K]; scales float32 [N][K/G]; shapes int16
[N][K/G][2] holding fp16 bit patterns (a, then b); x bfloat16 [M][K].
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

__all__ = [
    "Weight", "make_generator", "sample_shapes", "lognormal_scales",
    "codes_uniform", "codes_ternary", "codes_laplace", "activations",
    "make_weight", "single_config", "decode_config", "smallm_config",
    "prefill_config", "moe_routing", "moe_expert", "WORKLOADS",
]

# name -> (bits, group, N, K) of each weight matrix, plus M values
WORKLOADS = {
    "single": dict(bits=3, group=128, shapes=[(256, 512)], M=[4]),
    "decode": dict(bits=2, group=512, shapes=[(6144, 7168), (7168, 3072)], M=[1]),
    "smallm": dict(bits=4, group=128, shapes=[(6144, 7168), (7168, 3072)], M=[8, 64]),
    "moe": dict(bits=2, group=512, shapes=[(6144, 7168)], M=[64], experts=896, topk=16),
    "prefill": dict(bits=3, group=256, shapes=[(6144, 7168)], M=[4096]),
}


@dataclass
class Weight:
    codes: torch.Tensor      # int8 [N][K]
    scales: torch.Tensor     # float32 [N][K/G]
    shapes: torch.Tensor     # int16 [N][K/G][2] (fp16 bit patterns of a, b)
    bits: int
    group: int

    @property
    def N(self) -> int:
        return self.codes.shape[0]

    @property
    def K(self) -> int:
        return self.codes.shape[1]


def make_generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _fp16_bits(t: torch.Tensor) -> torch.Tensor:
    return t.to(torch.float16).view(torch.int16)


def sample_shapes(gen: torch.Generator, n: int, device="cpu") -> torch.Tensor:
    """n fp16 (a, b) pairs from the increasing region, as int16 bit patterns [n][2]."""
    out = []
    have = 0
    while have < n:
        m = max(64, int((n - have) * 3.2) + 64)
        a = torch.rand(m, generator=gen, device=device, dtype=torch.float64) * 4.0
        b = torch.rand(m, generator=gen, device=device, dtype=torch.float64) * 9.5 - 6.5
        a = a.to(torch.float16).to(torch.float64)
        b = b.to(torch.float16).to(torch.float64)
        c = 1.0 - a - b
        lo = torch.minimum(a, 3.0 - 2.0 * a - b)                 # q'(0), q'(1)
        safe_c = torch.where(c > 0, c, torch.ones_like(c))
        tstar = -b / (3.0 * safe_c)
        inner = (c > 0) & (tstar > 0) & (tstar < 1)
        lo = torch.where(inner, torch.minimum(lo, a - b * b / (3.0 * safe_c)), lo)
        keep = lo > 1e-9
        ab = torch.stack([a[keep], b[keep]], dim=1)
        out.append(ab)
        have += ab.shape[0]
    ab = torch.cat(out)[:n]
    return _fp16_bits(ab)


def lognormal_scales(gen: torch.Generator, n: int, median: float, sigma: float = 0.3,
                     device="cpu") -> torch.Tensor:
    z = torch.randn(n, generator=gen, device=device, dtype=torch.float64)
    return torch.exp(math.log(median) + sigma * z).to(torch.float32)


def codes_uniform(gen, N, K, kmax, device="cpu") -> torch.Tensor:
    return torch.randint(-kmax, kmax + 1, (N, K), generator=gen, device=device,
                         dtype=torch.int64).to(torch.int8)


def codes_ternary(gen, N, K, device="cpu") -> torch.Tensor:
    """P(0) = 1/2, P(+1) = P(-1) = 1/4."""
    u = torch.randint(0, 4, (N, K), generator=gen, device=device, dtype=torch.int64)
    return torch.where(u < 2, 0, torch.where(u == 2, 1, -1)).to(torch.int8)


def codes_laplace(gen, N, K, kmax=7, scale=0.25, device="cpu") -> torch.Tensor:
    """round(kmax * clip(Laplace(0, scale), -1, 1)) by inverse transform, ties to even."""
    u = torch.rand((N, K), generator=gen, device=device, dtype=torch.float64) - 0.5
    lap = -scale * torch.sign(u) * torch.log1p(-2.0 * u.abs())
    return torch.round(kmax * lap.clamp(-1.0, 1.0)).to(torch.int8)


def activations(gen, M, K, outlier_frac=0.0, outlier_mult=1.0, device="cpu") -> torch.Tensor:
    """bf16 [M][K] ~ N(0,1); round(frac*K) columns (without replacement) scaled in fp32."""
    x = torch.randn((M, K), generator=gen, device=device, dtype=torch.float32)
    n_out = int(round(outlier_frac * K))
    if n_out:
        cols = torch.randperm(K, generator=gen, device=device)[:n_out]
        x[:, cols] *= outlier_mult
    return x.to(torch.bfloat16)


def make_weight(gen, N, K, bits, group, codes_kind, median, device="cpu") -> Weight:
    km = (1 << (bits - 1)) - 1
    if codes_kind == "uniform":
        codes = codes_uniform(gen, N, K, km, device)
    elif codes_kind == "ternary":
        codes = codes_ternary(gen, N, K, device)
    elif codes_kind == "laplace":
        codes = codes_laplace(gen, N, K, km, 0.25, device)
    else:
        raise ValueError(codes_kind)
    ng = N * (K // group)
    scales = lognormal_scales(gen, ng, median, 0.3, device).reshape(N, K // group)
    shapes = sample_shapes(gen, ng, device).reshape(N, K // group, 2)
    return Weight(codes, scales, shapes, bits, group)


def single_config(seed=1, device="cpu"):
    """W3 G128, 256 x 512, M = 4; group 0 of row 0 is the uniform-INT case."""
    g = make_generator(seed, device)
    w = make_weight(g, 256, 512, 3, 128, "uniform", 0.02, device)
    w.shapes[0, 0] = _fp16_bits(torch.tensor([1.0, 0.0], dtype=torch.float64, device=device))
    x = activations(g, 4, 512, device=device)
    return w, x


def decode_config(seed=2, device="cpu"):
    """W2 G512, gate_up 6144 x 7168 and down 7168 x 3072, M = 1."""
    g = make_generator(seed, device)
    w_up = make_weight(g, 6144, 7168, 2, 512, "ternary", 0.015, device)
    w_down = make_weight(g, 7168, 3072, 2, 512, "ternary", 0.015, device)
    x_up = activations(g, 1, 7168, device=device)
    x_down = activations(g, 1, 3072, device=device)
    return (w_up, x_up), (w_down, x_down)


def smallm_config(M, seed=3, device="cpu"):
    """W4 G128, gate_up and down shapes, M rows with 1 % outlier columns x50."""
    g = make_generator(seed * 1000 + M, device)
    w_up = make_weight(g, 6144, 7168, 4, 128, "laplace", 0.02, device)
    w_down = make_weight(g, 7168, 3072, 4, 128, "laplace", 0.02, device)
    x_up = activations(g, M, 7168, 0.01, 50.0, device)
    x_down = activations(g, M, 3072, 0.01, 50.0, device)
    return (w_up, x_up), (w_down, x_down)


def prefill_config(seed=5, device="cpu", M=4096, N=6144, K=7168):
    """W3 G256, N x K weight, M rows with 0.5 % outlier columns x30."""
    g = make_generator(seed, device)
    w = make_weight(g, N, K, 3, 256, "uniform", 0.02, device)
    x = activations(g, M, K, 0.005, 30.0, device)
    return w, x


def moe_routing(seed=4, T=64, E=896, topk=16, K=7168, device="cpu"):
    """Token activations [T][K] and topk distinct expert ids per token (int32)."""
    g = make_generator(seed, device)
    x = activations(g, T, K, device=device)
    keys = torch.rand((T, E), generator=g, device=device)
    ids = torch.argsort(keys, dim=1)[:, :topk].to(torch.int32)
    return x, ids


def moe_expert(e, seed=4, N=6144, K=7168, bits=2, group=512, device="cpu") -> Weight:
    """Expert e of the pool, drawn from its own seed so any expert can be redrawn alone."""
    g = make_generator(seed * 1_000_003 + 7919 * (e + 1), device)
    return make_weight(g, N, K, bits, group, "ternary", 0.015, device)

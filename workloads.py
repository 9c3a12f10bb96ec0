"""Seeded synthetic workloads for the ternary-weight x int8-activation product.

This module only draws inputs: ternary int8 weight matrices, per-tensor weight
scales and float activations, with the shapes and value structure of the
workloads below.  It holds none of the method's arithmetic (no packing, no
quantization, no products), so the GPU path and the CPU oracle can both take
their inputs from it without sharing any of the computation.

Shapes follow the BitNet b1.58 2B-4T model metadata printed on the page
"ik_llama.cpp 运行 BitNet b1.58 2B 模型实战…" (section 二, the GGUF key/value
dump: hidden 2560, FFN 6912, 20 heads / 5 KV heads, 30 blocks) and a
Llama-3-70B-class shape (hidden 8192, FFN 28672, 64 / 8 heads, 80 blocks;
"LLM Quantization Paradigms…", section 6 names this model class).  Each block
has seven ternary projections q, k, v, o, gate, up, down ("BitNet Inference
Preprocessing…", Stage 1 lists them).  Outlier channels follow the
activation-outlier description of "LLM Quantization Paradigms…", section 2
(0.1-1 % of channels, up to 100x larger).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

MASTER_SEED = 20241021

PROJ_NAMES = ("q", "k", "v", "o", "gate", "up", "down")
# Which of the four per-layer inputs feeds each projection:
# 0 = attention input (q,k,v), 1 = attention output (o),
# 2 = FFN input (gate,up), 3 = FFN hidden (down).
PROJ_INPUT = (0, 0, 0, 1, 2, 2, 3)


def layer_shapes(hidden: int, ffn: int, heads: int, kv_heads: int,
                 head_dim: int = 128):
    """(M, K) = (out, in) of the seven projections of one block."""
    q = heads * head_dim
    kv = kv_heads * head_dim
    return ((q, hidden), (kv, hidden), (kv, hidden), (hidden, q),
            (ffn, hidden), (ffn, hidden), (hidden, ffn))


LAYER_2B = layer_shapes(2560, 6912, 20, 5)
LAYER_70B = layer_shapes(8192, 28672, 64, 8)


@dataclass(frozen=True)
class Workload:
    name: str
    index: int                      # seed offset of this workload
    description: str
    shapes: tuple                   # per-layer ((M, K), ...)
    layers: int
    batches: tuple                  # token counts N that are run
    x_dtype: str                    # "f32" or "bf16"
    y_dtype: str                    # "f32" or "bf16"
    weight_dist: str                # "uniform" or "p0_0.4"
    act_dist: str                   # "normal" or "student_t4"
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    fixed_scale: float | None = None
    proj_names: tuple = field(default=PROJ_NAMES)
    proj_input: tuple = field(default=PROJ_INPUT)

    @property
    def packed_bytes_per_layer(self) -> int:
        return sum(m * k // 4 for m, k in self.shapes)

    @property
    def packed_bytes_per_pass(self) -> int:
        return self.layers * self.packed_bytes_per_layer

    def input_widths(self):
        """K of each distinct input of a layer, in input-index order."""
        widths = {}
        for (m, k), src in zip(self.shapes, self.proj_input):
            widths.setdefault(src, k)
            assert widths[src] == k
        return [widths[i] for i in sorted(widths)]


GEMV_2560 = Workload(
    name="gemv_2560", index=1,
    description="single ternary GEMV, 1 token, K=2560 -> M=2560, uniform "
                "{-1,0,+1} weights, scale 0.02, fp32 N(0,1) activations",
    shapes=((2560, 2560),), layers=1, batches=(1,), x_dtype="f32",
    y_dtype="f32", weight_dist="uniform", act_dist="normal",
    fixed_scale=0.02, proj_names=("w",), proj_input=(0,))

LAYER2B_N1 = Workload(
    name="layer2b_n1", index=2,
    description="one BitNet-b1.58-2B-style block (7 projections), 1 token, "
                "P(0)=0.4, bf16 N(0,1) activations",
    shapes=LAYER_2B, layers=1, batches=(1,), x_dtype="bf16", y_dtype="bf16",
    weight_dist="p0_0.4", act_dist="normal")

LAYER2B_N64 = Workload(
    name="layer2b_n64", index=3,
    description="same block, batched decode of 64 tokens, bf16 N(0,1) with "
                "1% of channels x20",
    shapes=LAYER_2B, layers=1, batches=(64,), x_dtype="bf16", y_dtype="bf16",
    weight_dist="p0_0.4", act_dist="normal", outlier_frac=0.01,
    outlier_scale=20.0)

PREFILL2B_N2048 = Workload(
    name="prefill2b_n2048", index=4,
    description="prefill, 2048 tokens x the 7 projections of the 2560/6912 "
                "block, bf16 Student-t(4) activations",
    shapes=LAYER_2B, layers=1, batches=(2048,), x_dtype="bf16",
    y_dtype="bf16", weight_dist="p0_0.4", act_dist="student_t4")

STREAM70B = Workload(
    name="stream70b", index=5,
    description="80 blocks of hidden 8192 / FFN 28672 / 64 q + 8 kv heads "
                "(about 16 GB packed), 1 and 8 tokens, bf16 N(0,1) with 0.5% "
                "of channels x30",
    shapes=LAYER_70B, layers=80, batches=(1, 8), x_dtype="bf16",
    y_dtype="bf16", weight_dist="p0_0.4", act_dist="normal",
    outlier_frac=0.005, outlier_scale=30.0)

WORKLOADS = (GEMV_2560, LAYER2B_N1, LAYER2B_N64, PREFILL2B_N2048, STREAM70B)
BY_NAME = {w.name: w for w in WORKLOADS}


def weight_seed(wl: Workload, layer: int, proj: int) -> int:
    return MASTER_SEED + 1000 * wl.index + 10 * layer + proj


def act_seed(wl: Workload, layer: int, inp: int, n: int) -> int:
    return MASTER_SEED + 7_000_000 + 100_000 * wl.index + 1000 * n + 10 * layer + inp


def weight_scale(wl: Workload, proj: int) -> float:
    """Per-tensor weight scale of projection ``proj``: distinct per projection
    so that swapped tensors are caught."""
    if wl.fixed_scale is not None:
        return wl.fixed_scale
    return 0.02 * (1.0 + proj / 8.0)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def ternary_weights(M: int, K: int, dist: str, seed: int,
                    device="cpu") -> torch.Tensor:
    """int8 [M, K] with values in {-1, 0, +1}.

    "uniform": each state with probability 1/3.
    "p0_0.4":  P(0) = 0.4, P(+1) = P(-1) = 0.3.
    """
    g = _gen(seed, device)
    if dist == "uniform":
        return torch.randint(-1, 2, (M, K), generator=g, device=device,
                             dtype=torch.int8)
    if dist == "p0_0.4":
        u = torch.rand((M, K), generator=g, device=device)
        return ((u >= 0.7).to(torch.int8) - (u < 0.3).to(torch.int8))
    raise ValueError(dist)


def float_weights(M: int, K: int, dist: str, seed: int, dtype: str = "f32",
                  device="cpu") -> torch.Tensor:
    """Float weights [M, K] (float32 or bfloat16) for the weight quantizer.

    "normal":     N(0, 0.02^2), the spread of trained projection weights.
    "student_t4": 0.02 * Student-t with 4 degrees of freedom (heavy tails).
    "wide":       N(0, 1) * 2^u, u uniform on the integers [-130, 20]:
                  magnitudes spread over ~150 binades, subnormals included.
    "subnormal":  random float32 subnormal bit patterns with random signs.
    "zeros":      all zero.
    "ternarized": 0.0213 * t with t from ternary_weights(..., "p0_0.4"),
                  a tensor already rounded to {-g, 0, +g}.
    Values are drawn in float32 and cast (round to nearest) for bfloat16."""
    g = _gen(seed, device)
    if dist == "normal":
        w = torch.randn((M, K), generator=g, device=device) * 0.02
    elif dist == "student_t4":
        z = torch.randn((M, K), generator=g, device=device)
        chi2 = torch.zeros((M, K), device=device)
        for _ in range(4):
            e = torch.randn((M, K), generator=g, device=device)
            chi2 += e * e
        w = 0.02 * z / torch.sqrt(chi2 / 4.0)
    elif dist == "wide":
        z = torch.randn((M, K), generator=g, device=device)
        u = torch.randint(-130, 21, (M, K), generator=g, device=device)
        w = z * torch.exp2(u.to(torch.float32))
    elif dist == "subnormal":
        bits = torch.randint(0, 1 << 23, (M, K), generator=g, device=device,
                             dtype=torch.int32)
        sign = torch.randint(0, 2, (M, K), generator=g, device=device,
                             dtype=torch.int32) << 31
        w = (bits | sign).view(torch.float32)
    elif dist == "zeros":
        w = torch.zeros((M, K), device=device)
    elif dist == "ternarized":
        w = ternary_weights(M, K, "p0_0.4", seed, device).to(torch.float32) * 0.0213
    else:
        raise ValueError(dist)
    if dtype == "f32":
        return w.contiguous()
    if dtype == "bf16":
        return w.to(torch.bfloat16).contiguous()
    raise ValueError(dtype)


def activations(N: int, K: int, dist: str, seed: int, dtype: str,
                outlier_frac: float = 0.0, outlier_scale: float = 1.0,
                device="cpu") -> torch.Tensor:
    """Float activations [N, K] (float32 or bfloat16).

    Values are drawn in float32 ("normal": N(0,1); "student_t4": Student-t
    with 4 degrees of freedom, as z / sqrt(chi2_4 / 4)).  If outlier_frac > 0,
    round(outlier_frac * K) channels, picked by a seeded permutation and the
    same for every token, are multiplied by outlier_scale in float32 before
    the cast to bfloat16."""
    g = _gen(seed, device)
    if dist == "normal":
        x = torch.randn((N, K), generator=g, device=device)
    elif dist == "student_t4":
        z = torch.randn((N, K), generator=g, device=device)
        chi2 = torch.zeros((N, K), device=device)
        for _ in range(4):
            e = torch.randn((N, K), generator=g, device=device)
            chi2 += e * e
        x = z / torch.sqrt(chi2 / 4.0)
    else:
        raise ValueError(dist)
    if outlier_frac > 0.0:
        ch = outlier_channels(K, seed, outlier_frac, device)
        x[:, ch] *= outlier_scale
    if dtype == "f32":
        return x.contiguous()
    if dtype == "bf16":
        return x.to(torch.bfloat16).contiguous()
    raise ValueError(dtype)


def outlier_channels(K: int, seed: int, outlier_frac: float,
                     device="cpu") -> torch.Tensor:
    """The round(outlier_frac * K) channels that activations() scales for the
    same seed: the head of a permutation drawn from its own generator."""
    count = int(round(outlier_frac * K))
    g = _gen(seed + 1, device)
    return torch.randperm(K, generator=g, device=device)[:count]


def layer_weights(wl: Workload, layer: int, device="cpu"):
    """[(w_int8[M,K], scale), ...] for the seven (or one) projections."""
    out = []
    for p, (M, K) in enumerate(wl.shapes):
        w = ternary_weights(M, K, wl.weight_dist, weight_seed(wl, layer, p),
                            device)
        out.append((w, weight_scale(wl, p)))
    return out


def layer_inputs(wl: Workload, layer: int, N: int, device="cpu"):
    """The distinct float inputs of one layer, in input-index order."""
    return [activations(N, K, wl.act_dist, act_seed(wl, layer, i, N),
                        wl.x_dtype, wl.outlier_frac, wl.outlier_scale, device)
            for i, K in enumerate(wl.input_widths())]

"""Seeded synthetic workloads for the ConvRot linear (inputs only).

This module draws the inputs that both the HIP library and the CPU oracle are
fed.  It holds none of the method's arithmetic: no rotation, no quantization,
no matrix product.  All host-side draws use numpy's PCG64 (``default_rng``);
the 32-layer stack draws its weights on the device with torch's generator
because they total 6.2 G values.

The shapes stand in for the text-encoder workloads of the source pages
("MOSS-Image Qwen3.5-9B text encoder, INT8 (W8A8, ConvRot)", section
"Measured": a 32-decoder-layer encoder run over 34 prompts), which are not
available: activations are N(0, 1) with 1 % of the input channels scaled by 20
(outlier channels, the case ConvRot's rotation is for: "qwen3.5_4b_int8_convrot",
section "Why ConvRot"), weights are N(0, 0.02).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

OUTLIER_GAIN = 20.0
WEIGHT_STD = 0.02


@dataclass(frozen=True)
class Linear:
    name: str
    K: int
    N: int


@dataclass(frozen=True)
class Config:
    key: str
    description: str
    M: int
    linears: tuple
    n_outliers: tuple          # outlier channel count per linear (same order)
    seed: int
    wbits: int = 8
    group: int = 256
    layers: int = 1
    extra: dict = field(default_factory=dict)


def _one_percent(K: int) -> int:
    return int(round(0.01 * K))


# The five workloads.  C3u is the headline shape.
CONFIGS = {
    "C1": Config("C1", "single linear, M=16 K=512 N=256, 2 outlier channels",
                 16, (Linear("linear", 512, 256),), (2,), seed=0),
    "C2": Config("C2", "attention projection, M=512 K=4096 N=4096",
                 512, (Linear("proj", 4096, 4096),), (_one_percent(4096),), seed=1),
    "C3u": Config("C3u", "MLP up/gate, M=2048 K=4096 N=12288",
                  2048, (Linear("up", 4096, 12288),), (_one_percent(4096),), seed=2),
    "C3d": Config("C3d", "MLP down, M=2048 K=12288 N=4096",
                  2048, (Linear("down", 12288, 4096),), (_one_percent(12288),), seed=3),
    "C4": Config("C4", "32-layer decoder linear stack at 34 prompts x 256 tokens (M=8704)",
                 8704,
                 (Linear("q", 4096, 4096), Linear("k", 4096, 1024), Linear("v", 4096, 1024),
                  Linear("o", 4096, 4096), Linear("gate", 4096, 12288), Linear("up", 4096, 12288),
                  Linear("down", 12288, 4096)),
                 tuple(_one_percent(k) for k in (4096, 4096, 4096, 4096, 4096, 4096, 12288)),
                 seed=4, layers=32),
    "C5": Config("C5", "W4A8 variant, M=4096 K=4096 N=12288, int4 weights two per byte",
                 4096, (Linear("up", 4096, 12288),), (_one_percent(4096),), seed=8, wbits=4),
}

# In the stack, q/k/v share one input, gate/up share one, o and down have
# their own: four activation tensors per layer, drawn once with seeds 4..7
# and reused by every layer.
C4_INPUT_OF = {"q": 0, "k": 0, "v": 0, "o": 1, "gate": 2, "up": 2, "down": 3}
C4_INPUT_K = (4096, 4096, 4096, 12288)
C4_WEIGHT_SEED_BASE = 100


def float_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even) via torch's CPU cast;
    returns the raw bit patterns as uint16."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_float(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact fp32 values."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def outlier_channels(K: int, n_outliers: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng([seed, 1])
    return np.sort(rng.choice(K, size=n_outliers, replace=False))


def make_activations(M: int, K: int, n_outliers: int, seed: int) -> np.ndarray:
    """bf16 bits [M, K]: N(0, 1) with ``n_outliers`` input channels x20."""
    rng = np.random.default_rng([seed, 0])
    x = rng.standard_normal((M, K), dtype=np.float32)
    if n_outliers:
        x[:, outlier_channels(K, n_outliers, seed)] *= OUTLIER_GAIN
    return float_to_bf16_bits(x)


NORM_W_STD = 0.25


def make_norm_weight(K: int, n_outliers: int, seed: int) -> np.ndarray:
    """fp32 [K] stored RMSNorm weights w (the norm applies 1 + w), as left by
    a SmoothQuant fold: w ~ N(0, 0.25^2), and on the ``n_outliers`` outlier
    channels of ``make_activations(.., seed)`` the factor 1 + w is divided by
    sqrt(20) (the smoothing factor of a x20 channel at migration strength 0.5)."""
    rng = np.random.default_rng([seed, 3])
    w = rng.standard_normal(K, dtype=np.float32) * np.float32(NORM_W_STD)
    if n_outliers:
        ch = outlier_channels(K, n_outliers, seed)
        w[ch] = (np.float32(1) + w[ch]) / np.float32(np.sqrt(OUTLIER_GAIN)) - np.float32(1)
    return w.astype(np.float32)


def make_weight(N: int, K: int, seed: int) -> np.ndarray:
    """fp32 [N, K] drawn from N(0, 0.02^2)."""
    rng = np.random.default_rng([seed, 2])
    return (rng.standard_normal((N, K), dtype=np.float32) * np.float32(WEIGHT_STD)).astype(np.float32)


def make_weight_device(N: int, K: int, seed: int, device):
    """fp32 [N, K] N(0, 0.02^2) drawn on ``device`` with torch's generator
    (used for the 32-layer stack, whose weights are too many for the host)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.randn((N, K), generator=g, device=device, dtype=torch.float32) * WEIGHT_STD


def config_inputs(key: str):
    """(x_bf16_bits [M, K], w_fp32 [N, K]) for the single-linear configs."""
    cfg = CONFIGS[key]
    assert len(cfg.linears) == 1, "the stack config is drawn per layer"
    lin = cfg.linears[0]
    x = make_activations(cfg.M, lin.K, cfg.n_outliers[0], cfg.seed)
    w = make_weight(lin.N, lin.K, cfg.seed)
    return x, w


def stack_activations(layer_inputs=C4_INPUT_K, M: int = 8704, base_seed: int = 4):
    """The four shared activation tensors of the 32-layer stack (seeds 4..7)."""
    return [make_activations(M, K, _one_percent(K), base_seed + i) for i, K in enumerate(layer_inputs)]

"""Seeded synthetic inputs and layer shapes for the QLoRA linear layer.

This module holds no arithmetic of the method: it only names shapes and draws
random tensors.  Both the CPU oracle and the HIP path receive the same arrays
from here.

The pages' workloads are LLaMA finetunes (7B-65B) on instruction datasets; no
weights or data are available, so seeded Gaussian tensors of LLaMA layer
shapes stand in for them:
  W  ~ N(0, 0.02) fp32           (frozen base weight, before quantization)
  X, dY ~ N(0, 1)  -> bf16       (activations / output gradients)
  A, B  ~ N(0, 0.01) -> bf16     (LoRA pair; B is non-zero on purpose so the
                                  LoRA branch is exercised)
bf16 rounding of inputs uses torch's fp32 -> bf16 conversion (round to
nearest even).  Host tensors come from NumPy PCG64 with
seed = 1000 * config_index + tensor_index.
"""

from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np

W_STD = 0.02
ACT_STD = 1.0
LORA_STD = 0.01


@dataclass(frozen=True)
class Linear:
    name: str
    out_features: int   # N (rows of W)
    in_features: int    # K (columns of W)


@dataclass(frozen=True)
class LayerConfig:
    index: int
    name: str
    linears: Tuple[Linear, ...]
    tokens: int         # M
    rank: int           # r
    alpha: float
    layers: int = 1
    small_m: Tuple[int, ...] = field(default_factory=tuple)

    @property
    def scale(self) -> float:
        return float(np.float32(self.alpha) / np.float32(self.rank))


def llama_linears(hidden: int, ffn: int) -> Tuple[Linear, ...]:
    """The seven linears of a LLaMA decoder layer, W shape [out, in]."""
    return (
        Linear("q_proj", hidden, hidden),
        Linear("k_proj", hidden, hidden),
        Linear("v_proj", hidden, hidden),
        Linear("o_proj", hidden, hidden),
        Linear("gate_proj", ffn, hidden),
        Linear("up_proj", ffn, hidden),
        Linear("down_proj", hidden, ffn),
    )


CONFIGS: List[LayerConfig] = [
    LayerConfig(0, "linear_1024x1024_m128_r8",
                (Linear("linear", 1024, 1024),), tokens=128, rank=8, alpha=16.0),
    LayerConfig(1, "llama7b_layer_m8192_r64",
                llama_linears(4096, 11008), tokens=8192, rank=64, alpha=16.0),
    LayerConfig(2, "llama7b_layer_small_m_r64",
                llama_linears(4096, 11008), tokens=1, rank=64, alpha=16.0,
                small_m=(1, 16, 64)),
    LayerConfig(3, "llama33b_layer_m8192_r64",
                llama_linears(6656, 17920), tokens=8192, rank=64, alpha=16.0),
    LayerConfig(4, "llama65b_80layers_m16384_r64",
                llama_linears(8192, 22016), tokens=16384, rank=64, alpha=16.0,
                layers=80),
]


def seed_for(config_index: int, tensor_index: int) -> int:
    return 1000 * config_index + tensor_index


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal_fp32(shape, std: float, seed: int) -> np.ndarray:
    """N(0, std^2) as float32, drawn in float32 by PCG64."""
    g = _rng(seed)
    return (g.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16) via torch's round-to-nearest-even cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def weight(shape, seed: int) -> np.ndarray:
    return normal_fp32(shape, W_STD, seed)


def activation_bf16(shape, seed: int, std: float = ACT_STD) -> np.ndarray:
    return to_bf16_bits(normal_fp32(shape, std, seed))


def lora_bf16(shape, seed: int) -> np.ndarray:
    return to_bf16_bits(normal_fp32(shape, LORA_STD, seed))


def linear_inputs(cfg: LayerConfig, linear_index: int, tokens: int = None):
    """Host inputs for one linear of a config: dict of numpy arrays.

    Tensor indices within a config: 10*linear_index + {0: W, 1: X, 2: A, 3: B, 4: dY}.
    """
    lin = cfg.linears[linear_index]
    m = cfg.tokens if tokens is None else tokens
    n, k, r = lin.out_features, lin.in_features, cfg.rank
    base = 10 * linear_index
    s = lambda t: seed_for(cfg.index, base + t)
    return dict(
        W=weight((n, k), s(0)),
        X=activation_bf16((m, k), s(1)),
        A=lora_bf16((r, k), s(2)),
        B=lora_bf16((n, r), s(3)),
        dY=activation_bf16((m, n), s(4)),
        scale=cfg.scale, M=m, N=n, K=k, r=r,
    )


def device_normal(shape, std: float, seed: int, device, dtype=None):
    """N(0, std^2) drawn on a torch device with a seeded torch.Generator."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    t.mul_(std)
    return t if dtype is None else t.to(dtype)


def device_layer_weights(cfg: LayerConfig, layer: int, device):
    """The frozen weights of one layer of a multi-layer config, drawn on the
    device: one torch.Generator seeded 65000 + layer draws the layer's linears
    in order (q, k, v, o, gate, up, down) as N(0, W_STD^2) fp32 [out, in].
    Yields (linear, tensor); each tensor is a fresh allocation."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(65000 + layer)
    for lin in cfg.linears:
        t = torch.randn((lin.out_features, lin.in_features), generator=g, device=device, dtype=torch.float32)
        t.mul_(W_STD)
        yield lin, t

"""Seeded synthetic layers for the SparseGPT layer solver.

Random weights and calibration activations shaped like the decoder layers the
pages prune (7B-class 4096 / 11008 wide, 70B-class 8192 / 28672 wide).  This
module only draws random numbers: it holds none of the method's arithmetic, and
both the HIP path and the oracle receive the bytes it produces.

Distribution recipe (one reading of a terse spec, applied to every config):
  * W ~ N(0, std^2), then rounded to the layer dtype (bf16 round-to-nearest-even
    through torch's cast).
  * Per-channel activation scale s_c = exp(g_c), g_c ~ N(0, 1).
  * A set of outlier channels (uniform without replacement) has its scale
    multiplied by a factor (x20 for the attention/MLP-up inputs, x10 for the
    post-activation inputs, where the set is floor(1% of n) channels).
  * Token t, channel c: x = s_c * z  or  x = s_c * max(z, 0)  (post-activation),
    z ~ N(0, 1) i.i.d.; sequences are only a chunking unit.
  * Seeds: base + 1000 * config_id + stream, with stream 0 = W, 1 = scales,
    2 = outlier set, 100 + i = token chunk i.  Token chunks are drawn
    independently, so any chunk can be regenerated on its own.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import torch

BASE_SEED = 20231


@dataclass(frozen=True)
class LayerConfig:
    name: str
    m: int                 # rows of W (output channels)
    n: int                 # columns of W (input channels)
    tokens: int            # calibration tokens N
    w_std: float
    dtype: str             # "f32" or "bf16" (both W and X)
    act: str               # "linear" or "relu"
    outliers: int          # number of outlier channels
    outlier_factor: float
    patterns: Tuple[str, ...]
    blocksize: int
    damp: float = 0.01
    config_id: int = 0
    chunk_tokens: int = 32768
    x_source: Optional[str] = None   # reuse another config's activations


# The five workloads: a tiny parity layer, then attention-projection, MLP-up,
# MLP-down and large MLP-down shaped layers.
CONFIGS = {
    "tiny": LayerConfig("tiny", 64, 128, 512, 0.02, "f32", "linear", 0, 1.0,
                        ("0.5",), 32, config_id=0, chunk_tokens=512),
    "attn_4096": LayerConfig("attn_4096", 4096, 4096, 128 * 2048, 0.02, "bf16",
                             "linear", 8, 20.0, ("0.5",), 128, config_id=1),
    "mlp_up_11008": LayerConfig("mlp_up_11008", 11008, 4096, 128 * 2048, 0.02,
                                "bf16", "linear", 8, 20.0, ("2:4",), 128,
                                config_id=2, x_source="attn_4096"),
    "mlp_down_11008": LayerConfig("mlp_down_11008", 4096, 11008, 128 * 2048,
                                  0.015, "bf16", "relu", 110, 10.0,
                                  ("0.6", "4:8"), 128, config_id=3),
    "mlp_down_28672": LayerConfig("mlp_down_28672", 8192, 28672, 256 * 2048,
                                  0.01, "bf16", "relu", 286, 10.0,
                                  ("0.5", "2:4"), 128, config_id=4),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make_weight(cfg: LayerConfig, device="cpu") -> torch.Tensor:
    seed = BASE_SEED + 1000 * cfg.config_id + 0
    w = torch.randn(cfg.m, cfg.n, generator=_gen(seed, device), device=device,
                    dtype=torch.float32) * cfg.w_std
    return w.to(_torch_dtype(cfg.dtype)).contiguous()


def _x_cfg(cfg: LayerConfig) -> LayerConfig:
    return CONFIGS[cfg.x_source] if cfg.x_source else cfg


def channel_scales(cfg: LayerConfig, device="cpu") -> torch.Tensor:
    xc = _x_cfg(cfg)
    g = torch.randn(xc.n, generator=_gen(BASE_SEED + 1000 * xc.config_id + 1, device),
                    device=device, dtype=torch.float32)
    s = torch.exp(g)
    if xc.outliers > 0:
        perm = torch.randperm(xc.n, generator=_gen(BASE_SEED + 1000 * xc.config_id + 2, device),
                              device=device)
        s[perm[:xc.outliers]] *= xc.outlier_factor
    return s


def make_x_chunk(cfg: LayerConfig, index: int, tokens: int, device="cpu",
                 scales: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Token-major activation chunk [tokens, n] in the layer dtype."""
    xc = _x_cfg(cfg)
    if scales is None:
        scales = channel_scales(cfg, device)
    seed = BASE_SEED + 1000 * xc.config_id + 100 + index
    z = torch.randn(tokens, xc.n, generator=_gen(seed, device), device=device,
                    dtype=torch.float32)
    if xc.act == "relu":
        z.clamp_(min=0.0)
    z.mul_(scales[None, :])
    return z.to(_torch_dtype(xc.dtype)).contiguous()


def make_x(cfg: LayerConfig, device="cpu", tokens: Optional[int] = None,
           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """All calibration tokens as one token-major [N, n] tensor (chunked draw)."""
    xc = _x_cfg(cfg)
    N = tokens if tokens is not None else xc.tokens
    if out is None:
        out = torch.empty(N, xc.n, dtype=_torch_dtype(xc.dtype), device=device)
    scales = channel_scales(cfg, device)
    step = xc.chunk_tokens
    for i, t0 in enumerate(range(0, N, step)):
        t1 = min(N, t0 + step)
        out[t0:t1] = make_x_chunk(cfg, i, t1 - t0, device, scales)
    return out


def scaled_config(cfg: LayerConfig, m: int, n: int, tokens: int,
                  blocksize: Optional[int] = None, patterns=None,
                  name: Optional[str] = None) -> LayerConfig:
    """Same distribution at a smaller (oracle-sized) shape."""
    outl = cfg.outliers
    if cfg.act == "relu":
        outl = max(1, int(0.01 * n)) if cfg.outliers else 0
    else:
        outl = min(cfg.outliers, n // 4)
    return LayerConfig(name or f"{cfg.name}_{m}x{n}", m, n, tokens, cfg.w_std,
                       cfg.dtype, cfg.act, outl, cfg.outlier_factor,
                       tuple(patterns or cfg.patterns),
                       blocksize or cfg.blocksize, cfg.damp,
                       config_id=cfg.config_id + 50,
                       chunk_tokens=min(cfg.chunk_tokens, tokens))


def random_spd_inputs(seed: int, n: int, tokens: int, device="cpu",
                      corr: float = 0.5) -> torch.Tensor:
    """Correlated fp32 activations [tokens, n] for small algebra tests:
    x = z A with a random mixing matrix, plus log-normal channel scales."""
    g = _gen(seed, device)
    A = torch.eye(n, device=device) + corr * torch.randn(n, n, generator=g, device=device) / n ** 0.5
    z = torch.randn(tokens, n, generator=g, device=device)
    s = torch.exp(torch.randn(n, generator=g, device=device))
    return (z @ A) * s[None, :]


def random_weight(seed: int, m: int, n: int, std: float = 0.02, device="cpu") -> torch.Tensor:
    return torch.randn(m, n, generator=_gen(seed, device), device=device) * std

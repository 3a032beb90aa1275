"""Seeded synthetic inputs for ReHyAt hybrid attention (shared by the tests, the bench and smoke()).

This module draws random tensors and rounds them to the storage precision. It holds none of
the method's arithmetic: no feature map, no index sets, no attention. Both the float64
oracle and the HIP path consume exactly the tensors produced here.

Workload shapes are those of the Wan2.1-1.3B video DiT latents named on the ReHyAt pages:
the 21x30x52 latent of a 5 s video at 480x832 (sciencestack.ai abstract page of ReHyAt,
Fig. 4 caption) and the 320x480 / 480x832 resolutions of Fig. 5; 12 heads of width 128.
Tokens are time-major (frame f, spatial index s -> token f*HW+s), as in the papernotes.org
ReHyAt note, key design 1.

Recipe: one torch.Generator (CPU) seeded with the config's seed; draws in this order
  1. W  [D, F] ~ N(0, 1/D)                          (feature-map weights, shared by phi_q,
                                                     phi_k and every head)
  2. extras:  head_scale   -> s_h ~ U(0.5, 2) for each head h (applied to q, k, v of that
                              head in every batch item)
              frame_offset -> o_{b,h,f} ~ N(0, I_D) for every frame, added as 0.5*o to q and
                              k of every token of frame f
  3. q, k, v [B, H, N, D] ~ N(0, 1), float32, in that order.
Then every tensor is rounded to the storage dtype (bf16 with round-to-nearest-even, or kept
float32). torch's CPU generator gives the same draws for any thread count.

Parameters of the learned polynomial feature map (make_mlp_map_params), from a generator of
their own seed; per head when `heads` is given (leading dimension H), drawn in this order:
  W1 [D, h] ~ N(0, 1/D)              (so x W1 ~ N(0, 1) for x ~ N(0, I_D))
  b1 [h]    ~ N(0, b1_std^2)
  W2 [h, F] ~ N(0, 2 psi_std^2 / h)  (relu of a unit normal has second moment 1/2, so the
                                      random part of psi has standard deviation ~ psi_std)
  b2 [F]    = psi_mean[i] on the features of part i (no draw)
all rounded to bf16. psi_mean sets where psi sits; the feature products phi(q).phi(k) then
have a known sign and scale, as a trained map imitating exp would give.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np
import torch

__all__ = [
    "HybridConfig", "CONFIGS", "config", "make_inputs", "make_custom", "to_f64", "TORCH_DTYPE",
    "make_mlp_map_params", "make_upstream",
]

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class HybridConfig:
    """Shape, precision and form of one synthetic hybrid-attention workload."""
    name: str
    B: int
    H: int
    D: int
    T: int            # latent frames
    HW: int           # spatial tokens per frame
    Tc: int           # frames per chunk
    To: int           # overlap frames reaching back from each chunk
    F: int            # feature dimension of phi
    dtype: str        # "f32" or "bf16" (storage and MFMA operand type)
    mode: str         # "causal" or "bidir"
    form: str         # "fwd" (whole sequence, one call) or "stream" (one call per chunk)
    seed: int
    extra: str = "none"   # "none" | "head_scale" | "frame_offset"
    description: str = ""

    @property
    def N(self) -> int:
        return self.T * self.HW

    @property
    def n_chunks(self) -> int:
        return -(-self.T // self.Tc)

    def replace(self, **kw) -> "HybridConfig":
        return dataclasses.replace(self, **kw)


CONFIGS: List[HybridConfig] = [
    HybridConfig("c1_tiny_f32", B=1, H=2, D=64, T=6, HW=64, Tc=2, To=1, F=64,
                 dtype="f32", mode="causal", form="fwd", seed=1,
                 description="tiny causal, fp32, 6 frames x 8x8 tokens"),
    HybridConfig("c2_320x480_bidir", B=1, H=12, D=128, T=21, HW=600, Tc=3, To=1, F=128,
                 dtype="bf16", mode="bidir", form="fwd", seed=2,
                 description="21x20x30 latent (320x480), bidirectional chunked form"),
    HybridConfig("c3_480x832_causal", B=2, H=12, D=128, T=21, HW=1560, Tc=3, To=1, F=128,
                 dtype="bf16", mode="causal", form="fwd", seed=3, extra="head_scale",
                 description="21x30x52 latent (480x832, 5 s), batch 2 (cond/uncond), causal"),
    HybridConfig("c4_81f_stream", B=1, H=12, D=128, T=81, HW=1560, Tc=3, To=1, F=128,
                 dtype="bf16", mode="causal", form="stream", seed=4,
                 description="81x30x52 latent streamed as 27 recurrent steps"),
    HybridConfig("c5_wide_chunk", B=1, H=12, D=128, T=49, HW=1560, Tc=7, To=3, F=256,
                 dtype="bf16", mode="causal", form="fwd", seed=5, extra="frame_offset",
                 description="49x30x52 latent, Tc=7, To=3, F=256, frame-correlated q/k"),
]


def config(i_or_name) -> HybridConfig:
    """Config by 1-based index (1..5) or by name."""
    if isinstance(i_or_name, int):
        return CONFIGS[i_or_name - 1]
    for c in CONFIGS:
        if c.name == i_or_name:
            return c
    raise KeyError(i_or_name)


def make_custom(B: int, H: int, N: int, D: int, F: int, *, seed: int, dtype: str,
                HW: Optional[int] = None, extra: str = "none",
                w_std: Optional[float] = None) -> Dict[str, torch.Tensor]:
    """Draw W, q, k, v for an arbitrary shape with the recipe in the module docstring.

    Returns CPU tensors in the storage dtype: "W" [D, F], "q", "k", "v" [B, H, N, D], and
    "head_scale" [H] when that extra is used.
    """
    if dtype not in TORCH_DTYPE:
        raise ValueError(f"unknown dtype {dtype!r}")
    g = torch.Generator().manual_seed(int(seed))
    std = (1.0 / np.sqrt(D)) if w_std is None else float(w_std)
    W = torch.randn((D, F), generator=g) * std
    scale = None
    offset = None
    if extra == "head_scale":
        scale = torch.empty(H).uniform_(0.5, 2.0, generator=g)
    elif extra == "frame_offset":
        if HW is None or N % HW:
            raise ValueError("frame_offset needs HW dividing N")
        offset = torch.randn((B, H, N // HW, 1, D), generator=g)
    elif extra != "none":
        raise ValueError(f"unknown extra {extra!r}")
    out: Dict[str, torch.Tensor] = {"W": W.to(TORCH_DTYPE[dtype])}
    for name in ("q", "k", "v"):
        x = torch.randn((B, H, N, D), generator=g)
        if scale is not None:
            x.mul_(scale.view(1, H, 1, 1))
        if offset is not None and name in ("q", "k"):
            x.view(B, H, N // HW, HW, D).add_(offset, alpha=0.5)
        out[name] = x.to(TORCH_DTYPE[dtype])
        del x
    if scale is not None:
        out["head_scale"] = scale
    return out


def make_mlp_map_params(D: int, hidden: int, F: int, *, seed: int, P: int = 2,
                        heads: Optional[int] = None, psi_mean=None, psi_std: float = 0.05,
                        b1_std: float = 0.1) -> Dict[str, torch.Tensor]:
    """W1, b1, W2, b2 (bf16, CPU) of the learned feature map, recipe in the module
    docstring. psi_mean: one value per part (default: 1/sqrt(F/P) on part 1, 0 elsewhere)."""
    if F % P:
        raise ValueError("F must split into P parts")
    if psi_mean is None:
        psi_mean = [1.0 / np.sqrt(F // P)] + [0.0] * (P - 1)
    if len(psi_mean) != P:
        raise ValueError("psi_mean needs one value per part")
    g = torch.Generator().manual_seed(int(seed))
    lead = () if heads is None else (int(heads),)
    W1 = torch.randn(lead + (D, hidden), generator=g) / np.sqrt(D)
    b1 = torch.randn(lead + (hidden,), generator=g) * b1_std
    W2 = torch.randn(lead + (hidden, F), generator=g) * (psi_std * np.sqrt(2.0 / hidden))
    b2 = torch.tensor(np.repeat(np.asarray(psi_mean, dtype=np.float64), F // P),
                      dtype=torch.float32).expand(lead + (F,)).clone()
    return {n: t.to(torch.bfloat16) for n, t in (("W1", W1), ("b1", b1), ("W2", W2), ("b2", b2))}


def make_upstream(shape, *, seed: int, dtype: str) -> torch.Tensor:
    """Seeded upstream gradient dy ~ N(0, 1) of the given shape, rounded to `dtype`
    (generator seeded with seed + 7919, drawn after nothing else)."""
    g = torch.Generator().manual_seed(int(seed) + 7919)
    return torch.randn(tuple(shape), generator=g).to(TORCH_DTYPE[dtype])


def make_inputs(cfg: HybridConfig) -> Dict[str, torch.Tensor]:
    """Seeded inputs of one named workload (see the module docstring for the recipe)."""
    return make_custom(cfg.B, cfg.H, cfg.N, cfg.D, cfg.F, seed=cfg.seed, dtype=cfg.dtype,
                       HW=cfg.HW, extra=cfg.extra)


def to_f64(x: torch.Tensor) -> np.ndarray:
    """Exact float64 numpy copy of a stored (bf16 or fp32) CPU tensor."""
    return x.detach().to("cpu", torch.float64).numpy()

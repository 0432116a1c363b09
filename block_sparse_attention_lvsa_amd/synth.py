"""Seeded synthetic Q/K/V for the LVSA attention workloads.

This module holds no arithmetic of the method: it only draws seeded normal
samples of the workloads' shapes and rounds them to bf16.  It is the one
module that both the oracle-side tests and the HIP-side calls take their
inputs from.

Workloads (shapes from the pages' 480×832 video: 1560 tokens per latent
frame; horizons 1× and 6× of Wan 2.1 (21 and 121 latent frames); 1.5× and 2×
(49 and 65 latent frames) for the HunyuanVideo-like assumed shape):

  name        B  H  d    T    P     C   W   seed  distribution
  tiny        1  2  64   8    64    4   2   1     iid N(0,1)
  wan13b_1x   1  12 128  21   1560  21  9   2     iid N(0,1)  (mask is dense)
  wan13b_6x   1  12 128  121  1560  21  9   3     iid N(0,1)
  wan14b_6x   1  40 128  121  1560  21  9   4     iid N(0,1) + per-frame N(0,0.5²)
  syn_1p5x    1  16 128  49   1560  33  13  5     iid N(0,1)
  syn_2x      1  16 128  65   1560  33  13  6     iid N(0,1)
  wan13b_720p_6x  1 12 128 121 3600 21 9  7     iid N(0,1)
  wan22_720p_6x_h5 1 5 128 121 3600 21 9  8     iid N(0,1) + per-frame N(0,0.5²)

The two 720p workloads take the pages' 720×1280 runs (TechWalker article,
§五) with the latent grid assumed to shrink as at 480×832 (×8 spatially by
the VAE, ×2 by the patch embedding: 45×80 = 3600 tokens per latent frame).
``wan22_720p_6x_h5`` is one device's share of the Wan 2.2-A14B run, whose 40
heads the pages split over 8 devices by sequence parallelism: 5 heads at the
full sequence length.

Recipe: ``torch.Generator(device).manual_seed(seed)``; ``torch.randn`` in
float32 drawn in the order q, k, v (then the per-frame components z_q, z_k,
z_v of shape [B, H, T, d] for the temporally-correlated workload, added to
every token of the frame); then round-to-nearest-even to bf16.  The draw is
done on the device the tensors are used on; a CPU consumer receives exactly
the same bf16 values by copying them (or slices of them) back.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    D: int
    T: int
    P: int
    C: int
    W: int
    seed: int
    frame_std: float = 0.0
    steps: Tuple[int, ...] = field(default_factory=lambda: tuple(range(50)))

    @property
    def N(self) -> int:
        return self.T * self.P


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 64, 8, 64, 4, 2, 1, steps=tuple(range(8))),
    "wan13b_1x": Workload("wan13b_1x", 1, 12, 128, 21, 1560, 21, 9, 2),
    "wan13b_6x": Workload("wan13b_6x", 1, 12, 128, 121, 1560, 21, 9, 3),
    "wan14b_6x": Workload("wan14b_6x", 1, 40, 128, 121, 1560, 21, 9, 4, frame_std=0.5),
    "syn_1p5x": Workload("syn_1p5x", 1, 16, 128, 49, 1560, 33, 13, 5),
    "syn_2x": Workload("syn_2x", 1, 16, 128, 65, 1560, 33, 13, 6),
    "wan13b_720p_6x": Workload("wan13b_720p_6x", 1, 12, 128, 121, 3600, 21, 9, 7),
    "wan22_720p_6x_h5": Workload("wan22_720p_6x_h5", 1, 5, 128, 121, 3600, 21, 9, 8, frame_std=0.5),
}


def make_qkv(w: Workload, device="cpu", dtype=torch.bfloat16):
    """Seeded q, k, v of shape [B, H, T·P, d], rounded to ``dtype`` (RNE)."""
    dev = torch.device(device)
    g = torch.Generator(device=dev).manual_seed(w.seed)
    shape = (w.B, w.H, w.N, w.D)
    out = []
    for _ in range(3):
        x = torch.randn(shape, generator=g, device=dev, dtype=torch.float32)
        out.append(x)
    if w.frame_std > 0.0:
        for i in range(3):
            z = torch.randn((w.B, w.H, w.T, w.D), generator=g, device=dev,
                            dtype=torch.float32) * w.frame_std
            x = out[i].view(w.B, w.H, w.T, w.P, w.D)
            x += z.unsqueeze(3)
    return tuple(x.to(dtype) for x in out)


def make_random(shape, seed: int, device="cpu", dtype=torch.bfloat16, std: float = 1.0):
    """One seeded N(0, std²) tensor of ``shape`` rounded to ``dtype``."""
    dev = torch.device(device)
    g = torch.Generator(device=dev).manual_seed(seed)
    x = torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * std
    return x.to(dtype)

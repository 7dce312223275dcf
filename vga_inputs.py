"""Seeded synthetic inputs for alternating attention (shared by the tests, the
smoke check and the benchmark; holds none of the method's arithmetic).

Shapes follow the pages: a 518x518 frame cut into 14x14 patches gives a
37x37 grid of 1369 patch tokens ("VGGT (CVPR 2025) Dissection", section 2.5,
worked example), followed by special tokens; heads of width 64.

Two recipes:

* ``tiny_qkv`` -- Q, K, V i.i.d. N(0, 1), float32, drawn in that order from
  ``numpy.random.default_rng(seed)``.
* ``feature_field_qkv`` -- stands in for real multi-view scenes (the pages'
  dense 100-800 frame sequences; no dataset or trained weights are used).
  A shared 2D feature field F ~ N(0,1) of shape [gh+16, gw+16, C] is sampled
  per frame at an integer shift (dy, dx) in [-8, 8]^2; patch (r, c) of a
  frame takes F[r+8+dy, c+8+dx] + 0.1*eps; the S special tokens are one shared
  N(0,1) [S, C] block + 0.1*eps per frame; eps ~ N(0,1).  Q, K, V = X @ W with
  W ~ N(0, 1/C) [C, C], C = H*64, computed in fp32 and rounded to bf16, viewed
  as [T, H, 64].  Draw order: F, shifts, specials, eps, Wq, Wk, Wv, all from
  one ``torch.Generator`` on the target device seeded with ``seed``.
* ``feature_field_block`` -- the inputs of a whole attention block (the
  projections around the attention): the same token features X (before any
  projection) in bf16 [T, C], and the weights of the QKV projection
  W_qkv ~ N(0, 1/C) [3C, C] with bias b_qkv ~ N(0, 0.1^2) [3C], and of the
  output projection W_o ~ N(0, 1/C) [C, C] with b_o ~ N(0, 0.1^2) [C], drawn
  after X in that order from the same generator.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    num_frames: int
    grid_h: int
    grid_w: int
    num_special: int
    num_heads: int
    head_dim: int
    dtype: str          # "f32" or "bf16"
    seed: int

    @property
    def tokens_per_frame(self) -> int:
        return self.grid_h * self.grid_w + self.num_special

    @property
    def tokens(self) -> int:
        return self.num_frames * self.tokens_per_frame


# The five workloads: tiny oracle check, the N=4 worked example, and the
# 100 / 300 / 800-frame sequences (37x37 grid + 5 specials = 1374 tokens/frame).
TINY = Workload("tiny N=2 8x8+5 H=2 fp32", 2, 8, 8, 5, 2, 64, "f32", 0)
N4 = Workload("N=4 37x37+5 H=16 bf16", 4, 37, 37, 5, 16, 64, "bf16", 1)
N100 = Workload("N=100 37x37+5 H=16 bf16", 100, 37, 37, 5, 16, 64, "bf16", 2)
N300 = Workload("N=300 37x37+5 H=16 bf16", 300, 37, 37, 5, 16, 64, "bf16", 3)
N800 = Workload("N=800 37x37+5 H=16 bf16", 800, 37, 37, 5, 16, 64, "bf16", 4)
WORKLOADS = {"tiny": TINY, "n4": N4, "n100": N100, "n300": N300, "n800": N800}


def tiny_qkv(T: int, H: int, d: int = 64, seed: int = 0):
    """Q, K, V float32 [T, H, d], i.i.d. N(0,1), drawn Q then K then V."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, d)).astype(np.float32)
    k = rng.standard_normal((T, H, d)).astype(np.float32)
    v = rng.standard_normal((T, H, d)).astype(np.float32)
    return q, k, v


def feature_field_qkv(N: int, gh: int, gw: int, S: int, H: int, d: int = 64,
                      seed: int = 1, device="cpu", dtype=None):
    """Shifted-feature-field Q, K, V as torch tensors [N*L, H, d] (bf16 default)."""
    import torch

    dtype = dtype or torch.bfloat16
    C = H * d
    L = gh * gw + S
    T = N * L
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    field = torch.randn(gh + 16, gw + 16, C, generator=g, device=device)
    shifts = torch.randint(-8, 9, (N, 2), generator=g, device=device)
    specials = torch.randn(S, C, generator=g, device=device)
    x = torch.randn(T, C, generator=g, device=device)   # eps, scaled below
    x.mul_(0.1)
    rows = torch.arange(gh, device=device).view(gh, 1) + 8
    cols = torch.arange(gw, device=device).view(1, gw) + 8
    xv = x.view(N, L, C)
    # frame by frame keeps the temporary small at N = 800
    shifts = shifts.cpu()
    for f in range(N):
        dy, dx = int(shifts[f, 0]), int(shifts[f, 1])
        patch = field[rows + dy, cols + dx].reshape(gh * gw, C)
        xv[f, : gh * gw] += patch
        xv[f, gh * gw:] += specials
    out = []
    for _ in range(3):
        w = torch.randn(C, C, generator=g, device=device).mul_(C ** -0.5)
        out.append(torch.matmul(x, w).to(dtype).view(T, H, d))
        del w
    del x
    return tuple(out)


def feature_field_block(N: int, gh: int, gw: int, S: int, H: int, seed: int = 1,
                        device="cpu"):
    """(x, w_qkv, b_qkv, w_o, b_o) in bf16: shifted-feature-field tokens
    [N*L, 64H] and random projection weights (see the module docstring)."""
    import torch

    C = H * 64
    L = gh * gw + S
    T = N * L
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    field = torch.randn(gh + 16, gw + 16, C, generator=g, device=device)
    shifts = torch.randint(-8, 9, (N, 2), generator=g, device=device).cpu()
    specials = torch.randn(S, C, generator=g, device=device)
    x = torch.randn(T, C, generator=g, device=device).mul_(0.1)
    rows = torch.arange(gh, device=device).view(gh, 1) + 8
    cols = torch.arange(gw, device=device).view(1, gw) + 8
    xv = x.view(N, L, C)
    for f in range(N):
        dy, dx = int(shifts[f, 0]), int(shifts[f, 1])
        xv[f, : gh * gw] += field[rows + dy, cols + dx].reshape(gh * gw, C)
        xv[f, gh * gw:] += specials
    bf = torch.bfloat16
    w_qkv = torch.randn(3 * C, C, generator=g, device=device).mul_(C ** -0.5).to(bf)
    b_qkv = torch.randn(3 * C, generator=g, device=device).mul_(0.1).to(bf)
    w_o = torch.randn(C, C, generator=g, device=device).mul_(C ** -0.5).to(bf)
    b_o = torch.randn(C, generator=g, device=device).mul_(0.1).to(bf)
    return x.to(bf), w_qkv, b_qkv, w_o, b_o


def seeded_rows(T: int, count: int, seed: int) -> np.ndarray:
    """Sorted distinct query rows, uniform over [0, T), for sampled checks."""
    rng = np.random.default_rng(seed)
    count = min(count, T)
    return np.sort(rng.choice(T, size=count, replace=False)).astype(np.int64)

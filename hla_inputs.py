"""Seeded synthetic inputs for the gated linear / gated softmax attention path.

This module only draws random tensors and names workload shapes. It holds none of
the attention arithmetic, so both the fp64 oracle (``oracle/``) and the HIP path
(``softmax_attention_amd``) can take their inputs from it without sharing code.

Shapes follow the spatio-temporal latent token sequences the SANA-Video 2.0 pages
describe (480x832 video at 81/121/193 frames, "about 19,000 tokens" at 720p; page
"SANA-Video 2.0 ... (ai-papers.net)", sections on hybrid linear attention and on
experimental results). The pages publish no tensors, so every value here is
i.i.d. N(0, 1) from a seeded CPU generator, rounded to bf16 (round to nearest even)
for the bf16 workloads, or to OCP fp8 e4m3 for fp8 inputs (torch's cast; N(0, 1)
draws stay far inside its +-448 range). The same rounded tensors go to the GPU and,
upcast exactly, to the oracle.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

import torch

SEED_BASE = 20261203
# tensor slot inside a layer's seed: q, k, v, g, and the residual stream x0
SLOT = {"q": 0, "k": 1, "v": 2, "g": 3, "x0": 4, "summary": 5, "router": 6}

LINEAR = 0
SOFTMAX = 1


@dataclass(frozen=True)
class Workload:
    """One named workload: shape, dtype and which operators it exercises."""

    index: int          # 1-based workload number; part of the seed
    name: str
    B: int
    H: int
    N: int
    D: int
    dtype: str          # "f32", "bf16" or "fp8"
    latent: Tuple[int, int, int]  # (T, H, W) latent grid; N = T*H*W
    kinds: Tuple[int, ...] = (LINEAR, SOFTMAX)
    eps: float = 1e-6
    note: str = ""

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[self.dtype]

    @property
    def scale(self) -> float:
        return self.D ** -0.5


WORKLOADS: List[Workload] = [
    Workload(1, "tiny_f32", 1, 2, 256, 32, "f32", (4, 8, 8),
             note="one gated linear + one gated softmax layer, fp32"),
    Workload(2, "480p_81f", 2, 16, 8190, 128, "bf16", (21, 15, 26),
             note="480p x 81 frames, B=2 (CFG pair)"),
    Workload(3, "720p_81f", 2, 16, 19320, 128, "bf16", (21, 23, 40),
             note="720p x 81 frames, B=2 (CFG pair)"),
    Workload(4, "stack_720p_121f", 1, 16, 28520, 128, "bf16", (31, 23, 40),
             kinds=(LINEAR, LINEAR, LINEAR, SOFTMAX, LINEAR, LINEAR, LINEAR, SOFTMAX),
             note="3:1 hybrid stack of 8 layers, fp32 residual stream"),
    Workload(5, "long_720p_193f", 1, 16, 45080, 128, "bf16", (49, 23, 40),
             note="720p x 193 frames"),
]

BY_NAME = {w.name: w for w in WORKLOADS}

# Duration sweep at 720p (latent grid 23 x 40 per latent frame, T = (frames-1)/4 + 1):
# the pages report that the hybrid's advantage over full softmax grows with video
# duration, up to 720p / 60 s. (frames, note) pairs; 961 and 1441 frames are 60 s at
# 16 and 24 fps.
DURATION_FRAMES: List[Tuple[int, str]] = [
    (81, "3.4 s at 24 fps"), (121, "5 s at 24 fps"), (193, "8 s at 24 fps"),
    (481, "20 s at 24 fps"), (961, "60 s at 16 fps"), (1441, "60 s at 24 fps"),
]


def latent_720p(frames: int) -> Tuple[int, int, int]:
    """Latent (T, H, W) grid of a 720p clip of ``frames`` frames."""
    return ((frames - 1) // 4 + 1, 23, 40)


def duration_workload(frames: int, B: int = 1, H: int = 16) -> Workload:
    """A 720p workload of ``frames`` frames (index 6: its own seed range)."""
    T, Hl, Wl = latent_720p(frames)
    return Workload(6, f"720p_{frames}f", B, H, T * Hl * Wl, 128, "bf16", (T, Hl, Wl),
                    note=f"720p x {frames} frames")


def seed_for(workload_index: int, layer: int, slot: str) -> int:
    return SEED_BASE + 1000 * workload_index + 10 * layer + SLOT[slot]


def randn(shape, seed: int, dtype: torch.dtype) -> torch.Tensor:
    """N(0,1) drawn in fp32 on the CPU from ``seed``, then cast (RNE) to ``dtype``."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(seed))
    t = torch.randn(tuple(shape), generator=gen, dtype=torch.float32)
    return t if dtype == torch.float32 else t.to(dtype)


def layer_inputs(w: Workload, layer: int, B: int = None, H: int = None, N: int = None,
                 dtype: torch.dtype = None):
    """(q, k, v, g) CPU tensors of shape [B, H, N, D] for ``layer`` of workload ``w``.

    B/H/N may be overridden (smaller shapes for tests) while keeping the seeds;
    ``dtype`` overrides the workload's (e.g. fp8 inputs of a bf16 workload).
    """
    B = w.B if B is None else B
    H = w.H if H is None else H
    N = w.N if N is None else N
    dt = w.torch_dtype if dtype is None else dtype
    shape = (B, H, N, w.D)
    return tuple(randn(shape, seed_for(w.index, layer, s), dt) for s in ("q", "k", "v", "g"))


def residual_x0(w: Workload, B: int = None, H: int = None, N: int = None) -> torch.Tensor:
    """fp32 residual stream x0 for the hybrid stack (always fp32)."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    N = w.N if N is None else N
    return randn((B, H, N, w.D), seed_for(w.index, 0, "x0"), torch.float32)


def attnres_inputs(w: Workload, n_blocks: int, B: int = None, H: int = None, N: int = None):
    """(x, summaries, router) for the block-attention-residual routing.

    x and the ``n_blocks`` block summaries are fp32 [B, H, N, D], N(0, 1) (a block
    summary is a sum of layer outputs of about unit size); the router W is bf16
    [D, D] with N(0, 4/D) entries, so q = x W has entries of about 2 and the
    per-token scores q . s / sqrt(D) spread over a few units.
    """
    B = w.B if B is None else B
    H = w.H if H is None else H
    N = w.N if N is None else N
    shape = (B, H, N, w.D)
    x = randn(shape, seed_for(w.index, 0, "x0"), torch.float32)
    summaries = [randn(shape, seed_for(w.index, i, "summary"), torch.float32) for i in range(n_blocks)]
    router = (randn((w.D, w.D), seed_for(w.index, 0, "router"), torch.float32) * (2.0 / w.D ** 0.5))
    return x, summaries, router.to(torch.bfloat16)


def custom(shape, seed: int, dtype: torch.dtype = torch.float32, n: int = 4):
    """``n`` independent N(0,1) tensors of ``shape`` from consecutive seeds."""
    return tuple(randn(shape, seed + i, dtype) for i in range(n))

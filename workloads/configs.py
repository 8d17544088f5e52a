"""The five synthetic workloads of the owned-partition step, as data.

Shapes follow the pages' own examples: the 7.5B-parameter / Nd = 64 example
(trishampatil "The Full Progression, in One View"; upskillscore "In
practice"), GPT-2 1.5B (trishampatil "The Real Problem") and the 60B model
scaled to 400 GPUs (anthology note, claim C4; upskillscore "In practice").
Values are i.i.d. synthetic draws; no dataset or trained weights are used.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple


def gpt2_numels(n_layer: int, d: int, vocab: int = 50257, n_ctx: int = 1024) -> List[int]:
    """GPT-2 parameter list in module order, LM head tied to the token
    embedding: wte [V,d], wpe [n_ctx,d], per layer ln_1 (w,b), attn qkv (w,b),
    attn proj (w,b), ln_2 (w,b), mlp fc (w,b), mlp proj (w,b); final ln_f."""
    out = [vocab * d, n_ctx * d]
    for _ in range(n_layer):
        out += [d, d, d * 3 * d, 3 * d, d * d, d, d, d, d * 4 * d, 4 * d, 4 * d * d, d]
    out += [d, d]
    return out


def gpt2_layers(n_layer: int) -> List[Tuple[int, int]]:
    """Tensor index ranges [first, last) of the units a Pos+g+p forward
    gathers one at a time: the embeddings (wte, wpe), each transformer block
    (its 12 tensors), the final layer norm."""
    out = [(0, 2)]
    for i in range(n_layer):
        out.append((2 + 12 * i, 14 + 12 * i))
    out.append((2 + 12 * n_layer, 4 + 12 * n_layer))
    return out


def layer_ranges(numels, layers) -> List[Tuple[int, int]]:
    """Flat element ranges [lo, hi) of tensor index ranges in a packed list."""
    offs = [0]
    for n in numels:
        offs.append(offs[-1] + n)
    return [(offs[a], offs[b]) for a, b in layers]


@dataclass(frozen=True)
class Workload:
    key: str
    title: str
    numels: Tuple[int, ...]
    nd: int
    owners: Tuple[int, ...]
    steps: int
    param_sigma: float
    grad_sigma: float
    loss_scale: float
    dist: str                      # "normal" or "student_t3"
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    stage: int = 2                 # 0 DP, 1 Pos, 2 Pos+g, 3 Pos+g+p
    # (1-based step, slice index, window element or None for S//2)
    inject: Optional[Tuple[int, int, Optional[int]]] = None
    seed: int = 0

    @property
    def psi(self) -> int:
        return sum(self.numels)


C1 = Workload(
    key="c1", title="flat Psi=1,000,003, Nd=4, every rank x 3 steps",
    numels=(1_000_003,), nd=4, owners=(0, 1, 2, 3), steps=3,
    param_sigma=0.02, grad_sigma=1e-3, loss_scale=1024.0, dist="normal",
    stage=2, seed=1)

C2 = Workload(
    key="c2", title="GPT-2-small shaped (12 x 768, vocab 50257), Nd=8, Pos, rank 3 x 10 steps",
    numels=tuple(gpt2_numels(12, 768)), nd=8, owners=(3,), steps=10,
    param_sigma=0.02, grad_sigma=1e-3, loss_scale=1024.0, dist="normal",
    stage=1, seed=2)

C3 = Workload(
    key="c3", title="GPT-2-XL shaped (48 x 1600), Nd=16, Pos+g, AdamW wd=0.01, rank 0 x 5 steps",
    numels=tuple(gpt2_numels(48, 1600)), nd=16, owners=(0,), steps=5,
    param_sigma=0.02, grad_sigma=1e-4, loss_scale=4096.0, dist="normal",
    weight_decay=0.01, stage=2, seed=3)

C4 = Workload(
    key="c4", title="flat Psi=7.5e9, Nd=64, rank 0 x 3 steps",
    numels=(7_500_000_000,), nd=64, owners=(0,), steps=3,
    param_sigma=0.02, grad_sigma=1e-4, loss_scale=8192.0, dist="normal",
    stage=2, seed=4)

C5 = Workload(
    key="c5", title="flat Psi=6e10, Nd=400, Student-t(3) grads, +inf at step 2 slice 17, rank 0 x 4 steps",
    numels=(60_000_000_000,), nd=400, owners=(0,), steps=4,
    param_sigma=0.02, grad_sigma=1e-4, loss_scale=2048.0, dist="student_t3",
    stage=2, inject=(2, 17, None), seed=5)

ALL = {w.key: w for w in (C1, C2, C3, C4, C5)}


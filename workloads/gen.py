"""Seeded synthetic inputs for the owned-partition step.

Holds none of the method's arithmetic: it only draws parameters and fp16
gradient slices with the workloads' distributions.  Both the oracle side and
the HIP side of every test consume the same arrays produced here.

Host draws (numpy PCG64) are keyed by (seed, kind, step, owner, slice, chunk)
so any window is reproducible chunk by chunk.  Device draws (torch's Philox
generator on the GPU) are used for the full-size workloads, where only
sampled elements are copied back for the oracle.
"""
from __future__ import annotations

import numpy as np

CHUNK = 1 << 22
_SALT = 0x5EED


def rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([_SALT, *[int(k) for k in key]])))


def _draw(dist: str, g: np.random.Generator, n: int) -> np.ndarray:
    if dist == "normal":
        return g.standard_normal(n)
    if dist == "student_t3":
        return g.standard_t(3, n)
    raise ValueError(dist)


def host_params(seed: int, psi: int, lo: int, hi: int, sigma: float) -> np.ndarray:
    """fp32 parameters for global flat indices [lo, hi): N(0, sigma) for
    indices < psi, exact zeros for padding indices >= psi."""
    out = np.zeros(max(hi - lo, 0), dtype=np.float32)
    if hi <= lo:
        return out
    for c in range(lo // CHUNK, (hi - 1) // CHUNK + 1):
        a, b = max(lo, c * CHUNK), min(hi, (c + 1) * CHUNK)
        vals = rng(seed, 0, c).standard_normal(CHUNK)[a - c * CHUNK:b - c * CHUNK] * sigma
        out[a - lo:b - lo] = vals.astype(np.float32)
    # padding positions hold exact zeros
    if hi > psi:
        out[max(psi, lo) - lo:] = 0.0
    return out


def host_grad_slices(seed: int, step: int, owner: int, nd: int, n: int, window_base: int,
                     psi: int, sigma: float, loss_scale: float, dist: str = "normal") -> np.ndarray:
    """fp16 slices [nd, n]: slice k is rank k's gradient for the owner's
    window at global offset window_base, drawn as fp16(x * sigma * L) with x
    from ``dist``; padding positions (global index >= psi) are zero."""
    out = np.zeros((nd, n), dtype=np.float16)
    scale = sigma * loss_scale
    for k in range(nd):
        for c in range(0, max(n, 1), CHUNK):
            b = min(n, c + CHUNK)
            if b <= c:
                break
            x = _draw(dist, rng(seed, 1, step, owner, k, c // CHUNK), b - c)
            out[k, c:b] = (x * scale).astype(np.float16)
    valid = max(0, min(n, psi - window_base))
    out[:, valid:] = 0
    return out


# ------------------------------------------------------------------ device
def device_fill_params(t, seed: int, sigma: float, valid: int):
    """Fill fp32 device tensor ``t`` (1-D) with N(0, sigma); elements at
    index >= valid are zero (padding)."""
    import torch
    g = torch.Generator(device=t.device)
    g.manual_seed(int(seed) * 1_000_003 + 17)
    t.normal_(0.0, sigma, generator=g)
    if valid < t.numel():
        t[max(valid, 0):].zero_()
    return t


def device_fill_grads(slices, seed: int, step: int, sigma: float, loss_scale: float,
                      dist: str, valid: int, chunk: int = 1 << 26):
    """Fill fp16 device tensor ``slices`` [nd, stride] row by row; columns at
    index >= valid are zero (padding).  Student-t(3) is drawn as
    z / sqrt((z1^2 + z2^2 + z3^2) / 3) from four standard normals."""
    import torch
    nd, width = slices.shape
    g = torch.Generator(device=slices.device)
    scale = float(sigma * loss_scale)
    for k in range(nd):
        g.manual_seed(((int(seed) * 1009 + int(step)) * 100_003 + k) & ((1 << 62) - 1))
        for c in range(0, width, chunk):
            b = min(width, c + chunk)
            z = torch.randn(b - c, device=slices.device, generator=g, dtype=torch.float32)
            if dist == "student_t3":
                w = torch.randn(3, b - c, device=slices.device, generator=g, dtype=torch.float32)
                z = z / torch.sqrt((w * w).sum(0) / 3.0)
            elif dist != "normal":
                raise ValueError(dist)
            slices[k, c:b] = (z * scale).to(torch.float16)
    if valid < width:
        slices[:, max(valid, 0):].zero_()
    return slices

"""Helpers for the GPU parity tests: run the HIP path through the C ABI on
host-provided inputs and compare with the oracle's results."""
from __future__ import annotations

import numpy as np

F16, F32, F64 = np.float16, np.float32, np.float64
SENTINEL = 0x7E5A  # an fp16 NaN pattern no step ever writes


def torch_mod():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("no GPU visible")
    return torch


def ord16(bits: np.ndarray) -> np.ndarray:
    """Maps fp16 bit patterns to integers whose difference counts ulps."""
    u = bits.astype(np.int64)
    return np.where(u & 0x8000, -(u & 0x7FFF), u)


def assert_state_close(gpu, orc, what, rel=1e-5):
    """Elementwise |gpu - oracle| <= rel * |oracle| (equality where the oracle
    is zero); returns the fraction of bit-identical elements."""
    a = np.asarray(gpu, dtype=F32)
    b = np.asarray(orc, dtype=F32)
    assert a.shape == b.shape, what
    same = a.view(np.uint32) == b.view(np.uint32)
    if not same.all():
        a64, b64 = a.astype(F64), b.astype(F64)
        ok = np.abs(a64 - b64) <= rel * np.abs(b64)
        ok |= same
        bad = np.flatnonzero(~ok)
        assert bad.size == 0, (f"{what}: {bad.size} elements outside rel {rel}; first {bad[:5]}: "
                               f"gpu {a[bad[:5]]} oracle {b[bad[:5]]}")
    return float(same.mean()) if same.size else 1.0


def assert_fp16_close(gpu_bits, orc_bits, what, ulps=1):
    d = np.abs(ord16(gpu_bits) - ord16(orc_bits))
    bad = np.flatnonzero(d > ulps)
    assert bad.size == 0, f"{what}: {bad.size} fp16 elements beyond {ulps} ulp; first {bad[:5]}"
    return float((d == 0).mean()) if d.size else 1.0


class GpuShardRun:
    """Owned shard on the GPU with a guarded all-gather window and slices
    embedded in wider buffers (exercises elem_off and slice_stride)."""

    def __init__(self, master0: np.ndarray, nd: int, hp: dict, guard: int = 64, elem_off: int = 16,
                 stride_pad: int = 24):
        torch = torch_mod()
        from zero_partitioned_mixed_buffer_amd import OwnedShard
        self.torch = torch
        self.n = n = master0.size
        self.nd = nd
        self.guard = guard
        self.elem_off = elem_off
        self.stride = ((elem_off + n + 7) // 8) * 8 + stride_pad
        self.shard = OwnedShard(torch.from_numpy(master0.astype(F32)).cuda(), **hp)
        self.ag = torch.full((guard + n + guard,), SENTINEL, dtype=torch.int16, device="cuda")
        self.ag = self.ag.view(torch.float16)
        self.shard.emit(self.ag, guard)
        self.slices = torch.full((nd, self.stride), 7.0, dtype=torch.float16).cuda()

    def step(self, slices: np.ndarray, loss_scale: float):
        torch = self.torch
        assert slices.shape == (self.nd, self.n)
        self.slices[:, self.elem_off:self.elem_off + self.n] = torch.from_numpy(slices).cuda()
        self.shard.step(self.slices, loss_scale, elem_off=self.elem_off, allgather=self.ag,
                        allgather_off=self.guard)
        torch.cuda.synchronize()
        ctl = self.shard.control()
        p, m, v = (x.cpu().numpy() for x in self.shard.committed(ctl))
        bits = self.ag.view(torch.int16).cpu().numpy().view(np.uint16)
        return ctl, p, m, v, bits

    def window(self, bits):
        return bits[self.guard:self.guard + self.n]

    def guards_intact(self, bits):
        g = np.concatenate([bits[:self.guard], bits[self.guard + self.n:]])
        return bool(np.all(g == SENTINEL))

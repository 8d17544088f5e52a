"""GPU parity of the Pos+g+p on-demand parameter gather against the oracle.

The windows are separate device allocations (rank r's fp16 window of S
elements, as each rank would hold it), filled with seeded values.  A
gathered range must equal the oracle's gather bit for bit, and the guard
elements around the destination must stay untouched.  Full-size cases
gather every layer of the GPT-2-small and GPT-2-XL shaped parameter lists
into one constant-size layer buffer, reused from layer to layer (the
release).
"""
import sys

import numpy as np
import pytest

import oracle
from workloads import configs, gen

from gpu_util import SENTINEL, torch_mod

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gather] {msg}", file=sys.stderr, flush=True)


def _windows(torch, nd, part, seed, psi=None):
    """nd separate fp16 device windows of `part` elements, N(0, 0.02)
    values; flat indices >= psi are zero (padding)."""
    ws = []
    for r in range(nd):
        t = torch.empty(part, dtype=torch.float32, device="cuda")
        valid = part if psi is None else max(0, min(part, psi - r * part))
        gen.device_fill_params(t, seed + r, 0.02, valid)
        ws.append(t.to(torch.float16))
        del t
    return ws


def _gather_check(torch, B, ws, ws_host, part, lo, hi, dst_off, tag):
    n = hi - lo
    guard = 64
    buf = torch.full((dst_off + n + guard,), SENTINEL, dtype=torch.int16, device="cuda")
    B.gather_params(ws, part, lo, hi, buf[dst_off:].view(torch.float16))
    torch.cuda.synchronize()
    got = buf.cpu().numpy().view(np.uint16)
    want = oracle.gather(ws_host, part, lo, hi).view(np.uint16)
    assert np.array_equal(got[dst_off:dst_off + n], want), tag
    assert np.all(got[:dst_off] == SENTINEL) and np.all(got[dst_off + n:] == SENTINEL), f"{tag} guard"


def test_gather_ranges():
    """Ranges inside one window, across several, whole, empty, single
    elements at window boundaries; 16-byte-compatible and incompatible
    source/destination offsets (vector and element-wise paths)."""
    torch = torch_mod()
    from zero_partitioned_mixed_buffer_amd import binding as B
    nd, part = 5, 20008
    ws = _windows(torch, nd, part, 77)
    wh = [w.cpu().numpy() for w in ws]
    total = nd * part
    g = np.random.default_rng(3)
    cases = [(0, total), (0, 0), (part, part), (part - 1, part + 1), (3 * part - 1, 3 * part),
             (8, 8 + 8192 * 2 + 24), (16, part - 16), (part - 8, 4 * part + 8), (1, 2 * part + 3),
             (total - 5, total), (5, 5 + 8 * 8192 + 3)]
    for _ in range(12):
        lo = int(g.integers(0, total))
        cases.append((lo, int(g.integers(lo, total + 1))))
    for lo, hi in cases:
        for dst_off in (0, 8, 3):
            _gather_check(torch, B, ws, wh, part, lo, hi, dst_off, f"[{lo}, {hi}) dst+{dst_off}")


def test_gather_spanning_more_windows_than_one_launch_holds():
    """A range over 37 small windows (16 window pieces per launch, so three
    launches), on both copy paths."""
    torch = torch_mod()
    from zero_partitioned_mixed_buffer_amd import binding as B
    nd, part = 40, 1000
    ws = _windows(torch, nd, part, 9)
    wh = [w.cpu().numpy() for w in ws]
    for lo, hi in ((5, 37005), (0, nd * part), (16 * part - 3, 33 * part + 4)):
        for dst_off in (0, 8, 3):
            _gather_check(torch, B, ws, wh, part, lo, hi, dst_off, f"[{lo}, {hi}) dst+{dst_off}")


def test_gather_unused_windows_may_be_null():
    torch = torch_mod()
    from zero_partitioned_mixed_buffer_amd import binding as B
    nd, part = 4, 4096
    ws = _windows(torch, nd, part, 5)
    wh = [w.cpu().numpy() for w in ws]
    sparse = [None, ws[1], ws[2], None]
    out = torch.empty(part + 100, dtype=torch.float16, device="cuda")
    B.gather_params(sparse, part, part + 50, 2 * part + 150, out)
    torch.cuda.synchronize()
    want = oracle.gather(wh, part, part + 50, 2 * part + 150).view(np.uint16)
    assert np.array_equal(out.cpu().numpy().view(np.uint16), want)
    with pytest.raises(B.ZeroError):
        B.gather_params(sparse, part, 0, 10, out)  # window 0 is needed


class _DeviceSlices:
    """A device window that the oracle reads by slices: each slice is copied
    to the host on demand, so windows of several GB need not be."""

    def __init__(self, t):
        self.t = t
        self.dtype = np.float16

    def __getitem__(self, sl):
        return self.t[sl].cpu().numpy()


def test_gather_past_int32_offsets():
    """Two windows of 2^31 + 4096 elements: ranges whose offsets, in the
    flat buffer and inside a window, pass the int32 range (a window edge
    at 2^31 + 4096, the end of the flat buffer near 2^32, a 64M-element
    range across the edge), on both copy paths."""
    torch = torch_mod()
    from zero_partitioned_mixed_buffer_amd import binding as B
    torch.cuda.empty_cache()
    nd, part = 2, (1 << 31) + 4096
    ws = _windows(torch, nd, part, 31)
    wh = [_DeviceSlices(w) for w in ws]
    cases = [(part - 1000, part + 3000), (2 * part - 5003, 2 * part), ((1 << 31) - 8, (1 << 31) + 8200),
             (part - (1 << 25), part + (1 << 25))]
    for lo, hi in cases:
        for dst_off in (0, 8, 3):
            say(f"[{lo}, {hi}) dst+{dst_off}")
            _gather_check(torch, B, ws, wh, part, lo, hi, dst_off, f"[{lo}, {hi}) dst+{dst_off}")
    del ws, wh
    torch.cuda.empty_cache()


@pytest.mark.parametrize("key", ["c2", "c3"])
def test_gather_every_layer_full(key):
    """Every layer of the GPT-2 shaped list, gathered from the Nd windows of
    the workload's partition into one constant-size layer buffer."""
    torch = torch_mod()
    from zero_partitioned_mixed_buffer_amd import binding as B
    w = configs.ALL[key]
    plan, _ = B.plan_partitions(list(w.numels), w.nd, 256)
    part = plan["part"]
    n_layer = (len(w.numels) - 4) // 12
    ranges = configs.layer_ranges(w.numels, configs.gpt2_layers(n_layer))
    ws = _windows(torch, w.nd, part, w.seed * 1000, psi=w.psi)
    wh = [x.cpu().numpy() for x in ws]
    biggest = max(hi - lo for lo, hi in ranges)
    buf = torch.empty(biggest, dtype=torch.float16, device="cuda")
    say(f"{key}: {len(ranges)} layers, largest {biggest} elements, windows of {part}")
    for i, (lo, hi) in enumerate(ranges):
        B.gather_params(ws, part, lo, hi, buf)
        got = buf[:hi - lo].view(torch.int16).cpu().numpy().view(np.uint16)
        want = oracle.gather(wh, part, lo, hi).view(np.uint16)
        assert np.array_equal(got, want), f"{key} layer {i} [{lo}, {hi})"
    # the padding of the last window gathers as zeros
    if plan["pad"]:
        B.gather_params(ws, part, w.psi, plan["padded"], buf)
        assert torch.count_nonzero(buf[:plan["pad"]].view(torch.int16)).item() == 0

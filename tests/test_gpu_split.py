"""GPU parity of a long window, whose fused pass the library runs as several
consecutive launches (windows of more than 2^25 elements, of more than 2^24
from 32 slices up, of more than 2^23 from 256 slices up).

The same window is stepped twice on the device: by zero_adam_step (split
into launches) and in buckets of 2^20 elements (one launch each; the
bucketed step is compared with the oracle element by element in
test_gpu_buckets).  Every element of the state and of the all-gather
window must agree bit for bit, flags and step counts exactly, the sum of
g^2 within 1e-12 of a float64 torch sum.  Sampled elements, dense around
every multiple of 1024 (where any split into 16-byte aligned launches
puts its boundaries), are also compared with the oracle: flags and t
exact, fp32 state within 1e-5 relative, fp16 window within 1 ulp.
"""
import sys

import numpy as np
import pytest

import oracle
from workloads import gen

from gpu_util import assert_fp16_close, assert_state_close, torch_mod

pytestmark = pytest.mark.gpu

N = (1 << 25) + 5003  # a ragged tail group after the last full one
ND = 3
# From 32 slices up the library splits at 2^23 elements once a window is
# longer than 2^24: this window takes three launches there and one below.
N_BIG_ND = (1 << 24) + 5003
BIG_ND = 48
# From 256 slices up it splits at 2^22 once a window is longer than 2^23.
N_HUGE_ND = (1 << 23) + 5003
HUGE_ND = 260
SPLITS = [(ND, N), (BIG_ND, N_BIG_ND)]
L = 1024.0


def say(msg):
    print(f"[split] {msg}", file=sys.stderr, flush=True)


def _sample_idx(n):
    g = np.random.default_rng(5)
    every = 1024 if n <= (1 << 26) else (1 << 20)  # the oracle's share stays at seconds
    near = (np.arange(0, n, every, dtype=np.int64)[:, None] + np.arange(-4, 4, dtype=np.int64)).ravel()
    idx = np.unique(np.concatenate([near, g.integers(0, n, 1 << 15, dtype=np.int64),
                                    np.arange(n - 16, n, dtype=np.int64)]))
    return idx[(idx >= 0) & (idx < n)]


def _sumsq(torch, slices, scale=L):
    g = slices.to(torch.float64).sum(0) * (1.0 / scale)
    return float((g * g).sum().item())


@pytest.mark.parametrize("nd,n,dynamic", [(ND, N, False), (ND, N, True), (BIG_ND, N_BIG_ND, False),
                                          (HUGE_ND, N_HUGE_ND, False)])
def test_long_window_split_launches(nd, n, dynamic):
    """With dynamic loss scaling (interval 2, from 4096) the slices carry
    the control block's scale, and the scale trajectory must match the
    oracle's exactly."""
    torch = torch_mod()
    from zero_partitioned_mixed_buffer_amd import OwnedShard
    from zero_partitioned_mixed_buffer_amd import binding as B
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    if dynamic:
        hp.update(scale_interval=2, loss_scale=4096.0)
    master = torch.empty(n, dtype=torch.float32, device="cuda")
    gen.device_fill_params(master, 123, 0.02, n)
    idx = _sample_idx(n)
    tidx = torch.from_numpy(idx).cuda()
    ref = oracle.OwnedShard(master[tidx].cpu().numpy(), **hp)
    whole = OwnedShard(master, **hp)
    buck = OwnedShard(master, **hp)
    del master
    ag_w = torch.zeros(n + 16, dtype=torch.float16, device="cuda")
    ag_b = torch.zeros(n + 16, dtype=torch.float16, device="cuda")
    whole.emit(ag_w, 8)
    buck.emit(ag_b, 8)
    # slice stride a multiple of 8 elements; the columns past n are zero
    dsl = torch.empty((nd, (n + 7) // 8 * 8), dtype=torch.float16, device="cuda")
    bucket = 1 << 20
    say(f"n={n} nd={nd}: {idx.size} sampled elements")
    for step in range(1, 4):
        scale = ref.scale if dynamic else L  # the scale the slices carry
        gen.device_fill_grads(dsl, 77, step, 1e-3, scale, "normal", n)
        if step == 2:
            dsl[1, n - 10] = float("inf")  # in the last launch of the split (sampled)
        ovf, _ = ref.step(dsl[:, tidx].cpu().numpy(), L)
        sq_want = None if ovf else _sumsq(torch, dsl, scale)
        say(f"step {step}: split whole-window step, then {-(-n // bucket)} buckets")
        whole.step(dsl, L, allgather=ag_w, allgather_off=8)
        for o in range(0, n, bucket):
            k = min(bucket, n - o)
            phase = (B.BUCKET_FIRST if o == 0 else 0) | (B.BUCKET_LAST if o + k >= n else 0)
            buck.step_bucket(dsl, o, k, phase, L, elem_off=o, allgather=ag_b, allgather_off=8)
        torch.cuda.synchronize()
        cw, cb = whole.control(), buck.control()
        tag = f"step {step}"
        assert cw["overflow"] == cb["overflow"] == int(ovf), tag
        assert cw["t"] == cb["t"] == ref.t and cw["skipped"] == cb["skipped"], tag
        if dynamic:
            assert cw["loss_scale"] == cb["loss_scale"] == ref.scale, tag
            assert cw["good_steps"] == cb["good_steps"] == ref.good_steps, tag
        for a, b in zip(whole.committed(cw), buck.committed(cb)):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), tag
        assert torch.equal(ag_w.view(torch.int16), ag_b.view(torch.int16)), tag
        if not ovf:
            assert cw["sumsq"] == pytest.approx(sq_want, rel=1e-12), tag
            assert cb["sumsq"] == pytest.approx(sq_want, rel=1e-12), tag
        p, m, v = (x[tidx].cpu().numpy() for x in whole.committed(cw))
        for got, want, nm in ((p, ref.p, "p"), (m, ref.m, "m"), (v, ref.v, "v")):
            assert_state_close(got, want, f"{tag} {nm}")
        bits = ag_w.view(torch.int16)[8 + tidx].cpu().numpy().view(np.uint16)
        assert_fp16_close(bits, ref.window().view(np.uint16), f"{tag} window")
    assert ref.flags == [0, 1, 0] and ref.t == 2
    if dynamic:
        assert ref.scales == [4096.0, 4096.0, 2048.0]


def _sumsq32(torch, slices):
    tot = 0.0
    for c in range(0, slices.shape[1], 1 << 27):
        g = (slices[:, c:c + (1 << 27)].to(torch.float64).sum(0) * (1.0 / L)).to(torch.float32).to(torch.float64)
        tot += float((g * g).sum().item())
    return tot


@pytest.mark.parametrize("nd,n", SPLITS + [(1, (1 << 31) + 5003)])
def test_long_window_clipped_split(nd, n):
    """The clipped step on a long window, its passes split into launches
    (the reduce pass by the slice count's rule, the update pass past 2^25),
    also on a window of 2^31 + 5003 elements, past the int32 range:
    sampled elements (dense around every multiple of 1024, or of 2^20 on
    windows longer than 2^26) against the
    oracle given the window's norm from a float64 torch sum of the fp32
    gradients; the sum of squares and the clip coefficient within 1e-12
    (a piece missing from the norm would move both); a skipped step leaves
    state and window bit-identical."""
    torch = torch_mod()
    from zero_partitioned_mixed_buffer_amd import OwnedShard
    torch.cuda.empty_cache()
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_grad_norm=0.5)
    master = torch.empty(n, dtype=torch.float32, device="cuda")
    gen.device_fill_params(master, 321, 0.02, n)
    idx = _sample_idx(n)
    tidx = torch.from_numpy(idx).cuda()
    ref = oracle.OwnedShard(master[tidx].cpu().numpy(), **hp)
    sh = OwnedShard(master, **hp)
    del master
    ag = torch.zeros(n + 16, dtype=torch.float16, device="cuda")
    sh.emit(ag, 8)
    dsl = torch.empty((nd, (n + 7) // 8 * 8), dtype=torch.float16, device="cuda")
    for step in range(1, 4):
        gen.device_fill_grads(dsl, 78, step, 1e-3, L, "normal", n)
        injected = step == 2
        if injected:
            dsl[min(2, nd - 1), 2] = float("-inf")  # in the first launch of the split (sampled)
        sq32 = None if injected else _sumsq32(torch, dsl)
        ovf, _ = ref.step(dsl[:, tidx].cpu().numpy(), L, window_sumsq=sq32)
        assert ovf == injected
        if ovf:
            prev = [x.clone() for x in sh.committed()]
            prev_ag = ag.clone()
        say(f"clipped step {step}")
        sh.step(dsl, L, allgather=ag, allgather_off=8)
        torch.cuda.synchronize()
        ctl = sh.control()
        tag = f"clipped step {step}"
        assert ctl["overflow"] == int(ovf) and ctl["t"] == ref.t, tag
        if ovf:
            for a, b in zip(prev, sh.committed(ctl)):
                assert torch.equal(a.view(torch.int32), b.view(torch.int32)), tag
            assert torch.equal(prev_ag.view(torch.int16), ag.view(torch.int16)), tag
            del prev, prev_ag
        else:
            assert ctl["sumsq"] == pytest.approx(sq32, rel=1e-12), tag
            assert ctl["clip_coef"] == pytest.approx(ref.coefs[-1], rel=1e-12) and ref.coefs[-1] < 0.1, tag
        p, m, v = (x[tidx].cpu().numpy() for x in sh.committed(ctl))
        for got, want, nm in ((p, ref.p, "p"), (m, ref.m, "m"), (v, ref.v, "v")):
            assert_state_close(got, want, f"{tag} {nm}")
        bits = ag.view(torch.int16)[8 + tidx].cpu().numpy().view(np.uint16)
        assert_fp16_close(bits, ref.window().view(np.uint16), f"{tag} window")
    assert ref.flags == [0, 1, 0] and ref.t == 2


N_PAST_INT32 = (1 << 31) + 5003


def _sumsq_chunked(torch, slices, n, scale):
    tot = 0.0
    for c in range(0, n, 1 << 27):
        g = slices[:, c:min(n, c + (1 << 27))].to(torch.float64).sum(0) * (1.0 / scale)
        tot += float((g * g).sum().item())
    return tot


def test_window_past_int32_elements():
    """A window of 2^31 + 5003 elements (Nd = 1; about 125 GB of device
    memory for two shards), so element indices and offsets pass the int32
    range.  Two steps, the second skipped by an inf in the last element
    group: the commit then re-emits the whole window from the committed
    master in one launch.  The split fused step and a bucketed twin
    (buckets of 2^26 elements, so its boundaries differ from the split's)
    agree bit for bit over the whole window; sampled elements (around every
    multiple of 2^28, around 2^31 and the tail) match the oracle."""
    torch = torch_mod()
    from zero_partitioned_mixed_buffer_amd import OwnedShard
    from zero_partitioned_mixed_buffer_amd import binding as B
    torch.cuda.empty_cache()
    n, nd = N_PAST_INT32, 1
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    master = torch.empty(n, dtype=torch.float32, device="cuda")
    gen.device_fill_params(master, 124, 0.02, n)
    g = np.random.default_rng(9)
    near = (np.arange(0, n, 1 << 28, dtype=np.int64)[:, None] + np.arange(-8, 8, dtype=np.int64)).ravel()
    idx = np.unique(np.concatenate([near, (1 << 31) + np.arange(-16, 16, dtype=np.int64),
                                    g.integers(0, n, 1 << 14, dtype=np.int64), np.arange(n - 16, n, dtype=np.int64)]))
    idx = idx[(idx >= 0) & (idx < n)]
    tidx = torch.from_numpy(idx).cuda()
    ref = oracle.OwnedShard(master[tidx].cpu().numpy(), **hp)
    whole = OwnedShard(master, **hp)
    buck = OwnedShard(master, **hp)
    del master
    ag_w = torch.zeros(n + 16, dtype=torch.float16, device="cuda")
    ag_b = torch.zeros(n + 16, dtype=torch.float16, device="cuda")
    whole.emit(ag_w, 8)
    buck.emit(ag_b, 8)
    dsl = torch.empty((nd, (n + 7) // 8 * 8), dtype=torch.float16, device="cuda")
    bucket = 1 << 26
    say(f"n={n} nd={nd}: {idx.size} sampled elements")
    for step in range(1, 3):
        gen.device_fill_grads(dsl, 79, step, 1e-3, L, "normal", n)
        if step == 2:
            dsl[0, n - 10] = float("inf")
        ovf, _ = ref.step(dsl[:, tidx].cpu().numpy(), L)
        sq_want = None if ovf else _sumsq_chunked(torch, dsl, n, L)
        say(f"step {step}: split whole-window step, then {-(-n // bucket)} buckets")
        whole.step(dsl, L, allgather=ag_w, allgather_off=8)
        for o in range(0, n, bucket):
            k = min(bucket, n - o)
            phase = (B.BUCKET_FIRST if o == 0 else 0) | (B.BUCKET_LAST if o + k >= n else 0)
            buck.step_bucket(dsl, o, k, phase, L, elem_off=o, allgather=ag_b, allgather_off=8)
        torch.cuda.synchronize()
        cw, cb = whole.control(), buck.control()
        tag = f"step {step}"
        assert cw["overflow"] == cb["overflow"] == int(ovf), tag
        assert cw["t"] == cb["t"] == ref.t and cw["skipped"] == cb["skipped"], tag
        for a, b in zip(whole.committed(cw), buck.committed(cb)):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), tag
        assert torch.equal(ag_w.view(torch.int16), ag_b.view(torch.int16)), tag
        if not ovf:
            assert cw["sumsq"] == pytest.approx(sq_want, rel=1e-12), tag
            assert cb["sumsq"] == pytest.approx(sq_want, rel=1e-12), tag
        p, m, v = (x[tidx].cpu().numpy() for x in whole.committed(cw))
        for got, want, nm in ((p, ref.p, "p"), (m, ref.m, "m"), (v, ref.v, "v")):
            assert_state_close(got, want, f"{tag} {nm}")
        bits = ag_w.view(torch.int16)[8 + tidx].cpu().numpy().view(np.uint16)
        assert_fp16_close(bits, ref.window().view(np.uint16), f"{tag} window")
    assert ref.flags == [0, 1] and ref.t == 1
    del whole, buck, ag_w, ag_b, dsl
    torch.cuda.empty_cache()

"""GPU parity of the bucketed step (constant-size fused buffers) against the
oracle.

Each bucket's fp16 slices are copied into one constant-size receive buffer
(the simulated arrival of a reduce-scatter bucket), and the bucket is
stepped from it.  A bucketed step computes what the whole-window step
computes, so the oracle is the same OwnedShard.step; the bar is the fused
step's: flags, t and the scale trajectory bit-exact, fp32 state within
1e-5 relative per element, fp16 window within 1 ulp, sum of g^2 within
1e-12 relative.  The state must also be bit-identical to the fused GPU
step's (the per-element arithmetic is the same code).
"""
import sys

import numpy as np
import pytest

import oracle
from workloads import configs, gen

from gpu_util import F32, SENTINEL, GpuShardRun, assert_fp16_close, assert_state_close, torch_mod

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)


def say(msg):
    print(f"[buckets] {msg}", file=sys.stderr, flush=True)


def bucket_list(n, b, order, seed=0):
    """(win_off, len) of the buckets of a window of n elements, bucket size
    b (a multiple of 8), in the given arrival order."""
    bl = [(o, min(b, n - o)) for o in range(0, n, b)]
    if order == "reversed":
        bl = bl[::-1]
    elif order == "shuffled":
        perm = np.random.default_rng(seed + n).permutation(len(bl))
        bl = [bl[i] for i in perm]
    return bl


class BucketRun:
    """Owned shard on the GPU stepped bucket by bucket from one
    constant-size receive buffer, with a guarded all-gather window."""

    def __init__(self, master0, nd, hp, bucket, guard=64, recv_off=8):
        torch = torch_mod()
        from zero_partitioned_mixed_buffer_amd import OwnedShard
        self.torch = torch
        self.n = master0.size
        self.nd, self.bucket, self.guard, self.recv_off = nd, bucket, guard, recv_off
        self.shard = OwnedShard(torch.from_numpy(master0.astype(F32)).cuda(), **hp)
        self.ag = torch.full((guard + self.n + guard,), SENTINEL, dtype=torch.int16, device="cuda")
        self.ag = self.ag.view(torch.float16)
        self.shard.emit(self.ag, guard)
        # constant-size receive buffer [nd, recv_off + bucket + pad]
        self.recv = torch.full((nd, recv_off + bucket + 16), 7.0, dtype=torch.float16, device="cuda")

    def step(self, slices, loss_scale, order="forward", drop=None):
        """One step over all buckets (bucket index ``drop`` of the arrival
        order is left out, which the library must reject at commit)."""
        from zero_partitioned_mixed_buffer_amd import binding as B
        torch = self.torch
        dsl = torch.from_numpy(np.ascontiguousarray(slices)).cuda()
        bl = bucket_list(self.n, self.bucket, order, seed=self.nd)
        for i, (o, k) in enumerate(bl):
            phase = (B.BUCKET_FIRST if i == 0 else 0) | (B.BUCKET_LAST if i == len(bl) - 1 else 0)
            if i == drop:
                continue
            self.recv[:, self.recv_off:self.recv_off + k] = dsl[:, o:o + k]
            self.shard.step_bucket(self.recv, o, k, phase, loss_scale, elem_off=self.recv_off,
                                   allgather=self.ag, allgather_off=self.guard)
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


def _check(run, ref, got, sq, tag):
    ctl, p, m, v, bits = got
    assert ctl["overflow"] == ref.flags[-1] and ctl["t"] == ref.t, tag
    for a, b, nm in ((p, ref.p, "p"), (m, ref.m, "m"), (v, ref.v, "v")):
        assert_state_close(a, b, f"{tag} {nm}")
    assert_fp16_close(run.window(bits), ref.window().view(np.uint16), f"{tag} window")
    assert run.guards_intact(bits), tag
    if not ctl["overflow"]:
        assert ctl["sumsq"] == pytest.approx(sq, rel=1e-12, abs=1e-300), tag


@pytest.mark.parametrize("n,nd,bucket,order", [
    (50003, 4, 8192, "forward"),        # ragged last bucket and tail group
    (50003, 8, 4096, "reversed"),
    (65536 + 12, 16, 16384, "shuffled"),
    (20011, 3, 20016, "forward"),       # one bucket (FIRST | LAST)
    (9001, 1, 512, "shuffled"),         # 18 buckets, Nd = 1
    (40000, 20, 8000, "forward"),       # Nd > 16: the chunked sum
    (300001, 48, 65536, "shuffled"),    # Nd >= 32: 8-group visits cut by bucket edges
    (200003, 49, 40000, "forward"),     # odd Nd: a one-slice last chunk
    (600003, 64, 131072, "reversed"),
])
def test_bucketed_matches_oracle(n, nd, bucket, order):
    g = np.random.default_rng(n + nd)
    master0 = (g.standard_normal(n) * 0.02).astype(F32)
    ref = oracle.OwnedShard(master0, **HP)
    run = BucketRun(master0, nd, HP, bucket)
    for step in range(1, 5):
        sl = gen.host_grad_slices(n + nd, step, 0, nd, n, 0, n, 1e-3, 1024.0)
        if step == 3:  # an inf in a middle bucket skips the whole step
            sl[nd - 1, min(n - 1, bucket + 5)] = np.inf
        ovf, sq = ref.step(sl, 1024.0)
        got = run.step(sl, 1024.0, order)
        _check(run, ref, got, sq, f"n={n} nd={nd} B={bucket} {order} step={step}")
    assert ref.flags == [0, 0, 1, 0]


def test_bucketed_bit_identical_to_fused():
    """Same inputs through the fused whole-window step and the bucketed step:
    state and window bit-identical, sum of g^2 equal to 1e-12."""
    n, nd = 70001, 8
    g = np.random.default_rng(5)
    master0 = (g.standard_normal(n) * 0.02).astype(F32)
    fused = GpuShardRun(master0, nd, HP)
    buck = BucketRun(master0, nd, HP, 8192)
    for step in range(1, 4):
        sl = gen.host_grad_slices(5, step, 0, nd, n, 0, n, 1e-3, 1024.0)
        cf, pf, mf, vf, bf = fused.step(sl, 1024.0)
        cb, pb, mb, vb, bb = buck.step(sl, 1024.0, "shuffled")
        for a, b in ((pf, pb), (mf, mb), (vf, vb)):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), step
        assert np.array_equal(fused.window(bf), buck.window(bb)), step
        assert cb["sumsq"] == pytest.approx(cf["sumsq"], rel=1e-12) and cb["t"] == cf["t"] == step


def test_missing_bucket_skips_the_step():
    """A step whose buckets do not cover the window is skipped with
    overflow = 2: state bit-identical, t unchanged, window restored, the
    dynamic loss scale untouched; the next complete step commits."""
    n, nd, bucket = 30000, 5, 4096
    hp = dict(HP, scale_interval=2, loss_scale=1024.0)
    g = np.random.default_rng(11)
    master0 = (g.standard_normal(n) * 0.02).astype(F32)
    ref = oracle.OwnedShard(master0, **hp)
    run = BucketRun(master0, nd, hp, bucket)
    sl = gen.host_grad_slices(11, 1, 0, nd, n, 0, n, 1e-3, 1024.0)
    ovf, sq = ref.step(sl, 1024.0)
    got1 = run.step(sl, 1024.0)
    _check(run, ref, got1, sq, "step 1")
    sl2 = gen.host_grad_slices(11, 2, 0, nd, n, 0, n, 1e-3, 1024.0)
    ctl, p, m, v, bits = run.step(sl2, 1024.0, "forward", drop=2)
    assert ctl["overflow"] == 2 and ctl["t"] == 1 and ctl["skipped"] == 1
    assert ctl["loss_scale"] == got1[0]["loss_scale"] and ctl["good_steps"] == got1[0]["good_steps"]
    for a, b in ((got1[1], p), (got1[2], m), (got1[3], v)):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(got1[4], bits)
    # the same gradients, now complete: the oracle takes them as its step 2
    ovf, sq = ref.step(sl2, 1024.0)
    _check(run, ref, run.step(sl2, 1024.0, "reversed"), sq, "step 2 complete")
    assert ref.t == 2


def test_bucketed_dynamic_scaling():
    n, nd, bucket = 24000, 6, 8000
    hp = dict(HP, scale_interval=2, loss_scale=4096.0)
    g = np.random.default_rng(21)
    master0 = (g.standard_normal(n) * 0.02).astype(F32)
    ref = oracle.OwnedShard(master0, **hp)
    run = BucketRun(master0, nd, hp, bucket)
    for step in range(1, 8):
        sl = gen.host_grad_slices(21, step, 0, nd, n, 0, n, 1e-3, ref.scale)
        if step in (2, 5):
            sl[1, 17000 + step] = np.nan
        ovf, sq = ref.step(sl, 1.0)
        got = run.step(sl, 1.0, "shuffled")
        _check(run, ref, got, sq, f"step {step}")
        assert got[0]["loss_scale"] == ref.scale and got[0]["good_steps"] == ref.good_steps
    assert ref.flags == [0, 1, 0, 0, 1, 0, 0]


def test_c2_bucketed_full():
    """GPT-2-small shaped list, Nd = 8, rank 3: 3 steps ingested in
    constant-size buckets of 2^20 elements (the benchmark's bucketed
    configuration), compared element by element with the oracle."""
    torch = torch_mod()
    from zero_partitioned_mixed_buffer_amd import OwnedShard
    from zero_partitioned_mixed_buffer_amd import binding as B
    w = configs.C2
    owner, bucket = 3, 1 << 20
    plan, _ = B.plan_partitions(list(w.numels), w.nd, 256)
    S = plan["part"]
    valid = max(0, min(S, w.psi - owner * S))
    master = torch.empty(S, dtype=torch.float32, device="cuda")
    gen.device_fill_params(master, w.seed + owner, w.param_sigma, valid)
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay)
    ref = oracle.OwnedShard(master.cpu().numpy(), **hp)
    sh = OwnedShard(master, **hp)
    ag = torch.zeros(S, dtype=torch.float16, device="cuda")
    dsl = torch.empty((w.nd, S), dtype=torch.float16, device="cuda")
    recv = torch.empty((w.nd, bucket), dtype=torch.float16, device="cuda")
    for step in range(1, 4):
        say(f"c2 bucketed step {step}")
        gen.device_fill_grads(dsl, w.seed, step, w.grad_sigma, w.loss_scale, w.dist, valid)
        ovf, sq = ref.step(dsl.cpu().numpy(), w.loss_scale)
        bl = bucket_list(S, bucket, "forward")
        for i, (o, k) in enumerate(bl):
            phase = (B.BUCKET_FIRST if i == 0 else 0) | (B.BUCKET_LAST if i == len(bl) - 1 else 0)
            recv[:, :k] = dsl[:, o:o + k]
            sh.step_bucket(recv, o, k, phase, w.loss_scale, allgather=ag)
        torch.cuda.synchronize()
        ctl = sh.control()
        assert ctl["overflow"] == int(ovf) == 0 and ctl["t"] == ref.t == step
        assert ctl["sumsq"] == pytest.approx(sq, rel=1e-12)
        p, m, v = (x.cpu().numpy() for x in sh.committed(ctl))
        for got, want, nm in ((p, ref.p, "p"), (m, ref.m, "m"), (v, ref.v, "v")):
            assert_state_close(got, want, f"c2 bucketed step {step} {nm}")
    bits = ag.view(torch.int16).cpu().numpy().view(np.uint16)
    assert_fp16_close(bits, ref.window().view(np.uint16), "c2 bucketed window")

"""GPU parity of the calls that take several pieces at once: several
arrived buckets in one zero_adam_step_buckets call, and several layers in
one zero_gather_layers call.

Buckets: each bucket sits in its own receive buffer (constant-size,
several at once, as arrivals queue up); the step's buckets arrive in a
seeded order and are passed in groups.  Against the same step taken one
bucket per call: state and all-gather window bit for bit, flags, t and
coverage verdicts exact; against the oracle on the whole window: fp32 state
within 1e-5 relative per element, fp16 within 1 ulp, sum of g^2 within
1e-12.  Groups are long enough to fill several launches (16 runs per
launch), a bucket longer than two launch lengths is cut inside its call,
and one-bucket calls are mixed into a step.  Gathers: random layer ranges
(empty ones, ranges across many windows, more than 16 pieces per call)
against the oracle's gather, destinations guarded.
"""
import numpy as np
import pytest

import oracle
from workloads import gen

from gpu_util import F16, F32, SENTINEL, assert_fp16_close, assert_state_close, torch_mod

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _shard(torch, master0, hp, guard=64):
    from zero_partitioned_mixed_buffer_amd import OwnedShard
    sh = OwnedShard(torch.from_numpy(master0.astype(F32)).cuda(), **hp)
    ag = torch.full((guard + master0.size + guard,), SENTINEL, dtype=torch.int16, device="cuda")
    sh.emit(ag.view(torch.float16), guard)
    return sh, ag


def _buckets(n, b, seed):
    """Buckets of b elements (the last one ragged), or for b = 0 irregular
    ones: random multiples of 8 from 8 to 3000 elements, and the window's
    last 3 elements alone (a bucket with no full 4-element group); in a
    seeded arrival order."""
    g = np.random.default_rng(seed)
    if b > 0:
        bl = [(o, min(b, n - o)) for o in range(0, n, b)]
    else:
        bl, o = [], 0
        while o < n - 3:
            k = min(int(g.integers(1, 376)) * 8, n - 3 - o)
            bl.append((o, k))
            o += k
        bl.append((o, n - o))
    perm = g.permutation(len(bl))
    return [bl[i] for i in perm]


@pytest.mark.parametrize("n,nd,bucket,group", [
    (50003, 4, 2048, 5),         # 25 buckets in groups of 5, ragged last bucket
    (200003, 8, 4096, 40),       # 49 buckets: one call of 40 runs (3 launches), then one of 9
    (300001, 20, 8192, 7),       # Nd > 16: the chunked sum, visits cut by bucket edges
    (600003, 48, 65536, 3),      # Nd >= 32: 8-group visits
    (30011, 1, 512, 59),         # Nd = 1, 59 buckets in one call
    (300003, 8, 0, 16),          # irregular buckets, 16 runs per launch: a lane's step crosses several runs
    (100003, 16, 0, 33),         # the same at Nd = 16, calls of 33 buckets (three launches each)
    (2**23 + 2**21 + 12347, 32, 2**20, 16),  # Nd = 32, launches of 8 and 3 buckets: 8-group visits across buckets
])
def test_bucket_lists_match_single_buckets_and_oracle(n, nd, bucket, group):
    torch = torch_mod()
    from zero_partitioned_mixed_buffer_amd import binding as B
    g = np.random.default_rng(n + nd)
    master0 = (g.standard_normal(n) * 0.02).astype(F32)
    ref = oracle.OwnedShard(master0, **HP)
    one, ag1 = _shard(torch, master0, HP)
    many, agm = _shard(torch, master0, HP)
    bl = _buckets(n, bucket, nd)
    recv_off = 8
    # one receive buffer per bucket (the arrivals queue up); columns past
    # each bucket's own width stay 7.0
    width = max(k for _, k in bl)
    # receive buffers of four widths, so the buckets of one launch have different row strides
    recv = [torch.full((nd, recv_off + width + 16 + 8 * (i % 4)), 7.0, dtype=torch.float16, device="cuda")
            for i in range(len(bl))]
    for step in range(1, 5):
        sl = gen.host_grad_slices(n + nd, step, 0, nd, n, 0, n, 1e-3, 1024.0)
        if step == 3:  # an inf in one bucket skips the whole step
            o_inf, k_inf = bl[len(bl) // 2]
            sl[nd - 1, o_inf + min(3, k_inf - 1)] = np.inf
        ovf, sq = ref.step(sl, 1024.0)
        dsl = torch.from_numpy(sl).cuda()
        for r, (o, k) in zip(recv, bl):
            r[:, recv_off:recv_off + k] = dsl[:, o:o + k]
        # one bucket per call
        for i, ((o, k), r) in enumerate(zip(bl, recv)):
            phase = (B.BUCKET_FIRST if i == 0 else 0) | (B.BUCKET_LAST if i == len(bl) - 1 else 0)
            one.step_bucket(r, o, k, phase, 1024.0, elem_off=recv_off, allgather=ag1.view(torch.float16),
                            allgather_off=64)
        # groups of `group` buckets per call; the second group goes one
        # bucket per call, to mix both kinds in one step
        calls = [list(range(i, min(i + group, len(bl)))) for i in range(0, len(bl), group)]
        for c, idx in enumerate(calls):
            phase = (B.BUCKET_FIRST if c == 0 else 0) | (B.BUCKET_LAST if c == len(calls) - 1 else 0)
            if c == 1 and len(calls) > 2:  # a middle group: phase 0 for each of its one-bucket calls
                for i in idx:
                    many.step_bucket(recv[i], bl[i][0], bl[i][1], 0, 1024.0, elem_off=recv_off,
                                     allgather=agm.view(torch.float16), allgather_off=64)
                continue
            items = [(B.grad_src(recv[i], recv[i].shape[1], recv_off, bl[i][1], nd, 1024.0), bl[i][0])
                     for i in idx]
            B.adam_step_buckets(items, many.state, many.hp, n, agm.view(torch.float16), 64, phase,
                                many.workspace)
        torch.cuda.synchronize()
        c1, cm = one.control(), many.control()
        tag = f"n={n} nd={nd} step={step}"
        assert cm["overflow"] == c1["overflow"] == int(ovf) and cm["t"] == c1["t"] == ref.t, tag
        for a, b in zip(one.committed(c1), many.committed(cm)):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), tag
        assert torch.equal(ag1, agm), tag
        p, m, v = (x.cpu().numpy() for x in many.committed(cm))
        for got, want, nm in ((p, ref.p, "p"), (m, ref.m, "m"), (v, ref.v, "v")):
            assert_state_close(got, want, f"{tag} {nm}")
        bits = agm.cpu().numpy().view(np.uint16)
        assert_fp16_close(bits[64:64 + n], ref.window().view(np.uint16), f"{tag} window")
        assert np.all(bits[:64] == SENTINEL) and np.all(bits[64 + n:] == SENTINEL)
        if not ovf:
            assert cm["sumsq"] == pytest.approx(sq, rel=1e-12), tag
    assert ref.flags == [0, 0, 1, 0]


def test_bucket_list_long_bucket_and_missing_bucket():
    """A bucket longer than two launch lengths (2^24 below Nd = 32) is cut
    inside its call; a step whose calls miss a bucket is skipped with flag 2
    and leaves state and window as they were."""
    torch = torch_mod()
    from zero_partitioned_mixed_buffer_amd import binding as B
    nd, n = 2, (1 << 25) + (1 << 20) + 5003
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    master = (torch.randn(n, device="cuda", generator=g) * 0.02).float()
    from zero_partitioned_mixed_buffer_amd import OwnedShard
    a = OwnedShard(master, **HP)
    b = OwnedShard(master, **HP)
    aga = torch.zeros(n, dtype=torch.float16, device="cuda")
    agb = torch.zeros(n, dtype=torch.float16, device="cuda")
    a.emit(aga)
    b.emit(agb)
    stride = (n + 7) // 8 * 8
    dsl = torch.empty((nd, stride), dtype=torch.float16, device="cuda")
    gen.device_fill_grads(dsl, 9, 1, 1e-3, 1024.0, "normal", n)
    # a: the whole window as one step; b: a long bucket and a short one in one call
    a.step(dsl, 1024.0, allgather=aga)
    cut = 1 << 20
    items = [(B.grad_src(dsl, stride, cut, n - cut, nd, 1024.0), cut), (B.grad_src(dsl, stride, 0, cut, nd, 1024.0), 0)]
    B.adam_step_buckets(items, b.state, b.hp, n, agb, 0, B.BUCKET_FIRST | B.BUCKET_LAST, b.workspace)
    torch.cuda.synchronize()
    ca, cb = a.control(), b.control()
    assert ca["t"] == cb["t"] == 1 and ca["overflow"] == cb["overflow"] == 0
    for x, y in zip(a.committed(ca), b.committed(cb)):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
    assert torch.equal(aga.view(torch.int16), agb.view(torch.int16))
    assert cb["sumsq"] == pytest.approx(ca["sumsq"], rel=1e-12)
    before = [x.clone() for x in b.committed(cb)] + [agb.clone()]
    # the second step covers all but the first bucket: skipped, flag 2
    B.adam_step_buckets(items[:1], b.state, b.hp, n, agb, 0, B.BUCKET_FIRST | B.BUCKET_LAST, b.workspace)
    torch.cuda.synchronize()
    cb = b.control()
    assert cb["overflow"] == 2 and cb["t"] == 1 and cb["skipped"] == 1
    after = list(b.committed(cb)) + [agb]
    for x, y in zip(before, after):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("nd", [24, 40])
def test_bucket_list_big_and_tiny_runs(nd):
    """Four buckets of 2^19 elements, a 3-element bucket (no full group, so
    no visit) and 40 tiny ones of 8-3000 elements, in one call: the first
    launch holds 16 runs, the big ones among them, and at Nd = 40 takes the
    8-group visits (2^21 elements and more), at Nd = 24 the 4-group ones.
    Bit-identical to the one-window step over two steps."""
    torch = torch_mod()
    from zero_partitioned_mixed_buffer_amd import binding as B
    from zero_partitioned_mixed_buffer_amd import OwnedShard
    big = 1 << 19
    g = np.random.default_rng(nd)
    tiny, o = [], 4 * big
    while len(tiny) < 40:
        k = int(g.integers(1, 376)) * 8
        tiny.append((o, k))
        o += k
    n = o + 3
    buckets = [(i * big, big) for i in range(4)] + [(n - 3, 3)] + tiny
    master = torch.from_numpy((g.standard_normal(n) * 0.02).astype(F32)).cuda()
    a = OwnedShard(master, **HP)
    b = OwnedShard(master, **HP)
    aga = torch.zeros(n, dtype=torch.float16, device="cuda")
    agb = torch.zeros(n, dtype=torch.float16, device="cuda")
    a.emit(aga)
    b.emit(agb)
    stride = (n + 7) // 8 * 8
    dsl = torch.empty((nd, stride), dtype=torch.float16, device="cuda")
    for step in (1, 2):
        gen.device_fill_grads(dsl, 40 + nd, step, 1e-3, 1024.0, "normal", n)
        a.step(dsl, 1024.0, allgather=aga)
        items = [(B.grad_src(dsl, stride, o, k, nd, 1024.0), o) for o, k in buckets]
        B.adam_step_buckets(items, b.state, b.hp, n, agb, 0, B.BUCKET_FIRST | B.BUCKET_LAST, b.workspace)
        torch.cuda.synchronize()
        ca, cb = a.control(), b.control()
        tag = f"nd={nd} step={step}"
        assert ca["t"] == cb["t"] == step and ca["overflow"] == cb["overflow"] == 0, tag
        for x, y in zip(a.committed(ca), b.committed(cb)):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32)), tag
        assert torch.equal(aga.view(torch.int16), agb.view(torch.int16)), tag
        assert cb["sumsq"] == pytest.approx(ca["sumsq"], rel=1e-12), tag


@pytest.mark.parametrize("nd,part,nranges,seed", [(4, 1000, 7, 1), (16, 4096, 40, 2), (3, 64, 30, 3)])
def test_gather_layers_matches_oracle(nd, part, nranges, seed):
    torch = torch_mod()
    from zero_partitioned_mixed_buffer_amd import binding as B
    g = np.random.default_rng(seed)
    wins_h = [(g.standard_normal(part) * 0.02).astype(F16) for _ in range(nd)]
    wins = [torch.from_numpy(w).cuda() for w in wins_h]
    total = nd * part
    ranges = []
    for q in range(nranges):
        if q % 9 == 4:
            lo = int(g.integers(0, total + 1))
            ranges.append((lo, lo))  # empty
            continue
        lo = int(g.integers(0, total))
        hi = int(g.integers(lo, min(total, lo + 3 * part) + 1))
        ranges.append((lo, hi))
    ranges.append((0, total))  # every window: nd pieces in one range
    dsts = [torch.full((hi - lo + 16,), SENTINEL, dtype=torch.int16, device="cuda") for lo, hi in ranges]
    B.gather_layers(wins, part, ranges, [d[8:8 + (hi - lo)] for d, (lo, hi) in zip(dsts, ranges)])
    torch.cuda.synchronize()
    for d, (lo, hi) in zip(dsts, ranges):
        got = d.cpu().numpy().view(np.uint16)
        want = oracle.gather(wins_h, part, lo, hi).view(np.uint16)
        assert np.array_equal(got[8:8 + (hi - lo)], want), (lo, hi)
        assert np.all(got[:8] == SENTINEL) and np.all(got[8 + (hi - lo):] == SENTINEL)

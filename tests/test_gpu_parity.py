"""GPU parity of the HIP path (through the C ABI) against the oracle.

Bar: overflow flags and the committed step count bit-exact; fp32 master,
momentum and variance elementwise within relative 1e-5 of the oracle
(equality where the oracle is 0); the fp16 all-gather window within 1 ulp;
sum of g^2 within relative 1e-12; the buffer outside the window untouched.
"""
import numpy as np
import pytest

import oracle
from workloads import gen

from gpu_util import F16, F32, GpuShardRun, assert_fp16_close, assert_state_close, torch_mod

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)


def _compare_step(run, sh, ctl, p, m, v, bits, ovf, sq, t, tag):
    assert ctl["overflow"] == int(ovf), tag
    assert ctl["t"] == sh.t == t, tag
    stats = [assert_state_close(p, sh.p, f"{tag} master"),
             assert_state_close(m, sh.m, f"{tag} exp_avg"),
             assert_state_close(v, sh.v, f"{tag} exp_avg_sq"),
             assert_fp16_close(run.window(bits), sh.window().view(np.uint16), f"{tag} fp16 window")]
    assert run.guards_intact(bits), f"{tag}: all-gather buffer written outside the window"
    if not ovf:
        assert ctl["sumsq"] == pytest.approx(sq, rel=1e-12, abs=1e-300), tag
    return stats


def _run_case(n, nd, steps, seed, hp=HP, L=1024.0, sigma=1e-3, dist="normal", mutate=None):
    g = np.random.default_rng(seed)
    master0 = (g.standard_normal(n) * 0.02).astype(F32)
    sh = oracle.OwnedShard(master0, **hp)
    run = GpuShardRun(master0, nd, hp)
    stats = []
    for step in range(1, steps + 1):
        sl = gen.host_grad_slices(seed, step, 0, nd, n, 0, n, sigma, L, dist)
        if mutate is not None:
            sl = mutate(step, sl)
        ovf, sq = sh.step(sl, L)
        ctl, p, m, v, bits = run.step(sl, L)
        stats.append(_compare_step(run, sh, ctl, p, m, v, bits, ovf, sq, sh.t, f"n={n} nd={nd} step={step}"))
    return sh, run, stats


@pytest.mark.parametrize("n", [0, 8, 256, 2048 * 3 + 256, 5003, 65536 + 7])
@pytest.mark.parametrize("nd", [1, 2, 3, 17])
def test_fused_step_small(n, nd):
    _, _, stats = _run_case(n, nd, steps=3, seed=100 + n + nd)
    # the fixed float64 operation sequence is expected to agree bit for bit
    assert min(s[0] for s in stats) >= 0.999


@pytest.mark.parametrize("nd", list(range(1, 18)))
def test_fused_step_every_nd_many_groups_per_lane(nd):
    """Every slice count of the compile-time paths (one and two groups
    ahead, and the chunked sum past 16), on a window where each lane owns 6
    or 7 element groups (the prefetch rotations run several full cycles)
    and the last group is ragged."""
    n = 4 * 65536 * 6 + 4 * 1000 + 3
    _run_case(n, nd, steps=2, seed=300 + nd)


# Windows for the chunked sum past 16 slices, where one wave's visit covers 4
# (Nd < 32) or 8 (Nd >= 32) consecutive 256-element groups, so one pass of
# the 1024 waves covers 2^20 or 2^21 elements.  Each window runs past one
# full pass (or stops short of it), ends in a partial visit and a ragged
# group, and the slice counts take both chunk loops (Nd a multiple of the
# two-slice chunk, or one slice left over) on both sides of Nd = 32.
CHUNKED_CASES = [(17, 2**20 + 3 * 256 + 5), (18, 2**20 + 3 * 256 + 5), (31, 2**20 + 3 * 256 + 5),
                 (32, 2**21 + 2053), (47, 300001), (48, 2**21 + 2053), (64, 2**21 + 2053), (99, 600003)]


@pytest.mark.parametrize("nd,n", CHUNKED_CASES)
def test_fused_step_chunked_visits(nd, n):
    _run_case(n, nd, steps=2, seed=500 + nd)


# Windows one full pass and a fraction of another long, in visits of the
# launch's size: at most a quarter of a pass left (Nd >= 32 takes it in
# quarter visits), at most half (half visits), more than half (no split),
# for both visit sizes.
TAIL_SPLIT_CASES = [(56, 1224 * 2048 - 145), (40, 1424 * 2048 - 397), (33, 1900 * 2048 - 29),
                    (20, 1324 * 1024 - 41), (25, 1724 * 1024 - 17)]


@pytest.mark.parametrize("nd,n", TAIL_SPLIT_CASES)
def test_fused_step_partial_last_pass(nd, n):
    _run_case(n, nd, steps=2, seed=700 + nd)


@pytest.mark.parametrize("nd", [4, 8, 64])
def test_fused_step_adamw_many_steps(nd):
    hp = dict(HP, weight_decay=0.01)
    _, _, stats = _run_case(20000, nd, steps=20, seed=7 + nd, hp=hp, L=4096.0, sigma=1e-4)
    assert min(s[0] for s in stats) >= 0.999


def test_fused_step_student_t():
    _run_case(30000, 20, steps=4, seed=31, L=2048.0, sigma=1e-4, dist="student_t3")


def _edge_mutate(step, sl):
    g = np.random.default_rng(step)
    pool = np.array([0.0, -0.0, 65504.0, -65504.0, 2.0**-24, -(2.0**-24), 2.0**-14, -(2.0**-14),
                     6.1e-5, 1.0], dtype=F16)
    sl = sl.copy()
    pick = g.random(sl.shape) < 0.2
    sl[pick] = pool[g.integers(0, len(pool), int(pick.sum()))]
    sl[:, :4] = np.array([0.0, -0.0, 2.0**-24, -65504.0], dtype=F16)
    sl[:, -3:] = np.array([-0.0, 65504.0, 2.0**-24], dtype=F16)
    return sl


@pytest.mark.parametrize("nd", [5, 24, 64])
def test_fused_step_edge_values(nd):
    """Signed zeros, fp16 subnormals and +-65504 at the first, last and
    random elements; all-zero (padding-like) elements stay zero.  Nd 24 and
    64 take the chunked sum (its first chunk starts from slice 0, so an
    all -0 column sums to -0 there too)."""
    _run_case(4099, nd, steps=4, seed=5, mutate=_edge_mutate, L=1.0)


@pytest.mark.parametrize("nd", [6, 24, 64])
@pytest.mark.parametrize("where", ["first", "middle", "last"])
@pytest.mark.parametrize("bad", [np.inf, -np.inf, np.nan, "inf-inf"])
def test_overflow_skip(where, bad, nd):
    """An inf/NaN anywhere skips the step: state bit-identical, t unchanged,
    all-gather window restored; the following steps proceed normally (on
    the prefetch path and both chunked-sum visit shapes)."""
    n = 10000 + 3
    pos = {"first": 0, "middle": n // 2, "last": n - 1}[where]

    def mutate(step, sl):
        if step == 2:
            sl = sl.copy()
            if bad == "inf-inf":
                sl[1, pos], sl[4, pos] = np.inf, -np.inf
            else:
                sl[3, pos] = bad
        return sl

    sh, run, _ = _run_case(n, nd, steps=4, seed=9, mutate=mutate)
    assert sh.flags == [0, 1, 0, 0] and sh.t == 3
    ctl = run.shard.control()
    assert ctl["skipped"] == 1 and ctl["t"] == 3


def test_overflow_window_restored_bitwise():
    n, nd = 3000, 4
    g = np.random.default_rng(3)
    master0 = (g.standard_normal(n) * 0.02).astype(F32)
    run = GpuShardRun(master0, nd, HP)
    sl = gen.host_grad_slices(3, 1, 0, nd, n, 0, n, 1e-3, 1024.0)
    _, p1, m1, v1, bits1 = run.step(sl, 1024.0)
    sl2 = sl.copy()
    sl2[2, 1234] = np.inf
    ctl, p2, m2, v2, bits2 = run.step(sl2, 1024.0)
    assert ctl["overflow"] == 1 and ctl["t"] == 1
    for a, b in ((p1, p2), (m1, m2), (v1, v2)):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(bits1, bits2)


def _reduce_case(nd, n, seed):
    """The reduce pass against the oracle: fp32 g bit-exact, flag exact,
    sum of g^2 within 1e-12, nothing written past the window."""
    torch = torch_mod()
    from zero_partitioned_mixed_buffer_amd import binding as B
    sl = gen.host_grad_slices(seed, 1, 0, nd, n, 0, n, 1e-3, 1024.0)
    s = oracle.reduce_owned(sl)
    gg, ovf, sq = oracle.unscale(s, 1024.0)
    stride = (n + 7) // 8 * 8
    dsl = torch.zeros((nd, stride), dtype=torch.float16, device="cuda")
    dsl[:, :n] = torch.from_numpy(sl).cuda()
    out = torch.full((n + 8,), 123.0, dtype=torch.float32, device="cuda")
    flag = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    ssq = torch.zeros(1, dtype=torch.float64, device="cuda")
    ws = torch.zeros(B.workspace_bytes(), dtype=torch.uint8, device="cuda")
    B.reduce_owned(B.grad_src(dsl, stride, 0, n, nd, 1024.0), out, flag, ssq, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert int(flag.item()) == int(ovf) == 0
    assert np.array_equal(got[:n].view(np.uint32), gg.astype(F32).view(np.uint32))
    assert np.all(got[n:] == 123.0)  # nothing written past the window
    assert float(ssq.item()) == pytest.approx(sq, rel=1e-12)


@pytest.mark.parametrize("nd", list(range(1, 18)))
def test_reduce_owned_every_nd_many_groups_per_lane(nd):
    """The reduce pass for every slice count of its compile-time paths (two
    groups ahead up to Nd = 8, one ahead to 16, chunked past 16), with 6 or
    7 element groups per lane and a ragged tail."""
    _reduce_case(nd, 4 * 65536 * 6 + 4 * 1000 + 3, 400 + nd)


@pytest.mark.parametrize("nd,n", CHUNKED_CASES)
def test_reduce_owned_chunked_visits(nd, n):
    """The reduce pass on the chunked-sum windows of the fused step's test."""
    _reduce_case(nd, n, 600 + nd)


def test_reduce_owned_parity():
    torch = torch_mod()
    from zero_partitioned_mixed_buffer_amd import binding as B
    g = np.random.default_rng(17)
    for n, nd in ((0, 3), (5, 1), (8203, 7), (70001, 33)):
        sl = gen.host_grad_slices(17, 1, 0, nd, n, 0, n, 1e-3, 1024.0)
        sl = _edge_mutate(1, sl) if n > 8 else sl
        s = oracle.reduce_owned(sl)
        gg, ovf, sq = oracle.unscale(s, 1024.0)
        stride = (n + 7) // 8 * 8 + 8
        dsl = torch.zeros((nd, stride), dtype=torch.float16, device="cuda")
        dsl[:, :n] = torch.from_numpy(sl).cuda()
        out = torch.full((max(n, 1),), 123.0, dtype=torch.float32, device="cuda")
        flag = torch.full((1,), 7, dtype=torch.int32, device="cuda")
        ssq = torch.zeros(1, dtype=torch.float64, device="cuda")
        ws = torch.zeros(B.workspace_bytes(), dtype=torch.uint8, device="cuda")
        src = B.grad_src(dsl, stride, 0, n, nd, 1024.0)
        B.reduce_owned(src, out, flag, ssq, ws)
        torch.cuda.synchronize()
        assert int(flag.item()) == int(ovf)
        got = out.cpu().numpy()[:n]
        assert np.array_equal(got.view(np.uint32), gg.astype(F32).view(np.uint32))
        assert float(ssq.item()) == pytest.approx(sq, rel=1e-12, abs=1e-300)
        # second call on the same workspace (completion counter reset)
        sl2 = sl.copy()
        if n:
            sl2[nd - 1, n - 1] = np.nan
            dsl[:, :n] = torch.from_numpy(sl2).cuda()
            B.reduce_owned(src, None, flag, ssq, ws)
            torch.cuda.synchronize()
            assert int(flag.item()) == 1


def test_emit_parity():
    torch = torch_mod()
    from zero_partitioned_mixed_buffer_amd import binding as B
    g = np.random.default_rng(19)
    specials = np.array([int(r, 16) for r in
                         "3f801000 3f803000 477fe000 477ff000 33000000 33400000 387fe000 80000000 "
                         "7f800000 ff800000 00000001 80000001 7f7fffff 3dcccccd".split()],
                        dtype=np.uint32).view(F32)
    # the larger windows give each lane several groups a grid stride apart
    # (the emit loop takes four at a time, then the rest one by one)
    for n in (1, 7, 8, 4096 + 5, 300001, (1 << 24) + 5, 13000003):
        x = (g.standard_normal(n) * 10.0 ** g.uniform(-9, 5, n)).astype(F32)
        x[:min(n, specials.size)] = specials[:min(n, specials.size)]
        d = torch.from_numpy(x).cuda()
        ag = torch.full((n + 16,), 0x7E5A, dtype=torch.int16, device="cuda")
        B.emit_fp16(d, n, ag, 8)
        torch.cuda.synchronize()
        bits = ag.cpu().numpy().view(np.uint16)
        with np.errstate(over="ignore"):
            want = oracle.emit(x).view(np.uint16)
        assert np.array_equal(bits[8:8 + n], want)
        assert np.all(bits[:8] == 0x7E5A) and np.all(bits[8 + n:] == 0x7E5A)


def test_determinism_two_runs():
    n, nd = 100003, 9
    results = []
    for _ in range(2):
        g = np.random.default_rng(77)
        master0 = (g.standard_normal(n) * 0.02).astype(F32)
        run = GpuShardRun(master0, nd, HP)
        for step in range(1, 4):
            sl = gen.host_grad_slices(77, step, 0, nd, n, 0, n, 1e-3, 1024.0)
            ctl, p, m, v, bits = run.step(sl, 1024.0)
        results.append((ctl["sumsq"], p.tobytes(), m.tobytes(), v.tobytes(), bits.tobytes()))
    assert results[0] == results[1]


def test_fused_step_nd400_small_window():
    """Nd = 400 (the largest configuration's slice count) on a small ragged
    window: 200 chunks of 2 slices per element group, in visits of 8 groups
    (two full visits and a 3-element tail)."""
    _run_case(4099, 400, steps=2, seed=400, L=2048.0, sigma=1e-4, dist="student_t3")


def test_all_padding_window():
    """A window that is all padding (zero parameters and zero gradients)
    stays exactly +0 in every buffer, step after step."""
    n, nd = 4104, 5
    master0 = np.zeros(n, dtype=F32)
    sh = oracle.OwnedShard(master0, **HP)
    run = GpuShardRun(master0, nd, HP)
    for step in range(1, 4):
        sl = np.zeros((nd, n), dtype=F16)
        ovf, sq = sh.step(sl, 1024.0)
        ctl, p, m, v, bits = run.step(sl, 1024.0)
        _compare_step(run, sh, ctl, p, m, v, bits, ovf, sq, step, f"padding step {step}")
        for x in (p, m, v):
            assert not np.any(x.view(np.uint32)), "padding must stay +0"
        assert not np.any(run.window(bits))


def test_constant_gradient_twenty_steps():
    """The same gradient every step for 20 steps (the bias corrections run
    through their whole range), three slices with different values."""
    n, nd = 3000, 3

    def const(step, sl):
        out = np.empty_like(sl)
        out[0], out[1], out[2] = 0.25 * 1024, -0.125 * 1024, 2.0**-10 * 1024
        return out.astype(F16)

    _run_case(n, nd, steps=20, seed=9, mutate=const)


@pytest.mark.parametrize("L", [1000.0, 3.7, 65537.0])
def test_non_power_of_two_loss_scale(L):
    """g = s * (1/L) with an inexact reciprocal: the device and the oracle
    take the same two roundings."""
    _run_case(20011, 6, steps=3, seed=int(L) % 97, L=L, sigma=1e-3)


@pytest.mark.parametrize("hp", [
    dict(lr=0.0, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0),     # no movement
    dict(lr=1e-2, beta1=0.0, beta2=0.0, eps=1e-8, weight_decay=0.0),      # m = g, v = g^2
    dict(lr=1e-3, beta1=0.99, beta2=0.9999, eps=1.0, weight_decay=0.5),   # large eps, strong decay
    dict(lr=0.1, beta1=0.5, beta2=0.5, eps=1e-12, weight_decay=1e-4),
])
def test_hyperparameter_extremes(hp):
    _run_case(9001, 4, steps=4, seed=11, hp=hp)


def test_state_canaries():
    """Canary elements right after every state array (both ping-pong sets)
    and the fp32 gradient buffer are never written by the fused, clipped or
    bucketed paths on a ragged window."""
    torch = torch_mod()
    from zero_partitioned_mixed_buffer_amd import binding as B
    n, nd, pad = 4 * 65536 * 2 + 4003, 4, 64
    canary = float.fromhex("0x1.5555p+100")
    g = np.random.default_rng(13)
    arrays = []
    for k in range(7):  # p0 p1 m0 m1 v0 v1 grad
        t = torch.full((n + pad,), canary, dtype=torch.float32, device="cuda")
        if k < 6:
            t[:n] = 0.0
        arrays.append(t)
    arrays[0][:n] = torch.from_numpy((g.standard_normal(n) * 0.02).astype(F32)).cuda()
    ctl = torch.frombuffer(bytearray(B.ctl_init_bytes(1024.0)), dtype=torch.uint8).cuda()
    st = B.adam_state(arrays[0:2], arrays[2:4], arrays[4:6], ctl)
    ws = torch.zeros(B.workspace_bytes(), dtype=torch.uint8, device="cuda")
    ag = torch.zeros(n + pad, dtype=torch.float16, device="cuda")
    stride = (n + 7) // 8 * 8
    sl = torch.zeros((nd, stride), dtype=torch.float16, device="cuda")
    sl[:, :n] = torch.from_numpy(gen.host_grad_slices(13, 1, 0, nd, n, 0, n, 1e-3, 1024.0)).cuda()
    src = B.grad_src(sl, stride, 0, n, nd, 1024.0)
    B.adam_step(src, st, B.adam_hp(1e-3, 0.9, 0.999, 1e-8, 0.0), ag, 0, ws)
    B.adam_step_clipped(src, st, B.adam_hp(1e-3, 0.9, 0.999, 1e-8, 0.0, max_grad_norm=1e-3), arrays[6], ag, 0, ws)
    hp = B.adam_hp(1e-3, 0.9, 0.999, 1e-8, 0.0)
    bucket = 65536 * 4
    for i, o in enumerate(range(0, n, bucket)):
        k = min(bucket, n - o)
        phase = (B.BUCKET_FIRST if o == 0 else 0) | (B.BUCKET_LAST if o + k >= n else 0)
        B.adam_step_bucket(B.grad_src(sl, stride, o, k, nd, 1024.0), st, hp, o, n, ag, 0, phase, ws)
    torch.cuda.synchronize()
    c = B.ctl_from_bytes(bytes(ctl.cpu().numpy().tobytes()))
    assert c["t"] == 3 and c["skipped"] == 0
    for k, t in enumerate(arrays):
        tail = t[n:].cpu().numpy()
        assert np.all(tail == np.float32(canary)), f"array {k} written past its end"
    assert not torch.count_nonzero(ag[n:].view(torch.int16)).item()


def test_column_view_of_wider_slice_buffer():
    """Slices passed as a column view of a wider [Nd, W] buffer: the step
    reads the view's rows W elements apart (the tensor's row stride), not
    its width."""
    torch = torch_mod()
    from zero_partitioned_mixed_buffer_amd import OwnedShard
    n, nd, width = 5000, 5, 5024
    g = np.random.default_rng(29)
    master0 = (g.standard_normal(n) * 0.02).astype(F32)
    ref = oracle.OwnedShard(master0)
    sh = OwnedShard(torch.from_numpy(master0).cuda())
    wide = torch.full((nd, width), 3.0, dtype=torch.float16, device="cuda")
    for step in (1, 2):
        sl = gen.host_grad_slices(29, step, 0, nd, n, 0, n, 1e-3, 1024.0)
        wide[:, 8:8 + n] = torch.from_numpy(sl).cuda()
        ref.step(sl, 1024.0)
        sh.step(wide[:, 8:8 + n], 1024.0)
        torch.cuda.synchronize()
        ctl = sh.control()
        assert ctl["t"] == ref.t == step and ctl["overflow"] == 0
        p, m, v = (x.cpu().numpy() for x in sh.committed(ctl))
        for a, b, nm in ((p, ref.p, "p"), (m, ref.m, "m"), (v, ref.v, "v")):
            assert_state_close(a, b, f"column view step {step} {nm}")


def test_restore_skipped_second_window():
    """zero_restore_skipped re-derives another copy of the window from the
    committed master after a skipped step, and leaves it alone after a
    clean one."""
    torch = torch_mod()
    from zero_partitioned_mixed_buffer_amd import binding as B
    from gpu_util import SENTINEL
    n, nd = 20011, 3
    g = np.random.default_rng(31)
    master0 = (g.standard_normal(n) * 0.02).astype(F32)
    ref = oracle.OwnedShard(master0)
    run = GpuShardRun(master0, nd, {})
    other = torch.full((n + 16,), SENTINEL, dtype=torch.int16, device="cuda")
    for step in (1, 2):
        sl = gen.host_grad_slices(31, step, 0, nd, n, 0, n, 1e-3, 1024.0)
        if step == 2:
            sl[1, n // 3] = np.nan
        ovf, _ = ref.step(sl, 1024.0)
        ctl = run.step(sl, 1024.0)[0]
        assert ctl["overflow"] == int(ovf) == (step == 2)
        B.restore_skipped(run.shard.state, n, other, 8)
        torch.cuda.synchronize()
        bits = other.cpu().numpy().view(np.uint16)
        if step == 1:
            assert np.all(bits == SENTINEL)  # clean step: nothing written
        else:
            assert_fp16_close(bits[8:8 + n], ref.window().view(np.uint16), "restored window")
            assert np.all(bits[:8] == SENTINEL) and np.all(bits[8 + n:] == SENTINEL)


def test_largest_nd():
    """Nd = 8191, the largest the library accepts (float64 holds the sum of
    fewer than 2^13 fp16 values exactly): 4095 chunks of 2 slices and a
    remainder of 1.  One element carries 65504 in every slice (the largest
    finite fp16, sum 8191 * 65504), another alternating +-65504 (sum 65504);
    the step must match the oracle and stay finite."""
    nd, n = 8191, 1001

    def mutate(step, sl):
        sl[:, 5] = np.float16(65504.0)
        sl[:, 6] = np.where(np.arange(nd) % 2 == 0, np.float16(65504.0), np.float16(-65504.0))
        return sl

    sh, _, _ = _run_case(n, nd, 2, 83, L=65536.0, sigma=1e-4, mutate=mutate)
    assert sh.flags == [0, 0]


@pytest.mark.parametrize("nd,n,dist", [(7, 70001, "normal"), (16, 100003, "normal"),
                                       (48, 2**21 + 2053, "student_t3"), (400, 40961, "student_t3")])
def test_exact_sum_invariants(nd, n, dist):
    """Invariants of the exact Nd-way sum on the HIP path itself, beside the
    oracle comparison: permuting the slices, or doubling every gradient
    together with the loss scale (exact in fp16 here, and 1/L a power of
    two), gives the same state, window, Sigma g^2 and step count bit for bit.
    The prefetch paths, both visit shapes and Student-t tails are covered."""
    L = 1024.0 if dist == "normal" else 2048.0
    sigma = 1e-3 if dist == "normal" else 1e-4
    g = np.random.default_rng(nd * 7 + 1)
    master0 = (g.standard_normal(n) * 0.02).astype(F32)
    runs = [GpuShardRun(master0, nd, HP) for _ in range(3)]
    for step in range(1, 4):
        sl = gen.host_grad_slices(nd + 40, step, 0, nd, n, 0, n, sigma, L, dist)
        assert np.all(np.isfinite(sl.astype(np.float32) * 2)), "doubling must stay finite in fp16"
        perm = g.permutation(nd)
        outs = [runs[0].step(sl, L), runs[1].step(np.ascontiguousarray(sl[perm]), L),
                runs[2].step((sl.astype(np.float32) * 2).astype(F16), 2 * L)]
        ref_ctl, rp, rm, rv, rbits = outs[0]
        assert ref_ctl["overflow"] == 0 and ref_ctl["t"] == step
        for k, what in ((1, "permuted"), (2, "doubled")):
            ctl, p, m, v, bits = outs[k]
            tag = f"nd={nd} n={n} step={step} {what}"
            assert ctl["t"] == ref_ctl["t"] and ctl["overflow"] == 0, tag
            assert ctl["sumsq"] == ref_ctl["sumsq"], tag
            for a, b, name in ((p, rp, "master"), (m, rm, "exp_avg"), (v, rv, "exp_avg_sq")):
                assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{tag} {name}"
            assert np.array_equal(runs[k].window(bits), runs[0].window(rbits)), f"{tag} window"
            assert runs[k].guards_intact(bits), tag

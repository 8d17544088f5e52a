"""GPU parity of dynamic loss scaling and global-norm clipping against the
oracle.  Same bar as the fused step: flags, step counts and the scale
trajectory bit-exact; fp32 state within 1e-5 relative per element; fp16
window within 1 ulp; sum of g^2 and the clip coefficient within 1e-12."""
import numpy as np
import pytest

import oracle
from workloads import gen

from gpu_util import F16, F32, GpuShardRun, assert_fp16_close, assert_state_close

pytestmark = pytest.mark.gpu


def _run(n, nd, steps, seed, hp, bad_steps=(), sigma=1e-3, static_L=1024.0):
    g = np.random.default_rng(seed)
    master0 = (g.standard_normal(n) * 0.02).astype(F32)
    sh = oracle.OwnedShard(master0, **hp)
    run = GpuShardRun(master0, nd, hp)
    dynamic = hp.get("scale_interval", 0) > 0
    for step in range(1, steps + 1):
        L = sh.scale if dynamic else static_L
        sl = gen.host_grad_slices(seed, step, 0, nd, n, 0, n, sigma, L)
        if step in bad_steps:
            sl[step % nd, (step * 7919) % max(n, 1)] = np.nan if step % 2 else np.inf
        ovf, sq = sh.step(sl, static_L)
        ctl, p, m, v, bits = run.step(sl, static_L)
        tag = f"n={n} nd={nd} step={step}"
        assert ctl["overflow"] == int(ovf) and ctl["t"] == sh.t, tag
        if dynamic:
            assert ctl["loss_scale"] == sh.scale and ctl["good_steps"] == sh.good_steps, tag
        for got, want, nm in ((p, sh.p, "p"), (m, sh.m, "m"), (v, sh.v, "v")):
            assert_state_close(got, want, f"{tag} {nm}")
        assert_fp16_close(run.window(bits), sh.window().view(np.uint16), f"{tag} window")
        assert run.guards_intact(bits), tag
        if not ovf:
            assert ctl["sumsq"] == pytest.approx(sq, rel=1e-12, abs=1e-300), tag
            assert ctl["clip_coef"] == pytest.approx(sh.coefs[-1], rel=1e-12), tag
    return sh, run


HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)


@pytest.mark.parametrize("nd", [1, 4, 9, 24, 64])
def test_dynamic_scaling_fused(nd):
    """The scale trajectory through skips and growth, on the prefetch path
    (Nd <= 16) and both chunked-sum visit shapes (Nd 24 and 64)."""
    hp = dict(HP, scale_interval=2, loss_scale=4096.0)
    sh, _ = _run(20003, nd, 9, 40 + nd, hp, bad_steps=(2, 6, 7))
    assert sh.flags == [0, 1, 0, 0, 0, 1, 1, 0, 0]
    assert sh.scales == [4096.0, 4096.0, 2048.0, 2048.0, 4096.0, 4096.0, 2048.0, 1024.0, 1024.0]


@pytest.mark.parametrize("max_norm", [1e-3, 1e9])
@pytest.mark.parametrize("n,nd", [(5003, 3), (65536 + 12, 8)])
def test_clipped_step(n, nd, max_norm):
    hp = dict(HP, max_grad_norm=max_norm)
    sh, _ = _run(n, nd, 5, 50 + nd, hp, bad_steps=(3,))
    assert sh.flags == [0, 0, 1, 0, 0]
    if max_norm < 1:
        assert max(c for c in sh.coefs if c == c) < 1.0  # clipping was active
    else:
        assert all(c == 1.0 for c in sh.coefs if c == c)


@pytest.mark.parametrize("nd", [2, 8, 17, 24, 48, 99])
def test_clipped_many_groups_per_lane(nd):
    """Both clipped passes on a window where each lane owns 6 or 7 element
    groups (the prefetch rotations run several full cycles), ragged tail,
    clipping active, one skipped step.  Past 16 slices the reduce pass sums
    in chunks over visits of 4 (Nd < 32) or 8 groups, with Nd = 99 leaving
    a one-slice last chunk."""
    n = 4 * 65536 * 6 + 4 * 1000 + 3
    hp = dict(HP, weight_decay=0.01, max_grad_norm=0.05)
    sh, _ = _run(n, nd, 3, 70 + nd, hp, bad_steps=(2,))
    assert sh.flags == [0, 1, 0]
    assert max(c for c in sh.coefs if c == c) < 1.0


def test_clipped_adamw_dynamic_scaling():
    hp = dict(HP, weight_decay=0.01, max_grad_norm=5e-3, scale_interval=3, loss_scale=8192.0)
    sh, _ = _run(30000, 16, 8, 61, hp, bad_steps=(4,), sigma=1e-4)
    assert sh.flags == [0, 0, 0, 1, 0, 0, 0, 0]
    assert sh.scales[-1] != sh.scales[0]


def test_clipped_skip_leaves_window_and_state():
    """An overflowing clipped step touches neither the state nor the fp16
    window (no restore launch is made for the clipped path)."""
    n, nd = 4099, 5
    g = np.random.default_rng(7)
    master0 = (g.standard_normal(n) * 0.02).astype(F32)
    run = GpuShardRun(master0, nd, dict(HP, max_grad_norm=0.01))
    sl = gen.host_grad_slices(7, 1, 0, nd, n, 0, n, 1e-3, 1024.0)
    _, p1, m1, v1, bits1 = run.step(sl, 1024.0)
    sl2 = sl.copy()
    sl2[4, n - 1] = -np.inf
    ctl, p2, m2, v2, bits2 = run.step(sl2, 1024.0)
    assert ctl["overflow"] == 1 and ctl["t"] == 1 and ctl["skipped"] == 1
    for a, b in ((p1, p2), (m1, m2), (v1, v2)):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(bits1, bits2)


@pytest.mark.parametrize("nd", [3, 24])
def test_dynamic_scale_limits(nd):
    """Dynamic scaling at the ends of float64: a growth from 2^1023 would
    overflow, so the scale stays (the count resets); a backoff from
    2^-1073 reaches 2^-1074 and then 0, and with 1/L = inf every g is
    non-finite, so those steps are skipped and the state is never written.
    The slices are drawn at a fixed scale; only the control block's scale
    is extreme."""
    n = 20003
    g = np.random.default_rng(80 + nd)
    master0 = (g.standard_normal(n) * 0.02).astype(F32)
    for start, bad_steps, want_scales, want_flags in (
            (2.0 ** 1022, (3,), [2.0 ** 1022, 2.0 ** 1023, 2.0 ** 1023, 2.0 ** 1022],
             [0, 0, 1, 0]),
            (2.0 ** -1073, (), [2.0 ** -1073, 2.0 ** -1074, 0.0, 0.0], [1, 1, 1, 1])):
        hp = dict(HP, scale_interval=1, loss_scale=start)
        sh = oracle.OwnedShard(master0, **hp)
        run = GpuShardRun(master0, nd, hp)
        for step in range(1, 5):
            sl = gen.host_grad_slices(80 + nd, step, 0, nd, n, 0, n, 1e-3, 1024.0)
            if step in bad_steps:
                sl[1, 17] = np.inf
            ovf, sq = sh.step(sl)
            ctl, p, m, v, bits = run.step(sl, 1.0)
            tag = f"nd={nd} start={start} step={step}"
            assert ctl["overflow"] == int(ovf) and ctl["t"] == sh.t, tag
            assert ctl["loss_scale"] == sh.scale and ctl["good_steps"] == sh.good_steps, tag
            for got, want, nm in ((p, sh.p, "p"), (m, sh.m, "m"), (v, sh.v, "v")):
                assert_state_close(got, want, f"{tag} {nm}")
            assert_fp16_close(run.window(bits), sh.window().view(np.uint16), f"{tag} window")
            assert run.guards_intact(bits), tag
        assert sh.scales == want_scales and sh.flags == want_flags
        if want_flags == [1, 1, 1, 1]:
            assert np.array_equal(p.view(np.uint32), master0.view(np.uint32)) and not np.any(m)

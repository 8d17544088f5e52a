"""Pins of the oracle to facts outside itself (no GPU).

Each test ties one part of the oracle to what the pages print, to a closed
form of Adam, to exact rational arithmetic, to torch's float64 Adam, or to
hand-derived IEEE rounding results.  The last group plants plausible mistakes
into copies of the oracle's arithmetic and checks that the pins catch them.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import zero_oracle as zo

F16, F32, F64 = np.float16, np.float32, np.float64


# ----------------------------------------------------------------- memory model
def test_memory_table_printed(golden):
    """7.5B parameters, Nd = 64: 120 / 31.4 / 16.6 / 1.9 GB, 2Psi / 3Psi."""
    for psi, nd, stage, gb, red, comm in golden("memory_table.txt"):
        r = oracle.memory_model(float(psi), int(nd), int(stage))
        assert round(r["total_bytes"] / 1e9, 1) == float(gb)
        assert r["comm_elems"] == float(comm) * float(psi)
        if int(stage) in (0, 3):
            # 1x and 64x are exact at Nd = 64
            assert r["reduction_vs_dp"] == float(red)
        else:
            # 4x and 8x are the large-Nd limits of 16/(4+12/Nd), 16/(2+14/Nd)
            lim = oracle.memory_model(float(psi), 10**9, int(stage))["reduction_vs_dp"]
            assert abs(lim - float(red)) < 1e-6
            assert r["reduction_vs_dp"] < float(red)


def test_memory_gpt2_1p5b():
    """GPT-2 1.5B: 24 GB or more of model state against 3 GB of fp16 weights
    (trishampatil "The Real Problem")."""
    r = oracle.memory_model(1.5e9, 1, 0)
    assert r["total_bytes"] == 24e9
    assert r["params_bytes"] == 3e9
    # K = 12: fp32 copy + momentum + variance, 4 bytes each
    assert r["optim_bytes"] == 12 * 1.5e9


def test_memory_stage_structure():
    """Stage formulas: 16Psi, 4Psi+12Psi/Nd, 2Psi+14Psi/Nd, 16Psi/Nd; a
    single rank (Nd = 1) partitions nothing; comm 3Psi/2Psi = 1.5."""
    psi = 1e9
    for nd in (1, 2, 7, 64, 400):
        t = [oracle.memory_model(psi, nd, s)["total_bytes"] for s in range(4)]
        assert t[0] == 16 * psi
        assert math.isclose(t[1], 4 * psi + 12 * psi / nd, rel_tol=1e-15)
        assert math.isclose(t[2], 2 * psi + 14 * psi / nd, rel_tol=1e-15)
        assert math.isclose(t[3], 16 * psi / nd, rel_tol=1e-15)
        if nd == 1:
            assert t[0] == t[1] == t[2] == t[3]
        else:
            assert t[0] > t[1] > t[2] > t[3]
    c = [oracle.memory_model(psi, 8, s)["comm_elems"] for s in range(4)]
    assert c[0] == c[1] == c[2] == 2 * psi and c[3] / c[2] == 1.5
    assert oracle.memory_model(psi, 8, 2)["comm_elems_ring"] == 2 * psi * 7 / 8


def _ring_reduce_scatter(bufs, sent):
    """Ring reduce-scatter of Nd equal-length vectors (one per rank), run
    step by step: in step k rank r sends its partial of chunk (r - k) mod Nd
    to rank r + 1, which adds it to its own.  After Nd - 1 steps rank r holds
    the full sum of chunk (r + 1) mod Nd.  sent[r] counts the elements rank
    r put on the wire."""
    nd = len(bufs)
    n = bufs[0].size // nd
    acc = [b.astype(F64).copy() for b in bufs]
    for k in range(nd - 1):
        msgs = []
        for r in range(nd):
            c = (r - k) % nd
            msgs.append((r, c, acc[r][c * n:(c + 1) * n].copy()))
        for r, c, m in msgs:
            dst = (r + 1) % nd
            acc[dst][c * n:(c + 1) * n] += m
            sent[r] += m.size
    return {(r + 1) % nd: acc[r][((r + 1) % nd) * n:((r + 1) % nd + 1) * n] for r in range(nd)}


def _ring_all_gather(owned, nd, n, sent):
    """Ring all-gather: rank r starts with its chunk r; in step k it sends
    chunk (r - k) mod Nd to rank r + 1.  Returns every rank's full vector."""
    full = [np.full(nd * n, np.nan) for _ in range(nd)]
    for r in range(nd):
        full[r][r * n:(r + 1) * n] = owned[r]
    for k in range(nd - 1):
        msgs = [(r, (r - k) % nd) for r in range(nd)]
        data = [full[r][c * n:(c + 1) * n].copy() for r, c in msgs]
        for (r, c), m in zip(msgs, data):
            full[(r + 1) % nd][c * n:(c + 1) * n] = m
            sent[r] += m.size
    return full


@pytest.mark.parametrize("nd", [1, 2, 3, 8, 13])
def test_ring_volume_by_simulation(nd):
    """The ring variant of the communication volume, counted rather than
    computed: a ring reduce-scatter and ring all-gathers are run on data
    (their results are checked), the elements each rank sends are tallied,
    and the tally per stage (Pos / Pos+g: one reduce-scatter + one
    all-gather; Pos+g+p: two parameter all-gathers + one reduce-scatter) is
    compared with comm_elems_ring.  A factor such as Nd/(Nd-1) or
    2(Nd-1)/Nd per collective would fail here."""
    g = np.random.default_rng(nd)
    n = 5
    psi = nd * n
    grads = [g.integers(-50, 50, psi).astype(F64) for _ in range(nd)]
    sent_rs = np.zeros(nd, dtype=np.int64)
    owned = _ring_reduce_scatter(grads, sent_rs)
    total = np.sum(grads, axis=0)
    for r in range(nd):
        assert np.array_equal(owned[r], total[r * n:(r + 1) * n])
    params = g.standard_normal(psi)
    sent_ag = np.zeros(nd, dtype=np.int64)
    full = _ring_all_gather([params[r * n:(r + 1) * n] for r in range(nd)], nd, n, sent_ag)
    for r in range(nd):
        assert np.array_equal(full[r], params)
    # every rank sends the same amount in each collective
    assert len(set(sent_rs)) == 1 and len(set(sent_ag)) == 1
    per_stage = {0: sent_rs[0] + sent_ag[0], 1: sent_rs[0] + sent_ag[0], 2: sent_rs[0] + sent_ag[0],
                 3: sent_rs[0] + 2 * sent_ag[0]}
    for stage, want in per_stage.items():
        r = oracle.memory_model(psi, nd, stage)
        assert r["comm_elems_ring"] == pytest.approx(float(want), rel=1e-15, abs=1e-9)
        # and the nominal volume is the ring's without the (Nd-1)/Nd factor
        assert r["comm_elems"] == pytest.approx(float(want) * nd / max(nd - 1, 1) if nd > 1 else
                                                r["comm_elems"], rel=1e-15)


# ----------------------------------------------------------------- planner
@pytest.mark.parametrize("align", [8, 256])
def test_plan_bruteforce(align):
    g = np.random.default_rng(7)
    for _ in range(300):
        nt = int(g.integers(1, 6))
        numels = [int(x) for x in g.integers(0, 1200, nt)]
        nd = int(g.integers(1, 18))
        p = oracle.plan(numels, nd, align)
        psi = sum(numels)
        assert p.psi == psi and p.padded == nd * p.part and p.pad == p.padded - psi
        assert p.part % align == 0 and 0 <= p.pad < nd * align
        # S is the smallest multiple of align with nd * S >= psi
        assert nd * p.part >= psi and (p.part == 0 or nd * (p.part - align) < psi)
        # every tensor element is covered exactly once, inside one rank window
        cover = np.zeros(max(psi, 1), dtype=np.int64)
        base = np.concatenate([[0], np.cumsum(numels)])
        for f in p.frags:
            assert f.length > 0
            assert f.flat_off == base[f.tensor] + f.tensor_off
            assert f.rank * p.part + f.local_off == f.flat_off
            assert 0 <= f.local_off and f.local_off + f.length <= p.part
            assert 0 <= f.rank < nd
            cover[f.flat_off:f.flat_off + f.length] += 1
        assert np.all(cover[:psi] == 1)
        # fragments are maximal: consecutive pieces of a tensor change rank
        for a, b in zip(p.frags, p.frags[1:]):
            if a.tensor == b.tensor:
                assert b.rank == a.rank + 1 and b.local_off == 0


def test_plan_empty_and_single():
    p = oracle.plan([], 4, 256)
    assert p.part == 0 and p.padded == 0 and p.frags == []
    p = oracle.plan([0, 0], 3, 8)
    assert p.part == 0 and p.frags == []
    p = oracle.plan([1], 1, 256)
    assert p.part == 256 and p.pad == 255 and len(p.frags) == 1


# ----------------------------------------------------------------- reduction
def _edge_fp16(g, shape):
    pool = np.array([0.0, -0.0, 65504.0, -65504.0, 2.0**-24, -(2.0**-24), 2.0**-14,
                     1.0, -1.0, 0.5, 3.140625, 1000.0, -2.0**-23], dtype=F16)
    x = (g.standard_normal(shape) * 10.0).astype(F16)
    pick = g.random(shape) < 0.3
    x[pick] = pool[g.integers(0, len(pool), int(pick.sum()))]
    return x


def test_reduce_exact_vs_fractions():
    g = np.random.default_rng(3)
    for nd in (1, 2, 3, 17, 64):
        sl = _edge_fp16(g, (nd, 64))
        s = oracle.reduce_owned(sl)
        for j in range(sl.shape[1]):
            exact = sum(Fraction(float(sl[k, j])) for k in range(nd))
            assert s[j] == float(exact)  # exact sum is representable


def test_reduce_special_cases():
    g = np.random.default_rng(4)
    x = _edge_fp16(g, (1, 200))
    s1 = oracle.reduce_owned(x)
    assert np.array_equal(s1.view(np.uint64), x[0].astype(F64).view(np.uint64))
    same = np.repeat(x, 9, axis=0)
    s9 = oracle.reduce_owned(same)
    assert np.array_equal(s9, 9.0 * x[0].astype(F64))
    # permutation invariance, bit for bit (including zero signs away from 0)
    sl = _edge_fp16(g, (12, 300))
    a = oracle.reduce_owned(sl)
    b = oracle.reduce_owned(sl[g.permutation(12)])
    nz = a != 0
    assert np.array_equal(a[nz], b[nz])


def test_reduce_zero_sign_in_any_order():
    """The exact sum's sign of zero: -0 only when every term is -0, +0 for a
    mixed-sign zero column and for any exact cancellation (round to nearest
    gives +0 for x + (-x)).  All 24 orders of the four slices give the same
    bits, so the kernels' slice order cannot matter even for zeros."""
    from itertools import permutations
    tiny = 2.0**-24
    cols = np.array([
        [-0.0, -0.0, -0.0, -0.0],         # -0
        [0.0, -0.0, -0.0, -0.0],          # +0
        [1.0, -1.0, -0.0, -0.0],          # +0: exact cancellation
        [-0.0, tiny, -tiny, -0.0],        # +0
        [65504.0, -65504.0, -0.0, -0.0],  # +0
        [-0.0, -0.0, 1.0, -1.0],          # +0: cancellation after -0 + -0
        [-0.0, 3.0, -1.0, -0.0],          # 2
    ], dtype=F16).T  # [4 slices, 7 elements]
    want = np.array([-0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 2.0])
    for perm in permutations(range(4)):
        got = oracle.reduce_owned(cols[list(perm)])
        assert np.array_equal(got.view(np.uint64), want.view(np.uint64)), perm


def test_unscale_flag_and_norm():
    g = np.random.default_rng(5)
    sl = (g.standard_normal((5, 100)) * 300).astype(F16)
    s = oracle.reduce_owned(sl)
    gg, ovf, sq = oracle.unscale(s, 1024.0)
    assert not ovf
    exact = sum(Fraction(float(v)) ** 2 for v in gg)
    assert abs(Fraction(sq) - exact) <= abs(exact) * Fraction(1, 2**52)
    # g is s divided by L: exact for a power-of-two L
    assert all(Fraction(float(a)) == Fraction(float(b)) / 1024 for a, b in zip(gg, s))
    for bad in (np.inf, -np.inf, np.nan):
        sl2 = sl.copy()
        sl2[3, 57] = bad
        _, ovf2, _ = oracle.unscale(oracle.reduce_owned(sl2), 1024.0)
        assert ovf2
    sl3 = sl.copy()
    sl3[0, 1] = np.inf
    sl3[1, 1] = -np.inf  # +inf + -inf = NaN, still flagged
    assert oracle.unscale(oracle.reduce_owned(sl3), 1024.0)[1]


# ----------------------------------------------------------------- Adam
def _torch_adam_run(p0, grads, lr, b1, b2, eps, wd):
    torch = pytest.importorskip("torch")
    p = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    if wd:
        opt = torch.optim.AdamW([p], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd,
                                foreach=False, fused=False)
    else:
        opt = torch.optim.Adam([p], lr=lr, betas=(b1, b2), eps=eps, weight_decay=0.0,
                               foreach=False, fused=False)
    for gr in grads:
        p.grad = torch.tensor(gr, dtype=torch.float64)
        opt.step()
    st = opt.state[p]
    return p.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


def _oracle_run(p0, grads, lr, b1, b2, eps, wd, adam=None, scalars=None):
    adam = adam or zo.adam_update
    scalars = scalars or zo.step_scalars
    p = p0.astype(F64)
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    b1p = b2p = 1.0
    for gr in grads:
        sc = scalars(lr, b1, b2, eps, wd, b1p, b2p)
        p, m, v = adam(p, m, v, gr, sc)
        b1p, b2p = sc["b1t"], sc["b2t"]
    return p, m, v


def _close(a, b, scale):
    return bool(np.all(np.abs(a - b) <= 1e-12 * scale))


ADAM_CASES = [
    (1e-3, 0.9, 0.999, 1e-8, 0.0),
    (1e-3, 0.9, 0.999, 1e-8, 0.01),
    (3e-2, 0.8, 0.95, 1e-6, 0.1),
]


@pytest.mark.parametrize("lr,b1,b2,eps,wd", ADAM_CASES)
def test_adam_matches_torch_float64(lr, b1, b2, eps, wd):
    """The oracle's Adam/AdamW (float64 storage) against torch.optim's
    single-tensor Adam/AdamW in float64 over 12 steps."""
    g = np.random.default_rng(11)
    p0 = g.standard_normal(500) * 0.02
    grads = [g.standard_normal(500) * 10.0 ** g.uniform(-6, -1) for _ in range(12)]
    tp, tm, tv = _torch_adam_run(p0, grads, lr, b1, b2, eps, wd)
    op, om, ov = _oracle_run(p0, grads, lr, b1, b2, eps, wd)
    gs = max(np.max(np.abs(x)) for x in grads)
    assert _close(op, tp, 1.0) and _close(om, tm, gs) and _close(ov, tv, gs * gs)


def test_adam_first_step_closed_form():
    """Step 1: m = (1-b1) g, v = (1-b2) g^2, p = p0*(1-lr*wd) - lr*g/(|g|+eps);
    checked in float64 at 1e-12 and within 1 fp32 ulp after fp32 storage."""
    g = np.random.default_rng(12)
    p0 = (g.standard_normal(4000) * 0.02).astype(F32)
    gr = g.standard_normal(4000) * 1e-3
    gr[:5] = [0.0, 1e-12, -1e-12, 5.0, -5.0]
    for wd in (0.0, 0.01):
        sc = oracle.step_scalars(1e-3, 0.9, 0.999, 1e-8, wd, 1.0, 1.0)
        p64, m64, v64 = oracle.adam_update(p0.astype(F64), np.zeros(4000), np.zeros(4000), gr, sc)
        cf = p0.astype(F64) * (1 - 1e-3 * wd) - 1e-3 * gr / (np.abs(gr) + 1e-8)
        assert np.all(np.abs(p64 - cf) <= 1e-12 * np.maximum(np.abs(cf), 1e-3))
        assert np.allclose(m64, 0.1 * gr, rtol=1e-14, atol=0)
        assert np.allclose(v64, 0.001 * gr * gr, rtol=1e-14, atol=0)
        p32, m32, v32 = oracle.adam_update(p0, np.zeros(4000, F32), np.zeros(4000, F32), gr, sc)
        ulp = np.spacing(np.abs(cf.astype(F32)))
        assert np.all(np.abs(p32.astype(F64) - cf) <= ulp)


def test_adam_constant_gradient_and_skip():
    """Constant g: bias-corrected m-hat = g and v-hat = g^2, so every step
    moves p by lr*g/(|g|+eps); a skipped (overflowing) step must not advance
    t.  float64 storage, 20 steps, step 7 overflows."""
    n = 64
    g = np.random.default_rng(13)
    x = (g.standard_normal(n) * 100).astype(F16)
    x[0] = 0
    slices = np.stack([x, x, x])  # Nd = 3
    L = 256.0
    sh = oracle.OwnedShard(np.zeros(n), lr=1e-3, state_dtype=F64)
    bad = slices.copy()
    bad[1, 5] = np.inf
    clean = 0
    for step in range(1, 21):
        ovf, _ = sh.step(bad if step == 7 else slices, L)
        assert ovf == (step == 7)
        clean += not ovf
    assert sh.t == clean == 19
    gg = 3.0 * x.astype(F64) / L
    want = -clean * 1e-3 * gg / (np.abs(gg) + 1e-8)
    assert np.all(np.abs(sh.p - want) <= 1e-11 * np.maximum(np.abs(want), 1e-12))
    assert sh.flags == [0] * 6 + [1] + [0] * 13


def test_adam_zero_gradient():
    """g = 0: m -> b1*m, v -> b2*v, and with m = 0 the parameter moves only
    by the decoupled decay."""
    g = np.random.default_rng(14)
    p = (g.standard_normal(300) * 0.02).astype(F32)
    m = (g.standard_normal(300) * 1e-3).astype(F32)
    v = (g.random(300) * 1e-6).astype(F32)
    sc = oracle.step_scalars(1e-3, 0.9, 0.999, 1e-8, 0.0, 0.9, 0.999)
    _, m1, v1 = oracle.adam_update(p, m, v, np.zeros(300), sc)
    assert np.array_equal(m1, (0.9 * m.astype(F64)).astype(F32))
    assert np.array_equal(v1, (0.999 * v.astype(F64)).astype(F32))
    z = np.zeros(300, F32)
    p1, _, _ = oracle.adam_update(p, z, z, np.zeros(300), sc)
    assert np.array_equal(p1, p)
    sc2 = oracle.step_scalars(1e-3, 0.9, 0.999, 1e-8, 0.5, 1.0, 1.0)
    p2, _, _ = oracle.adam_update(p, z, z, np.zeros(300), sc2)
    assert np.array_equal(p2, (p.astype(F64) * (1 - 1e-3 * 0.5)).astype(F32))


def _shard_run(slices_steps, L, n, master=None, wd=0.0):
    sh = oracle.OwnedShard(master if master is not None else np.zeros(n, F32), weight_decay=wd)
    for sl in slices_steps:
        sh.step(sl, L)
    return sh


def test_shard_invariances():
    """Permuting slices and scaling grads and L together by 2 give identical
    bits; padding stays exactly zero."""
    g = np.random.default_rng(15)
    n, nd = 512, 6
    master = (g.standard_normal(n) * 0.02).astype(F32)
    master[-40:] = 0
    steps = []
    for _ in range(4):
        sl = (g.standard_normal((nd, n)) * 1e-3 * 1024).astype(F16)
        sl[:, -40:] = 0
        steps.append(sl)
    a = _shard_run(steps, 1024.0, n, master)
    b = _shard_run([s[g.permutation(nd)] for s in steps], 1024.0, n, master)
    c = _shard_run([(s.astype(F32) * 2).astype(F16) for s in steps], 2048.0, n, master)
    for x in (b, c):
        for name in ("p", "m", "v"):
            assert np.array_equal(getattr(a, name).view(np.uint32), getattr(x, name).view(np.uint32))
    for name in ("p", "m", "v"):
        assert np.all(getattr(a, name)[-40:].view(np.uint32) == 0)
    assert np.all(a.window()[-40:].view(np.uint16) == 0)


def test_overflow_skip_sequence():
    """A C5-like sequence on a small window: Nd = 20, +inf in slice 17 at
    step 2 of 4.  The skipped step leaves state and window bit-identical and
    t unchanged; flags are [0, 1, 0, 0]."""
    g = np.random.default_rng(16)
    n, nd = 256, 20
    sh = oracle.OwnedShard((g.standard_normal(n) * 0.02).astype(F32))
    for step in range(1, 5):
        sl = (g.standard_t(3, (nd, n)) * 1e-4 * 2048).astype(F16)
        if step == 2:
            sl[17, n // 2] = np.inf
            before = (sh.p.copy(), sh.m.copy(), sh.v.copy(), sh.window().copy(), sh.t)
        ovf, _ = sh.step(sl, 2048.0)
        if step == 2:
            assert ovf
            for x, y in zip(before[:4], (sh.p, sh.m, sh.v, sh.window())):
                assert np.array_equal(x.view(np.uint8), y.view(np.uint8))
            assert sh.t == before[4]
    assert sh.flags == [0, 1, 0, 0] and sh.t == 3


def test_emit_rne_golden(golden):
    for row in golden("fp16_rne.txt"):
        x = np.array([int(row[0], 16)], dtype=np.uint32).view(F32)
        with np.errstate(over="ignore"):
            h = oracle.emit(x).view(np.uint16)[0]
        assert h == int(row[1], 16), row
    nan = oracle.emit(np.array([np.nan], F32))
    assert np.isnan(nan[0])


# ----------------------------------------------------------------- planted mistakes
def _mut_scalars(kind):
    def f(lr, b1, b2, eps, wd, b1p, b2p):
        sc = zo.step_scalars(lr, b1, b2, eps, wd, b1p, b2p)
        if kind == "no_bias_correction":
            sc = dict(sc, ss=lr, isb=1.0)
        elif kind == "swap_betas":
            sc = dict(sc, b1=b2, b2=b1, omb1=1 - b2, omb2=1 - b1)
        elif kind == "decay_sign":
            sc = dict(sc, dcy=1.0 + lr * wd)
        elif kind == "eps_hat":
            sc = dict(sc, eps=eps * math.sqrt(1 - b2p * b2))
        elif kind == "bias_power_off_by_one":
            sc = dict(sc, ss=lr / (1 - sc["b1t"] * b1), isb=1.0 / math.sqrt(1 - sc["b2t"] * b2))
        return sc
    return f


def _mut_adam(kind):
    def f(p, m, v, g, sc):
        if kind == "eps_inside_sqrt":
            p64, m64, v64 = p.astype(F64), m.astype(F64), v.astype(F64)
            m1 = sc["b1"] * m64 + sc["omb1"] * g
            v1 = sc["b2"] * v64 + sc["omb2"] * g * g
            q = m1 / np.sqrt(v1 * sc["isb"] ** 2 + sc["eps"])
            return (p64 * sc["dcy"] - sc["ss"] * q).astype(p.dtype), m1.astype(p.dtype), v1.astype(p.dtype)
        if kind == "grad_not_squared":
            p64, m64, v64 = p.astype(F64), m.astype(F64), v.astype(F64)
            m1 = sc["b1"] * m64 + sc["omb1"] * g
            v1 = sc["b2"] * v64 + sc["omb2"] * np.abs(g)
            q = m1 / (np.sqrt(v1) * sc["isb"] + sc["eps"])
            return (p64 * sc["dcy"] - sc["ss"] * q).astype(p.dtype), m1.astype(p.dtype), v1.astype(p.dtype)
        if kind == "coupled_decay":
            p64, m64, v64 = p.astype(F64), m.astype(F64), v.astype(F64)
            gw = g + (1 - sc["dcy"]) / sc["ss"] * p64 if sc["dcy"] != 1 else g
            m1 = sc["b1"] * m64 + sc["omb1"] * gw
            v1 = sc["b2"] * v64 + sc["omb2"] * gw * gw
            q = m1 / (np.sqrt(v1) * sc["isb"] + sc["eps"])
            return (p64 - sc["ss"] * q).astype(p.dtype), m1.astype(p.dtype), v1.astype(p.dtype)
        raise ValueError(kind)
    return f


@pytest.mark.parametrize("kind", ["no_bias_correction", "swap_betas", "decay_sign", "eps_hat",
                                  "bias_power_off_by_one"])
def test_planted_scalar_mistakes_are_caught(kind):
    g = np.random.default_rng(21)
    p0 = g.standard_normal(200) * 0.02
    grads = [g.standard_normal(200) * 1e-7 for _ in range(5)]
    caught = False
    for lr, b1, b2, eps, wd in ADAM_CASES:
        tp, tm, tv = _torch_adam_run(p0, grads, lr, b1, b2, eps, wd)
        op, om, ov = _oracle_run(p0, grads, lr, b1, b2, eps, wd, scalars=_mut_scalars(kind))
        caught |= not (_close(op, tp, 1.0) and _close(om, tm, 1e-7) and _close(ov, tv, 1e-14))
    assert caught


@pytest.mark.parametrize("kind", ["eps_inside_sqrt", "grad_not_squared", "coupled_decay"])
def test_planted_update_mistakes_are_caught(kind):
    g = np.random.default_rng(22)
    p0 = g.standard_normal(200) * 0.02
    grads = [g.standard_normal(200) * 1e-3 for _ in range(5)]
    caught = False
    for lr, b1, b2, eps, wd in ADAM_CASES:
        tp, tm, tv = _torch_adam_run(p0, grads, lr, b1, b2, eps, wd)
        op, om, ov = _oracle_run(p0, grads, lr, b1, b2, eps, wd, adam=_mut_adam(kind))
        caught |= not (_close(op, tp, 1.0) and _close(om, tm, 1e-3) and _close(ov, tv, 1e-6))
    assert caught


def test_planted_reduce_mistakes_are_caught():
    """Summing in fp16, or dropping the last slice, breaks the exact-sum pin."""
    g = np.random.default_rng(23)
    sl = _edge_fp16(g, (9, 200))
    exact = np.array([float(sum(Fraction(float(sl[k, j])) for k in range(9))) for j in range(200)])

    def fp16_sum(x):
        s = x[0].copy()
        for k in range(1, x.shape[0]):
            s = (s + x[k]).astype(F16)
        return s.astype(F64)

    with np.errstate(over="ignore", invalid="ignore"):
        assert not np.array_equal(fp16_sum(sl), exact)
    assert not np.array_equal(oracle.reduce_owned(sl[:-1]), exact)
    assert np.array_equal(oracle.reduce_owned(sl), exact)


# ----------------------------------------------------------------- loss scaling and clipping
def test_scaler_matches_torch_amp_update():
    """The dynamic loss-scale rule against torch's own scaler update
    (torch._amp_update_scale_), over random overflow sequences."""
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(31)
    for interval in (1, 3, 7):
        flags = g.random(60) < 0.25
        scale, good = 2.0 ** 16, 0
        ts = torch.tensor([scale], dtype=torch.float32)
        tt = torch.zeros(1, dtype=torch.int32)
        for f in flags:
            scale, good = oracle.scaler_update(scale, good, bool(f), 2.0, 0.5, interval)
            torch._amp_update_scale_(ts, tt, torch.tensor([float(f)]), 2.0, 0.5, interval)
            assert scale == float(ts.item()) and good == int(tt.item())


def test_scaler_limits_match_torch():
    """Near the limits: a growth that overflows keeps the scale and still
    resets the count, and a backoff falls to 0 without a floor, as torch's
    update does at its own (float32) limits; the oracle's scale is float64."""
    torch = pytest.importorskip("torch")
    ts = torch.tensor([2.0 ** 127], dtype=torch.float32)
    tt = torch.tensor([2], dtype=torch.int32)
    torch._amp_update_scale_(ts, tt, torch.tensor([0.0]), 2.0, 0.5, 3)
    assert float(ts.item()) == 2.0 ** 127 and int(tt.item()) == 0
    assert oracle.scaler_update(2.0 ** 1023, 2, False, 2.0, 0.5, 3) == (2.0 ** 1023, 0)
    assert oracle.scaler_update(2.0 ** 1022, 2, False, 2.0, 0.5, 3) == (2.0 ** 1023, 0)
    ts = torch.tensor([2.0 ** -149], dtype=torch.float32)
    torch._amp_update_scale_(ts, tt, torch.tensor([1.0]), 2.0, 0.5, 3)
    assert float(ts.item()) == 0.0 and int(tt.item()) == 0
    assert oracle.scaler_update(2.0 ** -1074, 5, True, 2.0, 0.5, 3) == (0.0, 0)
    assert oracle.scaler_update(0.0, 0, True, 2.0, 0.5, 3) == (0.0, 0)


def test_flag_on_unscaled_gradient():
    """The overflow flag is raised by any non-finite unscaled gradient: a
    finite sum with a scale whose reciprocal overflows (2^-1074: 1/L = inf;
    0 after a long backoff) gives g = +-inf, or NaN for a zero sum, and the
    step is flagged; with a normal scale the flag is exactly the non-finite
    sums.  A flag on the sums alone would pass these steps and commit NaN."""
    s = np.array([0.0, 1.5, -3.0], dtype=F64)
    for L in (2.0 ** -1074, 0.0):
        g, ovf, _ = oracle.unscale(s, L)
        assert ovf and np.isnan(g[0]) and np.isposinf(g[1]) and np.isneginf(g[2])
        assert not np.any(~np.isfinite(s))  # the sums themselves are finite
        _, ovf32, _, _ = oracle.clipped_gradient(s, L, 1.0)
        assert ovf32
    g, ovf, _ = oracle.unscale(s, 2.0 ** -1000)  # 1/L = 2^1000: finite
    assert not ovf and g[1] == 1.5 * 2.0 ** 1000
    g, ovf, _ = oracle.unscale(np.array([np.inf, 1.0]), 1024.0)
    assert ovf
    # fp32 overflow of a finite float64 gradient flags the clipped step only
    big = np.array([1.0, 2.0 ** 100], dtype=F64)
    assert not oracle.unscale(big, 2.0 ** -60)[1]
    assert oracle.clipped_gradient(big, 2.0 ** -60, 1.0)[1]


def test_dynamic_scale_backed_off_to_zero_skips():
    """A dynamic scale that backs off to 0 skips every later step and never
    writes the state: t stays 0, the state is bit-identical."""
    g = np.random.default_rng(40)
    p0 = g.standard_normal(64).astype(F32) * 0.02
    sh = oracle.OwnedShard(p0, scale_interval=2, loss_scale=2.0 ** -1074)
    sl = (g.standard_normal((3, 64)) * 10).astype(F16)
    for _ in range(4):
        ovf, _ = sh.step(sl)
        assert ovf
    assert sh.t == 0 and sh.scales == [2.0 ** -1074, 0.0, 0.0, 0.0] and sh.scale == 0.0
    assert np.array_equal(sh.p.view(np.uint32), p0.view(np.uint32))
    assert not np.any(sh.m) and not np.any(sh.v)


def test_clip_matches_torch_clip_grad_norm():
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(32)
    for max_norm in (1e-4, 0.05, 1.0, 1e9):
        sl = (g.standard_normal((5, 3000)) * 0.3 * 1024).astype(F16)
        s = oracle.reduce_owned(sl)
        gg, ovf, sq, coef = oracle.clipped_gradient(s, 1024.0, max_norm)
        assert not ovf
        g32 = (s / 1024.0).astype(F32)
        t = torch.zeros(3000, dtype=torch.float64, requires_grad=True)
        t.grad = torch.tensor(g32.astype(F64))
        norm = torch.nn.utils.clip_grad_norm_([t], max_norm, foreach=False)
        assert float(norm) == pytest.approx(math.sqrt(sq), rel=1e-15)
        assert np.allclose(gg, t.grad.numpy(), rtol=1e-15, atol=0)
        assert coef == (1.0 if max_norm >= math.sqrt(sq) + 1e-6 else pytest.approx(max_norm / (math.sqrt(sq) + 1e-6), rel=1e-15))
    bad = (g.standard_normal((3, 50)) * 100).astype(F16)
    bad[1, 7] = np.inf
    assert oracle.clipped_gradient(oracle.reduce_owned(bad), 1024.0, 1.0)[1]


@pytest.mark.parametrize("wd", [0.0, 0.01])
def test_clipped_adam_matches_torch(wd):
    """float64 state: oracle's clipped steps against torch clip_grad_norm_
    followed by torch Adam/AdamW, 8 steps."""
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(33)
    n, L, max_norm = 400, 1024.0, 0.02
    p0 = g.standard_normal(n) * 0.02
    sh = oracle.OwnedShard(p0, weight_decay=wd, state_dtype=F64, max_grad_norm=max_norm)
    t = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = (torch.optim.AdamW([t], lr=1e-3, weight_decay=wd, foreach=False) if wd else
           torch.optim.Adam([t], lr=1e-3, foreach=False))
    for _ in range(8):
        sl = (g.standard_normal((4, n)) * 1e-3 * L).astype(F16)
        sh.step(sl, L)
        t.grad = torch.tensor((oracle.reduce_owned(sl) / L).astype(F32).astype(F64))
        torch.nn.utils.clip_grad_norm_([t], max_norm, foreach=False)
        opt.step()
    assert min(sh.coefs) < 1.0
    assert np.all(np.abs(sh.p - t.detach().numpy()) <= 1e-12)


def test_dynamic_scaling_sequence():
    """Overflows back the scale off and skip the step; clean runs grow it."""
    g = np.random.default_rng(34)
    n = 64
    sh = oracle.OwnedShard(np.zeros(n, F32), scale_interval=2, loss_scale=1024.0)
    flags = [0, 1, 0, 0, 0, 1, 1, 0, 0]
    for f in flags:
        sl = (g.standard_normal((3, n)) * 1e-3 * sh.scale).astype(F16)
        if f:
            sl[0, 5] = np.nan
        sh.step(sl)
    assert sh.flags == flags and sh.t == flags.count(0)
    assert sh.scales == [1024.0, 1024.0, 512.0, 512.0, 1024.0, 1024.0, 512.0, 256.0, 256.0]
    assert sh.scale == 512.0


@pytest.mark.parametrize("kind", ["eps_inside_sqrt", "max_instead_of_min", "clip_before_unscale"])
def test_planted_clip_mistakes_are_caught(kind):
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(35)
    sl = (g.standard_normal((5, 2000)) * 0.3 * 1024).astype(F16)
    s = oracle.reduce_owned(sl)
    g32 = (s / 1024.0).astype(F32).astype(F64)
    sq = math.fsum((g32 * g32).tolist())
    caught = False
    for max_norm in (1e-3, 1e9):
        if kind == "eps_inside_sqrt":
            c = min(1.0, max_norm / math.sqrt(sq + 1e-6))
            mine = g32 * c
        elif kind == "max_instead_of_min":
            mine = g32 * max(1.0, max_norm / (math.sqrt(sq) + 1e-6))
        else:
            c = min(1.0, max_norm / (math.sqrt(sq) * 1024.0 + 1e-6))
            mine = g32 * c
        t = torch.zeros(2000, dtype=torch.float64, requires_grad=True)
        t.grad = torch.tensor(g32.copy())
        torch.nn.utils.clip_grad_norm_([t], max_norm, foreach=False)
        caught |= not np.allclose(mine, t.grad.numpy(), rtol=1e-15, atol=0)
    assert caught


# ----------------------------------------------------------------- Pos+g+p gather
def _partitioned(numels, nd, align, seed):
    """Tensors of random fp16 values placed into the owners' windows by the
    planner's fragments (tensor_off -> rank, local_off): a placement written
    from the fragment description, independent of the gather's indexing."""
    g = np.random.default_rng(seed)
    tensors = [g.standard_normal(n).astype(F16) for n in numels]
    p = oracle.plan(numels, nd, align)
    windows = [np.zeros(p.part, dtype=F16) for _ in range(nd)]
    for f in p.frags:
        windows[f.rank][f.local_off:f.local_off + f.length] = tensors[f.tensor][f.tensor_off:f.tensor_off + f.length]
    return tensors, p, windows


def _gather_round_trips(gather, trials=60):
    """True if every run of consecutive tensors of random tensor lists,
    placed through the planner's fragments, gathers back unchanged and the
    padding gathers as zeros."""
    g = np.random.default_rng(41)
    for trial in range(trials):
        nt = int(g.integers(1, 12))
        numels = [int(x) for x in g.integers(0, 300, nt)]
        nd = int(g.integers(1, 9))
        align = int(g.choice([8, 16, 64]))
        tensors, p, windows = _partitioned(numels, nd, align, trial)
        offs = np.concatenate([[0], np.cumsum(numels)]).astype(int)
        for i in range(nt):
            for j in range(i + 1, nt + 1):
                got = gather(windows, p.part, int(offs[i]), int(offs[j]))
                want = np.concatenate([tensors[k] for k in range(i, j)])
                if got.shape != want.shape or not np.array_equal(got.view(np.uint16), want.view(np.uint16)):
                    return False
        pad = gather(windows, p.part, p.psi, p.padded)
        if pad.size != p.pad or np.any(pad.view(np.uint16)):
            return False
        # short ranges around every window boundary, against the tensors
        # laid end to end (plus the zero padding)
        flat = np.concatenate(tensors + [np.zeros(p.pad, dtype=F16)])
        for r in range(1, nd):
            b0 = r * p.part
            for lo, hi in ((b0 - 1, b0), (b0 - 1, b0 + 1), (b0 - 2, b0 + 3), (b0, b0 + 1)):
                lo, hi = max(lo, 0), min(hi, p.padded)
                got = gather(windows, p.part, lo, hi)
                if got.shape != (hi - lo,) or not np.array_equal(got.view(np.uint16), flat[lo:hi].view(np.uint16)):
                    return False
    return True


def test_gather_round_trip_through_plan():
    """Every tensor (and every run of consecutive tensors, a 'layer')
    gathered from the windows equals the tensor(s) placed there through the
    planner's fragments; the padding gathers as zeros."""
    assert _gather_round_trips(oracle.gather)


def test_gather_special_cases():
    tensors, p, windows = _partitioned([1000, 3, 2500, 17], 4, 8, 7)
    assert oracle.gather(windows, p.part, 5, 5).size == 0
    r = 2
    lo = r * p.part + 3
    assert np.array_equal(oracle.gather(windows, p.part, lo, lo + 10), windows[r][3:13])
    whole = oracle.gather(windows, p.part, 0, p.padded)
    assert np.array_equal(whole, np.concatenate(windows))
    # a range that starts and ends exactly on window boundaries
    assert np.array_equal(oracle.gather(windows, p.part, p.part, 3 * p.part), np.concatenate(windows[1:3]))


@pytest.mark.parametrize("kind", ["global_offset", "window_of_next_element", "last_piece_dropped"])
def test_planted_gather_mistakes_are_caught(kind):
    def bad_gather(windows, part, lo, hi):
        pieces, f = [], lo
        while f < hi:
            r = (f + 1) // part if kind == "window_of_next_element" else f // part
            off = f if kind == "global_offset" else f - r * part
            take = min(hi, (r + 1) * part) - f  # >= 1: every variant advances
            if not (kind == "last_piece_dropped" and f + take >= hi and f > lo):
                pieces.append(windows[r][max(off, 0):max(off, 0) + take])
            f += take
        return np.concatenate(pieces) if pieces else np.empty(0, F16)

    assert not _gather_round_trips(bad_gather)


def test_clipped_sample_with_window_norm_matches_full_window():
    """A shard holding a sample of a window's elements, given the window's
    sum of g32^2, takes exactly the steps the full window takes at those
    elements (the clip norm is the whole window's)."""
    g = np.random.default_rng(51)
    n, nd = 5000, 4
    master = (g.standard_normal(n) * 0.02).astype(F32)
    idx = np.sort(g.choice(n, 300, replace=False))
    full = oracle.OwnedShard(master, max_grad_norm=0.05, weight_decay=0.01)
    part = oracle.OwnedShard(master[idx], max_grad_norm=0.05, weight_decay=0.01)
    for step in range(4):
        sl = (g.standard_normal((nd, n)) * 1e-3 * 1024).astype(F16)
        full.step(sl, 1024.0)
        part.step(sl[:, idx], 1024.0, window_sumsq=full.sumsq[-1])
        assert part.coefs[-1] == full.coefs[-1] < 1.0
        for a, b in ((part.p, full.p[idx]), (part.m, full.m[idx]), (part.v, full.v[idx])):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    # without the window's norm the sample clips differently
    alone = oracle.OwnedShard(master[idx], max_grad_norm=0.05)
    alone.step(sl[:, idx], 1024.0)
    assert alone.coefs[-1] != full.coefs[-1]


@pytest.mark.parametrize("clip", [0.0, 0.05])
def test_step_chunks_matches_whole_window(clip):
    """The chunked step (column chunks of uneven width, mapped over a thread
    pool) gives the whole-window step's state bit for bit, the same flags,
    scale trajectory and step count, and the same sum of g^2 up to the
    rounding of adding the chunks' exact sums (and through the clip
    coefficient, within one fp32 rounding of the state)."""
    from concurrent.futures import ThreadPoolExecutor
    g = np.random.default_rng(90)
    n, nd = 10007, 5
    p0 = (g.standard_normal(n) * 0.02).astype(F32)
    hp = dict(weight_decay=0.01, max_grad_norm=clip, scale_interval=2, loss_scale=1024.0)
    a, b = oracle.OwnedShard(p0, **hp), oracle.OwnedShard(p0, **hp)
    edges = [0, 1, 8, 4096, 4100, 9000, n]
    with ThreadPoolExecutor(4) as ex:
        for step in range(1, 6):
            sl = (g.standard_normal((nd, n)) * 1e-3 * a.scale).astype(F16)
            if step == 3:
                sl[2, 4099] = np.inf
            ra = a.step(sl)
            chunks = [(lo, hi, sl[:, lo:hi]) for lo, hi in zip(edges, edges[1:])]
            rb = b.step_chunks(chunks, pmap=ex.map)
            assert ra[0] == rb[0]
            if not ra[0]:
                assert rb[1] == pytest.approx(ra[1], rel=1e-15)
            assert a.t == b.t and a.flags == b.flags and a.scales == b.scales
            tol = 0.0 if clip == 0 else 1.2e-7
            for x, y in ((a.p, b.p), (a.m, b.m), (a.v, b.v)):
                d = np.abs(x.astype(F64) - y.astype(F64))
                assert np.all(d <= tol * np.abs(x.astype(F64)))
    assert a.flags == [0, 0, 1, 0, 0]
    with pytest.raises(ValueError):
        b.step_chunks([(0, 8, sl[:, :8]), (9, n, sl[:, 9:])])

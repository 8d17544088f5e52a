"""Host-side checks of the C ABI (no GPU): the library loads and exports every
declared entry point; the C++ planner and memory model agree with the
oracle; argument validation rejects bad calls before any device work."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle
from workloads import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

B = pytest.importorskip("zero_partitioned_mixed_buffer_amd.binding")


def _declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(zero_[a-z0-9_]+)\s*\(", text))
    return names


@pytest.fixture(scope="module")
def L():
    return B.lib()


def test_exports_every_declared_symbol(L):
    declared = _declared_functions()
    assert {"zero_plan_partitions", "zero_reduce_owned", "zero_adam_step", "zero_emit_fp16",
            "zero_memory_model"} <= declared
    for name in declared:
        assert hasattr(L, name), name
    assert declared == set(B.EXPORTED)
    assert L.zero_abi_version() == B.ABI_VERSION == 7


def test_strerror(L):
    for st in (0, -1, -2, -3, -4, -5, -6, -99):
        assert isinstance(L.zero_strerror(st), bytes)


def _cmp_plan(numels, nd, align):
    cp, cf = B.plan_partitions(numels, nd, align)
    op = oracle.plan(numels, nd, align)
    assert (cp["psi"], cp["part"], cp["padded"], cp["pad"]) == (op.psi, op.part, op.padded, op.pad)
    assert cf == [(f.tensor, f.rank, f.tensor_off, f.flat_off, f.local_off, f.length) for f in op.frags]
    return cp


def test_plan_matches_oracle_random():
    g = np.random.default_rng(1)
    for _ in range(400):
        numels = [int(x) for x in g.integers(0, 5000, int(g.integers(0, 8)))]
        _cmp_plan(numels, int(g.integers(1, 70)), int(g.choice([8, 16, 256, 1024])))


@pytest.mark.parametrize("key", sorted(configs.ALL))
def test_plan_matches_oracle_workloads(key):
    w = configs.ALL[key]
    cp = _cmp_plan(list(w.numels), w.nd, 256)
    assert cp["padded"] - cp["pad"] == w.psi


def test_plan_errors(L):
    plan = B.Plan()
    n = C.c_int64()
    one = (C.c_int64 * 1)(10)
    assert L.zero_plan_partitions(one, 1, 0, 256, C.byref(plan), None, 0, C.byref(n)) == B.ZERO_EINVAL
    assert L.zero_plan_partitions(one, 1, 4, 12, C.byref(plan), None, 0, C.byref(n)) == B.ZERO_EINVAL
    assert L.zero_plan_partitions(one, 1, 4, 0, C.byref(plan), None, 0, C.byref(n)) == B.ZERO_EINVAL
    assert L.zero_plan_partitions(None, 1, 4, 256, C.byref(plan), None, 0, C.byref(n)) == B.ZERO_EINVAL
    neg = (C.c_int64 * 1)(-1)
    assert L.zero_plan_partitions(neg, 1, 4, 256, C.byref(plan), None, 0, C.byref(n)) == B.ZERO_EINVAL
    big = (C.c_int64 * 2)(2**62, 2**62)
    assert L.zero_plan_partitions(big, 2, 4, 256, C.byref(plan), None, 0, C.byref(n)) == B.ZERO_EOVERFLOW
    # psi = 2^63 - 1 fits, but padding it to 3 equal shards of 8-aligned size does not
    edge = (C.c_int64 * 2)(2**62, 2**62 - 1)
    assert L.zero_plan_partitions(edge, 2, 3, 8, C.byref(plan), None, 0, C.byref(n)) == B.ZERO_EOVERFLOW
    # two-call pattern: capacity error reports the needed count
    three = (C.c_int64 * 1)(1000)
    assert L.zero_plan_partitions(three, 1, 4, 8, C.byref(plan), None, 0, C.byref(n)) == B.ZERO_ECAPACITY
    assert n.value == 4 and plan.part == 256
    buf = (B.Frag * 4)()
    assert L.zero_plan_partitions(three, 1, 4, 8, C.byref(plan), buf, 4, C.byref(n)) == B.ZERO_OK


def test_memory_model_matches_oracle():
    for psi in (0.0, 1.0, 1.5e9, 7.5e9, 6e10, 124439808.0):
        for nd in (1, 4, 8, 16, 64, 400):
            for stage in range(4):
                for k in (12, 0, 16):
                    c = B.memory_model(psi, nd, stage, k)
                    o = oracle.memory_model(psi, nd, stage, k)
                    for key, val in o.items():
                        if np.isinf(val):
                            assert np.isinf(c[key])
                        else:
                            assert c[key] == pytest.approx(val, rel=1e-15, abs=0), (psi, nd, stage, k, key)


def test_memory_model_printed_values():
    """The C++ model reproduces the printed 7.5B / Nd = 64 numbers."""
    got = [round(B.memory_model(7.5e9, 64, s)["total_bytes"] / 1e9, 1) for s in range(4)]
    assert got == [120.0, 31.4, 16.6, 1.9]
    assert B.memory_model(7.5e9, 64, 3)["reduction_vs_dp"] == 64.0
    assert B.memory_model(7.5e9, 64, 3)["comm_elems"] / B.memory_model(7.5e9, 64, 2)["comm_elems"] == 1.5


def test_memory_model_errors(L):
    r = B.MemReport()
    for args in ((1e9, 0, 1, 12), (1e9, 4, 4, 12), (1e9, 4, -1, 12), (-1.0, 4, 1, 12), (float("nan"), 4, 1, 12),
                 (1e9, 4, 1, -1)):
        assert L.zero_memory_model(*args, C.byref(r)) == B.ZERO_EINVAL
    assert L.zero_memory_model(1e9, 4, 1, 12, None) == B.ZERO_EINVAL


def test_ctl_bytes_round_trip():
    c = B.ctl_from_bytes(B.ctl_init_bytes(512.0))
    c.update(cur=1, t=7, overflow=1, good_steps=3, beta1_pow=0.9 ** 7, skipped=2, sumsq=1.5)
    assert B.ctl_from_bytes(B.ctl_to_bytes(c)) == c
    assert len(B.ctl_to_bytes(c)) == B.CTL_BYTES


def test_ctl_init():
    c = B.ctl_from_bytes(B.ctl_init_bytes(4096.0))
    assert c == {"cur": 0, "t": 0, "overflow": 0, "good_steps": 0, "beta1_pow": 1.0, "beta2_pow": 1.0,
                 "sumsq": 0.0, "skipped": 0, "loss_scale": 4096.0, "clip_coef": 1.0}
    assert B.CTL_BYTES == 64


# Argument validation of the asynchronous calls: every case below fails
# before the library touches the HIP runtime, so it runs without a GPU.
A = 1 << 20  # fake, 16-byte aligned "device" addresses; never dereferenced


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


# fake addresses must never reach a real device, even through a validation bug
no_gpu = pytest.mark.skipif(_gpu_visible(), reason="uses fake device addresses; host-only check")


def _state(base=1 << 24, n=64, ctl=1 << 30):
    return B.adam_state([base, base + 4 * n * 2], [base + 4 * n * 4, base + 4 * n * 6],
                        [base + 4 * n * 8, base + 4 * n * 10], ctl)


@no_gpu
def test_step_validation(L):
    hp = B.adam_hp(1e-3, 0.9, 0.999, 1e-8, 0.0)
    ok_src = B.grad_src(A, 64, 0, 64, 4, 1024.0)
    st = _state()

    def step(src=ok_src, state=st, hpp=hp, ag=None, off=0, ws=1 << 28):
        return L.zero_adam_step(C.byref(src), C.byref(state), C.byref(hpp), ag, off, ws, None)

    assert step(src=B.grad_src(None, 64, 0, 64, 4, 1024.0)) == B.ZERO_EINVAL
    assert step(src=B.grad_src(A, 64, 0, 64, 0, 1024.0)) == B.ZERO_EINVAL
    assert step(src=B.grad_src(A, 64, 0, -1, 4, 1024.0)) == B.ZERO_EINVAL
    assert step(src=B.grad_src(A, 64, 0, 64, 4, 0.0)) == B.ZERO_EINVAL
    assert step(src=B.grad_src(A, 64, 0, 64, 4, float("inf"))) == B.ZERO_EINVAL
    assert step(src=B.grad_src(A, 64, 0, 64, 8192, 1024.0)) == B.ZERO_EINVAL
    assert step(src=B.grad_src(A + 2, 64, 0, 64, 4, 1024.0)) == B.ZERO_EALIGN
    assert step(src=B.grad_src(A, 60, 0, 64, 4, 1024.0)) == B.ZERO_EALIGN
    assert step(src=B.grad_src(A, 64, 4, 64, 4, 1024.0)) == B.ZERO_EALIGN
    assert step(src=B.grad_src(A, 2**62, 0, 64, 4, 1024.0)) == B.ZERO_EOVERFLOW
    for bad in (B.adam_hp(-1, 0.9, 0.999, 1e-8, 0), B.adam_hp(1e-3, 1.0, 0.999, 1e-8, 0),
                B.adam_hp(1e-3, 0.9, 1.0, 1e-8, 0), B.adam_hp(1e-3, 0.9, 0.999, 0.0, 0),
                B.adam_hp(1e-3, 0.9, 0.999, 1e-8, -0.1), B.adam_hp(float("nan"), 0.9, 0.999, 1e-8, 0),
                B.adam_hp(1e-3, 0.9, 0.999, 1e-8, 0, max_grad_norm=1.0),  # clipping needs the 2-pass call
                B.adam_hp(1e-3, 0.9, 0.999, 1e-8, 0, scale_interval=-1),
                B.adam_hp(1e-3, 0.9, 0.999, 1e-8, 0, scale_interval=5, scale_growth=0.0),
                B.adam_hp(1e-3, 0.9, 0.999, 1e-8, 0, scale_interval=5, scale_backoff=float("inf"))):
        assert step(hpp=bad) == B.ZERO_EINVAL
    odd = B.adam_hp(1e-3, 0.9, 0.999, 1e-8, 0)
    odd.reserved = 1
    assert step(hpp=odd) == B.ZERO_EINVAL
    assert step(state=_state(ctl=None)) == B.ZERO_EINVAL
    assert step(state=_state(base=(1 << 24) + 4)) == B.ZERO_EALIGN
    assert step(ws=None) == B.ZERO_EINVAL
    assert step(ws=(1 << 28) + 8) == B.ZERO_EALIGN
    # aliasing: ping and pong master overlap
    alias = B.adam_state([1 << 24, (1 << 24) + 128], [1 << 25, (1 << 25) + 4096],
                         [1 << 26, (1 << 26) + 4096], 1 << 30)
    assert step(state=alias) == B.ZERO_EALIAS
    # aliasing: all-gather window inside the gradient slices
    assert step(ag=A + 64, off=0) == B.ZERO_EALIAS
    # aliasing: state inside the gradient slices
    assert step(state=_state(base=A)) == B.ZERO_EALIAS
    # misaligned all-gather window
    assert step(ag=1 << 29, off=3) == B.ZERO_EALIGN
    # control block: 8-byte aligned, outside every data array
    assert step(state=_state(ctl=(1 << 30) + 4)) == B.ZERO_EALIGN
    assert step(state=_state(ctl=(1 << 24) + 64)) == B.ZERO_EALIAS     # inside master[0]
    assert step(state=_state(ctl=A + 8)) == B.ZERO_EALIAS              # inside the slices
    # workspace outside every data array and the control block
    assert step(ws=A) == B.ZERO_EALIAS
    assert step(ws=(1 << 30) - 256) == B.ZERO_EALIAS                   # covers the control block


@no_gpu
def test_clipped_validation(L):
    hp = B.adam_hp(1e-3, 0.9, 0.999, 1e-8, 0.0, max_grad_norm=1.0)
    src = B.grad_src(A, 64, 0, 64, 4, 1024.0)
    st = _state()

    def step(hpp=hp, gbuf=1 << 27, ag=None, off=0, ws=1 << 28):
        return L.zero_adam_step_clipped(C.byref(src), C.byref(st), C.byref(hpp), gbuf, ag, off, ws, None)

    assert step(gbuf=None) == B.ZERO_EINVAL
    assert step(gbuf=(1 << 27) + 4) == B.ZERO_EALIGN
    assert step(gbuf=1 << 24) == B.ZERO_EALIAS          # overlaps the master
    assert step(gbuf=A) == B.ZERO_EALIAS                # overlaps the gradient slices
    assert step(hpp=B.adam_hp(1e-3, 0.9, 0.999, 1e-8, 0.0)) == B.ZERO_EINVAL  # max_grad_norm must be > 0
    assert step(hpp=B.adam_hp(1e-3, 0.9, 0.999, 1e-8, 0.0, max_grad_norm=float("inf"))) == B.ZERO_EINVAL


@no_gpu
def test_bucket_validation(L):
    hp = B.adam_hp(1e-3, 0.9, 0.999, 1e-8, 0.0)
    src = B.grad_src(A, 16, 0, 16, 4, 1024.0)  # a bucket of 16 elements
    st = _state()                              # a window of 64 elements

    def step(src=src, off=0, window_n=64, phase=B.BUCKET_FIRST, hpp=hp, state=st, ag=None, ag_off=0):
        return L.zero_adam_step_bucket(C.byref(src), C.byref(state), C.byref(hpp), off, window_n, ag, ag_off,
                                       phase, 1 << 28, None)

    assert step(phase=4) == B.ZERO_EINVAL
    assert step(phase=-1) == B.ZERO_EINVAL
    assert step(off=-8) == B.ZERO_EINVAL
    assert step(off=56) == B.ZERO_EINVAL                # 56 + 16 > 64
    assert step(window_n=-1) == B.ZERO_EINVAL
    assert step(off=4) == B.ZERO_EALIGN                 # bucket offsets are multiples of 8
    assert step(off=2**62, window_n=2**62 + 64) == B.ZERO_EOVERFLOW
    assert step(hpp=B.adam_hp(1e-3, 0.9, 0.999, 1e-8, 0.0, max_grad_norm=1.0)) == B.ZERO_EINVAL
    assert step(state=_state(ctl=None)) == B.ZERO_EINVAL
    assert step(state=_state(base=A)) == B.ZERO_EALIAS  # state inside the receive buffer
    assert step(ag=1 << 29, ag_off=4) == B.ZERO_EALIGN  # window start + bucket offset misaligned
    assert step(ag=1 << 29, ag_off=-8) == B.ZERO_EINVAL
    assert L.zero_adam_step_bucket(None, C.byref(st), C.byref(hp), 0, 64, None, 0, 1, 1 << 28, None) == \
        B.ZERO_EINVAL


@no_gpu
def test_gather_validation(L):
    part = 1024
    wins = (C.c_void_p * 4)(1 << 24, 1 << 25, 1 << 26, 1 << 27)

    def g(lo, hi, dst=1 << 29, w=wins, nd=4, prt=part):
        return L.zero_gather_params(w, nd, prt, lo, hi, dst, None)

    assert g(0, 10, w=None) == B.ZERO_EINVAL
    assert g(0, 10, nd=0) == B.ZERO_EINVAL
    assert g(0, 10, prt=0) == B.ZERO_EINVAL
    assert g(-1, 10) == B.ZERO_EINVAL
    assert g(10, 9) == B.ZERO_EINVAL
    assert g(0, 4 * part + 1) == B.ZERO_EINVAL          # past the last window
    assert g(0, 10, dst=None) == B.ZERO_EINVAL
    assert g(0, 10, dst=(1 << 29) + 1) == B.ZERO_EALIGN  # fp16 elements are 2-byte aligned
    assert g(0, 10, prt=2**62) == B.ZERO_EOVERFLOW     # 4 windows of 2^62 elements
    odd = (C.c_void_p * 4)(1 << 24, (1 << 25) + 1, 1 << 26, 1 << 27)
    assert g(part, part + 8, w=odd) == B.ZERO_EALIGN
    holes = (C.c_void_p * 4)(1 << 24, None, 1 << 26, 1 << 27)
    assert g(part - 4, part + 4, w=holes) == B.ZERO_EINVAL  # window 1 is needed
    assert g(0, 2 * part, dst=(1 << 25) + 100) == B.ZERO_EALIAS  # dst inside window 1's piece
    assert g(7, 7) == B.ZERO_OK                          # empty: nothing launched


@no_gpu
def test_other_validation(L):
    src = B.grad_src(A, 64, 0, 64, 4, 1024.0)
    assert L.zero_reduce_owned(C.byref(src), None, None, 1 << 26, 1 << 28, None) == B.ZERO_EINVAL
    assert L.zero_reduce_owned(C.byref(src), A + 8, 1 << 25, 1 << 26, 1 << 28, None) == B.ZERO_EALIGN
    assert L.zero_reduce_owned(C.byref(src), A + 16, 1 << 25, 1 << 26, 1 << 28, None) == B.ZERO_EALIAS
    assert L.zero_reduce_owned(C.byref(src), None, (1 << 25) + 2, 1 << 26, 1 << 28, None) == B.ZERO_EALIGN
    assert L.zero_reduce_owned(C.byref(src), None, 1 << 25, (1 << 26) + 4, 1 << 28, None) == B.ZERO_EALIGN
    assert L.zero_reduce_owned(C.byref(src), None, A + 8, 1 << 26, 1 << 28, None) == B.ZERO_EALIAS
    assert L.zero_reduce_owned(C.byref(src), 1 << 24, (1 << 24) + 64, 1 << 26, 1 << 28, None) == B.ZERO_EALIAS
    assert L.zero_reduce_owned(C.byref(src), None, 1 << 25, (1 << 28) + 1024, 1 << 28, None) == B.ZERO_EALIAS
    assert L.zero_emit_fp16(None, 8, 1 << 29, 0, None) == B.ZERO_EINVAL
    assert L.zero_emit_fp16(1 << 24, -1, 1 << 29, 0, None) == B.ZERO_EINVAL
    assert L.zero_emit_fp16(1 << 24, 8, 1 << 29, 1, None) == B.ZERO_EALIGN
    assert L.zero_emit_fp16(1 << 24, 64, (1 << 24) + 64, 0, None) == B.ZERO_EALIAS
    assert L.zero_emit_fp16(1 << 24, 0, 1 << 29, 0, None) == B.ZERO_OK  # empty: nothing to do
    st = _state()
    assert L.zero_restore_skipped(C.byref(st), -1, 1 << 29, 0, None) == B.ZERO_EINVAL
    assert L.zero_restore_skipped(C.byref(st), 8, None, 0, None) == B.ZERO_EINVAL
    assert L.zero_restore_skipped(C.byref(st), 8, 1 << 29, 1, None) == B.ZERO_EALIGN
    assert L.zero_restore_skipped(C.byref(_state(ctl=(1 << 30) + 4)), 8, 1 << 29, 0, None) == B.ZERO_EALIGN
    assert L.zero_restore_skipped(C.byref(st), 64, 1 << 24, 0, None) == B.ZERO_EALIAS   # window on master[0]
    assert L.zero_restore_skipped(C.byref(st), 64, (1 << 30) - 64, 0, None) == B.ZERO_EALIAS  # covers the ctl


@no_gpu
def test_bucket_list_validation(L):
    hp = B.adam_hp(1e-3, 0.9, 0.999, 1e-8, 0.0)
    st = _state()  # a window of 64 elements

    def call(items, nb=None, window_n=64, phase=B.BUCKET_FIRST, hpp=hp, state=st, ag=None, ag_off=0):
        arr = (B.Bucket * max(len(items), 1))(*[B.Bucket(s, o) for s, o in items])
        return L.zero_adam_step_buckets(arr, len(items) if nb is None else nb, C.byref(state), C.byref(hpp),
                                        window_n, ag, ag_off, phase, 1 << 28, None)

    ok = [(B.grad_src(A, 16, 0, 16, 4, 1024.0), 0), (B.grad_src(A + 4096, 16, 0, 16, 4, 1024.0), 16)]
    assert call(ok, nb=0) == B.ZERO_EINVAL
    assert call(ok, nb=B.MAX_BUCKETS_PER_CALL + 1) == B.ZERO_EINVAL
    assert L.zero_adam_step_buckets(None, 1, C.byref(st), C.byref(hp), 64, None, 0, 1, 1 << 28, None) == \
        B.ZERO_EINVAL
    assert call(ok, phase=4) == B.ZERO_EINVAL
    assert call(ok, window_n=-1) == B.ZERO_EINVAL
    assert call([ok[0], (ok[1][0], 8)]) == B.ZERO_EINVAL           # two buckets cover elements 8..15
    assert call([ok[0], (ok[1][0], 56)]) == B.ZERO_EINVAL          # past the window
    assert call([ok[0], (ok[1][0], 20)]) == B.ZERO_EALIGN          # offsets are multiples of 8
    assert call([ok[0], (ok[1][0], -8)]) == B.ZERO_EINVAL
    assert call([ok[0], (B.grad_src(A + 4096, 16, 0, 16, 5, 1024.0), 16)]) == B.ZERO_EINVAL  # Nd differs
    assert call([ok[0], (B.grad_src(A + 4096, 16, 0, 16, 4, 512.0), 16)]) == B.ZERO_EINVAL   # scale differs
    assert call([ok[0], (B.grad_src(A + 4096, 16, 0, 16, 4, 0.0), 16)]) == B.ZERO_EINVAL
    assert call([ok[0], (B.grad_src(A + 4098, 16, 0, 16, 4, 1024.0), 16)]) == B.ZERO_EALIGN
    assert call([ok[0], (B.grad_src(1 << 24, 16, 0, 16, 4, 1024.0), 16)]) == B.ZERO_EALIAS  # slices on master[0]
    assert call(ok, hpp=B.adam_hp(1e-3, 0.9, 0.999, 1e-8, 0.0, max_grad_norm=1.0)) == B.ZERO_EINVAL
    assert call(ok, state=_state(ctl=None)) == B.ZERO_EINVAL
    assert call(ok, ag=1 << 29, ag_off=4) == B.ZERO_EALIGN
    assert call(ok, ag=A + 64) == B.ZERO_EALIAS                    # the all-gather window on bucket 0's slices
    assert call([(B.grad_src(A, 16, 0, 2 ** 62, 4, 1024.0), 2 ** 62)], window_n=2 ** 62) == B.ZERO_EOVERFLOW


@no_gpu
def test_gather_layers_validation(L):
    part = 1024
    wins = (C.c_void_p * 4)(1 << 24, 1 << 25, 1 << 26, 1 << 27)

    def g(ranges, dsts, w=wins, nd=4, prt=part, nr=None):
        rr = (C.c_int64 * max(2 * len(ranges), 1))(*[x for r in ranges for x in r])
        dd = (C.c_void_p * max(len(dsts), 1))(*dsts)
        return L.zero_gather_layers(w, nd, prt, rr, len(ranges) if nr is None else nr, dd, None)

    assert g([(0, 10)], [1 << 29], nr=-1) == B.ZERO_EINVAL
    assert g([(0, 10)], [1 << 29], w=None) == B.ZERO_EINVAL
    assert g([(0, 10), (10, 5)], [1 << 29, 1 << 30]) == B.ZERO_EINVAL          # hi < lo
    assert g([(0, 10), (0, 4 * part + 1)], [1 << 29, 1 << 30]) == B.ZERO_EINVAL
    assert g([(0, 10), (20, 30)], [1 << 29, None]) == B.ZERO_EINVAL
    assert g([(0, 10), (20, 30)], [1 << 29, (1 << 30) + 1]) == B.ZERO_EALIGN
    assert g([(0, 10), (20, 30)], [1 << 29, (1 << 29) + 8]) == B.ZERO_EALIAS     # destinations overlap
    assert g([(0, 10), (part, part + 8)], [1 << 29, (1 << 25) + 2]) == B.ZERO_EALIAS  # dst on window 1's piece
    assert g([(0, 10)], [1 << 29], prt=2 ** 62) == B.ZERO_EOVERFLOW
    holes = (C.c_void_p * 4)(1 << 24, None, 1 << 26, 1 << 27)
    assert g([(0, 10), (part - 4, part + 4)], [1 << 29, 1 << 30], w=holes) == B.ZERO_EINVAL
    assert g([], []) == B.ZERO_OK                                                # nothing to do
    assert g([(7, 7), (9, 9)], [None, None]) == B.ZERO_OK                        # empty ranges


@no_gpu
def test_calibration_validation(L):
    assert L.zero_calib_triad(1 << 24, 1 << 25, 1 << 26, 1.0, -1, None) == B.ZERO_EINVAL
    assert L.zero_calib_triad(None, 1 << 25, 1 << 26, 1.0, 8, None) == B.ZERO_EINVAL
    assert L.zero_calib_triad(1 << 24, 1 << 25, 1 << 26, 1.0, 0, None) == B.ZERO_OK  # empty
    assert L.zero_calib_triad((1 << 24) + 4, 1 << 25, 1 << 26, 1.0, 8, None) == B.ZERO_EALIGN
    assert L.zero_calib_triad(1 << 24, (1 << 24) + 16, 1 << 26, 1.0, 8, None) == B.ZERO_EALIAS
    assert L.zero_calib_triad(1 << 24, 1 << 25, 1 << 62, 1.0, 2 ** 61, None) == B.ZERO_EOVERFLOW
    src = B.grad_src(A, 64, 0, 64, 4, 1024.0)
    ins = (C.c_void_p * 3)(1 << 24, 1 << 25, 1 << 26)
    outs = (C.c_void_p * 3)(1 << 27, 1 << 28, 1 << 29)
    mix = L.zero_calib_stream_mix
    assert mix(C.byref(B.grad_src(A, 64, 0, 64, 0, 1024.0)), ins, outs, 1 << 30, None) == B.ZERO_EINVAL
    assert mix(C.byref(src), None, outs, 1 << 30, None) == B.ZERO_EINVAL
    assert mix(C.byref(src), ins, outs, None, None) == B.ZERO_EINVAL
    assert mix(C.byref(src), ins, (C.c_void_p * 3)(1 << 27, None, 1 << 29), 1 << 30, None) == B.ZERO_EINVAL
    assert mix(C.byref(src), ins, (C.c_void_p * 3)((1 << 27) + 8, 1 << 28, 1 << 29), 1 << 30, None) == \
        B.ZERO_EALIGN
    assert mix(C.byref(src), ins, outs, (1 << 30) + 2, None) == B.ZERO_EALIGN
    assert mix(C.byref(src), ins, (C.c_void_p * 3)(1 << 24, 1 << 28, 1 << 29), 1 << 30, None) == \
        B.ZERO_EALIAS  # an output on an input
    assert mix(C.byref(src), ins, outs, A + 32, None) == B.ZERO_EALIAS  # fp16 output in the slices
    assert mix(C.byref(src), ins, (C.c_void_p * 3)(1 << 27, (1 << 27) + 128, 1 << 29), 1 << 30, None) == \
        B.ZERO_EALIAS  # two outputs overlap
    assert mix(C.byref(B.grad_src(A, 64, 0, 0, 4, 1024.0)), ins, outs, 1 << 30, None) == B.ZERO_OK  # empty
    rd = L.zero_calib_slice_read
    assert rd(C.byref(B.grad_src(A, 64, 0, 64, 0, 1024.0)), 1 << 30, None) == B.ZERO_EINVAL  # Nd = 0
    assert rd(C.byref(B.grad_src(A, 64, 0, 64, 4, 0.0)), 1 << 30, None) == B.ZERO_EINVAL    # 1/L not finite
    assert rd(C.byref(src), None, None) == B.ZERO_EINVAL
    assert rd(C.byref(src), (1 << 30) + 2, None) == B.ZERO_EALIGN
    assert rd(C.byref(src), A + 32, None) == B.ZERO_EALIAS                                  # sink in the slices
    assert rd(C.byref(B.grad_src(A, 64, 0, 0, 4, 1024.0)), 1 << 30, None) == B.ZERO_OK       # empty


def test_missing_library_fails_loudly(monkeypatch):
    """Without the built library every entry point raises: there is no
    fallback path."""
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "_LIB_PATH", os.path.join(ROOT, "_no_such_dir", "libzero_dp.so"))
    with pytest.raises(RuntimeError, match="not built"):
        B.lib()
    with pytest.raises(RuntimeError, match="not built"):
        B.plan_partitions([10, 20], 2, 8)


def test_product_never_imports_the_oracle():
    """The package and its C sources name no oracle module; the oracle is
    test infrastructure."""
    pkg = os.path.join(ROOT, "zero_partitioned_mixed_buffer_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, fn)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, flags=re.M), fn
                assert "zero_oracle" not in text, fn


def test_binding_checks_torch_arguments():
    """The binding rejects torch tensors whose dtype, layout or extent does
    not fit the call before anything reaches the library (CPU tensors stop
    at the device check, which comes last)."""
    torch = pytest.importorskip("torch")
    h = torch.zeros((3, 64), dtype=torch.float16)
    with pytest.raises(ValueError, match="dtype"):
        B.grad_src(h.float(), 64, 0, 64, 3, 1.0)
    with pytest.raises(ValueError, match="2-D"):
        B.grad_src(h[:, ::2], 32, 0, 32, 3, 1.0)
    with pytest.raises(ValueError, match="rows"):
        B.grad_src(h, 32, 0, 32, 3, 1.0)  # rows are 64 apart, not 32
    with pytest.raises(ValueError, match="rows"):
        B.grad_src(h, 64, 0, 8, 4, 1.0)  # 4 slices asked, 3 held
    with pytest.raises(ValueError, match="columns"):
        B.grad_src(h, 64, 8, 64, 3, 1.0)  # past the end of a row
    with pytest.raises(ValueError, match="device"):
        B.grad_src(h, 64, 0, 64, 3, 1.0)
    # a column view of a wider buffer is fine up to the device check: its
    # rows keep the parent's stride
    with pytest.raises(ValueError, match="device"):
        B.grad_src(torch.zeros((3, 80), dtype=torch.float16)[:, 8:72], 80, 0, 64, 3, 1.0)
    with pytest.raises(ValueError, match="outside"):
        B.emit_fp16(0x1000, 16, torch.zeros(20, dtype=torch.float16), 8)  # an address passes through
    with pytest.raises(ValueError, match="dtype"):
        B.emit_fp16(0x1000, 16, torch.zeros(16, dtype=torch.float32), 0)
    with pytest.raises(ValueError, match="contiguous"):
        B.emit_fp16(0x1000, 16, torch.zeros(64, dtype=torch.float16)[::2], 0)
    with pytest.raises(ValueError, match="dtype"):
        B.adam_state([torch.zeros(8, dtype=torch.float64), 0x1000], [0x2000] * 2, [0x3000] * 2, 0x4000)
    with pytest.raises(ValueError, match="parameter window"):
        B.gather_params([torch.zeros(8, dtype=torch.float16)], 16, 0, 8, 0x1000)

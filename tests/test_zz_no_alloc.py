"""zero_adam_step_noalloc (the step on the library's own per-GPU scratch,
for callers that cannot allocate) against zero_adam_step with a caller's
workspace, through the C ABI on identical inputs: two calls in a row, the
second on a smaller window (a split long window, then a single launch
with fewer workgroups, the scratch still holding the first call's
partials), then a skipped step and a clean one.  State, fp16 window and
control block must be bit-identical; the small window is also checked
against the oracle."""
import numpy as np
import pytest

import oracle
from workloads import gen

from gpu_util import assert_fp16_close, assert_state_close, torch_mod

pytestmark = pytest.mark.gpu


def _pair(torch, n, hp, seed):
    from zero_partitioned_mixed_buffer_amd import OwnedShard
    master = torch.empty(n, dtype=torch.float32, device="cuda")
    gen.device_fill_params(master, seed, 0.02, n)
    shards = [OwnedShard(master, **hp) for _ in range(2)]
    ags = [torch.full((n + 16,), 0x7E5A, dtype=torch.int16, device="cuda") for _ in range(2)]
    for sh, ag in zip(shards, ags):
        sh.emit(ag, 8)
    return master.cpu().numpy(), shards, ags


def _step_both(torch, shards, ags, dsl, n, L):
    from zero_partitioned_mixed_buffer_amd import binding as B
    src = B.grad_src(dsl, dsl.stride(0), 0, n, dsl.shape[0], L)
    a, b = shards
    B.adam_step(src, a.state, a.hp, ags[0], 8, a.workspace)
    B.adam_step_noalloc(src, b.state, b.hp, ags[1], 8)
    torch.cuda.synchronize()
    ca, cb = a.control(), b.control()
    assert ca == cb, (ca, cb)
    for x, y in zip(a.committed(ca), b.committed(cb)):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
    assert torch.equal(ags[0], ags[1])
    return ca


def test_noalloc_matches_workspace_step():
    torch = torch_mod()
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    # call 1: a long window (taken in launches of about 2^24 elements, every
    # workgroup's slot accumulated across them)
    n1, nd1 = (1 << 25) + (1 << 24) + 5003, 4
    _, shards, ags = _pair(torch, n1, hp, 21)
    dsl = torch.empty((nd1, n1 + 5), dtype=torch.float16, device="cuda")
    gen.device_fill_grads(dsl, 21, 1, 1e-3, 1024.0, "normal", n1 + 5)
    c = _step_both(torch, shards, ags, dsl, n1, 1024.0)
    assert c["t"] == 1 and c["overflow"] == 0
    del shards, ags, dsl
    torch.cuda.empty_cache()
    # call 2 on: a smaller window in one launch of fewer workgroups, with
    # dynamic loss scaling; then a skipped step and a clean one
    n2, nd2 = 100003, 3
    hp2 = dict(hp, scale_interval=2, loss_scale=1024.0)
    m0, shards, ags = _pair(torch, n2, hp2, 22)
    ref = oracle.OwnedShard(m0, **hp2)
    stride = (n2 + 7) // 8 * 8
    dsl = torch.zeros((nd2, stride), dtype=torch.float16, device="cuda")
    for step in range(1, 4):
        sl = gen.host_grad_slices(22, step, 0, nd2, n2, 0, n2, 1e-3, ref.scale)
        if step == 2:
            sl[1, n2 // 2] = np.inf
        ovf, sq = ref.step(sl)
        dsl[:, :n2] = torch.from_numpy(sl).cuda()
        c = _step_both(torch, shards, ags, dsl, n2, 1024.0)
        assert c["overflow"] == int(ovf) and c["t"] == ref.t and c["loss_scale"] == ref.scale
        if not ovf:
            assert c["sumsq"] == pytest.approx(sq, rel=1e-12)
        p, m, v = (x.cpu().numpy() for x in shards[1].committed(c))
        for got, want, nm in ((p, ref.p, "p"), (m, ref.m, "m"), (v, ref.v, "v")):
            assert_state_close(got, want, f"noalloc step {step} {nm}")
        bits = ags[1].cpu().numpy().view(np.uint16)
        assert_fp16_close(bits[8:8 + n2], ref.window().view(np.uint16), f"noalloc step {step} window")
        assert np.all(bits[:8] == 0x7E5A) and np.all(bits[8 + n2:] == 0x7E5A)
    assert ref.flags == [0, 1, 0] and ref.t == 2


def test_noalloc_validates_like_the_step():
    """Invalid arguments are rejected before anything is enqueued, with the
    codes zero_adam_step returns."""
    torch = torch_mod()
    import ctypes as C
    from zero_partitioned_mixed_buffer_amd import binding as B
    L = B.lib()
    _, shards, ags = _pair(torch, 1000, dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0), 23)
    dsl = torch.zeros((2, 1000), dtype=torch.float16, device="cuda")
    sh = shards[0]
    ok = B.grad_src(dsl, 1000, 0, 1000, 2, 1024.0)
    stream = torch.cuda.current_stream().cuda_stream
    assert L.zero_adam_step_noalloc(C.byref(ok), C.byref(sh.state), C.byref(sh.hp), ags[0].data_ptr(), 8,
                                    stream) == B.ZERO_OK
    bad = B.grad_src(dsl, 1000, 0, 1000, 2, 0.0)
    assert L.zero_adam_step_noalloc(C.byref(bad), C.byref(sh.state), C.byref(sh.hp), ags[0].data_ptr(), 8,
                                    stream) == B.ZERO_EINVAL
    assert L.zero_adam_step_noalloc(C.byref(ok), C.byref(sh.state), C.byref(sh.hp), ags[0].data_ptr(), 9,
                                    stream) == B.ZERO_EALIGN
    assert L.zero_adam_step_noalloc(None, C.byref(sh.state), C.byref(sh.hp), None, 0, stream) == B.ZERO_EINVAL
    torch.cuda.synchronize()
    assert sh.control()["t"] == 1


def test_noalloc_steps_captured_in_a_graph():
    """The allocation-free step is for code under graph capture: two steps
    captured once and replayed four times, with fresh gradients written
    eagerly and the program synchronising between the replays, must match
    zero_adam_step with a workspace taken eagerly on a twin shard, bit for
    bit, through skipped steps and dynamic loss scaling."""
    torch = torch_mod()
    from zero_partitioned_mixed_buffer_amd import binding as B
    n, nd = 65536 * 2 + 777, 5
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, scale_interval=3, loss_scale=1024.0)
    _, shards, ags = _pair(torch, n, hp, 24)
    eager, graphed = shards
    stride = (n + 7) // 8 * 8
    bufs = [torch.zeros((nd, stride), dtype=torch.float16, device="cuda") for _ in range(2)]
    srcs = [B.grad_src(b, stride, 0, n, nd, 1.0) for b in bufs]

    def fill(step):
        for k, b in enumerate(bufs):
            sl = gen.host_grad_slices(24, 2 * step + k, 0, nd, n, 0, n, 1e-3, 1024.0)
            if (2 * step + k) % 5 == 3:
                sl[k, (step * 7919) % n] = np.inf  # some steps are skipped
            b[:, :n] = torch.from_numpy(sl).cuda()

    def graphed_steps(stream):
        for src in srcs:
            B.adam_step_noalloc(src, graphed.state, graphed.hp, ags[1], 8, stream)

    def eager_steps():
        for src in srcs:
            B.adam_step(src, eager.state, eager.hp, ags[0], 8, eager.workspace)

    fill(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # first calls off the capture (scratch address, launch sizes)
        graphed_steps(side)
    torch.cuda.current_stream().wait_stream(side)
    eager_steps()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        graphed_steps(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(4):
        fill(rep + 1)
        torch.cuda.synchronize()
        graph.replay()
        eager_steps()
        torch.cuda.synchronize()
        ce, cg = eager.control(), graphed.control()
        assert ce == cg, (rep, ce, cg)
        for a, b in zip(eager.committed(ce), graphed.committed(cg)):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), rep
        assert torch.equal(ags[0], ags[1]), rep
    assert ce["t"] + ce["skipped"] == 2 + 2 * 4 and ce["skipped"] > 0

"""The step is capturable in a HIP graph: it allocates nothing, never
synchronises, and decides commit or skip on the device.  A graph of two
steps, replayed several times with fresh gradients written eagerly between
the replays (and the program synchronising in between), must leave the
state, the control block and the all-gather window bit-identical to the
same steps taken eagerly on a twin shard."""
import numpy as np
import pytest

from workloads import gen

from gpu_util import F32, torch_mod

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager_steps():
    torch = torch_mod()
    from zero_partitioned_mixed_buffer_amd import OwnedShard
    n, nd = 65536 * 3 + 1003, 6
    g = np.random.default_rng(41)
    master0 = torch.from_numpy((g.standard_normal(n) * 0.02).astype(F32)).cuda()
    hp = dict(weight_decay=0.01, scale_interval=3, loss_scale=1024.0)
    eager, graphed = OwnedShard(master0, **hp), OwnedShard(master0, **hp)
    stride = (n + 7) // 8 * 8
    bufs = [torch.zeros((nd, stride), dtype=torch.float16, device="cuda") for _ in range(2)]
    ag_e = torch.zeros(n, dtype=torch.float16, device="cuda")
    ag_g = torch.zeros(n, dtype=torch.float16, device="cuda")
    eager.emit(ag_e)
    graphed.emit(ag_g)

    def fill(step):
        for k, b in enumerate(bufs):
            sl = gen.host_grad_slices(41, 2 * step + k, 0, nd, n, 0, n, 1e-3, 1024.0)
            if (2 * step + k) % 5 == 3:
                sl[k, (step * 7919) % n] = np.inf  # some steps are skipped
            b[:, :n] = torch.from_numpy(sl).cuda()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the capture (fills the launch-size cache)
        for b in bufs:
            graphed.step(b, allgather=ag_g)
    torch.cuda.current_stream().wait_stream(side)
    for b in bufs:
        eager.step(b, allgather=ag_e)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for b in bufs:
            graphed.step(b, allgather=ag_g)
    torch.cuda.synchronize()
    for rep in range(4):
        fill(rep)
        torch.cuda.synchronize()
        graph.replay()
        for b in bufs:
            eager.step(b, allgather=ag_e)
        torch.cuda.synchronize()
        ce, cg = eager.control(), graphed.control()
        assert ce == cg, (rep, ce, cg)
        for a, b in zip(eager.committed(ce), graphed.committed(cg)):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), rep
        assert torch.equal(ag_e.view(torch.int16), ag_g.view(torch.int16)), rep
    assert ce["t"] + ce["skipped"] == 2 + 2 * 4 and ce["skipped"] > 0

"""Steps of independent shards on two HIP streams at once.  The library
keeps no state between calls apart from the allocation-free step's scratch
(not used here), so each shard's results match the same steps taken alone,
one after another, bit for bit."""
import numpy as np
import pytest

from workloads import gen

from gpu_util import F32, torch_mod

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)


def _setup(torch, nd, n, seed, steps):
    g = np.random.default_rng(seed)
    master0 = (g.standard_normal(n) * 0.02).astype(F32)
    stride = (n + 7) // 8 * 8  # rows a multiple of 8 elements apart, as the library requires
    slices = []
    for s in range(1, steps + 1):
        t = torch.zeros((nd, stride), dtype=torch.float16, device="cuda")
        t[:, :n] = torch.from_numpy(gen.host_grad_slices(seed, s, 0, nd, n, 0, n, 1e-3, 1024.0)).cuda()
        slices.append(t)
    return master0, slices


def _state(torch, sh, ag):
    ctl = sh.control()
    p, m, v = (x.view(torch.int32).cpu().numpy() for x in sh.committed(ctl))
    return ctl, p, m, v, ag.view(torch.int16).cpu().numpy()


def test_two_streams_match_sequential():
    torch = torch_mod()
    from zero_partitioned_mixed_buffer_amd import OwnedShard
    cases = [(8, 3_000_017, 11, 3), (48, 1_000_003, 12, 3), (3, 2_000_005, 13, 3)]
    steps = 3
    data = [_setup(torch, nd, n, seed, steps) for nd, n, seed, _ in cases]
    streams = [torch.cuda.Stream() for _ in range(2)]  # default priority
    # concurrent: shard i on stream i % 2, launches interleaved step by step
    conc, conc_ag = [], []
    for (nd, n, _, _), (master0, _) in zip(cases, data):
        conc.append(OwnedShard(torch.from_numpy(master0).cuda(), **HP))
        conc_ag.append(torch.zeros(n, dtype=torch.float16, device="cuda"))
    torch.cuda.synchronize()
    for s in range(steps):
        for i, sh in enumerate(conc):
            sh.step(data[i][1][s], 1024.0, allgather=conc_ag[i], stream=streams[i % 2])
    torch.cuda.synchronize()
    # alone, on the current stream, one shard after another
    for i, ((nd, n, _, _), (master0, slices)) in enumerate(zip(cases, data)):
        ref = OwnedShard(torch.from_numpy(master0).cuda(), **HP)
        ref_ag = torch.zeros(n, dtype=torch.float16, device="cuda")
        for s in range(steps):
            ref.step(slices[s], 1024.0, allgather=ref_ag)
        torch.cuda.synchronize()
        c1, p1, m1, v1, a1 = _state(torch, conc[i], conc_ag[i])
        c2, p2, m2, v2, a2 = _state(torch, ref, ref_ag)
        tag = f"nd={nd} n={n}"
        assert c1["t"] == c2["t"] == steps and c1["overflow"] == c2["overflow"] == 0, tag
        assert c1["sumsq"] == c2["sumsq"], tag
        for x, y, nm in ((p1, p2, "master"), (m1, m2, "exp_avg"), (v1, v2, "exp_avg_sq"), (a1, a2, "window")):
            assert np.array_equal(x, y), f"{tag} {nm}"

"""Checkpoint and resume of an owned shard: a run saved after k steps and
resumed into a fresh shard must continue exactly as the uninterrupted run:
the same committed state and all-gather window bit for bit, the same step
count, beta powers, loss scale and clean-step count, through a skipped step
after the resume, with dynamic loss scaling and AdamW."""
import numpy as np
import pytest

from workloads import gen

from gpu_util import F32, torch_mod

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nd,n,k", [(4, 100003, 3), (24, 50021, 2)])
def test_resume_matches_uninterrupted(tmp_path, nd, n, k):
    torch = torch_mod()
    from zero_partitioned_mixed_buffer_amd import OwnedShard
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, scale_interval=2, loss_scale=4096.0)
    g = np.random.default_rng(n)
    master0 = torch.from_numpy((g.standard_normal(n) * 0.02).astype(F32)).cuda()
    a = OwnedShard(master0, **hp)   # uninterrupted
    b = OwnedShard(master0, **hp)   # saved after k steps
    aga = torch.zeros(n, dtype=torch.float16, device="cuda")
    agb = torch.zeros(n, dtype=torch.float16, device="cuda")
    a.emit(aga)
    b.emit(agb)
    stride = (n + 7) // 8 * 8
    dsl = torch.zeros((nd, stride), dtype=torch.float16, device="cuda")
    total = 7

    def slices(step, scale):
        sl = gen.host_grad_slices(n, step, 0, nd, n, 0, n, 1e-3, scale)
        if step == k + 2:  # a skipped step after the resume
            sl[1, n // 3] = np.inf
        dsl[:, :n] = torch.from_numpy(sl).cuda()
        return dsl

    for step in range(1, k + 1):
        sl = slices(step, a.control()["loss_scale"])
        a.step(sl, 1.0, allgather=aga)
        b.step(sl, 1.0, allgather=agb)
    path = str(tmp_path / "shard.npz")
    b.save(path)
    ctl_saved = b.control()
    del b
    c = OwnedShard(torch.zeros(n, dtype=torch.float32, device="cuda"), **hp)
    c.load(path)
    cc = c.control()
    assert cc["cur"] == 0
    assert {kk: v for kk, v in cc.items() if kk != "cur"} == {kk: v for kk, v in ctl_saved.items() if kk != "cur"}
    agc = torch.zeros(n, dtype=torch.float16, device="cuda")
    c.emit(agc)
    assert torch.equal(agc.view(torch.int16), agb.view(torch.int16))
    for step in range(k + 1, total + 1):
        sl = slices(step, a.control()["loss_scale"])
        a.step(sl, 1.0, allgather=aga)
        c.step(sl, 1.0, allgather=agc)
        torch.cuda.synchronize()
        ca, c2 = a.control(), c.control()
        assert {kk: v for kk, v in ca.items() if kk != "cur"} == {kk: v for kk, v in c2.items() if kk != "cur"}
        for x, y in zip(a.committed(ca), c.committed(c2)):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32)), step
        assert torch.equal(aga.view(torch.int16), agc.view(torch.int16)), step
    assert a.control()["skipped"] == 1 and a.control()["t"] == total - 1


def test_load_rejects_a_mismatched_checkpoint(tmp_path):
    torch = torch_mod()
    from zero_partitioned_mixed_buffer_amd import OwnedShard
    a = OwnedShard(torch.zeros(1000, dtype=torch.float32, device="cuda"))
    sd = a.state_dict()
    b = OwnedShard(torch.zeros(1008, dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError, match="float32"):
        b.load_state_dict(sd)
    sd["ctl"] = sd["ctl"][:10]
    with pytest.raises(ValueError, match="control block"):
        a.load_state_dict(sd)

"""Child process of tests/test_gpu_threads.py: in a fresh process (the
library's per-device launch-size cache still empty), four host threads
start together, each stepping its own shard on its own stream; then every
shard is stepped again alone on the current stream and the two must agree
bit for bit.  Prints "threads ok" on success."""
import os
import sys
import threading

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import torch  # noqa: E402  (before the library, as the binding expects)

from workloads import gen  # noqa: E402
from zero_partitioned_mixed_buffer_amd import OwnedShard  # noqa: E402

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
CASES = [(8, 1_000_003), (48, 2_000_005), (3, 500_001), (400, 100_003)]
STEPS = 3


def setup(nd, n, seed):
    g = np.random.default_rng(seed)
    master0 = (g.standard_normal(n) * 0.02).astype(np.float32)
    stride = (n + 7) // 8 * 8
    slices = []
    for s in range(1, STEPS + 1):
        t = torch.zeros((nd, stride), dtype=torch.float16, device="cuda")
        t[:, :n] = torch.from_numpy(gen.host_grad_slices(seed, s, 0, nd, n, 0, n, 1e-3, 1024.0)).cuda()
        slices.append(t)
    return master0, slices


def state(sh, ag):
    ctl = sh.control()
    return [ctl["t"], ctl["overflow"], ctl["sumsq"]] + [
        x.view(torch.int32).cpu().numpy() for x in sh.committed(ctl)] + [ag.view(torch.int16).cpu().numpy()]


def main():
    assert torch.cuda.is_available(), "no GPU visible"
    data = [setup(nd, n, 40 + i) for i, (nd, n) in enumerate(CASES)]
    torch.cuda.synchronize()
    shards = [OwnedShard(torch.from_numpy(m0).cuda(), **HP) for m0, _ in data]
    ags = [torch.zeros(n, dtype=torch.float16, device="cuda") for _, n in CASES]
    torch.cuda.synchronize()
    start = threading.Barrier(len(CASES))
    errors = []

    def work(i):
        try:
            stream = torch.cuda.Stream()  # default priority
            start.wait()
            for s in range(STEPS):
                shards[i].step(data[i][1][s], 1024.0, allgather=ags[i], stream=stream)
            stream.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(f"thread {i}: {e!r}")

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(CASES))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    if errors:
        print("\n".join(errors), flush=True)
        sys.exit(1)
    print("threads done", flush=True)
    for i, ((nd, n), (m0, slices)) in enumerate(zip(CASES, data)):
        ref = OwnedShard(torch.from_numpy(m0).cuda(), **HP)
        ag = torch.zeros(n, dtype=torch.float16, device="cuda")
        for s in range(STEPS):
            ref.step(slices[s], 1024.0, allgather=ag)
        torch.cuda.synchronize()
        a, b = state(shards[i], ags[i]), state(ref, ag)
        assert a[0] == b[0] == STEPS and a[1] == b[1] == 0 and a[2] == b[2], (nd, n, a[:3], b[:3])
        for x, y in zip(a[3:], b[3:]):
            assert np.array_equal(x, y), (nd, n)
        print(f"nd={nd} n={n}: threaded steps match", flush=True)
    print("threads ok", flush=True)


if __name__ == "__main__":
    main()

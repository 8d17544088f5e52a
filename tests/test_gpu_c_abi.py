"""The C ABI driven from plain C: tests/c_abi/zero_step_file (gcc, no
Python or torch in the process) takes owned-shard steps through
zero_emit_fp16 and zero_adam_step (or zero_adam_step_noalloc) on device
memory from the HIP runtime, and every step's committed state, control
block and whole all-gather buffer are compared with the oracle.

Bar (as for the other parity tests): flags, t and the skip count exact;
fp32 master, momentum and variance within relative 1e-5 of the oracle;
the fp16 window within 1 ulp; sum of g^2 within relative 1e-12; the
all-gather buffer outside the window unchanged.
"""
import numpy as np
import pytest

import oracle
from workloads import gen

from c_abi_io import ensure_built, read_output, run, write_input
from gpu_util import SENTINEL, assert_fp16_close, assert_state_close

pytestmark = pytest.mark.gpu

ADAM = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)
ADAMW = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


@pytest.mark.parametrize("n,nd,steps,hp,mode,inf_step", [
    (100003, 5, 3, ADAM, "step", 2),      # prefetch path, a skipped middle step
    (70001, 24, 2, ADAMW, "step", 0),     # chunked visits, AdamW
    (65536 + 13, 3, 3, ADAM, "noalloc", 3),  # the allocation-free entry point, skipped last step
    (0, 4, 2, ADAM, "step", 0),           # empty window
])
def test_c_consumer_matches_oracle(tmp_path, n, nd, steps, hp, mode, inf_step):
    exe = ensure_built()
    print(f"c consumer: n={n} nd={nd} steps={steps} mode={mode}", flush=True)
    seed = 900 + nd
    L = 1024.0
    master0 = gen.host_params(seed, n, 0, n, 0.02)
    # the window is rank 2 of 4 in a flat all-gather buffer; the rest holds a sentinel
    part = (n + 7) // 8 * 8
    ag_off, ag_len = 2 * part, 4 * part + 8
    ag0 = np.full(ag_len, SENTINEL, dtype=np.uint16)
    slices = []
    for step in range(1, steps + 1):
        sl = gen.host_grad_slices(seed, step, 0, nd, n, 0, n, 1e-3, L)
        if step == inf_step and n > 0:
            sl[nd - 1, n // 2] = np.inf
        slices.append(sl)
    fin, fout = str(tmp_path / "in.bin"), str(tmp_path / "out.bin")
    write_input(fin, master0, ag0, ag_off, nd, L, hp, slices)
    r = run(fin, fout, mode)
    assert r.returncode == 0, f"{exe} exited {r.returncode}: {r.stdout}"
    got = read_output(fout, n, ag_len, steps)

    sh = oracle.OwnedShard(master0, **hp)
    for step, (sl, g) in enumerate(zip(slices, got), start=1):
        tag = f"n={n} nd={nd} {mode} step {step}"
        ovf, sq = sh.step(sl, L)
        assert g["overflow"] == int(ovf), tag
        assert g["t"] == sh.t, tag
        assert g["skipped"] == step - sh.t, tag
        assert_state_close(g["p"], sh.p, f"{tag} master")
        assert_state_close(g["m"], sh.m, f"{tag} exp_avg")
        assert_state_close(g["v"], sh.v, f"{tag} exp_avg_sq")
        assert_fp16_close(g["ag"][ag_off:ag_off + n], sh.window().view(np.uint16), f"{tag} fp16 window")
        outside = np.concatenate([g["ag"][:ag_off], g["ag"][ag_off + n:]])
        assert np.all(outside == SENTINEL), f"{tag}: all-gather buffer written outside the window"
        if not ovf:
            assert g["sumsq"] == pytest.approx(sq, rel=1e-12, abs=1e-300), tag

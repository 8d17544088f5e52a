"""The benchmark's bandwidth calibration kernels, checked for what they
write (their traffic is what matters, but every byte they read must reach
an output and nothing outside the outputs may change): STREAM's triad, the
stream-mix kernel with the fused step's streams, and the slice reads alone
(both visit shapes, the prefetch path, split launch pieces, ragged
tails)."""
import numpy as np
import pytest

from gpu_util import torch_mod

pytestmark = pytest.mark.gpu


def test_triad_values():
    torch = torch_mod()
    from zero_partitioned_mixed_buffer_amd import binding as B
    for n in (0, 3, 4 * 1024 * 256 + 4 * 7 + 3, (1 << 22) + 13):
        g = torch.Generator(device="cuda")
        g.manual_seed(n)
        b = torch.randn(max(n, 1), device="cuda", generator=g)
        c = torch.randn(max(n, 1), device="cuda", generator=g)
        a = torch.full((max(n, 1) + 8,), 7.0, device="cuda")
        B.calib_triad(a, b, c, 0.375, n)
        torch.cuda.synchronize()
        want = b[:n].cpu().numpy() + np.float32(0.375) * c[:n].cpu().numpy()
        got = a.cpu().numpy()
        assert np.array_equal(got[:n], want), n
        assert np.all(got[n:] == 7.0)


def _mix_expected(sl, ins):
    nd, n = sl.shape
    g = n // 4
    x = np.zeros(g, dtype=np.uint32)
    if g:
        w = np.ascontiguousarray(sl[:, :4 * g]).view(np.uint32).reshape(nd, g, 2)
        x = np.bitwise_xor.reduce(np.bitwise_xor(w[:, :, 0], w[:, :, 1]), axis=0)
    v = ins[2].view(np.uint32).copy()
    v[:4 * g] ^= np.repeat(x, 4)
    if n > 4 * g:
        v[4 * g:] ^= np.bitwise_xor.reduce(sl[:, 4 * g:].astype(np.uint32), axis=0)
    out16 = (ins[0].view(np.uint32) >> 16).astype(np.uint16)
    return v.view(np.float32), out16


@pytest.mark.parametrize("nd,n", [(1, 1003), (3, 4 * 65536 + 5), (8, 262147), (16, 100003), (17, 300001),
                                  (24, 1000007), (31, 65543), (32, 200003), (48, 1 << 18), (99, 50021),
                                  (32, (1 << 24) + (1 << 22) + 5), (56, 1224 * 2048 - 145),
                                  (40, 1424 * 2048 - 397), (20, 1324 * 1024 - 41)])
def test_stream_mix_values(nd, n):
    torch = torch_mod()
    from zero_partitioned_mixed_buffer_amd import binding as B
    stride = (n + 7) // 8 * 8 + 16
    g = torch.Generator(device="cuda")
    g.manual_seed(nd * 7919 + n)
    sl = torch.randint(-32768, 32767, (nd, stride), dtype=torch.int16, device="cuda", generator=g)
    ins = [torch.randn(n, device="cuda", generator=g) for _ in range(3)]
    outs = [torch.full((n + 8,), 3.0, device="cuda") for _ in range(3)]
    o16 = torch.full((n + 8,), 0x7E5A, dtype=torch.int16, device="cuda")
    src = B.grad_src(sl.view(torch.float16), stride, 8, n, nd, 1.0)
    B.calib_stream_mix(src, ins, [o[:n] for o in outs], o16)
    torch.cuda.synchronize()
    h_sl = sl[:, 8:8 + n].cpu().numpy().view(np.uint16)
    h_in = [t.cpu().numpy() for t in ins]
    v_want, o16_want = _mix_expected(h_sl, h_in)
    got = [o.cpu().numpy() for o in outs]
    assert np.array_equal(got[0][:n].view(np.uint32), h_in[0].view(np.uint32))
    assert np.array_equal(got[1][:n].view(np.uint32), h_in[1].view(np.uint32))
    assert np.array_equal(got[2][:n].view(np.uint32), v_want.view(np.uint32))
    b16 = o16.cpu().numpy().view(np.uint16)
    assert np.array_equal(b16[:n], o16_want)
    assert all(np.all(x[n:] == 3.0) for x in got) and np.all(b16[n:] == 0x7E5A)


@pytest.mark.parametrize("nd,n", [(1, 1003), (3, 4 * 65536 + 5), (8, 262147), (16, 100003), (17, 300001),
                                  (24, 1000007), (31, 65543), (32, 200003), (48, 1 << 18), (99, 50021),
                                  (400, 40961), (32, (1 << 24) + (1 << 22) + 5), (260, (1 << 23) + (1 << 22) + 7),
                                  (56, 1224 * 2048 - 145), (40, 1424 * 2048 - 397), (20, 1324 * 1024 - 41)])
def test_slice_read_values(nd, n):
    """The fold: bits 0-15 the XOR of every slice's fp16 bits at the
    window's even elements, bits 16-31 at its odd elements, XORed into the
    sink's previous value."""
    torch = torch_mod()
    from zero_partitioned_mixed_buffer_amd import binding as B
    stride = (n + 7) // 8 * 8 + 16
    g = torch.Generator(device="cuda")
    g.manual_seed(nd * 104729 + n)
    sl = torch.randint(-32768, 32767, (nd, stride), dtype=torch.int16, device="cuda", generator=g)
    sink = torch.tensor([0x12345678], dtype=torch.int32, device="cuda")
    src = B.grad_src(sl.view(torch.float16), stride, 8, n, nd, 1.0)
    B.calib_slice_read(src, sink)
    torch.cuda.synchronize()
    row = sl[0, 8:8 + n].clone()
    for k in range(1, nd):
        row.bitwise_xor_(sl[k, 8:8 + n])
    h = row.cpu().numpy().view(np.uint16)
    lo = int(np.bitwise_xor.reduce(h[0::2])) if n > 0 else 0
    hi = int(np.bitwise_xor.reduce(h[1::2])) if n > 1 else 0
    want = 0x12345678 ^ (lo | (hi << 16))
    got = int(sink.cpu().numpy().view(np.uint32)[0])
    assert got == want, (hex(got), hex(want))

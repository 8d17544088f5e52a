"""ctypes binding of libzero_dp.so (argument marshalling only).

Every function here converts its arguments (torch tensors or raw device
addresses, Python numbers) into the C structs of include/zero_dp.h and calls
the library; all computation happens inside the library.  If the shared
library is missing, loading raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import List, Optional, Sequence, Tuple

# the in-tree build; ZERO_DP_LIBRARY names another build of the same ABI
# (the host-only sanitizer build that the host-side tests load)
_LIB_PATH = os.environ.get("ZERO_DP_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                              "libzero_dp.so")
_lib = None

ZERO_OK = 0
ZERO_EINVAL = -1
ZERO_EALIGN = -2
ZERO_EOVERFLOW = -3
ZERO_ECAPACITY = -4
ZERO_EALIAS = -5
ZERO_EHIP = -6

EXPORTED = (
    "zero_strerror", "zero_last_hip_error", "zero_abi_version", "zero_plan_partitions",
    "zero_memory_model", "zero_workspace_bytes", "zero_reduce_owned", "zero_ctl_init",
    "zero_adam_step", "zero_adam_step_clipped", "zero_adam_step_bucket", "zero_restore_skipped",
    "zero_emit_fp16", "zero_gather_params", "zero_adam_step_noalloc", "zero_calib_triad",
    "zero_calib_stream_mix", "zero_adam_step_buckets", "zero_gather_layers", "zero_calib_slice_read",
)
ABI_VERSION = 7
BUCKET_FIRST = 1
BUCKET_LAST = 2


class ZeroError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib().zero_strerror(status).decode()
        if status == ZERO_EHIP:
            msg += f" (hipError {lib().zero_last_hip_error()})"
        super().__init__(f"{where}: {msg} [{status}]")
        self.status = status


class Plan(C.Structure):
    _fields_ = [("psi", C.c_int64), ("nd", C.c_int32), ("align", C.c_int32), ("part", C.c_int64),
                ("padded", C.c_int64), ("pad", C.c_int64)]


class Frag(C.Structure):
    _fields_ = [("tensor", C.c_int32), ("rank", C.c_int32), ("tensor_off", C.c_int64),
                ("flat_off", C.c_int64), ("local_off", C.c_int64), ("len", C.c_int64)]


class MemReport(C.Structure):
    _fields_ = [(k, C.c_double) for k in ("params_bytes", "grads_bytes", "optim_bytes", "total_bytes",
                                          "comm_elems", "comm_elems_ring", "reduction_vs_dp")]


class GradSrc(C.Structure):
    _fields_ = [("base", C.c_void_p), ("slice_stride", C.c_int64), ("elem_off", C.c_int64),
                ("n", C.c_int64), ("nd", C.c_int32), ("reserved", C.c_int32), ("loss_scale", C.c_double)]


class StepCtl(C.Structure):
    _fields_ = [("cur", C.c_int32), ("t", C.c_int32), ("overflow", C.c_int32), ("good_steps", C.c_int32),
                ("beta1_pow", C.c_double), ("beta2_pow", C.c_double), ("sumsq", C.c_double),
                ("skipped", C.c_int64), ("loss_scale", C.c_double), ("clip_coef", C.c_double)]


class Bucket(C.Structure):
    _fields_ = [("src", GradSrc), ("win_off", C.c_int64)]


MAX_BUCKETS_PER_CALL = 1024


class AdamState(C.Structure):
    _fields_ = [("master", C.c_void_p * 2), ("exp_avg", C.c_void_p * 2), ("exp_avg_sq", C.c_void_p * 2),
                ("ctl", C.c_void_p)]


class AdamHp(C.Structure):
    _fields_ = [(k, C.c_double) for k in ("lr", "beta1", "beta2", "eps", "weight_decay", "max_grad_norm",
                                          "scale_growth", "scale_backoff")] + \
               [("scale_interval", C.c_int32), ("reserved", C.c_int32)]


def lib():
    """Loads libzero_dp.so from the package directory (raises if absent)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run "
                           "`python -m zero_partitioned_mixed_buffer_amd.build_lib`")
    # torch first: the library's libamdhip64.so.7 then resolves to the HIP
    # runtime torch has loaded, and the process holds one HIP runtime.
    # Loaded the other way round, torch loads a second copy of its own and
    # the library's runtime reports no device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = C.CDLL(_LIB_PATH)
    P = C.c_void_p
    L.zero_strerror.restype = C.c_char_p
    L.zero_strerror.argtypes = [C.c_int]
    L.zero_last_hip_error.restype = C.c_int
    L.zero_abi_version.restype = C.c_int
    L.zero_plan_partitions.argtypes = [C.POINTER(C.c_int64), C.c_int32, C.c_int32, C.c_int32,
                                       C.POINTER(Plan), C.POINTER(Frag), C.c_int64, C.POINTER(C.c_int64)]
    L.zero_memory_model.argtypes = [C.c_double, C.c_int32, C.c_int32, C.c_int32, C.POINTER(MemReport)]
    L.zero_workspace_bytes.restype = C.c_int64
    L.zero_reduce_owned.argtypes = [C.POINTER(GradSrc), P, P, P, P, P]
    L.zero_ctl_init.argtypes = [C.POINTER(StepCtl), C.c_double]
    L.zero_ctl_init.restype = None
    L.zero_adam_step.argtypes = [C.POINTER(GradSrc), C.POINTER(AdamState), C.POINTER(AdamHp), P,
                                 C.c_int64, P, P]
    L.zero_adam_step_noalloc.argtypes = [C.POINTER(GradSrc), C.POINTER(AdamState), C.POINTER(AdamHp), P,
                                         C.c_int64, P]
    L.zero_adam_step_clipped.argtypes = [C.POINTER(GradSrc), C.POINTER(AdamState), C.POINTER(AdamHp), P, P,
                                         C.c_int64, P, P]
    L.zero_adam_step_bucket.argtypes = [C.POINTER(GradSrc), C.POINTER(AdamState), C.POINTER(AdamHp), C.c_int64,
                                        C.c_int64, P, C.c_int64, C.c_int32, P, P]
    L.zero_restore_skipped.argtypes = [C.POINTER(AdamState), C.c_int64, P, C.c_int64, P]
    L.zero_emit_fp16.argtypes = [P, C.c_int64, P, C.c_int64, P]
    L.zero_gather_params.argtypes = [C.POINTER(C.c_void_p), C.c_int32, C.c_int64, C.c_int64, C.c_int64, P, P]
    L.zero_adam_step_buckets.argtypes = [C.POINTER(Bucket), C.c_int32, C.POINTER(AdamState), C.POINTER(AdamHp),
                                         C.c_int64, P, C.c_int64, C.c_int32, P, P]
    L.zero_gather_layers.argtypes = [C.POINTER(C.c_void_p), C.c_int32, C.c_int64, C.POINTER(C.c_int64), C.c_int32,
                                     C.POINTER(C.c_void_p), P]
    L.zero_calib_triad.argtypes = [P, P, P, C.c_float, C.c_int64, P]
    L.zero_calib_stream_mix.argtypes = [C.POINTER(GradSrc), C.POINTER(C.c_void_p), C.POINTER(C.c_void_p), P, P]
    L.zero_calib_slice_read.argtypes = [C.POINTER(GradSrc), P, P]
    for name in ("zero_plan_partitions", "zero_memory_model", "zero_reduce_owned", "zero_adam_step",
                 "zero_adam_step_noalloc", "zero_calib_triad", "zero_calib_stream_mix", "zero_adam_step_buckets",
                 "zero_gather_layers", "zero_calib_slice_read",
                 "zero_adam_step_clipped", "zero_adam_step_bucket", "zero_restore_skipped", "zero_emit_fp16",
                 "zero_gather_params"):
        getattr(L, name).restype = C.c_int
    if L.zero_abi_version() != ABI_VERSION:
        raise RuntimeError("libzero_dp.so ABI version mismatch")
    _lib = L
    return L


def _check(status: int, where: str):
    if status != ZERO_OK:
        raise ZeroError(status, where)


def _ptr(x) -> Optional[int]:
    """Device or host address of a torch tensor, or an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _is_tensor(x) -> bool:
    return x is not None and not isinstance(x, int)


_DTYPE_NAMES: dict = {}


def _dtype_name(t) -> str:
    d = t.dtype
    name = _DTYPE_NAMES.get(d)
    if name is None:
        name = _DTYPE_NAMES[d] = str(d).replace("torch.", "")
    return name


def _check_span(t, off: int, n: int, kinds: Tuple[str, ...], what: str):
    """For a torch tensor argument: dtype one of ``kinds``, elements laid out
    contiguously, [off, off + n) inside the tensor, on a GPU.  Raw addresses
    (ints) and None pass through (the library checks what it can)."""
    if t is None or isinstance(t, int):
        return
    if _dtype_name(t) not in kinds:
        raise ValueError(f"{what}: dtype {t.dtype}, expected one of {kinds}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: tensor must be contiguous")
    if off < 0 or n < 0 or off + n > t.numel():
        raise ValueError(f"{what}: elements [{off}, {off + n}) outside a tensor of {t.numel()}")
    if not t.is_cuda:
        raise ValueError(f"{what}: must be a device tensor")


_F16 = ("float16", "int16")


def _check_ws(ws):
    if ws is not None and not isinstance(ws, int) and (ws.numel() * ws.element_size() < workspace_bytes()
                                                      or not ws.is_cuda):
        raise ValueError(f"workspace: a device tensor of at least {workspace_bytes()} bytes")


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


# ------------------------------------------------------------------ host calls
def plan_partitions(numels: Sequence[int], nd: int, align: int = 256) -> Tuple[dict, List[tuple]]:
    L = lib()
    arr = (C.c_int64 * max(len(numels), 1))(*[int(x) for x in numels])
    plan = Plan()
    n = C.c_int64(0)
    st = L.zero_plan_partitions(arr, len(numels), nd, align, C.byref(plan), None, 0, C.byref(n))
    frags: List[tuple] = []
    if st == ZERO_ECAPACITY or (st == ZERO_OK and n.value > 0):
        buf = (Frag * n.value)()
        st = L.zero_plan_partitions(arr, len(numels), nd, align, C.byref(plan), buf, n.value, C.byref(n))
        frags = [(f.tensor, f.rank, f.tensor_off, f.flat_off, f.local_off, f.len) for f in buf]
    _check(st, "zero_plan_partitions")
    return ({"psi": plan.psi, "nd": plan.nd, "align": plan.align, "part": plan.part,
             "padded": plan.padded, "pad": plan.pad}, frags)


def memory_model(psi: float, nd: int, stage: int, k: int = 12) -> dict:
    r = MemReport()
    _check(lib().zero_memory_model(float(psi), nd, stage, k, C.byref(r)), "zero_memory_model")
    return {name: getattr(r, name) for name, _ in MemReport._fields_}


_ws_bytes: Optional[int] = None


def workspace_bytes() -> int:
    global _ws_bytes
    if _ws_bytes is None:
        _ws_bytes = int(lib().zero_workspace_bytes())
    return _ws_bytes


def ctl_init_bytes(loss_scale: float = 65536.0) -> bytes:
    c = StepCtl()
    lib().zero_ctl_init(C.byref(c), float(loss_scale))
    return bytes(c)


def ctl_from_bytes(b: bytes) -> dict:
    c = StepCtl.from_buffer_copy(b)
    return {name: getattr(c, name) for name, _ in StepCtl._fields_}


def ctl_to_bytes(fields: dict) -> bytes:
    """The control block's bytes from its fields (the inverse of ctl_from_bytes)."""
    c = StepCtl()
    for name, _ in StepCtl._fields_:
        setattr(c, name, fields[name])
    return bytes(c)


CTL_BYTES = C.sizeof(StepCtl)


# ------------------------------------------------------------------ device calls
def grad_src(base, slice_stride: int, elem_off: int, n: int, nd: int, loss_scale: float) -> GradSrc:
    """Gradient source: slice k of the window is base[k, elem_off:elem_off+n].
    A torch ``base`` must be a 2-D fp16 device tensor whose rows are
    ``slice_stride`` elements apart and that holds the whole window."""
    if _is_tensor(base):
        if _dtype_name(base) not in _F16:
            raise ValueError(f"gradient slices: dtype {base.dtype}, expected float16")
        if base.dim() != 2 or base.stride(1) != 1:
            raise ValueError("gradient slices: a 2-D tensor [Nd, stride] with unit element stride")
        if base.shape[0] < nd or (nd > 1 and base.stride(0) != slice_stride):
            raise ValueError(f"gradient slices: {base.shape[0]} rows {base.stride(0)} apart, "
                             f"expected {nd} rows {slice_stride} apart")
        if elem_off < 0 or n < 0 or elem_off + n > base.shape[1]:
            raise ValueError(f"gradient slices: columns [{elem_off}, {elem_off + n}) outside {base.shape[1]}")
        if not base.is_cuda:
            raise ValueError("gradient slices: must be a device tensor")
    return GradSrc(_ptr(base), int(slice_stride), int(elem_off), int(n), int(nd), 0, float(loss_scale))


def adam_state(master: Sequence, exp_avg: Sequence, exp_avg_sq: Sequence, ctl) -> AdamState:
    """Ping-pong state; with torch tensors, each a contiguous fp32 device
    array, and the steps then check that the window fits in all six."""
    s = AdamState()
    arrays = [*master, *exp_avg, *exp_avg_sq]
    for a in arrays:
        _check_span(a, 0, 0, ("float32",), "state array")
    for i in range(2):
        s.master[i] = _ptr(master[i])
        s.exp_avg[i] = _ptr(exp_avg[i])
        s.exp_avg_sq[i] = _ptr(exp_avg_sq[i])
    if _is_tensor(ctl) and (ctl.numel() * ctl.element_size() < CTL_BYTES or not ctl.is_cuda):
        raise ValueError(f"control block: a device tensor of at least {CTL_BYTES} bytes")
    s.ctl = _ptr(ctl)
    if all(_is_tensor(a) for a in arrays):
        s._numel = min(int(a.numel()) for a in arrays)
    return s


def _check_state(state: AdamState, n: int):
    cap = getattr(state, "_numel", None)
    if cap is not None and n > cap:
        raise ValueError(f"state arrays of {cap} elements cannot hold a window of {n}")


def adam_hp(lr: float, beta1: float, beta2: float, eps: float, weight_decay: float,
            max_grad_norm: float = 0.0, scale_interval: int = 0, scale_growth: float = 2.0,
            scale_backoff: float = 0.5) -> AdamHp:
    return AdamHp(float(lr), float(beta1), float(beta2), float(eps), float(weight_decay),
                  float(max_grad_norm), float(scale_growth), float(scale_backoff), int(scale_interval), 0)


def reduce_owned(src: GradSrc, grad_out, overflow, sumsq, workspace, stream=None):
    _check_span(grad_out, 0, src.n, ("float32",), "gradient output")
    _check_span(overflow, 0, 1, ("int32",), "overflow flag")
    _check_span(sumsq, 0, 1, ("float64",), "sum of squares")
    _check_ws(workspace)
    _check(lib().zero_reduce_owned(C.byref(src), _ptr(grad_out), _ptr(overflow), _ptr(sumsq),
                                   _ptr(workspace), _stream(stream)), "zero_reduce_owned")


def adam_step(src: GradSrc, state: AdamState, hp: AdamHp, allgather, allgather_off: int, workspace,
              stream=None):
    _check_state(state, src.n)
    _check_span(allgather, allgather_off, src.n, _F16, "all-gather buffer")
    _check_ws(workspace)
    _check(lib().zero_adam_step(C.byref(src), C.byref(state), C.byref(hp), _ptr(allgather),
                                int(allgather_off), _ptr(workspace), _stream(stream)), "zero_adam_step")


def adam_step_noalloc(src: GradSrc, state: AdamState, hp: AdamHp, allgather, allgather_off: int, stream=None):
    """zero_adam_step on the library's own per-GPU scratch (no workspace)."""
    _check_state(state, src.n)
    _check_span(allgather, allgather_off, src.n, _F16, "all-gather buffer")
    _check(lib().zero_adam_step_noalloc(C.byref(src), C.byref(state), C.byref(hp), _ptr(allgather),
                                        int(allgather_off), _stream(stream)), "zero_adam_step_noalloc")


def adam_step_clipped(src: GradSrc, state: AdamState, hp: AdamHp, grad_buf, allgather, allgather_off: int,
                      workspace, stream=None):
    _check_state(state, src.n)
    _check_span(grad_buf, 0, src.n, ("float32",), "gradient buffer")
    _check_span(allgather, allgather_off, src.n, _F16, "all-gather buffer")
    _check_ws(workspace)
    _check(lib().zero_adam_step_clipped(C.byref(src), C.byref(state), C.byref(hp), _ptr(grad_buf),
                                        _ptr(allgather), int(allgather_off), _ptr(workspace), _stream(stream)),
           "zero_adam_step_clipped")


def adam_step_bucket(src: GradSrc, state: AdamState, hp: AdamHp, win_off: int, window_n: int, allgather,
                     allgather_off: int, phase: int, workspace, stream=None):
    _check_state(state, window_n)
    _check_span(allgather, allgather_off, window_n, _F16, "all-gather buffer")
    _check_ws(workspace)
    _check(lib().zero_adam_step_bucket(C.byref(src), C.byref(state), C.byref(hp), int(win_off), int(window_n),
                                       _ptr(allgather), int(allgather_off), int(phase), _ptr(workspace),
                                       _stream(stream)), "zero_adam_step_bucket")


def bucket_array(buckets: Sequence[Tuple[GradSrc, int]]):
    """The zero_bucket array of (gradient source, window offset) pairs, for
    callers that pass the same buckets step after step."""
    return (Bucket * max(len(buckets), 1))(*[Bucket(src, int(off)) for src, off in buckets]), len(buckets)


def adam_step_buckets(buckets, state: AdamState, hp: AdamHp, window_n: int,
                      allgather, allgather_off: int, phase: int, workspace, stream=None):
    """Several arrived buckets of a bucketed step in one call: ``buckets``
    lists (gradient source, window offset) pairs, or is what bucket_array
    made of such a list."""
    _check_state(state, window_n)
    _check_span(allgather, allgather_off, window_n, _F16, "all-gather buffer")
    _check_ws(workspace)
    arr, nb = buckets if isinstance(buckets, tuple) else bucket_array(buckets)
    _check(lib().zero_adam_step_buckets(arr, nb, C.byref(state), C.byref(hp), int(window_n),
                                        _ptr(allgather), int(allgather_off), int(phase), _ptr(workspace),
                                        _stream(stream)), "zero_adam_step_buckets")


def restore_skipped(state: AdamState, n: int, allgather, allgather_off: int, stream=None):
    _check_state(state, n)
    _check_span(allgather, allgather_off, n, _F16, "all-gather buffer")
    _check(lib().zero_restore_skipped(C.byref(state), int(n), _ptr(allgather), int(allgather_off),
                                      _stream(stream)), "zero_restore_skipped")


def emit_fp16(master, n: int, allgather, allgather_off: int, stream=None):
    _check_span(master, 0, n, ("float32",), "master")
    _check_span(allgather, allgather_off, n, _F16, "all-gather buffer")
    _check(lib().zero_emit_fp16(_ptr(master), int(n), _ptr(allgather), int(allgather_off),
                                _stream(stream)), "zero_emit_fp16")


def gather_params(windows: Sequence, part: int, lo: int, hi: int, dst, stream=None):
    """Flat elements [lo, hi) of the partitioned fp16 parameters into dst;
    ``windows`` lists the Nd owners' windows (tensors, addresses or None)."""
    if part > 0 and hi > lo:  # the windows the range touches (the library rejects a null one)
        for w in windows[max(lo, 0) // part:min((hi - 1) // part + 1, len(windows))]:
            _check_span(w, 0, part, _F16, "parameter window")
    _check_span(dst, 0, max(hi - lo, 0), _F16, "layer buffer")
    arr = (C.c_void_p * max(len(windows), 1))(*[_ptr(w) for w in windows])
    _check(lib().zero_gather_params(arr, len(windows), int(part), int(lo), int(hi), _ptr(dst), _stream(stream)),
           "zero_gather_params")


def gather_layers(windows: Sequence, part: int, ranges: Sequence[Tuple[int, int]], dsts: Sequence, stream=None):
    """Flat ranges [lo, hi) of the partitioned fp16 parameters, range q into
    dsts[q], with the ranges' pieces sharing launches."""
    for (lo, hi), d in zip(ranges, dsts):
        if part > 0 and hi > lo:
            for w in windows[max(lo, 0) // part:min((hi - 1) // part + 1, len(windows))]:
                _check_span(w, 0, part, _F16, "parameter window")
        _check_span(d, 0, max(hi - lo, 0), _F16, "layer buffer")
    if len(ranges) != len(dsts):
        raise ValueError("one destination per range")
    arr = (C.c_void_p * max(len(windows), 1))(*[_ptr(w) for w in windows])
    rng = (C.c_int64 * max(2 * len(ranges), 1))(*[int(x) for r in ranges for x in r])
    dst = (C.c_void_p * max(len(dsts), 1))(*[_ptr(d) for d in dsts])
    _check(lib().zero_gather_layers(arr, len(windows), int(part), rng, len(ranges), dst, _stream(stream)),
           "zero_gather_layers")


# ------------------------------------------------------------------ calibration
def calib_triad(a, b, c, q: float, n: int, stream=None):
    """a[i] = b[i] + q * c[i] over n fp32 elements (STREAM's triad)."""
    for t, what in ((a, "a"), (b, "b"), (c, "c")):
        _check_span(t, 0, n, ("float32",), f"triad {what}")
    _check(lib().zero_calib_triad(_ptr(a), _ptr(b), _ptr(c), float(q), int(n), _stream(stream)),
           "zero_calib_triad")


def calib_stream_mix(src: GradSrc, ins: Sequence, outs: Sequence, out16, stream=None):
    """The fused step's streams with no arithmetic: src's slices and ins[0..2]
    read, outs[0..2] and out16 written, src.n elements each."""
    for t in (*ins, *outs):
        _check_span(t, 0, src.n, ("float32",), "stream-mix array")
    _check_span(out16, 0, src.n, _F16, "stream-mix fp16 output")
    pin = (C.c_void_p * 3)(*[_ptr(t) for t in ins])
    pout = (C.c_void_p * 3)(*[_ptr(t) for t in outs])
    _check(lib().zero_calib_stream_mix(C.byref(src), pin, pout, _ptr(out16), _stream(stream)),
           "zero_calib_stream_mix")


def calib_slice_read(src: GradSrc, sink, stream=None):
    """src's Nd slices read alone in the fused step's schedule; the XOR fold
    of the words read is XORed into sink (a device int32/uint32 word)."""
    if sink is not None and not isinstance(sink, int):
        if _dtype_name(sink) not in ("int32", "uint32") or sink.numel() < 1 or not sink.is_cuda:
            raise ValueError("slice-read sink: one device int32 word expected")
    _check(lib().zero_calib_slice_read(C.byref(src), _ptr(sink), _stream(stream)), "zero_calib_slice_read")

"""Oracle: a plain, slow, CPU implementation of one ZeRO-DP rank's step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's ``cpu_baseline`` leg may import or call this module.  It shares
no code with the HIP library: no kernels, headers, helpers or constants.

What it computes follows the ZeRO pages:

* "ZeRO: partitioning training state across GPUs" (upskillscore concept page),
  section "How it works": the model states of Psi parameters are divided
  among Nd ranks; a gradient partition is summed by its owner
  (reduce-scatter), which steps its own slice of the optimizer state, and
  the new fp16 parameters reach every rank by all-gather.  Memory 16Psi / 4Psi+12Psi/Nd /
  2Psi+14Psi/Nd / 16Psi/Nd; communication 2Psi (stages 0-2) or 3Psi.
* The trishampatil.com engineering dissection of ZeRO (page
  zero-memory-optimization-training-large-models), sections "The Real Problem" (2Psi + 2Psi + K Psi,
  K = 12 for fp32 copy, momentum, variance) and "The Full Progression, in One
  View" (the per-stage table and the 7.5B / Nd = 64 numbers).
* The anthology note on ZeRO (dmarx.github.io note-103), "Assumptions": Adam
  in mixed precision, fp16 params, fp32 param copy, momentum and variance.

Where the pages are silent (the Adam arithmetic, the loss scale, padding,
accumulation precision, the overflow policy) the plainest reading is taken:

* sum:      s_j = G_0[j] + G_1[j] + ... + G_{Nd-1}[j], left to right in
            float64.  Every fp16 value is an integer multiple of 2^-24 below
            2^16 in magnitude, so the float64 sum is exact for Nd < 8192 and
            any order gives the same bits (up to the sign of a zero sum, which
            the left-to-right order fixes).
* unscale:  g = s * (1/L);  overflow = any(!isfinite(g)) over the window
            (every non-finite s gives a non-finite g, and so does a scale
            whose reciprocal overflows, such as a dynamic scale backed off
            to 0); sumsq = sum of g*g, summed exactly and rounded once
            (math.fsum).
* Adam:     bias-corrected Adam with eps added after the square root of the
            corrected second moment, AdamW-style decoupled weight decay
            p * (1 - lr*wd).  All arithmetic in float64, one IEEE operation at
            a time (no fused multiply-add), state stored back as float32:
                m' = b1*m + (1-b1)*g
                v' = b2*v + (1-b2)*(g*g)
                d  = sqrt(v') * (1/sqrt(1-b2^t)) + eps
                q  = m' / d
                p' = p*(1-lr*wd) - (lr/(1-b1^t)) * q
            b1^t and b2^t are running products (t multiplications from 1.0).
* skip:     an overflowing step stores nothing and does not advance t.
* scaler:   dynamic loss scaling (mixed-precision practice): an overflowing
            step multiplies the scale by the backoff factor and resets the
            clean-step count; every `interval` consecutive clean steps
            multiply it by the growth factor (the old scale stays if the
            grown one is not finite) and reset the count.  The gradients of
            a step carry the scale in force when the step starts.
* clip:     global-norm clipping needs the norm before the update, so the
            reduced gradient is materialised as fp32 (g32 = fp32(s * (1/L)),
            overflow = any(!isfinite(g32))),
            its norm is sqrt(sum g32^2) (exact sum, rounded once), and the
            update uses g32 * min(1, max_norm / (norm + 1e-6)) in float64.
* emit:     allgather[off + j] = fp16 round-to-nearest-even of the fp32 master.
* plan:     tensors packed in list order; S = A*ceil(Psi/(Nd*A)); rank r owns
            [r*S, (r+1)*S); the padding sits at the tail of rank Nd-1.
* gather:   with the parameters partitioned too (Pos+g+p; dissection "ZeRO-3"
            and "Forward/Backward Under ZeRO-3": a layer's parameters are
            gathered when the computation reaches it, used, then released),
            flat element f is read from its owner's window, window f // S at
            position f % S; a layer is the flat range of its tensors.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Sequence

import numpy as np

F16 = np.float16
F32 = np.float32
F64 = np.float64


# --------------------------------------------------------------------------
# Partition plan.  Upskillscore "How it works": the optimizer state is
# divided among the Nd ranks and each rank steps its own; trishampatil "ZeRO's Core
# Idea" figure: GPU i holds shard i.  Padding/alignment is a reading (the
# pages do not fix it): equal shards of S = A*ceil(Psi/(Nd*A)) elements.
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Frag:
    tensor: int       # index in the tensor list
    rank: int         # owning rank
    tensor_off: int   # first element inside the tensor
    flat_off: int     # first element inside the flat buffer
    local_off: int    # first element inside the owner's shard
    length: int


@dataclass(frozen=True)
class Plan:
    psi: int
    nd: int
    align: int
    part: int         # S, elements per rank
    padded: int       # Nd * S
    pad: int          # padded - psi
    frags: List[Frag] = field(default_factory=list)

    def rank_offset(self, r: int) -> int:
        return r * self.part


def plan(numels: Sequence[int], nd: int, align: int = 256) -> Plan:
    if nd < 1 or align < 1:
        raise ValueError("nd and align must be >= 1")
    numels = [int(x) for x in numels]
    if any(x < 0 for x in numels):
        raise ValueError("negative tensor size")
    psi = sum(numels)
    # ceil(psi / (nd*align)) in exact integer arithmetic
    units = -(-psi // (nd * align))
    part = align * units
    padded = nd * part
    frags: List[Frag] = []
    flat = 0
    for ti, numel in enumerate(numels):
        done = 0
        while done < numel:
            pos = flat + done
            rank = pos // part
            local = pos - rank * part
            length = min(numel - done, part - local)
            frags.append(Frag(ti, rank, done, pos, local, length))
            done += length
        flat += numel
    return Plan(psi, nd, align, part, padded, padded - psi, frags)


# --------------------------------------------------------------------------
# Memory and communication model.  trishampatil "The Real Problem" (16 Psi =
# 2 Psi + 2 Psi + K Psi, K = 12), sections "ZeRO-1/2/3" and "The Full
# Progression, in One View" (per-stage memory and 2Psi/2Psi/2Psi/3Psi);
# upskillscore "How it works" (same formulas; 3Psi = two parameter
# all-gathers plus the gradient reduce-scatter).
# --------------------------------------------------------------------------
def memory_model(psi: float, nd: int, stage: int, k: int = 12) -> dict:
    if nd < 1 or stage not in (0, 1, 2, 3) or k < 0:
        raise ValueError("bad arguments")
    psi = float(psi)
    params = 2.0 * psi if stage < 3 else 2.0 * psi / nd
    grads = 2.0 * psi if stage < 2 else 2.0 * psi / nd
    optim = k * psi if stage < 1 else k * psi / nd
    total = params + grads + optim
    comm = 2.0 * psi if stage < 3 else 3.0 * psi
    dp_total = (2.0 + 2.0 + k) * psi
    return {
        "params_bytes": params,
        "grads_bytes": grads,
        "optim_bytes": optim,
        "total_bytes": total,
        "comm_elems": comm,
        # a ring collective moves (Nd-1)/Nd of the nominal volume per rank
        "comm_elems_ring": comm * (nd - 1) / nd,
        "reduction_vs_dp": dp_total / total if total > 0 else float("inf"),
    }


# --------------------------------------------------------------------------
# Local half of the reduce-scatter.  Upskillscore "How it works" (Pos+g: a
# gradient partition is summed on its owning rank alone);
# trishampatil "Forward/Backward Under ZeRO-3" (reduce-scatter gradients into
# shards).  Reading: the reduction is an exact sum.
# --------------------------------------------------------------------------
def reduce_owned(slices: np.ndarray) -> np.ndarray:
    """slices: float16 array [Nd, n] (slice k = rank k's contribution to the
    owned window).  Returns the float64 sum over k, left to right."""
    slices = np.asarray(slices)
    if slices.dtype != F16 or slices.ndim != 2 or slices.shape[0] < 1:
        raise ValueError("expected float16 [Nd >= 1, n]")
    s = slices[0].astype(F64)
    with np.errstate(invalid="ignore", over="ignore"):
        for k in range(1, slices.shape[0]):
            s = s + slices[k].astype(F64)
    return s


def _inverse(loss_scale: float) -> float:
    """1/L in float64; a scale of 0 (a dynamic scale backed off that far)
    or one whose reciprocal overflows gives inf."""
    if not (loss_scale >= 0 and math.isfinite(loss_scale)):
        raise ValueError("loss scale must be non-negative and finite")
    with np.errstate(divide="ignore", over="ignore"):
        return float(np.float64(1.0) / np.float64(loss_scale))


def unscale(s: np.ndarray, loss_scale: float):
    """Returns (g, overflow, sumsq).  Overflow is any non-finite unscaled
    gradient (mixed-precision practice cited by the anthology note,
    "Connections": Micikevicius et al.): every non-finite reduced value gives
    one, and so does a scale whose reciprocal is not finite.  sumsq is
    meaningful only without overflow."""
    inv = _inverse(loss_scale)
    with np.errstate(invalid="ignore", over="ignore"):
        g = s * inv
    overflow = bool(np.any(~np.isfinite(g)))
    if overflow:
        return g, True, float("nan")
    with np.errstate(over="ignore"):
        gg = g * g
    return g, False, math.fsum(gg.tolist())


# --------------------------------------------------------------------------
# Mixed-precision Adam.  Anthology note "Assumptions" and trishampatil "The
# Real Problem": fp32 parameter copy, momentum and variance (K = 12).
# --------------------------------------------------------------------------
def step_scalars(lr, beta1, beta2, eps, weight_decay, b1_pow_prev, b2_pow_prev):
    """Scalars of the step being taken, from the running powers of the
    committed steps (b^0 = 1.0).  Each line is one IEEE float64 operation."""
    b1t = b1_pow_prev * beta1
    b2t = b2_pow_prev * beta2
    bc1 = 1.0 - b1t
    bc2 = 1.0 - b2t
    return {
        "b1": float(beta1),
        "b2": float(beta2),
        "omb1": 1.0 - beta1,
        "omb2": 1.0 - beta2,
        "ss": lr / bc1,
        "isb": 1.0 / math.sqrt(bc2),
        "dcy": 1.0 - lr * weight_decay,
        "eps": float(eps),
        "b1t": b1t,
        "b2t": b2t,
    }


def adam_update(p, m, v, g, sc):
    """One Adam/AdamW update of (p, m, v) with unscaled gradient g (float64).

    Arithmetic in float64, one rounded operation per step in the order below;
    results are stored in the dtype of ``p`` (float32 for the 16-byte model,
    float64 when the test suite compares against a float64 library Adam)."""
    store = p.dtype
    p64 = p.astype(F64)
    m64 = m.astype(F64)
    v64 = v.astype(F64)
    g = np.asarray(g, dtype=F64)
    m1 = (sc["b1"] * m64) + (sc["omb1"] * g)
    v1 = (sc["b2"] * v64) + (sc["omb2"] * (g * g))
    d = (np.sqrt(v1) * sc["isb"]) + sc["eps"]
    q = m1 / d
    p1 = (p64 * sc["dcy"]) - (sc["ss"] * q)
    return p1.astype(store), m1.astype(store), v1.astype(store)


def emit(master: np.ndarray) -> np.ndarray:
    """fp16 copy of the fp32 master for the all-gather buffer (upskillscore
    "How it works": the new parameters reach every rank by all-gather).
    IEEE round-to-nearest-even; overflow to +-inf."""
    return np.asarray(master, dtype=F32).astype(F16)


# --------------------------------------------------------------------------
# One rank's owned shard across steps, with the skip/commit rule.
# --------------------------------------------------------------------------
# --------------------------------------------------------------------------
# Dynamic loss scaling and global-norm clipping (the pages cite
# mixed-precision training -- anthology note, "Connections" -- whose loss
# scale these implement; the pages themselves give no policy).
# --------------------------------------------------------------------------
def gather(windows: Sequence[np.ndarray], part: int, lo: int, hi: int) -> np.ndarray:
    """Flat elements [lo, hi) of the partitioned parameters, read from the
    owners' windows (each of `part` elements) one owner at a time."""
    pieces = []
    f = lo
    while f < hi:
        r = f // part
        take = min(hi, (r + 1) * part) - f
        pieces.append(windows[r][f - r * part:f - r * part + take])
        f += take
    if not pieces:
        return np.empty(0, dtype=windows[0].dtype if len(windows) else np.float16)
    return np.concatenate(pieces)


def scaler_update(scale: float, good: int, overflow: bool, growth: float, backoff: float,
                  interval: int):
    """Next (scale, good_steps) after a step with the given overflow flag.
    A growth that would make the scale non-finite keeps the old scale (the
    count still resets); a backoff is applied as it falls, down to 0."""
    if overflow:
        return scale * backoff, 0
    good += 1
    if good == interval:
        grown = scale * growth
        return (grown if math.isfinite(grown) else scale), 0
    return scale, good


CLIP_EPS = 1e-6


def clip_coefficient(sumsq: float, max_norm: float) -> float:
    """min(1, max_norm / (sqrt(sumsq) + 1e-6)), each step one IEEE float64
    operation."""
    c = max_norm / (math.sqrt(sumsq) + CLIP_EPS)
    return c if c < 1.0 else 1.0


def reduced_fp32(s: np.ndarray, loss_scale: float):
    """First pass of the clipping path over reduced values s: returns (g32,
    overflow, sumsq) with g32 = fp32(s * (1/L)) (as an fp32 gradient buffer
    holds it), overflow = any non-finite g32, and sumsq = sum g32^2 summed
    exactly and rounded once (NaN on overflow)."""
    inv = _inverse(loss_scale)
    with np.errstate(invalid="ignore", over="ignore"):
        g32 = (s * inv).astype(F32)
    if bool(np.any(~np.isfinite(g32))):
        return g32, True, float("nan")
    g64 = g32.astype(F64)
    return g32, False, math.fsum((g64 * g64).tolist())


def clipped_gradient(s: np.ndarray, loss_scale: float, max_norm: float, window_sumsq: float = None):
    """Two-pass gradient of the clipping path: returns (g, overflow, sumsq,
    coef) with g the float64 gradient the update uses.  The norm is the
    whole window's: when `s` holds only a sample of the window's elements,
    `window_sumsq` supplies the window's sum of g32^2 (computed elsewhere
    from the same inputs)."""
    g32, overflow, sumsq = reduced_fp32(s, loss_scale)
    if overflow:
        return None, True, float("nan"), float("nan")
    if window_sumsq is not None:
        sumsq = float(window_sumsq)
    coef = clip_coefficient(sumsq, max_norm)
    return g32.astype(F64) * coef, False, sumsq, coef


class OwnedShard:
    """Owned-partition state of one rank: fp32 master/m/v of S elements, the
    committed step count t and the running beta powers.  ``step`` performs
    reduce -> unscale/flag/sumsq -> Adam -> commit (or skip) -> emit."""

    def __init__(self, master: np.ndarray, lr=1e-3, beta1=0.9, beta2=0.999,
                 eps=1e-8, weight_decay=0.0, state_dtype=F32, max_grad_norm=0.0,
                 scale_interval=0, scale_growth=2.0, scale_backoff=0.5, loss_scale=65536.0):
        self.p = np.array(master, dtype=state_dtype, copy=True)
        self.m = np.zeros_like(self.p)
        self.v = np.zeros_like(self.p)
        self.hp = dict(lr=float(lr), beta1=float(beta1), beta2=float(beta2),
                       eps=float(eps), weight_decay=float(weight_decay))
        self.t = 0
        self.b1_pow = 1.0
        self.b2_pow = 1.0
        self.flags: List[int] = []
        self.sumsq: List[float] = []
        self.max_grad_norm = float(max_grad_norm)
        self.scale_interval = int(scale_interval)
        self.scale_growth = float(scale_growth)
        self.scale_backoff = float(scale_backoff)
        self.scale = float(loss_scale)   # used when scale_interval > 0
        self.good_steps = 0
        self.scales: List[float] = []
        self.coefs: List[float] = []

    def window(self) -> np.ndarray:
        return emit(self.p.astype(F32))

    def step(self, slices: np.ndarray, loss_scale: float = None, window_sumsq: float = None):
        """One step over the whole window: ``slices`` [Nd, S].  With dynamic
        scaling (scale_interval > 0) the slices carry self.scale and
        `loss_scale` is ignored.  `window_sumsq`: see clipped_gradient (a
        shard that holds a sample of a window)."""
        slices = np.asarray(slices)
        return self.step_chunks([(0, slices.shape[1], slices)], loss_scale, window_sumsq)

    def step_chunks(self, chunks, loss_scale: float = None, window_sumsq: float = None, pmap=map):
        """The same step with the window's slices given in column chunks:
        ``chunks`` yields (lo, hi, slices[:, lo:hi]) tiling [0, S) in order,
        so that a window too large for one [Nd, S] host array can be
        stepped.  Elements are independent; the only window-wide results
        are the flag (set if any chunk's is) and the sum of g^2: each
        chunk's exact sum, added with math.fsum (one chunk gives the exact
        sum of the window).  ``pmap`` maps the per-chunk work over the
        chunks: the built-in map, or a thread pool's (chunks share
        nothing).  Returns (skipped, sumsq)."""
        dynamic = self.scale_interval > 0
        L = self.scale if dynamic else float(loss_scale)
        clip = self.max_grad_norm > 0
        self.scales.append(L)

        def reduce_chunk(chunk):
            lo, hi, sl = chunk
            s = reduce_owned(sl)
            if s.shape[0] != hi - lo:
                raise ValueError("chunk width mismatch")
            g, ovf, sq = reduced_fp32(s, L) if clip else unscale(s, L)
            return lo, hi, g, ovf, sq

        parts = list(pmap(reduce_chunk, chunks))
        pos = 0
        for lo, hi, _, _, _ in parts:
            if lo != pos:
                raise ValueError("chunks must tile the window in order")
            pos = hi
        if pos != self.p.shape[0]:
            raise ValueError("window size mismatch")
        overflow = any(ovf for _, _, _, ovf, _ in parts)
        sq = float("nan") if overflow else math.fsum(x for _, _, _, _, x in parts)
        coef = 1.0
        if clip:
            if overflow:
                coef = float("nan")
            else:
                if window_sumsq is not None:
                    sq = float(window_sumsq)
                coef = clip_coefficient(sq, self.max_grad_norm)
        self.flags.append(int(overflow))
        self.sumsq.append(sq)
        self.coefs.append(coef)
        if dynamic:
            self.scale, self.good_steps = scaler_update(self.scale, self.good_steps, overflow,
                                                        self.scale_growth, self.scale_backoff,
                                                        self.scale_interval)
        if overflow:
            return True, sq
        sc = step_scalars(self.hp["lr"], self.hp["beta1"], self.hp["beta2"],
                          self.hp["eps"], self.hp["weight_decay"],
                          self.b1_pow, self.b2_pow)
        p1, m1, v1 = (np.empty_like(x) for x in (self.p, self.m, self.v))

        def update_chunk(part):
            lo, hi, g = part[0], part[1], part[2]
            if clip:
                g = g.astype(F64) * coef
            p1[lo:hi], m1[lo:hi], v1[lo:hi] = adam_update(self.p[lo:hi], self.m[lo:hi], self.v[lo:hi], g, sc)

        for _ in pmap(update_chunk, parts):
            pass
        self.p, self.m, self.v = p1, m1, v1
        self.t += 1
        self.b1_pow = sc["b1t"]
        self.b2_pow = sc["b2t"]
        return False, sq

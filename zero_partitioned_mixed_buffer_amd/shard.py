"""Device buffers of one rank's owned shard, allocated with torch.

Holds the ping-pong fp32 Adam state, the device control block and the
workspace, and forwards each step to the library (zero_adam_step, which
also restores the all-gather window of a skipped step).  torch is used
only to allocate device memory and to name the stream.  A shard can be
checkpointed (its committed state and control block) and resumed exactly.
"""
from __future__ import annotations

from typing import Optional

from . import binding as B


class OwnedShard:
    def __init__(self, master, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
                 max_grad_norm=0.0, scale_interval=0, scale_growth=2.0, scale_backoff=0.5,
                 loss_scale=65536.0):
        """max_grad_norm > 0 selects the two-pass clipped step (an fp32
        gradient buffer of n elements is allocated); scale_interval > 0
        selects dynamic loss scaling starting at `loss_scale`."""
        import torch
        if master.dtype != torch.float32 or master.dim() != 1 or not master.is_cuda:
            raise ValueError("master must be a 1-D float32 device tensor")
        dev = master.device
        n = master.numel()
        self.n = n
        self.master = [master.clone(), torch.empty(n, dtype=torch.float32, device=dev)]
        self.exp_avg = [torch.zeros(n, dtype=torch.float32, device=dev) for _ in range(2)]
        self.exp_avg_sq = [torch.zeros(n, dtype=torch.float32, device=dev) for _ in range(2)]
        ctl0 = torch.frombuffer(bytearray(B.ctl_init_bytes(loss_scale)), dtype=torch.uint8)
        self.ctl = ctl0.to(dev)
        self.workspace = torch.zeros(B.workspace_bytes(), dtype=torch.uint8, device=dev)
        self.state = B.adam_state(self.master, self.exp_avg, self.exp_avg_sq, self.ctl)
        self.hp = B.adam_hp(lr, beta1, beta2, eps, weight_decay, max_grad_norm, scale_interval,
                            scale_growth, scale_backoff)
        self.clipped = max_grad_norm > 0
        self.grad_buf = torch.empty(n, dtype=torch.float32, device=dev) if self.clipped else None

    def step(self, slices, loss_scale: float = 1.0, elem_off: int = 0, allgather=None, allgather_off: int = 0,
             stream=None):
        """One step; ``slices`` is a float16 device tensor [Nd, stride] whose
        columns [elem_off, elem_off + n) are the owned window.  With dynamic
        loss scaling the slices carry the control block's scale and
        ``loss_scale`` is ignored."""
        nd, stride = slices.shape[0], slices.stride(0)
        src = B.grad_src(slices, stride, elem_off, self.n, nd, loss_scale)
        if self.clipped:
            # a skipped clipped step leaves the all-gather window untouched
            B.adam_step_clipped(src, self.state, self.hp, self.grad_buf, allgather, allgather_off,
                                self.workspace, stream)
            return
        B.adam_step(src, self.state, self.hp, allgather, allgather_off, self.workspace, stream)

    def step_bucket(self, slices, win_off: int, n: int, phase: int, loss_scale: float = 1.0, elem_off: int = 0,
                    allgather=None, allgather_off: int = 0, stream=None):
        """One bucket of a bucketed step: columns [elem_off, elem_off + n) of
        ``slices`` [Nd, stride] hold the gradients of window elements
        [win_off, win_off + n).  ``phase`` carries B.BUCKET_FIRST on the
        step's first bucket and B.BUCKET_LAST on its last; the last also
        commits the step (restoring the all-gather window if it is skipped)."""
        if self.clipped:
            raise ValueError("a bucketed step cannot clip (the norm is needed before any bucket)")
        nd, stride = slices.shape[0], slices.stride(0)
        src = B.grad_src(slices, stride, elem_off, n, nd, loss_scale)
        B.adam_step_bucket(src, self.state, self.hp, win_off, self.n, allgather, allgather_off, phase,
                           self.workspace, stream)

    def emit(self, allgather, allgather_off: int = 0, stream=None):
        """fp16 copy of the committed master into the all-gather buffer."""
        B.emit_fp16(self.committed()[0], self.n, allgather, allgather_off, stream)

    def control(self) -> dict:
        """Reads the device control block (synchronises with the device)."""
        return B.ctl_from_bytes(bytes(self.ctl.cpu().numpy().tobytes()))

    def committed(self, ctl: Optional[dict] = None):
        cur = (ctl or self.control())["cur"]
        return self.master[cur], self.exp_avg[cur], self.exp_avg_sq[cur]

    # ------------------------------------------------------------ checkpoint
    def state_dict(self) -> dict:
        """The committed state, enough to resume bit for bit: host copies of
        the fp32 master, momentum and variance of the window, and the
        control block (step count, running beta powers, loss scale,
        clean-step count, last flag) as raw bytes.  Synchronises with the
        device."""
        import numpy as np
        ctl = self.control()
        p, m, v = (x.cpu().numpy() for x in self.committed(ctl))
        return {"master": p, "exp_avg": m, "exp_avg_sq": v,
                "ctl": np.frombuffer(bytes(self.ctl.cpu().numpy().tobytes()), dtype=np.uint8).copy()}

    def load_state_dict(self, sd: dict):
        """Restores a state_dict of a window of the same size: the state goes
        to buffer set 0 and the control block is restored with cur = 0, so
        the next step continues exactly where the saved shard left off."""
        import numpy as np
        import torch
        for k in ("master", "exp_avg", "exp_avg_sq"):
            a = np.asarray(sd[k])
            if a.dtype != np.float32 or a.shape != (self.n,):
                raise ValueError(f"{k}: expected float32[{self.n}], got {a.dtype}{list(a.shape)}")
        raw = np.asarray(sd["ctl"], dtype=np.uint8).tobytes()
        if len(raw) != B.CTL_BYTES:
            raise ValueError(f"control block: expected {B.CTL_BYTES} bytes, got {len(raw)}")
        fields = B.ctl_from_bytes(raw)
        fields["cur"] = 0
        dev = self.master[0].device
        for dst, k in ((self.master[0], "master"), (self.exp_avg[0], "exp_avg"), (self.exp_avg_sq[0], "exp_avg_sq")):
            dst.copy_(torch.from_numpy(np.ascontiguousarray(sd[k])).to(dev))
        self.ctl.copy_(torch.frombuffer(bytearray(B.ctl_to_bytes(fields)), dtype=torch.uint8).to(dev))
        torch.cuda.synchronize(dev)

    def save(self, path: str):
        """Writes state_dict() to a .npz file (plain arrays, no pickles)."""
        import numpy as np
        np.savez(path, **self.state_dict())

    def load(self, path: str):
        """Restores a file written by save() (loaded without pickles)."""
        import numpy as np
        with np.load(path, allow_pickle=False) as z:
            self.load_state_dict({k: z[k] for k in ("master", "exp_avg", "exp_avg_sq", "ctl")})

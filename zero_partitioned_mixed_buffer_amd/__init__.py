"""ZeRO-DP owned-partition step for AMD Instinct MI355X (gfx950).

One data-parallel rank's step over the window of the flat parameter buffer
it owns: the local half of the gradient reduce-scatter (exact Nd-way fp16
sum), unscale with inf/NaN detection and sum of squares, mixed-precision
Adam/AdamW on fp32 master/momentum/variance, and the fp16 write into the
flat all-gather buffer.  The computation lives in libzero_dp.so (HIP for
CDNA4, C ABI in include/zero_dp.h); this package only binds it.
"""
from . import binding  # noqa: F401  (loads the library lazily, on first call)
from .binding import (  # noqa: F401
    ZeroError,
    adam_hp,
    adam_state,
    adam_step,
    adam_step_bucket,
    adam_step_clipped,
    emit_fp16,
    gather_params,
    grad_src,
    memory_model,
    plan_partitions,
    reduce_owned,
    restore_skipped,
    workspace_bytes,
)
from .shard import OwnedShard  # noqa: F401

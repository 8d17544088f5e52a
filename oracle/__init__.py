"""CPU reference (oracle) for the ZeRO-DP owned-partition step.

Test infrastructure only: tests, the smoke check and the benchmark's CPU
baseline may import this package; the product path never does.
"""
from .zero_oracle import (  # noqa: F401
    Plan,
    Frag,
    plan,
    memory_model,
    reduce_owned,
    unscale,
    step_scalars,
    adam_update,
    emit,
    OwnedShard,
    scaler_update,
    clip_coefficient,
    clipped_gradient,
    reduced_fp32,
    gather,
)

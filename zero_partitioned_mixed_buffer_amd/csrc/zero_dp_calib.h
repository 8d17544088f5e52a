// Launchers of the bandwidth calibration kernels (zero_dp_calib.hip), which
// the benchmark runs beside the step to measure what HBM attains on the GPU
// it runs on.  None of them is part of the step.  Not part of the public ABI.
#pragma once

#include <cstdint>

#include "zero_dp_internal.h"

namespace zdp {

// STREAM's triad a[i] = b[i] + q * c[i] (fp32).
int launch_calib_triad(float* a, const float* b, const float* c, float q, int64_t n, void* stream);
// The fused step's streams with no arithmetic, in its launch shape.
int launch_calib_mix(const SrcArgs& src, const float* const* in, float* const* out, uint16_t* out16,
                     void* stream);
// The fused step's slice reads alone (its visit order and launch pieces),
// folded into one word XORed into *sink.
int launch_calib_slice_read(const SrcArgs& src, uint32_t* sink, void* stream);

}  // namespace zdp

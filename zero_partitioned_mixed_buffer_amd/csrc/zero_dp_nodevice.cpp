// Launchers of the host-only build of the library, which has no device
// translation unit: it exists to run the host code (planner, memory model,
// the argument validation of every entry point) under the address and
// undefined-behaviour sanitizers.  Every launch reports ZERO_EHIP with
// hipErrorNoDevice (100), so a call that passes validation fails loudly;
// nothing here computes anything.
#include "zero_dp_calib.h"
#include "zero_dp_internal.h"

namespace {

constexpr int kNoDevice = 100;  // hipErrorNoDevice

int no_device() {
    zdp::set_last_hip_error(kNoDevice);
    return ZERO_EHIP;
}

}  // namespace

namespace zdp {

int launch_reduce(const SrcArgs&, float*, int32_t*, double*, const Partials&, void*) { return no_device(); }
int launch_step(const SrcArgs&, const AdamArgs&, const Partials&, void*) { return no_device(); }
int launch_step_clipped(const SrcArgs&, const AdamArgs&, float*, double, const Partials&, void*) {
    return no_device();
}
int launch_bucket(const SrcArgs&, const AdamArgs&, const AdamArgs&, int32_t, const Partials&, void*) {
    return no_device();
}
int launch_buckets(const BucketRun*, int32_t, const SrcArgs&, const AdamArgs&, int32_t, const Partials&, void*) {
    return no_device();
}
int launch_gather(const uint16_t* const*, int64_t, const int64_t*, int32_t, uint16_t* const*, void*) {
    return no_device();
}
int launch_restore(const float*, const float*, const zero_step_ctl*, uint16_t*, int64_t, void*) {
    return no_device();
}
int launch_emit(const float*, uint16_t*, int64_t, void*) { return no_device(); }
int scratch_workspace(void**) { return no_device(); }
int launch_calib_triad(float*, const float*, const float*, float, int64_t, void*) { return no_device(); }
int launch_calib_mix(const SrcArgs&, const float* const*, float* const*, uint16_t*, void*) { return no_device(); }
int launch_calib_slice_read(const SrcArgs&, uint32_t*, void*) { return no_device(); }

}  // namespace zdp

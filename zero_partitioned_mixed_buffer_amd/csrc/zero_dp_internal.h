// Internal declarations shared by the host and device translation units of
// the ZeRO-DP owned-partition library.  Not part of the public ABI.
//
// The host translation unit zero_dp_calls.cpp validates every argument of
// the asynchronous C entry points and fills the kernel argument structs
// below; the device translation unit zero_dp_kernels.hip holds the step's
// kernels and the launchers declared here, which choose grids and enqueue
// the launches.  The calibration launchers are in zero_dp_calib.h.
#pragma once

#include <cstdint>

#include "../../include/zero_dp.h"

namespace zdp {

// Work decomposition of the streaming kernels: a workgroup of 256 lanes
// (four wave64s); each lane owns groups of consecutive elements (the group
// width is a compile-time choice of the device code).
constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;

// Upper bound on workgroups of the reducing kernels (one partial each).
constexpr int kMaxBlocks = 8192;

// Launch pieces of a long window: pieces of `len` elements (a multiple of
// 1024, so every piece starts 16-byte aligned); with `merge`, a remainder
// under half a piece joins the last piece, else it is a piece of its own.
struct Pieces {
    int64_t len;
    bool merge;
};

// The end of the piece of a window of n elements that starts at off.
inline int64_t piece_end(int64_t n, const Pieces& p, int64_t off) {
    const int64_t rest = n - off;
    if (p.merge) return rest < p.len + p.len / 2 ? n : off + p.len;
    return rest <= p.len ? n : off + p.len;
}

// Rounds of the grid the pieces take (round: q elements, one element group
// per lane or one visit per wave; a piece ending in a partial round still
// takes that whole round, most of its waves idle in it).
inline int64_t piece_rounds(int64_t n, const Pieces& p, int64_t q) {
    int64_t r = 0;
    for (int64_t off = 0; off < n;) {
        const int64_t e = piece_end(n, p, off);
        r += (e - off + q - 1) / q;
        off = e;
    }
    return r;
}

// Pieces of about `target` elements: equal ones, unless pieces of whole
// rounds (the remainder joining the last piece, so only the window's last
// launch ends in a partial round) take fewer rounds.  Equal pieces can end
// every launch in a partial round: at 3.1 rounds each, 4 pieces take 16
// rounds where whole-round pieces take 13.  Where both take as many rounds,
// equal pieces measured as fast or faster.
inline Pieces plan_pieces(int64_t n, int64_t target, int64_t q) {
    const int64_t np = (n + target - 1) / target;
    const Pieces eq{((n + np - 1) / np + 1023) / 1024 * 1024, false};
    const int64_t rounds = (target + q / 2) / q;
    const Pieces whole{(rounds > 0 ? rounds : 1) * q, true};
    return piece_rounds(n, whole, q) < piece_rounds(n, eq, q) ? whole : eq;
}

// Elements in one round of a grid of `grid` workgroups: a 4-element group
// per lane (Nd within one chunk), or a visit of `visit_groups` 256-element
// groups per wave.
inline int64_t round_elems(int64_t grid, bool visits, int visit_groups) {
    return visits ? grid * kWaves * 64 * 4 * visit_groups : grid * kBlock * 4;
}

// Workspace layout (bytes): completion counter, the elements a bucketed
// step's buckets have covered, then one slot per workgroup of partial sums
// of g^2 (double) and overflow flags (int32).
constexpr int64_t kWsTicket = 0;
constexpr int64_t kWsRunCount = 64;
constexpr int64_t kWsPartSq = 256;
constexpr int64_t kWsPartFlag = kWsPartSq + 8 * kMaxBlocks;
constexpr int64_t kWsBytes = kWsPartFlag + 4 * kMaxBlocks;

void set_last_hip_error(int e);
bool mul_overflows(int64_t a, int64_t b, int64_t* out);
bool add_overflows(int64_t a, int64_t b, int64_t* out);

// ------------------------------------------------------- kernel arguments
// Workgroup partials in the workspace.
struct Partials {
    uint32_t* ticket;
    double* sq;
    int32_t* flag;
};

// The gradient source of one launch.
struct SrcArgs {
    const uint16_t* win;       // base + elem_off: slice 0 of the window
    int64_t stride;
    int64_t n;
    int32_t nd;
    double inv_scale;          // 1/L of a static loss scale
    const zero_step_ctl* dyn;  // non-null: L = dyn->loss_scale (dynamic loss scaling)
};

// The Adam state, hyperparameters and outputs of a step.
struct AdamArgs {
    float* p[2];
    float* m[2];
    float* v[2];
    zero_step_ctl* ctl;
    double lr, b1, b2, eps, wd;
    uint16_t* ag;  // all-gather window start, or null
    double growth, backoff;  // dynamic loss scaling factors
    int32_t interval;        // > 0: dynamic loss scaling
    // bucketed step: this launch covers one bucket of the window; the
    // per-workgroup partials accumulate in their slots across the step's
    // launches and the elements covered in run_count
    int32_t bucket;          // 0: whole-window step; else ZERO_BUCKET_FIRST/LAST bits | 4
    int64_t window_n;        // elements the step's buckets must cover
    int64_t* run_count;
};

// ------------------------------------------------------------- launchers
// Every argument has been validated by the caller.  Each returns ZERO_OK
// or ZERO_EHIP (with the HIP error recorded by set_last_hip_error).  A
// build without a device translation unit links versions that return
// ZERO_EHIP for every launch.

// The decomposed reduce (zero_reduce_owned).
int launch_reduce(const SrcArgs& src, float* grad_out, int32_t* overflow, double* sumsq, const Partials& ws,
                  void* stream);
// The fused pass(es) over the whole window, then the commit (zero_adam_step).
int launch_step(const SrcArgs& src, const AdamArgs& a, const Partials& ws, void* stream);
// The clipped step's two passes and its commit (zero_adam_step_clipped).
int launch_step_clipped(const SrcArgs& src, const AdamArgs& a, float* grad_buf, double max_norm,
                        const Partials& ws, void* stream);
// One bucket (`a` holds the bucket's state and window pointers, `whole`
// the window's, for the commit after the last bucket).
int launch_bucket(const SrcArgs& src, const AdamArgs& a, const AdamArgs& whole, int32_t phase,
                  const Partials& ws, void* stream);
// One arrived bucket of a bucketed step: its slices (row stride `stride`,
// n elements) and its first window element.
struct BucketRun {
    const uint16_t* win;
    int64_t stride;
    int64_t n;
    int64_t win_off;
};
// Several buckets of one step in as few launches as fit (`a` holds the
// window's state and all-gather pointers and window_n; `common` the slice
// count and the loss scale); the commit follows when phase has LAST.
int launch_buckets(const BucketRun* runs, int32_t nruns, const SrcArgs& common, const AdamArgs& a,
                   int32_t phase, const Partials& ws, void* stream);
// The flat ranges [ranges[2q], ranges[2q+1]) of the windows into dsts[q]
// (zero_gather_params, zero_gather_layers).
int launch_gather(const uint16_t* const* windows, int64_t part, const int64_t* ranges, int32_t nranges,
                  uint16_t* const* dsts, void* stream);
// The window re-emit of a skipped step, decided on the device.
int launch_restore(const float* p0, const float* p1, const zero_step_ctl* ctl, uint16_t* ag, int64_t n,
                   void* stream);
// allgather window = fp16(master).
int launch_emit(const float* master, uint16_t* ag, int64_t n, void* stream);
// The current device's address of the library-held scratch that
// zero_adam_step_noalloc uses as its workspace (kWsBytes bytes), or
// ZERO_ECAPACITY if a step on this device would need more workgroup slots.
int scratch_workspace(void** ws);

}  // namespace zdp

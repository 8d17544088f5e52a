// Internal declarations shared by the host and device translation units of
// the ZeRO-DP owned-partition library.  Not part of the public ABI.
#pragma once

#include <cstdint>

namespace zdp {

// Work decomposition of the streaming kernels: a workgroup of 256 lanes
// (four wave64s); each lane owns groups of consecutive elements (the group
// width is a compile-time choice of the device code).
constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;

// Upper bound on workgroups of the reducing kernels (one partial each).
constexpr int kMaxBlocks = 8192;

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

}  // namespace zdp

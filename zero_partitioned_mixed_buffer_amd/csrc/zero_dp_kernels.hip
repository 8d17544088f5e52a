// Device side of the ZeRO-DP owned-partition step for CDNA4 (gfx950).
//
// One rank's step over its owned window, fused into a single streaming pass
// (upskillscore "How it works": the owner reduces its gradient partition by
// reduce-scatter, steps its own slice of the optimizer state, and the new
// parameters reach every rank by all-gather; trishampatil
// "Forward/Backward Under ZeRO-3": reduce-scatter -> update shard ->
// all-gather):
//
//   s_j  = G_0[j] + G_1[j] + ... + G_{Nd-1}[j]       exact in float64
//   g_j  = s_j * (1/L);  flag |= !isfinite(g_j);  sumsq += g_j^2
//   m'   = b1*m + (1-b1)*g          v' = b2*v + (1-b2)*(g*g)
//   d    = sqrt(v') * (1/sqrt(1-b2^t)) + eps          q = m'/d
//   p'   = p*(1-lr*wd) - (lr/(1-b1^t))*q
//   fp32 stores of p', m', v';  allgather[off+j] = fp16(fp32(p'))
//
// The flag tests g, not s: a non-finite s always gives a non-finite g, and
// so does a loss scale whose reciprocal overflows (a dynamic scale backed
// off to 0 or to a subnormal), which then skips the step instead of
// committing inf/NaN state.  Where g is stored as fp32 (the reduce pass),
// the fp32 value is tested, which also catches an fp32 overflow.
//
// Every floating-point operation above is one IEEE float64 operation with
// round-to-nearest-even; contraction into fused multiply-adds is disabled
// for this file, and division and square root are the correctly rounded
// sequences, so the results are reproducible bit for bit.  The fp16 values
// are integer multiples of 2^-24 below 2^16, so float64 holds the Nd-way sum
// exactly for Nd < 2^13 and the summation order does not matter.
//
// The work is HBM-bound (about 1 flop per byte), so there is no matrix-core
// work here; what matters is 16-byte coalesced vector access, enough bytes
// in flight per CU, and a single pass over every array.
//
// Kernels:
//   fused_step_kernel      the step above over the whole window, one piece
//                          of a long window, or one bucket (workgroup
//                          partials in the workspace for commit_kernel)
//   reduce_owned_kernel    the sum / unscale / flag / sum of g^2 alone; the
//                          first pass of the clipped step (fp32 g stored)
//   clipped_update_kernel  the clipped step's second pass: g * min(1,
//                          max_norm / (norm + 1e-6)), update, emit
//   commit_kernel          the launch after a step's passes: sums the
//                          workgroup partials in a fixed order, commits or
//                          skips the step in the control block, re-emits
//                          the window of a skipped fused step
//   emit_kernel, restore_kernel   fp16 window from the fp32 master (initial
//                          fill; re-emit on demand)
//   copy_f16_kernel        a Pos+g+p layer gather: the layer's pieces of up
//                          to 16 owners' windows in one launch (trishampatil
//                          "ZeRO-3": parameters gathered on demand, used,
//                          released)
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>

#include "../../include/zero_dp.h"
#include "zero_dp_internal.h"

#pragma clang fp contract(off)

// Device scratch of zero_adam_step_noalloc: the layout of a caller's
// workspace (one partial and one flag per workgroup, for up to
// zdp::kMaxBlocks workgroups, and the element count of a split window),
// one copy per GPU for the life of the process.  Host code never uses this
// name as an address: the device address comes from hipGetSymbolAddress,
// once per device with that device current (scratch_addr below).
static __device__ __align__(256) unsigned char scratch[zdp::kWsBytes];

namespace {

using zdp::AdamArgs;
using zdp::kBlock;
using zdp::kWaves;
using zdp::Partials;
using zdp::SrcArgs;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// Elements per lane per group: one 8-byte fp16 vector and one 16-byte fp32
// vector per array, so every load and store instruction of a wave covers a
// contiguous 512 B or 1 KiB.  (8 per lane splits the fp32 arrays over two
// half-line instructions; measured slower.)
constexpr int kV = 4;
typedef uint32_t hvec __attribute__((ext_vector_type(kV / 2)));  // kV fp16 values
typedef float fvec __attribute__((ext_vector_type(kV)));         // kV fp32 values

// ---------------------------------------------------------------- helpers
__device__ __forceinline__ double h2d(const hvec& w, int e) {
    const half2_t h = __builtin_bit_cast(half2_t, static_cast<uint32_t>(w[e >> 1]));
    return static_cast<double>(static_cast<float>((e & 1) ? h.y : h.x));
}

__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
    half2_t h;
    h.x = static_cast<_Float16>(a);  // IEEE round-to-nearest-even
    h.y = static_cast<_Float16>(b);
    return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ void init_v(double (&acc)[kV], const hvec& w) {
#pragma unroll
    for (int e = 0; e < kV; ++e) acc[e] = h2d(w, e);
}

__device__ __forceinline__ void add_v(double (&acc)[kV], const hvec& w) {
#pragma unroll
    for (int e = 0; e < kV; ++e) acc[e] += h2d(w, e);
}

__device__ __forceinline__ hvec pack_v(const float (&x)[kV]) {
    hvec h;
#pragma unroll
    for (int i = 0; i < kV / 2; ++i) h[i] = pack_f16(x[2 * i], x[2 * i + 1]);
    return h;
}

// Tuning knobs (compile-time; the defaults are the measured best on gfx950).
#ifndef ZDP_UNROLL
#define ZDP_UNROLL 16  // Nd up to which a group's slice loads are all issued together
#endif
#ifndef ZDP_NT_LOAD
#define ZDP_NT_LOAD 1  // streaming (non-temporal) loads of slices and state
#endif
#ifndef ZDP_NT_STORE
#define ZDP_NT_STORE 1  // streaming (non-temporal) stores of state and fp16
#endif
#ifndef ZDP_BPC
#define ZDP_BPC 1  // >0: at most this many workgroups per CU (fused step)
#endif
#ifndef ZDP_BPC_REDUCE
#define ZDP_BPC_REDUCE 1  // the same cap for the reduce pass
#endif
#ifndef ZDP_BPC_CLIP
#define ZDP_BPC_CLIP 1  // the same cap for the clipped update pass
#endif
#ifndef ZDP_BPC_COPY
#define ZDP_BPC_COPY 1  // workgroups per CU of the parameter gather copy
#endif
#ifndef ZDP_XCD_REMAP
#define ZDP_XCD_REMAP 1  // 1: consecutive logical workgroups on one XCD
#endif

template <typename T>
__device__ __forceinline__ T ldg(const T* p) {
#if ZDP_NT_LOAD
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}

template <typename T>
__device__ __forceinline__ void stg(T* p, const T& v) {
#if ZDP_NT_STORE
    __builtin_nontemporal_store(v, p);
#else
    *p = v;
#endif
}

__device__ __forceinline__ hvec ldh(const uint16_t* p) { return ldg(reinterpret_cast<const hvec*>(p)); }

// Nd-way sum of one window element, slices in index order (ragged tails).
__device__ __forceinline__ double sum_slices1(const uint16_t* p, int64_t stride, int nd) {
    double s = static_cast<double>(static_cast<float>(*reinterpret_cast<const _Float16*>(p)));
    for (int k = 1; k < nd; ++k)
        s += static_cast<double>(
            static_cast<float>(*reinterpret_cast<const _Float16*>(p + static_cast<int64_t>(k) * stride)));
    return s;
}

__device__ __forceinline__ bool finite(double x) { return __builtin_isfinite(x); }

// Deterministic workgroup reduction of one double and one flag; the result
// is valid in thread 0.
__device__ __forceinline__ void block_reduce(double& sq, int& flag) {
    __shared__ double s_sq[kWaves];
    __shared__ int s_flag[kWaves];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        sq += __shfl_xor(sq, o);
        flag |= __shfl_xor(flag, o);
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        s_sq[wave] = sq;
        s_flag[wave] = flag;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = s_sq[0];
        int f = s_flag[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) {
            t += s_sq[w];
            f |= s_flag[w];
        }
        sq = t;
        flag = f;
    }
    __syncthreads();
}

// Workgroups are dispatched round-robin over the 8 XCDs; with remapping,
// logical workgroup w runs on XCD w / (G/8) so each XCD streams one
// contiguous part of the window.
__device__ __forceinline__ int64_t logical_block() {
#if ZDP_XCD_REMAP
    const uint32_t g = gridDim.x, b = blockIdx.x;
    if (g % 8 == 0) return static_cast<int64_t>(b % 8) * (g / 8) + b / 8;
#endif
    return blockIdx.x;
}

// Iteration space of one lane over element groups [0, ngroups): grid
// stride, consecutive lanes on consecutive groups.  (Per-workgroup
// contiguous ranges measured 20-30% slower.)
struct GroupIter {
    int64_t gi, end, step;
    __device__ __forceinline__ GroupIter(int64_t ngroups) {
        gi = logical_block() * kBlock + threadIdx.x;
        end = ngroups;
        step = static_cast<int64_t>(gridDim.x) * kBlock;
    }
};


// Publishes this workgroup's partial and returns true in every thread of
// the workgroup that finishes last; that workgroup then holds the totals
// (fixed summation order: lane i sums partials i, i+256, ..., then the
// deterministic workgroup tree) in thread 0.
//
// Ordering: the ticket increment is an agent-scope acquire-release
// operation, which publishes this workgroup's partial (the release writes
// back the XCD's L2) and, in the last workgroup, acquires everyone else's;
// the last workgroup's other threads then take an agent-scope acquire fence
// (a cache invalidate, no write-back) before reading the partials.  Each
// agent-scope release costs an L2 write-back, so there is exactly one per
// workgroup: a full fence before the increment and another after it
// doubled the end-of-kernel cost (about 7 us per launch).
__device__ __forceinline__ bool last_block_totals(const Partials& ws, double& sq, int& flag) {
    __shared__ int s_last;
    block_reduce(sq, flag);
    if (threadIdx.x == 0) {
        ws.sq[blockIdx.x] = sq;
        ws.flag[blockIdx.x] = flag;
        const uint32_t prev =
            __hip_atomic_fetch_add(ws.ticket, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == gridDim.x - 1);
    }
    __syncthreads();
    if (!s_last) return false;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    double t = 0.0;
    int f = 0;
    for (uint32_t i = threadIdx.x; i < gridDim.x; i += kBlock) {
        t += __hip_atomic_load(ws.sq + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        f |= __hip_atomic_load(ws.flag + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    block_reduce(t, f);
    if (threadIdx.x == 0) {
        sq = t;
        flag = f;
        __hip_atomic_store(ws.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return true;
}

// Publishes this workgroup's partial in its own slot with plain stores (no
// ticket, no fence): the kernel boundary makes the slots visible to the
// next launch on the stream.  `accumulate` adds to the slot instead (a
// bucket after the first of a step, which must run on the same grid).
__device__ __forceinline__ void publish_partial(const Partials& ws, double sq, int flag, bool accumulate) {
    block_reduce(sq, flag);
    if (threadIdx.x == 0) {
        if (accumulate) {
            sq = ws.sq[blockIdx.x] + sq;
            flag |= ws.flag[blockIdx.x];
        }
        ws.sq[blockIdx.x] = sq;
        ws.flag[blockIdx.x] = flag;
    }
}

// Sum of the `nparts` published partials in the fixed order of
// last_block_totals (lane i sums slots i, i+256, ..., then the workgroup
// tree), in every thread of the workgroup: every workgroup of a launch
// computes the same bits.
__device__ __forceinline__ void sum_partials(const Partials& ws, int nparts, double& sq, int& flag) {
    __shared__ double s_sq;
    __shared__ int s_flag;
    double t = 0.0;
    int f = 0;
    for (int i = threadIdx.x; i < nparts; i += kBlock) {
        t += ws.sq[i];
        f |= ws.flag[i];
    }
    block_reduce(t, f);
    if (threadIdx.x == 0) {
        s_sq = t;
        s_flag = f;
    }
    __syncthreads();
    sq = s_sq;
    flag = s_flag;
}

// ---------------------------------------------------------------- kernels

// The kernel's view of the source with 1/L resolved (the same IEEE division
// as the host's 1.0 / L in every workgroup).
__device__ __forceinline__ SrcArgs resolve_scale(const SrcArgs& src) {
    SrcArgs s = src;
    if (src.dyn != nullptr) s.inv_scale = 1.0 / src.dyn->loss_scale;
    return s;
}

constexpr int kUnroll = ZDP_UNROLL;

// One reduced element group: g = (sum of slices) / L, the inf/NaN flag and
// the sum of squares, and the fp32 g into grad_out (when non-null).
// kNormOfStored: sum g^2 over the fp32-rounded g written to grad_out (the
// clipping path's norm) instead of the float64 g.
template <bool kNormOfStored>
__device__ __forceinline__ void reduce_finish(const double (&acc)[kV], const SrcArgs& src, float* grad_out,
                                              int64_t j, double& sq, int& bad) {
    float gf[kV];
#pragma unroll
    for (int e = 0; e < kV; ++e) {
        const double g = acc[e] * src.inv_scale;
        gf[e] = static_cast<float>(g);
        bad |= !finite(static_cast<double>(gf[e]));
        const double gn = kNormOfStored ? static_cast<double>(gf[e]) : g;
        sq += gn * gn;
    }
    if (grad_out != nullptr) {
        fvec o;
#pragma unroll
        for (int e = 0; e < kV; ++e) o[e] = gf[e];
        stg(reinterpret_cast<fvec*>(grad_out + j), o);
    }
}

// Elements [j, n) of the ragged tail, one at a time.
template <bool kNormOfStored>
__device__ void reduce_tail(int64_t j, const SrcArgs& src, float* grad_out, double& sq, int& bad) {
    for (int64_t e = j; e < src.n; ++e) {
        const double s = sum_slices1(src.win + e, src.stride, src.nd);
        const double g = s * src.inv_scale;
        const float g32 = static_cast<float>(g);
        bad |= !finite(static_cast<double>(g32));
        const double gn = kNormOfStored ? static_cast<double>(g32) : g;
        sq += gn * gn;
        if (grad_out != nullptr) grad_out[e] = g32;
    }
}

// Shapes of the chunked sum (Nd > kUnroll): U 256-element sub-groups per
// wave visit, R slices per chunk, PIPE = the next chunk's loads issued
// before this chunk's adds, XP = also across visits when Nd is a multiple
// of R (1: the next visit's first chunk, 2: also its state).  Windows with
// Nd >= ZDP_CH_BIG_ND take the "big" shape.  Measured in pairs on one MI355X
// against one 256-element group per visit and chunks of 16 (5.9 TB/s of
// slice reads at Nd = 64): the big shape is 7-14% faster for Nd 48-400,
// the small one 2-7% for Nd 17-32.  With launches of 2^23 for the big
// shape it also wins from Nd = 32 up (0.5-3% at Nd 32-40).  The big shape keeps only the next
// visit's first chunk ahead of the update: its state as well does not fit
// the registers of 8 groups per visit without spilling.
#ifndef ZDP_CH_BIG_ND
#define ZDP_CH_BIG_ND 32
#endif
#ifndef ZDP_CHB_U
#define ZDP_CHB_U 8
#endif
#ifndef ZDP_CHB_R
#define ZDP_CHB_R 2
#endif
#ifndef ZDP_CHB_PIPE
#define ZDP_CHB_PIPE 1
#endif
#ifndef ZDP_CHB_XP
#define ZDP_CHB_XP 1
#endif
#ifndef ZDP_CHS_U
#define ZDP_CHS_U 4
#endif
#ifndef ZDP_CHS_R
#define ZDP_CHS_R 2
#endif
#ifndef ZDP_CHS_PIPE
#define ZDP_CHS_PIPE 1
#endif
#ifndef ZDP_CHS_XP
#define ZDP_CHS_XP 2
#endif
static_assert(ZDP_CHB_R >= 1 && ZDP_CHB_R <= ZDP_UNROLL && ZDP_CHS_R >= 1 && ZDP_CHS_R <= ZDP_UNROLL,
              "the chunked path runs only for Nd > ZDP_UNROLL");

// The big visit shape needs at least one visit per wave: a launch with
// fewer (a window or bucket of under 2^21 elements at U = 8) leaves waves
// idle, so it takes the small shape, whose visits are half as long.
__device__ __forceinline__ bool big_visits(int nd, int64_t nfull) {
    return nd >= ZDP_CH_BIG_ND &&
           (nfull + 64 * ZDP_CHB_U - 1) / (64 * ZDP_CHB_U) >= static_cast<int64_t>(gridDim.x) * kWaves;
}


// Chunked sum for Nd > kUnroll.  A wave visits U consecutive 256-element
// sub-groups at a time (lane l holds elements 4l .. 4l+3 of each), so one
// load instruction per slice and sub-group covers a contiguous 512 B, and a
// chunk of R slices puts R*U of them in flight.  A scheduling barrier sits
// between a chunk's loads and its adds: left to itself the scheduler
// interleaves them and serialises half the loads behind full vmcnt waits.
template <int U, int R>
__device__ __forceinline__ void chu_load(hvec (&w)[R][U], const int64_t (&j)[U], const uint16_t* win,
                                         int64_t stride, int k0) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int u = 0; u < U; ++u) w[r][u] = ldh(win + j[u] + static_cast<int64_t>(k0 + r) * stride);
}

// Adds a chunk in slice order; the first chunk starts the sums from slice 0.
template <int U, int R, bool kFirst>
__device__ __forceinline__ void chu_add(double (&acc)[U][kV], const hvec (&w)[R][U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if constexpr (kFirst)
            init_v(acc[u], w[0][u]);
        else
            add_v(acc[u], w[0][u]);
#pragma unroll
        for (int r = 1; r < R; ++r) add_v(acc[u], w[r][u]);
    }
}

// The last chunk of r < R slices (r uniform), dispatched to a compile-time size.
template <int U, int RR>
__device__ __forceinline__ void chu_rem(double (&acc)[U][kV], const int64_t (&j)[U], const uint16_t* win,
                                        int64_t stride, int k0, int r) {
    if constexpr (RR >= 1) {
        if (r == RR) {
            hvec w[RR][U];
            chu_load<U, RR>(w, j, win, stride, k0);
            __builtin_amdgcn_sched_barrier(0);
            chu_add<U, RR, false>(acc, w);
            return;
        }
        chu_rem<U, RR - 1>(acc, j, win, stride, k0, r);
    }
}

// Nd-way sum (Nd >= R) of the U sub-groups at element offsets j[u].
template <int U, int R, bool PIPE>
__device__ __forceinline__ void chu_sum(double (&acc)[U][kV], const int64_t (&j)[U], const uint16_t* win,
                                        int64_t stride, int nd) {
    const int nfc = nd / R;
    hvec wa[R][U];
    chu_load<U, R>(wa, j, win, stride, 0);
    if constexpr (PIPE) {
    hvec wb[R][U];
    int c = 0;
    for (;;) {
        // two register sets in turn, so no set is copied while its loads are in flight
        if (c + 1 < nfc) chu_load<U, R>(wb, j, win, stride, (c + 1) * R);
        __builtin_amdgcn_sched_barrier(0);
        if (c == 0)
            chu_add<U, R, true>(acc, wa);
        else
            chu_add<U, R, false>(acc, wa);
        if (++c >= nfc) break;
        if (c + 1 < nfc) chu_load<U, R>(wa, j, win, stride, (c + 1) * R);
        __builtin_amdgcn_sched_barrier(0);
        chu_add<U, R, false>(acc, wb);
        if (++c >= nfc) break;
    }
    } else {
    __builtin_amdgcn_sched_barrier(0);
    chu_add<U, R, true>(acc, wa);
    for (int c = 1; c < nfc; ++c) {
        chu_load<U, R>(wa, j, win, stride, c * R);
        __builtin_amdgcn_sched_barrier(0);
        chu_add<U, R, false>(acc, wa);
    }
    }
    chu_rem<U, R - 1>(acc, j, win, stride, nfc * R, nd - nfc * R);
}

// Element offsets of visit vi's U sub-groups for this lane; a group past
// nfull is inactive and points at group 0 (its loads are not used).
template <int U>
__device__ __forceinline__ void visit_index(int64_t vi, int64_t nfull, int lane, int64_t (&j)[U], bool (&act)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t g = (vi * U + u) * 64 + lane;
        act[u] = g < nfull;
        j[u] = (act[u] ? g : 0) * kV;
    }
}

// The reduce pass for Nd > kUnroll: the fused step's visits and chunked sum
// without the state (one shape per Nd range, as there).
template <int U, int R, bool PIPE, bool kNormOfStored>
__device__ void rch_run(int64_t nfull, const SrcArgs& src, float* grad_out, double& sq, int& bad) {
    const int64_t wave = logical_block() * kWaves + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * kWaves;
    const int64_t nvis = (nfull + 64 * U - 1) / (64 * U);
    for (int64_t vi = wave; vi < nvis; vi += nwaves) {
        int64_t j[U];
        bool act[U];
        visit_index<U>(vi, nfull, lane, j, act);
        double acc[U][kV];
        chu_sum<U, R, PIPE>(acc, j, src.win, src.stride, src.nd);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (act[u]) reduce_finish<kNormOfStored>(acc[u], src, grad_out, j[u], sq, bad);
    }
    // the ragged tail group nfull, by the lane that would hold it
    if (src.n > nfull * kV && (nfull / (64 * U)) % nwaves == wave && nfull % 64 == lane)
        reduce_tail<kNormOfStored>(nfull * kV, src, grad_out, sq, bad);
}

#ifndef ZDP_RPF2_MAXR
#define ZDP_RPF2_MAXR 8  // Nd up to which the reduce pass loads two groups ahead
#endif

// Full groups gi, gi+step, ... < end with Nd = R <= one chunk: the next
// group's R loads are issued before the current group is summed, as in the
// fused step's prefetch path (past the end, group 0 is loaded and ignored).
template <int R, bool kNormOfStored>
__device__ void reduce_pf_run1(int64_t gi, int64_t end, int64_t step, const SrcArgs& src, float* grad_out,
                               double& sq, int& bad) {
    if (gi >= end) return;
    hvec w[R];
#pragma unroll
    for (int u = 0; u < R; ++u) w[u] = ldh(src.win + gi * kV + static_cast<int64_t>(u) * src.stride);
    for (;;) {
        const int64_t gn = gi + step;
        const int64_t gl = gn < end ? gn : 0;
        hvec wc[R];
#pragma unroll
        for (int u = 0; u < R; ++u) wc[u] = w[u];
#pragma unroll
        for (int u = 0; u < R; ++u) w[u] = ldh(src.win + gl * kV + static_cast<int64_t>(u) * src.stride);
        __builtin_amdgcn_sched_barrier(0);
        double acc[kV];
        init_v(acc, wc[0]);
#pragma unroll
        for (int u = 1; u < R; ++u) add_v(acc, wc[u]);
        reduce_finish<kNormOfStored>(acc, src, grad_out, gi * kV, sq, bad);
        if (gn >= end) break;
        gi = gn;
    }
}

// Two groups ahead from NB rotating register sets, as in the fused step;
// measured 30% faster at Nd = 2 and 4 and 8% at Nd = 8, slower from Nd = 12.
template <int R, bool kNormOfStored, int NB>
__device__ void reduce_pf_run2(int64_t gi, int64_t end, int64_t step, const SrcArgs& src, float* grad_out,
                               double& sq, int& bad) {
    if (gi >= end) return;
    hvec w[NB][R];
#pragma unroll
    for (int u = 0; u < R; ++u) w[0][u] = ldh(src.win + gi * kV + static_cast<int64_t>(u) * src.stride);
    {
        const int64_t g1 = gi + step < end ? gi + step : 0;
#pragma unroll
        for (int u = 0; u < R; ++u) w[1][u] = ldh(src.win + g1 * kV + static_cast<int64_t>(u) * src.stride);
    }
    bool more = true;
    while (more) {
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            if (more) {
                const int ld = (k + 2) % NB;
                const int64_t g2 = gi + 2 * step < end ? gi + 2 * step : 0;
#pragma unroll
                for (int u = 0; u < R; ++u)
                    w[ld][u] = ldh(src.win + g2 * kV + static_cast<int64_t>(u) * src.stride);
                __builtin_amdgcn_sched_barrier(0);
                double acc[kV];
                init_v(acc, w[k][0]);
#pragma unroll
                for (int u = 1; u < R; ++u) add_v(acc, w[k][u]);
                reduce_finish<kNormOfStored>(acc, src, grad_out, gi * kV, sq, bad);
                if (gi + step >= end)
                    more = false;
                else
                    gi += step;
            }
        }
    }
}

template <int R, bool kNormOfStored>
__device__ void reduce_pf_run(int64_t gi, int64_t end, int64_t step, const SrcArgs& src, float* grad_out,
                              double& sq, int& bad) {
    if constexpr (R <= ZDP_RPF2_MAXR)
        reduce_pf_run2<R, kNormOfStored, 4>(gi, end, step, src, grad_out, sq, bad);
    else
        reduce_pf_run1<R, kNormOfStored>(gi, end, step, src, grad_out, sq, bad);
}

template <int R, bool kNormOfStored>
__device__ __forceinline__ bool reduce_pf_dispatch(int nd, int64_t gi, int64_t end, int64_t step,
                                                   const SrcArgs& src, float* grad_out, double& sq, int& bad) {
    if constexpr (R >= 1) {
        if (nd == R) {
            reduce_pf_run<R, kNormOfStored>(gi, end, step, src, grad_out, sq, bad);
            return true;
        }
        return reduce_pf_dispatch<R - 1, kNormOfStored>(nd, gi, end, step, src, grad_out, sq, bad);
    }
    return false;
}

template <bool kNormOfStored>
__global__ void __launch_bounds__(kBlock) reduce_owned_kernel(SrcArgs src_in, float* grad_out,
                                                              int32_t* overflow, double* sumsq,
                                                              Partials ws, int32_t accumulate) {
    const SrcArgs src = resolve_scale(src_in);
    const int64_t ngroups = (src.n + kV - 1) / kV;
    const int64_t nfull = src.n / kV;
    double sq = 0.0;
    int bad = 0;
    bool done = false;
    if (src.nd <= kUnroll) {
        GroupIter it(ngroups);
        const int64_t endf = it.end < nfull ? it.end : nfull;
        done = reduce_pf_dispatch<kUnroll, kNormOfStored>(src.nd, it.gi, endf, it.step, src, grad_out, sq, bad);
        if (done && ngroups > nfull) {
            // the ragged tail group, by the lane whose sequence contains it
            const int64_t g = nfull;
            if (g >= it.gi && g < it.end && (g - it.gi) % it.step == 0)
                reduce_tail<kNormOfStored>(g * kV, src, grad_out, sq, bad);
        }
    }
    if (!done) {
        if (big_visits(src.nd, nfull))
            rch_run<ZDP_CHB_U, ZDP_CHB_R, ZDP_CHB_PIPE != 0, kNormOfStored>(nfull, src, grad_out, sq, bad);
        else
            rch_run<ZDP_CHS_U, ZDP_CHS_R, ZDP_CHS_PIPE != 0, kNormOfStored>(nfull, src, grad_out, sq, bad);
    }
    if constexpr (kNormOfStored) {
        // the clipped step's first pass: its second pass sums the partials
        // (a piece of a long window after the first adds to its slot)
        publish_partial(ws, sq, bad, accumulate != 0);
    } else if (last_block_totals(ws, sq, bad) && threadIdx.x == 0) {
        *overflow = bad;
        *sumsq = sq;
    }
}

// Per-element Adam/AdamW update (float64 arithmetic, fp32 storage).
struct AdamScalars {
    double b1, b2, omb1, omb2, ss, isb, dcy, eps;
};


// Scalars of the step being taken, t = committed + 1 (identical in every
// lane and workgroup: the same IEEE operations on the same inputs).
__device__ __forceinline__ AdamScalars step_scalars(const AdamArgs& a, double& b1t, double& b2t) {
    const zero_step_ctl* ctl = a.ctl;
    b1t = ctl->beta1_pow * a.b1;
    b2t = ctl->beta2_pow * a.b2;
    AdamScalars c;
    c.b1 = a.b1;
    c.b2 = a.b2;
    c.omb1 = 1.0 - a.b1;
    c.omb2 = 1.0 - a.b2;
    c.ss = a.lr / (1.0 - b1t);
    c.isb = 1.0 / __builtin_sqrt(1.0 - b2t);
    c.dcy = 1.0 - a.lr * a.wd;
    c.eps = a.eps;
    return c;
}

// Commit (or skip) a step for the whole window, and advance the dynamic
// loss scale; run by one lane after every workgroup has finished.  A
// bucketed step whose buckets did not cover the window (bad == 2) is
// skipped without touching the loss scale.
__device__ __forceinline__ void commit_step(const AdamArgs& a, int cur, double b1t, double b2t, int bad,
                                            double sq, double coef) {
    zero_step_ctl* w = a.ctl;
    w->overflow = bad;
    w->sumsq = sq;
    if (!bad) {
        w->cur = cur ^ 1;
        w->t = w->t + 1;
        w->beta1_pow = b1t;
        w->beta2_pow = b2t;
        w->clip_coef = coef;
    } else {
        w->skipped = w->skipped + 1;
    }
    if (a.interval > 0 && bad != 2) {
        if (bad) {
            w->loss_scale = w->loss_scale * a.backoff;
            w->good_steps = 0;
        } else {
            int g = w->good_steps + 1;
            if (g == a.interval) {
                // as torch's amp scaler: a growth that overflows keeps the scale
                const double grown = w->loss_scale * a.growth;
                if (__builtin_isfinite(grown)) w->loss_scale = grown;
                g = 0;
            }
            w->good_steps = g;
        }
    }
}

__device__ __forceinline__ void adam1(const AdamScalars& c, double g, float p, float m, float v,
                                      float& po, float& mo, float& vo) {
    const double m1 = (c.b1 * static_cast<double>(m)) + (c.omb1 * g);
    const double v1 = (c.b2 * static_cast<double>(v)) + (c.omb2 * (g * g));
    const double d = (__builtin_sqrt(v1) * c.isb) + c.eps;
    const double q = m1 / d;
    const double p1 = (static_cast<double>(p) * c.dcy) - (c.ss * q);
    mo = static_cast<float>(m1);
    vo = static_cast<float>(v1);
    po = static_cast<float>(p1);
}


// Buffers of one fused step after the ping-pong selection.
struct FusedPtrs {
    const float* pin;
    const float* min_;
    const float* vin;
    float* pout;
    float* mout;
    float* vout;
    uint16_t* ag;
};

template <int R>
__device__ __forceinline__ void pf_load(hvec (&w)[R], fvec& p, fvec& m, fvec& v, const SrcArgs& src,
                                        const FusedPtrs& f, int64_t j) {
    p = ldg(reinterpret_cast<const fvec*>(f.pin + j));
    m = ldg(reinterpret_cast<const fvec*>(f.min_ + j));
    v = ldg(reinterpret_cast<const fvec*>(f.vin + j));
#pragma unroll
    for (int u = 0; u < R; ++u) w[u] = ldh(src.win + j + static_cast<int64_t>(u) * src.stride);
}

template <int R>
__device__ __forceinline__ void pf_finish(const hvec (&w)[R], const fvec& pv, const fvec& mv, const fvec& vv,
                                          const SrcArgs& src, const FusedPtrs& f, const AdamScalars& c,
                                          int64_t j, double& sq, int& bad) {
    double acc[kV];
    init_v(acc, w[0]);
#pragma unroll
    for (int u = 1; u < R; ++u) add_v(acc, w[u]);
    float po[kV], mo[kV], vo[kV];
#pragma unroll
    for (int e = 0; e < kV; ++e) {
        const double g = acc[e] * src.inv_scale;
        bad |= !finite(g);
        sq += g * g;
        adam1(c, g, pv[e], mv[e], vv[e], po[e], mo[e], vo[e]);
    }
    fvec pw, mw, vw;
#pragma unroll
    for (int e = 0; e < kV; ++e) {
        pw[e] = po[e];
        mw[e] = mo[e];
        vw[e] = vo[e];
    }
    stg(reinterpret_cast<fvec*>(f.pout + j), pw);
    stg(reinterpret_cast<fvec*>(f.mout + j), mw);
    stg(reinterpret_cast<fvec*>(f.vout + j), vw);
    if (f.ag != nullptr) stg(reinterpret_cast<hvec*>(f.ag + j), pack_v(po));
}

#ifndef ZDP_PF_NB
#define ZDP_PF_NB 4  // register sets of the two-ahead prefetch
#endif
#ifndef ZDP_PF2_MINR
#define ZDP_PF2_MINR 7  // Nd range that prefetches two groups ahead
#endif
#ifndef ZDP_PF2_MAXR
#define ZDP_PF2_MAXR 9
#endif

// Full groups gi, gi+step, ... < end when all Nd = R slices fit in one
// chunk: the next group's R + 3 loads are issued before the current group
// is summed and updated, so its memory latency overlaps this group's fp64
// work.  Past the end a lane loads group 0 instead (the values are not
// used): every lane of a wave then reads the same few lines, which mostly
// hit L2, and the loop needs no branch around its loads.
template <int R>
__device__ void pf_run1(int64_t gi, int64_t end, int64_t step, const SrcArgs& src, const FusedPtrs& f,
                        const AdamScalars& c, double& sq, int& bad) {
    if (gi >= end) return;
    hvec w[R];
    fvec p, m, v;
    pf_load<R>(w, p, m, v, src, f, gi * kV);
    for (;;) {
        const int64_t gn = gi + step;
        const int64_t gl = gn < end ? gn : 0;
        hvec wc[R];
#pragma unroll
        for (int u = 0; u < R; ++u) wc[u] = w[u];
        const fvec pc = p, mc = m, vc = v;
        pf_load<R>(w, p, m, v, src, f, gl * kV);
        __builtin_amdgcn_sched_barrier(0);  // keep the next group's loads ahead of this group's work
        pf_finish<R>(wc, pc, mc, vc, src, f, c, gi * kV, sq, bad);
        if (gn >= end) break;
        gi = gn;
    }
}

// The same, two groups ahead: group gi + 2*step is loaded before group gi
// is finished, from NB register sets used in rotation (the loop is unrolled
// NB times, so no set is copied while its loads are in flight, and a set is
// reloaded NB - 2 phases after its last use).  Measured faster for
// 7 <= Nd <= 9 only; elsewhere one group ahead is as fast or faster.
template <int R, int NB>
__device__ void pf_run2(int64_t gi, int64_t end, int64_t step, const SrcArgs& src, const FusedPtrs& f,
                        const AdamScalars& c, double& sq, int& bad) {
    if (gi >= end) return;
    hvec w[NB][R];
    fvec p[NB], m[NB], v[NB];
    pf_load<R>(w[0], p[0], m[0], v[0], src, f, gi * kV);
    {
        const int64_t g1 = gi + step;
        pf_load<R>(w[1], p[1], m[1], v[1], src, f, (g1 < end ? g1 : 0) * kV);
    }
    bool more = true;
    while (more) {
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            if (more) {
                const int ld = (k + 2) % NB;
                const int64_t g2 = gi + 2 * step;
                pf_load<R>(w[ld], p[ld], m[ld], v[ld], src, f, (g2 < end ? g2 : 0) * kV);
                __builtin_amdgcn_sched_barrier(0);
                pf_finish<R>(w[k], p[k], m[k], v[k], src, f, c, gi * kV, sq, bad);
                if (gi + step >= end)
                    more = false;
                else
                    gi += step;
            }
        }
    }
}

template <int R>
__device__ void pf_run(int64_t gi, int64_t end, int64_t step, const SrcArgs& src, const FusedPtrs& f,
                       const AdamScalars& c, double& sq, int& bad) {
    if constexpr (ZDP_PF_NB >= 3 && R >= ZDP_PF2_MINR && R <= ZDP_PF2_MAXR)
        pf_run2<R, ZDP_PF_NB>(gi, end, step, src, f, c, sq, bad);
    else
        pf_run1<R>(gi, end, step, src, f, c, sq, bad);
}

template <int R>
__device__ __forceinline__ bool pf_dispatch(int nd, int64_t gi, int64_t end, int64_t step, const SrcArgs& src,
                                            const FusedPtrs& f, const AdamScalars& c, double& sq, int& bad) {
    if constexpr (R >= 1) {
        if (nd == R) {
            pf_run<R>(gi, end, step, src, f, c, sq, bad);
            return true;
        }
        return pf_dispatch<R - 1>(nd, gi, end, step, src, f, c, sq, bad);
    }
    return false;
}

// The fused step element by element over [e0, e1): the ragged tail.
__device__ void fused_elems(int64_t e0, int64_t e1, const SrcArgs& src, const FusedPtrs& f,
                            const AdamScalars& c, double& sq, int& bad) {
    for (int64_t e = e0; e < e1; ++e) {
        const double s = sum_slices1(src.win + e, src.stride, src.nd);
        const double g = s * src.inv_scale;
        bad |= !finite(g);
        sq += g * g;
        float po, mo, vo;
        adam1(c, g, f.pin[e], f.min_[e], f.vin[e], po, mo, vo);
        f.pout[e] = po;
        f.mout[e] = mo;
        f.vout[e] = vo;
        if (f.ag != nullptr) f.ag[e] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(po));
    }
}

template <int U>
__device__ __forceinline__ void visit_state(fvec (&pv)[U], fvec (&mv)[U], fvec (&vv)[U], const FusedPtrs& f,
                                            const int64_t (&j)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        pv[u] = ldg(reinterpret_cast<const fvec*>(f.pin + j[u]));
        mv[u] = ldg(reinterpret_cast<const fvec*>(f.min_ + j[u]));
        vv[u] = ldg(reinterpret_cast<const fvec*>(f.vin + j[u]));
    }
}

// Unscale, flag, sum of squares, Adam and the stores of one visit.
template <int U>
__device__ __forceinline__ void visit_finish(const double (&acc)[U][kV], const fvec (&pv)[U], const fvec (&mv)[U],
                                             const fvec (&vv)[U], const int64_t (&j)[U], const bool (&act)[U],
                                             const SrcArgs& src, const FusedPtrs& f, const AdamScalars& c,
                                             double& sq, int& bad) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (!act[u]) continue;
        float po[kV], mo[kV], vo[kV];
#pragma unroll
        for (int e = 0; e < kV; ++e) {
            const double g = acc[u][e] * src.inv_scale;
            bad |= !finite(g);
            sq += g * g;
            adam1(c, g, pv[u][e], mv[u][e], vv[u][e], po[e], mo[e], vo[e]);
        }
        fvec pw, mw, vw;
#pragma unroll
        for (int e = 0; e < kV; ++e) {
            pw[e] = po[e];
            mw[e] = mo[e];
            vw[e] = vo[e];
        }
        stg(reinterpret_cast<fvec*>(f.pout + j[u]), pw);
        stg(reinterpret_cast<fvec*>(f.mout + j[u]), mw);
        stg(reinterpret_cast<fvec*>(f.vout + j[u]), vw);
        if (f.ag != nullptr) stg(reinterpret_cast<hvec*>(f.ag + j[u]), pack_v(po));
    }
}

// Visits vi = wave, wave + waves, ... (in logical workgroup order); with
// U = 1 this is the same grid-stride order as GroupIter.
template <int U, int R, bool PIPE>
__device__ void ch_loop(int64_t nfull, int64_t wave, int lane, int64_t nwaves, const SrcArgs& src,
                        const FusedPtrs& f, const AdamScalars& c, double& sq, int& bad) {
    const int64_t nvis = (nfull + 64 * U - 1) / (64 * U);
    for (int64_t vi = wave; vi < nvis; vi += nwaves) {
        int64_t j[U];
        bool act[U];
        visit_index<U>(vi, nfull, lane, j, act);
        fvec pv[U], mv[U], vv[U];
        visit_state<U>(pv, mv, vv, f, j);
        double acc[U][kV];
        chu_sum<U, R, PIPE>(acc, j, src.win, src.stride, src.nd);
        visit_finish<U>(acc, pv, mv, vv, j, act, src, f, c, sq, bad);
    }
}

// The same for Nd a multiple of R, with the chunk loads one chunk ahead
// across visits: the last chunk of a visit is added while the next visit's
// first chunk (and with XS its state) is in flight, and those stay in
// flight through this visit's update.  Register sets w0 / w1 alternate
// within a visit; the next visit's first chunk goes to wx and moves to w0
// after the update.  Without XS a visit's state loads are issued at its
// start, behind its first chunk.
template <int U, int R, bool XS>
__device__ void ch_loop_xp(int64_t nfull, int64_t wave, int lane, int64_t nwaves, const SrcArgs& src,
                           const FusedPtrs& f, const AdamScalars& c, double& sq, int& bad) {
    const int64_t nvis = (nfull + 64 * U - 1) / (64 * U);
    if (wave >= nvis) return;
    const int nfc = src.nd / R;
    int64_t vi = wave;
    int64_t j[U];
    bool act[U];
    visit_index<U>(vi, nfull, lane, j, act);
    fvec pv[U], mv[U], vv[U];
    if constexpr (XS) visit_state<U>(pv, mv, vv, f, j);
    hvec w0[R][U];
    chu_load<U, R>(w0, j, src.win, src.stride, 0);
    for (;;) {
        if constexpr (!XS) visit_state<U>(pv, mv, vv, f, j);
        const int64_t vn = vi + nwaves;
        const bool more = vn < nvis;
        int64_t jn[U];
        bool actn[U];
        visit_index<U>(more ? vn : 0, more ? nfull : 0, lane, jn, actn);
        fvec pn[U], mn[U], vn_[U];
        hvec w1[R][U], wx[R][U];
        double acc[U][kV];
        int cc = 0;
        for (;;) {
            if (cc + 1 < nfc) {
                chu_load<U, R>(w1, j, src.win, src.stride, (cc + 1) * R);
            } else if (more) {
                if constexpr (XS) visit_state<U>(pn, mn, vn_, f, jn);
                chu_load<U, R>(wx, jn, src.win, src.stride, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (cc == 0)
                chu_add<U, R, true>(acc, w0);
            else
                chu_add<U, R, false>(acc, w0);
            if (++cc >= nfc) break;
            if (cc + 1 < nfc) {
                chu_load<U, R>(w0, j, src.win, src.stride, (cc + 1) * R);
            } else if (more) {
                if constexpr (XS) visit_state<U>(pn, mn, vn_, f, jn);
                chu_load<U, R>(wx, jn, src.win, src.stride, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            chu_add<U, R, false>(acc, w1);
            if (++cc >= nfc) break;
        }
        visit_finish<U>(acc, pv, mv, vv, j, act, src, f, c, sq, bad);
        if (!more) break;
        // the copies below wait for the next visit's loads: keep them after the update
        __builtin_amdgcn_sched_barrier(0);
        vi = vn;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            j[u] = jn[u];
            act[u] = actn[u];
            if constexpr (XS) {
                pv[u] = pn[u];
                mv[u] = mn[u];
                vv[u] = vn_[u];
            }
#pragma unroll
            for (int r = 0; r < R; ++r) w0[r][u] = wx[r][u];
        }
    }
}

// Full groups [g0, nfull) in visits of U groups, wave w taking visits w,
// w + W, ... of that range (no loads across visits).  A group past nfull
// is inactive and loads group g0.
template <int U, int R, bool PIPE>
__device__ void ch_loop_from(int64_t g0, int64_t nfull, int64_t wave, int lane, int64_t nwaves,
                             const SrcArgs& src, const FusedPtrs& f, const AdamScalars& c, double& sq, int& bad) {
    const int64_t ng = nfull - g0;
    const int64_t nvis = (ng + 64 * U - 1) / (64 * U);
    for (int64_t vi = wave; vi < nvis; vi += nwaves) {
        int64_t j[U];
        bool act[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t g = (vi * U + u) * 64 + lane;
            act[u] = g < ng;
            j[u] = (g0 + (act[u] ? g : 0)) * kV;
        }
        fvec pv[U], mv[U], vv[U];
        visit_state<U>(pv, mv, vv, f, j);
        double acc[U][kV];
        chu_sum<U, R, PIPE>(acc, j, src.win, src.stride, src.nd);
        visit_finish<U>(acc, pv, mv, vv, j, act, src, f, c, sq, bad);
    }
}

#ifndef ZDP_TAIL_SPLIT
#define ZDP_TAIL_SPLIT 1  // a launch's last partial round in smaller visits (0: as the others)
#endif

// Full groups [0, nfull) and the ragged tail for Nd > kUnroll, in one shape.
// A launch whose visits end in a partial round, most waves idle in it,
// takes that round in smaller visits over every wave: quarter visits when
// it holds at most a quarter of the waves' visits, half visits when at
// most half, so it fits one round of them.  (Measured at Nd = 400 on
// single launches of 2.12-3.5 visits per wave: 0.70-0.77 of 8 TB/s
// unsplit, 0.77-0.84 split; whole rounds run at 0.83-0.85.)
template <int U, int R, bool PIPE, int XP>
__device__ void ch_run(int64_t nfull, const SrcArgs& src, const FusedPtrs& f, const AdamScalars& c,
                       double& sq, int& bad) {
    const int64_t wave = logical_block() * kWaves + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * kWaves;
    int64_t nmain = nfull;
    int tail_u = 0;
    if constexpr (ZDP_TAIL_SPLIT != 0 && U >= 4) {
        const int64_t nvis = (nfull + 64 * U - 1) / (64 * U);
        const int64_t full = nvis / nwaves * nwaves;  // visits of the full rounds
        const int64_t t = nvis - full;
        if (full > 0 && t > 0) {
            if (U >= 8 && 4 * t <= nwaves)
                tail_u = U / 4;
            else if (2 * t <= nwaves)
                tail_u = U / 2;
            if (tail_u != 0) nmain = full * 64 * U;
        }
    }
    if (XP != 0 && src.nd % R == 0)
        ch_loop_xp<U, R, XP == 2>(nmain, wave, lane, nwaves, src, f, c, sq, bad);
    else
        ch_loop<U, R, PIPE>(nmain, wave, lane, nwaves, src, f, c, sq, bad);
    if constexpr (ZDP_TAIL_SPLIT != 0 && U >= 4) {
        if (tail_u == U / 2)
            ch_loop_from<U / 2, R, PIPE>(nmain, nfull, wave, lane, nwaves, src, f, c, sq, bad);
        if constexpr (U >= 8) {
            if (tail_u == U / 4)
                ch_loop_from<U / 4, R, PIPE>(nmain, nfull, wave, lane, nwaves, src, f, c, sq, bad);
        }
    }
    // the ragged tail group nfull, by the lane that would hold it
    if (src.n > nfull * kV && (nfull / (64 * U)) % nwaves == wave && nfull % 64 == lane)
        fused_elems(nfull * kV, src.n, src, f, c, sq, bad);
}

__device__ __forceinline__ void ch_dispatch(int64_t nfull, const SrcArgs& src, const FusedPtrs& f,
                                            const AdamScalars& c, double& sq, int& bad) {
    if (big_visits(src.nd, nfull))
        ch_run<ZDP_CHB_U, ZDP_CHB_R, ZDP_CHB_PIPE != 0, ZDP_CHB_XP>(nfull, src, f, c, sq, bad);
    else
        ch_run<ZDP_CHS_U, ZDP_CHS_R, ZDP_CHS_PIPE != 0, ZDP_CHS_XP>(nfull, src, f, c, sq, bad);
}

// The fused step over one contiguous run of the window: `src` holds the
// run's slices, `f` its state and all-gather pointers; sq and bad
// accumulate the run's sum of g^2 and flag.
__device__ __forceinline__ void fused_run(const SrcArgs& src, const FusedPtrs& f, const AdamScalars& c,
                                          double& sq, int& bad) {
    const int64_t ngroups = (src.n + kV - 1) / kV;
    const int64_t nfull = src.n / kV;
    bool done = false;
    if (src.nd <= kUnroll) {
        GroupIter it(ngroups);
        const int64_t endf = it.end < nfull ? it.end : nfull;
        done = pf_dispatch<kUnroll>(src.nd, it.gi, endf, it.step, src, f, c, sq, bad);
        if (done && ngroups > nfull) {
            // the ragged tail group, by the lane whose sequence contains it
            const int64_t g = nfull;
            if (g >= it.gi && g < it.end && (g - it.gi) % it.step == 0) fused_elems(g * kV, src.n, src, f, c, sq, bad);
        }
    }
    if (!done) ch_dispatch(nfull, src, f, c, sq, bad);
}

__global__ void __launch_bounds__(kBlock) fused_step_kernel(SrcArgs src_in, AdamArgs a, Partials ws) {
    const SrcArgs src = resolve_scale(src_in);
    const int cur = a.ctl->cur;
    double b1t, b2t;
    const AdamScalars c = step_scalars(a, b1t, b2t);
    const FusedPtrs f{a.p[cur], a.m[cur], a.v[cur], a.p[cur ^ 1], a.m[cur ^ 1], a.v[cur ^ 1], a.ag};
    double sq = 0.0;
    int bad = 0;
    fused_run(src, f, c, sq, bad);
    // partials for commit_kernel (a bucket after the first adds to its slot)
    const bool more = a.bucket != 0 && (a.bucket & ZERO_BUCKET_FIRST) == 0;
    publish_partial(ws, sq, bad, more);
    if (a.bucket != 0 && blockIdx.x == 0 && threadIdx.x == 0) *a.run_count = (more ? *a.run_count : 0) + src.n;
}

// Several runs of a bucketed step in one launch (the buckets that have
// arrived): run i reads its slices from win[i] (rows stride[i] apart) and
// steps window elements [off[i], off[i] + n[i]).  For Nd <= kUnroll the
// full groups of all the runs form one grid-stride sequence; for larger Nd
// the visits of all the runs do (below).  Each run's ragged tail is done by
// one lane.  Each workgroup's partial accumulates over the runs before it
// reaches its slot.
constexpr int kMaxRuns = 16;
struct RunList {
    const uint16_t* win[kMaxRuns];
    int64_t stride[kMaxRuns];
    int64_t n[kMaxRuns];
    int64_t off[kMaxRuns];
    int32_t count;
};

// The runs of one launch as LDS tables, read when a lane's next group lies
// in a later run: run i's slices, their row stride, its window offset, and
// pre[i], the number of full groups of the runs before it (pre[count] = all
// of them).
struct RunTab {
    const uint16_t* win[kMaxRuns];
    int64_t stride[kMaxRuns];
    int64_t off[kMaxRuns];
    int64_t pre[kMaxRuns + 1];
};

// A lane's current run: its full groups are [pre, hi) of the sequence over
// all the runs, its slices start at win (rows stride apart) and its first
// element is window element off.  Registers only; the LDS table is read
// when a lane's next group lies in a later run.
struct RunCur {
    int64_t pre, hi;
    const uint16_t* win;
    int64_t stride, off;
    int r;
};

__device__ __forceinline__ void run_seek(const RunTab& t, RunCur& c, int64_t g) {
    while (g >= c.hi) {
        ++c.r;
        c.pre = c.hi;
        c.hi = t.pre[c.r + 1];
        c.win = t.win[c.r];
        c.stride = t.stride[c.r];
        c.off = t.off[c.r];
    }
}

// Loads group g of run c (g in [c.pre, c.hi)) and returns its window
// element index.
template <int R>
__device__ __forceinline__ int64_t pfr_load(const RunCur& c, int64_t g, hvec (&w)[R], fvec& p, fvec& m, fvec& v,
                                            const FusedPtrs& f) {
    const int64_t jl = (g - c.pre) * kV;
    const int64_t js = c.off + jl;
    const uint16_t* sw = c.win + jl;
    p = ldg(reinterpret_cast<const fvec*>(f.pin + js));
    m = ldg(reinterpret_cast<const fvec*>(f.min_ + js));
    v = ldg(reinterpret_cast<const fvec*>(f.vin + js));
#pragma unroll
    for (int u = 0; u < R; ++u) w[u] = ldh(sw + static_cast<int64_t>(u) * c.stride);
    return js;
}

// The one-ahead prefetch loop of pf_run1 over the full groups of all the
// runs at once: a lane's grid-stride sequence runs on from one run into
// the next, so the pipeline fills and drains once per launch instead of
// once per run.  A lane's groups ascend, so its run only advances.  Past
// the end a lane loads the first full group of the launch (unused).
template <int R>
__device__ void pfr_run1(const RunTab& t, int64_t gi, int64_t end, int64_t step, const SrcArgs& src,
                         const FusedPtrs& f, const AdamScalars& c, double& sq, int& bad) {
    if (gi >= end) return;
    RunCur z{0, t.pre[1], t.win[0], t.stride[0], t.off[0], 0};
    run_seek(t, z, 0);  // the run that holds the first full group
    RunCur cur = z;
    run_seek(t, cur, gi);
    hvec w[R];
    fvec p, m, v;
    int64_t js = pfr_load<R>(cur, gi, w, p, m, v, f);
    for (;;) {
        const int64_t gn = gi + step;
        const bool more = gn < end;
        if (more) run_seek(t, cur, gn);
        hvec wc[R];
#pragma unroll
        for (int u = 0; u < R; ++u) wc[u] = w[u];
        const fvec pc = p, mc = m, vc = v;
        const int64_t jc = js;
        const RunCur& at = more ? cur : z;
        js = pfr_load<R>(at, more ? gn : z.pre, w, p, m, v, f);
        __builtin_amdgcn_sched_barrier(0);  // keep the next group's loads ahead of this group's work
        pf_finish<R>(wc, pc, mc, vc, src, f, c, jc, sq, bad);
        if (!more) break;
        gi = gn;
    }
}

// The same, two groups ahead (pf_run2's rotation of NB register sets) for
// 7 <= Nd <= 9: the run cursor follows the loads, two groups ahead of the
// group being finished, and each register set keeps its group's window
// element index.
template <int R, int NB>
__device__ void pfr_run2(const RunTab& t, int64_t gi, int64_t end, int64_t step, const SrcArgs& src,
                         const FusedPtrs& f, const AdamScalars& c, double& sq, int& bad) {
    if (gi >= end) return;
    RunCur z{0, t.pre[1], t.win[0], t.stride[0], t.off[0], 0};
    run_seek(t, z, 0);  // the run that holds the first full group
    RunCur cur = z;
    run_seek(t, cur, gi);
    hvec w[NB][R];
    fvec p[NB], m[NB], v[NB];
    int64_t js[NB];
    js[0] = pfr_load<R>(cur, gi, w[0], p[0], m[0], v[0], f);
    {
        const int64_t g1 = gi + step;
        const bool in = g1 < end;
        if (in) run_seek(t, cur, g1);
        const RunCur& at = in ? cur : z;
        js[1] = pfr_load<R>(at, in ? g1 : z.pre, w[1], p[1], m[1], v[1], f);
    }
    bool more = true;
    while (more) {
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            if (more) {
                const int ld = (k + 2) % NB;
                const int64_t g2 = gi + 2 * step;
                const bool in = g2 < end;
                if (in) run_seek(t, cur, g2);
                const RunCur& at = in ? cur : z;
                js[ld] = pfr_load<R>(at, in ? g2 : z.pre, w[ld], p[ld], m[ld], v[ld], f);
                __builtin_amdgcn_sched_barrier(0);
                pf_finish<R>(w[k], p[k], m[k], v[k], src, f, c, js[k], sq, bad);
                if (gi + step >= end)
                    more = false;
                else
                    gi += step;
            }
        }
    }
}

// The chunked sum over the visits of all the runs as one sequence: run r's
// full groups form ceil(nfull_r / (64 U)) visits, each within that run, and
// wave w takes visits w, w + W, ... of the sequence (as ch_loop does for
// one window), so short runs do not leave waves idle.  The wave index is
// made wave-uniform, so the run index and each run's pointers stay in
// scalar registers.
template <int U, int R, bool PIPE>
__device__ void chr_loop(const RunList& rl, const SrcArgs& base, const AdamArgs& a, int cur, const AdamScalars& c,
                         double& sq, int& bad) {
    const int64_t wave = __builtin_amdgcn_readfirstlane(static_cast<int>(logical_block() * kWaves + (threadIdx.x >> 6)));
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * kWaves;
    constexpr int64_t kVis = 64 * U;
    int r = 0;
    int64_t vbeg = 0, vend = (rl.n[0] / kV + kVis - 1) / kVis;
    for (int64_t vi = wave;; vi += nwaves) {
        while (vi >= vend && r + 1 < rl.count) {
            ++r;
            vbeg = vend;
            vend += (rl.n[r] / kV + kVis - 1) / kVis;
        }
        if (vi >= vend) break;
        SrcArgs s = base;
        s.win = rl.win[r];
        s.stride = rl.stride[r];
        s.n = rl.n[r];
        const int64_t o = rl.off[r];
        const FusedPtrs f{a.p[cur] + o,     a.m[cur] + o,     a.v[cur] + o,
                          a.p[cur ^ 1] + o, a.m[cur ^ 1] + o, a.v[cur ^ 1] + o,
                          a.ag != nullptr ? a.ag + o : nullptr};
        int64_t j[U];
        bool act[U];
        visit_index<U>(vi - vbeg, s.n / kV, lane, j, act);
        fvec pv[U], mv[U], vv[U];
        visit_state<U>(pv, mv, vv, f, j);
        double acc[U][kV];
        chu_sum<U, R, PIPE>(acc, j, s.win, s.stride, s.nd);
        visit_finish<U>(acc, pv, mv, vv, j, act, s, f, c, sq, bad);
    }
}

template <int R>
__device__ __forceinline__ bool pfr_dispatch(int nd, const RunTab& t, int64_t gi, int64_t end, int64_t step,
                                             const SrcArgs& src, const FusedPtrs& f, const AdamScalars& c,
                                             double& sq, int& bad) {
    if constexpr (R >= 1) {
        if (nd == R) {
            if constexpr (ZDP_PF_NB >= 3 && R >= ZDP_PF2_MINR && R <= ZDP_PF2_MAXR)
                pfr_run2<R, ZDP_PF_NB>(t, gi, end, step, src, f, c, sq, bad);
            else
                pfr_run1<R>(t, gi, end, step, src, f, c, sq, bad);
            return true;
        }
        return pfr_dispatch<R - 1>(nd, t, gi, end, step, src, f, c, sq, bad);
    }
    return false;
}

__global__ void __launch_bounds__(kBlock) fused_runs_kernel(RunList rl, SrcArgs src_in, AdamArgs a, Partials ws) {
    const SrcArgs base = resolve_scale(src_in);
    const int cur = a.ctl->cur;
    double b1t, b2t;
    const AdamScalars c = step_scalars(a, b1t, b2t);
    double sq = 0.0;
    int bad = 0;
    int64_t total = 0;
    for (int i = 0; i < rl.count; ++i) total += rl.n[i];
    if (base.nd <= kUnroll) {
        // Nd within one chunk: one grid-stride sequence over every run's
        // full groups, then each run's ragged tail by one lane
        __shared__ RunTab t;
        if (threadIdx.x < static_cast<unsigned>(rl.count)) {
            const int i = static_cast<int>(threadIdx.x);
            t.win[i] = rl.win[i];
            t.stride[i] = rl.stride[i];
            t.off[i] = rl.off[i];
        }
        if (threadIdx.x == 0) {
            int64_t g = 0;
            for (int i = 0; i < rl.count; ++i) {
                t.pre[i] = g;
                g += rl.n[i] / kV;
            }
            t.pre[rl.count] = g;
        }
        __syncthreads();
        const FusedPtrs f{a.p[cur],     a.m[cur],     a.v[cur],
                          a.p[cur ^ 1], a.m[cur ^ 1], a.v[cur ^ 1], a.ag};
        GroupIter it(t.pre[rl.count]);
        (void)pfr_dispatch<kUnroll>(base.nd, t, it.gi, it.end, it.step, base, f, c, sq, bad);
    } else {
        int64_t nfull = 0;
        for (int i = 0; i < rl.count; ++i) nfull += rl.n[i] / kV;
        if (big_visits(base.nd, nfull))
            chr_loop<ZDP_CHB_U, ZDP_CHB_R, ZDP_CHB_PIPE != 0>(rl, base, a, cur, c, sq, bad);
        else
            chr_loop<ZDP_CHS_U, ZDP_CHS_R, ZDP_CHS_PIPE != 0>(rl, base, a, cur, c, sq, bad);
    }
    // each run's ragged tail, by one lane
    const int64_t tid = logical_block() * kBlock + threadIdx.x;
    if (tid < rl.count && rl.n[tid] % kV != 0) {
        const int i = static_cast<int>(tid);
        SrcArgs s = base;
        s.win = rl.win[i];
        s.stride = rl.stride[i];
        s.n = rl.n[i];
        const int64_t o = rl.off[i];
        const FusedPtrs fi{a.p[cur] + o,     a.m[cur] + o,     a.v[cur] + o,
                           a.p[cur ^ 1] + o, a.m[cur ^ 1] + o, a.v[cur ^ 1] + o,
                           a.ag != nullptr ? a.ag + o : nullptr};
        fused_elems(s.n / kV * kV, s.n, s, fi, c, sq, bad);
    }
    const bool more = (a.bucket & ZERO_BUCKET_FIRST) == 0;
    publish_partial(ws, sq, bad, more);
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.run_count = (more ? *a.run_count : 0) + total;
}


// Second pass of the clipped step, per element group: g = g32 * coef from
// the materialised fp32 gradient, then the fused step's update and emit.
__device__ __forceinline__ void cu_load(fvec& g, fvec& p, fvec& m, fvec& v, const float* grad,
                                        const FusedPtrs& f, int64_t j) {
    g = ldg(reinterpret_cast<const fvec*>(grad + j));
    p = ldg(reinterpret_cast<const fvec*>(f.pin + j));
    m = ldg(reinterpret_cast<const fvec*>(f.min_ + j));
    v = ldg(reinterpret_cast<const fvec*>(f.vin + j));
}

__device__ __forceinline__ void cu_finish(const fvec& gv, const fvec& pv, const fvec& mv, const fvec& vv,
                                          const FusedPtrs& f, const AdamScalars& c, double coef, int64_t j) {
    float po[kV], mo[kV], vo[kV];
#pragma unroll
    for (int e = 0; e < kV; ++e)
        adam1(c, static_cast<double>(gv[e]) * coef, pv[e], mv[e], vv[e], po[e], mo[e], vo[e]);
    fvec pw, mw, vw;
#pragma unroll
    for (int e = 0; e < kV; ++e) {
        pw[e] = po[e];
        mw[e] = mo[e];
        vw[e] = vo[e];
    }
    stg(reinterpret_cast<fvec*>(f.pout + j), pw);
    stg(reinterpret_cast<fvec*>(f.mout + j), mw);
    stg(reinterpret_cast<fvec*>(f.vout + j), vw);
    if (f.ag != nullptr) stg(reinterpret_cast<hvec*>(f.ag + j), pack_v(po));
}

// Full groups gi, gi+step, ... < end, two groups ahead from NB rotating
// register sets (as the fused step's prefetch; past the end, group 0 is
// loaded and ignored).
template <int NB>
__device__ void cu_run(int64_t gi, int64_t end, int64_t step, const float* grad, const FusedPtrs& f,
                       const AdamScalars& c, double coef) {
    if (gi >= end) return;
    fvec g[NB], p[NB], m[NB], v[NB];
    cu_load(g[0], p[0], m[0], v[0], grad, f, gi * kV);
    cu_load(g[1], p[1], m[1], v[1], grad, f, (gi + step < end ? gi + step : 0) * kV);
    bool more = true;
    while (more) {
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            if (more) {
                const int ld = (k + 2) % NB;
                const int64_t g2 = gi + 2 * step < end ? gi + 2 * step : 0;
                cu_load(g[ld], p[ld], m[ld], v[ld], grad, f, g2 * kV);
                __builtin_amdgcn_sched_barrier(0);
                cu_finish(g[k], p[k], m[k], v[k], f, c, coef, gi * kV);
                if (gi + step >= end)
                    more = false;
                else
                    gi += step;
            }
        }
    }
}

// Second pass of the clipped step: g = g32 * coef from the materialised
// fp32 gradient, then the update, emit and commit of the fused step.  A
// step whose first pass found an inf/NaN touches nothing but the control
// block (so its all-gather window needs no restore).
__global__ void __launch_bounds__(kBlock) clipped_update_kernel(
    const float* __restrict__ grad, int64_t n, AdamArgs a, double max_norm, Partials ws, int32_t nparts) {
    double sq_in;
    int flag;
    sum_partials(ws, nparts, sq_in, flag);  // the first pass's, identical in every workgroup
    if (flag != 0) return;                  // skipped: commit_kernel records it
    const double r = max_norm / (__builtin_sqrt(sq_in) + 1e-6);
    const double coef = r < 1.0 ? r : 1.0;
    const int cur = a.ctl->cur;
    double b1t, b2t;
    const AdamScalars c = step_scalars(a, b1t, b2t);
    const FusedPtrs f{a.p[cur], a.m[cur], a.v[cur], a.p[cur ^ 1], a.m[cur ^ 1], a.v[cur ^ 1], a.ag};
    const int64_t ngroups = (n + kV - 1) / kV;
    const int64_t nfull = n / kV;
    GroupIter it(ngroups);
    cu_run<4>(it.gi, it.end < nfull ? it.end : nfull, it.step, grad, f, c, coef);
    if (ngroups > nfull) {
        // the ragged tail group, by the lane whose sequence contains it
        const int64_t g = nfull;
        if (g >= it.gi && g < it.end && (g - it.gi) % it.step == 0) {
            for (int64_t e = g * kV; e < n; ++e) {
                float po, mo, vo;
                adam1(c, static_cast<double>(grad[e]) * coef, f.pin[e], f.min_[e], f.vin[e], po, mo, vo);
                f.pout[e] = po;
                f.mout[e] = mo;
                f.vout[e] = vo;
                if (f.ag != nullptr) f.ag[e] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(po));
            }
        }
    }
    (void)b1t;  // the commit kernel recomputes the powers it commits
    (void)b2t;
}

// allgather[j] = fp16(src[j]) for j < n, in the grid-stride group order:
// kEmitU groups a grid stride apart per iteration, all their loads issued
// before their stores (one group at a time measured about 2.5 TB/s of
// read + write), then the remaining groups and the ragged tail one by one.
constexpr int kEmitU = 4;

__device__ __forceinline__ void emit_range(const float* __restrict__ src, uint16_t* __restrict__ ag,
                                           int64_t n) {
    const int64_t ngroups = (n + kV - 1) / kV;
    const int64_t nfull = n / kV;
    GroupIter it(ngroups);
    for (; it.gi + (kEmitU - 1) * it.step < nfull; it.gi += kEmitU * it.step) {
        fvec a[kEmitU];
#pragma unroll
        for (int u = 0; u < kEmitU; ++u) a[u] = ldg(reinterpret_cast<const fvec*>(src + (it.gi + u * it.step) * kV));
#pragma unroll
        for (int u = 0; u < kEmitU; ++u) {
            float x[kV];
#pragma unroll
            for (int e = 0; e < kV; ++e) x[e] = a[u][e];
            stg(reinterpret_cast<hvec*>(ag + (it.gi + u * it.step) * kV), pack_v(x));
        }
    }
    for (; it.gi < it.end; it.gi += it.step) {
        const int64_t gi = it.gi;
        const int64_t j = gi * kV;
        if (gi < nfull) {
            const fvec a = ldg(reinterpret_cast<const fvec*>(src + j));
            float x[kV];
#pragma unroll
            for (int e = 0; e < kV; ++e) x[e] = a[e];
            stg(reinterpret_cast<hvec*>(ag + j), pack_v(x));
        } else {
            for (int64_t e = j; e < n; ++e) {
                const _Float16 h = static_cast<_Float16>(src[e]);
                ag[e] = __builtin_bit_cast(uint16_t, h);
            }
        }
    }
}

__global__ void __launch_bounds__(kBlock) emit_kernel(const float* src, uint16_t* ag, int64_t n) {
    emit_range(src, ag, n);
}

__global__ void __launch_bounds__(kBlock) restore_kernel(const float* p0, const float* p1,
                                                         const zero_step_ctl* ctl, uint16_t* ag,
                                                         int64_t n) {
    if (ctl->overflow == 0) return;
    emit_range(ctl->cur ? p1 : p0, ag, n);
}

// The commit of a fused (or bucketed) step, one launch after it: every
// workgroup sums the step's partials in the same fixed order, workgroup 0
// commits the step in the control block (or records the skip and backs
// off the loss scale), and on a skip every workgroup re-emits its share of
// the all-gather window from the committed master.  A skip never changes
// ctl->cur, so the workgroups that read it race with no write.
//
// Clipped mode (max_norm > 0, one workgroup, after the clipped step's second
// pass): the partials are the first pass's; the coefficient is recomputed
// with the same operations as the second pass used, and a skipped clipped
// step wrote nothing, so there is nothing to re-emit.
__global__ void __launch_bounds__(kBlock) commit_kernel(AdamArgs a, Partials ws, int32_t nparts, int64_t n,
                                                        double max_norm) {
    double sq;
    int flag;
    sum_partials(ws, nparts, sq, flag);
    if (a.bucket != 0 && *a.run_count != a.window_n) flag = 2;  // the buckets missed part of the window
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        double b1t, b2t;
        (void)step_scalars(a, b1t, b2t);
        double coef = 1.0;
        if (max_norm > 0.0) {
            const double r = max_norm / (__builtin_sqrt(sq) + 1e-6);
            coef = r < 1.0 ? r : 1.0;
        }
        commit_step(a, a.ctl->cur, b1t, b2t, flag, sq, flag ? 1.0 : coef);
    }
    if (max_norm == 0.0 && flag != 0 && a.ag != nullptr) emit_range(a.p[a.ctl->cur], a.ag, n);
}

// ------------------------------------------------- Pos+g+p parameter gather
#ifndef ZDP_COPY_U
#define ZDP_COPY_U 4
#endif
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kCopyU = ZDP_COPY_U;  // 16-byte vectors per lane per iteration

// dst[i] = src[i] for i < n (fp16 bit patterns): one piece of a layer
// gather, from one owner's window, by the whole grid.  When src and dst
// agree modulo 16 bytes the body moves 16-byte vectors, kCopyU per lane per
// iteration with all loads issued before the stores, each instruction
// lane-contiguous, and each workgroup a contiguous chunk; the head and tail
// go element-wise.  Otherwise every element moves on its own (2-byte
// accesses, coalesced).  The chunks of a launch's pieces are dealt to the
// workgroups in one rotation (rot: the workgroup next in turn), so no
// workgroup takes the extra chunk of every piece.
__device__ __forceinline__ void copy_piece(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                           int64_t n, int64_t& rot) {
    const uintptr_t sa = reinterpret_cast<uintptr_t>(src), da = reinterpret_cast<uintptr_t>(dst);
    if (((sa ^ da) & 15u) != 0) {
        const int64_t nlanes = static_cast<int64_t>(gridDim.x) * kBlock;
        for (int64_t i = logical_block() * kBlock + threadIdx.x; i < n; i += nlanes) dst[i] = src[i];
        return;
    }
    int64_t head = static_cast<int64_t>(((16u - (da & 15u)) & 15u) / 2u);
    if (head > n) head = n;
    const int64_t nv = (n - head) / 8;
    const u32x4* __restrict__ sv = reinterpret_cast<const u32x4*>(src + head);
    u32x4* __restrict__ dv = reinterpret_cast<u32x4*>(dst + head);
    // full chunks of kCopyU * kBlock vectors, one per workgroup at a time
    // (no predicates, so all kCopyU loads are in flight together)
    constexpr int64_t kChunk = static_cast<int64_t>(kCopyU) * kBlock;
    const int64_t nfull = nv / kChunk;
    const int64_t G = gridDim.x;
    const int64_t lb = logical_block();
    const int64_t first = ((lb - rot) % G + G) % G;
    for (int64_t c = first; c < nfull; c += G) {
        const int64_t base = c * kChunk + threadIdx.x;
        u32x4 v[kCopyU];
#pragma unroll
        for (int u = 0; u < kCopyU; ++u) v[u] = ldg(sv + base + u * kBlock);
#pragma unroll
        for (int u = 0; u < kCopyU; ++u) stg(dv + base + u * kBlock, v[u]);
    }
    // the last partial chunk, the head and the tail: the workgroup next in turn
    if (lb == (rot + nfull) % G) {
        for (int64_t i = nfull * kChunk + threadIdx.x; i < nv; i += kBlock) stg(dv + i, ldg(sv + i));
        for (int64_t i = threadIdx.x; i < head; i += kBlock) dst[i] = src[i];
        for (int64_t i = head + nv * 8 + threadIdx.x; i < n; i += kBlock) dst[i] = src[i];
    }
    rot = (rot + nfull + 1) % G;
}

// The pieces of one launch of a gather (a layer's parts of consecutive
// windows, or the parts of several layers): piece i copies len[i]
// elements from src[i] to dst[i].
constexpr int kMaxPieces = 16;
struct CopyPieces {
    const uint16_t* src[kMaxPieces];
    uint16_t* dst[kMaxPieces];
    int64_t len[kMaxPieces];
    int32_t np;
};

__global__ void __launch_bounds__(kBlock) copy_f16_kernel(CopyPieces t) {
    int64_t rot = 0;
    for (int i = 0; i < t.np; ++i) copy_piece(t.src[i], t.dst[i], t.len[i], rot);
}

// ---------------------------------------------------------------- launchers
constexpr int kMaxDevices = 64;
enum KernelId { kReduce = 0, kFused = 1, kEmit = 2, kRestore = 3, kClip = 4, kCopy = 5, kCommit = 6, kKernels = 7 };
std::atomic<int> g_grid_cache[kKernels][kMaxDevices];  // 0 = not computed yet

// Workgroups that keep every CU of the current device busy at the kernel's
// occupancy (grid-stride loops then cover any n).
int resident_blocks(KernelId id) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 1024;
    int cached = g_grid_cache[id][dev].load(std::memory_order_relaxed);
    if (cached > 0) return cached;
    int cus = 0, per_cu = 0;
    const void* fn = nullptr;
    switch (id) {
        case kReduce: fn = reinterpret_cast<const void*>(reduce_owned_kernel<true>); break;
        case kFused: fn = reinterpret_cast<const void*>(fused_step_kernel); break;
        case kEmit: fn = reinterpret_cast<const void*>(emit_kernel); break;
        case kRestore: fn = reinterpret_cast<const void*>(restore_kernel); break;
        case kClip: fn = reinterpret_cast<const void*>(clipped_update_kernel); break;
        case kCopy: fn = reinterpret_cast<const void*>(copy_f16_kernel); break;
        case kCommit: fn = reinterpret_cast<const void*>(commit_kernel); break;
        default: return 1024;
    }
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kBlock, 0) != hipSuccess ||
        cus <= 0 || per_cu <= 0) {
        (void)hipGetLastError();
        return 1024;
    }
    const int cap = id == kFused    ? ZDP_BPC
                    : id == kReduce ? ZDP_BPC_REDUCE
                    : id == kClip   ? ZDP_BPC_CLIP
                    : id == kCopy   ? ZDP_BPC_COPY
                    : id == kCommit ? 1
                                    : 0;
    if (cap > 0 && per_cu > cap) per_cu = cap;
    int blocks = cus * per_cu;
    if (blocks > zdp::kMaxBlocks) blocks = zdp::kMaxBlocks;
    g_grid_cache[id][dev].store(blocks, std::memory_order_relaxed);
    return blocks;
}

int grid_for(KernelId id, int64_t n) {
    const int64_t groups = (n + kV - 1) / kV;
    const int64_t need = (groups + kBlock - 1) / kBlock;
    int64_t cap = resident_blocks(id);
    if (cap > zdp::kMaxBlocks) cap = zdp::kMaxBlocks;
    int64_t g = need < cap ? need : cap;
    return static_cast<int>(g < 1 ? 1 : g);
}

// Workgroups of one gather piece of n elements: enough chunks of kCopyU
// vectors per lane, at most the resident limit (a multiple of 8, so the
// XCD-contiguous order applies).
int copy_grid(int64_t n) {
    const int64_t chunk = static_cast<int64_t>(kCopyU) * kBlock * 8;
    const int64_t need = (n + chunk - 1) / chunk;
    const int64_t cap = resident_blocks(kCopy);
    const int64_t g = need < cap ? need : cap;
    return static_cast<int>(g < 1 ? 1 : g);
}

int finish_launch() {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        zdp::set_last_hip_error(static_cast<int>(e));
        return ZERO_EHIP;
    }
    return ZERO_OK;
}

// The grid of every launch of a step that accumulates workgroup slots
// (buckets, split windows): the same on every launch on a device.
int fixed_grid(KernelId id) {
    const int r = resident_blocks(id);
    return r < zdp::kMaxBlocks ? r : zdp::kMaxBlocks;
}

#ifndef ZDP_SPLIT_LOG2
#define ZDP_SPLIT_LOG2 24  // elements per launch of a long window: about 2^24 (0: one launch)
#endif
#ifndef ZDP_SPLIT_BIG_LOG2
#define ZDP_SPLIT_BIG_LOG2 23  // the same for Nd >= ZDP_CH_BIG_ND (the 8-group visits)
#endif
#ifndef ZDP_SPLIT_HUGE_ND
#define ZDP_SPLIT_HUGE_ND 256  // from this Nd on, launches of about 2^(ZDP_SPLIT_BIG_LOG2 - 1)
#endif

// A window longer than two launch lengths is stepped in launches of about
// 2^24 elements (2^23 for the big visit shape, Nd >= ZDP_CH_BIG_ND; 2^22
// from Nd = ZDP_SPLIT_HUGE_ND).  One grid-stride launch over 10^8
// elements measured 3-16% slower than the same work in such launches (Nd
// 16, 64 and 400); shorter windows take one launch, where the few
// microseconds an extra launch costs outweigh the gain.  The 8-group visits
// of the big shape run 1-2% faster in launches of 2^23 than of 2^24 (the
// GPT-2-XL shard at Nd = 16 runs 1.4% slower there).  Launches of 2^22
// measured 0.9-1% faster than 2^23 at Nd = 400 and 1-6% slower at Nd 32,
// 48, 64 and 100 (paired, in one process); 256 is a boundary between the
// two measured sides.
int64_t split_elems(int32_t nd) {
    const int l = nd >= ZDP_SPLIT_HUGE_ND ? ZDP_SPLIT_BIG_LOG2 - 1
                  : nd >= ZDP_CH_BIG_ND   ? ZDP_SPLIT_BIG_LOG2
                                          : ZDP_SPLIT_LOG2;
    return l > 0 ? (int64_t{1} << l) : 0;
}

bool split_window(int64_t n, int32_t nd) {
    const int64_t e = split_elems(nd);
    return e > 0 && n > 2 * e;
}

// The launch pieces of a window of n elements at Nd = nd on a grid of
// `grid` workgroups: one piece, or pieces of about split_elems(nd) elements
// when split_window(n, nd) (zdp::plan_pieces).
zdp::Pieces pieces_for(int64_t n, int32_t nd, int64_t grid) {
    if (!split_window(n, nd)) return zdp::Pieces{n, false};
    const int u = nd >= ZDP_CH_BIG_ND ? ZDP_CHB_U : ZDP_CHS_U;
    return zdp::plan_pieces(n, split_elems(nd), zdp::round_elems(grid, nd > kUnroll, u));
}

// Calls launch(off, k) for consecutive pieces [off, off + k) that cover
// [0, n), as pieces_for(n, nd, grid) places them.
template <class Launch>
int for_each_piece(int64_t n, int32_t nd, int64_t grid, Launch&& launch) {
    const zdp::Pieces pc = pieces_for(n, nd, grid);
    int64_t off = 0;
    do {
        const int64_t end = zdp::piece_end(n, pc, off);
        const int rc = launch(off, end - off);
        if (rc != ZERO_OK) return rc;
        off = end;
    } while (off < n);
    return ZERO_OK;
}

SrcArgs piece_src(const SrcArgs& src, int64_t off, int64_t k) {
    SrcArgs sub = src;
    sub.win = src.win + off;
    sub.n = k;
    return sub;
}

AdamArgs piece_args(const AdamArgs& a, int64_t off) {
    AdamArgs b = a;
    for (int i = 0; i < 2; ++i) {
        b.p[i] = a.p[i] + off;
        b.m[i] = a.m[i] + off;
        b.v[i] = a.v[i] + off;
    }
    b.ag = a.ag != nullptr ? a.ag + off : nullptr;
    return b;
}

// Launches the fused kernel over the elements of `src`, whose state and
// all-gather pointers are those of `a`, piece by piece (for_each_piece).
// Every launch accumulates into the workgroup slots except the first when
// `first` (the first launch of a step).  a.window_n must be set.
int launch_fused_range(const SrcArgs& src, const AdamArgs& a, bool first, int grid, const Partials& ws,
                       hipStream_t s) {
    return for_each_piece(src.n, src.nd, grid, [&](int64_t off, int64_t k) {
        AdamArgs b = piece_args(a, off);
        b.bucket = 4 | (first && off == 0 ? ZERO_BUCKET_FIRST : 0);
        fused_step_kernel<<<grid, kBlock, 0, s>>>(piece_src(src, off, k), b, ws);
        return finish_launch();
    });
}

// ---------------------------------------------- allocation-free step
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_addr[kMaxDevices];

// The current device's scratch address (looked up on its first use).
int scratch_addr(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        zdp::set_last_hip_error(e != hipSuccess ? static_cast<int>(e) : static_cast<int>(hipErrorInvalidDevice));
        return ZERO_EHIP;
    }
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || p == nullptr) {
                zdp::set_last_hip_error(e != hipSuccess ? static_cast<int>(e) : static_cast<int>(hipErrorUnknown));
                return ZERO_EHIP;
            }
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return ZERO_OK;
}

}  // namespace

namespace zdp {

int launch_reduce(const SrcArgs& src, float* grad_out, int32_t* overflow, double* sumsq, const Partials& ws,
                  void* stream) {
    const int grid = grid_for(kReduce, src.n);
    (void)hipGetLastError();
    reduce_owned_kernel<false><<<grid, kBlock, 0, static_cast<hipStream_t>(stream)>>>(src, grad_out, overflow,
                                                                                      sumsq, ws, 0);
    return finish_launch();
}

int launch_step(const SrcArgs& whole, const AdamArgs& a_in, const Partials& ws, void* stream) {
    AdamArgs a = a_in;
    const int64_t n = whole.n;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (!split_window(n, whole.nd)) {
        const int grid = grid_for(kFused, n);
        fused_step_kernel<<<grid, kBlock, 0, s>>>(whole, a, ws);
        const int rc = finish_launch();
        if (rc != ZERO_OK) return rc;
        commit_kernel<<<grid_for(kCommit, n), kBlock, 0, s>>>(a, ws, grid, n, 0.0);
        return finish_launch();
    }
    // a long window: consecutive launches accumulating the workgroup slots,
    // as the buckets of one step, then the commit
    a.window_n = n;
    const int grid = fixed_grid(kFused);
    const int rc = launch_fused_range(whole, a, true, grid, ws, s);
    if (rc != ZERO_OK) return rc;
    a.bucket = ZERO_BUCKET_LAST | 4;
    commit_kernel<<<grid_for(kCommit, n), kBlock, 0, s>>>(a, ws, grid, n, 0.0);
    return finish_launch();
}

int launch_step_clipped(const SrcArgs& whole, const AdamArgs& a, float* grad_buf, double max_norm,
                        const Partials& ws, void* stream) {
    const int64_t n = whole.n;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    // a long window takes each pass in pieces; the first pass's pieces run
    // on one grid and accumulate in the workgroup slots
    const int grid1 = split_window(n, whole.nd) ? fixed_grid(kReduce) : grid_for(kReduce, n);
    (void)hipGetLastError();
    int rc = for_each_piece(n, whole.nd, grid1, [&](int64_t off, int64_t k) {
        reduce_owned_kernel<true><<<grid1, kBlock, 0, s>>>(piece_src(whole, off, k), grad_buf + off, nullptr,
                                                            nullptr, ws, off != 0);
        return finish_launch();
    });
    if (rc != ZERO_OK) return rc;
    // the update pass streams g and the state alone: pieces as for small Nd
    rc = for_each_piece(n, 1, fixed_grid(kClip), [&](int64_t off, int64_t k) {
        clipped_update_kernel<<<grid_for(kClip, k), kBlock, 0, s>>>(grad_buf + off, k, piece_args(a, off),
                                                                   max_norm, ws, grid1);
        return finish_launch();
    });
    if (rc != ZERO_OK) return rc;
    commit_kernel<<<1, kBlock, 0, s>>>(a, ws, grid1, n, max_norm);
    return finish_launch();
}

int launch_bucket(const SrcArgs& src, const AdamArgs& a, const AdamArgs& whole, int32_t phase,
                  const Partials& ws, void* stream) {
    // every bucket of a step runs on the same grid: each workgroup adds its
    // partial to its own slot
    const int grid = fixed_grid(kFused);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const int rc = launch_fused_range(src, a, (phase & ZERO_BUCKET_FIRST) != 0, grid, ws, s);
    if (rc != ZERO_OK || (phase & ZERO_BUCKET_LAST) == 0) return rc;
    // the commit, over the whole window
    commit_kernel<<<grid_for(kCommit, whole.window_n), kBlock, 0, s>>>(whole, ws, grid, whole.window_n, 0.0);
    return finish_launch();
}

int launch_buckets(const BucketRun* runs, int32_t nruns, const SrcArgs& common, const AdamArgs& a_in,
                   int32_t phase, const Partials& ws, void* stream) {
    // every launch of a step runs on the same grid (each workgroup adds its
    // partial to its own slot); a run longer than two launch lengths is cut
    // into pieces as a long window is, and consecutive pieces share a
    // launch while they fit in one launch length and kMaxRuns
    const int grid = fixed_grid(kFused);
    const int64_t cap = split_elems(common.nd) > 0 ? split_elems(common.nd) : (int64_t{1} << 62);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    AdamArgs a = a_in;
    bool first = (phase & ZERO_BUCKET_FIRST) != 0;
    RunList rl{};
    int64_t total = 0;
    (void)hipGetLastError();
    auto flush = [&]() {
        if (rl.count == 0) return ZERO_OK;
        a.bucket = 4 | (first ? ZERO_BUCKET_FIRST : 0);
        fused_runs_kernel<<<grid, kBlock, 0, s>>>(rl, common, a, ws);
        first = false;
        rl = RunList{};
        total = 0;
        return finish_launch();
    };
    for (int32_t i = 0; i < nruns; ++i) {
        const BucketRun& r = runs[i];
        const zdp::Pieces pc = pieces_for(r.n, common.nd, grid);
        int64_t off = 0;
        do {
            const int64_t k = zdp::piece_end(r.n, pc, off) - off;
            if (rl.count == kMaxRuns || (rl.count > 0 && total + k > cap)) {
                const int rc = flush();
                if (rc != ZERO_OK) return rc;
            }
            rl.win[rl.count] = r.win + off;
            rl.stride[rl.count] = r.stride;
            rl.n[rl.count] = k;
            rl.off[rl.count] = r.win_off + off;
            ++rl.count;
            total += k;
            off += k;
        } while (off < r.n);
    }
    const int rc = flush();
    if (rc != ZERO_OK || (phase & ZERO_BUCKET_LAST) == 0) return rc;
    a.bucket = ZERO_BUCKET_LAST | 4;
    commit_kernel<<<grid_for(kCommit, a.window_n), kBlock, 0, s>>>(a, ws, grid, a.window_n, 0.0);
    return finish_launch();
}

int launch_gather(const uint16_t* const* windows, int64_t part, const int64_t* ranges, int32_t nranges,
                  uint16_t* const* dsts, void* stream) {
    // the ranges' pieces in order, kMaxPieces per launch (one launch for a
    // layer that touches at most kMaxPieces windows)
    const hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    CopyPieces t{};
    int64_t total = 0;
    auto flush = [&]() {
        if (t.np == 0) return ZERO_OK;
        copy_f16_kernel<<<copy_grid(total), kBlock, 0, s>>>(t);
        t = CopyPieces{};
        total = 0;
        return finish_launch();
    };
    for (int32_t q = 0; q < nranges; ++q) {
        const int64_t lo = ranges[2 * q], hi = ranges[2 * q + 1];
        for (int64_t f = lo; f < hi;) {
            const int64_t r = f / part;
            const int64_t take = ((r + 1) * part < hi ? (r + 1) * part : hi) - f;
            t.src[t.np] = windows[r] + (f - r * part);
            t.dst[t.np] = dsts[q] + (f - lo);
            t.len[t.np] = take;
            ++t.np;
            total += take;
            f += take;
            if (t.np == kMaxPieces) {
                const int rc = flush();
                if (rc != ZERO_OK) return rc;
            }
        }
    }
    return flush();
}

int launch_restore(const float* p0, const float* p1, const zero_step_ctl* ctl, uint16_t* ag, int64_t n,
                   void* stream) {
    const int grid = grid_for(kRestore, n);
    (void)hipGetLastError();
    restore_kernel<<<grid, kBlock, 0, static_cast<hipStream_t>(stream)>>>(p0, p1, ctl, ag, n);
    return finish_launch();
}

int launch_emit(const float* master, uint16_t* ag, int64_t n, void* stream) {
    const int grid = grid_for(kEmit, n);
    (void)hipGetLastError();
    emit_kernel<<<grid, kBlock, 0, static_cast<hipStream_t>(stream)>>>(master, ag, n);
    return finish_launch();
}

int scratch_workspace(void** ws) {
    // every launch of a step uses one slot per workgroup; the scratch holds
    // kMaxBlocks of them (a grid never has more: resident_blocks caps it)
    if (fixed_grid(kFused) > kMaxBlocks || resident_blocks(kCommit) > kMaxBlocks) return ZERO_ECAPACITY;
    return scratch_addr(ws);
}

}  // namespace zdp

// Bandwidth calibration kernels for gfx950, used only by the benchmark to
// measure what HBM attains on the box it runs on, beside the fused step.
//
//   triad_kernel       a[i] = b[i] + q * c[i] (fp32, STREAM's triad: two
//                      read streams and one write stream)
//   stream_mix_kernel  the fused step's exact streams with no arithmetic:
//                      per owned element Nd fp16 slice reads, three fp32
//                      state reads, three fp32 state writes and one fp16
//                      write, with the fused kernel's launch shape (one
//                      256-lane workgroup per CU in XCD-contiguous order,
//                      4 elements per lane per group, non-temporal access,
//                      the same launch pieces of a long window) and its
//                      visit order (the next group's loads ahead for
//                      Nd <= 16; visits of 4 or 8 consecutive 256-element
//                      groups summed in chunks of 2 slices, one chunk
//                      ahead, above; 8 from Nd = 32 when a launch holds at
//                      least one such visit per wave).  The slices are combined with XOR
//                      into the third output, so every load is used; the
//                      other outputs are copies of the inputs.
//   slice_read_kernel  the same launch shape, visit order and launch pieces
//                      with the slice reads alone (2 * Nd bytes per owned
//                      element, nothing stored but one word per workgroup):
//                      the rate the step's slice streams attain without the
//                      state streams and the stores beside them.
//
// Neither kernel is part of the step; the step's kernels live in
// zero_dp_kernels.hip.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/zero_dp.h"
#include "zero_dp_calib.h"
#include "zero_dp_internal.h"

namespace {

constexpr int kBlock = zdp::kBlock;
constexpr int kWaves = zdp::kWaves;
constexpr int kV = 4;  // elements per lane per group
typedef uint32_t hvec __attribute__((ext_vector_type(2)));  // 4 fp16 values
typedef float fvec __attribute__((ext_vector_type(4)));     // 4 fp32 values
typedef uint32_t uvec __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ T ldg(const T* p) {
    return __builtin_nontemporal_load(p);
}

template <typename T>
__device__ __forceinline__ void stg(T* p, const T& v) {
    __builtin_nontemporal_store(v, p);
}

__device__ __forceinline__ int64_t logical_block() {
    const uint32_t g = gridDim.x, b = blockIdx.x;
    if (g % 8 == 0) return static_cast<int64_t>(b % 8) * (g / 8) + b / 8;
    return blockIdx.x;
}

// ------------------------------------------------------------------ triad
constexpr int kTriadU = 4;  // 16-byte vectors per lane per stream in flight

__global__ void __launch_bounds__(kBlock) triad_kernel(float* __restrict__ a, const float* __restrict__ b,
                                                       const float* __restrict__ c, float q, int64_t n) {
    const int64_t nv = n / 4;
    fvec* av = reinterpret_cast<fvec*>(a);
    const fvec* bv = reinterpret_cast<const fvec*>(b);
    const fvec* cv = reinterpret_cast<const fvec*>(c);
    constexpr int64_t kChunk = static_cast<int64_t>(kTriadU) * kBlock;
    const int64_t nfull = nv / kChunk;
    for (int64_t ch = logical_block(); ch < nfull; ch += gridDim.x) {
        const int64_t base = ch * kChunk + threadIdx.x;
        fvec x[kTriadU], y[kTriadU];
#pragma unroll
        for (int u = 0; u < kTriadU; ++u) {
            x[u] = ldg(bv + base + u * kBlock);
            y[u] = ldg(cv + base + u * kBlock);
        }
#pragma unroll
        for (int u = 0; u < kTriadU; ++u) {
            fvec r;
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = x[u][e] + q * y[u][e];
            stg(av + base + u * kBlock, r);
        }
    }
    if (blockIdx.x == gridDim.x - 1) {
        for (int64_t i = nfull * kChunk + threadIdx.x; i < nv; i += kBlock) {
            const fvec x = ldg(bv + i), y = ldg(cv + i);
            fvec r;
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = x[e] + q * y[e];
            stg(av + i, r);
        }
        for (int64_t i = nv * 4 + threadIdx.x; i < n; i += kBlock) a[i] = b[i] + q * c[i];
    }
}

// The step's choice of visit shape: 8-group visits from Nd = 32 when the
// launch holds at least one per wave, else 4-group visits.
__device__ __forceinline__ bool big_visits(int nd, int64_t nfull) {
    return nd >= 32 && (nfull + 64 * 8 - 1) / (64 * 8) >= static_cast<int64_t>(gridDim.x) * kWaves;
}

// ------------------------------------------------------------- stream mix
struct MixArgs {
    const uint16_t* win;  // slice 0 of the window
    int64_t stride;       // elements between slices
    int64_t n;
    int32_t nd;
    const float* in[3];
    float* out[3];
    uint16_t* out16;
};

__device__ __forceinline__ hvec ldh(const uint16_t* p) { return ldg(reinterpret_cast<const hvec*>(p)); }

__device__ __forceinline__ uint32_t xor_words(const hvec& w) { return w[0] ^ w[1]; }

// Stores of one group: outputs 0 and 1 copy the inputs, output 2 is input 2
// with the slices' XOR folded into its bits, the fp16 output the top half
// of input 0's bits.
__device__ __forceinline__ void mix_store(const MixArgs& a, int64_t j, const fvec& p, const fvec& m,
                                          const fvec& v, uint32_t x) {
    stg(reinterpret_cast<fvec*>(a.out[0] + j), p);
    stg(reinterpret_cast<fvec*>(a.out[1] + j), m);
    const uvec vb = __builtin_bit_cast(uvec, v);
    uvec vo;
#pragma unroll
    for (int e = 0; e < 4; ++e) vo[e] = vb[e] ^ x;
    stg(reinterpret_cast<fvec*>(a.out[2] + j), __builtin_bit_cast(fvec, vo));
    const uvec pb = __builtin_bit_cast(uvec, p);
    hvec h;
    h[0] = (pb[0] >> 16) | (pb[1] & 0xffff0000u);
    h[1] = (pb[2] >> 16) | (pb[3] & 0xffff0000u);
    stg(reinterpret_cast<hvec*>(a.out16 + j), h);
}

// Elements [e0, n) one at a time (the ragged tail).
__device__ void mix_elems(const MixArgs& a, int64_t e0) {
    for (int64_t e = e0; e < a.n; ++e) {
        uint32_t x = 0;
        for (int k = 0; k < a.nd; ++k) x ^= a.win[e + static_cast<int64_t>(k) * a.stride];
        const float p = a.in[0][e];
        a.out[0][e] = p;
        a.out[1][e] = a.in[1][e];
        a.out[2][e] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, a.in[2][e]) ^ x);
        a.out16[e] = static_cast<uint16_t>(__builtin_bit_cast(uint32_t, p) >> 16);
    }
}

// Nd = R <= 16: one group per lane at a time in grid-stride order, the next
// group's R + 3 loads issued before this group's stores (past the end a
// lane loads group 0 and ignores it).
template <int R>
__device__ void mix_pf(const MixArgs& a, int64_t nfull) {
    int64_t gi = logical_block() * kBlock + threadIdx.x;
    const int64_t step = static_cast<int64_t>(gridDim.x) * kBlock;
    if (gi >= nfull) return;
    hvec w[R];
    fvec p, m, v;
    auto load = [&](int64_t g) {
        const int64_t j = g * kV;
        p = ldg(reinterpret_cast<const fvec*>(a.in[0] + j));
        m = ldg(reinterpret_cast<const fvec*>(a.in[1] + j));
        v = ldg(reinterpret_cast<const fvec*>(a.in[2] + j));
#pragma unroll
        for (int k = 0; k < R; ++k) w[k] = ldh(a.win + j + static_cast<int64_t>(k) * a.stride);
    };
    load(gi);
    for (;;) {
        const int64_t gn = gi + step;
        hvec wc[R];
#pragma unroll
        for (int k = 0; k < R; ++k) wc[k] = w[k];
        const fvec pc = p, mc = m, vc = v;
        load(gn < nfull ? gn : 0);
        __builtin_amdgcn_sched_barrier(0);
        uint32_t x = 0;
#pragma unroll
        for (int k = 0; k < R; ++k) x ^= xor_words(wc[k]);
        mix_store(a, gi * kV, pc, mc, vc, x);
        if (gn >= nfull) break;
        gi = gn;
    }
}

template <int R>
__device__ __forceinline__ bool mix_pf_dispatch(const MixArgs& a, int64_t nfull) {
    if constexpr (R >= 1) {
        if (a.nd == R) {
            mix_pf<R>(a, nfull);
            return true;
        }
        return mix_pf_dispatch<R - 1>(a, nfull);
    }
    return false;
}

template <int U, int R>
__device__ __forceinline__ void mix_chunk_load(hvec (&w)[R][U], const int64_t (&j)[U], const uint16_t* win,
                                               int64_t stride, int k0) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int u = 0; u < U; ++u) w[r][u] = ldh(win + j[u] + static_cast<int64_t>(k0 + r) * stride);
}

template <int U, int R>
__device__ __forceinline__ void mix_chunk_xor(uint32_t (&x)[U], const hvec (&w)[R][U]) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] ^= xor_words(w[r][u]);
}

// The step's rule for a launch whose visits of U groups end in a partial
// round: that round runs in quarter visits when it holds at most a quarter
// of the waves' visits (U >= 8), in half visits when at most half.  Returns
// the tail's visit size (0: no split) and sets nmain, the groups before it.
__device__ __forceinline__ int tail_visit_groups(int64_t nfull, int u, int64_t nwaves, int64_t& nmain) {
    nmain = nfull;
    const int64_t nvis = (nfull + 64 * u - 1) / (64 * u);
    const int64_t full = nvis / nwaves * nwaves;
    const int64_t t = nvis - full;
    if (full == 0 || t == 0) return 0;
    int tu = 0;
    if (u >= 8 && 4 * t <= nwaves)
        tu = u / 4;
    else if (2 * t <= nwaves)
        tu = u / 2;
    if (tu != 0) nmain = full * 64 * u;
    return tu;
}

// Nd > 16: groups [g0, nfull), wave w taking visits w, w + W, ... of U
// consecutive 256-element groups (lane l holds elements 4l .. 4l+3 of
// each); a visit's slices come in chunks of R, the next chunk's loads
// issued before this chunk is folded.  Groups past nfull load group g0
// and store nothing.
template <int U, int R>
__device__ void mix_visits_from(const MixArgs& a, int64_t g0, int64_t nfull, int64_t wave, int lane,
                                int64_t nwaves) {
    const int64_t ng = nfull - g0;
    const int64_t nvis = (ng + 64 * U - 1) / (64 * U);
    const int nfc = a.nd / R;
    for (int64_t vi = wave; vi < nvis; vi += nwaves) {
        int64_t j[U];
        bool act[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t g = (vi * U + u) * 64 + lane;
            act[u] = g < ng;
            j[u] = (g0 + (act[u] ? g : 0)) * kV;
        }
        fvec p[U], m[U], v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            p[u] = ldg(reinterpret_cast<const fvec*>(a.in[0] + j[u]));
            m[u] = ldg(reinterpret_cast<const fvec*>(a.in[1] + j[u]));
            v[u] = ldg(reinterpret_cast<const fvec*>(a.in[2] + j[u]));
        }
        uint32_t x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = 0;
        hvec wa[R][U], wb[R][U];
        mix_chunk_load<U, R>(wa, j, a.win, a.stride, 0);
        int c = 0;
        for (;;) {
            if (c + 1 < nfc) mix_chunk_load<U, R>(wb, j, a.win, a.stride, (c + 1) * R);
            __builtin_amdgcn_sched_barrier(0);
            mix_chunk_xor<U, R>(x, wa);
            if (++c >= nfc) break;
            if (c + 1 < nfc) mix_chunk_load<U, R>(wa, j, a.win, a.stride, (c + 1) * R);
            __builtin_amdgcn_sched_barrier(0);
            mix_chunk_xor<U, R>(x, wb);
            if (++c >= nfc) break;
        }
        for (int k = nfc * R; k < a.nd; ++k)
#pragma unroll
            for (int u = 0; u < U; ++u) x[u] ^= xor_words(ldh(a.win + j[u] + static_cast<int64_t>(k) * a.stride));
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (act[u]) mix_store(a, j[u], p[u], m[u], v[u], x[u]);
    }
}

template <int U, int R>
__device__ void mix_visits(const MixArgs& a, int64_t nfull) {
    const int64_t wave = logical_block() * kWaves + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * kWaves;
    int64_t nmain;
    const int tu = tail_visit_groups(nfull, U, nwaves, nmain);
    mix_visits_from<U, R>(a, 0, nmain, wave, lane, nwaves);
    if (tu == U / 2) mix_visits_from<U / 2, R>(a, nmain, nfull, wave, lane, nwaves);
    if constexpr (U >= 8) {
        if (tu == U / 4) mix_visits_from<U / 4, R>(a, nmain, nfull, wave, lane, nwaves);
    }
    // the ragged tail, by the lane that would hold group nfull
    if (a.n > nfull * kV && (nfull / (64 * U)) % nwaves == wave && nfull % 64 == lane) mix_elems(a, nfull * kV);
}

__global__ void __launch_bounds__(kBlock) stream_mix_kernel(MixArgs a) {
    const int64_t nfull = a.n / kV;
    if (a.nd <= 16) {
        (void)mix_pf_dispatch<16>(a, nfull);
        // the ragged tail group, by the lane whose grid-stride sequence holds it
        const int64_t gi = logical_block() * kBlock + threadIdx.x;
        const int64_t step = static_cast<int64_t>(gridDim.x) * kBlock;
        if (a.n > nfull * kV && nfull >= gi && (nfull - gi) % step == 0) mix_elems(a, nfull * kV);
    } else if (big_visits(a.nd, nfull)) {
        mix_visits<8, 2>(a, nfull);
    } else {
        mix_visits<4, 2>(a, nfull);
    }
}

// ------------------------------------------------------------- slice read
struct ReadArgs {
    const uint16_t* win;  // slice 0 of the window (this launch's piece)
    int64_t stride;       // elements between slices
    int64_t n;
    int32_t nd;
    uint32_t* sink;
};

// Elements [e0, n) one at a time: the XOR of element e's slices goes to the
// low half of the word for even e and to the high half for odd e (a piece
// starts at an even element of the window, so the halves agree with the
// 4-element groups' word pairs).
__device__ uint32_t read_elems(const ReadArgs& a, int64_t e0) {
    uint32_t x = 0;
    for (int64_t e = e0; e < a.n; ++e) {
        uint32_t y = 0;
        for (int k = 0; k < a.nd; ++k) y ^= a.win[e + static_cast<int64_t>(k) * a.stride];
        x ^= (e & 1) ? (y << 16) : y;
    }
    return x;
}

// Nd = R <= 16: one group per lane at a time in grid-stride order, the next
// group's R loads issued before this group is folded (past the end a lane
// loads group 0 and ignores it).
template <int R>
__device__ uint32_t read_pf(const ReadArgs& a, int64_t nfull) {
    int64_t gi = logical_block() * kBlock + threadIdx.x;
    const int64_t step = static_cast<int64_t>(gridDim.x) * kBlock;
    uint32_t x = 0;
    if (gi >= nfull) return x;
    hvec w[R];
    auto load = [&](int64_t g) {
#pragma unroll
        for (int k = 0; k < R; ++k) w[k] = ldh(a.win + g * kV + static_cast<int64_t>(k) * a.stride);
    };
    load(gi);
    for (;;) {
        const int64_t gn = gi + step;
        hvec wc[R];
#pragma unroll
        for (int k = 0; k < R; ++k) wc[k] = w[k];
        load(gn < nfull ? gn : 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < R; ++k) x ^= xor_words(wc[k]);
        if (gn >= nfull) break;
        gi = gn;
    }
    return x;
}

template <int R>
__device__ __forceinline__ uint32_t read_pf_dispatch(const ReadArgs& a, int64_t nfull) {
    if constexpr (R >= 1) {
        if (a.nd == R) return read_pf<R>(a, nfull);
        return read_pf_dispatch<R - 1>(a, nfull);
    }
    return 0;
}

// Nd > 16: the stream-mix kernel's visits over groups [g0, nfull) (U
// consecutive 256-element groups per wave visit, chunks of R slices, the
// next chunk ahead) with no state loads and no stores.  Groups past nfull
// load group g0 and are not folded.
template <int U, int R>
__device__ uint32_t read_visits_from(const ReadArgs& a, int64_t g0, int64_t nfull, int64_t wave, int lane,
                                     int64_t nwaves) {
    const int64_t ng = nfull - g0;
    const int64_t nvis = (ng + 64 * U - 1) / (64 * U);
    const int nfc = a.nd / R;
    uint32_t x = 0;
    for (int64_t vi = wave; vi < nvis; vi += nwaves) {
        int64_t j[U];
        bool act[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t g = (vi * U + u) * 64 + lane;
            act[u] = g < ng;
            j[u] = (g0 + (act[u] ? g : 0)) * kV;
        }
        uint32_t xs[U];
#pragma unroll
        for (int u = 0; u < U; ++u) xs[u] = 0;
        hvec wa[R][U], wb[R][U];
        mix_chunk_load<U, R>(wa, j, a.win, a.stride, 0);
        int c = 0;
        for (;;) {
            if (c + 1 < nfc) mix_chunk_load<U, R>(wb, j, a.win, a.stride, (c + 1) * R);
            __builtin_amdgcn_sched_barrier(0);
            mix_chunk_xor<U, R>(xs, wa);
            if (++c >= nfc) break;
            if (c + 1 < nfc) mix_chunk_load<U, R>(wa, j, a.win, a.stride, (c + 1) * R);
            __builtin_amdgcn_sched_barrier(0);
            mix_chunk_xor<U, R>(xs, wb);
            if (++c >= nfc) break;
        }
        for (int k = nfc * R; k < a.nd; ++k)
#pragma unroll
            for (int u = 0; u < U; ++u) xs[u] ^= xor_words(ldh(a.win + j[u] + static_cast<int64_t>(k) * a.stride));
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (act[u]) x ^= xs[u];
    }
    return x;
}

template <int U, int R>
__device__ uint32_t read_visits(const ReadArgs& a, int64_t nfull) {
    const int64_t wave = logical_block() * kWaves + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * kWaves;
    int64_t nmain;
    const int tu = tail_visit_groups(nfull, U, nwaves, nmain);
    uint32_t x = read_visits_from<U, R>(a, 0, nmain, wave, lane, nwaves);
    if (tu == U / 2) x ^= read_visits_from<U / 2, R>(a, nmain, nfull, wave, lane, nwaves);
    if constexpr (U >= 8) {
        if (tu == U / 4) x ^= read_visits_from<U / 4, R>(a, nmain, nfull, wave, lane, nwaves);
    }
    // the ragged tail, by the lane that would hold group nfull
    if (a.n > nfull * kV && (nfull / (64 * U)) % nwaves == wave && nfull % 64 == lane) x ^= read_elems(a, nfull * kV);
    return x;
}

__global__ void __launch_bounds__(kBlock) slice_read_kernel(ReadArgs a) {
    const int64_t nfull = a.n / kV;
    uint32_t x;
    if (a.nd <= 16) {
        x = read_pf_dispatch<16>(a, nfull);
        const int64_t gi = logical_block() * kBlock + threadIdx.x;
        const int64_t step = static_cast<int64_t>(gridDim.x) * kBlock;
        if (a.n > nfull * kV && nfull >= gi && (nfull - gi) % step == 0) x ^= read_elems(a, nfull * kV);
    } else if (big_visits(a.nd, nfull)) {
        x = read_visits<8, 2>(a, nfull);
    } else {
        x = read_visits<4, 2>(a, nfull);
    }
    // one word per workgroup: the waves' XORs, then one atomic XOR
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), o));
    __shared__ uint32_t part[kWaves];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) t ^= part[w];
        atomicXor(a.sink, t);
    }
}

// One workgroup per CU of the current device (a multiple of 8 on MI355X,
// so the XCD-contiguous order applies).
int cu_grid() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                 hipSuccess || cus <= 0) {
        (void)hipGetLastError();
        return 256;
    }
    return cus;
}

// The fused step's launch pieces: about 2^22 elements from Nd = 256 up,
// 2^23 from Nd = 32 and 2^24 below, placed as the step places them
// (zdp::plan_pieces; multiples of 1024, so every piece starts at an even
// element), when the window is longer than two of them, else one launch.
zdp::Pieces pieces_for(int64_t n, int32_t nd, int grid) {
    const int64_t e = nd >= 256 ? (int64_t{1} << 22) : nd >= 32 ? (int64_t{1} << 23) : (int64_t{1} << 24);
    if (n <= 2 * e) return zdp::Pieces{n, false};
    return zdp::plan_pieces(n, e, zdp::round_elems(grid, nd > 16, nd >= 32 ? 8 : 4));
}

int finish() {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        zdp::set_last_hip_error(static_cast<int>(e));
        return ZERO_EHIP;
    }
    return ZERO_OK;
}

}  // namespace

namespace zdp {

int launch_calib_triad(float* a, const float* b, const float* c, float q, int64_t n, void* stream) {
    (void)hipGetLastError();
    triad_kernel<<<cu_grid(), kBlock, 0, static_cast<hipStream_t>(stream)>>>(a, b, c, q, n);
    return finish();
}

int launch_calib_mix(const SrcArgs& src, const float* const* in, float* const* out, uint16_t* out16, void* stream) {
    const int64_t n = src.n;
    const int grid = cu_grid();
    const zdp::Pieces pc = pieces_for(n, src.nd, grid);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    int64_t off = 0;
    do {
        const int64_t k = zdp::piece_end(n, pc, off) - off;
        MixArgs a;
        a.win = src.win + off;
        a.stride = src.stride;
        a.n = k;
        a.nd = src.nd;
        for (int i = 0; i < 3; ++i) {
            a.in[i] = in[i] + off;
            a.out[i] = out[i] + off;
        }
        a.out16 = out16 + off;
        stream_mix_kernel<<<grid, kBlock, 0, s>>>(a);
        const int rc = finish();
        if (rc != ZERO_OK) return rc;
        off += k;
    } while (off < n);
    return ZERO_OK;
}


int launch_calib_slice_read(const SrcArgs& src, uint32_t* sink, void* stream) {
    const int64_t n = src.n;
    const int grid = cu_grid();
    const zdp::Pieces pc = pieces_for(n, src.nd, grid);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    int64_t off = 0;
    do {
        const int64_t k = zdp::piece_end(n, pc, off) - off;
        ReadArgs a;
        a.win = src.win + off;
        a.stride = src.stride;
        a.n = k;
        a.nd = src.nd;
        a.sink = sink;
        slice_read_kernel<<<grid, kBlock, 0, s>>>(a);
        const int rc = finish();
        if (rc != ZERO_OK) return rc;
        off += k;
    } while (off < n);
    return ZERO_OK;
}

}  // namespace zdp

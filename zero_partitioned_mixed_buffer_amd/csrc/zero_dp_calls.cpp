// Asynchronous entry points of the ZeRO-DP owned-partition library: the
// host-side argument validation of every call, then the device launchers
// (zero_dp_kernels.hip).  Plain C++ with no HIP types, so that this unit
// can also be built for the host alone (with sanitizers), against launchers
// that never reach a device.
//
// Every call checks what the host can check before anything is enqueued:
// null pointers, counts, alignment of the 16-byte vector operands, int64
// overflow of every size and offset, and the overlap of every output with
// every input (an output that aliases an input would be read after it was
// written in a single streaming pass).
#include <cstdint>

#include "../../include/zero_dp.h"
#include "zero_dp_calib.h"
#include "zero_dp_internal.h"

namespace {

using zdp::AdamArgs;
using zdp::Partials;
using zdp::SrcArgs;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

// Two non-empty byte ranges share a byte.
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo < a.hi && b.lo < b.hi; }

Range bytes_of(const void* p, int64_t n, int64_t elem) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + static_cast<uintptr_t>(n) * static_cast<uintptr_t>(elem)};
}

bool any_overlap(const Range* r, int nr) {
    for (int i = 0; i < nr; ++i)
        for (int k = i + 1; k < nr; ++k)
            if (overlap(r[i], r[k])) return true;
    return false;
}

// Validates a gradient source and returns the byte span its slices cover.
int check_src(const zero_grad_src* src, Range* span) {
    if (src == nullptr || src->nd < 1 || src->nd >= 8192 || src->n < 0 || src->elem_off < 0 ||
        src->reserved != 0)
        return ZERO_EINVAL;
    if (src->base == nullptr && src->n != 0) return ZERO_EINVAL;
    if (!(src->loss_scale > 0.0) || !__builtin_isfinite(src->loss_scale) ||
        !__builtin_isfinite(1.0 / src->loss_scale))
        return ZERO_EINVAL;
    if (src->nd > 1 && src->slice_stride < 0) return ZERO_EINVAL;
    if (!aligned16(src->base) || src->elem_off % 8 != 0) return ZERO_EALIGN;
    if (src->nd > 1 && src->slice_stride % 8 != 0) return ZERO_EALIGN;
    int64_t last = 0, end = 0, bytes = 0;
    const int64_t stride = src->nd > 1 ? src->slice_stride : 0;
    if (zdp::mul_overflows(static_cast<int64_t>(src->nd - 1), stride, &last) ||
        zdp::add_overflows(last, src->elem_off, &last) || zdp::add_overflows(last, src->n, &end) ||
        zdp::mul_overflows(end, 2, &bytes))
        return ZERO_EOVERFLOW;
    span->lo = reinterpret_cast<uintptr_t>(src->base + src->elem_off);
    span->hi = reinterpret_cast<uintptr_t>(src->base) + static_cast<uintptr_t>(bytes);
    return ZERO_OK;
}

// The kernels' view of a validated source: 1/L is the host's IEEE division
// (the kernels repeat the same division for a dynamic scale).
SrcArgs make_src(const zero_grad_src* src, const zero_step_ctl* dyn = nullptr) {
    SrcArgs s;
    s.win = src->base + src->elem_off;
    s.stride = src->nd > 1 ? src->slice_stride : 0;
    s.n = src->n;
    s.nd = src->nd;
    s.inv_scale = 1.0 / src->loss_scale;
    s.dyn = dyn;
    return s;
}

Partials make_ws(void* workspace) {
    char* w = static_cast<char*>(workspace);
    Partials p;
    p.ticket = reinterpret_cast<uint32_t*>(w + zdp::kWsTicket);
    p.sq = reinterpret_cast<double*>(w + zdp::kWsPartSq);
    p.flag = reinterpret_cast<int32_t*>(w + zdp::kWsPartFlag);
    return p;
}

// Validates the state, hyperparameters, all-gather window, control block
// and workspace of a step over a window of n elements, fills the kernel
// arguments (the window's pointers), and lists the byte ranges the step
// writes or owns in r[0 .. *nr) (r holds at least 10).  `grad_buf` (the
// clipped path's fp32 gradient) may be null.
int check_window(const zero_adam_state* st, const zero_adam_hp* hp, int64_t n, uint16_t* allgather,
                 int64_t allgather_off, void* workspace, float* grad_buf, AdamArgs* a, Range* r, int* nr) {
    if (st == nullptr || hp == nullptr || st->ctl == nullptr || workspace == nullptr) return ZERO_EINVAL;
    if (!(hp->lr >= 0.0) || !__builtin_isfinite(hp->lr) || !(hp->beta1 >= 0.0 && hp->beta1 < 1.0) ||
        !(hp->beta2 >= 0.0 && hp->beta2 < 1.0) || !(hp->eps > 0.0) || !__builtin_isfinite(hp->eps) ||
        !(hp->weight_decay >= 0.0) || !__builtin_isfinite(hp->weight_decay) ||
        !(hp->max_grad_norm >= 0.0) || !__builtin_isfinite(hp->max_grad_norm) || hp->reserved != 0 ||
        hp->scale_interval < 0)
        return ZERO_EINVAL;
    if (hp->scale_interval > 0 &&
        (!(hp->scale_growth > 0.0) || !__builtin_isfinite(hp->scale_growth) || !(hp->scale_backoff > 0.0) ||
         !__builtin_isfinite(hp->scale_backoff)))
        return ZERO_EINVAL;
    int64_t b4 = 0;
    if (n < 0) return ZERO_EINVAL;
    if (zdp::mul_overflows(n, 4, &b4)) return ZERO_EOVERFLOW;
    float* arrs[7] = {st->master[0],     st->master[1],     st->exp_avg[0], st->exp_avg[1],
                      st->exp_avg_sq[0], st->exp_avg_sq[1], grad_buf};
    int k = 0;
    for (int i = 0; i < 7; ++i) {
        if (i == 6 && grad_buf == nullptr) continue;
        if (arrs[i] == nullptr && n != 0) return ZERO_EINVAL;
        if (!aligned16(arrs[i])) return ZERO_EALIGN;
        r[k++] = bytes_of(arrs[i], n, 4);
    }
    if (!aligned16(workspace)) return ZERO_EALIGN;
    uint16_t* ag = nullptr;
    if (allgather != nullptr) {
        if (allgather_off < 0) return ZERO_EINVAL;
        int64_t e = 0;
        if (zdp::add_overflows(allgather_off, n, &e) || zdp::mul_overflows(e, 2, &e)) return ZERO_EOVERFLOW;
        ag = allgather + allgather_off;
        if (!aligned16(ag)) return ZERO_EALIGN;
        r[k++] = bytes_of(ag, n, 2);
    }
    // the control block and the workspace must not overlap any data either
    if ((reinterpret_cast<uintptr_t>(st->ctl) & 7u) != 0) return ZERO_EALIGN;
    r[k++] = bytes_of(st->ctl, 1, static_cast<int64_t>(sizeof(zero_step_ctl)));
    r[k++] = bytes_of(workspace, 1, zdp::kWsBytes);
    if (any_overlap(r, k)) return ZERO_EALIAS;
    *nr = k;
    for (int i = 0; i < 2; ++i) {
        a->p[i] = st->master[i];
        a->m[i] = st->exp_avg[i];
        a->v[i] = st->exp_avg_sq[i];
    }
    a->ctl = st->ctl;
    a->lr = hp->lr;
    a->b1 = hp->beta1;
    a->b2 = hp->beta2;
    a->eps = hp->eps;
    a->wd = hp->weight_decay;
    a->ag = ag;
    a->growth = hp->scale_growth;
    a->backoff = hp->scale_backoff;
    a->interval = hp->scale_interval;
    a->bucket = 0;
    a->window_n = n;
    a->run_count = reinterpret_cast<int64_t*>(static_cast<char*>(workspace) + zdp::kWsRunCount);
    return ZERO_OK;
}

// Validates the arguments of a step (fused or clipped) over the window of
// src->n elements and fills the kernel arguments.
int check_step(const zero_grad_src* src, const zero_adam_state* st, const zero_adam_hp* hp,
               uint16_t* allgather, int64_t allgather_off, void* workspace, float* grad_buf, AdamArgs* a) {
    Range span{};
    const int rc = check_src(src, &span);
    if (rc != ZERO_OK) return rc;
    Range r[11];
    int nr = 0;
    const int rc2 = check_window(st, hp, src->n, allgather, allgather_off, workspace, grad_buf, a, r, &nr);
    if (rc2 != ZERO_OK) return rc2;
    for (int i = 0; i < nr; ++i)
        if (overlap(r[i], span)) return ZERO_EALIAS;
    return ZERO_OK;
}

// Validates gather ranges [lo, hi) of a Psi = nd * part flat buffer, their
// windows and destinations; an empty range is valid and gathers nothing.
int check_gather(const uint16_t* const* windows, int32_t nd, int64_t part, const int64_t* ranges,
                 int32_t nranges, uint16_t* const* dsts) {
    if (windows == nullptr || nd < 1 || part < 1 || nranges < 0 || (nranges > 0 && (ranges == nullptr ||
                                                                                      dsts == nullptr)))
        return ZERO_EINVAL;
    int64_t total = 0;
    if (zdp::mul_overflows(static_cast<int64_t>(nd), part, &total)) return ZERO_EOVERFLOW;
    for (int32_t q = 0; q < nranges; ++q) {
        const int64_t lo = ranges[2 * q], hi = ranges[2 * q + 1];
        if (lo < 0 || hi < lo || hi > total) return ZERO_EINVAL;
        const int64_t n = hi - lo;
        if (n == 0) continue;  // nothing to gather
        uint16_t* dst = dsts[q];
        int64_t bytes = 0;
        if (dst == nullptr) return ZERO_EINVAL;
        if (zdp::mul_overflows(n, 2, &bytes)) return ZERO_EOVERFLOW;
        if ((reinterpret_cast<uintptr_t>(dst) & 1u) != 0) return ZERO_EALIGN;
        const Range out = bytes_of(dst, n, 2);
        // every piece is validated before anything is launched; a
        // destination may overlap no window piece any range reads, nor
        // another range's destination
        for (int32_t q2 = 0; q2 < nranges; ++q2) {
            const int64_t lo2 = ranges[2 * q2], hi2 = ranges[2 * q2 + 1];
            if (lo2 < 0 || hi2 < lo2 || hi2 > total) return ZERO_EINVAL;
            if (q2 != q && hi2 > lo2 && dsts[q2] != nullptr && overlap(out, bytes_of(dsts[q2], hi2 - lo2, 2)))
                return ZERO_EALIAS;
            for (int64_t f = lo2; f < hi2;) {
                const int64_t r = f / part;
                const int64_t take = ((r + 1) * part < hi2 ? (r + 1) * part : hi2) - f;
                const uint16_t* w = windows[r];
                if (w == nullptr) return ZERO_EINVAL;
                if ((reinterpret_cast<uintptr_t>(w) & 1u) != 0) return ZERO_EALIGN;
                if (overlap(bytes_of(w + (f - r * part), take, 2), out)) return ZERO_EALIAS;
                f += take;
            }
        }
    }
    return ZERO_OK;
}

}  // namespace

extern "C" {

int64_t zero_workspace_bytes(void) { return zdp::kWsBytes; }

int zero_reduce_owned(const zero_grad_src* src, float* grad_out, int32_t* overflow, double* sumsq,
                      void* workspace, void* stream) {
    Range span{};
    const int rc = check_src(src, &span);
    if (rc != ZERO_OK) return rc;
    if (overflow == nullptr || sumsq == nullptr || workspace == nullptr) return ZERO_EINVAL;
    if (!aligned16(workspace) || (reinterpret_cast<uintptr_t>(overflow) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(sumsq) & 7u) != 0)
        return ZERO_EALIGN;
    Range r[5];
    int nr = 0;
    r[nr++] = span;
    r[nr++] = bytes_of(overflow, 1, 4);
    r[nr++] = bytes_of(sumsq, 1, 8);
    r[nr++] = bytes_of(workspace, 1, zdp::kWsBytes);
    if (grad_out != nullptr) {
        if (!aligned16(grad_out)) return ZERO_EALIGN;
        int64_t b = 0;
        if (zdp::mul_overflows(src->n, 4, &b)) return ZERO_EOVERFLOW;
        r[nr++] = bytes_of(grad_out, src->n, 4);
    }
    if (any_overlap(r, nr)) return ZERO_EALIAS;
    return zdp::launch_reduce(make_src(src), grad_out, overflow, sumsq, make_ws(workspace), stream);
}

int zero_adam_step(const zero_grad_src* src, const zero_adam_state* st, const zero_adam_hp* hp,
                   uint16_t* allgather, int64_t allgather_off, void* workspace, void* stream) {
    AdamArgs a;
    const int rc = check_step(src, st, hp, allgather, allgather_off, workspace, nullptr, &a);
    if (rc != ZERO_OK) return rc;
    if (hp->max_grad_norm != 0.0) return ZERO_EINVAL;  // clipping needs the two-pass entry point
    return zdp::launch_step(make_src(src, hp->scale_interval > 0 ? st->ctl : nullptr), a, make_ws(workspace),
                            stream);
}

int zero_adam_step_noalloc(const zero_grad_src* src, const zero_adam_state* st, const zero_adam_hp* hp,
                           uint16_t* allgather, int64_t allgather_off, void* stream) {
    // the step of zero_adam_step on this device's library-held scratch:
    // its first launch writes every slot and the count its commit reads, so
    // nothing needs clearing between calls
    void* ws = nullptr;
    const int rc = zdp::scratch_workspace(&ws);
    if (rc != ZERO_OK) return rc;
    return zero_adam_step(src, st, hp, allgather, allgather_off, ws, stream);
}

int zero_adam_step_clipped(const zero_grad_src* src, const zero_adam_state* st, const zero_adam_hp* hp,
                           float* grad_buf, uint16_t* allgather, int64_t allgather_off, void* workspace,
                           void* stream) {
    AdamArgs a;
    if (grad_buf == nullptr && src != nullptr && src->n != 0) return ZERO_EINVAL;
    const int rc = check_step(src, st, hp, allgather, allgather_off, workspace, grad_buf, &a);
    if (rc != ZERO_OK) return rc;
    if (!(hp->max_grad_norm > 0.0) || !__builtin_isfinite(hp->max_grad_norm)) return ZERO_EINVAL;
    return zdp::launch_step_clipped(make_src(src, hp->scale_interval > 0 ? st->ctl : nullptr), a, grad_buf,
                                    hp->max_grad_norm, make_ws(workspace), stream);
}

int zero_adam_step_bucket(const zero_grad_src* src, const zero_adam_state* st, const zero_adam_hp* hp,
                          int64_t win_off, int64_t window_n, uint16_t* allgather, int64_t allgather_off,
                          int32_t phase, void* workspace, void* stream) {
    if (src == nullptr || st == nullptr || hp == nullptr) return ZERO_EINVAL;
    if ((phase & ~(ZERO_BUCKET_FIRST | ZERO_BUCKET_LAST)) != 0 || win_off < 0 || window_n < 0 || src->n < 0)
        return ZERO_EINVAL;
    int64_t end = 0, b = 0;
    if (zdp::add_overflows(win_off, src->n, &end) || zdp::mul_overflows(window_n, 4, &b)) return ZERO_EOVERFLOW;
    if (end > window_n) return ZERO_EINVAL;
    if (win_off % 8 != 0) return ZERO_EALIGN;
    // the bucket's view of the state and of the all-gather window
    zero_adam_state sub = *st;
    for (int i = 0; i < 2; ++i) {
        if (st->master[i] == nullptr || st->exp_avg[i] == nullptr || st->exp_avg_sq[i] == nullptr) {
            if (window_n != 0) return ZERO_EINVAL;
            continue;
        }
        sub.master[i] = st->master[i] + win_off;
        sub.exp_avg[i] = st->exp_avg[i] + win_off;
        sub.exp_avg_sq[i] = st->exp_avg_sq[i] + win_off;
    }
    int64_t ag_off = 0;
    if (allgather != nullptr && (allgather_off < 0 || zdp::add_overflows(allgather_off, win_off, &ag_off)))
        return allgather_off < 0 ? ZERO_EINVAL : ZERO_EOVERFLOW;
    AdamArgs a;
    const int rc = check_step(src, &sub, hp, allgather, ag_off, workspace, nullptr, &a);
    if (rc != ZERO_OK) return rc;
    if (hp->max_grad_norm != 0.0) return ZERO_EINVAL;  // clipping needs the norm before any bucket
    // the whole window's all-gather range, for the re-emit of a skipped step
    uint16_t* ag_window = nullptr;
    if (allgather != nullptr) {
        int64_t e = 0;
        if (zdp::add_overflows(allgather_off, window_n, &e) || zdp::mul_overflows(e, 2, &e)) return ZERO_EOVERFLOW;
        ag_window = allgather + allgather_off;
        if (!aligned16(ag_window)) return ZERO_EALIGN;
    }
    a.bucket = phase | 4;  // the commit checks the buckets' coverage
    a.window_n = window_n;
    // the commit's view: the whole window
    AdamArgs whole = a;
    for (int i = 0; i < 2; ++i) {
        whole.p[i] = st->master[i];
        whole.m[i] = st->exp_avg[i];
        whole.v[i] = st->exp_avg_sq[i];
    }
    whole.ag = ag_window;
    return zdp::launch_bucket(make_src(src, hp->scale_interval > 0 ? st->ctl : nullptr), a, whole, phase,
                              make_ws(workspace), stream);
}

int zero_adam_step_buckets(const zero_bucket* buckets, int32_t nb, const zero_adam_state* st,
                           const zero_adam_hp* hp, int64_t window_n, uint16_t* allgather, int64_t allgather_off,
                           int32_t phase, void* workspace, void* stream) {
    if (buckets == nullptr || nb < 1 || nb > ZERO_MAX_BUCKETS_PER_CALL) return ZERO_EINVAL;
    if ((phase & ~(ZERO_BUCKET_FIRST | ZERO_BUCKET_LAST)) != 0 || window_n < 0) return ZERO_EINVAL;
    AdamArgs a;
    Range r[11];
    int nr = 0;
    const int rc = check_window(st, hp, window_n, allgather, allgather_off, workspace, nullptr, &a, r, &nr);
    if (rc != ZERO_OK) return rc;
    if (hp->max_grad_norm != 0.0) return ZERO_EINVAL;  // clipping needs the norm before any bucket
    zdp::BucketRun runs[ZERO_MAX_BUCKETS_PER_CALL];
    for (int32_t i = 0; i < nb; ++i) {
        const zero_bucket& b = buckets[i];
        Range span{};
        const int rc2 = check_src(&b.src, &span);
        if (rc2 != ZERO_OK) return rc2;
        if (b.src.nd != buckets[0].src.nd || b.src.loss_scale != buckets[0].src.loss_scale || b.win_off < 0)
            return ZERO_EINVAL;
        int64_t end = 0;
        if (zdp::add_overflows(b.win_off, b.src.n, &end)) return ZERO_EOVERFLOW;
        if (end > window_n) return ZERO_EINVAL;
        if (b.win_off % 8 != 0) return ZERO_EALIGN;
        // a bucket's slices may overlap nothing the step writes or owns
        for (int k = 0; k < nr; ++k)
            if (overlap(r[k], span)) return ZERO_EALIAS;
        // nor may two buckets of one call cover the same window element
        for (int32_t j = 0; j < i; ++j)
            if (b.win_off < runs[j].win_off + runs[j].n && runs[j].win_off < end && b.src.n > 0 && runs[j].n > 0)
                return ZERO_EINVAL;
        runs[i] = zdp::BucketRun{b.src.base + b.src.elem_off, b.src.nd > 1 ? b.src.slice_stride : 0, b.src.n,
                                 b.win_off};
    }
    return zdp::launch_buckets(runs, nb, make_src(&buckets[0].src, hp->scale_interval > 0 ? st->ctl : nullptr), a,
                               phase, make_ws(workspace), stream);
}

int zero_gather_params(const uint16_t* const* windows, int32_t nd, int64_t part, int64_t lo, int64_t hi,
                       uint16_t* dst, void* stream) {
    const int64_t range[2] = {lo, hi};
    const int rc = check_gather(windows, nd, part, range, 1, &dst);
    if (rc != ZERO_OK) return rc;
    if (hi == lo) return ZERO_OK;  // nothing to gather
    return zdp::launch_gather(windows, part, range, 1, &dst, stream);
}

int zero_gather_layers(const uint16_t* const* windows, int32_t nd, int64_t part, const int64_t* ranges,
                       int32_t nranges, uint16_t* const* dsts, void* stream) {
    const int rc = check_gather(windows, nd, part, ranges, nranges, dsts);
    if (rc != ZERO_OK) return rc;
    int64_t total = 0;
    for (int32_t q = 0; q < nranges; ++q) total += ranges[2 * q + 1] - ranges[2 * q];
    if (total == 0) return ZERO_OK;  // nothing to gather
    return zdp::launch_gather(windows, part, ranges, nranges, dsts, stream);
}

int zero_restore_skipped(const zero_adam_state* st, int64_t n, uint16_t* allgather,
                         int64_t allgather_off, void* stream) {
    if (st == nullptr || st->ctl == nullptr || n < 0 || allgather_off < 0) return ZERO_EINVAL;
    if (n != 0 && (allgather == nullptr || st->master[0] == nullptr || st->master[1] == nullptr))
        return ZERO_EINVAL;
    int64_t e = 0;
    if (zdp::mul_overflows(n, 4, &e) || zdp::add_overflows(allgather_off, n, &e) ||
        zdp::mul_overflows(e, 2, &e))
        return ZERO_EOVERFLOW;
    if (n == 0) return ZERO_OK;  // nothing to restore
    uint16_t* ag = allgather + allgather_off;
    if (!aligned16(ag) || !aligned16(st->master[0]) || !aligned16(st->master[1]) ||
        (reinterpret_cast<uintptr_t>(st->ctl) & 7u) != 0)
        return ZERO_EALIGN;
    const Range w = bytes_of(ag, n, 2);
    if (overlap(w, bytes_of(st->master[0], n, 4)) || overlap(w, bytes_of(st->master[1], n, 4)) ||
        overlap(w, bytes_of(st->ctl, 1, static_cast<int64_t>(sizeof(zero_step_ctl)))))
        return ZERO_EALIAS;
    return zdp::launch_restore(st->master[0], st->master[1], st->ctl, ag, n, stream);
}

int zero_emit_fp16(const float* master, int64_t n, uint16_t* allgather, int64_t allgather_off,
                   void* stream) {
    if (n < 0 || allgather_off < 0) return ZERO_EINVAL;
    if (n == 0) return ZERO_OK;  // nothing to write
    if (master == nullptr || allgather == nullptr) return ZERO_EINVAL;
    int64_t e = 0;
    if (zdp::mul_overflows(n, 4, &e) || zdp::add_overflows(allgather_off, n, &e) ||
        zdp::mul_overflows(e, 2, &e))
        return ZERO_EOVERFLOW;
    uint16_t* ag = allgather + allgather_off;
    if (!aligned16(ag) || !aligned16(master)) return ZERO_EALIGN;
    if (overlap(bytes_of(master, n, 4), bytes_of(ag, n, 2))) return ZERO_EALIAS;
    return zdp::launch_emit(master, ag, n, stream);
}

int zero_calib_triad(float* a, const float* b, const float* c, float q, int64_t n, void* stream) {
    if (n < 0) return ZERO_EINVAL;
    if (n == 0) return ZERO_OK;
    if (a == nullptr || b == nullptr || c == nullptr) return ZERO_EINVAL;
    int64_t bytes = 0;
    if (zdp::mul_overflows(n, 4, &bytes)) return ZERO_EOVERFLOW;
    if (!aligned16(a) || !aligned16(b) || !aligned16(c)) return ZERO_EALIGN;
    if (overlap(bytes_of(a, n, 4), bytes_of(b, n, 4)) || overlap(bytes_of(a, n, 4), bytes_of(c, n, 4)))
        return ZERO_EALIAS;
    return zdp::launch_calib_triad(a, b, c, q, n, stream);
}

int zero_calib_stream_mix(const zero_grad_src* src, const float* const* in, float* const* out, uint16_t* out16,
                          void* stream) {
    Range span{};
    const int rc = check_src(src, &span);
    if (rc != ZERO_OK) return rc;
    if (in == nullptr || out == nullptr) return ZERO_EINVAL;
    const int64_t n = src->n;
    int64_t bytes = 0;
    if (zdp::mul_overflows(n, 4, &bytes)) return ZERO_EOVERFLOW;
    if (n == 0) return ZERO_OK;
    Range r[8];
    int nr = 0;
    for (int i = 0; i < 3; ++i) {
        if (in[i] == nullptr || out[i] == nullptr) return ZERO_EINVAL;
        if (!aligned16(in[i]) || !aligned16(out[i])) return ZERO_EALIGN;
    }
    if (out16 == nullptr) return ZERO_EINVAL;
    if (!aligned16(out16)) return ZERO_EALIGN;
    // the outputs must not overlap each other or any input
    for (int i = 0; i < 3; ++i) r[nr++] = bytes_of(out[i], n, 4);
    r[nr++] = bytes_of(out16, n, 2);
    if (any_overlap(r, nr)) return ZERO_EALIAS;
    const Range ins[4] = {span, bytes_of(in[0], n, 4), bytes_of(in[1], n, 4), bytes_of(in[2], n, 4)};
    for (int i = 0; i < nr; ++i)
        for (const Range& x : ins)
            if (overlap(r[i], x)) return ZERO_EALIAS;
    return zdp::launch_calib_mix(make_src(src), in, out, out16, stream);
}

int zero_calib_slice_read(const zero_grad_src* src, uint32_t* sink, void* stream) {
    Range span{};
    const int rc = check_src(src, &span);
    if (rc != ZERO_OK) return rc;
    if (sink == nullptr) return ZERO_EINVAL;
    if (reinterpret_cast<uintptr_t>(sink) % 4 != 0) return ZERO_EALIGN;
    if (src->n == 0) return ZERO_OK;
    if (overlap(bytes_of(sink, 1, 4), span)) return ZERO_EALIAS;
    return zdp::launch_calib_slice_read(make_src(src), sink, stream);
}

}  // extern "C"

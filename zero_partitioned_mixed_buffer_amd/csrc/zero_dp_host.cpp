// Host side of the ZeRO-DP owned-partition library: partition planner,
// memory/communication model, status strings.  No device code here.
//
// Planner: the flat buffer of packed tensors is split into Nd equal windows,
// one per data-parallel rank (trishampatil "ZeRO's Core Idea": GPU i holds
// shard i; upskillscore "How it works": states split into Nd parts).  The
// window size is padded to a multiple of `align` so that every window starts
// on a 16-byte boundary for fp16 and fp32 data.
//
// Memory model: trishampatil "The Real Problem" (2Psi + 2Psi + K Psi with
// K = 12) and "The Full Progression, in One View" (per-stage bytes and the
// 2Psi / 3Psi communication volumes); upskillscore "How it works".
#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/zero_dp.h"
#include "zero_dp_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

}  // namespace

namespace zdp {

void set_last_hip_error(int e) { g_last_hip_error = e; }

bool mul_overflows(int64_t a, int64_t b, int64_t* out) {
    return __builtin_mul_overflow(a, b, out);
}

bool add_overflows(int64_t a, int64_t b, int64_t* out) {
    return __builtin_add_overflow(a, b, out);
}

}  // namespace zdp

extern "C" {

const char* zero_strerror(int status) {
    switch (status) {
        case ZERO_OK: return "ok";
        case ZERO_EINVAL: return "invalid argument";
        case ZERO_EALIGN: return "misaligned operand (16-byte vectors, offsets in multiples of 8 elements)";
        case ZERO_EOVERFLOW: return "size or offset overflows int64";
        case ZERO_ECAPACITY: return "fragment array too small";
        case ZERO_EALIAS: return "output overlaps an input";
        case ZERO_EHIP: return "HIP runtime or launch failure";
        default: return "unknown status";
    }
}

int zero_last_hip_error(void) { return g_last_hip_error; }

int zero_abi_version(void) { return ZERO_DP_ABI_VERSION; }

int zero_plan_partitions(const int64_t* numels, int32_t n_tensors, int32_t nd, int32_t align_elems,
                         zero_plan* plan, zero_frag* frags, int64_t frag_cap, int64_t* n_frags) {
    if (plan == nullptr || n_frags == nullptr || n_tensors < 0 || nd < 1 || frag_cap < 0)
        return ZERO_EINVAL;
    if (align_elems < 8 || align_elems % 8 != 0) return ZERO_EINVAL;
    if (n_tensors > 0 && numels == nullptr) return ZERO_EINVAL;
    if (frag_cap > 0 && frags == nullptr) return ZERO_EINVAL;

    int64_t psi = 0;
    for (int32_t i = 0; i < n_tensors; ++i) {
        if (numels[i] < 0) return ZERO_EINVAL;
        if (zdp::add_overflows(psi, numels[i], &psi)) return ZERO_EOVERFLOW;
    }
    int64_t unit = 0;  // elements in one "row" of Nd aligned blocks
    if (zdp::mul_overflows(static_cast<int64_t>(nd), static_cast<int64_t>(align_elems), &unit))
        return ZERO_EOVERFLOW;
    // ceil(psi / unit) without overflow: psi >= 0, unit >= 8
    const int64_t units = psi / unit + (psi % unit != 0 ? 1 : 0);
    int64_t part = 0, padded = 0;
    if (zdp::mul_overflows(units, static_cast<int64_t>(align_elems), &part)) return ZERO_EOVERFLOW;
    if (zdp::mul_overflows(part, static_cast<int64_t>(nd), &padded)) return ZERO_EOVERFLOW;

    plan->psi = psi;
    plan->nd = nd;
    plan->align = align_elems;
    plan->part = part;
    plan->padded = padded;
    plan->pad = padded - psi;

    // Fragments: cut each tensor's flat range at multiples of S.
    int64_t count = 0;
    int64_t flat = 0;
    for (int32_t i = 0; i < n_tensors; ++i) {
        const int64_t numel = numels[i];
        int64_t done = 0;
        while (done < numel) {
            const int64_t pos = flat + done;
            const int64_t rank = pos / part;
            const int64_t local = pos - rank * part;
            const int64_t room = part - local;
            const int64_t len = (numel - done) < room ? (numel - done) : room;
            if (count < frag_cap) {
                zero_frag& f = frags[count];
                f.tensor = i;
                f.rank = static_cast<int32_t>(rank);
                f.tensor_off = done;
                f.flat_off = pos;
                f.local_off = local;
                f.len = len;
            }
            ++count;
            done += len;
        }
        flat += numel;
    }
    *n_frags = count;
    return count > frag_cap ? ZERO_ECAPACITY : ZERO_OK;
}

int zero_memory_model(double psi, int32_t nd, int32_t stage, int32_t k, zero_mem_report* out) {
    if (out == nullptr || !(psi >= 0.0) || !std::isfinite(psi) || nd < 1 || stage < 0 || stage > 3 ||
        k < 0)
        return ZERO_EINVAL;
    const double n = static_cast<double>(nd);
    const double kk = static_cast<double>(k);
    // fp16 parameters: replicated until stage 3 (Pos+g+p) shards them.
    out->params_bytes = stage >= 3 ? 2.0 * psi / n : 2.0 * psi;
    // fp16 gradients: sharded from stage 2 (Pos+g) on.
    out->grads_bytes = stage >= 2 ? 2.0 * psi / n : 2.0 * psi;
    // K bytes of optimizer state: sharded from stage 1 (Pos) on.
    out->optim_bytes = stage >= 1 ? kk * psi / n : kk * psi;
    out->total_bytes = out->params_bytes + out->grads_bytes + out->optim_bytes;
    out->comm_elems = stage >= 3 ? 3.0 * psi : 2.0 * psi;
    out->comm_elems_ring = out->comm_elems * (n - 1.0) / n;
    const double dp = (4.0 + kk) * psi;
    out->reduction_vs_dp = out->total_bytes > 0.0 ? dp / out->total_bytes : INFINITY;
    return ZERO_OK;
}

void zero_ctl_init(zero_step_ctl* ctl, double loss_scale) {
    if (ctl == nullptr) return;
    std::memset(ctl, 0, sizeof(*ctl));
    ctl->beta1_pow = 1.0;
    ctl->beta2_pow = 1.0;
    ctl->loss_scale = loss_scale;
    ctl->clip_coef = 1.0;
}

}  // extern "C"

// Host side of the library: the flat-bucket partitioner, the model-state and
// communication accounting, the workspace size and the error channel.
//
// Partition (L18 notes §2.1, §3.2 and exercise 6; Illustrated ZeRO §8.4):
// Adam is elementwise, so the flat parameter vector is cut into equal
// contiguous pieces, one per data-parallel rank, and a tensor may straddle two
// ranks.  Stage 3 partitions each unit (layer) on its own so that one layer can
// be gathered into a contiguous buffer.  All arithmetic here is int64.
//
// Pages cited by short name:
//   L18 notes         CMU 11-868 Lecture 18 notes, "Memory Optimization in Distributed Training: ZeRO" (semidirectx.com)
//   Illustrated ZeRO  "图解分布式训练（八）—— ZeRO 学习" (llm.jiangnianmeng.cn)

#include <algorithm>
#include <new>
#include <string>

#include "internal.h"

namespace zf {

namespace {
thread_local std::string g_error;
}  // namespace

int fail(int code, const std::string& msg) {
    g_error = msg;
    return code;
}

int ok() {
    g_error.clear();
    return ZERO_OK;
}

int64_t partial_blocks(int64_t n) {
    const int64_t b = (n + kPartialElems - 1) / kPartialElems;
    return b < 1 ? 1 : b;
}

}  // namespace zf

namespace zf {

// Maximal runs (old owner, old shard offset, new shard offset, length) that
// fill `rank`'s shard under `neu` from the shards of `old`, in new-shard
// order.  Both plans must partition the same number of parameters; the flat
// parameter order (units concatenated) identifies a parameter.
void reshard_runs(const zero_plan& old, const zero_plan& neu, int rank, std::vector<zero_reshard_segment>& runs) {
    runs.clear();
    const int r_new = neu.owners == 1 ? 0 : rank;
    size_t k = 0;            // old unit holding flat position g
    int64_t old_flat = 0;    // flat base of old unit k
    int64_t new_flat = 0;    // flat base of the new unit
    for (const auto& u : neu.units) {
        const int64_t lo = std::min(int64_t(r_new) * u.slice_numel, u.numel);
        const int64_t hi = std::min(int64_t(r_new + 1) * u.slice_numel, u.numel);
        int64_t g = new_flat + lo;
        const int64_t g_end = new_flat + hi;
        int64_t j = u.shard_base + lo - int64_t(r_new) * u.slice_numel;
        while (g < g_end) {
            while (g >= old_flat + old.units[k].numel) old_flat += old.units[k++].numel;
            const auto& ou = old.units[k];
            const int64_t local = g - old_flat;
            const int64_t r_old = old.owners == 1 ? 0 : local / ou.slice_numel;
            const int64_t piece_end =
                std::min({g_end, old_flat + ou.numel, old_flat + (r_old + 1) * ou.slice_numel});
            const int64_t len = piece_end - g;
            const int64_t k_off = ou.shard_base + local - r_old * ou.slice_numel;
            zero_reshard_segment* last = runs.empty() ? nullptr : &runs.back();
            if (last && last->old_rank == r_old && last->old_offset + last->len == k_off &&
                last->new_offset + last->len == j)
                last->len += len;
            else
                runs.push_back({r_old, k_off, j, len});
            g += len;
            j += len;
        }
        new_flat += u.numel;
    }
}

int64_t plan_psi(const zero_plan& p) {
    int64_t psi = 0;
    for (const auto& u : p.units) psi += u.numel;
    return psi;
}

}  // namespace zf

extern "C" {

const char* zero_last_error(void) { return zf::g_error.c_str(); }

int zero_version(void) { return 10301; }

int zero_plan_create(const int64_t* unit_numels, int n_units, int nd, int stage,
                     int64_t align_elems, zero_plan** out) {
    if (out == nullptr) return zf::fail(ZERO_EINVAL, "zero_plan_create: out is NULL");
    *out = nullptr;
    if (unit_numels == nullptr || n_units < 1)
        return zf::fail(ZERO_EINVAL, "zero_plan_create: need at least one unit");
    if (nd < 1 || nd > ZERO_MAX_RANKS)
        return zf::fail(ZERO_EINVAL, "zero_plan_create: nd must be in [1, 1024]");
    if (stage < 0 || stage > 3)
        return zf::fail(ZERO_EINVAL, "zero_plan_create: stage must be 0, 1, 2 or 3");
    if (align_elems < 1 || align_elems > (int64_t(1) << 30))
        return zf::fail(ZERO_EINVAL, "zero_plan_create: align must be in [1, 2^30]");
    int64_t total = 0;
    for (int i = 0; i < n_units; ++i) {
        if (unit_numels[i] < 0) return zf::fail(ZERO_EINVAL, "zero_plan_create: negative unit size");
        if (unit_numels[i] > (int64_t(1) << 50) - total)
            return zf::fail(ZERO_EINVAL, "zero_plan_create: more than 2^50 elements");
        total += unit_numels[i];
    }
    if (total == 0) return zf::fail(ZERO_EINVAL, "zero_plan_create: no elements");

    zero_plan* p = new (std::nothrow) zero_plan;
    if (p == nullptr) return zf::fail(ZERO_ENOMEM, "zero_plan_create: out of host memory");
    p->nd = nd;
    p->stage = stage;
    p->owners = stage == 0 ? 1 : nd;
    p->align = align_elems;
    std::vector<int64_t> sizes;
    if (stage == 3)
        sizes.assign(unit_numels, unit_numels + n_units);
    else
        sizes.push_back(total);
    int64_t full_base = 0, shard_base = 0;
    try {
        for (int64_t u : sizes) {
            int64_t per = (u + p->owners - 1) / p->owners;
            int64_t s = (per + align_elems - 1) / align_elems * align_elems;
            // padding can outgrow the 2^50 real elements (up to align per unit
            // and owner): keep the padded layout within 2^52 elements
            if (s > (int64_t(1) << 52) / p->owners || full_base > (int64_t(1) << 52) - int64_t(p->owners) * s) {
                delete p;
                return zf::fail(ZERO_EINVAL, "zero_plan_create: the padded layout exceeds 2^52 elements");
            }
            p->units.push_back({u, s, full_base, shard_base});
            full_base += int64_t(p->owners) * s;
            shard_base += s;
        }
    } catch (const std::bad_alloc&) {
        delete p;
        return zf::fail(ZERO_ENOMEM, "zero_plan_create: out of host memory");
    }
    p->shard_numel = shard_base;
    p->full_numel = full_base;
    *out = p;
    return zf::ok();
}

void zero_plan_destroy(zero_plan* plan) { delete plan; }

int zero_plan_info(const zero_plan* plan, int* n_units, int* owners, int* nd, int* stage) {
    if (plan == nullptr) return zf::fail(ZERO_EINVAL, "zero_plan_info: plan is NULL");
    if (n_units) *n_units = int(plan->units.size());
    if (owners) *owners = plan->owners;
    if (nd) *nd = plan->nd;
    if (stage) *stage = plan->stage;
    return zf::ok();
}

int zero_plan_rank(const zero_plan* plan, int rank, int64_t* shard_numel, int64_t* real_numel) {
    if (plan == nullptr) return zf::fail(ZERO_EINVAL, "zero_plan_rank: plan is NULL");
    if (rank < 0 || rank >= plan->nd) return zf::fail(ZERO_EINVAL, "zero_plan_rank: rank out of range");
    int r = plan->owners == 1 ? 0 : rank;
    int64_t real = 0;
    for (const auto& u : plan->units) {
        int64_t lo = std::min(int64_t(r) * u.slice_numel, u.numel);
        int64_t hi = std::min(int64_t(r + 1) * u.slice_numel, u.numel);
        real += hi - lo;
    }
    if (shard_numel) *shard_numel = plan->shard_numel;
    if (real_numel) *real_numel = real;
    return zf::ok();
}

int zero_plan_unit(const zero_plan* plan, int unit, int64_t* numel, int64_t* slice_numel,
                   int64_t* full_base, int64_t* shard_base) {
    if (plan == nullptr) return zf::fail(ZERO_EINVAL, "zero_plan_unit: plan is NULL");
    if (unit < 0 || unit >= int(plan->units.size()))
        return zf::fail(ZERO_EINVAL, "zero_plan_unit: unit out of range");
    const auto& u = plan->units[unit];
    if (numel) *numel = u.numel;
    if (slice_numel) *slice_numel = u.slice_numel;
    if (full_base) *full_base = u.full_base;
    if (shard_base) *shard_base = u.shard_base;
    return zf::ok();
}

int zero_plan_full_numel(const zero_plan* plan, int64_t* padded) {
    if (plan == nullptr || padded == nullptr)
        return zf::fail(ZERO_EINVAL, "zero_plan_full_numel: NULL argument");
    *padded = plan->full_numel;
    return zf::ok();
}

int zero_plan_segments(const zero_plan* plan, const int64_t* tensor_numels, int n_tensors, int rank,
                       zero_segment* out, int cap, int* count) {
    if (plan == nullptr || count == nullptr || (n_tensors > 0 && tensor_numels == nullptr))
        return zf::fail(ZERO_EINVAL, "zero_plan_segments: NULL argument");
    if (n_tensors < 0 || cap < 0 || (cap > 0 && out == nullptr))
        return zf::fail(ZERO_EINVAL, "zero_plan_segments: bad count or capacity");
    if (rank < 0 || rank >= plan->nd) return zf::fail(ZERO_EINVAL, "zero_plan_segments: rank out of range");
    // Validate that the tensors fill the units exactly, before writing anything.
    {
        size_t ui = 0;
        int64_t pos = 0, sum = 0;
        for (int t = 0; t < n_tensors; ++t) {
            int64_t len = tensor_numels[t];
            if (len < 0) return zf::fail(ZERO_EINVAL, "zero_plan_segments: negative tensor size");
            if (len == 0) continue;
            while (ui < plan->units.size() && pos == plan->units[ui].numel) { ++ui; pos = 0; }
            if (ui >= plan->units.size() || len > plan->units[ui].numel - pos)
                return zf::fail(ZERO_EINVAL, "zero_plan_segments: tensors do not fill the units");
            pos += len;
            sum += len;
        }
        int64_t psi = 0;
        for (const auto& u : plan->units) psi += u.numel;
        if (sum != psi) return zf::fail(ZERO_EINVAL, "zero_plan_segments: tensor sizes do not add up");
    }
    int r = plan->owners == 1 ? 0 : rank;
    int written = 0;
    size_t ui = 0;
    int64_t pos = 0;
    for (int t = 0; t < n_tensors; ++t) {
        int64_t len = tensor_numels[t];
        if (len == 0) continue;
        while (pos == plan->units[ui].numel) { ++ui; pos = 0; }
        const auto& u = plan->units[ui];
        int64_t lo = std::min(int64_t(r) * u.slice_numel, u.numel);
        int64_t hi = std::min(int64_t(r + 1) * u.slice_numel, u.numel);
        int64_t a = std::max(lo, pos), b = std::min(hi, pos + len);
        if (a < b) {
            if (written < cap)
                out[written] = {t, a - pos, u.shard_base + (a - int64_t(r) * u.slice_numel), b - a};
            ++written;
        }
        pos += len;
    }
    *count = written;
    return zf::ok();
}


int zero_plan_reshard(const zero_plan* old_plan, const zero_plan* new_plan, int new_rank, zero_reshard_segment* out,
                      int cap, int* count) {
    if (old_plan == nullptr || new_plan == nullptr || count == nullptr)
        return zf::fail(ZERO_EINVAL, "zero_plan_reshard: NULL argument");
    if (cap < 0 || (cap > 0 && out == nullptr)) return zf::fail(ZERO_EINVAL, "zero_plan_reshard: bad capacity");
    if (new_rank < 0 || new_rank >= new_plan->nd)
        return zf::fail(ZERO_EINVAL, "zero_plan_reshard: rank out of range");
    if (zf::plan_psi(*old_plan) != zf::plan_psi(*new_plan))
        return zf::fail(ZERO_EINVAL, "zero_plan_reshard: the plans partition different parameter counts");
    std::vector<zero_reshard_segment> runs;
    try {
        zf::reshard_runs(*old_plan, *new_plan, new_rank, runs);
    } catch (const std::bad_alloc&) {
        return zf::fail(ZERO_ENOMEM, "zero_plan_reshard: out of host memory");
    }
    if (runs.size() > size_t(INT32_MAX)) return zf::fail(ZERO_EINVAL, "zero_plan_reshard: too many runs");
    for (size_t i = 0; i < runs.size() && i < size_t(cap); ++i) out[i] = runs[i];
    *count = int(runs.size());
    return zf::ok();
}

int zero_model_state_bytes(double psi, int nd, int stage, int k_bytes, double* out) {
    if (out == nullptr || nd < 1 || !(psi >= 0) || k_bytes < 0)
        return zf::fail(ZERO_EINVAL, "zero_model_state_bytes: bad argument");
    double k = k_bytes;
    switch (stage) {
        case 0: *out = psi * (4.0 + k); break;
        case 1: *out = psi * (4.0 + k / nd); break;
        case 2: *out = psi * (2.0 + (2.0 + k) / nd); break;
        case 3: *out = psi * ((4.0 + k) / nd); break;
        default: return zf::fail(ZERO_EINVAL, "zero_model_state_bytes: stage must be 0..3");
    }
    return zf::ok();
}

int zero_comm_volume(double psi, int nd, int stage, double* elems_sent) {
    if (elems_sent == nullptr || nd < 1 || !(psi >= 0) || stage < 0 || stage > 3)
        return zf::fail(ZERO_EINVAL, "zero_comm_volume: bad argument");
    double passes = stage == 3 ? 3.0 : 2.0;
    *elems_sent = passes * psi * double(nd - 1) / double(nd);
    return zf::ok();
}

int64_t zero_workspace_bytes(int64_t n, int n_sets) {
    if (n < 0 || n > ZERO_MAX_ELEMS || n_sets < 0 || n_sets > ZERO_MAX_RANKS) {
        zf::fail(ZERO_EINVAL, "zero_workspace_bytes: bad argument");
        return -1;
    }
    zf::ok();
    return zf::kPartialsOffset + int64_t(n_sets) * zf::partial_blocks(n) * int64_t(sizeof(double));
}

}  // extern "C"

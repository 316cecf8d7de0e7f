// The library's host code (partitioner, host AdamW with its worker threads,
// sharded checkpoints) exercised through the C ABI, for builds under the
// compiler's address, undefined-behaviour and thread sanitizers.  No device is
// used: only host-memory paths run.  Self-checking; prints "ok" and exits 0
// when every check holds.
//
// Usage: host_sanitize_driver TMPDIR
// Test fixture: compiled and run by tests/test_host_sanitizers.py.

#include <sys/stat.h>
#include <unistd.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "zero_flat.h"

namespace {

int g_failures = 0;
long g_checks = 0;

#define CHECK(cond, ...)                                                    \
    do {                                                                    \
        ++g_checks;                                                         \
        if (!(cond)) {                                                      \
            std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);       \
            std::fprintf(stderr, __VA_ARGS__);                              \
            std::fprintf(stderr, " [%s]\n", zero_last_error());             \
            ++g_failures;                                                   \
        }                                                                   \
    } while (0)

// splitmix64: a small deterministic generator for the layouts and values.
struct Rng {
    uint64_t s;
    uint64_t next() {
        uint64_t z = (s += 0x9E3779B97F4A7C15ull);
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }
    int64_t range(int64_t lo, int64_t hi) { return lo + int64_t(next() % uint64_t(hi - lo + 1)); }
    double unit() { return double(next() >> 11) * (1.0 / 9007199254740992.0); }
};

struct Plan {
    zero_plan* p = nullptr;
    ~Plan() { zero_plan_destroy(p); }
};

// ---------------------------------------------------------------------------
// a0: partitions, tensor segments and reshard runs on random layouts
// ---------------------------------------------------------------------------

void check_plans() {
    Rng rng{1};
    for (int trial = 0; trial < 300; ++trial) {
        const int n_units = int(rng.range(1, 24));
        std::vector<int64_t> units(static_cast<size_t>(n_units));
        int64_t psi = 0;
        for (auto& u : units) psi += (u = rng.range(0, 3000));
        const int nd = int(rng.range(1, 70)), stage = int(rng.range(0, 3));
        const int64_t aligns[4] = {1, 2, 8, 64};
        const int64_t align = aligns[rng.range(0, 3)];
        Plan plan;
        const int rc = zero_plan_create(units.data(), n_units, nd, stage, align, &plan.p);
        if (psi == 0) {
            CHECK(rc == ZERO_EINVAL && plan.p == nullptr, "an empty layout must be refused");
            continue;
        }
        CHECK(rc == ZERO_OK, "zero_plan_create trial %d", trial);
        if (rc != ZERO_OK) continue;
        int nu = 0, owners = 0, nd2 = 0, st = 0;
        CHECK(zero_plan_info(plan.p, &nu, &owners, &nd2, &st) == ZERO_OK, "info");
        CHECK(owners == (stage == 0 ? 1 : nd) && nd2 == nd && st == stage, "info values");
        int64_t full = 0;
        CHECK(zero_plan_full_numel(plan.p, &full) == ZERO_OK, "full_numel");

        // Every real element is owned once: the owners' real counts add up to psi.
        int64_t real_sum = 0, shard = -1;
        for (int r = 0; r < nd; ++r) {
            int64_t s = 0, real = 0;
            CHECK(zero_plan_rank(plan.p, r, &s, &real) == ZERO_OK, "rank %d", r);
            CHECK(real >= 0 && real <= s, "rank %d: real %lld of %lld", r, (long long)real, (long long)s);
            CHECK(shard < 0 || s == shard, "every rank holds the same shard length");
            shard = s;
            if (r < owners) real_sum += real;
        }
        CHECK(real_sum == psi, "owners' real elements %lld != psi %lld", (long long)real_sum, (long long)psi);
        CHECK(full == int64_t(owners) * shard, "full = owners x shard");

        // Segments of a random split of the units into tensors: in bounds, no
        // overlap inside a shard, all of psi over the owners.
        std::vector<int64_t> tensors;
        for (int64_t u : units) {
            int64_t left = u;
            while (left > 0) {
                const int64_t t = rng.range(1, left);
                tensors.push_back(t);
                left -= t;
            }
            if (rng.range(0, 3) == 0) tensors.push_back(0);
        }
        int64_t covered = 0;
        for (int r = 0; r < owners; ++r) {
            int count = -1;
            CHECK(zero_plan_segments(plan.p, tensors.data(), int(tensors.size()), r, nullptr, 0, &count) == ZERO_OK,
                  "segments count");
            std::vector<zero_segment> segs(size_t(count > 0 ? count : 1));
            int count2 = -1;
            CHECK(zero_plan_segments(plan.p, tensors.data(), int(tensors.size()), r, segs.data(), count, &count2) ==
                      ZERO_OK && count2 == count,
                  "segments fill");
            std::vector<char> used(size_t(shard), 0);
            for (int i = 0; i < count; ++i) {
                const zero_segment& g = segs[size_t(i)];
                const bool in = g.tensor >= 0 && g.tensor < int64_t(tensors.size()) && g.len > 0 &&
                                g.tensor_off >= 0 && g.tensor_off + g.len <= tensors[size_t(g.tensor)] &&
                                g.shard_off >= 0 && g.shard_off + g.len <= shard;
                CHECK(in, "segment %d of rank %d out of bounds", i, r);
                if (!in) continue;
                for (int64_t k = g.shard_off; k < g.shard_off + g.len; ++k) {
                    CHECK(!used[size_t(k)], "shard position %lld used twice", (long long)k);
                    used[size_t(k)] = 1;
                }
                covered += g.len;
            }
        }
        CHECK(covered == psi, "segments cover %lld of %lld", (long long)covered, (long long)psi);

        // Reshard runs into another random partition of the same units.
        Plan other;
        const int nd_b = int(rng.range(1, 70)), stage_b = int(rng.range(0, 3));
        CHECK(zero_plan_create(units.data(), n_units, nd_b, stage_b, aligns[rng.range(0, 3)], &other.p) == ZERO_OK,
              "second plan");
        int owners_b = 0, x = 0;
        zero_plan_info(other.p, &x, &owners_b, &x, &x);
        int64_t moved = 0;
        for (int r = 0; r < owners_b; ++r) {
            int64_t s_b = 0, real_b = 0;
            zero_plan_rank(other.p, r, &s_b, &real_b);
            int count = -1;
            CHECK(zero_plan_reshard(plan.p, other.p, r, nullptr, 0, &count) == ZERO_OK, "reshard count");
            std::vector<zero_reshard_segment> runs(size_t(count > 0 ? count : 1));
            int count2 = -1;
            CHECK(zero_plan_reshard(plan.p, other.p, r, runs.data(), count, &count2) == ZERO_OK && count2 == count,
                  "reshard fill");
            int64_t run_sum = 0;
            for (int i = 0; i < count; ++i) {
                const zero_reshard_segment& g = runs[size_t(i)];
                CHECK(g.old_rank >= 0 && g.old_rank < owners && g.len > 0 && g.old_offset >= 0 &&
                          g.old_offset + g.len <= shard && g.new_offset >= 0 && g.new_offset + g.len <= s_b,
                      "run %d of rank %d out of bounds", i, r);
                run_sum += g.len;
            }
            CHECK(run_sum == real_b, "runs of rank %d move %lld of %lld", r, (long long)run_sum, (long long)real_b);
            moved += run_sum;
        }
        CHECK(moved == psi, "reshard moves %lld of %lld", (long long)moved, (long long)psi);
    }

    // Refusals, with nothing written and no crash.
    zero_plan* p = reinterpret_cast<zero_plan*>(1);
    const int64_t one = 10, neg = -1;
    CHECK(zero_plan_create(&one, 1, 0, 1, 8, &p) == ZERO_EINVAL && p == nullptr, "nd 0");
    CHECK(zero_plan_create(&one, 1, 2, 4, 8, &p) == ZERO_EINVAL, "stage 4");
    CHECK(zero_plan_create(&neg, 1, 2, 1, 8, &p) == ZERO_EINVAL, "negative unit");
    CHECK(zero_plan_create(nullptr, 1, 2, 1, 8, &p) == ZERO_EINVAL, "NULL units");
    CHECK(zero_plan_create(&one, 1, 2, 1, 0, &p) == ZERO_EINVAL, "align 0");
    CHECK(zero_plan_create(&one, 1, 2, 1, 8, nullptr) == ZERO_EINVAL, "NULL out");
    Plan ok;
    CHECK(zero_plan_create(&one, 1, 2, 1, 8, &ok.p) == ZERO_OK, "small plan");
    int count = 0;
    CHECK(zero_plan_segments(ok.p, &one, 1, 2, nullptr, 0, &count) == ZERO_EINVAL, "rank out of range");
    const int64_t wrong = 9;
    CHECK(zero_plan_segments(ok.p, &wrong, 1, 0, nullptr, 0, &count) == ZERO_EINVAL, "tensors must add up");
    CHECK(zero_workspace_bytes(-1, 1) < 0 && zero_workspace_bytes(1, 1) > 0, "workspace size");
    double out = 0;
    CHECK(zero_model_state_bytes(1e9, 0, 1, 12, &out) == ZERO_EINVAL, "model state nd 0");
    CHECK(zero_comm_volume(1e9, 4, 5, &out) == ZERO_EINVAL, "comm volume stage 5");
}

// ---------------------------------------------------------------------------
// host AdamW: every instruction set, thread count and size gives the scalar
// single-thread bits; concurrent callers share the worker pool safely
// ---------------------------------------------------------------------------

struct AdamCase {
    std::vector<float> p, m, v;
    std::vector<uint16_t> g, out;
};

// A finite 16-bit gradient of either sign with a bounded exponent (fp16
// subnormals included).
uint16_t grad_bits(int dt, Rng& rng) {
    const uint16_t sign = uint16_t(rng.range(0, 1) << 15);
    if (dt == ZERO_BF16) return uint16_t(sign | uint16_t(rng.range(0x3000, 0x3f7f)));
    return uint16_t(sign | uint16_t(rng.range(0x0001, 0x2bff)));
}

AdamCase make_case(int64_t n, int gdt, uint64_t seed) {
    Rng rng{seed};
    AdamCase c;
    c.p.resize(size_t(n));
    c.m.resize(size_t(n));
    c.v.resize(size_t(n));
    c.g.resize(size_t(n));
    c.out.assign(size_t(n), 0xAAAA);
    for (int64_t i = 0; i < n; ++i) {
        c.p[size_t(i)] = float((rng.unit() - 0.5) * 0.04);
        c.m[size_t(i)] = float((rng.unit() - 0.5) * 1e-4);
        c.v[size_t(i)] = float(rng.unit() * 1e-6);
        c.g[size_t(i)] = grad_bits(gdt, rng);
    }
    return c;
}

int adam(AdamCase& c, int gdt, int pdt, int threads, float coef) {
    const zero_adam_hparams hp = {3e-4f, 0.9f, 0.95f, 1e-8f, 0.1f, 0.0625f, 3};
    return zero_cpu_adam_step(c.p.data(), c.m.data(), c.v.data(), c.g.data(), gdt, int64_t(c.p.size()), &hp, coef,
                              0, c.out.data(), pdt, threads);
}

bool same(const AdamCase& a, const AdamCase& b) {
    const size_t n = a.p.size();
    if (n == 0) return b.p.empty();
    return std::memcmp(a.p.data(), b.p.data(), 4 * n) == 0 && std::memcmp(a.m.data(), b.m.data(), 4 * n) == 0 &&
           std::memcmp(a.v.data(), b.v.data(), 4 * n) == 0 && std::memcmp(a.out.data(), b.out.data(), 2 * n) == 0;
}

void check_host_adam() {
    const int detected = zero_cpu_isa();
    const int64_t sizes[] = {0, 1, 7, 63, 64, 65, 1000, 4099, 100003};
    const int dts[3][2] = {{ZERO_BF16, ZERO_BF16}, {ZERO_F16, ZERO_F16}, {ZERO_F16, ZERO_BF16}};
    for (const auto& dt : dts) {
        for (int64_t n : sizes) {
            AdamCase ref = make_case(n, dt[0], uint64_t(n) * 7 + uint64_t(dt[0]));
            CHECK(zero_cpu_set_isa(ZERO_CPU_SCALAR) == ZERO_OK, "scalar isa");
            CHECK(adam(ref, dt[0], dt[1], 1, 0.75f) == ZERO_OK, "scalar reference n=%lld", (long long)n);
            for (int isa = ZERO_CPU_SCALAR; isa <= detected; ++isa) {
                CHECK(zero_cpu_set_isa(isa) == ZERO_OK, "isa %d", isa);
                for (int threads : {1, 3, 16}) {
                    AdamCase got = make_case(n, dt[0], uint64_t(n) * 7 + uint64_t(dt[0]));
                    CHECK(adam(got, dt[0], dt[1], threads, 0.75f) == ZERO_OK, "adam");
                    CHECK(same(got, ref), "isa %d, %d threads, n=%lld, dtypes %d/%d differ from the scalar bits", isa,
                          threads, (long long)n, dt[0], dt[1]);
                }
            }
        }
    }
    CHECK(zero_cpu_set_isa(detected) == ZERO_OK, "restore isa");

    // Two threads calling at once: each result equals a call made alone.
    AdamCase alone[2] = {make_case(50001, ZERO_BF16, 11), make_case(70001, ZERO_BF16, 12)};
    for (int k = 0; k < 2; ++k)
        for (int rep = 0; rep < 5; ++rep) CHECK(adam(alone[k], ZERO_BF16, ZERO_BF16, 8, 1.0f) == ZERO_OK, "alone");
    AdamCase both[2] = {make_case(50001, ZERO_BF16, 11), make_case(70001, ZERO_BF16, 12)};
    int rcs[2] = {0, 0};
    std::thread t0([&] { for (int rep = 0; rep < 5; ++rep) rcs[0] |= adam(both[0], ZERO_BF16, ZERO_BF16, 8, 1.0f); });
    std::thread t1([&] { for (int rep = 0; rep < 5; ++rep) rcs[1] |= adam(both[1], ZERO_BF16, ZERO_BF16, 12, 1.0f); });
    t0.join();
    t1.join();
    CHECK(rcs[0] == ZERO_OK && rcs[1] == ZERO_OK, "concurrent calls");
    CHECK(same(both[0], alone[0]) && same(both[1], alone[1]), "concurrent calls differ from calls made alone");

    // Refusals.
    AdamCase c = make_case(100, ZERO_BF16, 3);
    const zero_adam_hparams hp = {3e-4f, 0.9f, 0.95f, 1e-8f, 0.1f, 1.0f, 1};
    CHECK(zero_cpu_adam_step(c.p.data(), c.p.data(), c.v.data(), c.g.data(), ZERO_BF16, 100, &hp, 1.0f, 0,
                             c.out.data(), ZERO_BF16, 4) == ZERO_EALIAS, "master = m");
    CHECK(zero_cpu_adam_step(c.p.data(), c.m.data(), c.v.data(), c.g.data(), 7, 100, &hp, 1.0f, 0, c.out.data(),
                             ZERO_BF16, 4) == ZERO_EINVAL, "bad dtype");
    CHECK(zero_cpu_adam_step(c.p.data(), c.m.data(), c.v.data(), c.g.data(), ZERO_BF16, 100, &hp, 1.0f, 0,
                             c.out.data(), ZERO_BF16, 0) == ZERO_EINVAL, "0 threads");
    CHECK(zero_cpu_adam_step(nullptr, c.m.data(), c.v.data(), c.g.data(), ZERO_BF16, 100, &hp, 1.0f, 0,
                             c.out.data(), ZERO_BF16, 4) == ZERO_EINVAL, "NULL master");
    CHECK(zero_cpu_adam_step(c.p.data(), c.m.data(), c.v.data(), c.g.data(), ZERO_BF16, 100, nullptr, 1.0f, 0,
                             c.out.data(), ZERO_BF16, 4) == ZERO_EINVAL, "NULL hp");

    // A delayed-offload handle starts and stops its workers without an update.
    zero_offload* h = nullptr;
    CHECK(zero_offload_create(4, &h) == ZERO_OK && h != nullptr, "offload create");
    int applied = -1;
    CHECK(zero_offload_end(h, nullptr, &applied, nullptr) == ZERO_EINVAL, "end with nothing begun");
    zero_offload_destroy(h);
    CHECK(zero_offload_create(0, &h) == ZERO_EINVAL, "0 workers");
}

// ---------------------------------------------------------------------------
// sharded checkpoints in host memory: save under one partition, restore under
// another, and refuse damaged or missing files
// ---------------------------------------------------------------------------

struct Aligned {
    void* p = nullptr;
    explicit Aligned(size_t bytes) : p(std::aligned_alloc(64, (bytes + 63) / 64 * 64)) {}
    ~Aligned() { std::free(p); }
};

void check_checkpoints(const std::string& dir) {
    const int64_t units[3] = {1000, 300007, 517};
    Plan old_plan, new_plan;
    CHECK(zero_plan_create(units, 3, 4, 3, 8, &old_plan.p) == ZERO_OK, "old plan");
    CHECK(zero_plan_create(units, 3, 3, 1, 64, &new_plan.p) == ZERO_OK, "new plan");
    int64_t n_old = 0, real = 0, n_new = 0;
    zero_plan_rank(old_plan.p, 0, &n_old, &real);
    zero_plan_rank(new_plan.p, 0, &n_new, &real);
    Aligned staging(ZERO_CKPT_MIN_STAGING);
    std::vector<std::vector<float>> old_state(4 * 3);
    std::vector<std::string> paths;
    for (int r = 0; r < 4; ++r) {
        for (int a = 0; a < 3; ++a) {
            auto& s = old_state[size_t(r * 3 + a)];
            s.resize(size_t(n_old));
            for (int64_t i = 0; i < n_old; ++i) s[size_t(i)] = float(r * 1000003 + a * 7919) + float(i) * 0.5f;
        }
        paths.push_back(dir + "/rank" + std::to_string(r) + ".zck");
        CHECK(zero_ckpt_save(paths.back().c_str(), old_plan.p, r, 42, old_state[size_t(r * 3)].data(),
                             old_state[size_t(r * 3 + 1)].data(), old_state[size_t(r * 3 + 2)].data(), ZERO_LOC_HOST,
                             staging.p, ZERO_CKPT_MIN_STAGING, nullptr) == ZERO_OK,
              "save rank %d", r);
    }
    std::vector<const char*> cpaths;
    for (const auto& p : paths) cpaths.push_back(p.c_str());
    for (int r = 0; r < 3; ++r) {
        std::vector<float> st[3];
        for (auto& s : st) s.assign(size_t(n_new), -1.0f);
        int64_t step = -1;
        CHECK(zero_ckpt_load(cpaths.data(), 4, new_plan.p, r, st[0].data(), st[1].data(), st[2].data(),
                             ZERO_LOC_HOST, &step, staging.p, ZERO_CKPT_MIN_STAGING, nullptr) == ZERO_OK,
              "load rank %d", r);
        CHECK(step == 42, "saved step");
        int count = 0;
        zero_plan_reshard(old_plan.p, new_plan.p, r, nullptr, 0, &count);
        std::vector<zero_reshard_segment> runs(size_t(count > 0 ? count : 1));
        zero_plan_reshard(old_plan.p, new_plan.p, r, runs.data(), count, &count);
        std::vector<char> placed(size_t(n_new), 0);
        for (int i = 0; i < count; ++i) {
            const auto& g = runs[size_t(i)];
            for (int a = 0; a < 3; ++a)
                CHECK(std::memcmp(st[a].data() + g.new_offset,
                                  old_state[size_t(g.old_rank * 3 + a)].data() + g.old_offset, size_t(4 * g.len)) == 0,
                      "rank %d run %d array %d", r, i, a);
            std::memset(placed.data() + g.new_offset, 1, size_t(g.len));
        }
        for (int64_t i = 0; i < n_new; ++i)
            if (!placed[size_t(i)])
                for (int a = 0; a < 3; ++a) CHECK(st[a][size_t(i)] == 0.0f, "padding %lld is zero", (long long)i);
    }

    std::vector<float> a(static_cast<size_t>(n_new)), b(static_cast<size_t>(n_new)), c(static_cast<size_t>(n_new));
    int64_t step = 0;
    // one saved file too few
    CHECK(zero_ckpt_load(cpaths.data(), 3, new_plan.p, 0, a.data(), b.data(), c.data(), ZERO_LOC_HOST, &step,
                         staging.p, ZERO_CKPT_MIN_STAGING, nullptr) == ZERO_EINVAL, "three of four files");
    // a missing file
    const std::string gone = dir + "/missing.zck";
    std::vector<const char*> missing = cpaths;
    missing[2] = gone.c_str();
    CHECK(zero_ckpt_load(missing.data(), 4, new_plan.p, 0, a.data(), b.data(), c.data(), ZERO_LOC_HOST, &step,
                         staging.p, ZERO_CKPT_MIN_STAGING, nullptr) == ZERO_EIO, "missing file");
    // a damaged byte in the last file's state
    {
        FILE* f = std::fopen(paths[3].c_str(), "r+b");
        CHECK(f != nullptr, "open for damage");
        if (f) {
            std::fseek(f, -5, SEEK_END);
            const int ch = std::fgetc(f);
            std::fseek(f, -5, SEEK_END);
            std::fputc(ch ^ 0x40, f);
            std::fclose(f);
        }
        int rc = ZERO_OK;
        for (int r = 0; r < 3 && rc == ZERO_OK; ++r)
            rc = zero_ckpt_load(cpaths.data(), 4, new_plan.p, r, a.data(), b.data(), c.data(), ZERO_LOC_HOST, &step,
                                staging.p, ZERO_CKPT_MIN_STAGING, nullptr);
        CHECK(rc == ZERO_EIO, "a damaged block must be found");
    }
    // a truncated file
    CHECK(::truncate(paths[1].c_str(), 1000) == 0, "truncate");
    CHECK(zero_ckpt_load(cpaths.data(), 4, new_plan.p, 0, a.data(), b.data(), c.data(), ZERO_LOC_HOST, &step,
                         staging.p, ZERO_CKPT_MIN_STAGING, nullptr) == ZERO_EIO, "truncated file");
    // refusals before any file is touched
    CHECK(zero_ckpt_save((dir + "/x.zck").c_str(), old_plan.p, 0, 1, old_state[0].data(), old_state[1].data(),
                         old_state[2].data(), ZERO_LOC_HOST, staging.p, 64, nullptr) == ZERO_EINVAL, "small staging");
    CHECK(zero_ckpt_save((dir + "/x.zck").c_str(), old_plan.p, 9, 1, old_state[0].data(), old_state[1].data(),
                         old_state[2].data(), ZERO_LOC_HOST, staging.p, ZERO_CKPT_MIN_STAGING, nullptr) == ZERO_EINVAL,
          "rank out of range");
    struct stat sb;
    CHECK(::stat((dir + "/x.zck").c_str(), &sb) != 0, "a refused save writes no file");
    for (const auto& p : paths) ::unlink(p.c_str());
}

}  // namespace

int main(int argc, char** argv) {
    if (argc != 2) {
        std::fprintf(stderr, "usage: host_sanitize_driver TMPDIR\n");
        return 2;
    }
    check_plans();
    check_host_adam();
    check_checkpoints(argv[1]);
    if (g_failures) {
        std::fprintf(stderr, "%d check(s) failed\n", g_failures);
        return 1;
    }
    std::printf("ok: %ld checks, host AdamW instruction set %d\n", g_checks, zero_cpu_isa());
    return 0;
}

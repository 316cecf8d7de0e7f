// Sharded checkpoints: one file per rank holding that rank's fp32 optimizer
// state and the partition it was saved under, and a restore of any rank's
// shard under another partition from the files of all old ranks.
//
// Sharded training leaves every process with only its own slice of the
// weights and optimizer state; restoring at a different degree of
// parallelism has to re-own the state while keeping the parameter order and
// the moments attached to their parameters, and a missing process file must
// fail explicitly rather than produce an incomplete model (026 notes §五).
//
// File layout (little-endian):
//   Header (128 bytes) | unit sizes (int64 x n_units) |
//   block checksums (uint64 x 3 x n_blocks) | zero padding to a 4 KiB multiple |
//   master | m | v   (fp32, shard_numel each, padding positions included)
// Every array is cut into blocks of ZERO_CKPT_BLOCK elements with one
// checksum each, so a restore verifies exactly the blocks it reads.
//
// Pages cited by short name:
//   026 notes  "026｜ZeRO：数据并行中，没必要让每张卡保存全部训练状态" (wq-win.github.io)

#include <fcntl.h>
#include <hip/hip_runtime_api.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <atomic>
#include <cerrno>
#include <cstdint>
#include <cstring>
#include <string>
#include <vector>

#include "internal.h"

namespace zf {
namespace {

constexpr char kMagic[8] = {'Z', 'F', 'C', 'K', 'P', 'T', '0', '1'};
constexpr uint32_t kVersion = 1;
constexpr int64_t kBlock = ZERO_CKPT_BLOCK;
constexpr int64_t kBlockBytes = 4 * kBlock;
constexpr int kArrays = 3;

struct Header {
    char magic[8];
    uint32_t version;
    uint32_t reserved;
    int32_t nd, stage, owners, rank;
    int64_t align, n_units, psi, shard_numel, step;
    int64_t block_elems, n_blocks, data_offset;
    uint64_t meta_sum;  // checksum of the header (this field zero), the unit sizes and the block checksums
    char pad[24];
};
static_assert(sizeof(Header) == 128, "checkpoint header layout");

// 64-bit checksum of a byte range (a multiple of 4 bytes): four independent
// multiply/xor-shift lanes over 8-byte words, folded with the length.  It
// detects corruption and truncation; it is not a cryptographic hash.
uint64_t checksum(const void* data, int64_t bytes) {
    const unsigned char* p = static_cast<const unsigned char*>(data);
    constexpr uint64_t kMul = 0x9E3779B97F4A7C15ull;
    uint64_t h[4] = {0x243F6A8885A308D3ull, 0x13198A2E03707344ull, 0xA4093822299F31D0ull, 0x082EFA98EC4E6C89ull};
    const int64_t words = bytes / 8;
    int64_t i = 0;
    for (; i + 4 <= words; i += 4) {
        for (int l = 0; l < 4; ++l) {
            uint64_t w;
            std::memcpy(&w, p + 8 * (i + l), 8);
            h[l] = (h[l] ^ w) * kMul;
            h[l] ^= h[l] >> 29;
        }
    }
    for (; i < words; ++i) {
        uint64_t w;
        std::memcpy(&w, p + 8 * i, 8);
        h[i & 3] = (h[i & 3] ^ w) * kMul;
        h[i & 3] ^= h[i & 3] >> 29;
    }
    if (bytes % 8) {
        uint32_t w;
        std::memcpy(&w, p + 8 * words, 4);
        h[0] = (h[0] ^ w) * kMul;
        h[0] ^= h[0] >> 29;
    }
    uint64_t out = uint64_t(bytes) * kMul;
    for (int l = 0; l < 4; ++l) {
        out = (out ^ h[l]) * kMul;
        out ^= out >> 31;
    }
    return out;
}

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

std::string sys_reason() { return std::strerror(errno); }

struct Fd {
    int fd = -1;
    Fd() = default;
    Fd(const Fd&) = delete;
    Fd& operator=(const Fd&) = delete;
    ~Fd() {
        if (fd >= 0) ::close(fd);
    }
};

struct Events {
    hipEvent_t e[2] = {nullptr, nullptr};
    bool pending[2] = {false, false};
    Events() = default;
    Events(const Events&) = delete;
    Events& operator=(const Events&) = delete;
    ~Events() {
        for (auto& x : e)
            if (x) (void)hipEventDestroy(x);
    }
};

// Waits for the stream on every exit, so no copy still touches the caller's
// staging buffer or arrays once a call has returned (errors included).
struct StreamDrain {
    hipStream_t s;
    bool active;
    ~StreamDrain() {
        if (active) (void)hipStreamSynchronize(s);
    }
};

bool write_all(int fd, const void* buf, int64_t bytes, int64_t offset) {
    const char* p = static_cast<const char*>(buf);
    while (bytes > 0) {
        const ssize_t w = ::pwrite(fd, p, size_t(std::min<int64_t>(bytes, int64_t(1) << 30)), offset);
        if (w < 0 && errno == EINTR) continue;
        if (w <= 0) return false;
        p += w;
        bytes -= w;
        offset += w;
    }
    return true;
}

bool read_all(int fd, void* buf, int64_t bytes, int64_t offset) {
    char* p = static_cast<char*>(buf);
    while (bytes > 0) {
        const ssize_t r = ::pread(fd, p, size_t(std::min<int64_t>(bytes, int64_t(1) << 30)), offset);
        if (r < 0 && errno == EINTR) continue;
        if (r <= 0) return false;
        p += r;
        bytes -= r;
        offset += r;
    }
    return true;
}

uint64_t meta_checksum(Header h, const std::vector<int64_t>& units, const std::vector<uint64_t>& sums) {
    h.meta_sum = 0;
    std::vector<unsigned char> buf(sizeof(Header) + 8 * units.size() + 8 * sums.size());
    std::memcpy(buf.data(), &h, sizeof(Header));
    if (!units.empty()) std::memcpy(buf.data() + sizeof(Header), units.data(), 8 * units.size());
    if (!sums.empty()) std::memcpy(buf.data() + sizeof(Header) + 8 * units.size(), sums.data(), 8 * sums.size());
    return checksum(buf.data(), int64_t(buf.size()));
}

int check_staging(const char* fn, void* staging, int64_t staging_bytes) {
    if (staging == nullptr || (reinterpret_cast<uintptr_t>(staging) & 63) || staging_bytes < ZERO_CKPT_MIN_STAGING)
        return fail(ZERO_EINVAL, std::string(fn) + ": staging must be 64-byte aligned and at least " +
                                     std::to_string(ZERO_CKPT_MIN_STAGING) + " bytes");
    return ZERO_OK;
}

int hip_error(hipError_t e, const char* fn) {
    return fail(ZERO_EHIP, std::string(fn) + ": " + hipGetErrorString(e));
}

// A saved file, opened and checked.
struct SavedFile {
    Fd fd;
    Header h{};
    std::vector<int64_t> units;
    std::vector<uint64_t> sums;  // [array][block]
};

int open_saved(const char* fn, const char* path, int index, SavedFile& f) {
    const std::string who = std::string(fn) + ": rank " + std::to_string(index) + " file '" + path + "'";
    f.fd.fd = ::open(path, O_RDONLY | O_CLOEXEC);
    if (f.fd.fd < 0) return fail(ZERO_EIO, who + " cannot be opened: " + sys_reason());
    if (!read_all(f.fd.fd, &f.h, sizeof(Header), 0)) return fail(ZERO_EIO, who + " is too short for a header");
    if (std::memcmp(f.h.magic, kMagic, 8) != 0) return fail(ZERO_EIO, who + " is not a checkpoint file");
    if (f.h.version != kVersion)
        return fail(ZERO_EIO, who + " has format version " + std::to_string(f.h.version) + ", expected " +
                                  std::to_string(kVersion));
    if (f.h.n_units < 1 || f.h.n_units > (int64_t(1) << 24) || f.h.shard_numel < 0 || f.h.block_elems != kBlock ||
        f.h.n_blocks != (f.h.shard_numel + kBlock - 1) / kBlock || f.h.owners < 1 || f.h.owners > ZERO_MAX_RANKS)
        return fail(ZERO_EIO, who + " has a corrupt header");
    try {
        f.units.resize(size_t(f.h.n_units));
        f.sums.resize(size_t(kArrays * f.h.n_blocks));
    } catch (const std::bad_alloc&) {
        return fail(ZERO_ENOMEM, who + ": out of host memory");
    }
    if (!read_all(f.fd.fd, f.units.data(), 8 * f.h.n_units, sizeof(Header)) ||
        (!f.sums.empty() && !read_all(f.fd.fd, f.sums.data(), 8 * int64_t(f.sums.size()),
                                      sizeof(Header) + 8 * f.h.n_units)))
        return fail(ZERO_EIO, who + " is truncated inside its header");
    if (meta_checksum(f.h, f.units, f.sums) != f.h.meta_sum) return fail(ZERO_EIO, who + " has a corrupt header");
    struct stat st;
    if (::fstat(f.fd.fd, &st) != 0) return fail(ZERO_EIO, who + ": " + sys_reason());
    const int64_t want = f.h.data_offset + int64_t(kArrays) * 4 * f.h.shard_numel;
    if (int64_t(st.st_size) != want)
        return fail(ZERO_EIO, who + " holds " + std::to_string(int64_t(st.st_size)) + " bytes, expected " +
                                  std::to_string(want) + " (truncated or foreign)");
    if (f.h.rank != index)
        return fail(ZERO_EINVAL, who + " holds rank " + std::to_string(f.h.rank) + "'s state");
    return ZERO_OK;
}

bool same_run(const SavedFile& a, const SavedFile& b) {
    return a.h.nd == b.h.nd && a.h.stage == b.h.stage && a.h.owners == b.h.owners && a.h.align == b.h.align &&
           a.h.psi == b.h.psi && a.h.shard_numel == b.h.shard_numel && a.h.step == b.h.step && a.units == b.units;
}

}  // namespace
}  // namespace zf

using namespace zf;

extern "C" {

int zero_ckpt_save(const char* path, const zero_plan* plan, int rank, int64_t step, const float* master,
                   const float* m, const float* v, int location, void* staging, int64_t staging_bytes,
                   void* stream) {
    const char* fn = "zero_ckpt_save";
    if (path == nullptr || plan == nullptr) return fail(ZERO_EINVAL, std::string(fn) + ": NULL path or plan");
    if (rank < 0 || rank >= plan->nd) return fail(ZERO_EINVAL, std::string(fn) + ": rank out of range");
    if (rank >= plan->owners) return fail(ZERO_EINVAL, std::string(fn) + ": this rank owns no shard");
    if (step < 0) return fail(ZERO_EINVAL, std::string(fn) + ": step < 0");
    if (location != ZERO_LOC_DEVICE && location != ZERO_LOC_HOST)
        return fail(ZERO_EINVAL, std::string(fn) + ": location must be ZERO_LOC_DEVICE or ZERO_LOC_HOST");
    const int64_t n = plan->shard_numel;
    const float* arrays[kArrays] = {master, m, v};
    for (const float* a : arrays)
        if (n > 0 && (a == nullptr || (reinterpret_cast<uintptr_t>(a) & 3)))
            return fail(ZERO_EINVAL, std::string(fn) + ": master, m and v must be non-NULL and 4-byte aligned");
    if (int rc = check_staging(fn, staging, staging_bytes)) return rc;

    Header h{};
    std::memcpy(h.magic, kMagic, 8);
    h.version = kVersion;
    h.nd = plan->nd;
    h.stage = plan->stage;
    h.owners = plan->owners;
    h.rank = rank;
    h.align = plan->align;
    h.n_units = int64_t(plan->units.size());
    h.psi = plan_psi(*plan);
    h.shard_numel = n;
    h.step = step;
    h.block_elems = kBlock;
    h.n_blocks = (n + kBlock - 1) / kBlock;
    h.data_offset = round_up(int64_t(sizeof(Header)) + 8 * h.n_units + 8 * kArrays * h.n_blocks, 4096);
    std::vector<int64_t> units;
    std::vector<uint64_t> sums;
    try {
        for (const auto& u : plan->units) units.push_back(u.numel);
        sums.assign(size_t(kArrays * h.n_blocks), 0);
    } catch (const std::bad_alloc&) {
        return fail(ZERO_ENOMEM, std::string(fn) + ": out of host memory");
    }
    // A stage-3 plan lists its units; stages 0-2 merge them into one, which
    // loses nothing a restore needs (the flat order is the same).

    // The temporary name is unique to this process and call, so two saves to
    // one path never write the same file; the last rename wins, whole.
    static std::atomic<uint64_t> save_serial{0};
    const std::string tmp = std::string(path) + ".tmp." + std::to_string(::getpid()) + "." +
                            std::to_string(save_serial.fetch_add(1));
    Fd out;
    out.fd = ::open(tmp.c_str(), O_WRONLY | O_CREAT | O_EXCL | O_CLOEXEC, 0644);
    if (out.fd < 0) return fail(ZERO_EIO, std::string(fn) + ": cannot create '" + tmp + "': " + sys_reason());
    auto abandon = [&](int rc) {
        ::close(out.fd);
        out.fd = -1;
        ::unlink(tmp.c_str());
        return rc;
    };

    // Items (array, first element) in file order, each at most one staging slot.
    const int64_t slot_elems = std::max<int64_t>(1, staging_bytes / 2 / kBlockBytes) * kBlock;
    char* slots[2] = {static_cast<char*>(staging), static_cast<char*>(staging) + 4 * slot_elems};
    struct Item {
        int a;
        int64_t lo, len;
    };
    std::vector<Item> items;
    for (int a = 0; a < kArrays; ++a)
        for (int64_t lo = 0; lo < n; lo += slot_elems) items.push_back({a, lo, std::min(slot_elems, n - lo)});
    hipStream_t s = static_cast<hipStream_t>(stream);
    Events ev;
    StreamDrain drain{s, location == ZERO_LOC_DEVICE};
    if (location == ZERO_LOC_DEVICE)
        for (auto& e : ev.e)
            if (hipError_t err = hipEventCreateWithFlags(&e, hipEventDisableTiming)) return abandon(hip_error(err, fn));
    auto fetch = [&](size_t k) -> int {  // device -> slot k&1
        const Item& it = items[k];
        hipError_t e = hipMemcpyAsync(slots[k & 1], arrays[it.a] + it.lo, size_t(4 * it.len), hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipEventRecord(ev.e[k & 1], s);
        return e == hipSuccess ? ZERO_OK : hip_error(e, fn);
    };
    if (location == ZERO_LOC_DEVICE && !items.empty())
        if (int rc = fetch(0)) return abandon(rc);
    for (size_t k = 0; k < items.size(); ++k) {
        const Item& it = items[k];
        const void* src;
        if (location == ZERO_LOC_DEVICE) {
            if (k + 1 < items.size())
                if (int rc = fetch(k + 1)) return abandon(rc);
            if (hipError_t e = hipEventSynchronize(ev.e[k & 1])) return abandon(hip_error(e, fn));
            src = slots[k & 1];
        } else {
            src = arrays[it.a] + it.lo;
        }
        // item boundaries fall on block boundaries (slot_elems is a multiple of kBlock)
        for (int64_t b = it.lo / kBlock; b * kBlock < it.lo + it.len; ++b) {
            const int64_t e0 = b * kBlock, e1 = std::min(n, e0 + kBlock);
            sums[size_t(it.a * h.n_blocks + b)] =
                checksum(static_cast<const char*>(src) + 4 * (e0 - it.lo), 4 * (e1 - e0));
        }
        const int64_t off = h.data_offset + (int64_t(it.a) * n + it.lo) * 4;
        if (!write_all(out.fd, src, 4 * it.len, off))
            return abandon(fail(ZERO_EIO, std::string(fn) + ": writing '" + tmp + "': " + sys_reason()));
    }
    h.meta_sum = meta_checksum(h, units, sums);
    std::vector<unsigned char> meta(size_t(h.data_offset), 0);
    std::memcpy(meta.data(), &h, sizeof(Header));
    std::memcpy(meta.data() + sizeof(Header), units.data(), 8 * units.size());
    if (!sums.empty()) std::memcpy(meta.data() + sizeof(Header) + 8 * units.size(), sums.data(), 8 * sums.size());
    if (!write_all(out.fd, meta.data(), h.data_offset, 0))
        return abandon(fail(ZERO_EIO, std::string(fn) + ": writing '" + tmp + "': " + sys_reason()));
    if (n == 0 && ::ftruncate(out.fd, h.data_offset) != 0)
        return abandon(fail(ZERO_EIO, std::string(fn) + ": sizing '" + tmp + "': " + sys_reason()));
    // On stable storage before it takes the final name, and the name itself after.
    if (::fsync(out.fd) != 0)
        return abandon(fail(ZERO_EIO, std::string(fn) + ": flushing '" + tmp + "': " + sys_reason()));
    if (::close(out.fd) != 0) {
        out.fd = -1;
        ::unlink(tmp.c_str());
        return fail(ZERO_EIO, std::string(fn) + ": closing '" + tmp + "': " + sys_reason());
    }
    out.fd = -1;
    if (::rename(tmp.c_str(), path) != 0) {
        ::unlink(tmp.c_str());
        return fail(ZERO_EIO, std::string(fn) + ": renaming to '" + path + "': " + sys_reason());
    }
    const std::string p(path);
    const size_t slash = p.find_last_of('/');
    const std::string dir = slash == std::string::npos ? "." : (slash == 0 ? "/" : p.substr(0, slash));
    Fd d;
    d.fd = ::open(dir.c_str(), O_RDONLY | O_DIRECTORY | O_CLOEXEC);
    if (d.fd < 0 || ::fsync(d.fd) != 0)
        return fail(ZERO_EIO, std::string(fn) + ": flushing directory '" + dir + "': " + sys_reason());
    return ok();
}

int zero_ckpt_load(const char* const* paths, int n_paths, const zero_plan* plan, int rank, float* master, float* m,
                   float* v, int location, int64_t* step_out, void* staging, int64_t staging_bytes, void* stream) {
    const char* fn = "zero_ckpt_load";
    if (paths == nullptr || plan == nullptr || step_out == nullptr)
        return fail(ZERO_EINVAL, std::string(fn) + ": NULL paths, plan or step_out");
    if (n_paths < 1 || n_paths > ZERO_MAX_RANKS) return fail(ZERO_EINVAL, std::string(fn) + ": n_paths out of range");
    if (rank < 0 || rank >= plan->nd) return fail(ZERO_EINVAL, std::string(fn) + ": rank out of range");
    if (location != ZERO_LOC_DEVICE && location != ZERO_LOC_HOST)
        return fail(ZERO_EINVAL, std::string(fn) + ": location must be ZERO_LOC_DEVICE or ZERO_LOC_HOST");
    const int64_t n_new = plan->shard_numel;
    float* dst[kArrays] = {master, m, v};
    for (float* a : dst)
        if (n_new > 0 && (a == nullptr || (reinterpret_cast<uintptr_t>(a) & 3)))
            return fail(ZERO_EINVAL, std::string(fn) + ": master, m and v must be non-NULL and 4-byte aligned");
    for (int i = 0; i < n_paths; ++i)
        if (paths[i] == nullptr) return fail(ZERO_EINVAL, std::string(fn) + ": paths[" + std::to_string(i) + "] is NULL");
    if (int rc = check_staging(fn, staging, staging_bytes)) return rc;

    // Every old rank's file must be present and from the same run.
    std::vector<SavedFile> files(static_cast<size_t>(n_paths));
    for (int i = 0; i < n_paths; ++i)
        if (int rc = open_saved(fn, paths[i], i, files[size_t(i)])) return rc;
    const Header& h0 = files[0].h;
    if (n_paths != h0.owners)
        return fail(ZERO_EINVAL, std::string(fn) + ": the saved run has " + std::to_string(h0.owners) +
                                     " shard files, got " + std::to_string(n_paths));
    for (int i = 1; i < n_paths; ++i)
        if (!same_run(files[0], files[size_t(i)]))
            return fail(ZERO_EINVAL, std::string(fn) + ": rank " + std::to_string(i) + " file '" + paths[i] +
                                         "' belongs to another run or step than rank 0's");
    zero_plan* old_raw = nullptr;
    if (int rc = zero_plan_create(files[0].units.data(), int(h0.n_units), h0.nd, h0.stage, h0.align, &old_raw))
        return fail(rc, std::string(fn) + ": the saved partition is invalid: " + zero_last_error());
    struct PlanGuard {
        zero_plan* p;
        ~PlanGuard() { zero_plan_destroy(p); }
    } old_guard{old_raw};
    if (old_raw->shard_numel != h0.shard_numel || plan_psi(*old_raw) != h0.psi)
        return fail(ZERO_EIO, std::string(fn) + ": rank 0 file '" + paths[0] + "' disagrees with its own partition");
    if (h0.psi != plan_psi(*plan))
        return fail(ZERO_EINVAL, std::string(fn) + ": the saved run has " + std::to_string(h0.psi) +
                                     " parameters, the plan " + std::to_string(plan_psi(*plan)));
    std::vector<zero_reshard_segment> runs;
    try {
        reshard_runs(*old_raw, *plan, rank, runs);
    } catch (const std::bad_alloc&) {
        return fail(ZERO_ENOMEM, std::string(fn) + ": out of host memory");
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    Events ev;
    StreamDrain drain{s, location == ZERO_LOC_DEVICE};
    // Padding positions (in no run) are zero.
    {
        int64_t pos = 0;
        auto zero = [&](int64_t lo, int64_t hi) -> int {
            if (hi <= lo) return ZERO_OK;
            for (float* a : dst) {
                if (location == ZERO_LOC_HOST) {
                    std::memset(a + lo, 0, size_t(4 * (hi - lo)));
                } else if (hipError_t e = hipMemsetAsync(a + lo, 0, size_t(4 * (hi - lo)), s)) {
                    return hip_error(e, fn);
                }
            }
            return ZERO_OK;
        };
        for (const auto& r : runs) {
            if (int rc = zero(pos, r.new_offset)) return rc;
            pos = r.new_offset + r.len;
        }
        if (int rc = zero(pos, n_new)) return rc;
    }

    // Copy every run block by block through the two staging slots; each block
    // read is verified before any of it is used.
    const int64_t n_old = h0.shard_numel;
    const int64_t slot_elems = std::max<int64_t>(1, staging_bytes / 2 / kBlockBytes) * kBlock;
    char* slots[2] = {static_cast<char*>(staging), static_cast<char*>(staging) + 4 * slot_elems};
    if (location == ZERO_LOC_DEVICE)
        for (auto& e : ev.e)
            if (hipError_t err = hipEventCreateWithFlags(&e, hipEventDisableTiming)) return hip_error(err, fn);
    int slot = 0;
    for (int a = 0; a < kArrays; ++a) {
        for (const auto& r : runs) {
            const SavedFile& f = files[size_t(r.old_rank)];
            int64_t x = r.old_offset;  // next old-shard element of this run to place
            const int64_t x_end = r.old_offset + r.len;
            while (x < x_end) {
                const int64_t b_lo = x / kBlock;
                const int64_t span_lo = b_lo * kBlock;
                const int64_t span_hi = std::min({n_old, span_lo + slot_elems, round_up(x_end, kBlock)});
                if (location == ZERO_LOC_DEVICE && ev.pending[slot]) {
                    if (hipError_t e = hipEventSynchronize(ev.e[slot])) return hip_error(e, fn);
                    ev.pending[slot] = false;
                }
                char* buf = slots[slot];
                const int64_t off = f.h.data_offset + (int64_t(a) * n_old + span_lo) * 4;
                if (!read_all(f.fd.fd, buf, 4 * (span_hi - span_lo), off))
                    return fail(ZERO_EIO, std::string(fn) + ": rank " + std::to_string(r.old_rank) + " file '" +
                                              paths[r.old_rank] + "': read failed: " + sys_reason());
                for (int64_t b = b_lo; b * kBlock < span_hi; ++b) {
                    const int64_t e0 = b * kBlock, e1 = std::min(n_old, e0 + kBlock);
                    if (checksum(buf + 4 * (e0 - span_lo), 4 * (e1 - e0)) != f.sums[size_t(a * f.h.n_blocks + b)])
                        return fail(ZERO_EIO, std::string(fn) + ": rank " + std::to_string(r.old_rank) + " file '" +
                                                  paths[r.old_rank] + "': block " + std::to_string(b) + " of array " +
                                                  std::to_string(a) + " is corrupt");
                }
                const int64_t take = std::min(x_end, span_hi) - x;
                float* to = dst[a] + r.new_offset + (x - r.old_offset);
                const char* from = buf + 4 * (x - span_lo);
                if (location == ZERO_LOC_HOST) {
                    std::memcpy(to, from, size_t(4 * take));
                } else {
                    hipError_t e = hipMemcpyAsync(to, from, size_t(4 * take), hipMemcpyHostToDevice, s);
                    if (e == hipSuccess) e = hipEventRecord(ev.e[slot], s);
                    if (e != hipSuccess) return hip_error(e, fn);
                    ev.pending[slot] = true;
                    slot ^= 1;
                }
                x += take;
            }
        }
    }
    if (location == ZERO_LOC_DEVICE)
        if (hipError_t e = hipStreamSynchronize(s)) return hip_error(e, fn);
    *step_out = h0.step;
    return ok();
}

}  // extern "C"

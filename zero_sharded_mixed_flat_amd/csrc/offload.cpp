// CPU-offloaded optimizer (ZeRO-Offload): AdamW on host-resident fp32 state,
// and the step that streams the reduced gradient from HBM to the host, runs
// the host AdamW chunk by chunk and streams the 16-bit parameters back.
//
// ZeRO-Offload keeps only the 16-bit parameters and gradients on the GPU and
// moves the fp32 master, m and v (12 bytes per parameter) to host memory,
// where a multi-threaded, vectorised Adam updates them; each step sends the
// gradient to the host and the 16-bit parameters back (L18 notes §4.4).
//
// Arithmetic: the GPU kernel's sequence -- the fp32 state, the 16-bit gradient
// and the fp32 scalars widened to fp64, one IEEE fp64 rounding per operation
// with no fused multiply-add, correctly rounded division and square root, and
// one rounding of m', v' and p' to fp32 -- so the AVX-512, AVX2 and scalar
// paths give identical bits on every x86-64 host, and the same bits as the
// GPU.  fp16 conversions use the F16C instructions on the vector paths (round
// to nearest even) and an exact software conversion on the scalar path; bf16
// uses integer rounding.
//
// Pages cited by short name:
//   L18 notes  CMU 11-868 Lecture 18 notes, "Memory Optimization in Distributed Training: ZeRO" (semidirectx.com)

#include <hip/hip_runtime_api.h>
#include <immintrin.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <condition_variable>
#include <cstdint>
#include <cstring>
#include <functional>
#include <memory>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "internal.h"

namespace zf {
namespace {

// The step's scalars widened to fp64 (exactly: each is an fp32 value; gs is
// inv_loss_scale times the clip multiplier, exact because the former is a
// power of two).
struct HostAdam {
    double lr, b1, b2, omb1, omb2, eps, wd, gs, bc1, bc2;
};

// ---------------------------------------------------------------------------
// scalar 16-bit <-> fp32, exact, from the IEEE 754 encodings
// ---------------------------------------------------------------------------

inline float bits_to_float(uint32_t u) {
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

inline uint32_t float_to_bits(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return u;
}

inline float widen_scalar(uint16_t b, int dt) {
    if (dt == ZERO_BF16) return bits_to_float(uint32_t(b) << 16);
    const uint32_t sign = uint32_t(b & 0x8000u) << 16;
    const uint32_t e = (b >> 10) & 0x1fu, mant = b & 0x3ffu;
    if (e == 0x1f) return bits_to_float(sign | 0x7f800000u | (mant << 13));
    if (e == 0) {
        const float mag = float(mant) * 0x1p-24f;  // subnormal: mant units of 2^-24, exact
        return sign ? -mag : mag;
    }
    return bits_to_float(sign | ((e + 112u) << 23) | (mant << 13));
}

inline uint16_t narrow_scalar(float x, int dt) {
    uint32_t u = float_to_bits(x);
    if (dt == ZERO_BF16) {
        if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
        return uint16_t((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
    }
    const uint16_t sign = uint16_t((u >> 16) & 0x8000u);
    u &= 0x7fffffffu;
    if (u > 0x7f800000u) return sign | 0x7e00u;        // NaN
    if (u >= 0x477ff000u) return sign | 0x7c00u;       // at least 65520: rounds to infinity
    if (u >= 0x38800000u) {                            // normal fp16 range (>= 2^-14)
        uint32_t r = u - 0x38000000u;                  // rebias the exponent by 127 - 15
        r += 0x0fffu + ((r >> 13) & 1u);               // round to nearest even on 13 dropped bits
        return uint16_t(sign | (r >> 13));
    }
    if (u <= 0x33000000u) return sign;                 // at most 2^-25: rounds to zero
    const uint32_t e = u >> 23, m = (u & 0x7fffffu) | 0x800000u;
    const uint32_t shift = 126u - e;                   // value = m * 2^(e - 150) = (m >> shift) units of 2^-24
    uint32_t q = m >> shift;
    const uint32_t rem = m & ((1u << shift) - 1u), half = 1u << (shift - 1u);
    if (rem > half || (rem == half && (q & 1u))) ++q;
    return uint16_t(sign | q);
}

inline void adam_scalar(const HostAdam& c, float* p, float* m, float* v, const uint16_t* g16, int gdt,
                        uint16_t* out, int pdt, int64_t lo, int64_t hi) {
    for (int64_t i = lo; i < hi; ++i) {
        const double g = double(widen_scalar(g16[i], gdt)) * c.gs;
        const double m2 = c.b1 * double(m[i]) + c.omb1 * g;
        const double v2 = c.b2 * double(v[i]) + c.omb2 * (g * g);
        const double p0 = double(p[i]);
        const double p2 = p0 - c.lr * ((m2 / c.bc1) / (std::sqrt(v2 / c.bc2) + c.eps) + c.wd * p0);
        m[i] = float(m2);
        v[i] = float(v2);
        p[i] = float(p2);
        out[i] = narrow_scalar(p[i], pdt);
    }
}

// ---------------------------------------------------------------------------
// AVX-512: 8 elements (one register of fp64) per iteration
// ---------------------------------------------------------------------------

__attribute__((target("avx512f,avx512bw,avx512vl,avx2,f16c"))) void adam_avx512(
    const HostAdam& c, float* p, float* m, float* v, const uint16_t* g16, int gdt, uint16_t* out, int pdt,
    int64_t lo, int64_t hi) {
    const __m512d b1 = _mm512_set1_pd(c.b1), b2 = _mm512_set1_pd(c.b2), omb1 = _mm512_set1_pd(c.omb1),
                  omb2 = _mm512_set1_pd(c.omb2), eps = _mm512_set1_pd(c.eps), lr = _mm512_set1_pd(c.lr),
                  wd = _mm512_set1_pd(c.wd), gs = _mm512_set1_pd(c.gs), bc1 = _mm512_set1_pd(c.bc1),
                  bc2 = _mm512_set1_pd(c.bc2);
    const __m256i abs_mask = _mm256_set1_epi32(0x7fffffff), inf = _mm256_set1_epi32(0x7f800000),
                  round = _mm256_set1_epi32(0x7fff), one = _mm256_set1_epi32(1),
                  qnan = _mm256_set1_epi32(0x7fc0);
    // The 16-bit output is written once and never read here: streaming stores
    // skip the read of each line a plain store would do first (2 bytes of host
    // traffic per element).  They need 16-byte alignment, which a range keeps
    // once its first element has it, and a fence before the range is done.
    const bool stream = (reinterpret_cast<uintptr_t>(out + lo) & 15) == 0;
    int64_t i = lo;
    for (; i + 8 <= hi; i += 8) {
        const __m128i graw = _mm_loadu_si128(reinterpret_cast<const __m128i*>(g16 + i));
        const __m256 g32 = gdt == ZERO_BF16 ? _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_cvtepu16_epi32(graw), 16))
                                            : _mm256_cvtph_ps(graw);
        const __m512d g = _mm512_mul_pd(_mm512_cvtps_pd(g32), gs);
        const __m512d p0 = _mm512_cvtps_pd(_mm256_loadu_ps(p + i));
        const __m512d m2 =
            _mm512_add_pd(_mm512_mul_pd(b1, _mm512_cvtps_pd(_mm256_loadu_ps(m + i))), _mm512_mul_pd(omb1, g));
        const __m512d v2 = _mm512_add_pd(_mm512_mul_pd(b2, _mm512_cvtps_pd(_mm256_loadu_ps(v + i))),
                                         _mm512_mul_pd(omb2, _mm512_mul_pd(g, g)));
        const __m512d denom = _mm512_add_pd(_mm512_sqrt_pd(_mm512_div_pd(v2, bc2)), eps);
        const __m512d upd = _mm512_add_pd(_mm512_div_pd(_mm512_div_pd(m2, bc1), denom), _mm512_mul_pd(wd, p0));
        const __m256 pf = _mm512_cvtpd_ps(_mm512_sub_pd(p0, _mm512_mul_pd(lr, upd)));
        _mm256_storeu_ps(m + i, _mm512_cvtpd_ps(m2));
        _mm256_storeu_ps(v + i, _mm512_cvtpd_ps(v2));
        _mm256_storeu_ps(p + i, pf);
        __m128i o;
        if (pdt == ZERO_BF16) {
            const __m256i u = _mm256_castps_si256(pf);
            const __mmask8 nan = _mm256_cmpgt_epi32_mask(_mm256_and_si256(u, abs_mask), inf);
            const __m256i lsb = _mm256_and_si256(_mm256_srli_epi32(u, 16), one);
            __m256i r = _mm256_srli_epi32(_mm256_add_epi32(_mm256_add_epi32(u, round), lsb), 16);
            r = _mm256_mask_mov_epi32(r, nan, qnan);
            o = _mm256_cvtepi32_epi16(r);
        } else {
            o = _mm256_cvtps_ph(pf, _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC);
        }
        if (stream)
            _mm_stream_si128(reinterpret_cast<__m128i*>(out + i), o);
        else
            _mm_storeu_si128(reinterpret_cast<__m128i*>(out + i), o);
    }
    if (stream) _mm_sfence();
    adam_scalar(c, p, m, v, g16, gdt, out, pdt, i, hi);
}

// ---------------------------------------------------------------------------
// AVX2: 8 elements (two registers of fp64) per iteration
// ---------------------------------------------------------------------------

__attribute__((target("avx2,f16c"))) void adam_avx2(const HostAdam& c, float* p, float* m, float* v,
                                                     const uint16_t* g16, int gdt, uint16_t* out, int pdt,
                                                     int64_t lo, int64_t hi) {
    const __m256d b1 = _mm256_set1_pd(c.b1), b2 = _mm256_set1_pd(c.b2), omb1 = _mm256_set1_pd(c.omb1),
                  omb2 = _mm256_set1_pd(c.omb2), eps = _mm256_set1_pd(c.eps), lr = _mm256_set1_pd(c.lr),
                  wd = _mm256_set1_pd(c.wd), gs = _mm256_set1_pd(c.gs), bc1 = _mm256_set1_pd(c.bc1),
                  bc2 = _mm256_set1_pd(c.bc2);
    const __m256i abs_mask = _mm256_set1_epi32(0x7fffffff), inf = _mm256_set1_epi32(0x7f800000),
                  round = _mm256_set1_epi32(0x7fff), one = _mm256_set1_epi32(1),
                  qnan = _mm256_set1_epi32(0x7fc0);
    const bool stream = (reinterpret_cast<uintptr_t>(out + lo) & 15) == 0;   // as in the AVX-512 path
    int64_t i = lo;
    for (; i + 8 <= hi; i += 8) {
        const __m128i graw = _mm_loadu_si128(reinterpret_cast<const __m128i*>(g16 + i));
        const __m256 g32 = gdt == ZERO_BF16 ? _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_cvtepu16_epi32(graw), 16))
                                            : _mm256_cvtph_ps(graw);
        __m128 ph[2];
        for (int h = 0; h < 2; ++h) {
            const int64_t j = i + 4 * h;
            const __m128 gh = h ? _mm256_extractf128_ps(g32, 1) : _mm256_castps256_ps128(g32);
            const __m256d g = _mm256_mul_pd(_mm256_cvtps_pd(gh), gs);
            const __m256d p0 = _mm256_cvtps_pd(_mm_loadu_ps(p + j));
            const __m256d m2 =
                _mm256_add_pd(_mm256_mul_pd(b1, _mm256_cvtps_pd(_mm_loadu_ps(m + j))), _mm256_mul_pd(omb1, g));
            const __m256d v2 = _mm256_add_pd(_mm256_mul_pd(b2, _mm256_cvtps_pd(_mm_loadu_ps(v + j))),
                                             _mm256_mul_pd(omb2, _mm256_mul_pd(g, g)));
            const __m256d denom = _mm256_add_pd(_mm256_sqrt_pd(_mm256_div_pd(v2, bc2)), eps);
            const __m256d upd =
                _mm256_add_pd(_mm256_div_pd(_mm256_div_pd(m2, bc1), denom), _mm256_mul_pd(wd, p0));
            ph[h] = _mm256_cvtpd_ps(_mm256_sub_pd(p0, _mm256_mul_pd(lr, upd)));
            _mm_storeu_ps(m + j, _mm256_cvtpd_ps(m2));
            _mm_storeu_ps(v + j, _mm256_cvtpd_ps(v2));
            _mm_storeu_ps(p + j, ph[h]);
        }
        const __m256 pf = _mm256_set_m128(ph[1], ph[0]);
        __m128i o;
        if (pdt == ZERO_BF16) {
            const __m256i u = _mm256_castps_si256(pf);
            const __m256i nan = _mm256_cmpgt_epi32(_mm256_and_si256(u, abs_mask), inf);
            const __m256i lsb = _mm256_and_si256(_mm256_srli_epi32(u, 16), one);
            __m256i r = _mm256_srli_epi32(_mm256_add_epi32(_mm256_add_epi32(u, round), lsb), 16);
            r = _mm256_blendv_epi8(r, qnan, nan);
            o = _mm_packus_epi32(_mm256_castsi256_si128(r), _mm256_extracti128_si256(r, 1));
        } else {
            o = _mm256_cvtps_ph(pf, _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC);
        }
        if (stream)
            _mm_stream_si128(reinterpret_cast<__m128i*>(out + i), o);
        else
            _mm_storeu_si128(reinterpret_cast<__m128i*>(out + i), o);
    }
    if (stream) _mm_sfence();
    adam_scalar(c, p, m, v, g16, gdt, out, pdt, i, hi);
}

// ---------------------------------------------------------------------------
// dispatch and threads
// ---------------------------------------------------------------------------

int detect_isa() {
    __builtin_cpu_init();
    if (__builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
        __builtin_cpu_supports("avx512vl") && __builtin_cpu_supports("f16c"))
        return ZERO_CPU_AVX512;
    if (__builtin_cpu_supports("avx2") && __builtin_cpu_supports("f16c")) return ZERO_CPU_AVX2;
    return ZERO_CPU_SCALAR;
}

const int g_detected_isa = detect_isa();
std::atomic<int> g_isa{g_detected_isa};

void adam_range(int isa, const HostAdam& c, float* p, float* m, float* v, const uint16_t* g16, int gdt,
                uint16_t* out, int pdt, int64_t lo, int64_t hi) {
    if (isa == ZERO_CPU_AVX512)
        adam_avx512(c, p, m, v, g16, gdt, out, pdt, lo, hi);
    else if (isa == ZERO_CPU_AVX2)
        adam_avx2(c, p, m, v, g16, gdt, out, pdt, lo, hi);
    else
        adam_scalar(c, p, m, v, g16, gdt, out, pdt, lo, hi);
}

constexpr int kMaxThreads = 256;
constexpr int64_t kMinPerThread = 1 << 15;  // smaller ranges are not worth a thread

// Worker threads that live across calls.  start() hands parts 0..parts-1 of
// a job to the workers and returns; wait() returns once every part is done.
// One job at a time: the owner of the pool orders start and wait.
class WorkerPool {
  public:
    explicit WorkerPool(int n) {
        threads_.reserve(n);
        for (int i = 0; i < n; ++i) threads_.emplace_back([this] { loop(); });
    }
    ~WorkerPool() {
        {
            std::lock_guard<std::mutex> lock(mu_);
            stop_ = true;
        }
        work_.notify_all();
        for (auto& t : threads_) t.join();
    }
    int size() const { return int(threads_.size()); }
    void start(int parts, std::function<void(int)> fn) {
        std::lock_guard<std::mutex> lock(mu_);
        job_ = std::move(fn);
        parts_ = parts;
        next_ = 0;
        done_ = 0;
        ++generation_;
        work_.notify_all();
    }
    void wait() {
        std::unique_lock<std::mutex> lock(mu_);
        finished_.wait(lock, [this] { return done_ == parts_; });
        job_ = nullptr;
    }

  private:
    void loop() {
        uint64_t seen = 0;
        std::unique_lock<std::mutex> lock(mu_);
        for (;;) {
            work_.wait(lock, [&] { return stop_ || (generation_ != seen && next_ < parts_); });
            if (stop_) return;
            seen = generation_;
            while (next_ < parts_) {
                const int k = next_++;
                lock.unlock();
                job_(k);
                lock.lock();
                if (++done_ == parts_) finished_.notify_all();
            }
        }
    }
    std::mutex mu_;
    std::condition_variable work_, finished_;
    std::vector<std::thread> threads_;
    std::function<void(int)> job_;
    int parts_ = 0, next_ = 0, done_ = 0;
    uint64_t generation_ = 0;
    bool stop_ = false;
};

// Contiguous, 64-element-aligned parts of [0, n), at most n_threads of them.
struct Split {
    int parts;
    int64_t per;
};

Split split(int64_t n, int n_threads) {
    const int64_t by_size = std::max<int64_t>(1, n / kMinPerThread);
    const int t = int(std::min<int64_t>(n_threads, by_size));
    const int64_t per = ((n + t - 1) / t + 63) / 64 * 64;
    return Split{int((n + per - 1) / per), per};
}

std::function<void(int)> adam_job(const HostAdam& c, float* p, float* m, float* v, const uint16_t* g16, int gdt,
                                  uint16_t* out, int pdt, int64_t n, int64_t per) {
    const int isa = g_isa.load();
    return [=](int k) {
        const int64_t lo = std::min<int64_t>(n, k * per), hi = std::min<int64_t>(n, lo + per);
        if (lo < hi) adam_range(isa, c, p, m, v, g16, gdt, out, pdt, lo, hi);
    };
}

// The workers of the synchronous host AdamW calls, shared by the process and
// grown to the largest thread count asked for (calls run one at a time).
std::mutex g_pool_mutex;
std::unique_ptr<WorkerPool> g_pool;

// The whole range on n_threads workers; returns when the update is done.
void adam_threads(const HostAdam& c, float* p, float* m, float* v, const uint16_t* g16, int gdt, uint16_t* out,
                  int pdt, int64_t n, int n_threads) {
    const Split sp = split(n, n_threads);
    if (sp.parts <= 1) {
        adam_range(g_isa.load(), c, p, m, v, g16, gdt, out, pdt, 0, n);
        return;
    }
    std::lock_guard<std::mutex> lock(g_pool_mutex);
    if (!g_pool || g_pool->size() < sp.parts) {
        g_pool.reset();
        g_pool = std::make_unique<WorkerPool>(sp.parts);
    }
    g_pool->start(sp.parts, adam_job(c, p, m, v, g16, gdt, out, pdt, n, sp.per));
    g_pool->wait();
}

constexpr int64_t kOffloadMinStaging = ZERO_OFFLOAD_MIN_STAGING;  // head room + four slots of 64 values
static_assert(ZERO_OFFLOAD_MIN_STAGING == 64 + 8 * 64, "staging layout");

int hip_fail(hipError_t e, const char* where) {
    return fail(ZERO_EHIP, std::string(where) + ": " + hipGetErrorString(e));
}

bool valid_dtype_h(int dt) { return dt == ZERO_F16 || dt == ZERO_BF16; }

uintptr_t addr_h(const void* p) { return reinterpret_cast<uintptr_t>(p); }

bool overlaps_h(const void* a, int64_t ab, const void* b, int64_t bb) {
    if (ab <= 0 || bb <= 0) return false;
    return addr_h(a) < addr_h(b) + uintptr_t(bb) && addr_h(b) < addr_h(a) + uintptr_t(ab);
}

bool pow2_positive_h(float x) {
    if (!(x > 0.0f) || !std::isfinite(x)) return false;
    int e;
    return std::frexp(x, &e) == 0.5f;
}

// Shared validation of the hyperparameters; fills the fp32 constants.
int make_consts(const char* fn, const zero_adam_hparams* hp, float coef, HostAdam* c) {
    if (hp == nullptr) return fail(ZERO_EINVAL, std::string(fn) + ": hp is NULL");
    if (!std::isfinite(hp->lr) || !std::isfinite(hp->eps) || !std::isfinite(hp->weight_decay) ||
        !(hp->beta1 >= 0.0f && hp->beta1 < 1.0f) || !(hp->beta2 >= 0.0f && hp->beta2 < 1.0f))
        return fail(ZERO_EINVAL, std::string(fn) + ": hyperparameters must be finite, betas in [0, 1)");
    if (hp->step < 1) return fail(ZERO_EINVAL, std::string(fn) + ": step must be >= 1");
    if (!pow2_positive_h(hp->inv_loss_scale))
        return fail(ZERO_EINVAL, std::string(fn) + ": inv_loss_scale must be a positive power of two");
    if (!std::isfinite(coef) || !(coef > 0.0f))
        return fail(ZERO_EINVAL, std::string(fn) + ": coef must be finite and positive");
    const float bc1 = float(1.0 - std::pow(double(hp->beta1), double(hp->step)));
    const float bc2 = float(1.0 - std::pow(double(hp->beta2), double(hp->step)));
    if (!(bc1 > 0.0f) || !(bc2 > 0.0f)) return fail(ZERO_EINVAL, std::string(fn) + ": bias correction is zero");
    c->lr = hp->lr;
    c->b1 = hp->beta1;
    c->b2 = hp->beta2;
    c->omb1 = float(1.0 - double(hp->beta1));
    c->omb2 = float(1.0 - double(hp->beta2));
    c->eps = hp->eps;
    c->wd = hp->weight_decay;
    c->gs = double(hp->inv_loss_scale) * double(coef);
    c->bc1 = bc1;
    c->bc2 = bc2;
    return ZERO_OK;
}

int check_host_buffers(const char* fn, float* master, float* m, float* v, const void* grad, const void* param,
                       int64_t n) {
    if (!master || !m || !v || !grad || !param) return fail(ZERO_EINVAL, std::string(fn) + ": NULL buffer");
    if ((addr_h(master) | addr_h(m) | addr_h(v)) & 3)
        return fail(ZERO_EINVAL, std::string(fn) + ": fp32 buffers must be 4-byte aligned");
    if ((addr_h(grad) | addr_h(param)) & 1)
        return fail(ZERO_EINVAL, std::string(fn) + ": 16-bit buffers must be 2-byte aligned");
    const void* outs[4] = {master, m, v, param};
    const int64_t ob[4] = {4 * n, 4 * n, 4 * n, 2 * n};
    for (int i = 0; i < 4; ++i) {
        for (int j = i + 1; j < 4; ++j)
            if (overlaps_h(outs[i], ob[i], outs[j], ob[j]))
                return fail(ZERO_EALIAS, std::string(fn) + ": master, m, v and the parameters must not overlap");
        if (overlaps_h(outs[i], ob[i], grad, 2 * n))
            return fail(ZERO_EALIAS, std::string(fn) + ": an output overlaps the gradient");
    }
    return ZERO_OK;
}

using HostUpdate = std::function<void(const HostAdam&, float*, float*, float*, const uint16_t*, uint16_t*, int64_t)>;

// The offloaded update of [0, n) in chunks through two gradient slots and two
// parameter slots of pinned staging, on stream s: chunk k's gradient comes to
// the host (slot k%2), the host AdamW updates it, its parameters go back from
// slot k%2.  The copy of chunk k+1 is queued before chunk k is updated, and a
// slot's parameters are rewritten only after their copy to the device is
// done.  Returns once every copy has been queued; the caller synchronises s.
int stream_chunks(const char* fn, const HostAdam& c, float* master, float* m, float* v, const uint16_t* g_dev,
                  int grad_dtype, uint16_t* p_dev, int param_dtype, int64_t n, uint16_t* const gslot[2],
                  uint16_t* const pslot[2], int64_t chunk, hipEvent_t got[2], hipEvent_t sent[2], hipStream_t s,
                  const HostUpdate& update) {
    (void)grad_dtype;
    (void)param_dtype;
    auto status = [&](hipError_t e) { return e == hipSuccess ? ZERO_OK : hip_fail(e, fn); };
    const int64_t n_chunks = (n + chunk - 1) / chunk;
    auto enqueue_in = [&](int64_t k) {
        const int64_t lo = k * chunk, len = std::min(chunk, n - lo);
        hipError_t e = hipMemcpyAsync(gslot[k & 1], g_dev + lo, 2 * len, hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipEventRecord(got[k & 1], s);
        return status(e);
    };
    int rc = enqueue_in(0);
    bool sent_pending[2] = {false, false};
    for (int64_t k = 0; k < n_chunks && rc == ZERO_OK; ++k) {
        const int64_t lo = k * chunk, len = std::min(chunk, n - lo);
        if (k + 1 < n_chunks) rc = enqueue_in(k + 1);
        if (rc == ZERO_OK) rc = status(hipEventSynchronize(got[k & 1]));
        if (rc == ZERO_OK && sent_pending[k & 1]) rc = status(hipEventSynchronize(sent[k & 1]));
        if (rc != ZERO_OK) break;
        update(c, master + lo, m + lo, v + lo, gslot[k & 1], pslot[k & 1], len);
        rc = status(hipMemcpyAsync(p_dev + lo, pslot[k & 1], 2 * len, hipMemcpyHostToDevice, s));
        if (rc == ZERO_OK) rc = status(hipEventRecord(sent[k & 1], s));
        sent_pending[k & 1] = true;
    }
    return rc;
}

// State of a one-step-delayed update between its begin and end calls.
struct Pending {
    bool active = false;
    bool applied = false;
    int64_t n = 0;
    uint16_t* next_params = nullptr;   // the parameters in flight, in the caller's device buffer
};

}  // namespace
}  // namespace zf

// The host side of the delayed ZeRO-Offload update: persistent workers for the
// host AdamW and, while an update is in flight, the thread that drives its
// copies on a stream of its own.
struct zero_offload {
    std::unique_ptr<zf::WorkerPool> pool;
    std::thread driver;
    int driver_rc = ZERO_OK;
    std::string driver_msg;
    zf::Pending pending;
};

using namespace zf;

extern "C" {

int zero_cpu_isa(void) { return g_isa.load(); }

int zero_cpu_set_isa(int isa) {
    if (isa < ZERO_CPU_SCALAR || isa > g_detected_isa)
        return fail(ZERO_EINVAL, "zero_cpu_set_isa: not supported by this CPU");
    g_isa.store(isa);
    return ok();
}

int zero_cpu_adam_step(float* master, float* m, float* v, const void* grad, int grad_dtype, int64_t n,
                       const zero_adam_hparams* hp, float coef, int skip, void* param_out, int param_dtype,
                       int n_threads) {
    const char* fn = "zero_cpu_adam_step";
    if (n < 0 || n > ZERO_MAX_ELEMS) return fail(ZERO_EINVAL, std::string(fn) + ": n must be in [0, 2^34]");
    if (!valid_dtype_h(grad_dtype) || !valid_dtype_h(param_dtype))
        return fail(ZERO_EINVAL, std::string(fn) + ": dtypes must be ZERO_F16 or ZERO_BF16");
    if (n_threads < 1 || n_threads > kMaxThreads)
        return fail(ZERO_EINVAL, std::string(fn) + ": n_threads must be in [1, 256]");
    HostAdam c;
    if (int rc = make_consts(fn, hp, coef, &c)) return rc;
    if (n == 0 || skip) return ok();
    if (int rc = check_host_buffers(fn, master, m, v, grad, param_out, n)) return rc;
    adam_threads(c, master, m, v, static_cast<const uint16_t*>(grad), grad_dtype, static_cast<uint16_t*>(param_out),
                 param_dtype, n, n_threads);
    return ok();
}

int zero_offload_adam_step(float* master, float* m, float* v, const void* grad_dev, int grad_dtype, int64_t n,
                           const zero_adam_hparams* hp, const float* coef_dev, const int32_t* flag_dev,
                           void* param_dev, int param_dtype, void* staging, int64_t staging_bytes, int n_threads,
                           void* stream) {
    const char* fn = "zero_offload_adam_step";
    if (n < 0 || n > ZERO_MAX_ELEMS) return fail(ZERO_EINVAL, std::string(fn) + ": n must be in [0, 2^34]");
    if (!valid_dtype_h(grad_dtype) || !valid_dtype_h(param_dtype))
        return fail(ZERO_EINVAL, std::string(fn) + ": dtypes must be ZERO_F16 or ZERO_BF16");
    if (n_threads < 1 || n_threads > kMaxThreads)
        return fail(ZERO_EINVAL, std::string(fn) + ": n_threads must be in [1, 256]");
    HostAdam c;
    if (int rc = make_consts(fn, hp, 1.0f, &c)) return rc;
    if (coef_dev == nullptr || (addr_h(coef_dev) & 3) || flag_dev == nullptr || (addr_h(flag_dev) & 3))
        return fail(ZERO_EINVAL, std::string(fn) + ": coef_dev or flag NULL or misaligned");
    if (n == 0) return ok();
    if (int rc = check_host_buffers(fn, master, m, v, grad_dev, param_dev, n)) return rc;
    if (staging == nullptr || (addr_h(staging) & 63) || staging_bytes < kOffloadMinStaging)
        return fail(ZERO_EINVAL, std::string(fn) + ": staging must be 64-byte aligned and at least " +
                                     std::to_string(kOffloadMinStaging) + " bytes");
    if (overlaps_h(staging, staging_bytes, master, 4 * n) || overlaps_h(staging, staging_bytes, m, 4 * n) ||
        overlaps_h(staging, staging_bytes, v, 4 * n))
        return fail(ZERO_EALIAS, std::string(fn) + ": staging overlaps the host state");

    hipStream_t s = static_cast<hipStream_t>(stream);
    // Staging: 8 bytes of head room for the clip multiplier and the flag, then
    // two gradient slots and two parameter slots of `chunk` 16-bit values.
    char* st = static_cast<char*>(staging);
    float* coef_h = reinterpret_cast<float*>(st);
    int32_t* flag_h = reinterpret_cast<int32_t*>(st + 4);
    const int64_t chunk = std::min<int64_t>(n, (staging_bytes - 64) / 8 / 64 * 64);
    uint16_t* gslot[2] = {reinterpret_cast<uint16_t*>(st + 64), reinterpret_cast<uint16_t*>(st + 64) + chunk};
    uint16_t* pslot[2] = {gslot[1] + chunk, gslot[1] + 2 * chunk};
    const uint16_t* g_dev = static_cast<const uint16_t*>(grad_dev);
    uint16_t* p_dev = static_cast<uint16_t*>(param_dev);

    auto status = [&](hipError_t e) { return e == hipSuccess ? ZERO_OK : hip_fail(e, fn); };
    hipEvent_t got[2] = {nullptr, nullptr}, sent[2] = {nullptr, nullptr};
    int rc = ZERO_OK;
    for (int k = 0; k < 2 && rc == ZERO_OK; ++k) {
        rc = status(hipEventCreateWithFlags(&got[k], hipEventDisableTiming));
        if (rc == ZERO_OK) rc = status(hipEventCreateWithFlags(&sent[k], hipEventDisableTiming));
    }
    auto cleanup = [&]() {
        for (int k = 0; k < 2; ++k) {
            if (got[k]) (void)hipEventDestroy(got[k]);
            if (sent[k]) (void)hipEventDestroy(sent[k]);
        }
    };
    if (rc != ZERO_OK) {
        cleanup();
        return rc;
    }
    // The clip multiplier and the skip flag come first: the update needs both.
    rc = status(hipMemcpyAsync(coef_h, coef_dev, 4, hipMemcpyDeviceToHost, s));
    if (rc == ZERO_OK) rc = status(hipMemcpyAsync(flag_h, flag_dev, 4, hipMemcpyDeviceToHost, s));
    if (rc == ZERO_OK) rc = status(hipStreamSynchronize(s));
    if (rc == ZERO_OK && *flag_h != 0) {  // skipped step: nothing moves
        cleanup();
        return ok();
    }
    if (rc == ZERO_OK && !(std::isfinite(*coef_h) && *coef_h > 0.0f))
        rc = fail(ZERO_EINVAL, std::string(fn) + ": the clip multiplier on the device is not finite and positive");
    if (rc == ZERO_OK) c.gs = double(hp->inv_loss_scale) * double(*coef_h);

    if (rc == ZERO_OK)
        rc = stream_chunks(fn, c, master, m, v, g_dev, grad_dtype, p_dev, param_dtype, n, gslot, pslot, chunk, got,
                           sent, s, [&](const HostAdam& cc, float* pp, float* mm, float* vv, const uint16_t* gg,
                                        uint16_t* oo, int64_t len) {
                               adam_threads(cc, pp, mm, vv, gg, grad_dtype, oo, param_dtype, len, n_threads);
                           });
    // The staging buffer is the caller's again only once every copy has ended.
    const hipError_t e = hipStreamSynchronize(s);
    if (rc == ZERO_OK) rc = status(e);
    cleanup();
    return rc == ZERO_OK ? ok() : rc;
}

int zero_offload_create(int n_threads, zero_offload** out) {
    const char* fn = "zero_offload_create";
    if (out == nullptr) return fail(ZERO_EINVAL, std::string(fn) + ": out is NULL");
    *out = nullptr;
    if (n_threads < 1 || n_threads > kMaxThreads)
        return fail(ZERO_EINVAL, std::string(fn) + ": n_threads must be in [1, 256]");
    std::unique_ptr<zero_offload> h(new (std::nothrow) zero_offload());
    if (!h) return fail(ZERO_ENOMEM, std::string(fn) + ": out of host memory");
    h->pool = std::make_unique<WorkerPool>(n_threads);
    *out = h.release();
    return ok();
}

void zero_offload_destroy(zero_offload* h) {
    if (h == nullptr) return;
    if (h->driver.joinable()) h->driver.join();
    delete h;
}

int zero_offload_begin(zero_offload* h, float* master, float* m, float* v, const void* grad_dev, int grad_dtype,
                       int64_t n, const zero_adam_hparams* hp, const float* coef_dev, const int32_t* flag_dev,
                       int param_dtype, void* device_buffer, int64_t device_bytes, void* staging,
                       int64_t staging_bytes, void* stream) {
    const char* fn = "zero_offload_begin";
    if (h == nullptr) return fail(ZERO_EINVAL, std::string(fn) + ": handle is NULL");
    if (h->pending.active) return fail(ZERO_EINVAL, std::string(fn) + ": the previous update has not ended");
    if (n < 0 || n > ZERO_MAX_ELEMS) return fail(ZERO_EINVAL, std::string(fn) + ": n must be in [0, 2^34]");
    if (!valid_dtype_h(grad_dtype) || !valid_dtype_h(param_dtype))
        return fail(ZERO_EINVAL, std::string(fn) + ": dtypes must be ZERO_F16 or ZERO_BF16");
    HostAdam c;
    if (int rc = make_consts(fn, hp, 1.0f, &c)) return rc;
    if (coef_dev == nullptr || (addr_h(coef_dev) & 3) || flag_dev == nullptr || (addr_h(flag_dev) & 3))
        return fail(ZERO_EINVAL, std::string(fn) + ": coef_dev or flag NULL or misaligned");
    if (staging == nullptr || (addr_h(staging) & 63) || staging_bytes < kOffloadMinStaging)
        return fail(ZERO_EINVAL, std::string(fn) + ": staging must be 64-byte aligned and at least " +
                                     std::to_string(kOffloadMinStaging) + " bytes");
    if (n > 0) {
        if (!master || !m || !v || !grad_dev) return fail(ZERO_EINVAL, std::string(fn) + ": NULL buffer");
        if ((addr_h(master) | addr_h(m) | addr_h(v)) & 3)
            return fail(ZERO_EINVAL, std::string(fn) + ": fp32 buffers must be 4-byte aligned");
        if ((addr_h(grad_dev) | addr_h(device_buffer)) & 1)
            return fail(ZERO_EINVAL, std::string(fn) + ": 16-bit buffers must be 2-byte aligned");
        if (device_buffer == nullptr || device_bytes < 4 * n)
            return fail(ZERO_EINVAL, std::string(fn) + ": device_buffer NULL or smaller than 4 * n bytes");
        const void* outs[3] = {master, m, v};
        for (int i = 0; i < 3; ++i) {
            for (int j = i + 1; j < 3; ++j)
                if (overlaps_h(outs[i], 4 * n, outs[j], 4 * n))
                    return fail(ZERO_EALIAS, std::string(fn) + ": master, m and v must not overlap");
            if (overlaps_h(outs[i], 4 * n, staging, staging_bytes))
                return fail(ZERO_EALIAS, std::string(fn) + ": staging overlaps the host state");
        }
        if (overlaps_h(device_buffer, 4 * n, grad_dev, 2 * n))
            return fail(ZERO_EALIAS, std::string(fn) + ": device_buffer overlaps the gradient");
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* st = static_cast<char*>(staging);
    float* coef_h = reinterpret_cast<float*>(st);
    int32_t* flag_h = reinterpret_cast<int32_t*>(st + 4);
    hipError_t e = hipMemcpyAsync(coef_h, coef_dev, 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipMemcpyAsync(flag_h, flag_dev, 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, fn);
    if (*flag_h != 0 || n == 0) {            // a skipped step moves nothing
        h->pending = Pending{true, false, n, nullptr};
        return ok();
    }
    if (!(std::isfinite(*coef_h) && *coef_h > 0.0f))
        return fail(ZERO_EINVAL, std::string(fn) + ": the clip multiplier on the device is not finite and positive");
    c.gs = double(hp->inv_loss_scale) * double(*coef_h);

    // The gradient is copied aside on the device (stream order), so the caller's
    // next step may overwrite it at once; the update's parameters collect in the
    // second half of device_buffer until zero_offload_end.
    uint16_t* snapshot = static_cast<uint16_t*>(device_buffer);
    uint16_t* next_params = snapshot + n;
    hipEvent_t ready = nullptr;
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ready, hipEventDisableTiming);
    if (e == hipSuccess) e = hipMemcpyAsync(snapshot, grad_dev, size_t(2 * n), hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess) e = hipEventRecord(ready, s);
    if (e != hipSuccess) {
        if (ready) (void)hipEventDestroy(ready);
        return hip_fail(e, fn);
    }
    const int64_t chunk = std::min<int64_t>(n, (staging_bytes - 64) / 8 / 64 * 64);
    h->pending = Pending{true, true, n, next_params};
    h->driver_rc = ZERO_OK;
    h->driver_msg.clear();
    WorkerPool* pool = h->pool.get();
    h->driver = std::thread([h, pool, c, master, m, v, snapshot, next_params, grad_dtype, param_dtype, n, st, chunk,
                             ready, dev]() {
        const char* dfn = "zero_offload_begin (update in flight)";
        hipStream_t s2 = nullptr;
        hipEvent_t got[2] = {nullptr, nullptr}, sent[2] = {nullptr, nullptr};
        hipError_t e2 = hipSetDevice(dev);
        if (e2 == hipSuccess) e2 = hipStreamCreateWithFlags(&s2, hipStreamNonBlocking);
        if (e2 == hipSuccess) e2 = hipStreamWaitEvent(s2, ready, 0);
        for (int k = 0; k < 2 && e2 == hipSuccess; ++k) {
            e2 = hipEventCreateWithFlags(&got[k], hipEventDisableTiming);
            if (e2 == hipSuccess) e2 = hipEventCreateWithFlags(&sent[k], hipEventDisableTiming);
        }
        int rc = e2 == hipSuccess ? ZERO_OK : hip_fail(e2, dfn);
        if (rc == ZERO_OK) {
            uint16_t* gslot[2] = {reinterpret_cast<uint16_t*>(st + 64), reinterpret_cast<uint16_t*>(st + 64) + chunk};
            uint16_t* pslot[2] = {gslot[1] + chunk, gslot[1] + 2 * chunk};
            rc = stream_chunks(dfn, c, master, m, v, snapshot, grad_dtype, next_params, param_dtype, n, gslot, pslot,
                               chunk, got, sent, s2,
                               [&](const HostAdam& cc, float* pp, float* mm, float* vv, const uint16_t* gg,
                                   uint16_t* oo, int64_t len) {
                                   const Split sp = split(len, pool->size());
                                   pool->start(sp.parts, adam_job(cc, pp, mm, vv, gg, grad_dtype, oo, param_dtype,
                                                                  len, sp.per));
                                   pool->wait();
                               });
        }
        if (s2 != nullptr) {
            const hipError_t e3 = hipStreamSynchronize(s2);   // every copy of the update has ended
            if (rc == ZERO_OK && e3 != hipSuccess) rc = hip_fail(e3, dfn);
            (void)hipStreamDestroy(s2);
        }
        for (int k = 0; k < 2; ++k) {
            if (got[k]) (void)hipEventDestroy(got[k]);
            if (sent[k]) (void)hipEventDestroy(sent[k]);
        }
        (void)hipEventDestroy(ready);
        h->driver_rc = rc;
        if (rc != ZERO_OK) h->driver_msg = zero_last_error();
    });
    return ok();
}

int zero_offload_end(zero_offload* h, void* param_dev, int* applied, void* stream) {
    const char* fn = "zero_offload_end";
    if (h == nullptr) return fail(ZERO_EINVAL, std::string(fn) + ": handle is NULL");
    if (!h->pending.active) return fail(ZERO_EINVAL, std::string(fn) + ": no update has begun");
    const Pending pd = h->pending;
    if (pd.applied && (param_dev == nullptr || (addr_h(param_dev) & 1)))
        return fail(ZERO_EINVAL, std::string(fn) + ": param_dev NULL or misaligned");
    if (pd.applied && overlaps_h(param_dev, 2 * pd.n, pd.next_params - pd.n, 4 * pd.n))
        return fail(ZERO_EALIAS, std::string(fn) + ": param_dev overlaps the update's device buffer");
    if (h->driver.joinable()) h->driver.join();
    h->pending = Pending{};
    if (applied != nullptr) *applied = pd.applied ? 1 : 0;
    if (h->driver_rc != ZERO_OK) {
        const int rc = h->driver_rc;
        h->driver_rc = ZERO_OK;
        return fail(rc, h->driver_msg);
    }
    if (!pd.applied) return ok();
    const hipError_t e = hipMemcpyAsync(param_dev, pd.next_params, size_t(2 * pd.n), hipMemcpyDeviceToDevice,
                                        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, fn);
}

}  // extern "C"

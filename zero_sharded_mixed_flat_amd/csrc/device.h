// Device and launch helpers shared by the HIP sources of the library:
// vector types, streaming (non-temporal) accesses, 16-bit <-> fp32
// conversions, the deterministic block sum, index spans, argument checks and
// a launch wrapper that reports the launch's own status.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <string>
#include <tuple>
#include <utility>

#include "internal.h"

namespace zf {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ T ld_stream(const T* p) {
    return __builtin_nontemporal_load(p);
}

template <typename T>
__device__ __forceinline__ void st_stream(T* p, T v) {
    __builtin_nontemporal_store(v, p);
}

// ---------------------------------------------------------------------------
// 16-bit <-> fp32
// ---------------------------------------------------------------------------

template <int DT>
__device__ __forceinline__ float widen(uint32_t b);

template <>
__device__ __forceinline__ float widen<ZERO_F16>(uint32_t b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
}

template <>
__device__ __forceinline__ float widen<ZERO_BF16>(uint32_t b) {
    return __uint_as_float(b << 16);
}

// Round to nearest, ties to even.  fp16 uses the hardware conversion (IEEE
// mode, subnormals kept); bf16 is the upper half of the fp32 pattern after
// adding 0x7FFF plus the lowest kept bit, NaN mapped to 0x7FC0.
template <int DT>
__device__ __forceinline__ uint32_t narrow(float x);

template <>
__device__ __forceinline__ uint32_t narrow<ZERO_F16>(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

template <>
__device__ __forceinline__ uint32_t narrow<ZERO_BF16>(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

template <int DT>
__device__ __forceinline__ bool finite16(uint32_t b) {
    constexpr uint32_t e = DT == ZERO_F16 ? 0x7c00u : 0x7f80u;
    return (b & e) != e;
}

// Four 16-bit values packed in a u2 (little-endian order).
__device__ __forceinline__ uint32_t half_of(const u2& w, int k) {
    const uint32_t word = (k < 2) ? w.x : w.y;
    return (k & 1) ? (word >> 16) : (word & 0xffffu);
}

__device__ __forceinline__ u2 pack4(const uint32_t (&h)[4]) {
    return u2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
}

// ---------------------------------------------------------------------------
// Deterministic block reduction: xor-butterfly inside each 64-lane wave, then
// thread 0 adds the per-wave sums in wave order.  Same tree on every run.
// ---------------------------------------------------------------------------

template <int BLOCK>
__device__ __forceinline__ double block_sum(double v) {
    constexpr int kWaves = BLOCK / 64;
    __shared__ double wave_sums[kWaves];
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) wave_sums[wave] = v;
    __syncthreads();
    double total = 0.0;
    if (threadIdx.x == 0) {
        for (int w = 0; w < kWaves; ++w) total += wave_sums[w];
    }
    return total;  // valid in thread 0 only
}

// ---------------------------------------------------------------------------
// Index spaces
// ---------------------------------------------------------------------------

// With `vec` set, elements [head, head + 4*nq) form the quad body (every
// pointer aligned for quad accesses there) and the `head` elements before and
// the tail after it (fewer than 8 in all) are done one by one by the last
// block.  Without it every element is done one by one, block b taking a
// contiguous range of elements.
struct Span {
    int64_t n;
    int64_t head;
    int64_t nq;
    int vec;
};

struct Ptrs64 {
    const uint16_t* p[64];
};

// ---------------------------------------------------------------------------
// Host-side helpers
// ---------------------------------------------------------------------------

inline bool valid_dtype(int dt) { return dt == ZERO_F16 || dt == ZERO_BF16; }

inline uintptr_t addr(const void* p) { return reinterpret_cast<uintptr_t>(p); }

inline bool overlaps(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
    if (a_bytes <= 0 || b_bytes <= 0) return false;
    const uintptr_t a0 = addr(a), b0 = addr(b);
    return a0 < b0 + uintptr_t(b_bytes) && b0 < a0 + uintptr_t(a_bytes);
}

inline bool pow2_positive(float x) {
    if (!(x > 0.0f) || !std::isfinite(x)) return false;
    int e;
    return std::frexp(x, &e) == 0.5f;
}

// Quad span for a set of arrays: `head` elements (0..3) bring every 16-bit
// pointer to an 8-byte and every fp32 pointer to a 16-byte boundary.  If no
// common head exists (or n is tiny) every element goes one by one.
inline Span make_span(int64_t n, const void* const* ptrs16, int n16, const void* const* ptrs32, int n32) {
    Span sp{n, 0, 0, 0};
    if (n == 0) return sp;
    int64_t head;
    if (n16 > 0) {
        const uintptr_t mis = addr(ptrs16[0]) & 7;
        if (mis & 1) return sp;
        head = int64_t((8 - mis) & 7) / 2;
    } else {
        const uintptr_t mis = addr(ptrs32[0]) & 15;
        if (mis & 3) return sp;
        head = int64_t((16 - mis) & 15) / 4;
    }
    for (int i = 0; i < n16; ++i)
        if (((addr(ptrs16[i]) + 2 * uintptr_t(head)) & 7) != 0) return sp;
    for (int i = 0; i < n32; ++i)
        if (((addr(ptrs32[i]) + 4 * uintptr_t(head)) & 15) != 0) return sp;
    if (head + 4 > n) return sp;
    sp.head = head;
    sp.nq = (n - head) / 4;
    sp.vec = 1;
    return sp;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int hip_status(hipError_t e, const char* where) {
    if (e != hipSuccess) return fail(ZERO_EHIP, std::string(where) + ": " + hipGetErrorString(e));
    return ok();
}

// More than 64 rank pointers reach the kernels through a table copied from
// host memory into the workspace.  A captured graph would keep that copy's
// host address, not the pointers, so such calls refuse to be captured.
inline int refuse_capture(hipStream_t s, const char* fn) {
    hipStreamCaptureStatus status = hipStreamCaptureStatusNone;
    const hipError_t e = hipStreamIsCapturing(s, &status);
    if (e != hipSuccess) return hip_status(e, fn);
    if (status != hipStreamCaptureStatusNone)
        return fail(ZERO_EINVAL, std::string(fn) +
                                     ": more than 64 ranks cannot be captured in a graph (the pointer table is "
                                     "copied from host memory)");
    return ZERO_OK;
}

// Launches `kernel` and returns the status of THIS launch.  hipGetLastError()
// is not used: it also reports earlier failures of other libraries' calls on
// this thread.  The arguments are converted to the kernel's parameter types.
template <typename... KArgs, typename... Actual>
hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t s, Actual&&... a) {
    static_assert(sizeof...(KArgs) == sizeof...(Actual), "argument count");
    std::tuple<KArgs...> args(std::forward<Actual>(a)...);
    return std::apply(
        [&](auto&... x) {
            void* argv[] = {static_cast<void*>(&x)...};
            return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, s);
        },
        args);
}

}  // namespace
}  // namespace zf

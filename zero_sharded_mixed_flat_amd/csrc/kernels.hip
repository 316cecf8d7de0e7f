// Device side of one ZeRO rank's share of a mixed-precision Adam step, for
// MI355X (gfx950, wave64), plus the C-ABI entry points that validate their
// arguments and launch it.
//
// Every kernel here streams HBM: nothing is a contraction, so there is no
// MFMA.  The design points are 16-byte vector loads and stores (8 16-bit
// values per lane per access), grid-stride loops over 64-bit indices, one
// read and one write of each fp32 state array per step, and a deterministic
// two-level (wave shuffle, then LDS) fp64 reduction for the norm whose tree
// depends only on the element count.
//
//   reduce_kernel   a1: Nd contributions -> rank-order fp32 mean -> 16-bit,
//                   fused per-block fp64 sums of squares and the inf/NaN flag
//                   (L18 notes §2.2 step 3, §2.5).
//   sumsq_kernel    a2: the same sums of squares over an already-reduced
//                   gradient.
//   finalize_kernel a2: fixed-order fp64 sum of the partials -> norm and the
//                   clip multiplier (L18 notes §1.4; L3.2 §4.2).
//   adam_kernel     a3: AdamW on fp32 master/m/v, cast to 16 bits (L18 notes
//                   §2.2 step 4).
//   gather_kernel   a4: 16-bit shards -> the unit's slice of the full buffer
//                   (L18 notes §2.2 step 5; Illustrated ZeRO §8.4).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <string>
#include <tuple>
#include <utility>
#include <vector>

#include "internal.h"

namespace zf {
namespace {

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

__device__ __forceinline__ void unpack8(const uint4& w, uint32_t (&h)[8]) {
    h[0] = w.x & 0xffffu; h[1] = w.x >> 16;
    h[2] = w.y & 0xffffu; h[3] = w.y >> 16;
    h[4] = w.z & 0xffffu; h[5] = w.z >> 16;
    h[6] = w.w & 0xffffu; h[7] = w.w >> 16;
}

__device__ __forceinline__ uint4 pack8(const uint32_t (&h)[8]) {
    return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                      h[6] | (h[7] << 16));
}

// ---------------------------------------------------------------------------
// Deterministic block reduction: xor-butterfly inside each 64-lane wave, then
// wave 0 adds the per-wave sums in wave order.  Same tree on every run.
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
// a1: reduce
// ---------------------------------------------------------------------------

struct Ptrs64 {
    const uint16_t* p[64];
};

// Elements [head, head + 8*nvec) go through the 16-byte vector body; the
// `head` elements before and the tail after it through the scalar loop.
struct Span {
    int64_t n;
    int64_t head;
    int64_t nvec;
};

// ND > 0: rank count known at compile time (<= 64), pointers in kernel args.
// ND == 0: runtime rank count <= 64, pointers in kernel args.
// ND < 0: runtime rank count > 64, pointers in a device table (workspace).
template <int DT, int ND>
__global__ __launch_bounds__(kBlock) void reduce_kernel(Ptrs64 tab, const uint16_t* const* dtab,
                                                        int nd, Span sp, float inv_nd, float nd_f,
                                                        int pow2, float inv_s,
                                                        uint16_t* __restrict__ out,
                                                        double* __restrict__ partials,
                                                        int32_t* __restrict__ flag) {
#pragma clang fp contract(off)
    const int64_t tid = int64_t(blockIdx.x) * kBlock + threadIdx.x;
    const int64_t stride = int64_t(gridDim.x) * kBlock;
    const int ranks = ND > 0 ? ND : nd;
    double sq = 0.0;
    int bad = 0;

    auto src = [&](int r) -> const uint16_t* {
        if constexpr (ND >= 0) return tab.p[r];
        else return dtab[r];
    };
    auto finish = [&](float acc) -> uint32_t {
        const float mean = pow2 ? acc * inv_nd : acc / nd_f;
        const uint32_t o = narrow<DT>(mean);
        bad |= !finite16<DT>(o);
        const double d = double(widen<DT>(o)) * double(inv_s);
        sq += d * d;
        return o;
    };

    for (int64_t i = tid; i < sp.nvec; i += stride) {
        const int64_t e = sp.head + i * 8;
        float acc[8];
        uint32_t h[8];
        unpack8(*reinterpret_cast<const uint4*>(src(0) + e), h);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = widen<DT>(h[k]);
        if constexpr (ND > 0) {
#pragma unroll
            for (int r = 1; r < ND; ++r) {
                unpack8(*reinterpret_cast<const uint4*>(src(r) + e), h);
#pragma unroll
                for (int k = 0; k < 8; ++k) acc[k] = acc[k] + widen<DT>(h[k]);
            }
        } else {
            for (int r = 1; r < ranks; ++r) {
                unpack8(*reinterpret_cast<const uint4*>(src(r) + e), h);
#pragma unroll
                for (int k = 0; k < 8; ++k) acc[k] = acc[k] + widen<DT>(h[k]);
            }
        }
        uint32_t o[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = finish(acc[k]);
        *reinterpret_cast<uint4*>(out + e) = pack8(o);
    }

    const int64_t tail0 = sp.head + 8 * sp.nvec;
    const int64_t nscalar = sp.head + (sp.n - tail0);
    for (int64_t k = tid; k < nscalar; k += stride) {
        const int64_t e = k < sp.head ? k : tail0 + (k - sp.head);
        float acc = widen<DT>(src(0)[e]);
        for (int r = 1; r < ranks; ++r) acc = acc + widen<DT>(src(r)[e]);
        out[e] = static_cast<uint16_t>(finish(acc));
    }

    const double total = block_sum<kBlock>(sq);
    const int any_bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) {
        partials[blockIdx.x] = total;
        if (any_bad) atomicOr(flag, ZERO_FLAG_NONFINITE_GRAD);
    }
}

// ---------------------------------------------------------------------------
// a2: sums of squares of a pre-reduced gradient, and the finalize
// ---------------------------------------------------------------------------

template <int DT>
__global__ __launch_bounds__(kBlock) void sumsq_kernel(const uint16_t* __restrict__ g, Span sp,
                                                       float inv_s, double* __restrict__ partials,
                                                       int32_t* __restrict__ flag) {
    const int64_t tid = int64_t(blockIdx.x) * kBlock + threadIdx.x;
    const int64_t stride = int64_t(gridDim.x) * kBlock;
    double sq = 0.0;
    int bad = 0;
    auto add = [&](uint32_t b) {
        bad |= !finite16<DT>(b);
        const double d = double(widen<DT>(b)) * double(inv_s);
        sq += d * d;
    };
    for (int64_t i = tid; i < sp.nvec; i += stride) {
        uint32_t h[8];
        unpack8(*reinterpret_cast<const uint4*>(g + sp.head + i * 8), h);
#pragma unroll
        for (int k = 0; k < 8; ++k) add(h[k]);
    }
    const int64_t tail0 = sp.head + 8 * sp.nvec;
    const int64_t nscalar = sp.head + (sp.n - tail0);
    for (int64_t k = tid; k < nscalar; k += stride) add(g[k < sp.head ? k : tail0 + (k - sp.head)]);

    const double total = block_sum<kBlock>(sq);
    const int any_bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) {
        partials[blockIdx.x] = total;
        if (any_bad) atomicOr(flag, ZERO_FLAG_NONFINITE_GRAD);
    }
}

constexpr int kFinalizeBlock = 1024;

__global__ __launch_bounds__(kFinalizeBlock) void finalize_kernel(
    const double* __restrict__ partials, int64_t count, const double* __restrict__ extra,
    int n_extra, float max_norm, int32_t* __restrict__ flag, double* __restrict__ norm_out,
    float* __restrict__ coef_out) {
    double s = 0.0;
    for (int64_t k = threadIdx.x; k < count; k += kFinalizeBlock) s += partials[k];
    double total = block_sum<kFinalizeBlock>(s);
    if (threadIdx.x == 0) {
        for (int j = 0; j < n_extra; ++j) total += extra[j];
        const double norm = sqrt(total);
        double coef = 1.0;
        if (max_norm > 0.0f) coef = fmin(1.0, double(max_norm) / (norm + 1e-6));
        if (!isfinite(total)) *flag |= ZERO_FLAG_NONFINITE_NORM;
        *norm_out = norm;
        *coef_out = static_cast<float>(coef);
    }
}

// ---------------------------------------------------------------------------
// a3: AdamW
// ---------------------------------------------------------------------------

struct AdamConsts {
    float lr, b1, b2, omb1, omb2, eps, wd, inv_s, inv_bc1, inv_bc2;
};

// Elements [head, head + 8*nvec) use 16-byte accesses for the 16-bit arrays
// and two 16-byte accesses per fp32 array.
template <int GDT, int PDT>
__global__ __launch_bounds__(kBlock) void adam_kernel(float* __restrict__ master,
                                                      float* __restrict__ m,
                                                      float* __restrict__ v,
                                                      const uint16_t* __restrict__ grad, Span sp,
                                                      AdamConsts c,
                                                      const float* __restrict__ coef_dev,
                                                      const int32_t* __restrict__ flag,
                                                      uint16_t* __restrict__ param) {
    if (*flag != 0) return;  // a skipped step writes nothing
    const float gs = c.inv_s * *coef_dev;
    const int64_t tid = int64_t(blockIdx.x) * kBlock + threadIdx.x;
    const int64_t stride = int64_t(gridDim.x) * kBlock;

    auto update = [&](float& p, float& mm, float& vv, uint32_t gb) -> uint32_t {
        const float g = widen<GDT>(gb) * gs;
        mm = c.b1 * mm + c.omb1 * g;
        vv = c.b2 * vv + c.omb2 * (g * g);
        const float denom = sqrtf(vv * c.inv_bc2) + c.eps;
        p = p - c.lr * ((mm * c.inv_bc1) / denom + c.wd * p);
        return narrow<PDT>(p);
    };

    for (int64_t i = tid; i < sp.nvec; i += stride) {
        const int64_t e = sp.head + i * 8;
        uint32_t h[8];
        unpack8(*reinterpret_cast<const uint4*>(grad + e), h);
        float4 p0 = *reinterpret_cast<const float4*>(master + e);
        float4 p1 = *reinterpret_cast<const float4*>(master + e + 4);
        float4 m0 = *reinterpret_cast<const float4*>(m + e);
        float4 m1 = *reinterpret_cast<const float4*>(m + e + 4);
        float4 v0 = *reinterpret_cast<const float4*>(v + e);
        float4 v1 = *reinterpret_cast<const float4*>(v + e + 4);
        uint32_t o[8];
        o[0] = update(p0.x, m0.x, v0.x, h[0]);
        o[1] = update(p0.y, m0.y, v0.y, h[1]);
        o[2] = update(p0.z, m0.z, v0.z, h[2]);
        o[3] = update(p0.w, m0.w, v0.w, h[3]);
        o[4] = update(p1.x, m1.x, v1.x, h[4]);
        o[5] = update(p1.y, m1.y, v1.y, h[5]);
        o[6] = update(p1.z, m1.z, v1.z, h[6]);
        o[7] = update(p1.w, m1.w, v1.w, h[7]);
        *reinterpret_cast<float4*>(master + e) = p0;
        *reinterpret_cast<float4*>(master + e + 4) = p1;
        *reinterpret_cast<float4*>(m + e) = m0;
        *reinterpret_cast<float4*>(m + e + 4) = m1;
        *reinterpret_cast<float4*>(v + e) = v0;
        *reinterpret_cast<float4*>(v + e + 4) = v1;
        *reinterpret_cast<uint4*>(param + e) = pack8(o);
    }
    const int64_t tail0 = sp.head + 8 * sp.nvec;
    const int64_t nscalar = sp.head + (sp.n - tail0);
    for (int64_t k = tid; k < nscalar; k += stride) {
        const int64_t e = k < sp.head ? k : tail0 + (k - sp.head);
        float p = master[e], mm = m[e], vv = v[e];
        const uint32_t o = update(p, mm, vv, grad[e]);
        master[e] = p;
        m[e] = mm;
        v[e] = vv;
        param[e] = static_cast<uint16_t>(o);
    }
}

// ---------------------------------------------------------------------------
// a4: gather one unit
// ---------------------------------------------------------------------------

// Block (x, r) copies part of owner r's slice of one unit.  `vec` selects
// 16-byte copies (everything aligned) or 2-byte copies.
template <bool DEVICE_TABLE>
__global__ __launch_bounds__(kBlock) void gather_kernel(Ptrs64 tab, const uint16_t* const* dtab,
                                                        int64_t slice, int64_t shard_base,
                                                        int64_t full_base, int vec,
                                                        uint16_t* __restrict__ full) {
    const int r = blockIdx.y;
    const uint16_t* src;
    if constexpr (DEVICE_TABLE) src = dtab[r];
    else src = tab.p[r];
    src += shard_base;
    uint16_t* dst = full + full_base + int64_t(r) * slice;
    const int64_t tid = int64_t(blockIdx.x) * kBlock + threadIdx.x;
    const int64_t stride = int64_t(gridDim.x) * kBlock;
    if (vec) {
        const int64_t nv = slice / 8;
        const uint4* s4 = reinterpret_cast<const uint4*>(src);
        uint4* d4 = reinterpret_cast<uint4*>(dst);
        for (int64_t i = tid; i < nv; i += stride) d4[i] = s4[i];
    } else {
        for (int64_t i = tid; i < slice; i += stride) dst[i] = src[i];
    }
}

// ---------------------------------------------------------------------------
// Host-side helpers
// ---------------------------------------------------------------------------

bool valid_dtype(int dt) { return dt == ZERO_F16 || dt == ZERO_BF16; }

uintptr_t addr(const void* p) { return reinterpret_cast<uintptr_t>(p); }

bool overlaps(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
    if (a_bytes <= 0 || b_bytes <= 0) return false;
    const uintptr_t a0 = addr(a), b0 = addr(b);
    return a0 < b0 + uintptr_t(b_bytes) && b0 < a0 + uintptr_t(a_bytes);
}

bool pow2_positive(float x) {
    if (!(x > 0.0f) || !std::isfinite(x)) return false;
    int e;
    return std::frexp(x, &e) == 0.5f;
}

// Vector span for a set of arrays: `head` scalar elements bring every pointer
// to a 16-byte boundary; if no common head exists everything is scalar.
Span make_span(int64_t n, const void* const* ptrs16, int n16, const void* const* ptrs32, int n32) {
    Span sp{n, n, 0};
    if (n == 0) return sp;
    const void* lead = n16 > 0 ? ptrs16[0] : ptrs32[0];
    int64_t head;
    if (n16 > 0) {
        const uintptr_t mis = addr(lead) & 15;
        if (mis & 1) return sp;
        head = int64_t((16 - mis) & 15) / 2;
    } else {
        const uintptr_t mis = addr(lead) & 15;
        if (mis & 3) return sp;
        head = int64_t((16 - mis) & 15) / 4;
    }
    for (int i = 0; i < n16; ++i)
        if (((addr(ptrs16[i]) + 2 * uintptr_t(head)) & 15) != 0) return sp;
    for (int i = 0; i < n32; ++i)
        if (((addr(ptrs32[i]) + 4 * uintptr_t(head)) & 15) != 0) return sp;
    if (head >= n) return sp;
    sp.head = head;
    sp.nvec = (n - head) / 8;
    return sp;
}

unsigned grid_for(int64_t work_items, int64_t max_blocks) {
    int64_t b = (work_items + kBlock - 1) / kBlock;
    if (b < 1) b = 1;
    if (b > max_blocks) b = max_blocks;
    return unsigned(b);
}

int hip_status(hipError_t e, const char* where) {
    if (e != hipSuccess) return fail(ZERO_EHIP, std::string(where) + ": " + hipGetErrorString(e));
    return ok();
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

template <int DT>
hipError_t launch_reduce(int nd, dim3 grid, hipStream_t s, const Ptrs64& tab,
                         const uint16_t* const* dtab, Span sp, float inv_nd, float nd_f, int pow2,
                         float inv_s, uint16_t* out, double* partials, int32_t* flag) {
#define ZF_REDUCE(ND_)                                                                             \
    return launch(reduce_kernel<DT, ND_>, grid, dim3(kBlock), s, tab, dtab, nd, sp, inv_nd, nd_f, \
                  pow2, inv_s, out, partials, flag)
    switch (dtab ? -1 : nd) {
        case -1: ZF_REDUCE(-1);
        case 1: ZF_REDUCE(1);
        case 2: ZF_REDUCE(2);
        case 4: ZF_REDUCE(4);
        case 8: ZF_REDUCE(8);
        case 16: ZF_REDUCE(16);
        case 32: ZF_REDUCE(32);
        case 64: ZF_REDUCE(64);
        default: ZF_REDUCE(0);
    }
#undef ZF_REDUCE
}

template <int GDT>
hipError_t launch_adam(int pdt, dim3 grid, hipStream_t s, float* master, float* m, float* v,
                       const uint16_t* grad, Span sp, const AdamConsts& c, const float* coef,
                       const int32_t* flag, uint16_t* param) {
    if (pdt == ZERO_F16)
        return launch(adam_kernel<GDT, ZERO_F16>, grid, dim3(kBlock), s, master, m, v, grad, sp, c,
                      coef, flag, param);
    return launch(adam_kernel<GDT, ZERO_BF16>, grid, dim3(kBlock), s, master, m, v, grad, sp, c, coef,
                  flag, param);
}

constexpr int64_t kMaxAdamBlocks = 2048;
constexpr int64_t kMaxGatherBlocksX = 1024;

}  // namespace
}  // namespace zf

using namespace zf;

extern "C" {

int zero_reduce_shard(const void* const* contribs, int nd, int64_t n, int dtype, float inv_loss_scale,
                      void* reduced_out, void* workspace, int64_t workspace_bytes, int set,
                      int32_t* flag, void* stream) {
    const char* fn = "zero_reduce_shard";
    if (nd < 1 || nd > ZERO_MAX_RANKS) return fail(ZERO_EINVAL, std::string(fn) + ": nd must be in [1, 1024]");
    if (n < 0) return fail(ZERO_EINVAL, std::string(fn) + ": n < 0");
    if (!valid_dtype(dtype)) return fail(ZERO_EINVAL, std::string(fn) + ": dtype must be ZERO_F16 or ZERO_BF16");
    if (!pow2_positive(inv_loss_scale))
        return fail(ZERO_EINVAL, std::string(fn) + ": inv_loss_scale must be a positive power of two");
    if (set < 0 || set >= ZERO_MAX_RANKS) return fail(ZERO_EINVAL, std::string(fn) + ": set out of range");
    if (workspace == nullptr || (addr(workspace) & 7))
        return fail(ZERO_EINVAL, std::string(fn) + ": workspace NULL or not 8-byte aligned");
    if (workspace_bytes < zero_workspace_bytes(n, set + 1))
        return fail(ZERO_EINVAL, std::string(fn) + ": workspace too small");
    if (flag == nullptr || (addr(flag) & 3)) return fail(ZERO_EINVAL, std::string(fn) + ": flag NULL or misaligned");
    const int64_t bytes = 2 * n;
    if (n > 0) {
        if (contribs == nullptr) return fail(ZERO_EINVAL, std::string(fn) + ": contribs is NULL");
        if (reduced_out == nullptr || (addr(reduced_out) & 1))
            return fail(ZERO_EINVAL, std::string(fn) + ": reduced_out NULL or misaligned");
        for (int r = 0; r < nd; ++r) {
            if (contribs[r] == nullptr || (addr(contribs[r]) & 1))
                return fail(ZERO_EINVAL, std::string(fn) + ": contribution " + std::to_string(r) + " NULL or misaligned");
            if (overlaps(contribs[r], bytes, reduced_out, bytes))
                return fail(ZERO_EALIAS, std::string(fn) + ": reduced_out overlaps contribution " + std::to_string(r));
            if (overlaps(contribs[r], bytes, workspace, workspace_bytes))
                return fail(ZERO_EALIAS, std::string(fn) + ": workspace overlaps contribution " + std::to_string(r));
        }
        if (overlaps(reduced_out, bytes, workspace, workspace_bytes))
            return fail(ZERO_EALIAS, std::string(fn) + ": reduced_out overlaps the workspace");
        if (overlaps(reduced_out, bytes, flag, 4) || overlaps(workspace, workspace_bytes, flag, 4))
            return fail(ZERO_EALIAS, std::string(fn) + ": flag overlaps an output");
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t blocks = partial_blocks(n);
    double* partials = reinterpret_cast<double*>(static_cast<char*>(workspace) + kTableBytes) + int64_t(set) * blocks;
    Ptrs64 tab{};
    const uint16_t* const* dtab = nullptr;
    std::vector<const void*> ptrs(nd, nullptr);
    if (n > 0) {
        for (int r = 0; r < nd; ++r) ptrs[r] = contribs[r];
    }
    if (nd <= 64) {
        for (int r = 0; r < nd; ++r) tab.p[r] = static_cast<const uint16_t*>(ptrs[r]);
    } else {
        // The runtime stages a pageable source before returning, so `ptrs`
        // may go out of scope once the call is back.
        dtab = static_cast<const uint16_t* const*>(workspace);
        const hipError_t e = hipMemcpyAsync(workspace, ptrs.data(), sizeof(void*) * nd, hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return hip_status(e, fn);
    }
    std::vector<const void*> all16(ptrs);
    all16.push_back(reduced_out);
    const Span sp = n > 0 ? make_span(n, all16.data(), int(all16.size()), nullptr, 0) : Span{0, 0, 0};
    int e2;
    const bool pow2 = std::frexp(double(nd), &e2) == 0.5;
    const float inv_nd = pow2 ? 1.0f / float(nd) : 0.0f;
    const dim3 grid{unsigned(blocks)};
    const hipError_t e =
        dtype == ZERO_F16
            ? launch_reduce<ZERO_F16>(nd, grid, s, tab, dtab, sp, inv_nd, float(nd), pow2, inv_loss_scale,
                                      static_cast<uint16_t*>(reduced_out), partials, flag)
            : launch_reduce<ZERO_BF16>(nd, grid, s, tab, dtab, sp, inv_nd, float(nd), pow2, inv_loss_scale,
                                       static_cast<uint16_t*>(reduced_out), partials, flag);
    return hip_status(e, fn);
}

int zero_grad_norm(const void* grad, int64_t n, int dtype, float inv_loss_scale, void* workspace,
                   int64_t workspace_bytes, int n_sets, const double* extra_sumsq, int n_extra,
                   float max_norm, int32_t* flag, double* norm_out, float* coef_out, void* stream) {
    const char* fn = "zero_grad_norm";
    if (n < 0) return fail(ZERO_EINVAL, std::string(fn) + ": n < 0");
    if (n_sets < 1 || n_sets > ZERO_MAX_RANKS) return fail(ZERO_EINVAL, std::string(fn) + ": n_sets must be in [1, 1024]");
    if (n_extra < 0 || (n_extra > 0 && (extra_sumsq == nullptr || (addr(extra_sumsq) & 7))))
        return fail(ZERO_EINVAL, std::string(fn) + ": bad extra_sumsq");
    if (!std::isfinite(max_norm)) return fail(ZERO_EINVAL, std::string(fn) + ": max_norm must be finite");
    if (workspace == nullptr || (addr(workspace) & 7))
        return fail(ZERO_EINVAL, std::string(fn) + ": workspace NULL or not 8-byte aligned");
    if (workspace_bytes < zero_workspace_bytes(n, n_sets))
        return fail(ZERO_EINVAL, std::string(fn) + ": workspace too small");
    if (flag == nullptr || (addr(flag) & 3) || norm_out == nullptr || (addr(norm_out) & 7) ||
        coef_out == nullptr || (addr(coef_out) & 3))
        return fail(ZERO_EINVAL, std::string(fn) + ": flag, norm_out or coef_out NULL or misaligned");
    if (grad != nullptr) {
        if (!valid_dtype(dtype)) return fail(ZERO_EINVAL, std::string(fn) + ": dtype must be ZERO_F16 or ZERO_BF16");
        if (!pow2_positive(inv_loss_scale))
            return fail(ZERO_EINVAL, std::string(fn) + ": inv_loss_scale must be a positive power of two");
        if (n > 0 && (addr(grad) & 1)) return fail(ZERO_EINVAL, std::string(fn) + ": grad misaligned");
        if (overlaps(grad, 2 * n, workspace, workspace_bytes))
            return fail(ZERO_EALIAS, std::string(fn) + ": workspace overlaps grad");
    }
    if (overlaps(norm_out, 8, workspace, workspace_bytes) || overlaps(coef_out, 4, workspace, workspace_bytes) ||
        overlaps(flag, 4, workspace, workspace_bytes) || overlaps(norm_out, 8, coef_out, 4))
        return fail(ZERO_EALIAS, std::string(fn) + ": outputs overlap");

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t blocks = partial_blocks(n);
    double* partials = reinterpret_cast<double*>(static_cast<char*>(workspace) + kTableBytes);
    if (grad != nullptr && n > 0) {
        const void* p16[1] = {grad};
        const Span sp = n > 0 ? make_span(n, p16, 1, nullptr, 0) : Span{0, 0, 0};
        const uint16_t* g16 = static_cast<const uint16_t*>(grad);
        const hipError_t e =
            dtype == ZERO_F16
                ? launch(sumsq_kernel<ZERO_F16>, dim3(unsigned(blocks)), dim3(kBlock), s, g16, sp,
                         inv_loss_scale, partials, flag)
                : launch(sumsq_kernel<ZERO_BF16>, dim3(unsigned(blocks)), dim3(kBlock), s, g16, sp,
                         inv_loss_scale, partials, flag);
        if (e != hipSuccess) return hip_status(e, fn);
    }
    // With n = 0 every partial sum is zero by definition: none is read, so an
    // empty gradient needs no partials pass and no earlier launch.
    const int64_t count = n > 0 ? int64_t(n_sets) * blocks : 0;
    return hip_status(launch(finalize_kernel, dim3(1), dim3(kFinalizeBlock), s, partials, count,
                             extra_sumsq, n_extra, max_norm, flag, norm_out, coef_out),
                      fn);
}

int zero_adam_step(float* master, float* m, float* v, const void* grad, int grad_dtype, int64_t n,
                   const zero_adam_hparams* hp, const float* coef_dev, const int32_t* flag,
                   void* param_out, int param_dtype, void* stream) {
    const char* fn = "zero_adam_step";
    if (n < 0) return fail(ZERO_EINVAL, std::string(fn) + ": n < 0");
    if (!valid_dtype(grad_dtype) || !valid_dtype(param_dtype))
        return fail(ZERO_EINVAL, std::string(fn) + ": dtypes must be ZERO_F16 or ZERO_BF16");
    if (hp == nullptr) return fail(ZERO_EINVAL, std::string(fn) + ": hp is NULL");
    if (!std::isfinite(hp->lr) || !std::isfinite(hp->eps) || !std::isfinite(hp->weight_decay) ||
        !(hp->beta1 >= 0.0f && hp->beta1 < 1.0f) || !(hp->beta2 >= 0.0f && hp->beta2 < 1.0f))
        return fail(ZERO_EINVAL, std::string(fn) + ": hyperparameters must be finite, betas in [0, 1)");
    if (hp->step < 1) return fail(ZERO_EINVAL, std::string(fn) + ": step must be >= 1");
    if (!pow2_positive(hp->inv_loss_scale))
        return fail(ZERO_EINVAL, std::string(fn) + ": inv_loss_scale must be a positive power of two");
    if (coef_dev == nullptr || (addr(coef_dev) & 3) || flag == nullptr || (addr(flag) & 3))
        return fail(ZERO_EINVAL, std::string(fn) + ": coef_dev or flag NULL or misaligned");
    if (n > 0) {
        if (!master || !m || !v || !grad || !param_out)
            return fail(ZERO_EINVAL, std::string(fn) + ": NULL buffer");
        if ((addr(master) | addr(m) | addr(v)) & 3)
            return fail(ZERO_EINVAL, std::string(fn) + ": fp32 buffers must be 4-byte aligned");
        if ((addr(grad) | addr(param_out)) & 1)
            return fail(ZERO_EINVAL, std::string(fn) + ": 16-bit buffers must be 2-byte aligned");
        const void* outs[4] = {master, m, v, param_out};
        const int64_t ob[4] = {4 * n, 4 * n, 4 * n, 2 * n};
        for (int i = 0; i < 4; ++i) {
            for (int j = i + 1; j < 4; ++j)
                if (overlaps(outs[i], ob[i], outs[j], ob[j]))
                    return fail(ZERO_EALIAS, std::string(fn) + ": master, m, v and param_out must not overlap");
            if (overlaps(outs[i], ob[i], grad, 2 * n) || overlaps(outs[i], ob[i], coef_dev, 4) ||
                overlaps(outs[i], ob[i], flag, 4))
                return fail(ZERO_EALIAS, std::string(fn) + ": an output overlaps grad, coef or flag");
        }
    }
    if (n == 0) return ok();

    AdamConsts c;
    c.lr = hp->lr;
    c.b1 = hp->beta1;
    c.b2 = hp->beta2;
    c.omb1 = float(1.0 - double(hp->beta1));
    c.omb2 = float(1.0 - double(hp->beta2));
    c.eps = hp->eps;
    c.wd = hp->weight_decay;
    c.inv_s = hp->inv_loss_scale;
    const float bc1 = float(1.0 - std::pow(double(hp->beta1), double(hp->step)));
    const float bc2 = float(1.0 - std::pow(double(hp->beta2), double(hp->step)));
    if (!(bc1 > 0.0f) || !(bc2 > 0.0f)) return fail(ZERO_EINVAL, std::string(fn) + ": bias correction is zero");
    c.inv_bc1 = float(1.0 / double(bc1));
    c.inv_bc2 = float(1.0 / double(bc2));

    const void* p16[2] = {grad, param_out};
    const void* p32[3] = {master, m, v};
    const Span sp = make_span(n, p16, 2, p32, 3);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid(grid_for(sp.nvec > 0 ? sp.nvec : n, kMaxAdamBlocks));
    const uint16_t* g16 = static_cast<const uint16_t*>(grad);
    uint16_t* p16o = static_cast<uint16_t*>(param_out);
    const hipError_t e =
        grad_dtype == ZERO_F16
            ? launch_adam<ZERO_F16>(param_dtype, grid, s, master, m, v, g16, sp, c, coef_dev, flag, p16o)
            : launch_adam<ZERO_BF16>(param_dtype, grid, s, master, m, v, g16, sp, c, coef_dev, flag, p16o);
    return hip_status(e, fn);
}

int zero_gather_params(const zero_plan* plan, const void* const* shards, int unit_begin, int unit_end,
                       int dtype, void* full, void* workspace, int64_t workspace_bytes, void* stream) {
    const char* fn = "zero_gather_params";
    if (plan == nullptr) return fail(ZERO_EINVAL, std::string(fn) + ": plan is NULL");
    const int n_units = int(plan->units.size());
    if (unit_begin < 0 || unit_end < unit_begin || unit_end > n_units)
        return fail(ZERO_EINVAL, std::string(fn) + ": unit range out of bounds");
    if (!valid_dtype(dtype)) return fail(ZERO_EINVAL, std::string(fn) + ": dtype must be ZERO_F16 or ZERO_BF16");
    if (unit_begin == unit_end) return ok();
    const int owners = plan->owners;
    if (shards == nullptr || full == nullptr || (addr(full) & 1))
        return fail(ZERO_EINVAL, std::string(fn) + ": shards or full NULL, or full misaligned");
    const int64_t shard_bytes = 2 * plan->shard_numel, full_bytes = 2 * plan->full_numel;
    for (int r = 0; r < owners; ++r) {
        if (shards[r] == nullptr || (addr(shards[r]) & 1))
            return fail(ZERO_EINVAL, std::string(fn) + ": shard " + std::to_string(r) + " NULL or misaligned");
        if (overlaps(shards[r], shard_bytes, full, full_bytes))
            return fail(ZERO_EALIAS, std::string(fn) + ": shard " + std::to_string(r) + " overlaps the full buffer");
    }
    const bool device_table = owners > 64;
    if (device_table) {
        if (workspace == nullptr || (addr(workspace) & 7) || workspace_bytes < kTableBytes)
            return fail(ZERO_EINVAL, std::string(fn) + ": more than 64 owners need a workspace of zero_workspace_bytes(0, 0) bytes");
        if (overlaps(workspace, kTableBytes, full, full_bytes))
            return fail(ZERO_EALIAS, std::string(fn) + ": workspace overlaps the full buffer");
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    Ptrs64 tab{};
    const uint16_t* const* dtab = nullptr;
    bool aligned = (addr(full) & 15) == 0 && plan->align % 8 == 0;
    for (int r = 0; r < owners; ++r) aligned = aligned && (addr(shards[r]) & 15) == 0;
    if (device_table) {
        dtab = static_cast<const uint16_t* const*>(workspace);
        const hipError_t e = hipMemcpyAsync(workspace, shards, sizeof(void*) * owners, hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return hip_status(e, fn);
    } else {
        for (int r = 0; r < owners; ++r) tab.p[r] = static_cast<const uint16_t*>(shards[r]);
    }
    for (int u = unit_begin; u < unit_end; ++u) {
        const UnitInfo& ui = plan->units[u];
        if (ui.slice_numel == 0) continue;
        const int vec = aligned ? 1 : 0;
        const int64_t items = vec ? ui.slice_numel / 8 : ui.slice_numel;
        const dim3 grid(grid_for(items, kMaxGatherBlocksX), unsigned(owners));
        uint16_t* f16 = static_cast<uint16_t*>(full);
        const hipError_t e =
            device_table ? launch(gather_kernel<true>, grid, dim3(kBlock), s, tab, dtab, ui.slice_numel,
                                  ui.shard_base, ui.full_base, vec, f16)
                         : launch(gather_kernel<false>, grid, dim3(kBlock), s, tab, dtab, ui.slice_numel,
                                  ui.shard_base, ui.full_base, vec, f16);
        if (e != hipSuccess) return hip_status(e, fn);
    }
    return ok();
}

}  // extern "C"

// Block-quantised 16-bit parameters for the gather (ZeRO++ quantised
// weights), for MI355X (gfx950, wave64), and their C-ABI entry points.
//
// ZeRO++ sends the ZeRO-3 parameter all-gather in 8 or 4 bits with one scale
// per block of values (L18 notes §4.5).  Blocks are 256 elements; a 64-lane
// wave owns one block at a time (4 elements per lane, an 8-byte load), takes
// the block's absmax with a shuffle tree, and writes its codes and scale.
// The receiving side dequantises straight into the layer's place in the full
// parameter buffer, so a gathered element costs 1 (or 0.5) code byte read and
// 2 bytes written instead of 2 + 2.  All streams are HBM-bound; nothing is a
// contraction.
//
//   quantize_span_kernel   16-bit shard -> codes + fp32 scales (aligned inputs)
//   quantize_kernel        the same for any 8-byte-aligned input
//   dequantize_kernel      codes + scales -> 16-bit
//   gather_dequant_kernel  every owner's codes of one unit -> the unit's
//                          16-bit slices of the full buffer
//
// Pages cited by short name:
//   L18 notes  CMU 11-868 Lecture 18 notes, "Memory Optimization in Distributed Training: ZeRO" (semidirectx.com)

#include <cstring>
#include <string>
#include <vector>

#include "device.h"

namespace zf {
namespace {

constexpr int kQBlock = ZERO_QBLOCK;
static_assert(kQBlock == 64 * 4, "a quantisation block is one wave of quads");

template <int BITS>
constexpr float qmax_of() {
    return BITS == 8 ? 127.0f : 7.0f;
}

// Code for x given the block scale: clamp(round_half_even(x / scale)).
template <int BITS>
__device__ __forceinline__ int code_of(float x, float scale) {
    if (!(scale > 0.0f)) return 0;
    const float r = rintf(x / scale);
    return static_cast<int>(fminf(fmaxf(r, -qmax_of<BITS>()), qmax_of<BITS>()));
}

// ---------------------------------------------------------------------------
// quantise
// ---------------------------------------------------------------------------

constexpr int kQuantWaves = 4;
constexpr int kQuantThreads = 64 * kQuantWaves;
constexpr int kQuantBlocksPerWave = 4;

template <int DT, int BITS>
__global__ __launch_bounds__(kQuantThreads) void quantize_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                                 int64_t nblocks, uint8_t* __restrict__ codes,
                                                                 float* __restrict__ scales) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t first = (int64_t(blockIdx.x) * kQuantWaves + wave) * kQuantBlocksPerWave;
    float v[kQuantBlocksPerWave][4];
#pragma unroll
    for (int j = 0; j < kQuantBlocksPerWave; ++j) {
        const int64_t e0 = (first + j) * kQBlock + 4 * lane;
        if (e0 + 4 <= n) {
            const u2 w = ld_stream(reinterpret_cast<const u2*>(x + e0));
#pragma unroll
            for (int k = 0; k < 4; ++k) v[j][k] = widen<DT>(half_of(w, k));
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) v[j][k] = e0 + k < n ? widen<DT>(x[e0 + k]) : 0.0f;
        }
    }
#pragma unroll
    for (int j = 0; j < kQuantBlocksPerWave; ++j) {
        const int64_t blk = first + j;
        if (blk >= nblocks) break;  // uniform over the wave
        float amax = fmaxf(fmaxf(fabsf(v[j][0]), fabsf(v[j][1])), fmaxf(fabsf(v[j][2]), fabsf(v[j][3])));
        for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
        const float scale = amax / qmax_of<BITS>();
        int q[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) q[k] = code_of<BITS>(v[j][k], scale);
        if (lane == 0) scales[blk] = scale;
        const int64_t e0 = blk * kQBlock + 4 * lane;
        if constexpr (BITS == 8) {
            if (e0 + 4 <= n) {
                const uint32_t packed = uint32_t(q[0] & 0xff) | (uint32_t(q[1] & 0xff) << 8) |
                                        (uint32_t(q[2] & 0xff) << 16) | (uint32_t(q[3] & 0xff) << 24);
                st_stream(reinterpret_cast<uint32_t*>(codes + e0), packed);
            } else {
                for (int k = 0; k < 4; ++k)
                    if (e0 + k < n) codes[e0 + k] = static_cast<uint8_t>(q[k] & 0xff);
            }
        } else {
            if (e0 + 4 <= n) {
                const uint16_t packed = static_cast<uint16_t>((q[0] & 0xf) | ((q[1] & 0xf) << 4) |
                                                              ((q[2] & 0xf) << 8) | ((q[3] & 0xf) << 12));
                st_stream(reinterpret_cast<uint16_t*>(codes + e0 / 2), packed);
            } else {
                for (int p = 0; p < 2; ++p) {
                    const int64_t e = e0 + 2 * p;
                    if (e < n) {
                        const int hi = e + 1 < n ? (q[2 * p + 1] & 0xf) : 0;
                        codes[e / 2] = static_cast<uint8_t>((q[2 * p] & 0xf) | (hi << 4));
                    }
                }
            }
        }
    }
}

// Aligned inputs: a wave takes 1024-element spans.  Lane l loads 8 elements
// (16 bytes) at span offsets 8l and 512 + 8l, so each load instruction reads
// one contiguous KiB; lanes 0-31 / 32-63 of a load hold one 256-element block,
// whose absmax is a 32-lane shuffle reduction.  Codes go out 8 per lane per
// store (8 bytes of INT8 or 4 bytes of INT4), again contiguous per
// instruction.  x must be 16-byte aligned, INT8 codes 8-byte aligned.
constexpr int kQSpan = 1024;
constexpr int kQSpansPerWave = 2;

template <int BITS>
__device__ __forceinline__ void store_codes8(uint8_t* codes, int64_t e, const int (&q)[8]) {
    if constexpr (BITS == 8) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            lo |= uint32_t(q[k] & 0xff) << (8 * k);
            hi |= uint32_t(q[4 + k] & 0xff) << (8 * k);
        }
        st_stream(reinterpret_cast<u2*>(codes + e), u2{lo, hi});
    } else {
        uint32_t w = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) w |= uint32_t(q[k] & 0xf) << (4 * k);
        st_stream(reinterpret_cast<uint32_t*>(codes + e / 2), w);
    }
}

template <int DT, int BITS>
__global__ __launch_bounds__(kQuantThreads) void quantize_span_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                                      int64_t nblocks, uint8_t* __restrict__ codes,
                                                                      float* __restrict__ scales) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t span0 = (int64_t(blockIdx.x) * kQuantWaves + wave) * kQSpansPerWave;
    float v[kQSpansPerWave][2][8];
#pragma unroll
    for (int j = 0; j < kQSpansPerWave; ++j) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t e0 = (span0 + j) * kQSpan + 512 * h + 8 * lane;
            if (e0 + 8 <= n) {
                const u4 w = ld_stream(reinterpret_cast<const u4*>(x + e0));
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    v[j][h][2 * k] = widen<DT>(w[k] & 0xffffu);
                    v[j][h][2 * k + 1] = widen<DT>(w[k] >> 16);
                }
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k) v[j][h][k] = e0 + k < n ? widen<DT>(x[e0 + k]) : 0.0f;
            }
        }
    }
#pragma unroll
    for (int j = 0; j < kQSpansPerWave; ++j) {
        if ((span0 + j) * kQSpan >= n) break;  // uniform over the wave
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t blk = (span0 + j) * (kQSpan / kQBlock) + 2 * h + (lane >> 5);
            float amax = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[j][h][k]));
            for (int off = 16; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
            const float scale = amax / qmax_of<BITS>();
            int q[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) q[k] = code_of<BITS>(v[j][h][k], scale);
            if ((lane & 31) == 0 && blk < nblocks) scales[blk] = scale;
            const int64_t e0 = (span0 + j) * kQSpan + 512 * h + 8 * lane;
            if (e0 + 8 <= n) {
                store_codes8<BITS>(codes, e0, q);
            } else if constexpr (BITS == 8) {
                for (int k = 0; k < 8; ++k)
                    if (e0 + k < n) codes[e0 + k] = static_cast<uint8_t>(q[k] & 0xff);
            } else {
                for (int k = 0; k < 8; k += 2) {
                    const int64_t e = e0 + k;
                    if (e < n) {
                        const int hi = e + 1 < n ? (q[k + 1] & 0xf) : 0;
                        codes[e / 2] = static_cast<uint8_t>((q[k] & 0xf) | (hi << 4));
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// dequantise
// ---------------------------------------------------------------------------

constexpr int kDeqThreads = 512;
constexpr int kDeqQuadsPerLane = 2;
constexpr int64_t kDeqTileQuads = int64_t(kDeqThreads) * kDeqQuadsPerLane;

// Four codes starting at element e (a multiple of 4) as sign-extended ints.
template <int BITS>
__device__ __forceinline__ void load_codes4(const uint8_t* codes, int64_t e, int (&q)[4]) {
    if constexpr (BITS == 8) {
        const uint32_t w = ld_stream(reinterpret_cast<const uint32_t*>(codes + e));
#pragma unroll
        for (int k = 0; k < 4; ++k) q[k] = static_cast<int8_t>((w >> (8 * k)) & 0xff);
    } else {
        const uint32_t w = ld_stream(reinterpret_cast<const uint16_t*>(codes + e / 2));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int nib = (w >> (4 * k)) & 0xf;
            q[k] = nib > 7 ? nib - 16 : nib;
        }
    }
}

template <int BITS>
__device__ __forceinline__ int load_code1(const uint8_t* codes, int64_t e) {
    if constexpr (BITS == 8) {
        return static_cast<int8_t>(codes[e]);
    } else {
        const int nib = (codes[e / 2] >> (4 * (e & 1))) & 0xf;
        return nib > 7 ? nib - 16 : nib;
    }
}

template <int DT, int BITS>
__global__ __launch_bounds__(kDeqThreads) void dequantize_kernel(const uint8_t* __restrict__ codes,
                                                                 const float* __restrict__ scales, int64_t n,
                                                                 uint16_t* __restrict__ y) {
    const int64_t q0 = int64_t(blockIdx.x) * kDeqTileQuads + threadIdx.x;
#pragma unroll
    for (int u = 0; u < kDeqQuadsPerLane; ++u) {
        const int64_t e = 4 * (q0 + u * kDeqThreads);
        if (e >= n) break;
        const float scale = scales[e / kQBlock];
        if (e + 4 <= n) {
            int q[4];
            load_codes4<BITS>(codes, e, q);
            uint32_t o[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] = narrow<DT>(float(q[k]) * scale);
            st_stream(reinterpret_cast<u2*>(y + e), pack4(o));
        } else {
            for (int64_t k = e; k < n; ++k) y[k] = static_cast<uint16_t>(narrow<DT>(float(load_code1<BITS>(codes, k)) * scale));
        }
    }
}

// ---------------------------------------------------------------------------
// gather + dequantise, one unit
// ---------------------------------------------------------------------------

struct CodePtrs64 {
    const uint8_t* p[64];
};
struct ScalePtrs64 {
    const float* p[64];
};

// Eight codes (an "oct") starting at element e, a multiple of 8: 8 bytes of
// INT8 codes or 4 bytes of INT4 nibbles.  Lanes take consecutive octs, so each
// load and each 16-byte store of a wave covers one contiguous span.
template <int BITS>
struct OctCodes;
template <>
struct OctCodes<8> {
    u2 w;
    __device__ __forceinline__ void load(const uint8_t* codes, int64_t e) {
        w = ld_stream(reinterpret_cast<const u2*>(codes + e));
    }
    __device__ __forceinline__ int get(int k) const {  // sign-extended byte k
        const uint32_t word = k < 4 ? w.x : w.y;
        return static_cast<int>(word << (24 - 8 * (k & 3))) >> 24;
    }
};
template <>
struct OctCodes<4> {
    uint32_t w;
    __device__ __forceinline__ void load(const uint8_t* codes, int64_t e) {
        w = ld_stream(reinterpret_cast<const uint32_t*>(codes + e / 2));
    }
    __device__ __forceinline__ int get(int k) const {  // sign-extended nibble k
        return static_cast<int>(w << (28 - 4 * k)) >> 28;
    }
};

constexpr int kGDThreads = 256;
constexpr int kGDOctsPerLane = 4;
constexpr int64_t kGDTileOcts = int64_t(kGDThreads) * kGDOctsPerLane;

// Block (x, r) writes tile x of owner r's slice of one unit.  The slice and
// the unit's shard base are multiples of 256, so every oct is whole and lies
// in one quantisation block; the code shards and the full buffer are 16-byte
// aligned.  All loads of a lane are issued before the first store.
template <int DT, int BITS, bool DEVICE_TABLE>
__global__ __launch_bounds__(kGDThreads) void gather_dequant_kernel(
    CodePtrs64 ctab, ScalePtrs64 stab, const uint8_t* const* dctab, const float* const* dstab, int64_t slice,
    int64_t shard_base, int64_t full_base, uint16_t* __restrict__ full) {
    const int r = blockIdx.y;
    const uint8_t* codes;
    const float* scales;
    if constexpr (DEVICE_TABLE) {
        codes = dctab[r];
        scales = dstab[r];
    } else {
        codes = ctab.p[r];
        scales = stab.p[r];
    }
    uint16_t* dst = full + full_base + int64_t(r) * slice;
    const int64_t q0 = int64_t(blockIdx.x) * kGDTileOcts + threadIdx.x;
    OctCodes<BITS> c[kGDOctsPerLane];
    float sc[kGDOctsPerLane];
#pragma unroll
    for (int u = 0; u < kGDOctsPerLane; ++u) {
        const int64_t j = 8 * (q0 + u * kGDThreads);
        if (j < slice) {
            c[u].load(codes, shard_base + j);
            sc[u] = scales[(shard_base + j) / kQBlock];
        }
    }
#pragma unroll
    for (int u = 0; u < kGDOctsPerLane; ++u) {
        const int64_t j = 8 * (q0 + u * kGDThreads);
        if (j >= slice) break;
        uint32_t h[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) h[k] = narrow<DT>(float(c[u].get(k)) * sc[u]);
        st_stream(reinterpret_cast<u4*>(dst + j), u4{h[0] | (h[1] << 16), h[2] | (h[3] << 16),
                                                     h[4] | (h[5] << 16), h[6] | (h[7] << 16)});
    }
}

inline bool valid_bits(int bits) { return bits == 8 || bits == 4; }

inline int64_t code_bytes(int64_t n, int bits) { return bits == 8 ? n : (n + 1) / 2; }

template <int DT>
hipError_t launch_quantize(int bits, bool spans, hipStream_t s, const uint16_t* x, int64_t n, int64_t nb,
                           uint8_t* codes, float* scales) {
    if (spans) {
        const int64_t waves = ceil_div(ceil_div(n, int64_t(kQSpan)), int64_t(kQSpansPerWave));
        const dim3 grid{unsigned(ceil_div(waves, int64_t(kQuantWaves)))};
        if (bits == 8)
            return launch(quantize_span_kernel<DT, 8>, grid, dim3(kQuantThreads), s, x, n, nb, codes, scales);
        return launch(quantize_span_kernel<DT, 4>, grid, dim3(kQuantThreads), s, x, n, nb, codes, scales);
    }
    const dim3 grid{unsigned(ceil_div(nb, int64_t(kQuantWaves) * kQuantBlocksPerWave))};
    if (bits == 8) return launch(quantize_kernel<DT, 8>, grid, dim3(kQuantThreads), s, x, n, nb, codes, scales);
    return launch(quantize_kernel<DT, 4>, grid, dim3(kQuantThreads), s, x, n, nb, codes, scales);
}

template <int DT>
hipError_t launch_dequantize(int bits, dim3 grid, hipStream_t s, const uint8_t* codes, const float* scales,
                             int64_t n, uint16_t* y) {
    if (bits == 8) return launch(dequantize_kernel<DT, 8>, grid, dim3(kDeqThreads), s, codes, scales, n, y);
    return launch(dequantize_kernel<DT, 4>, grid, dim3(kDeqThreads), s, codes, scales, n, y);
}

template <int DT, int BITS>
hipError_t launch_gather_dequant(bool device_table, dim3 grid, hipStream_t s, const CodePtrs64& ct,
                                 const ScalePtrs64& st, const uint8_t* const* dct, const float* const* dst,
                                 int64_t slice, int64_t shard_base, int64_t full_base, uint16_t* full) {
    if (device_table)
        return launch(gather_dequant_kernel<DT, BITS, true>, grid, dim3(kGDThreads), s, ct, st, dct, dst, slice,
                      shard_base, full_base, full);
    return launch(gather_dequant_kernel<DT, BITS, false>, grid, dim3(kGDThreads), s, ct, st, dct, dst, slice,
                  shard_base, full_base, full);
}

}  // namespace
}  // namespace zf

using namespace zf;

extern "C" {

int64_t zero_quant_code_bytes(int64_t n, int bits) {
    if (n < 0 || !valid_bits(bits)) {
        fail(ZERO_EINVAL, "zero_quant_code_bytes: n < 0 or bits not 8 or 4");
        return -1;
    }
    ok();
    return code_bytes(n, bits);
}

int64_t zero_quant_scale_count(int64_t n) {
    if (n < 0) {
        fail(ZERO_EINVAL, "zero_quant_scale_count: n < 0");
        return -1;
    }
    ok();
    return ceil_div(n, kQBlock);
}

int zero_quantize_blocks(const void* x, int dtype, int64_t n, int bits, void* codes, float* scales, void* stream) {
    const char* fn = "zero_quantize_blocks";
    if (n < 0 || n > ZERO_MAX_ELEMS) return fail(ZERO_EINVAL, std::string(fn) + ": n must be in [0, 2^34]");
    if (!valid_dtype(dtype)) return fail(ZERO_EINVAL, std::string(fn) + ": dtype must be ZERO_F16 or ZERO_BF16");
    if (!valid_bits(bits)) return fail(ZERO_EINVAL, std::string(fn) + ": bits must be 8 or 4");
    if (n == 0) return ok();
    if (x == nullptr || (addr(x) & 7)) return fail(ZERO_EINVAL, std::string(fn) + ": x NULL or not 8-byte aligned");
    if (codes == nullptr || (addr(codes) & 3)) return fail(ZERO_EINVAL, std::string(fn) + ": codes NULL or not 4-byte aligned");
    if (scales == nullptr || (addr(scales) & 3)) return fail(ZERO_EINVAL, std::string(fn) + ": scales NULL or misaligned");
    const int64_t cb = code_bytes(n, bits), nb = ceil_div(n, kQBlock);
    if (overlaps(x, 2 * n, codes, cb) || overlaps(x, 2 * n, scales, 4 * nb) || overlaps(codes, cb, scales, 4 * nb))
        return fail(ZERO_EALIAS, std::string(fn) + ": x, codes and scales must not overlap");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint16_t* x16 = static_cast<const uint16_t*>(x);
    uint8_t* c8 = static_cast<uint8_t*>(codes);
    const bool spans = (addr(x) & 15) == 0 && (bits == 4 || (addr(codes) & 7) == 0);
    const hipError_t e = dtype == ZERO_F16 ? launch_quantize<ZERO_F16>(bits, spans, s, x16, n, nb, c8, scales)
                                           : launch_quantize<ZERO_BF16>(bits, spans, s, x16, n, nb, c8, scales);
    return hip_status(e, fn);
}

int zero_dequantize_blocks(const void* codes, const float* scales, int64_t n, int bits, void* y, int dtype,
                           void* stream) {
    const char* fn = "zero_dequantize_blocks";
    if (n < 0 || n > ZERO_MAX_ELEMS) return fail(ZERO_EINVAL, std::string(fn) + ": n must be in [0, 2^34]");
    if (!valid_dtype(dtype)) return fail(ZERO_EINVAL, std::string(fn) + ": dtype must be ZERO_F16 or ZERO_BF16");
    if (!valid_bits(bits)) return fail(ZERO_EINVAL, std::string(fn) + ": bits must be 8 or 4");
    if (n == 0) return ok();
    if (codes == nullptr || (addr(codes) & 3)) return fail(ZERO_EINVAL, std::string(fn) + ": codes NULL or not 4-byte aligned");
    if (scales == nullptr || (addr(scales) & 3)) return fail(ZERO_EINVAL, std::string(fn) + ": scales NULL or misaligned");
    if (y == nullptr || (addr(y) & 7)) return fail(ZERO_EINVAL, std::string(fn) + ": y NULL or not 8-byte aligned");
    const int64_t cb = code_bytes(n, bits), nb = ceil_div(n, kQBlock);
    if (overlaps(y, 2 * n, codes, cb) || overlaps(y, 2 * n, scales, 4 * nb))
        return fail(ZERO_EALIAS, std::string(fn) + ": y overlaps an input");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid{unsigned(ceil_div(ceil_div(n, 4), kDeqTileQuads))};
    const uint8_t* c8 = static_cast<const uint8_t*>(codes);
    uint16_t* y16 = static_cast<uint16_t*>(y);
    const hipError_t e = dtype == ZERO_F16 ? launch_dequantize<ZERO_F16>(bits, grid, s, c8, scales, n, y16)
                                           : launch_dequantize<ZERO_BF16>(bits, grid, s, c8, scales, n, y16);
    return hip_status(e, fn);
}

int zero_gather_dequant(const zero_plan* plan, const void* const* code_shards, const float* const* scale_shards,
                        int unit_begin, int unit_end, int bits, int dtype, void* full, void* workspace,
                        int64_t workspace_bytes, void* stream) {
    const char* fn = "zero_gather_dequant";
    if (plan == nullptr) return fail(ZERO_EINVAL, std::string(fn) + ": plan is NULL");
    const int n_units = int(plan->units.size());
    if (unit_begin < 0 || unit_end < unit_begin || unit_end > n_units)
        return fail(ZERO_EINVAL, std::string(fn) + ": unit range out of bounds");
    if (!valid_dtype(dtype)) return fail(ZERO_EINVAL, std::string(fn) + ": dtype must be ZERO_F16 or ZERO_BF16");
    if (!valid_bits(bits)) return fail(ZERO_EINVAL, std::string(fn) + ": bits must be 8 or 4");
    if (plan->align % kQBlock != 0)
        return fail(ZERO_EINVAL, std::string(fn) + ": the plan's align must be a multiple of 256");
    if (unit_begin == unit_end) return ok();
    for (int u = unit_begin; u < unit_end; ++u)
        if (plan->units[u].slice_numel > ZERO_MAX_ELEMS)
            return fail(ZERO_EINVAL, std::string(fn) + ": unit " + std::to_string(u) + "'s slice exceeds 2^34 elements");
    const int owners = plan->owners;
    if (code_shards == nullptr || scale_shards == nullptr || full == nullptr || (addr(full) & 15))
        return fail(ZERO_EINVAL, std::string(fn) + ": NULL argument or full not 16-byte aligned");
    const int64_t cb = code_bytes(plan->shard_numel, bits), sb = 4 * ceil_div(plan->shard_numel, kQBlock);
    const int64_t full_bytes = 2 * plan->full_numel;
    for (int r = 0; r < owners; ++r) {
        if (code_shards[r] == nullptr || (addr(code_shards[r]) & 15) || scale_shards[r] == nullptr ||
            (addr(scale_shards[r]) & 3))
            return fail(ZERO_EINVAL, std::string(fn) + ": shard " + std::to_string(r) + " NULL or misaligned");
        if (overlaps(code_shards[r], cb, full, full_bytes) || overlaps(scale_shards[r], sb, full, full_bytes))
            return fail(ZERO_EALIAS, std::string(fn) + ": shard " + std::to_string(r) + " overlaps the full buffer");
    }
    const bool device_table = owners > 64;
    if (device_table) {
        if (workspace == nullptr || (addr(workspace) & 7) || workspace_bytes < kPartialsOffset)
            return fail(ZERO_EINVAL, std::string(fn) + ": more than 64 owners need a workspace of zero_workspace_bytes(0, 0) bytes");
        if (overlaps(workspace, kPartialsOffset, full, full_bytes))
            return fail(ZERO_EALIAS, std::string(fn) + ": workspace overlaps the full buffer");
        for (int r = 0; r < owners; ++r)
            if (overlaps(workspace, kPartialsOffset, code_shards[r], cb) ||
                overlaps(workspace, kPartialsOffset, scale_shards[r], sb))
                return fail(ZERO_EALIAS, std::string(fn) + ": workspace overlaps shard " + std::to_string(r));
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    CodePtrs64 ct{};
    ScalePtrs64 st{};
    const uint8_t* const* dct = nullptr;
    const float* const* dst = nullptr;
    if (device_table) {
        if (int rc = refuse_capture(s, fn)) return rc;
        char* w = static_cast<char*>(workspace);
        dct = reinterpret_cast<const uint8_t* const*>(w);
        dst = reinterpret_cast<const float* const*>(w + kTableBytes);
        // Copied from the library's own pageable copies of the pointers, which the
        // runtime stages before returning: the caller may reuse its arrays at
        // once, whatever memory they are in.
        const std::vector<const void*> codes(code_shards, code_shards + owners), scales(scale_shards, scale_shards + owners);
        hipError_t e = hipMemcpyAsync(w, codes.data(), sizeof(void*) * owners, hipMemcpyHostToDevice, s);
        if (e == hipSuccess)
            e = hipMemcpyAsync(w + kTableBytes, scales.data(), sizeof(void*) * owners, hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return hip_status(e, fn);
    } else {
        for (int r = 0; r < owners; ++r) {
            ct.p[r] = static_cast<const uint8_t*>(code_shards[r]);
            st.p[r] = scale_shards[r];
        }
    }
    uint16_t* f16 = static_cast<uint16_t*>(full);
    for (int u = unit_begin; u < unit_end; ++u) {
        const UnitInfo& ui = plan->units[u];
        if (ui.slice_numel == 0) continue;
        const dim3 grid(unsigned(ceil_div(ui.slice_numel / 8, kGDTileOcts)), unsigned(owners));
        hipError_t e;
        if (dtype == ZERO_F16)
            e = bits == 8 ? launch_gather_dequant<ZERO_F16, 8>(device_table, grid, s, ct, st, dct, dst, ui.slice_numel,
                                                              ui.shard_base, ui.full_base, f16)
                          : launch_gather_dequant<ZERO_F16, 4>(device_table, grid, s, ct, st, dct, dst, ui.slice_numel,
                                                              ui.shard_base, ui.full_base, f16);
        else
            e = bits == 8 ? launch_gather_dequant<ZERO_BF16, 8>(device_table, grid, s, ct, st, dct, dst, ui.slice_numel,
                                                               ui.shard_base, ui.full_base, f16)
                          : launch_gather_dequant<ZERO_BF16, 4>(device_table, grid, s, ct, st, dct, dst, ui.slice_numel,
                                                               ui.shard_base, ui.full_base, f16);
        if (e != hipSuccess) return hip_status(e, fn);
    }
    return ok();
}

}  // extern "C"

// Device side of one ZeRO rank's share of a mixed-precision Adam step, for
// MI355X (gfx950, wave64), plus the C-ABI entry points that validate their
// arguments and launch it.
//
// Every kernel here streams HBM: nothing is a contraction, so there is no
// MFMA.  Design points, chosen by measurement on MI355X:
//   * one contiguous tile per block (no grid-stride loop): the set of active
//     addresses is one window sliding through memory, which keeps all HBM
//     channels evenly loaded (power-of-two grid strides measured 10-20% slower);
//   * 4 elements per lane per access, so each wave-wide load or store covers a
//     contiguous span (8-byte accesses for 16-bit data, 16-byte for fp32);
//   * all loads of a lane's tile issued before its stores;
//   * non-temporal loads and stores: nothing is reused, so the caches are
//     bypassed;
//   * each fp32 state array is read once and written once per step;
//   * a deterministic two-level (wave shuffle, then LDS) fp64 reduction whose
//     tree depends only on the element count.
//
//   reduce_kernel   a1: Nd contributions -> rank-order fp32 mean -> 16-bit,
//                   fused per-block fp64 sums of squares and the inf/NaN flag
//                   (L18 notes §2.2 step 3, §2.5).
//   sumsq_kernel    a2: the same sums of squares over an already-reduced
//                   gradient, one 2048-element range per wave.
//   finalize_kernel a2: fixed-order fp64 sum of the partials -> norm and the
//                   clip multiplier (L18 notes §1.4; L3.2 §4.2).
//   adam_kernel     a3: AdamW on fp32 master/m/v, cast to 16 bits (L18 notes
//                   §2.2 step 4).
//   gather_kernel   a4: 16-bit shards -> the unit's slice of the full buffer
//                   (L18 notes §2.2 step 5; Illustrated ZeRO §8.4).
//
// Pages cited by short name:
//   L18 notes         CMU 11-868 Lecture 18 notes, "Memory Optimization in Distributed Training: ZeRO" (semidirectx.com)
//   L3.2              "L3.2 显存优化与 ZeRO" (yulong.wang)
//   Illustrated ZeRO  "图解分布式训练（八）—— ZeRO 学习" (llm.jiangnianmeng.cn)

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <tuple>
#include <utility>
#include <vector>

#include "device.h"

namespace zf {
namespace {

// ---------------------------------------------------------------------------
// a1: reduce
// ---------------------------------------------------------------------------

#ifndef ZF_RANK_UNROLL_FULL
#define ZF_RANK_UNROLL_FULL 8
#endif
#ifndef ZF_RANK_UNROLL_WIDE
#define ZF_RANK_UNROLL_WIDE 4
#endif
constexpr int kRankUnrollFull = ZF_RANK_UNROLL_FULL;
constexpr int kRankUnrollWide = ZF_RANK_UNROLL_WIDE;

// Element offsets of emulated owner o's slices (blockIdx.y = o): its
// contribution from rank r starts `contrib` elements past owner 0's, its output
// `out` past, its partial sums `partials` sums past.  All zero for one owner.
struct OwnerStrides {
    int64_t contrib, out, partials;
};

// ND > 0: rank count known at compile time (<= 64), pointers in kernel args.
// ND == 0: runtime rank count <= 64, pointers in kernel args.
// ND < 0: runtime rank count > 64, pointers in a device table (workspace).
// Block (b, o) covers quads [b*kPartialQuads, (b+1)*kPartialQuads) of owner
// o's body (or elements [b*kPartialElems, ...) without `vec`) and writes
// owner o's partials[b].
template <int DT, int ND>
__global__ __launch_bounds__(kReduceBlock) void reduce_kernel(Ptrs64 tab, const uint16_t* const* dtab,
                                                        int nd, Span sp, OwnerStrides os, float inv_nd,
                                                        float nd_f, int pow2, float inv_s,
                                                        uint16_t* __restrict__ out,
                                                        double* __restrict__ partials,
                                                        int32_t* __restrict__ flag) {
#pragma clang fp contract(off)
    const int ranks = ND > 0 ? ND : nd;
    const int64_t owner = blockIdx.y;
    const int64_t coff = owner * os.contrib;
    out += owner * os.out;
    partials += owner * os.partials;
    double sq = 0.0;
    int bad = 0;

    auto src = [&](int r) -> const uint16_t* {
        if constexpr (ND >= 0) return tab.p[r] + coff;
        else return dtab[r] + coff;
    };
    auto finish = [&](float acc) -> uint32_t {
        const float mean = pow2 ? acc * inv_nd : acc / nd_f;
        const uint32_t o = narrow<DT>(mean);
        bad |= !finite16<DT>(o);
        const double d = double(widen<DT>(o)) * double(inv_s);
        sq += d * d;
        return o;
    };
    auto quad_src = [&](int r) { return reinterpret_cast<const u2*>(src(r) + sp.head); };
    u2* qout = reinterpret_cast<u2*>(out + sp.head);
    auto one_element = [&](int64_t e) {
        float acc = widen<DT>(src(0)[e]);
        for (int r = 1; r < ranks; ++r) acc = acc + widen<DT>(src(r)[e]);
        out[e] = static_cast<uint16_t>(finish(acc));
    };

    if (sp.vec) {
        const int64_t q0 = int64_t(blockIdx.x) * kPartialQuads + threadIdx.x;
        for (int t = 0; t < kPartialTiles; ++t) {
            const int64_t tq = q0 + int64_t(t) * kReduceTileQuads;
            if (tq - threadIdx.x + kReduceTileQuads <= sp.nq) {
                // Full tile: this lane's kReduceQuadsPerLane quads, loads before math.
                float acc[kReduceQuadsPerLane][4];
#pragma unroll
                for (int u = 0; u < kReduceQuadsPerLane; ++u) {
                    const u2 w = ld_stream(quad_src(0) + tq + u * kReduceBlock);
#pragma unroll
                    for (int k = 0; k < 4; ++k) acc[u][k] = widen<DT>(half_of(w, k));
                }
                if constexpr (ND > 0) {
                    // Up to kRankUnrollFull ranks unroll fully; beyond, the rank
                    // loop unrolls by kRankUnrollWide, so that many ranks' loads
                    // are in flight at a time (a full unroll of 16 or more ranks
                    // holds them all in registers and halves the waves per SIMD).
                    // The summation order is rank order either way.
                    constexpr int kRankUnroll = ND > kRankUnrollFull ? kRankUnrollWide : ND;
#pragma unroll kRankUnroll
                    for (int r = 1; r < ND; ++r) {
                        u2 w[kReduceQuadsPerLane];
#pragma unroll
                        for (int u = 0; u < kReduceQuadsPerLane; ++u) w[u] = ld_stream(quad_src(r) + tq + u * kReduceBlock);
#pragma unroll
                        for (int u = 0; u < kReduceQuadsPerLane; ++u)
#pragma unroll
                            for (int k = 0; k < 4; ++k) acc[u][k] = acc[u][k] + widen<DT>(half_of(w[u], k));
                    }
                } else {
                    for (int r = 1; r < ranks; ++r) {
                        u2 w[kReduceQuadsPerLane];
#pragma unroll
                        for (int u = 0; u < kReduceQuadsPerLane; ++u) w[u] = ld_stream(quad_src(r) + tq + u * kReduceBlock);
#pragma unroll
                        for (int u = 0; u < kReduceQuadsPerLane; ++u)
#pragma unroll
                            for (int k = 0; k < 4; ++k) acc[u][k] = acc[u][k] + widen<DT>(half_of(w[u], k));
                    }
                }
#pragma unroll
                for (int u = 0; u < kReduceQuadsPerLane; ++u) {
                    uint32_t o[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) o[k] = finish(acc[u][k]);
                    st_stream(qout + tq + u * kReduceBlock, pack4(o));
                }
            } else {
                // Last, partial tile of the body.
                for (int u = 0; u < kReduceQuadsPerLane; ++u) {
                    const int64_t q = tq + u * kReduceBlock;
                    if (q >= sp.nq) break;
                    float acc[4];
                    u2 w = quad_src(0)[q];
#pragma unroll
                    for (int k = 0; k < 4; ++k) acc[k] = widen<DT>(half_of(w, k));
                    for (int r = 1; r < ranks; ++r) {
                        w = quad_src(r)[q];
#pragma unroll
                        for (int k = 0; k < 4; ++k) acc[k] = acc[k] + widen<DT>(half_of(w, k));
                    }
                    uint32_t o[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) o[k] = finish(acc[k]);
                    qout[q] = pack4(o);
                }
                break;
            }
        }
        if (blockIdx.x == gridDim.x - 1) {
            const int64_t tail0 = sp.head + 4 * sp.nq;
            const int64_t nscalar = sp.head + (sp.n - tail0);
            for (int64_t k = threadIdx.x; k < nscalar; k += kReduceBlock)
                one_element(k < sp.head ? k : tail0 + (k - sp.head));
        }
    } else {
        const int64_t e0 = int64_t(blockIdx.x) * kPartialElems;
        const int64_t e1 = e0 + kPartialElems < sp.n ? e0 + kPartialElems : sp.n;
        for (int64_t e = e0 + threadIdx.x; e < e1; e += kReduceBlock) one_element(e);
    }

    const double total = block_sum<kReduceBlock>(sq);
    const int any_bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) {
        partials[blockIdx.x] = total;
        if (any_bad) atomicOr(flag, ZERO_FLAG_NONFINITE_GRAD);
    }
}

// ---------------------------------------------------------------------------
// a2: sums of squares of a pre-reduced gradient, and the finalize
// ---------------------------------------------------------------------------

// Each 64-lane wave owns whole partial ranges (kPartialQuads quads, i.e. one
// range of the reduce's partial sums) and sums each with a fixed shuffle tree;
// a block of kSumsqWaves waves covers kSumsqWaves * kSumsqRangesPerWave
// consecutive ranges, so a block streams enough bytes to keep HBM busy even
// though the kernel reads a single array.
constexpr int kSumsqWaves = 4;
constexpr int kSumsqBlock = 64 * kSumsqWaves;
constexpr int kSumsqRangesPerWave = 4;
constexpr int kSumsqQuadsPerLane = int(kPartialQuads / 64);

__device__ __forceinline__ double wave_sum(double v) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;  // every lane holds the total
}

template <int DT>
__global__ __launch_bounds__(kSumsqBlock) void sumsq_kernel(const uint16_t* __restrict__ g, Span sp,
                                                            float inv_s, int64_t n_ranges,
                                                            double* __restrict__ partials,
                                                            int32_t* __restrict__ flag) {
    static_assert(kPartialQuads % 64 == 0, "a range must split evenly over a wave");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int bad = 0;
    auto term = [&](uint32_t b) -> double {
        bad |= !finite16<DT>(b);
        const double d = double(widen<DT>(b)) * double(inv_s);
        return d * d;
    };
    const u2* qg = reinterpret_cast<const u2*>(g + sp.head);
    const int64_t first = (int64_t(blockIdx.x) * kSumsqWaves + wave) * kSumsqRangesPerWave;
    for (int j = 0; j < kSumsqRangesPerWave; ++j) {
        const int64_t range = first + j;
        if (range >= n_ranges) break;
        double sq = 0.0;
        if (sp.vec) {
            const int64_t q0 = range * kPartialQuads + lane;
            if (range * kPartialQuads + kPartialQuads <= sp.nq) {
                u2 w[kSumsqQuadsPerLane];
#pragma unroll
                for (int u = 0; u < kSumsqQuadsPerLane; ++u) w[u] = ld_stream(qg + q0 + u * 64);
#pragma unroll
                for (int u = 0; u < kSumsqQuadsPerLane; ++u)
#pragma unroll
                    for (int k = 0; k < 4; ++k) sq += term(half_of(w[u], k));
            } else {
                for (int u = 0; u < kSumsqQuadsPerLane; ++u) {
                    const int64_t q = q0 + u * 64;
                    if (q >= sp.nq) break;
                    const u2 w = qg[q];
#pragma unroll
                    for (int k = 0; k < 4; ++k) sq += term(half_of(w, k));
                }
            }
            if (range == n_ranges - 1) {
                const int64_t tail0 = sp.head + 4 * sp.nq;
                const int64_t nscalar = sp.head + (sp.n - tail0);
                for (int64_t k = lane; k < nscalar; k += 64) sq += term(g[k < sp.head ? k : tail0 + (k - sp.head)]);
            }
        } else {
            const int64_t e0 = range * kPartialElems;
            const int64_t e1 = e0 + kPartialElems < sp.n ? e0 + kPartialElems : sp.n;
            for (int64_t e = e0 + lane; e < e1; e += 64) sq += term(g[e]);
        }
        const double total = wave_sum(sq);
        if (lane == 0) partials[range] = total;
    }
    if (__any(bad) && lane == 0) atomicOr(flag, ZERO_FLAG_NONFINITE_GRAD);
}

constexpr int kFinalizeBlock = 1024;
constexpr int kStageBlock = 256;
// Up to this many partial sums the finalize reads them directly; above it a
// first stage folds contiguous chunks into at most kLevel2Max sums.
constexpr int64_t kSingleStageMax = 8192;
constexpr int64_t kStageChunkMin = 4096;

// Sums x[lo..hi) with thread t taking x[lo + t], x[lo + t + B], ... into
// eight accumulators (its j-th value into accumulator j mod 8, eight loads in
// flight), combined in a fixed order.  The result is the same on every run.
template <int B>
__device__ __forceinline__ double thread_sum(const double* __restrict__ x, int64_t lo, int64_t hi) {
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int64_t k = lo + threadIdx.x;
    for (; k + 7 * B < hi; k += 8 * B) {
        double v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = x[k + i * B];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    for (int i = 0; k < hi; k += B, ++i) acc[i] += x[k];
    return ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
}

// First stage: block b folds partials [b*chunk, min((b+1)*chunk, count)).
__global__ __launch_bounds__(kStageBlock) void fold_kernel(const double* __restrict__ partials,
                                                           int64_t count, int64_t chunk,
                                                           double* __restrict__ level2) {
    const int64_t lo = int64_t(blockIdx.x) * chunk;
    const int64_t hi = lo + chunk < count ? lo + chunk : count;
    const double total = block_sum<kStageBlock>(thread_sum<kStageBlock>(partials, lo, hi));
    if (threadIdx.x == 0) level2[blockIdx.x] = total;
}

// Sum of `count` values, plus extra[0..n_extra) in order -> norm, clip
// multiplier, and the non-finite flag.
__global__ __launch_bounds__(kFinalizeBlock) void finalize_kernel(
    const double* __restrict__ values, int64_t count, const double* __restrict__ extra,
    int n_extra, float max_norm, int32_t* __restrict__ flag, double* __restrict__ norm_out,
    float* __restrict__ coef_out) {
    double total = block_sum<kFinalizeBlock>(thread_sum<kFinalizeBlock>(values, 0, count));
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
    float lr, b1, b2, omb1, omb2, eps, wd, inv_s, bc1, bc2;
};

// Where an AdamW launch takes its scalars from.
enum ConstsFrom { kConstsArg = 0, kConstsDevice = 1, kConstsTable = 2 };

// Element offsets of emulated owner o's arrays (blockIdx.y = o).
struct AdamStrides {
    int64_t state, grad, param;
};

// Block (b, o) covers quads [b*kAdamTileQuads, (b+1)*kAdamTileQuads) of owner
// o's body (or elements [b*kAdamTileElems, ...) without `vec`).
// CF selects the scalars: the kernel argument c_arg; *c_src, so a captured
// graph can replay the launch with new ones; or c_src[state->step -
// state->table_t0], a table entry per step chosen by the device step counter
// (an entry outside the table skips the step and sets ZERO_FLAG_NO_CONSTS).
// The update widens the fp32 state, the 16-bit gradient and the fp32 scalars
// to fp64 and evaluates it there one operation at a time, in the order
// written, with no fused multiply-adds and with correctly rounded division
// and square root; m', v' and p' are each rounded to fp32 once.  That is the
// unsharded update's own definition, so every output is the one the plain
// data-parallel step gives (L18 notes §2.5), and the host AdamW, which
// evaluates the same sequence, gives the same bits.
template <int GDT, int PDT, int CF>
__global__ __launch_bounds__(kAdamBlock) void adam_kernel(float* __restrict__ master,
                                                      float* __restrict__ m,
                                                      float* __restrict__ v,
                                                      const uint16_t* __restrict__ grad, Span sp,
                                                      AdamStrides as, AdamConsts c_arg,
                                                      const AdamConsts* __restrict__ c_src, int64_t table_len,
                                                      const zero_step_state* __restrict__ state,
                                                      const float* __restrict__ coef_dev,
                                                      int32_t* __restrict__ flag,
                                                      uint16_t* __restrict__ param) {
#pragma clang fp contract(off)
    if (*flag != 0) return;  // a skipped step writes nothing
    AdamConsts c = c_arg;
    if constexpr (CF == kConstsDevice) {
        c = *c_src;
    } else if constexpr (CF == kConstsTable) {
        // Every block takes the same decision from the same inputs.
        const int64_t idx = state->step - state->table_t0;
        if (idx < 0 || idx >= table_len) {
            if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) atomicOr(flag, ZERO_FLAG_NO_CONSTS);
            return;
        }
        c = c_src[idx];
    }
    {
        const int64_t owner = blockIdx.y;
        master += owner * as.state;
        m += owner * as.state;
        v += owner * as.state;
        grad += owner * as.grad;
        param += owner * as.param;
    }
    // inv_s is a power of two, so this product is exact and g below is the
    // 16-bit value times inv_s times coef with a single rounding.
    const double gs = double(c.inv_s) * double(*coef_dev);
    const double b1 = c.b1, b2 = c.b2, omb1 = c.omb1, omb2 = c.omb2, lr = c.lr, eps = c.eps, wd = c.wd,
                 bc1 = c.bc1, bc2 = c.bc2;

    auto update = [&](float& p, float& mm, float& vv, uint32_t gb) -> uint32_t {
        const double g = double(widen<GDT>(gb)) * gs;
        const double m2 = b1 * double(mm) + omb1 * g;
        const double v2 = b2 * double(vv) + omb2 * (g * g);
        const double p0 = double(p);
        const double p2 = p0 - lr * ((m2 / bc1) / (sqrt(v2 / bc2) + eps) + wd * p0);
        mm = static_cast<float>(m2);
        vv = static_cast<float>(v2);
        p = static_cast<float>(p2);
        return narrow<PDT>(p);
    };
    auto update4 = [&](f4& p, f4& mm, f4& vv, const u2& g) -> u2 {
        float pp[4] = {p.x, p.y, p.z, p.w}, ma[4] = {mm.x, mm.y, mm.z, mm.w}, va[4] = {vv.x, vv.y, vv.z, vv.w};
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = update(pp[k], ma[k], va[k], half_of(g, k));
        p = f4{pp[0], pp[1], pp[2], pp[3]};
        mm = f4{ma[0], ma[1], ma[2], ma[3]};
        vv = f4{va[0], va[1], va[2], va[3]};
        return pack4(o);
    };
    auto one_element = [&](int64_t e) {
        float p = master[e], mm = m[e], vv = v[e];
        const uint32_t o = update(p, mm, vv, grad[e]);
        master[e] = p;
        m[e] = mm;
        v[e] = vv;
        param[e] = static_cast<uint16_t>(o);
    };

    if (sp.vec) {
        f4* qp = reinterpret_cast<f4*>(master + sp.head);
        f4* qm = reinterpret_cast<f4*>(m + sp.head);
        f4* qv = reinterpret_cast<f4*>(v + sp.head);
        const u2* qg = reinterpret_cast<const u2*>(grad + sp.head);
        u2* qo = reinterpret_cast<u2*>(param + sp.head);
        const int64_t tq = int64_t(blockIdx.x) * kAdamTileQuads + threadIdx.x;
        if (tq - threadIdx.x + kAdamTileQuads <= sp.nq) {
            u2 g[kAdamQuadsPerLane];
            f4 p[kAdamQuadsPerLane], mm[kAdamQuadsPerLane], vv[kAdamQuadsPerLane];
#pragma unroll
            for (int u = 0; u < kAdamQuadsPerLane; ++u) {
                const int64_t q = tq + u * kAdamBlock;
                g[u] = ld_stream(qg + q);
                p[u] = ld_stream(qp + q);
                mm[u] = ld_stream(qm + q);
                vv[u] = ld_stream(qv + q);
            }
#pragma unroll
            for (int u = 0; u < kAdamQuadsPerLane; ++u) {
                const int64_t q = tq + u * kAdamBlock;
                const u2 o = update4(p[u], mm[u], vv[u], g[u]);
                st_stream(qp + q, p[u]);
                st_stream(qm + q, mm[u]);
                st_stream(qv + q, vv[u]);
                st_stream(qo + q, o);
            }
        } else {
            for (int u = 0; u < kAdamQuadsPerLane; ++u) {
                const int64_t q = tq + u * kAdamBlock;
                if (q >= sp.nq) break;
                f4 p = qp[q], mm = qm[q], vv = qv[q];
                const u2 o = update4(p, mm, vv, qg[q]);
                qp[q] = p;
                qm[q] = mm;
                qv[q] = vv;
                qo[q] = o;
            }
        }
        if (blockIdx.x == gridDim.x - 1) {
            const int64_t tail0 = sp.head + 4 * sp.nq;
            const int64_t nscalar = sp.head + (sp.n - tail0);
            for (int64_t k = threadIdx.x; k < nscalar; k += kAdamBlock)
                one_element(k < sp.head ? k : tail0 + (k - sp.head));
        }
    } else {
        const int64_t e0 = int64_t(blockIdx.x) * kAdamTileElems;
        const int64_t e1 = e0 + kAdamTileElems < sp.n ? e0 + kAdamTileElems : sp.n;
        for (int64_t e = e0 + threadIdx.x; e < e1; e += kAdamBlock) one_element(e);
    }
}

// One thread closes a step: an applied step (flag 0) advances the device step
// counter; a skipped one is counted; the flag is recorded and cleared for the
// next step.
__global__ __launch_bounds__(64) void step_end_kernel(int32_t* __restrict__ flag,
                                                      zero_step_state* __restrict__ st) {
    if (threadIdx.x != 0) return;
    const int32_t f = *flag;
    st->last_flag = f;
    if (f == 0) {
        st->step += 1;
        st->applied += 1;
    } else {
        st->skipped += 1;
    }
    *flag = 0;
}

// ---------------------------------------------------------------------------
// a4: gather one unit
// ---------------------------------------------------------------------------

constexpr int kGatherBlock = 512;
constexpr int kGatherOctsPerLane = 2;                                     // 16-byte pieces
constexpr int64_t kGatherTileOcts = int64_t(kGatherBlock) * kGatherOctsPerLane;
constexpr int64_t kGatherTileElems = 8 * kGatherTileOcts;

// The hardware hands consecutive blocks of a launch to the eight XCDs in turn
// (block b to XCD b mod 8).  xcd_grouped(b, G) renumbers the G blocks so that
// the blocks one XCD receives take one contiguous run of tiles, the first
// G mod 8 XCDs one tile more than the rest; it is a bijection on [0, G).  For
// this two-stream copy that order measured 4.5% faster than launch order; the
// other kernels, with more streams or narrower reads, were slower with it and
// keep launch order.
__device__ __forceinline__ int64_t xcd_grouped(int64_t b, int64_t G) {
    const int64_t xcd = b & 7, local = b >> 3, per = G >> 3, extra = G & 7;
    return xcd < extra ? xcd * (per + 1) + local : extra * (per + 1) + (xcd - extra) * per + local;
}

// Logical block (x, r), after xcd_grouped over the whole grid, copies tile x of
// owner r's slice of one unit.  `vec` selects 16-byte pieces (everything
// 16-byte aligned, slice a multiple of 8) or element-by-element copies.
template <bool DEVICE_TABLE>
__global__ __launch_bounds__(kGatherBlock) void gather_kernel(Ptrs64 tab, const uint16_t* const* dtab,
                                                        int64_t slice, int64_t shard_base,
                                                        int64_t full_base, int vec,
                                                        uint16_t* __restrict__ full) {
    const int64_t gx = gridDim.x;
    const int64_t b = xcd_grouped(int64_t(blockIdx.y) * gx + blockIdx.x, gx * gridDim.y);
    const int64_t bx = b % gx;
    const int r = static_cast<int>(b / gx);
    const uint16_t* src;
    if constexpr (DEVICE_TABLE) src = dtab[r];
    else src = tab.p[r];
    src += shard_base;
    uint16_t* dst = full + full_base + int64_t(r) * slice;
    if (vec) {
        const u4* s4 = reinterpret_cast<const u4*>(src);
        u4* d4 = reinterpret_cast<u4*>(dst);
        const int64_t nv = slice / 8;
        const int64_t t0 = bx * kGatherTileOcts + threadIdx.x;
        if (t0 - threadIdx.x + kGatherTileOcts <= nv) {
            u4 x[kGatherOctsPerLane];
#pragma unroll
            for (int u = 0; u < kGatherOctsPerLane; ++u) x[u] = ld_stream(s4 + t0 + u * kGatherBlock);
#pragma unroll
            for (int u = 0; u < kGatherOctsPerLane; ++u) st_stream(d4 + t0 + u * kGatherBlock, x[u]);
        } else {
            for (int u = 0; u < kGatherOctsPerLane; ++u) {
                const int64_t i = t0 + u * kGatherBlock;
                if (i < nv) d4[i] = s4[i];
            }
        }
    } else {
        const int64_t e0 = bx * kGatherTileElems;
        const int64_t e1 = e0 + kGatherTileElems < slice ? e0 + kGatherTileElems : slice;
        for (int64_t e = e0 + threadIdx.x; e < e1; e += kGatherBlock) dst[e] = src[e];
    }
}

// ---------------------------------------------------------------------------
// Launch dispatch
// ---------------------------------------------------------------------------

template <int DT>
hipError_t launch_reduce(int nd, dim3 grid, hipStream_t s, const Ptrs64& tab,
                         const uint16_t* const* dtab, Span sp, const OwnerStrides& os, float inv_nd, float nd_f,
                         int pow2, float inv_s, uint16_t* out, double* partials, int32_t* flag) {
#define ZF_REDUCE(ND_)                                                                                  \
    return launch(reduce_kernel<DT, ND_>, grid, dim3(kReduceBlock), s, tab, dtab, nd, sp, os, inv_nd, nd_f, \
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

// The scalars of one AdamW launch: by value, from device memory, or from a
// per-step table chosen by the device step counter.
struct AdamSource {
    int from;
    AdamConsts arg;
    const AdamConsts* src;
    int64_t table_len;
    const zero_step_state* state;
};

struct AdamArgs {
    float* master;
    float* m;
    float* v;
    const uint16_t* grad;
    uint16_t* param;
    AdamStrides strides;
    const float* coef;
    int32_t* flag;
};

template <int GDT, int PDT, int CF>
hipError_t launch_adam_c(dim3 grid, hipStream_t s, Span sp, const AdamArgs& a, const AdamSource& src) {
    return launch(adam_kernel<GDT, PDT, CF>, grid, dim3(kAdamBlock), s, a.master, a.m, a.v, a.grad, sp, a.strides,
                  src.arg, src.src, src.table_len, src.state, a.coef, a.flag, a.param);
}

template <int GDT, int PDT>
hipError_t launch_adam_p(dim3 grid, hipStream_t s, Span sp, const AdamArgs& a, const AdamSource& src) {
    if (src.from == kConstsTable) return launch_adam_c<GDT, PDT, kConstsTable>(grid, s, sp, a, src);
    if (src.from == kConstsDevice) return launch_adam_c<GDT, PDT, kConstsDevice>(grid, s, sp, a, src);
    return launch_adam_c<GDT, PDT, kConstsArg>(grid, s, sp, a, src);
}

hipError_t launch_adam(int gdt, int pdt, dim3 grid, hipStream_t s, Span sp, const AdamArgs& a,
                       const AdamSource& src) {
    if (gdt == ZERO_F16)
        return pdt == ZERO_F16 ? launch_adam_p<ZERO_F16, ZERO_F16>(grid, s, sp, a, src)
                               : launch_adam_p<ZERO_F16, ZERO_BF16>(grid, s, sp, a, src);
    return pdt == ZERO_F16 ? launch_adam_p<ZERO_BF16, ZERO_F16>(grid, s, sp, a, src)
                           : launch_adam_p<ZERO_BF16, ZERO_BF16>(grid, s, sp, a, src);
}

static_assert(sizeof(zero_adam_consts) == sizeof(AdamConsts), "zero_adam_consts mirrors AdamConsts");

// The fp32 scalars of an AdamW step from its hyperparameters (validated).
int adam_consts(const char* fn, const zero_adam_hparams* hp, AdamConsts* c) {
    if (hp == nullptr) return fail(ZERO_EINVAL, std::string(fn) + ": hp is NULL");
    if (!std::isfinite(hp->lr) || !std::isfinite(hp->eps) || !std::isfinite(hp->weight_decay) ||
        !(hp->beta1 >= 0.0f && hp->beta1 < 1.0f) || !(hp->beta2 >= 0.0f && hp->beta2 < 1.0f))
        return fail(ZERO_EINVAL, std::string(fn) + ": hyperparameters must be finite, betas in [0, 1)");
    if (hp->step < 1) return fail(ZERO_EINVAL, std::string(fn) + ": step must be >= 1");
    if (!pow2_positive(hp->inv_loss_scale))
        return fail(ZERO_EINVAL, std::string(fn) + ": inv_loss_scale must be a positive power of two");
    c->lr = hp->lr;
    c->b1 = hp->beta1;
    c->b2 = hp->beta2;
    c->omb1 = float(1.0 - double(hp->beta1));
    c->omb2 = float(1.0 - double(hp->beta2));
    c->eps = hp->eps;
    c->wd = hp->weight_decay;
    c->inv_s = hp->inv_loss_scale;
    c->bc1 = float(1.0 - std::pow(double(hp->beta1), double(hp->step)));
    c->bc2 = float(1.0 - std::pow(double(hp->beta2), double(hp->step)));
    if (!(c->bc1 > 0.0f) || !(c->bc2 > 0.0f))
        return fail(ZERO_EINVAL, std::string(fn) + ": bias correction is zero");
    return ZERO_OK;
}

// Owner strides are bounded so that every extent below fits in int64.
constexpr int64_t kMaxOwnerStride = int64_t(1) << 40;

// Owner o's slices of an array sit o * stride elements past owner 0's.  With
// several owners the vector path needs every stride to keep each owner's
// alignment (a multiple of 4 elements); otherwise every element goes one by one.
inline Span owners_span(Span sp, int owners, const int64_t* strides, int n_strides) {
    if (owners > 1)
        for (int i = 0; i < n_strides; ++i)
            if (strides[i] % 4 != 0) return Span{sp.n, 0, 0, 0};
    return sp;
}

// Bytes from owner 0's first element to the last owner's last one.
inline int64_t owners_extent(int owners, int64_t stride, int64_t n, int64_t elem) {
    return elem * (int64_t(owners - 1) * stride + n);
}

// Checks the buffers of an AdamW launch over `owners` emulated owners and
// enqueues it with the scalars `src` names.
int adam_enqueue(const char* fn, float* master, float* m, float* v, int64_t state_stride, const void* grad,
                 int grad_dtype, int64_t grad_stride, int64_t n, int owners, void* param_out, int64_t param_stride,
                 int param_dtype, const AdamSource& src, const float* coef_dev, const int32_t* flag, void* stream) {
    if (n < 0 || n > ZERO_MAX_ELEMS) return fail(ZERO_EINVAL, std::string(fn) + ": n must be in [0, 2^34]");
    if (owners < 1 || owners > ZERO_MAX_RANKS) return fail(ZERO_EINVAL, std::string(fn) + ": owners must be in [1, 1024]");
    if (owners > 1 && (state_stride < n || param_stride < n || grad_stride < 0 || state_stride > kMaxOwnerStride ||
                       param_stride > kMaxOwnerStride || grad_stride > kMaxOwnerStride))
        return fail(ZERO_EINVAL, std::string(fn) + ": owner strides must be in [n, 2^40] (state, param) and "
                                                   "[0, 2^40] (grad)");
    if (!valid_dtype(grad_dtype) || !valid_dtype(param_dtype))
        return fail(ZERO_EINVAL, std::string(fn) + ": dtypes must be ZERO_F16 or ZERO_BF16");
    if (coef_dev == nullptr || (addr(coef_dev) & 3) || flag == nullptr || (addr(flag) & 3))
        return fail(ZERO_EINVAL, std::string(fn) + ": coef_dev or flag NULL or misaligned");
    const int64_t src_bytes = src.from == kConstsTable ? src.table_len * int64_t(sizeof(AdamConsts))
                                                       : src.from == kConstsDevice ? int64_t(sizeof(AdamConsts)) : 0;
    if (n > 0) {
        if (!master || !m || !v || !grad || !param_out)
            return fail(ZERO_EINVAL, std::string(fn) + ": NULL buffer");
        if ((addr(master) | addr(m) | addr(v)) & 3)
            return fail(ZERO_EINVAL, std::string(fn) + ": fp32 buffers must be 4-byte aligned");
        if ((addr(grad) | addr(param_out)) & 1)
            return fail(ZERO_EINVAL, std::string(fn) + ": 16-bit buffers must be 2-byte aligned");
        const int64_t sb = owners_extent(owners, state_stride, n, 4), pb = owners_extent(owners, param_stride, n, 2);
        const int64_t gb = owners_extent(owners, grad_stride, n, 2);
        const void* outs[4] = {master, m, v, param_out};
        const int64_t ob[4] = {sb, sb, sb, pb};
        for (int i = 0; i < 4; ++i) {
            for (int j = i + 1; j < 4; ++j)
                if (overlaps(outs[i], ob[i], outs[j], ob[j]))
                    return fail(ZERO_EALIAS, std::string(fn) + ": master, m, v and param_out must not overlap");
            if (overlaps(outs[i], ob[i], grad, gb) || overlaps(outs[i], ob[i], coef_dev, 4) ||
                overlaps(outs[i], ob[i], flag, 4) || overlaps(outs[i], ob[i], src.src, src_bytes) ||
                (src.state != nullptr && overlaps(outs[i], ob[i], src.state, int64_t(sizeof(zero_step_state)))))
                return fail(ZERO_EALIAS, std::string(fn) + ": an output overlaps grad, coef, flag or the scalars");
        }
    }
    if (n == 0) return ok();
    const void* p16[2] = {grad, param_out};
    const void* p32[3] = {master, m, v};
    const int64_t strides[3] = {state_stride, grad_stride, param_stride};
    const Span sp = owners_span(make_span(n, p16, 2, p32, 3), owners, strides, 3);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t blocks = sp.vec ? std::max<int64_t>(1, ceil_div(sp.nq, kAdamTileQuads)) : ceil_div(n, kAdamTileElems);
    const dim3 grid{unsigned(blocks), unsigned(owners)};
    const AdamArgs a{master, m, v, static_cast<const uint16_t*>(grad), static_cast<uint16_t*>(param_out),
                     AdamStrides{owners > 1 ? state_stride : 0, owners > 1 ? grad_stride : 0,
                                 owners > 1 ? param_stride : 0},
                     coef_dev, const_cast<int32_t*>(flag)};
    return hip_status(launch_adam(grad_dtype, param_dtype, grid, s, sp, a, src), fn);
}

// zero_reduce_shard / zero_reduce_owners: the checks and the launch, owners
// o = 0..owners-1 writing partial sets set + o (fn names the entry point).
int reduce_enqueue(const char* fn, const void* const* contribs, int nd, int64_t n, int owners,
                   int64_t contrib_stride, int dtype, float inv_loss_scale, void* reduced_out,
                   int64_t reduced_stride, void* workspace, int64_t workspace_bytes, int set, int32_t* flag,
                   void* stream) {
    if (nd < 1 || nd > ZERO_MAX_RANKS) return fail(ZERO_EINVAL, std::string(fn) + ": nd must be in [1, 1024]");
    if (n < 0 || n > ZERO_MAX_ELEMS) return fail(ZERO_EINVAL, std::string(fn) + ": n must be in [0, 2^34]");
    if (owners < 1 || owners > ZERO_MAX_RANKS) return fail(ZERO_EINVAL, std::string(fn) + ": owners must be in [1, 1024]");
    if (owners > 1 && (contrib_stride < 0 || reduced_stride < n || contrib_stride > kMaxOwnerStride ||
                       reduced_stride > kMaxOwnerStride))
        return fail(ZERO_EINVAL, std::string(fn) + ": owner strides must be in [0, 2^40] (contributions) and "
                                                   "[n, 2^40] (output)");
    if (!valid_dtype(dtype)) return fail(ZERO_EINVAL, std::string(fn) + ": dtype must be ZERO_F16 or ZERO_BF16");
    if (!pow2_positive(inv_loss_scale))
        return fail(ZERO_EINVAL, std::string(fn) + ": inv_loss_scale must be a positive power of two");
    if (set < 0 || set + owners > ZERO_MAX_RANKS) return fail(ZERO_EINVAL, std::string(fn) + ": set out of range");
    if (workspace == nullptr || (addr(workspace) & 7))
        return fail(ZERO_EINVAL, std::string(fn) + ": workspace NULL or not 8-byte aligned");
    if (workspace_bytes < zero_workspace_bytes(n, set + owners))
        return fail(ZERO_EINVAL, std::string(fn) + ": workspace too small");
    if (flag == nullptr || (addr(flag) & 3)) return fail(ZERO_EINVAL, std::string(fn) + ": flag NULL or misaligned");
    const int64_t bytes = owners_extent(owners, reduced_stride, n, 2);        // all owners' outputs
    const int64_t cbytes = owners_extent(owners, contrib_stride, n, 2);       // one rank's contributions
    if (n > 0) {
        if (contribs == nullptr) return fail(ZERO_EINVAL, std::string(fn) + ": contribs is NULL");
        if (reduced_out == nullptr || (addr(reduced_out) & 1))
            return fail(ZERO_EINVAL, std::string(fn) + ": reduced_out NULL or misaligned");
        // In place is allowed: reduced_out may be exactly one contribution
        // (each element is read from every rank before it is written).
        const bool same_layout = owners == 1 || reduced_stride == contrib_stride;
        for (int r = 0; r < nd; ++r) {
            if (contribs[r] == nullptr || (addr(contribs[r]) & 1))
                return fail(ZERO_EINVAL, std::string(fn) + ": contribution " + std::to_string(r) + " NULL or misaligned");
            const bool in_place = contribs[r] == reduced_out && same_layout;
            if (!in_place && overlaps(contribs[r], cbytes, reduced_out, bytes))
                return fail(ZERO_EALIAS, std::string(fn) + ": reduced_out overlaps contribution " + std::to_string(r));
            if (overlaps(contribs[r], cbytes, workspace, workspace_bytes))
                return fail(ZERO_EALIAS, std::string(fn) + ": workspace overlaps contribution " + std::to_string(r));
        }
        if (overlaps(reduced_out, bytes, workspace, workspace_bytes))
            return fail(ZERO_EALIAS, std::string(fn) + ": reduced_out overlaps the workspace");
        if (overlaps(reduced_out, bytes, flag, 4) || overlaps(workspace, workspace_bytes, flag, 4))
            return fail(ZERO_EALIAS, std::string(fn) + ": flag overlaps an output");
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t blocks = partial_blocks(n);
    double* partials = reinterpret_cast<double*>(static_cast<char*>(workspace) + kPartialsOffset) + int64_t(set) * blocks;
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
        if (int rc = refuse_capture(s, fn)) return rc;
        dtab = static_cast<const uint16_t* const*>(workspace);
        const hipError_t e = hipMemcpyAsync(workspace, ptrs.data(), sizeof(void*) * nd, hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return hip_status(e, fn);
    }
    std::vector<const void*> all16(ptrs);
    all16.push_back(reduced_out);
    const int64_t strides[2] = {contrib_stride, reduced_stride};
    const Span sp = owners_span(make_span(n, all16.data(), int(all16.size()), nullptr, 0), owners, strides, 2);
    const OwnerStrides os{owners > 1 ? contrib_stride : 0, owners > 1 ? reduced_stride : 0, owners > 1 ? blocks : 0};
    int e2;
    const bool pow2 = std::frexp(double(nd), &e2) == 0.5;
    const float inv_nd = pow2 ? 1.0f / float(nd) : 0.0f;
    const dim3 grid{unsigned(blocks), unsigned(owners)};
    const hipError_t e =
        dtype == ZERO_F16
            ? launch_reduce<ZERO_F16>(nd, grid, s, tab, dtab, sp, os, inv_nd, float(nd), pow2, inv_loss_scale,
                                      static_cast<uint16_t*>(reduced_out), partials, flag)
            : launch_reduce<ZERO_BF16>(nd, grid, s, tab, dtab, sp, os, inv_nd, float(nd), pow2, inv_loss_scale,
                                       static_cast<uint16_t*>(reduced_out), partials, flag);
    return hip_status(e, fn);
}

// zero_grad_norm's checks and launches, on a workspace the caller passes or
// on the static scratch (fn names the entry point in error messages).
int grad_norm_enqueue(const char* fn, const void* grad, int64_t n, int dtype, float inv_loss_scale,
                      void* workspace, int64_t workspace_bytes, int n_sets, const double* extra_sumsq,
                      int n_extra, float max_norm, int32_t* flag, double* norm_out, float* coef_out,
                      void* stream) {
    if (n < 0 || n > ZERO_MAX_ELEMS) return fail(ZERO_EINVAL, std::string(fn) + ": n must be in [0, 2^34]");
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
    double* partials = reinterpret_cast<double*>(static_cast<char*>(workspace) + kPartialsOffset);
    double* level2 = reinterpret_cast<double*>(static_cast<char*>(workspace) + kTableBytes);
    if (grad != nullptr && n > 0) {
        const void* p16[1] = {grad};
        const Span sp = make_span(n, p16, 1, nullptr, 0);
        const uint16_t* g16 = static_cast<const uint16_t*>(grad);
        const dim3 grid{unsigned(ceil_div(blocks, int64_t(kSumsqWaves) * kSumsqRangesPerWave))};
        const hipError_t e =
            dtype == ZERO_F16
                ? launch(sumsq_kernel<ZERO_F16>, grid, dim3(kSumsqBlock), s, g16, sp, inv_loss_scale, blocks,
                         partials, flag)
                : launch(sumsq_kernel<ZERO_BF16>, grid, dim3(kSumsqBlock), s, g16, sp, inv_loss_scale, blocks,
                         partials, flag);
        if (e != hipSuccess) return hip_status(e, fn);
    }
    // With n = 0 every partial sum is zero by definition: none is read, so an
    // empty gradient needs no partials pass and no earlier launch.
    const int64_t count = n > 0 ? int64_t(n_sets) * blocks : 0;
    const double* values = partials;
    int64_t n_values = count;
    if (count > kSingleStageMax) {
        const int64_t groups = std::min<int64_t>(kLevel2Max, ceil_div(count, kStageChunkMin));
        const int64_t chunk = ceil_div(count, groups);
        const int64_t used = ceil_div(count, chunk);
        const hipError_t e = launch(fold_kernel, dim3(unsigned(used)), dim3(kStageBlock), s, partials, count,
                                    chunk, level2);
        if (e != hipSuccess) return hip_status(e, fn);
        values = level2;
        n_values = used;
    }
    return hip_status(launch(finalize_kernel, dim3(1), dim3(kFinalizeBlock), s, values, n_values,
                             extra_sumsq, n_extra, max_norm, flag, norm_out, coef_out),
                      fn);
}

// ---------------------------------------------------------------------------
// Static scratch for the allocation-free norm (zero_grad_norm_noalloc)
// ---------------------------------------------------------------------------

// Laid out as a workspace of one set at the largest n: pointer table, second-
// level sums, then one fp64 partial sum per 2048 elements.
constexpr int64_t kNoAllocScratchBytes = kPartialsOffset + int64_t(sizeof(double)) * (ZERO_NOALLOC_MAX_ELEMS / kPartialElems);
static_assert(ZERO_NOALLOC_MAX_ELEMS % kPartialElems == 0, "the largest n fills whole partial ranges");
static_assert(ZERO_NOALLOC_SCRATCH_BYTES == kNoAllocScratchBytes, "the header states the scratch size");

}  // namespace
}  // namespace zf

// Each GPU the library runs on holds its own copy until the process ends.  In
// host code this name is a stand-in, not a device address: every use goes
// through the per-device address from hipGetSymbolAddress below.
static __device__ __align__(256) unsigned char scratch[zf::kNoAllocScratchBytes];

namespace zf {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, resolved on the first call on
// that device (with it current) and kept.
int noalloc_scratch(const char* fn, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, fn);
    if (dev < 0 || dev >= kMaxDevices) return fail(ZERO_EINVAL, std::string(fn) + ": device index beyond 63");
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, fn);
        if (ptr == nullptr || (addr(ptr) & 255))
            return fail(ZERO_EHIP, std::string(fn) + ": the scratch array has no usable device address");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return ZERO_OK;
}

}  // namespace
}  // namespace zf

using namespace zf;

extern "C" {

int zero_reduce_shard(const void* const* contribs, int nd, int64_t n, int dtype, float inv_loss_scale,
                      void* reduced_out, void* workspace, int64_t workspace_bytes, int set,
                      int32_t* flag, void* stream) {
    return reduce_enqueue("zero_reduce_shard", contribs, nd, n, 1, 0, dtype, inv_loss_scale, reduced_out, 0,
                          workspace, workspace_bytes, set, flag, stream);
}

int zero_reduce_owners(const void* const* contribs, int nd, int64_t n, int owners, int64_t contrib_stride,
                       int dtype, float inv_loss_scale, void* reduced_out, int64_t reduced_stride, void* workspace,
                       int64_t workspace_bytes, int32_t* flag, void* stream) {
    return reduce_enqueue("zero_reduce_owners", contribs, nd, n, owners, contrib_stride, dtype, inv_loss_scale,
                          reduced_out, reduced_stride, workspace, workspace_bytes, 0, flag, stream);
}

int zero_grad_norm(const void* grad, int64_t n, int dtype, float inv_loss_scale, void* workspace,
                   int64_t workspace_bytes, int n_sets, const double* extra_sumsq, int n_extra,
                   float max_norm, int32_t* flag, double* norm_out, float* coef_out, void* stream) {
    return grad_norm_enqueue("zero_grad_norm", grad, n, dtype, inv_loss_scale, workspace, workspace_bytes, n_sets,
                             extra_sumsq, n_extra, max_norm, flag, norm_out, coef_out, stream);
}

int zero_grad_norm_noalloc(const void* grad, int64_t n, int dtype, float inv_loss_scale,
                           const double* extra_sumsq, int n_extra, float max_norm, int32_t* flag,
                           double* norm_out, float* coef_out, void* stream) {
    const char* fn = "zero_grad_norm_noalloc";
    if (grad == nullptr) return fail(ZERO_EINVAL, std::string(fn) + ": grad is NULL (the partials pass is required)");
    if (n < 0 || n > ZERO_NOALLOC_MAX_ELEMS)
        return fail(ZERO_EINVAL, std::string(fn) + ": n must be in [0, ZERO_NOALLOC_MAX_ELEMS = 2^34]");
    void* ws = nullptr;
    if (int rc = noalloc_scratch(fn, &ws)) return rc;
    return grad_norm_enqueue(fn, grad, n, dtype, inv_loss_scale, ws, kNoAllocScratchBytes, 1, extra_sumsq, n_extra,
                             max_norm, flag, norm_out, coef_out, stream);
}

int zero_adam_step(float* master, float* m, float* v, const void* grad, int grad_dtype, int64_t n,
                   const zero_adam_hparams* hp, const float* coef_dev, const int32_t* flag,
                   void* param_out, int param_dtype, void* stream) {
    const char* fn = "zero_adam_step";
    AdamSource src{kConstsArg, {}, nullptr, 0, nullptr};
    if (int rc = adam_consts(fn, hp, &src.arg)) return rc;
    return adam_enqueue(fn, master, m, v, 0, grad, grad_dtype, 0, n, 1, param_out, 0, param_dtype, src, coef_dev,
                        flag, stream);
}

int zero_adam_consts_fill(const zero_adam_hparams* hp, zero_adam_consts* out) {
    const char* fn = "zero_adam_consts_fill";
    if (out == nullptr) return fail(ZERO_EINVAL, std::string(fn) + ": out is NULL");
    AdamConsts c;
    if (int rc = adam_consts(fn, hp, &c)) return rc;
    std::memcpy(out, &c, sizeof(c));
    return ok();
}

int zero_adam_step_consts(float* master, float* m, float* v, const void* grad, int grad_dtype, int64_t n,
                          const zero_adam_consts* consts_dev, const float* coef_dev, const int32_t* flag,
                          void* param_out, int param_dtype, void* stream) {
    const char* fn = "zero_adam_step_consts";
    if (consts_dev == nullptr || (addr(consts_dev) & 3))
        return fail(ZERO_EINVAL, std::string(fn) + ": consts_dev NULL or not 4-byte aligned");
    const AdamSource src{kConstsDevice, {}, reinterpret_cast<const AdamConsts*>(consts_dev), 1, nullptr};
    return adam_enqueue(fn, master, m, v, 0, grad, grad_dtype, 0, n, 1, param_out, 0, param_dtype, src, coef_dev,
                        flag, stream);
}

int zero_adam_step_owners(float* master, float* m, float* v, int64_t state_stride, const void* grad,
                          int grad_dtype, int64_t grad_stride, int64_t n, int owners,
                          const zero_adam_consts* table_dev, int64_t table_len, const zero_step_state* state_dev,
                          const float* coef_dev, int32_t* flag, void* param_out, int64_t param_stride,
                          int param_dtype, void* stream) {
    const char* fn = "zero_adam_step_owners";
    if (table_dev == nullptr || (addr(table_dev) & 3) || table_len < 1 || table_len > (int64_t(1) << 31))
        return fail(ZERO_EINVAL, std::string(fn) + ": table_dev NULL or misaligned, or table_len not in [1, 2^31]");
    if (state_dev == nullptr || (addr(state_dev) & 7))
        return fail(ZERO_EINVAL, std::string(fn) + ": state_dev NULL or not 8-byte aligned");
    const AdamSource src{kConstsTable, {}, reinterpret_cast<const AdamConsts*>(table_dev), table_len, state_dev};
    return adam_enqueue(fn, master, m, v, state_stride, grad, grad_dtype, grad_stride, n, owners, param_out,
                        param_stride, param_dtype, src, coef_dev, flag, stream);
}

int zero_step_end(int32_t* flag, zero_step_state* state_dev, void* stream) {
    const char* fn = "zero_step_end";
    if (flag == nullptr || (addr(flag) & 3)) return fail(ZERO_EINVAL, std::string(fn) + ": flag NULL or misaligned");
    if (state_dev == nullptr || (addr(state_dev) & 7))
        return fail(ZERO_EINVAL, std::string(fn) + ": state_dev NULL or not 8-byte aligned");
    if (overlaps(flag, 4, state_dev, int64_t(sizeof(zero_step_state))))
        return fail(ZERO_EALIAS, std::string(fn) + ": flag overlaps the step state");
    return hip_status(launch(step_end_kernel, dim3(1), dim3(64), static_cast<hipStream_t>(stream), flag, state_dev),
                      fn);
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
    for (int u = unit_begin; u < unit_end; ++u)
        if (plan->units[u].slice_numel > ZERO_MAX_ELEMS)
            return fail(ZERO_EINVAL, std::string(fn) + ": unit " + std::to_string(u) + "'s slice exceeds 2^34 elements");
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
        for (int r = 0; r < owners; ++r)
            if (overlaps(workspace, kTableBytes, shards[r], shard_bytes))
                return fail(ZERO_EALIAS, std::string(fn) + ": workspace overlaps shard " + std::to_string(r));
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    Ptrs64 tab{};
    const uint16_t* const* dtab = nullptr;
    bool aligned = (addr(full) & 15) == 0 && plan->align % 8 == 0;
    for (int r = 0; r < owners; ++r) aligned = aligned && (addr(shards[r]) & 15) == 0;
    if (device_table) {
        if (int rc = refuse_capture(s, fn)) return rc;
        dtab = static_cast<const uint16_t* const*>(workspace);
        // Copied from the library's own pageable copy of the pointers, which the
        // runtime stages before returning: the caller may reuse `shards` at once,
        // whatever memory it is in.
        const std::vector<const void*> ptrs(shards, shards + owners);
        const hipError_t e = hipMemcpyAsync(workspace, ptrs.data(), sizeof(void*) * owners, hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return hip_status(e, fn);
    } else {
        for (int r = 0; r < owners; ++r) tab.p[r] = static_cast<const uint16_t*>(shards[r]);
    }
    for (int u = unit_begin; u < unit_end; ++u) {
        const UnitInfo& ui = plan->units[u];
        if (ui.slice_numel == 0) continue;
        const int vec = aligned ? 1 : 0;
        const int64_t bx = vec ? ceil_div(ui.slice_numel / 8, kGatherTileOcts) : ceil_div(ui.slice_numel, kGatherTileElems);
        const dim3 grid(unsigned(std::max<int64_t>(bx, 1)), unsigned(owners));
        uint16_t* f16 = static_cast<uint16_t*>(full);
        const hipError_t e =
            device_table ? launch(gather_kernel<true>, grid, dim3(kGatherBlock), s, tab, dtab, ui.slice_numel,
                                  ui.shard_base, ui.full_base, vec, f16)
                         : launch(gather_kernel<false>, grid, dim3(kGatherBlock), s, tab, dtab, ui.slice_numel,
                                  ui.shard_base, ui.full_base, vec, f16);
        if (e != hipSuccess) return hip_status(e, fn);
    }
    return ok();
}

}  // extern "C"

// Internal declarations shared by the host partitioner (plan.cpp) and the
// device launch glue (kernels.hip).  Not part of the public ABI.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/zero_flat.h"

namespace zf {

// Sets the calling thread's error message and returns `code`.
int fail(int code, const std::string& msg);
// Clears the calling thread's error message and returns ZERO_OK.
int ok();

struct UnitInfo {
    int64_t numel;        // real elements
    int64_t slice_numel;  // per-owner slice (padded)
    int64_t full_base;    // base in the padded full buffer
    int64_t shard_base;   // base inside every shard
};

}  // namespace zf

struct zero_plan {
    int nd;
    int stage;
    int owners;
    int64_t align;
    int64_t shard_numel;
    int64_t full_numel;
    std::vector<zf::UnitInfo> units;
};

namespace zf {

// Runs that fill `rank`'s shard under `neu` from the shards of `old` (same
// parameter count), merged maximally, in new-shard order.
void reshard_runs(const zero_plan& old, const zero_plan& neu, int rank, std::vector<zero_reshard_segment>& runs);

int64_t plan_psi(const zero_plan& p);

}  // namespace zf

namespace zf {

// Tiling of the streaming kernels.  A lane handles 4 consecutive elements (a
// "quad") per access, so every load or store instruction of a wave touches
// one contiguous span; a block owns a contiguous tile of quads.  The reduce
// and sum-of-squares kernels give each block kPartialTiles consecutive tiles
// and write one fp64 partial sum per block, so the number of partial sums per
// set depends only on n.  The values are build-time settings (defaults are
// the fastest measured on MI355X).
#ifndef ZF_REDUCE_BLOCK
#define ZF_REDUCE_BLOCK 256
#endif
#ifndef ZF_REDUCE_QUADS
#define ZF_REDUCE_QUADS 2
#endif
#ifndef ZF_PARTIAL_TILES
#define ZF_PARTIAL_TILES 1
#endif
#ifndef ZF_ADAM_BLOCK
#define ZF_ADAM_BLOCK 256
#endif
#ifndef ZF_ADAM_QUADS
#define ZF_ADAM_QUADS 4
#endif
constexpr int kReduceBlock = ZF_REDUCE_BLOCK;
constexpr int kReduceQuadsPerLane = ZF_REDUCE_QUADS;
constexpr int kPartialTiles = ZF_PARTIAL_TILES;
constexpr int64_t kReduceTileQuads = int64_t(kReduceBlock) * kReduceQuadsPerLane;
constexpr int64_t kPartialQuads = kReduceTileQuads * kPartialTiles;
constexpr int64_t kPartialElems = 4 * kPartialQuads;
constexpr int kAdamBlock = ZF_ADAM_BLOCK;
constexpr int kAdamQuadsPerLane = ZF_ADAM_QUADS;
constexpr int64_t kAdamTileQuads = int64_t(kAdamBlock) * kAdamQuadsPerLane;
constexpr int64_t kAdamTileElems = 4 * kAdamTileQuads;
// Workspace layout: a device pointer table, the second-level partial sums of
// the norm, then the per-block partial sums of each set.
constexpr int64_t kTableBytes = int64_t(ZERO_MAX_RANKS) * 8;
constexpr int kLevel2Max = 1024;
constexpr int64_t kLevel2Bytes = int64_t(kLevel2Max) * 8;
constexpr int64_t kPartialsOffset = kTableBytes + kLevel2Bytes;

// Partial sums per set: max(1, ceil(n / kPartialElems)).
int64_t partial_blocks(int64_t n);

}  // namespace zf

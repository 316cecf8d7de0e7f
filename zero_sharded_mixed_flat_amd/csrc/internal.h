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

// Block size of every streaming kernel and the largest grid the partial-sum
// launches use; the number of partial sums per set depends only on n.
constexpr int kBlock = 256;
constexpr int64_t kMaxPartialBlocks = 2048;
// Device pointer table in front of the partial sums in the workspace.
constexpr int64_t kTableBytes = int64_t(ZERO_MAX_RANKS) * 8;

int64_t partial_blocks(int64_t n);

}  // namespace zf

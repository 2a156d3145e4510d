// Internal constants and helpers shared by the host planner and the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

constexpr int kHeadDim = 128;   // head dimension the kernels are built for
constexpr int kBlock = 16;      // tokens per KV block
constexpr int kGroup = 4;       // query heads per KV head (grouped-query attention)
constexpr int kDecodeWaves = 8;       // wavefronts per decode workgroup
constexpr int kMaxSplitBlocks = 64 * kDecodeWaves;   // one block id per lane of each wavefront
constexpr int kPrefillQ = 16;   // new tokens per prefill tile (x kGroup heads = 64 MFMA rows)

inline bool geometry_supported(const pa_geometry* g)
{
    return g->head_dim == kHeadDim && g->block_size == kBlock && g->num_kv_heads > 0 &&
           g->num_q_heads == g->num_kv_heads * kGroup && g->num_blocks > 0;
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace of a batch whose decode rows are split:
//   [0, 64 KiB)   uint32 completion counters, one per (row, KV head); zero before the
//                 first use of the buffer, and every call leaves them zero again
//   part_o        normalised FP32 split outputs [num_reqs][max_splits][Hq][head_dim]
//   part_lse      per-split log2-sum-exp [num_reqs][max_splits][Hq]
// The counters sit at a fixed place so that no call's partials ever land on them.
constexpr size_t kCounterBytes = 64 * 1024;
constexpr int64_t kMaxCounters = kCounterBytes / sizeof(uint32_t);

struct WorkspaceLayout {
    size_t counters = 0, part_o = 0, part_lse = 0, total = 0;
};

inline WorkspaceLayout workspace_layout(int32_t num_reqs, int32_t max_splits, int32_t num_q_heads)
{
    WorkspaceLayout w;
    if (max_splits <= 1 || num_reqs <= 0)
        return w;
    size_t n = (size_t)num_reqs * (size_t)max_splits * (size_t)num_q_heads;
    w.counters = 0;
    w.part_o = kCounterBytes;
    w.part_lse = align256(w.part_o + n * kHeadDim * sizeof(float));
    w.total = align256(w.part_lse + n * sizeof(float));
    return w;
}

}  // namespace pa

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
constexpr int kPrefillQ = 32;   // new tokens per prefill tile (x kGroup heads = 128 MFMA rows)
constexpr int kPrefillKeys = 128;     // keys per prefill step (eight blocks)
constexpr int kMaxPrefillSplits = 64; // most key splits of one prefill tile
// q8_0 pool: 32 values of a token's head row share one binary16 scale.  A (block, KV
// head) tile is [kBlock][kHeadDim] int8 codes followed by [kBlock][kHeadDim / 32] scales.
constexpr int kQ8Group = 32;
constexpr int kQ8CodeBytes = kBlock * kHeadDim;
constexpr int kQ8TileBytes = kQ8CodeBytes + kBlock * (kHeadDim / kQ8Group) * 2;
static_assert(kQ8TileBytes % 16 == 0, "q8_0 tiles stay 16-byte aligned");
static_assert(kQ8TileBytes == PA_Q8_TILE_BYTES, "header and kernels agree on the q8_0 tile");

inline bool geometry_supported(const pa_geometry* g)
{
    return g->head_dim == kHeadDim && g->block_size == kBlock && g->num_kv_heads > 0 && g->num_q_heads > 0 &&
           g->num_q_heads % g->num_kv_heads == 0 && g->num_blocks > 0;
}

// Workgroups serve kGroup query heads of one KV head.  A KV head with G = Hq / Hkv query
// heads is served in ceil(G / kGroup) slices ("virtual KV heads"); slice s holds its query
// heads kGroup s .. kGroup s + kGroup - 1, of which min(kGroup, G - kGroup s) exist (G < 4
// leaves head slots empty).  Virtual head v = s * Hkv + kvh, so that the slices of one KV
// head land on the same XCD when workgroups go round-robin to the eight XCDs.
inline int32_t num_vheads(int32_t num_q_heads, int32_t num_kv_heads)
{
    const int32_t g = num_q_heads / num_kv_heads;
    return num_kv_heads * ((g + kGroup - 1) / kGroup);
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace of a batch whose decode rows or prefill tiles are split:
//   [0, 64 KiB)   uint32 completion counters: decode (row, virtual KV head) pairs at r * V + v,
//                 prefill (tile, virtual KV head) pairs after them at num_reqs * V + tile * V + v;
//                 zero before the first use of the buffer, and every call leaves them zero
//   part_o        normalised FP32 decode split outputs [num_reqs][max_splits][V * 4][head_dim]
//                 (V virtual KV heads of 4 head slots each; V * 4 = Hq when Hq / Hkv is a multiple of 4)
//                 (also present with one split per row when there are shared-prefix groups)
//   part_lse      per-split log2-sum-exp [num_reqs][max_splits][V * 4]
//   pf_part_o     normalised FP32 prefill split outputs, 128 x 128 floats per (tile, KV head,
//                 split), in the order the prefill kernel's lanes hold them
//   pf_part_lse   their log2-sum-exp, 512 floats per (tile, KV head, split), also in lane order
//   px_part_o     normalised FP32 outputs over a row's shared-prefix blocks, per (request,
//                 prefix split, head slot): [num_reqs][prefix_splits][V * 4][head_dim]
//   px_part_lse   their log2-sum-exp [num_reqs][prefix_splits][V * 4]
// The counters sit at a fixed place so that no call's partials ever land on them.
constexpr size_t kCounterBytes = 64 * 1024;
constexpr int64_t kMaxCounters = kCounterBytes / sizeof(uint32_t);
constexpr int64_t kPrefillPartFloats = (int64_t)kPrefillQ * kGroup * kHeadDim;
// one log2-sum-exp per lane of each row group's two row blocks: 4 x 2 x 64 (each row's
// value is held by its four k-slice lanes)
constexpr int64_t kPrefillPartLseFloats = 4 * 2 * 64;

struct WorkspaceLayout {
    size_t counters = 0, part_o = 0, part_lse = 0, pf_part_o = 0, pf_part_lse = 0, px_part_o = 0, px_part_lse = 0,
           total = 0;
    int64_t pf_counter_base = 0;   // index of the first prefill counter
    int64_t counters_used = 0;     // counters the layout needs
};

inline WorkspaceLayout workspace_layout(int32_t num_reqs, int32_t max_splits, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t prefill_tiles, int32_t prefill_splits,
                                        int32_t prefix_splits = 0)
{
    WorkspaceLayout w;
    // partials are indexed by head slot (kGroup per virtual KV head), counters by virtual head
    const int32_t vheads = num_vheads(num_q_heads, num_kv_heads);
    const int32_t slots = vheads * kGroup;
    // decode partials: split rows, and every row of a shared-prefix group (its decode
    // result waits there for the group's prefix partials)
    const bool decode = (max_splits > 1 || prefix_splits > 0) && num_reqs > 0;
    const bool prefill = prefill_splits > 1 && prefill_tiles > 0;
    const bool prefix = prefix_splits > 0 && num_reqs > 0;
    if (!decode && !prefill && !prefix)
        return w;
    w.pf_counter_base = (int64_t)num_reqs * vheads;
    w.counters_used = prefill ? w.pf_counter_base + (int64_t)prefill_tiles * vheads
                              : decode ? (int64_t)num_reqs * vheads : 0;
    size_t at = kCounterBytes;
    if (decode) {
        const size_t n = (size_t)num_reqs * (size_t)max_splits * (size_t)slots;
        w.part_o = at;
        w.part_lse = align256(w.part_o + n * kHeadDim * sizeof(float));
        at = align256(w.part_lse + n * sizeof(float));
    }
    if (prefill) {
        const size_t n = (size_t)prefill_tiles * (size_t)vheads * (size_t)prefill_splits;
        w.pf_part_o = at;
        w.pf_part_lse = align256(w.pf_part_o + n * (size_t)kPrefillPartFloats * sizeof(float));
        at = align256(w.pf_part_lse + n * (size_t)kPrefillPartLseFloats * sizeof(float));
    }
    if (prefix) {
        const size_t n = (size_t)num_reqs * (size_t)prefix_splits * (size_t)slots;
        w.px_part_o = at;
        w.px_part_lse = align256(w.px_part_o + n * kHeadDim * sizeof(float));
        at = align256(w.px_part_lse + n * sizeof(float));
    }
    w.total = at;
    return w;
}

}  // namespace pa

// Host side of the library: the work planner, the content validators and the
// status strings.  No device code and no HIP calls.
#include <string.h>

#include <algorithm>
#include <unordered_set>
#include <map>
#include <vector>

#include "pa_internal.h"

namespace {

// Decode workgroups (of pa::kDecodeWaves wavefronts each) per CU the automatic split aims
// for: one workgroup fills a CU with two wavefronts per SIMD.
constexpr int kWorkgroupsPerCu = 1;
// Shortest automatic split: each split also costs a partial write and a merge read of
// Hq * (head_dim + 1) floats, so very short splits waste bandwidth.
constexpr int kMinAutoSplitBlocks = 8;
// Fixed cost of one decode workgroup (start-up latency, merge), in block-times.
constexpr int kWorkgroupOverheadBlocks = 4;
// Prefill workgroup costs in 128-key step times: start-up and output of any workgroup,
// and the partial write plus merge read that a split tile adds.
constexpr int kPrefillOverheadSteps = 2;
constexpr int kPrefillMergeSteps = 1;
// Shortest automatic prefill split, in steps.
constexpr int kMinAutoPrefillSplitSteps = 4;

int32_t ceil_div(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }

// Blocks a decode row streams: its whole table, less the leading blocks a shared-prefix
// group reads for it (skip[r], or none).
int32_t decode_blocks(const int32_t* kv_len, const int32_t* skip, int32_t r)
{
    return ceil_div(kv_len[r], pa::kBlock) - (skip ? skip[r] : 0);
}

// Decode split length and the resulting split count and work-item count.  split_blocks
// > 0 forces the length; otherwise candidate lengths divide the longest row evenly and
// each is scored by the estimated makespan in block-times: rounds of resident workgroups
// (one per CU) times the blocks one workgroup streams plus its fixed cost.  Ties go to
// the longer split, which needs fewer partials.
void choose_decode_splits(const pa_geometry* g, int32_t num_reqs, const int32_t* qo_len, const int32_t* kv_len,
                          const int32_t* skip, int32_t num_cus, int32_t split_blocks, pa_plan_t* plan)
{
    const int32_t vheads = pa::num_vheads(g->num_q_heads, g->num_kv_heads);   // workgroups per split of a row
    int32_t longest = 1;
    for (int32_t r = 0; r < num_reqs; ++r)
        if (qo_len[r] == 1)
            longest = std::max(longest, decode_blocks(kv_len, skip, r));
    int32_t sb;
    if (split_blocks > 0) {
        sb = std::min(split_blocks, pa::kMaxSplitBlocks);
    } else {
        const int64_t target = (int64_t)std::max(num_cus, 1) * kWorkgroupsPerCu;
        int64_t best_cost = INT64_MAX;
        sb = std::min(longest, pa::kMaxSplitBlocks);
        for (int32_t parts = 1; parts <= 256; ++parts) {
            const int32_t cand = ceil_div(longest, parts);
            if (cand > pa::kMaxSplitBlocks)
                continue;
            if (cand < kMinAutoSplitBlocks && parts > 1)
                break;
            int64_t wgs = 0;
            for (int32_t r = 0; r < num_reqs; ++r)
                if (qo_len[r] == 1)
                    wgs += (int64_t)ceil_div(decode_blocks(kv_len, skip, r), cand) * vheads;
            const int64_t cost = (wgs + target - 1) / target * (cand + kWorkgroupOverheadBlocks);
            if (cost < best_cost) {
                best_cost = cost;
                sb = cand;
            }
        }
    }
    plan->split_blocks = sb;
    int64_t items = 0;
    int32_t max_splits = 0;
    for (int32_t r = 0; r < num_reqs; ++r) {
        if (qo_len[r] != 1)
            continue;
        const int32_t s = ceil_div(decode_blocks(kv_len, skip, r), sb);
        max_splits = std::max(max_splits, s);
        items += (int64_t)s * vheads;
    }
    plan->max_splits = max_splits;
    plan->decode_items = (int32_t)std::min<int64_t>(items, INT32_MAX);
}

// Shared-prefix workgroups and decode workgroups run in one launch: the prefix ones first
// in the grid, then the decode ones split-major, each dispatched to the first CU that
// frees up (one workgroup per CU).  Makespan of that launch in decode block-times, from a
// greedy list-scheduling simulation over batches of identical workgroups (a map from
// free time to the number of CUs free then).  A decode workgroup costs its blocks plus a
// fixed cost, and the last split of a row also merges its partials (a cost per eight);
// a prefix workgroup costs a fixed amount, an amount per 128-key step and one per
// request of its group.
struct MakespanCosts {
    double decode_fixed, merge_per8, prefix_fixed, prefix_step, prefix_per_req;
};
// One model for both choices per pool format, each fitted to plans measured with HIP
// events over prefix splits 4 .. 24 and decode split lengths of 1 .. 6 parts of the
// longest suffix.  bf16 (and FP8) pools: 240 plans -- 4, 8, 16 and 32 requests sharing a
// 6144-token prefix with 2048-token suffixes, and the 36-layer sweep's batches 8, 16, 32
// and 64 (half the rows sharing the prefix); rms log error 0.086; the joint search over
// the candidates below picks a plan within 1.00-1.07 of each batch's best measured one
// (FP8 pools, measured on the four shared-prefix batches: within 1.00-1.14).  q8_0
// pools: 120 plans over the four shared-prefix batches, rms log error 0.12, picks within
// 1.00-1.06 (the 128-row q8_0 prefix tile makes a prefix workgroup dearer).  Costs are
// in decode block-times of the pool's format.  Prefix splits past 16 were slower on
// every batch measured and are not candidates.
constexpr MakespanCosts kCascadeCosts = {34.3, 0.0, 69.5, 7.66, 0.90};
constexpr MakespanCosts kCascadeCostsQ8 = {28.5, 0.0, 78.8, 14.6, 3.34};
constexpr int32_t kPrefixSplitCandidates[] = {4, 6, 8, 12, 16};
constexpr int32_t kMaxAutoDecodeParts = 8;

double fused_makespan(const pa_plan_t& plan, const std::vector<int32_t>& suffix_blocks, const int32_t* qo_len,
                      int32_t num_vheads, int32_t num_cus, int32_t prefix_splits, int32_t split_blocks,
                      const MakespanCosts& c)
{
    std::map<double, int64_t> free_at;     // time -> CUs that become free then
    free_at[0.0] = std::max(num_cus, 1);
    double end = 0.0;
    auto run = [&](int64_t count, double d) {
        while (count > 0) {
            auto it = free_at.begin();
            const double t = it->first;
            const int64_t n = std::min(count, it->second);
            if ((it->second -= n) == 0)
                free_at.erase(it);
            free_at[t + d] += n;
            end = std::max(end, t + d);
            count -= n;
        }
    };
    for (int32_t gi = 0; gi < plan.num_prefix_groups; ++gi) {
        const int32_t steps = ceil_div((int64_t)plan.prefix_blocks[gi] * pa::kBlock, pa::kPrefillKeys);
        for (int32_t sp = 0; sp < prefix_splits; ++sp) {
            const int32_t n = (sp + 1) * steps / prefix_splits - sp * steps / prefix_splits;
            run(num_vheads, c.prefix_fixed + c.prefix_step * n + c.prefix_per_req * plan.prefix_num_reqs[gi]);
        }
    }
    int32_t max_splits = 0;
    for (size_t r = 0; r < suffix_blocks.size(); ++r)
        if (qo_len[r] == 1)
            max_splits = std::max(max_splits, ceil_div(suffix_blocks[r], split_blocks));
    for (int32_t sp = 0; sp < max_splits; ++sp)
        for (size_t r = 0; r < suffix_blocks.size(); ++r) {
            if (qo_len[r] != 1)
                continue;
            const int32_t ns = ceil_div(suffix_blocks[r], split_blocks);
            const int32_t n = std::min(split_blocks, suffix_blocks[r] - sp * split_blocks);
            if (n <= 0)
                continue;
            const double merge = sp == ns - 1 ? c.merge_per8 * (ceil_div(ns, 8) + ceil_div(prefix_splits, 8)) : 0.0;
            run(num_vheads, c.decode_fixed + n + merge);
        }
    return end;
}

pa_status finish_workspace(const pa_geometry* g, pa_plan_t* plan)
{
    const pa::WorkspaceLayout ws =
        pa::workspace_layout(plan->num_reqs, plan->max_splits, g->num_q_heads, g->num_kv_heads, plan->prefill_tiles,
                             plan->prefill_splits, plan->num_prefix_groups > 0 ? plan->prefix_splits : 0);
    if (ws.counters_used > pa::kMaxCounters)
        return PA_ERR_UNSUPPORTED;   // more completion counters than the workspace holds
    plan->workspace_bytes = ws.total;
    return PA_OK;
}

}  // namespace

extern "C" pa_status pa_plan(const pa_geometry* g, int32_t num_reqs, const int32_t* qo_len,
                             const int32_t* kv_len, int32_t num_cus, int32_t split_blocks, int32_t prefill_splits,
                             pa_plan_t* plan)
{
    if (!g || !plan || (num_reqs > 0 && (!qo_len || !kv_len)))
        return PA_ERR_NULL;
    if (!pa::geometry_supported(g))
        return PA_ERR_UNSUPPORTED;
    if (num_reqs < 0 || prefill_splits < 0 || prefill_splits > pa::kMaxPrefillSplits)
        return PA_ERR_SHAPE;
    memset(plan, 0, sizeof(*plan));
    plan->num_q_heads = g->num_q_heads;
    plan->num_kv_heads = g->num_kv_heads;
    plan->num_reqs = num_reqs;

    int64_t total_q = 0;
    int32_t max_prefill_steps = 0, max_prefill_q = 0;
    for (int32_t r = 0; r < num_reqs; ++r) {
        if (qo_len[r] < 1 || kv_len[r] < qo_len[r])
            return PA_ERR_SHAPE;
        total_q += qo_len[r];
        if (qo_len[r] > 1)
            max_prefill_q = std::max(max_prefill_q, qo_len[r]);
    }
    // Query tile: 32 new tokens x 4 query heads = 128 MFMA rows; when every chunk row fits
    // a tile of 8 or 16 tokens, that smaller tile, whose rows keep all wavefronts (and all
    // four SIMDs of the CU) busy, where a 32-token tile would leave row groups idle.
    plan->prefill_tile_tokens = max_prefill_q <= 8 ? 8 : max_prefill_q <= 16 ? 16 : pa::kPrefillQ;
    plan->prefix_tile_rows = pa::kPrefillQ * pa::kGroup;
    for (int32_t r = 0; r < num_reqs; ++r) {
        if (qo_len[r] == 1) {
            plan->num_decode_rows++;
        } else {
            if (plan->num_prefill_rows >= PA_MAX_PREFILL_ROWS)
                return PA_ERR_UNSUPPORTED;
            int32_t i = plan->num_prefill_rows++;
            plan->prefill_req[i] = r;
            plan->prefill_tile_start[i + 1] =
                plan->prefill_tile_start[i] + ceil_div(qo_len[r], plan->prefill_tile_tokens);
            max_prefill_steps = std::max(max_prefill_steps, ceil_div(kv_len[r], pa::kPrefillKeys));
        }
    }
    if (total_q > INT32_MAX)
        return PA_ERR_SHAPE;
    plan->total_q = (int32_t)total_q;
    plan->prefill_tiles = plan->prefill_tile_start[plan->num_prefill_rows];

    // Split length: split the decode rows' KV over enough (row, KV head, split) items
    // to give every CU several wavefronts, on whole blocks.
    choose_decode_splits(g, num_reqs, qo_len, kv_len, nullptr, num_cus, split_blocks, plan);

    // Prefill key splits: a tile's causal key range is cut into contiguous step ranges,
    // one workgroup each, when the (tile, KV head) pairs alone would leave CUs idle.
    // Candidates are scored like the decode splits: rounds of resident workgroups times
    // the steps of the longest range plus the fixed and merge costs.
    int32_t ps = 1;
    if (plan->prefill_tiles > 0) {
        if (prefill_splits > 0) {
            ps = prefill_splits;
        } else {
            const int32_t vheads = pa::num_vheads(g->num_q_heads, g->num_kv_heads);
            const int64_t base = (int64_t)plan->prefill_tiles * vheads;
            const int64_t cus = std::max(num_cus, 1);
            int64_t best_cost = INT64_MAX;
            for (int32_t cand = 1; cand <= pa::kMaxPrefillSplits; ++cand) {
                const int32_t steps = ceil_div(std::max(max_prefill_steps, 1), cand);
                if (cand > 1 && steps < kMinAutoPrefillSplitSteps)
                    break;
                const int64_t rounds = (base * cand + cus - 1) / cus;
                const int64_t cost =
                    rounds * (steps + kPrefillOverheadSteps + (cand > 1 ? kPrefillMergeSteps : 0));
                if (cost < best_cost) {
                    best_cost = cost;
                    ps = cand;
                }
            }
            // fall back to unsplit tiles when the counters would not fit
            if (ps > 1 && (int64_t)num_reqs * vheads + base > pa::kMaxCounters)
                ps = 1;
        }
    }
    plan->prefill_splits = plan->prefill_tiles > 0 ? ps : 0;
    return finish_workspace(g, plan);
}

static pa_status plan_shared_prefix(bool q8, const pa_geometry* g, const int32_t* qo_len, const int32_t* kv_len,
                                    const int32_t* bt, int32_t max_blocks, int32_t num_cus, int32_t min_shared_blocks,
                                    int32_t prefix_splits, int32_t split_blocks, pa_plan_t* plan)
{
    if (!g || !plan)
        return PA_ERR_NULL;
    const int32_t R = plan->num_reqs;
    if (R > 0 && (!qo_len || !kv_len || !bt))
        return PA_ERR_NULL;
    if (!pa::geometry_supported(g) || plan->num_q_heads != g->num_q_heads || plan->num_kv_heads != g->num_kv_heads)
        return PA_ERR_UNSUPPORTED;
    if (max_blocks < 1 && R > 0)
        return PA_ERR_SHAPE;
    if (prefix_splits < 0 || prefix_splits > pa::kMaxPrefillSplits || split_blocks < 0)
        return PA_ERR_SHAPE;
    int64_t total_q = 0;
    for (int32_t r = 0; r < R; ++r) {
        if (qo_len[r] < 1 || kv_len[r] < qo_len[r] || ceil_div(kv_len[r], pa::kBlock) > max_blocks)
            return PA_ERR_SHAPE;
        total_q += qo_len[r];
    }
    if (total_q != plan->total_q)
        return PA_ERR_SHAPE;
    const int32_t min_shared = min_shared_blocks > 0 ? min_shared_blocks : 16;
    // Whole blocks of decode row r that may be shared: those before its last block.
    auto shareable = [&](int32_t r) { return (kv_len[r] - 1) / pa::kBlock; };

    // Greedy runs: from each decode row, extend over the following decode rows while
    // the common leading part of their tables stays at least min_shared blocks long.
    pa_plan_t out = *plan;
    out.num_prefix_groups = 0;
    int32_t max_prefix_blocks = 0;
    const int32_t vheads = pa::num_vheads(g->num_q_heads, g->num_kv_heads);
    for (int32_t r = 0; r < R && out.num_prefix_groups < PA_MAX_PREFIX_GROUPS;) {
        if (qo_len[r] != 1 || shareable(r) < min_shared) {
            ++r;
            continue;
        }
        int32_t common = shareable(r), end = r + 1;
        const int32_t* t0 = bt + (int64_t)r * max_blocks;
        for (int32_t r2 = r + 1; r2 < R && r2 - r < PA_MAX_PREFIX_GROUP_REQS && qo_len[r2] == 1; ++r2) {
            const int32_t* t2 = bt + (int64_t)r2 * max_blocks;
            int32_t c = 0;
            const int32_t lim = std::min(common, shareable(r2));
            while (c < lim && t2[c] == t0[c])
                ++c;
            if (c < min_shared)
                break;
            common = c;
            end = r2 + 1;
        }
        if (end - r >= 2) {
            const int32_t i = out.num_prefix_groups++;
            out.prefix_first_req[i] = r;
            out.prefix_num_reqs[i] = end - r;
            out.prefix_blocks[i] = common;
            max_prefix_blocks = std::max(max_prefix_blocks, common);
            r = end;
        } else {
            ++r;
        }
    }
    if (out.num_prefix_groups == 0)
        return PA_OK;

    // Key splits of the shared blocks and the decode split length over the private
    // suffixes, chosen together for the one launch: the pair with the smallest simulated
    // makespan under the pool format's costs.
    std::vector<int32_t> skip(R, 0), suffix(R, 0);
    for (int32_t i = 0; i < out.num_prefix_groups; ++i)
        for (int32_t k = 0; k < out.prefix_num_reqs[i]; ++k)
            skip[out.prefix_first_req[i] + k] = out.prefix_blocks[i];
    int32_t longest = 1;
    for (int32_t r = 0; r < R; ++r) {
        suffix[r] = decode_blocks(kv_len, skip.data(), r);
        if (qo_len[r] == 1)
            longest = std::max(longest, suffix[r]);
    }
    const int32_t steps = ceil_div((int64_t)max_prefix_blocks * pa::kBlock, pa::kPrefillKeys);
    // one makespan model for both choices, searched jointly (ties to fewer prefix splits,
    // then to the longer split length)
    const MakespanCosts& costs = q8 ? kCascadeCostsQ8 : kCascadeCosts;
    int32_t best_ps = 0, best_sb = 0;
    double best = 0.0;
    bool have = false;
    auto consider = [&](int32_t ps, int32_t sb) {
        const double t = fused_makespan(out, suffix, qo_len, vheads, num_cus, ps, sb, costs);
        if (!have || t < best - 1e-9) {
            have = true;
            best = t;
            best_ps = ps;
            best_sb = sb;
        }
    };
    auto over_lengths = [&](int32_t ps) {
        if (split_blocks > 0) {
            consider(ps, split_blocks);
            return;
        }
        bool any = false;
        for (int32_t parts = 1; parts <= kMaxAutoDecodeParts; ++parts) {
            const int32_t sb = ceil_div(longest, parts);
            if (sb > pa::kMaxSplitBlocks)
                continue;
            if (sb < kMinAutoSplitBlocks && parts > 1)
                break;
            consider(ps, sb);
            any = true;
        }
        if (!any)                                      // every cut longer than the largest split
            consider(ps, pa::kMaxSplitBlocks);
    };
    if (prefix_splits > 0) {
        over_lengths(prefix_splits);
    } else {
        for (const int32_t cand : kPrefixSplitCandidates)
            over_lengths(std::max(1, std::min({cand, steps, (int32_t)pa::kMaxPrefillSplits})));
    }
    out.prefix_splits = best_ps;
    // the prefix tile: 4 rows per request of the largest group; a q8_0 pool runs the full tile
    int32_t most_reqs = 0;
    for (int32_t i = 0; i < out.num_prefix_groups; ++i)
        most_reqs = std::max(most_reqs, out.prefix_num_reqs[i]);
    out.prefix_tile_rows = q8 ? 128 : most_reqs <= 8 ? 32 : most_reqs <= 16 ? 64 : 128;
    choose_decode_splits(g, R, qo_len, kv_len, skip.data(), num_cus, best_sb, &out);
    const pa_status st = finish_workspace(g, &out);
    if (st != PA_OK)
        return st;
    *plan = out;
    return PA_OK;
}

extern "C" pa_status pa_plan_shared_prefix(const pa_geometry* g, const int32_t* qo_len, const int32_t* kv_len,
                                           const int32_t* bt, int32_t max_blocks, int32_t num_cus,
                                           int32_t min_shared_blocks, int32_t prefix_splits, int32_t split_blocks,
                                           pa_plan_t* plan)
{
    return plan_shared_prefix(false, g, qo_len, kv_len, bt, max_blocks, num_cus, min_shared_blocks, prefix_splits,
                              split_blocks, plan);
}

extern "C" pa_status pa_plan_shared_prefix_q8(const pa_geometry* g, const int32_t* qo_len, const int32_t* kv_len,
                                              const int32_t* bt, int32_t max_blocks, int32_t num_cus,
                                              int32_t min_shared_blocks, int32_t prefix_splits,
                                              int32_t split_blocks, pa_plan_t* plan)
{
    return plan_shared_prefix(true, g, qo_len, kv_len, bt, max_blocks, num_cus, min_shared_blocks, prefix_splits,
                              split_blocks, plan);
}

extern "C" pa_status pa_validate_batch(const pa_geometry* g, int32_t num_reqs, const int32_t* qo_len,
                                       const int32_t* kv_len, const int32_t* block_tables,
                                       int32_t max_blocks_per_req, int32_t* bad_index)
{
    if (bad_index)
        *bad_index = -1;
    if (!g || (num_reqs > 0 && (!qo_len || !kv_len || !block_tables)))
        return PA_ERR_NULL;
    if (num_reqs < 0 || max_blocks_per_req < 0 || g->block_size <= 0)
        return PA_ERR_SHAPE;
    for (int32_t r = 0; r < num_reqs; ++r) {
        if (qo_len[r] < 1 || kv_len[r] < qo_len[r] || ceil_div(kv_len[r], g->block_size) > max_blocks_per_req) {
            if (bad_index)
                *bad_index = r;
            return PA_ERR_SHAPE;
        }
        int32_t nb = ceil_div(kv_len[r], g->block_size);
        const int32_t* row = block_tables + (size_t)r * max_blocks_per_req;
        for (int32_t b = 0; b < nb; ++b) {
            if (row[b] < 0 || row[b] >= g->num_blocks) {
                if (bad_index)
                    *bad_index = r;
                return PA_ERR_RANGE;
            }
        }
    }
    return PA_OK;
}

extern "C" pa_status pa_validate_copy(const pa_geometry* g, const int32_t* src, const int32_t* dst, int32_t n,
                                      int32_t* bad_index)
{
    if (bad_index)
        *bad_index = -1;
    if (!g || (n > 0 && (!src || !dst)))
        return PA_ERR_NULL;
    if (n < 0)
        return PA_ERR_SHAPE;
    std::unordered_set<int32_t> dsts, srcs;
    for (int32_t i = 0; i < n; ++i)
        srcs.insert(src[i]);
    for (int32_t i = 0; i < n; ++i) {
        const bool bad = src[i] < 0 || src[i] >= g->num_blocks || dst[i] < 0 || dst[i] >= g->num_blocks ||
                         !dsts.insert(dst[i]).second || srcs.count(dst[i]);
        if (bad) {
            if (bad_index)
                *bad_index = i;
            return PA_ERR_RANGE;
        }
    }
    return PA_OK;
}

extern "C" pa_status pa_validate_append(const pa_geometry* g, const int32_t* slot_mapping, int32_t n_tokens,
                                        int32_t* bad_index)
{
    if (bad_index)
        *bad_index = -1;
    if (!g || (n_tokens > 0 && !slot_mapping))
        return PA_ERR_NULL;
    if (n_tokens < 0)
        return PA_ERR_SHAPE;
    const int64_t num_slots = (int64_t)g->num_blocks * g->block_size;
    std::unordered_set<int32_t> seen;
    seen.reserve((size_t)n_tokens * 2);
    for (int32_t t = 0; t < n_tokens; ++t) {
        int32_t s = slot_mapping[t];
        if (s < 0)
            continue;
        if (s >= num_slots || !seen.insert(s).second) {
            if (bad_index)
                *bad_index = t;
            return PA_ERR_RANGE;
        }
    }
    return PA_OK;
}

extern "C" const char* pa_status_string(pa_status s)
{
    switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "inconsistent lengths (need 1 <= qo_len <= kv_len and enough table entries)";
    case PA_ERR_RANGE: return "block id or slot outside the pool, or a repeated slot";
    case PA_ERR_WORKSPACE: return "workspace smaller than the plan needs";
    case PA_ERR_UNSUPPORTED: return "unsupported geometry (need head_dim 128, block_size 16, query heads a multiple of KV heads)";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_NO_BLOCKS: return "not enough free blocks";
    }
    return "unknown status";
}

extern "C" size_t pa_plan_struct_bytes(void) { return sizeof(pa_plan_t); }

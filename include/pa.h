/*
 * pa.h -- paged-KV attention for a continuous batch that mixes decode rows
 * (qo_len = 1) with chunked-prefill rows (qo_len = chunk, causal), on AMD
 * Instinct MI355X (gfx950).  Plain C ABI: host or device pointers and sizes,
 * no framework types.
 *
 * Vocabulary, from the pages this library implements:
 *   - KV is stored in fixed-size blocks of `block_size` tokens; each request has
 *     a block table mapping logical block -> physical block, and a physical
 *     block may sit anywhere in the pool (AI-infra book ch. 8 "Inference
 *     optimisation", section 8.3.1 and fig. 8-10; serving tutorial, section
 *     "PagedAttention: KV cache in pages", which also gives 16-token blocks).
 *   - Several block tables may point at the same physical blocks (a shared
 *     prefix is stored once: book section 8.3.1 fig. 8-13 and section 8.3.2).
 *   - qo_len is a row's number of new (query) tokens and kv_len the number of
 *     KV entries it attends over; decode rows have qo_len = 1 (Perplexity blog
 *     on disaggregated prefill and decode, section on prefill vs decode).
 *   - A chunk of c new tokens at context h attends causally: the i-th new
 *     token (0-based) sees keys 0 .. h + i (book section 8.2.3, N_pair sum).
 *   - Inside a block the pool is laid out head-major ("HND"): one KV head's
 *     block_size x head_dim rows are contiguous (Perplexity blog, paragraph on
 *     NHD vs HND page layout).
 *
 * Layouts (bf16 = 16-bit brain float, stored as its bit pattern):
 *   k_pool, v_pool  bf16 [num_blocks][num_kv_heads][block_size][head_dim]
 *   q, out          bf16 [total_q][num_q_heads][head_dim]; the rows of request r
 *                   are qo_indptr[r] .. qo_indptr[r+1]-1, in token order
 *   lse             float [total_q][num_q_heads], natural log of the softmax
 *                   denominator sum_j exp(scale * q.k_j)
 *   block_tables    int32 [num_reqs][max_blocks_per_req]; entries past
 *                   ceil(kv_len / block_size) are never read
 *   k_new, v_new    bf16 [n_tokens][num_kv_heads][head_dim]
 *   slot_mapping    int32 [n_tokens]: block_id * block_size + offset, < 0 = skip
 *
 * Semantics (per request r, new token i, query head h):
 *   kvh = h / (num_q_heads / num_kv_heads)   (grouped-query attention, contiguous groups)
 *   p   = kv_len[r] - qo_len[r] + i           (position of the token; keys 0..p visible)
 *   out = sum_j softmax_j(scale * q.k_j) v_j  over j = 0..p, with k_j, v_j read at
 *         pool[block_tables[r][j / block_size]][kvh][j % block_size]
 * kv_len counts the tokens after this step's append, so a row sees its own new
 * token: call pa_append_kv before pa_attention_batch on the same stream.
 *
 * Work is cut per "virtual KV head": a workgroup serves four query heads of one KV
 * head, so a KV head with G = num_q_heads / num_kv_heads query heads takes
 * ceil(G / 4) virtual heads (G < 4 leaves head slots idle).  Counts of
 * (row, KV head) or (tile, KV head) pairs below are over virtual KV heads.
 *
 * Ownership and ordering: the caller allocates and owns every buffer (device
 * memory for everything the kernels touch, host memory for plans and the
 * validators' inputs).  The library allocates no device memory and keeps no
 * global state.  Every device call is asynchronous on `stream` (a hipStream_t;
 * NULL means the null stream).  A block may be freed or rewritten only after the
 * stream work that reads it has completed (book section 8.3.2: release needs the
 * last reference gone *and* the device done with the block); an append must
 * never target a block that another request's table still reads (copy-on-write
 * is the caller's job, book section 8.3.2 fig. 8-15).
 *
 * Errors: every entry point returns a pa_status and never aborts.  Cheap checks
 * (null pointers, supported geometry, plan / workspace consistency) run before
 * any launch.  Content checks that need a scan of host copies (block ids in
 * range, 1 <= qo_len <= kv_len, slots in range and not repeated) are in
 * pa_validate_batch / pa_validate_append.  The kernels bound-check what they read
 * and write: a block id outside the pool or a row whose lengths disagree with the
 * plan is not read and that row's output is set to NaN; an out-of-range slot is
 * not written.  A failed launch maps to PA_ERR_HIP.  With PA_VALIDATE=1 in the
 * environment, pa_append_kv(_q8) and pa_attention_batch(_q8) also copy their index
 * arrays to the host in stream order (waiting for the stream; PA_ERR_UNSUPPORTED under
 * graph capture) and run the validators' checks first, returning their status with
 * nothing launched.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_NULL = -1,        /* a required pointer is NULL                        */
    PA_ERR_SHAPE = -2,       /* lengths inconsistent (qo_len < 1, kv_len < qo_len, ...) */
    PA_ERR_RANGE = -3,       /* a block id or slot outside the pool, a repeated slot */
    PA_ERR_WORKSPACE = -4,   /* workspace too small for the plan                   */
    PA_ERR_UNSUPPORTED = -5, /* geometry the kernels are not built for             */
    PA_ERR_HIP = -6,         /* a HIP runtime call or kernel launch failed         */
    PA_ERR_NO_BLOCKS = -7    /* the block allocator has too few free blocks         */
} pa_status;

/* One layer's attention geometry and pool size. */
typedef struct pa_geometry {
    int32_t num_q_heads;   /* query heads (32 for Qwen3-8B)                                   */
    int32_t num_kv_heads;  /* KV heads (8 for Qwen3-8B); must divide num_q_heads               */
    int32_t head_dim;      /* must be 128                                                      */
    int32_t block_size;    /* tokens per block; must be 16                                     */
    int32_t num_blocks;    /* physical blocks in each of the K and V pools                     */
    float scale;           /* score scale, normally 1 / sqrt(head_dim)                         */
} pa_geometry;

/* Most rows with qo_len > 1 that one plan can hold. */
#define PA_MAX_PREFILL_ROWS 128
/* Most shared-prefix (cascade) groups one plan can hold, and most requests per group. */
#define PA_MAX_PREFIX_GROUPS 16
#define PA_MAX_PREFIX_GROUP_REQS 32

/*
 * The host-side work plan for one batch.  A pure function of the host copies of
 * qo_len / kv_len, the geometry and the CU count; it can be reused for every
 * layer of a step (all layers share the lengths).  Plain data: copy it freely.
 */
typedef struct pa_plan_t {
    int32_t num_q_heads, num_kv_heads;   /* geometry the plan was made for                    */
    int32_t num_reqs;                    /* rows of the batch                                 */
    int32_t total_q;                     /* sum of qo_len                                     */
    int32_t num_decode_rows;             /* rows with qo_len == 1                             */
    int32_t num_prefill_rows;            /* rows with qo_len > 1                              */
    int32_t split_blocks;                /* KV blocks per decode split (one workgroup each)   */
    int32_t max_splits;                  /* largest split count of any decode row             */
    int32_t decode_items;                /* (row, virtual KV head, split) decode workgroups   */
    int32_t prefill_tiles;               /* query tiles over all prefill rows                 */
    int32_t prefill_splits;              /* key splits per prefill tile (one workgroup each)  */
    int32_t prefill_req[PA_MAX_PREFILL_ROWS];       /* request index of each prefill row      */
    int32_t prefill_tile_start[PA_MAX_PREFILL_ROWS + 1]; /* prefix sums of tiles per row      */
    int32_t num_prefix_groups;           /* shared-prefix groups (pa_plan_shared_prefix)      */
    int32_t prefix_splits;               /* key splits of each group's shared blocks          */
    int32_t prefix_first_req[PA_MAX_PREFIX_GROUPS]; /* first request of each group            */
    int32_t prefix_num_reqs[PA_MAX_PREFIX_GROUPS];  /* consecutive decode requests in it      */
    int32_t prefix_blocks[PA_MAX_PREFIX_GROUPS];    /* leading blocks all of them share       */
    int32_t prefill_tile_tokens;         /* new tokens per query tile: 32, or 16 / 8 when every
                                            row with qo_len > 1 fits one such tile (the tile's
                                            MFMA rows are then all busy, spread over all four
                                            SIMDs of a CU); a q8_0 pool always runs 32      */
    int32_t prefix_tile_rows;            /* MFMA rows of a shared-prefix group's tile: 128, or
                                            64 / 32 when every group has at most 16 / 8 rows */
    int32_t one_launch;                  /* a batch with chunk tiles and decode rows (and no
                                            shared-prefix group, bf16 pool): 0 launches the
                                            chunk tiles, then the decode rows; 1 runs both in
                                            one launch, chunk tiles first in the grid; 2 the
                                            same with the two kinds interleaved.  Results are
                                            bit-identical.  pa_plan sets 0 (measured fastest
                                            on a one-GPU MI355X); the caller may override   */
    uint64_t workspace_bytes;            /* device workspace pa_attention_batch needs         */
} pa_plan_t;

/*
 * Build the plan.  qo_len_host / kv_len_host: host int32 [num_reqs].  num_cus: the
 * device's compute-unit count (256 on MI355X; see pa_query_num_cus).
 * split_blocks: 0 picks the decode split length automatically: a decode row is
 * split over kv_len only when its (row, KV head) pairs alone would leave CUs idle
 * (the pages motivate splitting attention over kv_len as well as over requests when
 * a batch has few tokens: Perplexity blog, section on prefill vs decode); > 0 forces
 * that many blocks per split (clamped to 1 .. 512).
 * prefill_splits: 0 picks how many contiguous key ranges each 32-token prefill tile
 * is cut into (one workgroup per range, merged by the last one to finish) so that
 * the tiles fill the CUs; > 0 forces that count (1 .. 64; ranges may then be empty).
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE (qo_len < 1, kv_len < qo_len, prefill_splits
 * out of range), PA_ERR_UNSUPPORTED (geometry, more than PA_MAX_PREFILL_ROWS prefill
 * rows, or split work needing more than 16384 completion counters: one per
 * (request, KV head) plus one per (prefill tile, KV head)).
 */
pa_status pa_plan(const pa_geometry* geometry, int32_t num_reqs, const int32_t* qo_len_host,
                  const int32_t* kv_len_host, int32_t num_cus, int32_t split_blocks, int32_t prefill_splits,
                  pa_plan_t* plan);

/*
 * Add shared-prefix (cascade) groups to a plan built by pa_plan from the same lengths.
 * A group is a run of at least two consecutive decode rows (qo_len == 1) whose block
 * tables start with the same physical blocks: the pages keep one physical copy of a
 * common prefix, referenced from every request's table (book section 8.3.2, shared
 * blocks with reference counts; Hugging Face continuous-batching page, prefix caching).
 * pa_attention_batch then reads each group's shared blocks once per KV head, for all
 * of the group's query rows together, in the same launch as the decode rows, and
 * merges that partial result with each row's private suffix by the log-sum-exp rule.
 * The prefix key splits and the decode split length are chosen together for that
 * launch.  Groups never overlap (pa_attention_batch returns PA_ERR_SHAPE for a plan
 * whose groups share a row).  Only whole blocks that precede every row's
 * last block are shared, and a run needs at least min_shared_blocks of them (0 picks
 * 16).  block_tables_host: host int32 [num_reqs][max_blocks_per_req], the tables the
 * batch will use (a device table that differs gives wrong results).  Runs longer than
 * PA_MAX_PREFIX_GROUP_REQS are cut; at most PA_MAX_PREFIX_GROUPS groups are kept.
 * Recomputes the decode splits over the private suffixes and the workspace size; a
 * plan with no group found is left as it was.  prefix_splits: 0 lets the planner
 * choose how many key ranges each group's shared blocks are cut into (one workgroup
 * per range and KV head); > 0 forces that count (1 .. 64).  split_blocks: 0 lets the
 * planner choose the decode split length over the private suffixes; > 0 forces it
 * (clamped to 1 .. 512).  Errors: PA_ERR_NULL, PA_ERR_SHAPE (lengths differ from
 * the plan's, prefix_splits or split_blocks out of range), PA_ERR_UNSUPPORTED
 * (completion counters, as for pa_plan).
 */
pa_status pa_plan_shared_prefix(const pa_geometry* geometry, const int32_t* qo_len_host, const int32_t* kv_len_host,
                                const int32_t* block_tables_host, int32_t max_blocks_per_req, int32_t num_cus,
                                int32_t min_shared_blocks, int32_t prefix_splits, int32_t split_blocks,
                                pa_plan_t* plan);

/*
 * pa_plan_shared_prefix for a batch that runs on a q8_0 pool (pa_attention_batch_q8):
 * the same groups, arguments, overrides and errors; the automatic choice of prefix splits
 * and split length uses the q8_0 kernels' costs (prefix steps dearer, decode blocks
 * cheaper than on bf16), which favours more, shorter prefix splits.
 */
pa_status pa_plan_shared_prefix_q8(const pa_geometry* geometry, const int32_t* qo_len_host,
                                   const int32_t* kv_len_host, const int32_t* block_tables_host,
                                   int32_t max_blocks_per_req, int32_t num_cus, int32_t min_shared_blocks,
                                   int32_t prefix_splits, int32_t split_blocks, pa_plan_t* plan);

/*
 * Write this step's new K/V rows into the pools through the slot mapping
 * (book section 8.3.1: a token's KV goes to a slot of the block its table
 * names; Perplexity blog: the per-layer append happens before attention).
 * Device pointers: k_pool, v_pool (written in place), k_new, v_new, slot_mapping.
 * Slots < 0 are skipped; slots >= num_blocks * block_size are not written.
 * Repeated slots are invalid (pa_validate_append reports them); which write wins
 * is then unspecified.  Errors: PA_ERR_NULL, PA_ERR_UNSUPPORTED, PA_ERR_SHAPE
 * (n_tokens < 0), PA_ERR_HIP.
 */
pa_status pa_append_kv(const pa_geometry* geometry, void* k_pool, void* v_pool, const void* k_new,
                       const void* v_new, const int32_t* slot_mapping, int32_t n_tokens, void* stream);

/*
 * Attention for the whole mixed batch (decode rows and chunked-prefill rows).
 * plan: host pointer to a plan built from the same lengths.  Device pointers: q,
 * k_pool, v_pool, block_tables, qo_indptr (int32 [num_reqs + 1], prefix sums of
 * qo_len), kv_len (int32 [num_reqs]), out, lse, workspace (at least
 * plan->workspace_bytes bytes, 256-byte aligned; may be NULL when that is 0).
 * The workspace holds split partials and, in its first 64 KiB, the completion
 * counters of split work (one per (row, KV head) and one per (prefill tile, KV
 * head)): allocate it zeroed once; every call leaves the counters zero again, so
 * the buffer can be reused by later calls (of any plan) on the same stream.  Two
 * calls that run concurrently must not share a workspace.
 * Errors: PA_ERR_NULL, PA_ERR_UNSUPPORTED (geometry differs from the plan's),
 * PA_ERR_WORKSPACE, PA_ERR_HIP.
 */
pa_status pa_attention_batch(const pa_geometry* geometry, const pa_plan_t* plan, const void* q,
                             const void* k_pool, const void* v_pool, const int32_t* block_tables,
                             int32_t max_blocks_per_req, const int32_t* qo_indptr, const int32_t* kv_len,
                             void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step of a layer with the append fused into the attention launch: for a
 * batch of decode rows only (qo_len = 1), row r's new K / V (k_new / v_new row
 * qo_indptr[r], bf16 [total_q][num_kv_heads][head_dim]) is written to the slot of its
 * position kv_len[r] - 1 -- block_tables[r][(kv_len[r] - 1) / block_size], offset
 * (kv_len[r] - 1) % block_size -- and attention reads it from k_new / v_new directly.
 * The result equals pa_append_kv (with those slots) followed by pa_attention_batch, in
 * one launch: the per-layer append is the step's other kernel (book section 8.3.1; the
 * Perplexity blog orders the per-layer append before attention).  Shared-prefix groups
 * are supported; a row's last block must be its own (the planner never shares it).
 * PA_ERR_UNSUPPORTED for a plan with rows of qo_len > 1; other arguments and errors as
 * for pa_attention_batch (PA_VALIDATE=1 also checks that no two rows write one slot).
 */
pa_status pa_decode_step(const pa_geometry* geometry, const pa_plan_t* plan, const void* q, void* k_pool,
                         void* v_pool, const void* k_new, const void* v_new, const int32_t* block_tables,
                         int32_t max_blocks_per_req, const int32_t* qo_indptr, const int32_t* kv_len, void* out,
                         float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * One step of a layer for any batch (decode rows and chunked-prefill rows) with the
 * append fused into the step: row r's qo_len new K / V rows (k_new / v_new rows
 * qo_indptr[r] .. qo_indptr[r + 1] - 1, bf16 [total_q][num_kv_heads][head_dim]) are
 * written to the slots of positions kv_len[r] - qo_len .. kv_len[r] - 1 through
 * block_tables.  Decode rows do it inside the decode launch (attention reads the new
 * token from k_new / v_new); chunk rows' tokens go into the pool in extra workgroups of
 * that launch, which then runs before the chunk tiles (with no decode rows, or with
 * shared-prefix groups, in a short launch of their own before the tiles); the tiles read
 * the pool.  The result equals pa_append_kv (with those
 * slots) followed by pa_attention_batch (book section 8.3.1: a token's KV goes to a slot
 * of the block its table names; the Perplexity blog orders the per-layer append before
 * attention).  The slots a step writes must be distinct and in blocks no other row of the
 * batch reads (copy-on-write of shared blocks is the caller's, as for pa_append_kv).
 * Arguments and errors as for pa_attention_batch; PA_ERR_NULL for missing k_new / v_new;
 * PA_VALIDATE=1 also checks that no two new tokens share a slot.
 */
pa_status pa_attention_step(const pa_geometry* geometry, const pa_plan_t* plan, const void* q, void* k_pool,
                            void* v_pool, const void* k_new, const void* v_new, const int32_t* block_tables,
                            int32_t max_blocks_per_req, const int32_t* qo_indptr, const int32_t* kv_len, void* out,
                            float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Host-side content checks on host copies of a batch's arguments: 1 <= qo_len <=
 * kv_len, ceil(kv_len / block_size) <= max_blocks_per_req, and every table entry
 * a row reads names a block in [0, num_blocks).  Returns PA_OK, PA_ERR_NULL,
 * PA_ERR_SHAPE or PA_ERR_RANGE; *bad_index (may be NULL) receives the offending
 * request index.
 */
pa_status pa_validate_batch(const pa_geometry* geometry, int32_t num_reqs, const int32_t* qo_len_host,
                            const int32_t* kv_len_host, const int32_t* block_tables_host,
                            int32_t max_blocks_per_req, int32_t* bad_index);

/*
 * Host-side check of a slot mapping: every slot is < 0 or below
 * num_blocks * block_size, and no non-negative slot repeats.  Returns PA_OK,
 * PA_ERR_NULL, PA_ERR_SHAPE or PA_ERR_RANGE; *bad_index (may be NULL) receives
 * the offending token index.
 */
pa_status pa_validate_append(const pa_geometry* geometry, const int32_t* slot_mapping_host, int32_t n_tokens,
                             int32_t* bad_index);

/*
 * Copy whole blocks inside the pools: for i < n, the K and V tiles of every KV head of
 * block src[i] are copied to block dst[i].  This is the copy-on-write step of a shared
 * block that one request is about to write into: the request gets a private copy and
 * its table is pointed at it (book section 8.3.2, copy-on-write of a shared tail
 * block).  Device pointers: k_pool, v_pool (written in place), src_blocks, dst_blocks
 * (int32 [n]).  Pairs with an id outside [0, num_blocks) are skipped.  A dst that is
 * also a src, or a dst that repeats, is invalid (pa_validate_copy reports it); the
 * result is then unspecified.  Errors: PA_ERR_NULL, PA_ERR_UNSUPPORTED, PA_ERR_SHAPE
 * (n < 0), PA_ERR_HIP.
 */
pa_status pa_copy_blocks(const pa_geometry* geometry, void* k_pool, void* v_pool, const int32_t* src_blocks,
                         const int32_t* dst_blocks, int32_t n, void* stream);

/*
 * Host-side check of a block-copy list: every id is in [0, num_blocks), no dst repeats
 * and no dst is also a src.  Returns PA_OK, PA_ERR_NULL, PA_ERR_SHAPE or PA_ERR_RANGE;
 * *bad_index (may be NULL) receives the offending pair index.
 */
pa_status pa_validate_copy(const pa_geometry* geometry, const int32_t* src_blocks_host,
                           const int32_t* dst_blocks_host, int32_t n, int32_t* bad_index);

/*
 * q8_0 KV pool (book section 8.4.2 and fig. 8-23: 32 values share one 2-byte scale and
 * are stored as 8-bit codes, 34 bytes in place of 64).  A group is 32 consecutive dims
 * of one token's row for one KV head.  A K (or V) tile of one (block, KV head) is
 * PA_Q8_TILE_BYTES bytes: the block's [block_size][head_dim] int8 codes, then its
 * [block_size][head_dim / 32] IEEE binary16 scales; a code c with scale d stands for
 * c * d.  One pool holds both: uint8 [num_blocks][num_kv_heads][2][PA_Q8_TILE_BYTES],
 * each (block, KV head) its K tile, then its V tile, so a block's K and V for one head
 * are read as one contiguous 4352-byte piece.  Q, the outputs and the new rows stay bf16.
 */
#define PA_Q8_TILE_BYTES (16 * 128 + 16 * (128 / 32) * 2)

/*
 * pa_append_kv into a q8_0 pool: each new bf16 row is quantised per 32-value group with
 * scale d = binary16(min(max|x| / 127, 65504)) (binary32 division, conversion to
 * nearest even) and codes rint(x / d) in binary32 (ties to even) clamped to [-127, 127],
 * 0 where d = 0.  New rows must be finite.  Device pointers: kv_pool_q8 (written in
 * place), k_new, v_new, slot_mapping; slot rules and errors as for pa_append_kv.
 */
pa_status pa_append_kv_q8(const pa_geometry* geometry, void* kv_pool_q8, const void* k_new, const void* v_new,
                          const int32_t* slot_mapping, int32_t n_tokens, void* stream);

/*
 * pa_attention_batch over a q8_0 pool, for any batch pa_attention_batch takes (decode
 * rows, chunked-prefill rows, shared-prefix groups from pa_plan_shared_prefix): the values
 * are the codes times their scales, and everything else (outputs, splits, workspace) is
 * as for pa_attention_batch.  Q is converted to binary16 toward zero (exact for bf16
 * values of magnitude in [2^-14, 65504]; larger ones saturate at 65504).  Every path
 * takes the K codes as exact binary16 integers and applies the K scales to the scores in
 * binary32.  V: on decode rows each V scale d is folded into its token's softmax weight p
 * (p <= 2^8, as the running maximum is raised lazily) and p * d is rounded to binary16
 * toward zero; on chunk rows and prefix groups each V value code * d is rounded to
 * binary16 (nearest) and the weights p to binary16 (nearest).  Limits that follow: (1) a
 * V group with scale d below 2^-14 (largest |value| below about 0.008) gives decode
 * weights, or chunk-row values, in binary16's subnormal range, so the output's relative
 * error grows as the V values shrink (about 0.4% of |O| at |V| ~ 1e-3, several percent at
 * 1e-4); (2) p * d and code * d must stay below 65504, which holds for d <= 255 (largest
 * |V| <= 32,000).  K scales have no such limit.  The new rows must already be in the pool
 * (pa_append_kv_q8 first), or use the fused steps below.
 */
pa_status pa_attention_batch_q8(const pa_geometry* geometry, const pa_plan_t* plan, const void* q,
                                const void* kv_pool_q8, const int32_t* block_tables, int32_t max_blocks_per_req,
                                const int32_t* qo_indptr, const int32_t* kv_len, void* out, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_step / pa_attention_step over a q8_0 pool: the append of the new rows fused
 * into the step (into the decode launch for decode rows; chunk rows' new tokens go into the
 * pool in a short launch before the tiles).  Each new 32-value group is quantised exactly as
 * pa_append_kv_q8 quantises it (the same scale and codes: a group's largest magnitude is
 * gathered from the lanes that hold its pieces) and written to the slot of its position;
 * the attention uses the stored codes and scales, so outputs, LSEs and the pool are
 * bit-identical to pa_append_kv_q8 + pa_attention_batch_q8.  Arguments, rules and errors as
 * for pa_decode_step / pa_attention_step, with the one q8_0 pool in place of k_pool / v_pool.
 */
pa_status pa_decode_step_q8(const pa_geometry* geometry, const pa_plan_t* plan, const void* q, void* kv_pool_q8,
                            const void* k_new, const void* v_new, const int32_t* block_tables,
                            int32_t max_blocks_per_req, const int32_t* qo_indptr, const int32_t* kv_len, void* out,
                            float* lse, void* workspace, size_t workspace_bytes, void* stream);
pa_status pa_attention_step_q8(const pa_geometry* geometry, const pa_plan_t* plan, const void* q, void* kv_pool_q8,
                               const void* k_new, const void* v_new, const int32_t* block_tables,
                               int32_t max_blocks_per_req, const int32_t* qo_indptr, const int32_t* kv_len, void* out,
                               float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* pa_copy_blocks for a q8_0 pool (all of a block's tiles); same rules and errors. */
pa_status pa_copy_blocks_q8(const pa_geometry* geometry, void* kv_pool_q8, const int32_t* src_blocks,
                            const int32_t* dst_blocks, int32_t n, void* stream);

/*
 * FP8 KV pools (book section 8.4.4: KV stored in FP8 while Q stays BF16, figs. 8-27 and
 * 8-28; section 8.4.2's cost model ΔT = ΔD/β − T_c).  Two pools with the bf16 pools'
 * layout, uint8 [num_blocks][num_kv_heads][block_size][head_dim], one OCP FP8 E4M3 code
 * per value (1 sign bit, 4 exponent bits with bias 7, 3 fraction bits; largest magnitude
 * 448; S.1111.111 is NaN), and one binary32 scale per pool: a code c stands for
 * decode(c) * k_scale in the K pool and decode(c) * v_scale in the V pool.  Scales must be
 * finite and > 0 (else PA_ERR_SHAPE).
 *
 * pa_append_kv_fp8: each new bf16 value x is stored as the code of x / scale (binary32
 * division), to nearest with ties to even, magnitudes above 448 (infinities too)
 * saturating to 448, a NaN as the NaN code 0x7F.  Slot rules and errors as for
 * pa_append_kv.
 */
pa_status pa_append_kv_fp8(const pa_geometry* geometry, void* k_pool_fp8, void* v_pool_fp8, const void* k_new,
                           const void* v_new, const int32_t* slot_mapping, int32_t n_tokens, float k_scale,
                           float v_scale, void* stream);

/*
 * pa_attention_batch over FP8 pools, for any batch pa_attention_batch takes (decode rows,
 * chunked-prefill rows, shared-prefix groups); outputs, splits, workspace and errors as for
 * pa_attention_batch.  Every E4M3 value is a bf16 value, so the codes are widened to bf16
 * exactly and the bf16 arithmetic runs on them; k_scale multiplies the scores (folded
 * into the score scale in binary32) and v_scale each normalised output.  The new rows must
 * already be in the pools (pa_append_kv_fp8 first), or use the fused steps below.
 */
pa_status pa_attention_batch_fp8(const pa_geometry* geometry, const pa_plan_t* plan, const void* q,
                                 const void* k_pool_fp8, const void* v_pool_fp8, const int32_t* block_tables,
                                 int32_t max_blocks_per_req, const int32_t* qo_indptr, const int32_t* kv_len,
                                 void* out, float* lse, void* workspace, size_t workspace_bytes, float k_scale,
                                 float v_scale, void* stream);

/*
 * pa_decode_step / pa_attention_step over FP8 pools: the append of the new rows fused into
 * the step (into the decode launch for decode rows; chunk rows' new tokens go into the
 * pools in a short launch before the tiles).  Each new value is encoded exactly as
 * pa_append_kv_fp8 encodes it (the same binary32 quotient, saturation and NaN rule) and
 * written to the slot of its position; the attention uses the value its code represents,
 * so outputs, LSEs and pools are bit-identical to pa_append_kv_fp8 + pa_attention_batch_fp8.
 * Arguments, rules and errors as for pa_decode_step / pa_attention_step, plus the scales.
 */
pa_status pa_decode_step_fp8(const pa_geometry* geometry, const pa_plan_t* plan, const void* q, void* k_pool_fp8,
                             void* v_pool_fp8, const void* k_new, const void* v_new, const int32_t* block_tables,
                             int32_t max_blocks_per_req, const int32_t* qo_indptr, const int32_t* kv_len, void* out,
                             float* lse, void* workspace, size_t workspace_bytes, float k_scale, float v_scale,
                             void* stream);
pa_status pa_attention_step_fp8(const pa_geometry* geometry, const pa_plan_t* plan, const void* q, void* k_pool_fp8,
                                void* v_pool_fp8, const void* k_new, const void* v_new, const int32_t* block_tables,
                                int32_t max_blocks_per_req, const int32_t* qo_indptr, const int32_t* kv_len,
                                void* out, float* lse, void* workspace, size_t workspace_bytes, float k_scale,
                                float v_scale, void* stream);

/* pa_copy_blocks for FP8 pools (one byte per value); same rules and errors. */
pa_status pa_copy_blocks_fp8(const pa_geometry* geometry, void* k_pool_fp8, void* v_pool_fp8,
                             const int32_t* src_blocks, const int32_t* dst_blocks, int32_t n, void* stream);

/*
 * Reference-counted block allocator with stream-deferred release (host side; book
 * section 8.3.2 and figs. 8-14 / 8-15): a physical block carries one reference per block
 * table that points at it, so a shared prefix is a set of blocks with counts above one;
 * a request about to write into a shared block first gets a private copy; and a block
 * returns to the free pool only when its last reference is gone and the device has
 * finished the work that reads it.  The allocator hands out block ids of one pool (the
 * same ids serve every layer's pools); the caller fills block tables with them.  It owns
 * no device memory; an allocator is not thread-safe (one per host thread, or a lock).
 */
typedef struct pa_block_allocator pa_block_allocator;

/* A pool of num_blocks free blocks.  Errors: PA_ERR_NULL, PA_ERR_SHAPE (num_blocks < 1). */
pa_status pa_allocator_create(int32_t num_blocks, pa_block_allocator** allocator);

/* Frees the allocator (pending releases are dropped).  NULL is ignored. */
void pa_allocator_destroy(pa_block_allocator* allocator);

/*
 * n free blocks, each with one reference, into blocks_out (host int32 [n]).  Deferred
 * releases whose stream work has completed are reclaimed first.  All or nothing:
 * PA_ERR_NO_BLOCKS when fewer than n are free.
 */
pa_status pa_allocator_alloc(pa_block_allocator* allocator, int32_t n, int32_t* blocks_out);

/* One more reference to each listed block (a table that starts sharing them).
 * PA_ERR_RANGE (nothing changed) if a block is not allocated. */
pa_status pa_allocator_retain(pa_block_allocator* allocator, const int32_t* blocks, int32_t n);

/*
 * Drops one reference per list entry (a block may be listed more than once).  A block
 * whose count reaches zero becomes free: at once when deferred is 0 (the caller knows
 * no queued device work reads it), else once the work queued on `stream` at this call
 * has completed (an event recorded now; not allowed while the stream is being captured
 * into a graph: PA_ERR_UNSUPPORTED).  PA_ERR_RANGE (nothing changed) if a block is not
 * allocated or would drop below zero; PA_ERR_HIP if the event cannot be recorded.
 */
pa_status pa_allocator_release(pa_block_allocator* allocator, const int32_t* blocks, int32_t n, void* stream,
                               int32_t deferred);

/*
 * Copy-on-write before a request writes into `block`: if the block has one reference
 * it is returned as is (write in place); otherwise a fresh block is allocated and
 * returned, and the shared block loses this request's reference.  The caller then
 * copies the data (pa_copy_blocks or pa_copy_blocks_q8, on the stream of the write) and
 * points its table at the returned block.  PA_ERR_RANGE, PA_ERR_NO_BLOCKS.
 */
pa_status pa_allocator_cow(pa_block_allocator* allocator, int32_t block, int32_t* block_out);

/* Current reference count of a block (0 when free or awaiting a deferred release). */
pa_status pa_allocator_refcount(const pa_block_allocator* allocator, int32_t block, int32_t* count);

/* Free blocks after reclaiming completed deferred releases, and blocks still waiting
 * (either pointer may be NULL). */
pa_status pa_allocator_num_free(pa_block_allocator* allocator, int32_t* free_blocks, int32_t* pending_blocks);

/* Waits for every deferred release's stream work, then reclaims.  PA_ERR_HIP on failure. */
pa_status pa_allocator_sync(pa_block_allocator* allocator);

/*
 * pa_attention_batch for callers that cannot allocate device memory or pass a workspace:
 * code being captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc.  It takes no workspace: the split partials and completion counters live in a
 * fixed scratch array of PA_NOALLOC_SCRATCH_BYTES bytes that the library holds on every
 * device it runs on until the process ends.  The call allocates nothing (no hipMalloc, no
 * hipFree, no allocating library routine).  Arguments, layouts and results are those of
 * pa_attention_batch; the stream must belong to the current device (PA_ERR_UNSUPPORTED
 * otherwise).  PA_ERR_WORKSPACE, with nothing launched, when plan->workspace_bytes exceeds
 * PA_NOALLOC_SCRATCH_BYTES.  The first call on a device looks the scratch array up and
 * zeroes its counters on `stream`; every call leaves them zero again.  All calls on one
 * device share that device's array: two calls whose work overlaps in time on one device
 * (different streams, or different host threads without ordering) race and give wrong
 * results; calls ordered on one stream are safe.
 */
#define PA_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)
pa_status pa_attention_batch_noalloc(const pa_geometry* geometry, const pa_plan_t* plan, const void* q,
                                     const void* k_pool, const void* v_pool, const int32_t* block_tables,
                                     int32_t max_blocks_per_req, const int32_t* qo_indptr, const int32_t* kv_len,
                                     void* out, float* lse, void* stream);

/* Compute-unit count of a HIP device (for pa_plan).  PA_ERR_HIP on failure. */
pa_status pa_query_num_cus(int32_t device, int32_t* num_cus);

/* sizeof(pa_plan_t) as this library was compiled, for bindings that mirror the struct. */
size_t pa_plan_struct_bytes(void);

/* Static text for a status code. */
const char* pa_status_string(pa_status status);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */

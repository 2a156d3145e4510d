// HIP kernels for gfx950 (MI355X) and the device-side C entry points.
//
//   pa_append_scatter   new K/V rows -> pool slots named by the slot mapping
//   pa_decode_split     one wavefront per (decode row, KV head, KV split): block-table
//                       gather with several blocks of loads in flight, QK^T with bf16
//                       dot2, online softmax in FP32, PV accumulation in FP32, and the
//                       log-sum-exp merge of the splits done by the last split to finish
//   pa_prefill_tile     chunked-prefill rows: one workgroup per (row, KV head, 32 new
//                       tokens x 4 query heads); K / V copied straight into LDS,
//                       S^T = K Q^T and O^T = V^T P^T on BF16 MFMA with FP32
//                       accumulation, causal mask, online softmax
//   pa_append_q8_scatter, pa_decode_split<true>
//                       the same append and decode over a q8_0 pool
//
// Pool layout: [block][kv_head][token-in-block][dim] (head-major inside a block), so one
// (block, KV head) tile is 16 x 128 bf16 = 4 KiB of contiguous memory.  A q8_0 tile is
// the 16 x 128 int8 codes followed by the 16 x 4 binary16 scales, 2176 bytes, and the
// q8_0 pool keeps each (block, KV head)'s K tile and V tile side by side (4352 bytes):
// half-size tiles read as separate 2 KiB pieces stream markedly slower from HBM.
#include <hip/hip_runtime.h>

#include <cmath>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <stdlib.h>

#include <mutex>
#include <type_traits>
#include <vector>

#include "pa_internal.h"

namespace {

using pa::kBlock;
using pa::kGroup;
using pa::kHeadDim;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float kLn2 = 0.69314718055994531f;
constexpr float kLog2e = 1.44269504088896341f;
// Lazy rescaling threshold in log2 units: the running maximum is only raised when a
// score exceeds it by more than this, so unnormalised weights stay below 2^8.
constexpr float kRescaleSlack = 8.0f;

__device__ inline float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Round two floats to bf16 (nearest even) and pack them, low half first.
__device__ inline uint32_t pack_bf16(float a, float b)
{
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ inline float dot2_bf16(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

template <int kCtrl>
__device__ inline float dpp(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;   // lane i <-> 7 - i inside each half-row

__device__ inline float shfl_xor(float x, int mask) { return __shfl_xor(x, mask, 64); }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Relaxed agent-scope accesses: coherent across the XCDs without cache maintenance.
__device__ inline void store_agent(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline float load_agent(const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// Running log-sum-exp merge of normalised partial results (o_s, lse_s in log2 units):
// out = sum_s 2^lse_s o_s / sum_s 2^lse_s, with the weights taken relative to the largest
// lse seen so far.  An empty partial (lse = -inf) adds nothing; a NaN lse poisons the
// result.
struct LseMerge {
    float lmax = -INFINITY, wsum = 0.f, o = 0.f;
    bool nan = false;
    __device__ void add(float ls, float os)
    {
        nan |= ls != ls;
        if (!(ls > -INFINITY))
            return;
        if (ls > lmax) {
            const float a = lmax == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(lmax - ls);
            wsum *= a;
            o *= a;
            lmax = ls;
        }
        const float c = __builtin_amdgcn_exp2f(ls - lmax);
        wsum += c;
        o = fmaf(c, os, o);
    }
};

// Adds partials s = 0 .. n - 1 to m, eight at a time: all loads of a group of eight are
// issued before any is used, so n partials cost about n / 8 memory round trips.
template <typename LoadLse, typename LoadO>
__device__ inline void merge_partials(LseMerge& m, int n, LoadLse load_lse, LoadO load_o)
{
    for (int s0 = 0; s0 < n; s0 += 8) {
        float ls[8], os[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int s = min(s0 + u, n - 1);
            ls[u] = load_lse(s);
            os[u] = load_o(s);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (s0 + u < n)
                m.add(ls[u], os[u]);
    }
}

__device__ inline float readlane_f(float x, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// The query heads one workgroup serves: virtual KV head vkv = slice * Hkv + kvh holds query
// heads head0 .. head0 + 3 of KV head kvh, head0 = kvh * G + 4 * slice (G = Hq / Hkv), of
// which `heads` = min(4, G - 4 * slice) exist; the others are empty slots (zero queries,
// nothing written).  Partials are indexed by head slot, vkv * 4 + h.
struct HeadSlice {
    int kvh, slice, head0, heads, slot0;
};
__device__ inline HeadSlice head_slice(int vkv, int num_q_heads, int num_kv_heads)
{
    HeadSlice hs;
    const int g = num_q_heads / num_kv_heads;
    hs.kvh = vkv % num_kv_heads;
    hs.slice = vkv / num_kv_heads;
    hs.head0 = hs.kvh * g + kGroup * hs.slice;
    hs.heads = min(kGroup, g - kGroup * hs.slice);
    hs.slot0 = vkv * kGroup;
    return hs;
}

__device__ inline float half_bits_to_float(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }

// Two floats -> binary16 pair (toward zero), low half first.
__device__ inline uint32_t pack_half_rtz(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

__device__ inline float dot2_f16(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}

// q8_0 codes as exact binary16 numbers: the int8 code c becomes 1152 + c (= 1024 + (c + 128),
// whose bit pattern is 0x64 : (c ^ 0x80)).  The products then carry a bias of 1152 times
// the other operand, which the callers take off once.  `sel` picks, through v_perm, the
// two code bytes that go to the low and high halves (byte slots 0 and 2).
constexpr float kQ8Bias = 1152.0f;
__device__ inline uint32_t q8_to_half2(uint32_t hi_src, uint32_t lo_src, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi_src, lo_src, sel) ^ 0x64806480u;
}

// ------------------------------------------------------------------------------ append

// One thread moves one 16-byte chunk of K and the matching chunk of V.
__global__ __launch_bounds__(256) void pa_append_scatter(uint16_t* __restrict__ k_pool, uint16_t* __restrict__ v_pool,
                                                         const uint16_t* __restrict__ k_new,
                                                         const uint16_t* __restrict__ v_new,
                                                         const int32_t* __restrict__ slot_mapping, int32_t n_tokens,
                                                         int32_t num_kv_heads, int64_t num_slots)
{
    constexpr int kChunks = kHeadDim * 2 / 16;   // 16-byte chunks per (token, head) row
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per_token = (int64_t)num_kv_heads * kChunks;
    if (idx >= (int64_t)n_tokens * per_token)
        return;
    const int32_t t = (int32_t)(idx / per_token);
    const int32_t rem = (int32_t)(idx - (int64_t)t * per_token);
    const int32_t h = rem / kChunks, c = rem % kChunks;
    const int32_t slot = slot_mapping[t];
    if (slot < 0 || (int64_t)slot >= num_slots)
        return;
    const int64_t blk = slot / kBlock, off = slot % kBlock;
    const int64_t dst = ((blk * num_kv_heads + h) * kBlock + off) * kHeadDim / 8 + c;   // in 16-byte units
    const int64_t src = ((int64_t)t * num_kv_heads + h) * kHeadDim / 8 + c;
    reinterpret_cast<u32x4*>(k_pool)[dst] = reinterpret_cast<const u32x4*>(k_new)[src];
    reinterpret_cast<u32x4*>(v_pool)[dst] = reinterpret_cast<const u32x4*>(v_new)[src];
}

// q8_0 quantisation shared by the append and the fused steps (so that the codes they
// store agree bit for bit).  Scale of a 32-value group from its largest magnitude:
// binary16(min(amax / 127, 65504)), the division in binary32 rounded to nearest; returns
// the scale as a float and its binary16 bits in `bits`.
__device__ inline float q8_group_scale(float amax, uint32_t& bits)
{
    float d = amax / 127.0f;
    if (d > 65504.0f)
        d = 65504.0f;
    const _Float16 dh = (_Float16)d;
    bits = __builtin_bit_cast(uint16_t, dh);
    return (float)dh;
}

// Codes of four values with scale dw: rint(x / dw) clamped to +-127 (0 when dw = 0), as
// int8 bytes, first value in the low byte.
__device__ inline uint32_t q8_codes4(float x0, float x1, float x2, float x3, float dw)
{
    const float x[4] = {x0, x1, x2, x3};
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float c = 0.f;
        if (dw != 0.f)
            c = fminf(fmaxf(rintf(x[j] / dw), -127.f), 127.f);
        word |= ((uint32_t)(int32_t)c & 0xffu) << (8 * j);
    }
    return word;
}

// Largest magnitude of eight bf16 values (four pairs), from 0: the append's amax over a
// group is the largest of these over the group's pieces.
__device__ inline float bf16x8_amax(const u32x4 w)
{
    float a = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        a = fmaxf(a, fmaxf(fabsf(bf16_lo(w[j])), fabsf(bf16_hi(w[j]))));
    return a;
}

// Codes of eight bf16 values (four pairs) with scale dw.
__device__ inline u32x2 q8_codes8(const u32x4 w, float dw)
{
    return u32x2{q8_codes4(bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1]), dw),
                 q8_codes4(bf16_lo(w[2]), bf16_hi(w[2]), bf16_lo(w[3]), bf16_hi(w[3]), dw)};
}

// One thread quantises one 32-value group of one (token, KV head) row, K and V: scale
// d = binary16(min(amax / 127, 65504)), codes rint(x / d) clamped to +-127 (0 when d = 0),
// the divisions in binary32 rounded to nearest.
// Group grp of new row src (element offset (token * Hkv + h) * head_dim) of K and of V,
// quantised into slot off of block blk, KV head h.
__device__ inline void q8_append_group(uint8_t* kv_pool, const uint16_t* k_new, const uint16_t* v_new, int64_t src,
                                       int grp, int64_t blk, int off, int h, int num_kv_heads)
{
    constexpr int kGroups = kHeadDim / pa::kQ8Group;
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const u32x4* in = reinterpret_cast<const u32x4*>((which ? v_new : k_new) + src + grp * pa::kQ8Group);
        u32x4 w[4];
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[i] = in[i];
            amax = fmaxf(amax, bf16x8_amax(w[i]));
        }
        uint32_t bits;
        const float dw = q8_group_scale(amax, bits);
        u32x2 c[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            c[i] = q8_codes8(w[i], dw);
        uint8_t* tile = kv_pool + ((blk * num_kv_heads + h) * 2 + which) * pa::kQ8TileBytes;
        u32x4* codes = reinterpret_cast<u32x4*>(tile + off * kHeadDim + grp * pa::kQ8Group);
        codes[0] = u32x4{c[0].x, c[0].y, c[1].x, c[1].y};
        codes[1] = u32x4{c[2].x, c[2].y, c[3].x, c[3].y};
        reinterpret_cast<uint16_t*>(tile + pa::kQ8CodeBytes)[off * kGroups + grp] = (uint16_t)bits;
    }
}

__global__ __launch_bounds__(256) void pa_append_q8_scatter(uint8_t* __restrict__ kv_pool,
                                                            const uint16_t* __restrict__ k_new,
                                                            const uint16_t* __restrict__ v_new,
                                                            const int32_t* __restrict__ slot_mapping,
                                                            int32_t n_tokens, int32_t num_kv_heads, int64_t num_slots)
{
    constexpr int kGroups = kHeadDim / pa::kQ8Group;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per_token = (int64_t)num_kv_heads * kGroups;
    if (idx >= (int64_t)n_tokens * per_token)
        return;
    const int32_t t = (int32_t)(idx / per_token);
    const int32_t rem = (int32_t)(idx - (int64_t)t * per_token);
    const int32_t h = rem / kGroups, grp = rem % kGroups;
    const int32_t slot = slot_mapping[t];
    if (slot < 0 || (int64_t)slot >= num_slots)
        return;
    q8_append_group(kv_pool, k_new, v_new, ((int64_t)t * num_kv_heads + h) * kHeadDim, grp, slot / kBlock,
                    slot % kBlock, h, num_kv_heads);
}

// E4M3 codes of eight bf16 values x (four bf16 pairs, first value in the low half): the code
// of x / scale (binary32 division), clamped to +-448 first so that the conversion, which
// rounds to nearest with ties to even, saturates instead of producing NaN; a NaN quotient
// becomes the NaN code 0x7F.  The append and the fused steps share it, so the codes they
// store agree bit for bit.
__device__ inline u32x2 e4m3x8_from_bf16(const u32x4 w, float scale)
{
    uint32_t out[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        float y[4] = {bf16_lo(w[2 * j]) / scale, bf16_hi(w[2 * j]) / scale, bf16_lo(w[2 * j + 1]) / scale,
                      bf16_hi(w[2 * j + 1]) / scale};
        uint32_t nan_bytes = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            nan_bytes |= y[e] != y[e] ? 0xFFu << (8 * e) : 0u;
            y[e] = fminf(fmaxf(y[e], -448.0f), 448.0f);
        }
        uint32_t word = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0u, false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], word, true);
        out[j] = (word & ~nan_bytes) | (0x7F7F7F7Fu & nan_bytes);
    }
    return u32x2{out[0], out[1]};
}

// Eight E4M3 codes -> eight bf16 values (four bf16 pairs, first code in the low half).
__device__ inline u32x4 e4m3x8_to_bf16(const u32x2 w)
{
    return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, true)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, true))};
}

// Append into FP8 pools (the bf16 layout, one E4M3 code per value): one thread per 16 values
// of one (new token, KV head) row, K and V, each value stored as e4m3x8_from_bf16 encodes it.
// 16 values (chunk c) of new row src (element offset (token * Hkv + h) * head_dim) of K and
// of V, encoded into the slot row at byte offset dst (of the (block, KV head) tile's row).
__device__ inline void fp8_append_chunk(uint8_t* k_pool, uint8_t* v_pool, const uint16_t* k_new, const uint16_t* v_new,
                                        int64_t src, int c, int64_t dst, float k_scale, float v_scale)
{
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const u32x4* in = reinterpret_cast<const u32x4*>((which ? v_new : k_new) + src + 16 * c);
        const float sc = which ? v_scale : k_scale;
        const u32x2 lo = e4m3x8_from_bf16(in[0], sc), hi = e4m3x8_from_bf16(in[1], sc);
        *reinterpret_cast<u32x4*>((which ? v_pool : k_pool) + dst + 16 * c) = u32x4{lo.x, lo.y, hi.x, hi.y};
    }
}

__global__ __launch_bounds__(256) void pa_append_fp8_scatter(uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
                                                             const uint16_t* __restrict__ k_new,
                                                             const uint16_t* __restrict__ v_new,
                                                             const int32_t* __restrict__ slot_mapping, int32_t n_tokens,
                                                             int32_t num_kv_heads, int64_t num_slots, float k_scale,
                                                             float v_scale)
{
    constexpr int kChunks = kHeadDim / 16;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per_token = (int64_t)num_kv_heads * kChunks;
    if (idx >= (int64_t)n_tokens * per_token)
        return;
    const int32_t t = (int32_t)(idx / per_token);
    const int32_t rem = (int32_t)(idx - (int64_t)t * per_token);
    const int32_t h = rem / kChunks, c = rem % kChunks;
    const int32_t slot = slot_mapping[t];
    if (slot < 0 || (int64_t)slot >= num_slots)
        return;
    const int64_t blk = slot / kBlock, off = slot % kBlock;
    fp8_append_chunk(k_pool, v_pool, k_new, v_new, ((int64_t)t * num_kv_heads + h) * kHeadDim, c,
                     ((blk * num_kv_heads + h) * kBlock + off) * kHeadDim, k_scale, v_scale);
}

// ------------------------------------------------------------------------------ block copy

// One thread per 16 bytes of a block: pairs x npools x blk_chunks threads, where a block
// of one pool is blk_chunks 16-byte chunks (bf16: two pools, Hkv x 256 chunks each; q8_0:
// one pool, Hkv x 272 chunks); consecutive threads move contiguous memory.
__global__ __launch_bounds__(256) void pa_copy_scatter(u32x4* __restrict__ k_pool, u32x4* __restrict__ v_pool,
                                                       const int32_t* __restrict__ src, const int32_t* __restrict__ dst,
                                                       int32_t n, int32_t num_blocks, int64_t blk_chunks, int32_t npools)
{
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t pair = t / (npools * blk_chunks);
    if (pair >= n)
        return;
    const int32_t s = src[pair], d = dst[pair];
    if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks)
        return;
    const int64_t rem = t - pair * npools * blk_chunks;
    u32x4* pool = rem >= blk_chunks ? v_pool : k_pool;
    const int64_t within = rem % blk_chunks;
    pool[(int64_t)d * blk_chunks + within] = pool[(int64_t)s * blk_chunks + within];
}

// ------------------------------------------------------------------------------ decode

struct DecodeParams {
    const uint16_t* q;
    const uint16_t* k_pool;
    const uint16_t* v_pool;
    const int32_t* block_tables;
    const int32_t* qo_indptr;
    const int32_t* kv_len;
    uint16_t* out;
    float* lse;
    uint32_t* counters;   // one per (row, KV head): splits finished so far
    float* part_o;
    float* part_lse;
    int32_t max_blocks;
    int32_t num_reqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t num_vheads;    // workgroups per (row, split): virtual KV heads of four head slots
    int32_t num_blocks;
    int32_t split_blocks;
    int32_t max_splits;
    float scale_log2;   // score scale times log2(e): softmax runs in base 2 (times the K scale of an FP8 pool)
    float v_scale;      // FP8 pool: the V scale, applied to each normalised output (1 otherwise)
    float k_div, v_div; // FP8 pool with the append fused: the scales new K / V values are divided by
    // shared-prefix groups: rows first .. first + count - 1 skip their first `blocks`
    // blocks, whose partial results (prefix_splits of them per row and head) an earlier
    // launch left in px_part_o / px_part_lse
    int32_t num_prefix_groups;
    int32_t prefix_splits;
    int32_t prefix_first[PA_MAX_PREFIX_GROUPS];
    int32_t prefix_count[PA_MAX_PREFIX_GROUPS];
    int32_t prefix_blocks[PA_MAX_PREFIX_GROUPS];
    const float* px_part_o;
    const float* px_part_lse;
    // fused append (decode steps): row r's new token, k_new / v_new row qo_indptr[r], is
    // written to the slot of position kv_len - 1 and read from these rows directly
    const uint16_t* k_new;
    const uint16_t* v_new;
};

#ifndef PA_DECODE_DEPTH
#define PA_DECODE_DEPTH 1
#endif
// KV blocks whose loads are in flight while a block is being processed.
constexpr int kDecodeDepth = PA_DECODE_DEPTH;
#ifndef PA_DECODE_DEPTH_Q8
#define PA_DECODE_DEPTH_Q8 1
#endif
constexpr int kDecodeDepthQ8 = PA_DECODE_DEPTH_Q8;   // deeper was measured slower
#ifndef PA_DECODE_DEPTH_FP8
#define PA_DECODE_DEPTH_FP8 1
#endif
constexpr int kDecodeDepthFp8 = PA_DECODE_DEPTH_FP8;
constexpr int kDecodeWaves = pa::kDecodeWaves;

// One (block, KV head) tile is 16 tokens x 256 bytes, read by four 16-byte loads per lane.
// K: lane = 8 * t8 + c8 reads tokens t8 and t8 + 8, 16-byte chunks c8 and c8 + 8; each load
//    instruction covers eight whole 128-byte lines (one half-row of each of 8 tokens).
//    k[0] = (t8, c8), k[1] = (t8, c8 + 8), k[2] = (t8 + 8, c8), k[3] = (t8 + 8, c8 + 8).
// V: lane = 16 * tg + c16 reads tokens tg + 4i, chunk c16: four contiguous 1 KiB loads.
struct KvStage {
    u32x4 k[4];
    u32x4 v[4];
};

__device__ inline void load_stage(KvStage& s, const uint16_t* ktile, const uint16_t* vtile, int lane)
{
    const u32x4* kp = reinterpret_cast<const u32x4*>(ktile);
    const u32x4* vp = reinterpret_cast<const u32x4*>(vtile) + lane;
    const int t8 = lane >> 3, c8 = lane & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        s.k[i] = __builtin_nontemporal_load(kp + (t8 + 8 * (i >> 1)) * 16 + c8 + 8 * (i & 1));
#pragma unroll
    for (int i = 0; i < 4; ++i)
        s.v[i] = __builtin_nontemporal_load(vp + 64 * i);
}

// FP8 pool: the bf16 tile's layout with one E4M3 code per value, read at the same element
// positions as load_stage (8 bytes where it reads 16) and widened to bf16 before use:
// every E4M3 value is a bf16 value, so the widening is exact and the bf16 arithmetic runs
// unchanged (the K scale is folded into the score scale, the V scale into the output).
struct KvStageFp8 {
    u32x2 k[4];
    u32x2 v[4];
};

__device__ inline void load_stage_fp8(KvStageFp8& s, const uint8_t* ktile, const uint8_t* vtile, int lane)
{
    const u32x2* kp = reinterpret_cast<const u32x2*>(ktile);
    const u32x2* vp = reinterpret_cast<const u32x2*>(vtile) + lane;
    const int t8 = lane >> 3, c8 = lane & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        s.k[i] = __builtin_nontemporal_load(kp + (t8 + 8 * (i >> 1)) * 16 + c8 + 8 * (i & 1));
#pragma unroll
    for (int i = 0; i < 4; ++i)
        s.v[i] = __builtin_nontemporal_load(vp + 64 * i);
}


__device__ inline KvStage widen(const KvStageFp8& s)
{
    KvStage o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o.k[i] = e4m3x8_to_bf16(s.k[i]);
        o.v[i] = e4m3x8_to_bf16(s.v[i]);
    }
    return o;
}
__device__ inline KvStage widen(const KvStage& s) { return s; }

// q8_0 tile: codes [16][128] int8, then scales [16][4] binary16.
// K: lane = 8 * t8 + c8 reads the 16 codes of dims 16 c8 .. 16 c8 + 15 (one scale group,
//    c8 / 2) of tokens t8 and t8 + 8; each load covers 1 KiB, eight whole 128-byte rows.
// V: lane = 16 * tg + c16 reads the 8 codes of dims 8 c16 .. 8 c16 + 7 (group c16 / 4) of
//    tokens tg + 4 i, i = 0..3: 512 contiguous bytes per load.
// Scales: each lane reads the scales of its own tokens and group (2 for K, 4 for V).
struct KvStageQ8 {
    u32x4 k[2];
    u32x2 v[4];
    uint32_t ks[2], vs[4];
};

__device__ inline void load_stage_q8(KvStageQ8& s, const uint8_t* ktile, const uint8_t* vtile, int lane)
{
    const int t8 = lane >> 3, c8 = lane & 7, tg = lane >> 4, c16 = lane & 15;
    s.k[0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ktile + t8 * kHeadDim + 16 * c8));
    s.k[1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ktile + (t8 + 8) * kHeadDim + 16 * c8));
#pragma unroll
    for (int i = 0; i < 4; ++i)
        s.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(vtile + (tg + 4 * i) * kHeadDim + 8 * c16));
    const uint16_t* ksc = reinterpret_cast<const uint16_t*>(ktile + pa::kQ8CodeBytes);
    const uint16_t* vsc = reinterpret_cast<const uint16_t*>(vtile + pa::kQ8CodeBytes);
    s.ks[0] = __builtin_nontemporal_load(ksc + t8 * 4 + (c8 >> 1));
    s.ks[1] = __builtin_nontemporal_load(ksc + (t8 + 8) * 4 + (c8 >> 1));
#pragma unroll
    for (int i = 0; i < 4; ++i)
        s.vs[i] = __builtin_nontemporal_load(vsc + (tg + 4 * i) * 4 + (c16 >> 2));
}

__device__ inline float dot16(const u32x4& q, const u32x4& k, float acc)
{
    acc = dot2_bf16(q.x, k.x, acc);
    acc = dot2_bf16(q.y, k.y, acc);
    acc = dot2_bf16(q.z, k.z, acc);
    return dot2_bf16(q.w, k.w, acc);
}

// Reduce-scatter over the eight lanes of a half-row: lane c (0..7) holds eight partial
// sums v[0..7] and returns the full sum of v[c] over the eight lanes.  Three halving
// steps pair lanes that differ in one bit of c: the half-row mirror (c <-> 7 - c, bit 2),
// then quad xor 2 (bit 1), then quad xor 1 (bit 0); at each step a lane keeps the half of
// its values that its bit selects and adds the partner's copy of that half.
__device__ inline float reduce_scatter8(const float (&v)[8], int c)
{
    const bool b2 = c & 4, b1 = c & 2, b0 = c & 1;
    float k4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float keep = b2 ? v[4 + i] : v[i];
        const float send = b2 ? v[i] : v[4 + i];
        k4[i] = keep + dpp<kRowHalfMirror>(send);
    }
    float k2[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float keep = b1 ? k4[2 + i] : k4[i];
        const float send = b1 ? k4[i] : k4[2 + i];
        k2[i] = keep + dpp<kQuadXor2>(send);
    }
    const float keep = b0 ? k2[1] : k2[0];
    const float send = b0 ? k2[0] : k2[1];
    return keep + dpp<kQuadXor1>(send);
}

// Orders this wavefront's LDS accesses around a cross-lane exchange.  LDS executes one
// wavefront's instructions in order, so only the compiler has to be kept from moving them.
__device__ inline void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Decode splits of row r whose first `skip` blocks a shared-prefix pass covers, or -1 when
// the row is not a decode row or its lengths disagree with the plan.  The decode kernel and
// the shared-prefix pass both count into a (row, KV head) counter and use this one test, so
// they agree on how many arrivals complete it.
__device__ inline int decode_splits_of(const DecodeParams& p, int r, int skip)
{
    if (p.qo_indptr[r + 1] - p.qo_indptr[r] != 1)
        return -1;
    const int kvlen = p.kv_len[r];
    const int nblk = (kvlen + kBlock - 1) / kBlock;
    if (kvlen < 1 || nblk > p.max_blocks || nblk <= skip || p.split_blocks < 1 ||
        p.split_blocks > pa::kMaxSplitBlocks)
        return -1;
    const int nsplit = (nblk - skip + p.split_blocks - 1) / p.split_blocks;
    return nsplit > p.max_splits ? -1 : nsplit;
}

// Shared-prefix blocks of row r under the plan's groups (0 outside every group).
__device__ inline int prefix_skip_of(const DecodeParams& p, int r)
{
    int skip = 0;
    for (int gi = 0; gi < p.num_prefix_groups; ++gi)
        if (r >= p.prefix_first[gi] && r < p.prefix_first[gi] + p.prefix_count[gi])
            skip = p.prefix_blocks[gi];
    return skip;
}

// Final outputs of rows rows[0 .. nrows - 1] for virtual KV head vkv: each row's decode partials
// (as many as decode_splits_of gives), then its nprefix shared-prefix partials, merged by
// the log-sum-exp rule in that fixed order, whichever workgroup arrived last.  Each thread
// owns one (head, dim) value of every row.  kChunk rows are merged together, kBatch
// partials of each loaded before any is used, so a workgroup finishing several rows pays
// about one row's load latency per kChunk rows (and one row with up to kBatch partials,
// one round trip).  All partials were written with agent-scope stores that completed
// before their writer counted in, so agent-scope loads see them.
static_assert(kGroup * kHeadDim == 64 * kDecodeWaves, "one output value per thread");
template <int kChunk, int kBatch>
__device__ inline void merge_rows_results(const DecodeParams& p, const int* rows, int nrows, int vkv, int nprefix)
{
    const HeadSlice hs = head_slice(vkv, p.num_q_heads, p.num_kv_heads);
    const int head0 = hs.head0, slots = p.num_vheads * kGroup;
    const int idx = threadIdx.x, h = idx / kHeadDim, d = idx & (kHeadDim - 1);
    const float nan = __builtin_nanf("");
    // The partial buffers, held in vector registers so that picking a partial's buffer is
    // a select; left to the compiler, each pick reloads the pointer from the kernel
    // arguments and waits for that scalar load before the partial's loads can go out.
    const float* dec_lse = p.part_lse;
    const float* dec_o = p.part_o;
    const float* pfx_lse = p.px_part_lse;
    const float* pfx_o = p.px_part_o;
    asm volatile("" : "+v"(dec_lse), "+v"(dec_o), "+v"(pfx_lse), "+v"(pfx_o));
    for (int c0 = 0; c0 < nrows; c0 += kChunk) {
        int rr[kChunk], ns[kChunk], tot[kChunk];
        int most = 0;
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            const bool valid = c0 + j < nrows;
            rr[j] = rows[valid ? c0 + j : c0];
            ns[j] = valid ? max(0, decode_splits_of(p, rr[j], prefix_skip_of(p, rr[j]))) : 0;
            tot[j] = valid ? ns[j] + nprefix : 0;
            most = max(most, tot[j]);
        }
        LseMerge mg[kChunk];
        for (int s0 = 0; s0 < most; s0 += kBatch) {
            float ls[kChunk][kBatch], os[kChunk][kBatch];
#pragma unroll
            for (int j = 0; j < kChunk; ++j)
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    const int sidx = min(s0 + u, max(tot[j], 1) - 1);
                    const int64_t pi = sidx < ns[j]
                                           ? ((int64_t)rr[j] * p.max_splits + sidx) * slots + hs.slot0 + h
                                           : ((int64_t)rr[j] * p.prefix_splits + (sidx - ns[j])) * slots +
                                                 hs.slot0 + h;
                    const float* lsrc = sidx < ns[j] ? dec_lse : pfx_lse;
                    const float* osrc = sidx < ns[j] ? dec_o : pfx_o;
                    ls[j][u] = tot[j] > 0 ? load_agent(lsrc + pi) : 0.f;
                    os[j][u] = tot[j] > 0 ? load_agent(osrc + pi * kHeadDim + d) : 0.f;
                }
#pragma unroll
            for (int j = 0; j < kChunk; ++j)
#pragma unroll
                for (int u = 0; u < kBatch; ++u)
                    if (s0 + u < tot[j])
                        mg[j].add(ls[j][u], os[j][u]);
        }
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            if (c0 + j >= nrows || h >= hs.heads)
                continue;
            const int q_row = p.qo_indptr[rr[j]];
            p.out[((int64_t)q_row * p.num_q_heads + head0) * kHeadDim + idx] =
                __builtin_bit_cast(uint16_t, (__bf16)(mg[j].nan ? nan : mg[j].o / mg[j].wsum));
            if (d == 0)
                p.lse[(int64_t)q_row * p.num_q_heads + head0 + h] =
                    mg[j].nan ? nan : (mg[j].lmax + fast_log2(mg[j].wsum)) * kLn2;
        }
    }
}

// merge_rows_results for the many rows a prefix-group workgroup can finish: four rows at
// a time, two wavefronts per row, each lane merging four consecutive dims of one head, so
// a row's partials (up to kBatch at once) are all requested before any is used.
__device__ inline void merge_group_rows(const DecodeParams& p, const int* rows, int nrows, int vkv, int nprefix)
{
    constexpr int kBatch = 12;
    const HeadSlice hs = head_slice(vkv, p.num_q_heads, p.num_kv_heads);
    const int head0 = hs.head0, slots = p.num_vheads * kGroup;
    const int t = threadIdx.x, slot = t >> 7, h = (t >> 5) & 3, d4 = (t & 31) * 4;
    const float nan = __builtin_nanf("");
    const float* dec_lse = p.part_lse;            // in vector registers: see merge_rows_results
    const float* dec_o = p.part_o;
    const float* pfx_lse = p.px_part_lse;
    const float* pfx_o = p.px_part_o;
    asm volatile("" : "+v"(dec_lse), "+v"(dec_o), "+v"(pfx_lse), "+v"(pfx_o));
    for (int c0 = 0; c0 < nrows; c0 += 4) {
        const int j = c0 + slot;                  // the same for both wavefronts of a row
        if (j >= nrows)
            continue;
        const int rr = rows[j];
        const int ns = max(0, decode_splits_of(p, rr, prefix_skip_of(p, rr)));
        const int tot = ns + nprefix;
        LseMerge mg[4];
        for (int s0 = 0; s0 < tot; s0 += kBatch) {
            float ls[kBatch], os[kBatch][4];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int sidx = min(s0 + u, tot - 1);
                const int64_t pi = sidx < ns ? ((int64_t)rr * p.max_splits + sidx) * slots + hs.slot0 + h
                                             : ((int64_t)rr * p.prefix_splits + (sidx - ns)) * slots + hs.slot0 + h;
                const float* lsrc = sidx < ns ? dec_lse : pfx_lse;
                const float* osrc = (sidx < ns ? dec_o : pfx_o) + pi * kHeadDim + d4;
                ls[u] = load_agent(lsrc + pi);
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    os[u][k] = load_agent(osrc + k);
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
                if (s0 + u < tot)
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        mg[k].add(ls[u], os[u][k]);
        }
        if (h >= hs.heads)
            continue;
        const int q_row = p.qo_indptr[rr];
        const int64_t orow = (int64_t)q_row * p.num_q_heads + head0 + h;
        float v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            v[k] = mg[k].nan ? nan : mg[k].o / mg[k].wsum;
        *reinterpret_cast<u32x2*>(p.out + orow * kHeadDim + d4) = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
        if (d4 == 0)
            p.lse[orow] = mg[0].nan ? nan : (mg[0].lmax + fast_log2(mg[0].wsum)) * kLn2;
    }
}

// Grid: max_splits * num_reqs * V workgroups of kDecodeWaves wavefronts (V virtual KV
// heads of four query-head slots each: one per KV head when it serves four query heads),
// virtual head fastest: workgroups go round-robin to the eight XCDs, so with eight KV
// heads each XCD serves one KV head of every row and reads that head's shared-prefix
// blocks from one L2.
//
// A workgroup owns one (row, virtual KV head, split); its blocks are cut into kDecodeWaves
// contiguous runs, one per wavefront.  Each wavefront streams its run with kDecodeDepth
// blocks of loads in flight.  Per block: scores of 16 tokens x 4 heads (bf16 dot2, FP32
// accumulation, reduced over 8 lanes), the online softmax with one (token, head) pair per
// lane, and PV, where each lane accumulates 4 heads x 8 dims over its 4 tokens after the
// weights pass through LDS.  The running maximum is raised lazily (only when a score
// passes it by kRescaleSlack), which keeps exact results and skips most rescales.
//
// The wavefronts' results are merged through LDS with the log-sum-exp rule
//   L = max_w L_w,  c_w = 2^(L_w - L),  O = sum_w c_w O_w / sum_w c_w,  LSE = L + log2 sum_w c_w.
// With one split per row the workgroup writes the final output.  Otherwise it writes a
// partial, and the last split of the (row, KV head) to finish -- found with an agent-scope
// counter that it then resets -- merges the partials by the same rule.
//
// With a q8_0 pool (kQ8) the loads are half as large and the codes enter the products as
// binary16 numbers 1152 + code (see q8_to_half2): each score starts from -1152 times the
// sum of its 16 query values and is then scaled by its group's scale; each PV weight is
// the softmax weight times the value's scale, and -1152 times the weights' sum is taken
// off the accumulators at the end.  Q is widened to binary16, which holds every bf16
// value of magnitude in [2^-14, 65504] exactly.
template <bool kQ8, bool kFused, bool kFp8 = false>
__device__ __attribute__((always_inline)) inline void decode_body(const DecodeParams& p, int bid)
{
    static_assert(!(kFp8 && kQ8), "one pool format");
    constexpr int kDepth = kQ8 ? kDecodeDepthQ8 : kFp8 ? kDecodeDepthFp8 : kDecodeDepth;
    using Stage = std::conditional_t<kQ8, KvStageQ8, std::conditional_t<kFp8, KvStageFp8, KvStage>>;
    __shared__ float p_lds[kDecodeWaves][kBlock * kGroup];
    __shared__ float o_lds[kDecodeWaves][kGroup * kHeadDim];
    __shared__ float l_lds[kDecodeWaves][kGroup];
    __shared__ uint32_t last_lds;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int vkv = bid % p.num_vheads;
    const int rest = bid / p.num_vheads;
    const int r = rest % p.num_reqs;
    const int split = rest / p.num_reqs;
    const HeadSlice hsl = head_slice(vkv, p.num_q_heads, p.num_kv_heads);
    const int kvh = hsl.kvh, head0 = hsl.head0;
    const float nan = __builtin_nanf("");

    // Wavefront w takes blocks g0 + w, g0 + w + 8, ... of the split.  Their table entries
    // (lane i holds entry i) and the first kDepth blocks' K / V are requested before
    // the row's lengths arrive, so the start-up waits for one memory round trip less.  The
    // early requests are bounded by the table row and the pool; entries past the row's
    // last block are never used.
    const int skip = prefix_skip_of(p, r);            // blocks a shared-prefix group reads for this row
    const int g0 = skip + split * p.split_blocks;
    const int bidx = g0 + wave + kDecodeWaves * lane;
    int my_blk = 0;
    if (lane * kDecodeWaves < p.split_blocks && bidx < p.max_blocks)
        my_blk = p.block_tables[(int64_t)r * p.max_blocks + bidx];
    const int q_row = p.qo_indptr[r];
    const int q_end = p.qo_indptr[r + 1];
    const int kvlen = p.kv_len[r];

    const int t8 = lane >> 3, c8 = lane & 7;          // score role
    const int ts = t8 + 8 * (c8 >> 2), hs = c8 & 3;   // softmax role: token ts, head hs
    const int c16 = lane & 15, tg = lane >> 4;        // PV role

    // j < 0: a spare load whose data is never used; it reads pool block 0, which the
    // other spare loads keep in L2 (a re-read of the run's own last block would often
    // miss, the K / V loads being nontemporal)
    auto issue = [&](Stage& st, int j) __attribute__((always_inline)) {
        int id = __builtin_amdgcn_readlane(my_blk, j < 0 ? 0 : j);
        id = (j >= 0 && id >= 0 && id < p.num_blocks) ? id : 0;
        if constexpr (kQ8) {
            const uint8_t* kt = reinterpret_cast<const uint8_t*>(p.k_pool) +
                                ((int64_t)id * p.num_kv_heads + kvh) * (2 * pa::kQ8TileBytes);
            load_stage_q8(st, kt, kt + pa::kQ8TileBytes, lane);
        } else if constexpr (kFp8) {
            const int64_t off = ((int64_t)id * p.num_kv_heads + kvh) * kBlock * kHeadDim;   // one byte per value
            load_stage_fp8(st, reinterpret_cast<const uint8_t*>(p.k_pool) + off,
                           reinterpret_cast<const uint8_t*>(p.v_pool) + off, lane);
        } else {
            const int64_t off = ((int64_t)id * p.num_kv_heads + kvh) * kBlock * kHeadDim;
            load_stage(st, p.k_pool + off, p.v_pool + off, lane);
        }
    };
    Stage st[kDepth + 1];
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
        issue(st[d], d);

    if (q_end - q_row != 1)
        return;                                       // not a decode row
    const int nblk = (kvlen + kBlock - 1) / kBlock;
    const int nsplit = decode_splits_of(p, r, skip);
    if (nsplit < 0) {                                 // lengths disagree with the plan
        if (split == 0)
            for (int i = tid; i < hsl.heads * kHeadDim; i += 64 * kDecodeWaves) {
                p.out[((int64_t)q_row * p.num_q_heads + head0) * kHeadDim + i] = 0x7FC0;
                if (i < hsl.heads)
                    p.lse[(int64_t)q_row * p.num_q_heads + head0 + i] = nan;
            }
        return;
    }
    if (split >= nsplit)
        return;
    const int g_end = min(nblk, g0 + p.split_blocks);
    const int nb = g_end > g0 + wave ? (g_end - g0 - wave + kDecodeWaves - 1) / kDecodeWaves : 0;
    bool bad = lane < nb && (my_blk < 0 || my_blk >= p.num_blocks);
    bad = __syncthreads_or(bad);                      // a block id outside the pool: its data is not used

    // Fused append: the workgroup whose blocks include the new token's block writes the
    // token's K / V row into the pool and uses the new values for that block directly
    // (no other workgroup of the launch reads that block).
    const int new_blk = (kvlen - 1) / kBlock, new_off = (kvlen - 1) % kBlock;
    u32x4 kn0 = u32x4{0u, 0u, 0u, 0u}, kn1 = kn0, vn = kn0;
    // q8_0 pool: the new row quantised as the append quantises it -- this lane's K codes
    // (dims 16 c8 .., group c8 / 2) and V codes (dims 8 c16 .., group c16 / 4) with their
    // groups' scale bits; a group's largest magnitude is gathered from the lanes holding it
    u32x4 kq = u32x4{0u, 0u, 0u, 0u};
    u32x2 vq = u32x2{0u, 0u};
    uint32_t kqs = 0u, vqs = 0u;
    if constexpr (kFused && kQ8) {
        if (new_blk >= g0 && new_blk < g_end) {
            const u32x4* kr = reinterpret_cast<const u32x4*>(p.k_new + ((int64_t)q_row * p.num_kv_heads + kvh) * kHeadDim);
            const u32x4* vr = reinterpret_cast<const u32x4*>(p.v_new + ((int64_t)q_row * p.num_kv_heads + kvh) * kHeadDim);
            const u32x4 ka = kr[2 * c8], kb = kr[2 * c8 + 1], vv = vr[c16];
            float am = fmaxf(bf16x8_amax(ka), bf16x8_amax(kb));
            am = fmaxf(am, shfl_xor(am, 1));                    // the other half of the group
            const float kdw = q8_group_scale(am, kqs);
            const u32x2 k0 = q8_codes8(ka, kdw), k1 = q8_codes8(kb, kdw);
            kq = u32x4{k0.x, k0.y, k1.x, k1.y};
            float av = bf16x8_amax(vv);
            av = fmaxf(av, shfl_xor(av, 1));
            av = fmaxf(av, shfl_xor(av, 2));                    // the four lanes of the group
            vq = q8_codes8(vv, q8_group_scale(av, vqs));
            const int phys = p.block_tables[(int64_t)r * p.max_blocks + new_blk];
            if (hsl.slice == 0 && phys >= 0 && phys < p.num_blocks) {   // one slice writes
                uint8_t* kt = reinterpret_cast<uint8_t*>(const_cast<uint16_t*>(p.k_pool)) +
                              ((int64_t)phys * p.num_kv_heads + kvh) * (2 * pa::kQ8TileBytes);
                uint8_t* vt = kt + pa::kQ8TileBytes;
                if (wave == 0 && t8 == 0) {
                    *reinterpret_cast<u32x4*>(kt + new_off * kHeadDim + 16 * c8) = kq;
                    if ((c8 & 1) == 0)
                        reinterpret_cast<uint16_t*>(kt + pa::kQ8CodeBytes)[new_off * 4 + (c8 >> 1)] = (uint16_t)kqs;
                }
                if (wave == 0 && tg == 0) {
                    *reinterpret_cast<u32x2*>(vt + new_off * kHeadDim + 8 * c16) = vq;
                    if ((c16 & 3) == 0)
                        reinterpret_cast<uint16_t*>(vt + pa::kQ8CodeBytes)[new_off * 4 + (c16 >> 2)] = (uint16_t)vqs;
                }
            }
        }
    } else if constexpr (kFused) {
        if (new_blk >= g0 && new_blk < g_end) {
            const u32x4* kr = reinterpret_cast<const u32x4*>(p.k_new + ((int64_t)q_row * p.num_kv_heads + kvh) * kHeadDim);
            const u32x4* vr = reinterpret_cast<const u32x4*>(p.v_new + ((int64_t)q_row * p.num_kv_heads + kvh) * kHeadDim);
            kn0 = kr[c8];
            kn1 = kr[c8 + 8];
            vn = vr[c16];
            if constexpr (kFp8) {
                // the new row as its codes represent it (the stage holds widened codes)
                kn0 = e4m3x8_to_bf16(e4m3x8_from_bf16(kn0, p.k_div));
                kn1 = e4m3x8_to_bf16(e4m3x8_from_bf16(kn1, p.k_div));
                vn = e4m3x8_to_bf16(e4m3x8_from_bf16(vn, p.v_div));
            }
            const int phys = p.block_tables[(int64_t)r * p.max_blocks + new_blk];
            if (tid < 16 && hsl.slice == 0 && phys >= 0 && phys < p.num_blocks) {   // one slice writes
                const int64_t row = (((int64_t)phys * p.num_kv_heads + kvh) * kBlock + new_off) * (kHeadDim / 8);
                if constexpr (kFp8) {
                    reinterpret_cast<u32x2*>(const_cast<uint16_t*>(p.k_pool))[row + tid] = e4m3x8_from_bf16(kr[tid], p.k_div);
                    reinterpret_cast<u32x2*>(const_cast<uint16_t*>(p.v_pool))[row + tid] = e4m3x8_from_bf16(vr[tid], p.v_div);
                } else {
                    reinterpret_cast<u32x4*>(const_cast<uint16_t*>(p.k_pool))[row + tid] = kr[tid];
                    reinterpret_cast<u32x4*>(const_cast<uint16_t*>(p.v_pool))[row + tid] = vr[tid];
                }
            }
        }
    }

    u32x4 qv[kGroup][2];       // bf16 pool: bf16 pairs of dims 8 c8 .. and 64 + 8 c8 ..
    uint32_t qh[kGroup][8];    // q8_0 pool: binary16 pairs of dims 16 c8 + 2 j, + 1
    float qbias[kGroup];       // q8_0 pool: -1152 times the sum of those 16 values
    {
        const u32x4* qb = reinterpret_cast<const u32x4*>(p.q + ((int64_t)q_row * p.num_q_heads + head0) * kHeadDim);
#pragma unroll
        for (int h = 0; h < kGroup; ++h) {
            const bool has = h < hsl.heads;             // empty head slots hold zero queries
            if constexpr (kQ8) {
                const u32x4 z = u32x4{0u, 0u, 0u, 0u};
                const u32x4 a = has ? qb[h * 16 + 2 * c8] : z, b = has ? qb[h * 16 + 2 * c8 + 1] : z;
                const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
                float sum = 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float lo = bf16_lo(w[j]), hi = bf16_hi(w[j]);
                    qh[h][j] = pack_half_rtz(lo, hi);
                    sum += half_bits_to_float(qh[h][j] & 0xffffu) + half_bits_to_float(qh[h][j] >> 16);
                }
                qbias[h] = -kQ8Bias * sum;
            } else {
                qv[h][0] = has ? qb[h * 16 + c8] : u32x4{0u, 0u, 0u, 0u};
                qv[h][1] = has ? qb[h * 16 + c8 + 8] : u32x4{0u, 0u, 0u, 0u};
            }
        }
    }

    float m = -INFINITY;   // running max (base 2) of head hs, equal in every lane of that head
    float lsum = 0.f;      // this lane's share of head hs's softmax denominator
    float acc[kGroup][8];
    float wsum[kGroup];        // q8_0 pool: sum of this lane's PV weights per head
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
        wsum[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[h][e] = 0.f;
    }

    float* pw = p_lds[wave];

    auto process = [&](const Stage& st_in, int j) __attribute__((always_inline)) {
        auto st = [&]() {
            if constexpr (kQ8)
                return st_in;
            else
                return widen(st_in);                  // FP8 codes -> bf16 (exact); bf16 as is
        }();
        if constexpr (kFused && kQ8) {
            if (g0 + wave + kDecodeWaves * j == new_blk) {   // the block that holds the new token
                if (t8 == new_off) {
                    st.k[0] = kq;
                    st.ks[0] = kqs;
                }
                if (t8 + 8 == new_off) {
                    st.k[1] = kq;
                    st.ks[1] = kqs;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (tg + 4 * i == new_off) {
                        st.v[i] = vq;
                        st.vs[i] = vqs;
                    }
            }
        } else if constexpr (kFused) {
            if (g0 + wave + kDecodeWaves * j == new_blk) {   // the block that holds the new token
                if (t8 == new_off) {
                    st.k[0] = kn0;
                    st.k[1] = kn1;
                }
                if (t8 + 8 == new_off) {
                    st.k[2] = kn0;
                    st.k[3] = kn1;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (tg + 4 * i == new_off)
                        st.v[i] = vn;
            }
        }
        // scores of tokens t8 + 8 tt for the four heads, partial over this lane's 16 dims,
        // index 4 tt + h; the reduce-scatter leaves lane c8 with the full score of token
        // ts = t8 + 8 (c8 / 4), head hs = c8 % 4
        float sc[2 * kGroup];
        if constexpr (kQ8) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const float dk = half_bits_to_float(st.ks[tt]);
                const u32x4 w = st.k[tt];
                uint32_t kc[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    kc[2 * i] = q8_to_half2(w[i], w[i], 0x0c010c00u);       // codes 4i, 4i + 1
                    kc[2 * i + 1] = q8_to_half2(w[i], w[i], 0x0c030c02u);   // codes 4i + 2, 4i + 3
                }
#pragma unroll
                for (int h = 0; h < kGroup; ++h) {
                    float a = qbias[h];
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        a = dot2_f16(qh[h][i], kc[i], a);
                    sc[tt * kGroup + h] = a * dk;
                }
            }
        } else {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int h = 0; h < kGroup; ++h)
                    sc[tt * kGroup + h] = dot16(qv[h][1], st.k[2 * tt + 1], dot16(qv[h][0], st.k[2 * tt], 0.f));
        }
        float x = reduce_scatter8(sc, c8);
        x *= p.scale_log2;
        const int pos0 = (g0 + wave + kDecodeWaves * j) * kBlock;
        if (pos0 + ts >= kvlen)
            x = -INFINITY;
        if (__any(x > m + kRescaleSlack)) {
            float mx = fmaxf(m, x);
            mx = fmaxf(mx, shfl_xor(mx, 4));
            mx = fmaxf(mx, shfl_xor(mx, 8));
            mx = fmaxf(mx, shfl_xor(mx, 16));
            mx = fmaxf(mx, shfl_xor(mx, 32));
            const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - mx);
            m = mx;
            lsum *= alpha;
#pragma unroll
            for (int h = 0; h < kGroup; ++h) {
                const float a = readlane_f(alpha, h);   // lane h holds head h (t8 = 0, c8 = h)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc[h][e] *= a;
                if constexpr (kQ8)
                    wsum[h] *= a;
            }
        }
        // The softmax statistics stay FP32; the weights enter PV as bf16, as in the MFMA
        // prefill path (relative error <= 2^-9 per weight in the numerator only).
        const float pr = fast_exp2(x - m);
        lsum += pr;
        pw[ts * kGroup + hs] = pr;                    // [token][head]
        wave_lds_sync();
        const int valid = kvlen - pos0;               // tokens of this block that exist
        if constexpr (kQ8) {
            // PV on binary16 dot2 over token pairs (tg + 8 pair, tg + 8 pair + 4); the weight
            // of a token is its softmax weight times its scale for this lane's dims (group
            // c16 / 4); a slot past kv_len gets weight 0 whatever its scale holds.
            float dv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dv[i] = half_bits_to_float(st.vs[i]);
                if (tg + 4 * i >= valid)
                    dv[i] = 0.f;
            }
#pragma unroll
            for (int pair = 0; pair < 2; ++pair) {
                const f32x4 pa = *reinterpret_cast<const f32x4*>(&pw[(tg + 8 * pair) * kGroup]);
                const f32x4 pb = *reinterpret_cast<const f32x4*>(&pw[(tg + 8 * pair + 4) * kGroup]);
                const float da = dv[2 * pair], db = dv[2 * pair + 1];
                const uint32_t wk[kGroup] = {pack_half_rtz(pa.x * da, pb.x * db), pack_half_rtz(pa.y * da, pb.y * db),
                                             pack_half_rtz(pa.z * da, pb.z * db), pack_half_rtz(pa.w * da, pb.w * db)};
#pragma unroll
                for (int h = 0; h < kGroup; ++h)
                    wsum[h] = dot2_f16(wk[h], 0x3c003c00u, wsum[h]);   // (1, 1)
                const u32x2 va = st.v[2 * pair], vb = st.v[2 * pair + 1];
#pragma unroll
                for (int d = 0; d < 8; ++d) {
                    const uint32_t b = d & 3;
                    const uint32_t cp = q8_to_half2(vb[d >> 2], va[d >> 2], 0x0c000c00u | ((4u + b) << 16) | b);
#pragma unroll
                    for (int h = 0; h < kGroup; ++h)
                        acc[h][d] = dot2_f16(wk[h], cp, acc[h][d]);
                }
            }
        } else {
        // PV on bf16 dot2: tokens are taken in pairs (tg, tg + 4) and (tg + 8, tg + 12);
        // a pair's V values for one dim and the pair's weights for one head are packed
        // into bf16x2 operands.
        u32x4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] = st.v[i];
        if (valid < kBlock) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (tg + 4 * i >= valid)
                    v[i] = u32x4{0u, 0u, 0u, 0u};     // slots past kv_len may hold anything
        }
#pragma unroll
        for (int pair = 0; pair < 2; ++pair) {
            const f32x4 pa = *reinterpret_cast<const f32x4*>(&pw[(tg + 8 * pair) * kGroup]);
            const f32x4 pb = *reinterpret_cast<const f32x4*>(&pw[(tg + 8 * pair + 4) * kGroup]);
            const uint32_t pk[kGroup] = {pack_bf16(pa.x, pb.x), pack_bf16(pa.y, pb.y), pack_bf16(pa.z, pb.z),
                                         pack_bf16(pa.w, pb.w)};
            const u32x4& va = v[2 * pair];
            const u32x4& vb = v[2 * pair + 1];
            const uint32_t wa[4] = {va.x, va.y, va.z, va.w};
            const uint32_t wb[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t lo = __builtin_amdgcn_perm(wb[w], wa[w], 0x05040100u);   // dim 2w of both tokens
                const uint32_t hi = __builtin_amdgcn_perm(wb[w], wa[w], 0x07060302u);   // dim 2w + 1
#pragma unroll
                for (int h = 0; h < kGroup; ++h) {
                    acc[h][2 * w] = dot2_bf16(pk[h], lo, acc[h][2 * w]);
                    acc[h][2 * w + 1] = dot2_bf16(pk[h], hi, acc[h][2 * w + 1]);
                }
            }
        }
        }
        wave_lds_sync();
    };

    if (!bad && nb > 0) {
        // Loads for block j + kDepth are issued before block j is processed (the first
        // kDepth were issued above).  Past the end of the run a spare load is issued
        // instead, so every iteration issues the same loads, and the stages in flight at
        // the top of the steady-state loop are the same on entry and on every trip: the
        // compiler can then wait for exactly the oldest stage.
        int j0 = 0;
        for (; j0 + kDepth + 1 <= nb; j0 += kDepth + 1) {
#pragma unroll
            for (int u = 0; u <= kDepth; ++u) {
                issue(st[(u + kDepth) % (kDepth + 1)], j0 + u + kDepth < nb ? j0 + u + kDepth : -1);
                process(st[u], j0 + u);
            }
        }
        // the last nb - j0 < kDepth + 1 blocks are already in flight
#pragma unroll
        for (int u = 0; u < kDepth; ++u)
            if (j0 + u < nb)
                process(st[u], j0 + u);
    }

    if constexpr (kQ8) {
#pragma unroll
        for (int h = 0; h < kGroup; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[h][e] = fmaf(-kQ8Bias, wsum[h], acc[h][e]);   // the codes' 1152 offset
    }
    // this wavefront's totals: denominators over its 16 token slots, numerators over its
    // four token groups
    float ltot = lsum;
    ltot += shfl_xor(ltot, 4);
    ltot += shfl_xor(ltot, 8);
    ltot += shfl_xor(ltot, 16);
    ltot += shfl_xor(ltot, 32);
#pragma unroll
    for (int h = 0; h < kGroup; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            acc[h][e] += shfl_xor(acc[h][e], 16);
            acc[h][e] += shfl_xor(acc[h][e], 32);
        }
    const bool empty = nb == 0 || bad;
    if (lane < 16) {
#pragma unroll
        for (int h = 0; h < kGroup; ++h) {
            const float inv = empty ? 0.f : p.v_scale / readlane_f(ltot, h);
            f32x4* dst = reinterpret_cast<f32x4*>(&o_lds[wave][h * kHeadDim + c16 * 8]);
            dst[0] = f32x4{acc[h][0] * inv, acc[h][1] * inv, acc[h][2] * inv, acc[h][3] * inv};
            dst[1] = f32x4{acc[h][4] * inv, acc[h][5] * inv, acc[h][6] * inv, acc[h][7] * inv};
        }
    }
    if (lane < kGroup)
        l_lds[wave][lane] = empty ? -INFINITY : m + fast_log2(ltot);   // lane = head (t8 = 0, c8 = head)
    __syncthreads();

    // merge the wavefronts: thread -> (head h, dim d); 512 outputs, kDecodeWaves * 64 threads
    float res[kGroup * kHeadDim / (64 * kDecodeWaves)];
    float res_lse[kGroup * kHeadDim / (64 * kDecodeWaves)];
    constexpr int kPerThread = kGroup * kHeadDim / (64 * kDecodeWaves);
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        const int idx = tid + k * 64 * kDecodeWaves;
        const int h = idx / kHeadDim;
        float L = -INFINITY;
#pragma unroll
        for (int w = 0; w < kDecodeWaves; ++w)
            L = fmaxf(L, l_lds[w][h]);
        float wsum = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < kDecodeWaves; ++w) {
            const float c = (l_lds[w][h] == -INFINITY) ? 0.f : fast_exp2(l_lds[w][h] - L);
            wsum += c;
            o = fmaf(c, o_lds[w][idx], o);
        }
        res[k] = bad ? nan : o / wsum;
        res_lse[k] = bad ? nan : L + fast_log2(wsum);
    }

    const int64_t out_base = ((int64_t)q_row * p.num_q_heads + head0) * kHeadDim;
    const bool prefix = skip > 0 && p.prefix_splits > 0;
    if (nsplit == 1 && !prefix) {
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) {
            const int idx = tid + k * 64 * kDecodeWaves;
            if (idx / kHeadDim >= hsl.heads)
                continue;
            p.out[out_base + idx] = __builtin_bit_cast(uint16_t, (__bf16)res[k]);
            if ((idx & (kHeadDim - 1)) == 0)
                p.lse[(int64_t)q_row * p.num_q_heads + head0 + idx / kHeadDim] = res_lse[k] * kLn2;
        }
        return;
    }

    // Partials are written with agent-scope stores (coherent across the XCDs' separate L2
    // caches) and every thread waits until its stores have completed before the
    // workgroup counts itself in; the last arrival reads them with agent-scope loads.
    // This needs no L2 writeback or invalidation, which a device fence would do for every
    // split.  A row of a shared-prefix group also waits for its group's prefix splits,
    // which count into the same counter from the same launch.
    const int64_t mine = ((int64_t)r * p.max_splits + split) * (p.num_vheads * kGroup) + hsl.slot0;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        const int idx = tid + k * 64 * kDecodeWaves;
        store_agent(p.part_o + mine * kHeadDim + idx, res[k]);
        if ((idx & (kHeadDim - 1)) == 0)
            store_agent(p.part_lse + mine + idx / kHeadDim, res_lse[k]);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int nprefix = prefix ? p.prefix_splits : 0;
    uint32_t* counter = p.counters + (int64_t)r * p.num_vheads + vkv;
    if (tid == 0) {
        const uint32_t done = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = done == (uint32_t)(nsplit + nprefix - 1);
        if (last)
            __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // ready for the next call
        last_lds = last;
    }
    __syncthreads();
    if (last_lds)
        merge_rows_results<1, 32>(p, &r, 1, vkv, nprefix);
}

template <bool kQ8, bool kFused, bool kFp8 = false>
__global__ __launch_bounds__(64 * kDecodeWaves) void pa_decode_split(DecodeParams p)
{
    decode_body<kQ8, kFused, kFp8>(p, blockIdx.x);
}

// ------------------------------------------------------------------------------ prefill

struct PrefillParams {
    const uint16_t* q;
    const uint16_t* k_pool;
    const uint16_t* v_pool;
    const int32_t* block_tables;
    const int32_t* qo_indptr;
    const int32_t* kv_len;
    uint16_t* out;
    float* lse;
    uint32_t* counters;         // one per (tile, KV head); used when splits > 1
    float* part_o;              // split partials, kPfRows * kHeadDim floats per (tile, KV head, split)
    float* part_lse;            // 4 x 2 x 64 floats (lane order) per (tile, KV head, split)
    int32_t max_blocks;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t num_vheads;         // virtual KV heads (see HeadSlice)
    int32_t num_blocks;
    int32_t num_prefill_rows;
    int32_t splits;             // key splits per tile
    float scale_log2;
    float v_scale;      // FP8 pool: the V scale, applied to each normalised output (1 otherwise)
    float k_div, v_div; // FP8 pool with the append fused: the scales new K / V values are divided by
    int32_t prefill_req[PA_MAX_PREFILL_ROWS];
    int32_t tile_start[PA_MAX_PREFILL_ROWS + 1];
    // shared-prefix mode: one tile per group, its rows (request, head) of the group's
    // decode requests, its keys the group's shared blocks
    int32_t group_first[PA_MAX_PREFIX_GROUPS];
    int32_t group_count[PA_MAX_PREFIX_GROUPS];
    int32_t group_blocks[PA_MAX_PREFIX_GROUPS];
    float* px_part_o;           // [num_reqs][splits][Hq][head_dim]
    float* px_part_lse;         // [num_reqs][splits][Hq]
    // fused append (chunked-prefill rows of a step): row r's new tokens, k_new / v_new
    // rows qo_indptr[r] .., are written to the slots of positions kv_len - qo_len .. and
    // read from these rows directly
    const uint16_t* k_new;
    const uint16_t* v_new;
};

constexpr int kPfKeys = pa::kPrefillKeys;  // keys per step: eight 16-token blocks
constexpr int kPfWaves = 8;                // 4 row groups x 2 key halves
constexpr int kPfRows = pa::kPrefillQ * kGroup;   // 128 MFMA rows: (token, head) pairs
static_assert(kPfRows * kHeadDim == pa::kPrefillPartFloats, "a prefill split partial holds every row of its tile");
constexpr int kPfAcc = 16;                 // f32x4 O^T accumulators per lane: 2 row blocks x 8 dim blocks
constexpr int kTileChunks = kPfKeys * kHeadDim * 2 / 16;   // 16-byte chunks in one K or V tile

// Swizzle of the 16-byte chunk index inside a staged K / V tile row (one key, 256 bytes).
// A bijection of the low four bits of the key: the S^T operand reads (16 consecutive keys,
// one chunk) and the transposed V reads (8 consecutive keys, two adjacent chunks) then hit
// distinct LDS banks.
__device__ inline int pf_swz(int key) { return ((key & 7) << 1) | ((key >> 3) & 1); }

// s_waitcnt for vector memory only (expcnt and lgkmcnt left at their maxima).
template <int kVm>
__device__ inline void wait_vmcnt()
{
    __builtin_amdgcn_s_waitcnt((kVm & 15) | ((kVm >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Transposed LDS read: within each group of 16 lanes, if lane m points at four consecutive
// bf16 values (row m of a 16 x 4 tile), lane i receives the values at [4k + i/4][i%4],
// k = 0..3.
__device__ inline uint2 lds_read_tr16(const void* p)
{
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(const_cast<void*>(p)));
    return __builtin_bit_cast(uint2, v);
}

// Largest of three floats, NaN-propagating (v_maximum3_f32); the scores are never NaN on
// a valid row, and fmaxf would add a canonicalising instruction per input.
__device__ inline float max3f(float a, float b, float c)
{
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

static_assert(4 * kPfAcc * 4 * 64 == pa::kPrefillPartFloats, "prefill partial size differs from the workspace's");
static_assert(4 * 2 * 64 == pa::kPrefillPartLseFloats, "prefill partial LSE size differs from the workspace's");

// Cache-policy bits of a tile kernel's K / V copies: nt (2) for the 64- / 32-row chunk
// tiles, whose copies no other workgroup reads again.
template <bool kCascade, int kRG>
constexpr int kPfCopyAux = (!kCascade && kRG == 2) ? 2 : 0;

template <bool kCascade, int kRG>
using PfCopy = std::integral_constant<int, kPfCopyAux<kCascade, kRG>>;

// One 16-byte-per-lane LDS-DMA copy (global_load_lds_dwordx4) from per-lane addresses, for
// the one-launch mixed batch's fused chunk tiles, whose lanes may read the new rows or the
// pool; cache-policy bits aux as the tags say.
using CopyDefault = std::integral_constant<int, 0>;
using CopyStream = std::integral_constant<int, 2>;
__device__ inline void lds_copy16(const void* src, void* lds, CopyDefault)
{
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// The same copy through a buffer resource (buffer_load_dwordx4 ... lds): lane bytes
// off .. off + 15 of the `bytes` bytes at the wavefront-uniform address of pf_rsrc (a lane
// past them reads zeros).  The tiles stage their pool blocks this way: while a copy in the
// global form is in flight, the compiler cannot tell its completion apart from that of the
// LDS reads (it counts it as a flat access that may finish out of order) and waits for
// every outstanding LDS read before each product instead of only for the operands that
// product needs.
__device__ inline __amdgpu_buffer_rsrc_t pf_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ inline void lds_copy16(__amdgpu_buffer_rsrc_t rs, uint32_t off, void* lds, CopyDefault)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, 0);
}
__device__ inline void lds_copy16(__amdgpu_buffer_rsrc_t rs, uint32_t off, void* lds, CopyStream)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, 2);
}

template <int N>
struct BufSel {
    static constexpr int value = N;
};

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedValu = 0x2;
constexpr int kSchedMfma = 0x8;
constexpr int kSchedVmemRead = 0x20;
constexpr int kSchedDsRead = 0x100;

// exp2 of eight scores (a 32-key chunk of one row block) against the running maximum,
// packed as that chunk's P^T operand; returns their sum.  Chunk c's operand holds this
// lane's keys 32 c + 4 kslice + 0..3 and 32 c + 16 + 4 kslice + 0..3, i.e. x[8 c .. 8 c + 7].
__device__ __forceinline__ float pf_exp8(const float* x, float neg_m, float scale_log2, bf16x8& pb)
{
    float pe[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        pe[i] = fast_exp2(fmaf(x[i], scale_log2, neg_m));
    pb = __builtin_bit_cast(bf16x8, u32x4{pack_bf16(pe[0], pe[1]), pack_bf16(pe[2], pe[3]), pack_bf16(pe[4], pe[5]),
                                          pack_bf16(pe[6], pe[7])});
    return ((pe[0] + pe[1]) + (pe[2] + pe[3])) + ((pe[4] + pe[5]) + (pe[6] + pe[7]));
}

// Transposed V operand of 32-key chunk c: v_addr[db] is this lane's byte offset for dim
// block db; the chunk adds 8 KiB and its upper 16 keys another 4 KiB.
__device__ __forceinline__ void pf_read_v(const char* vt, const int (&v_addr)[8], int c, bf16x8 (&vop)[8])
{
#pragma unroll
    for (int db = 0; db < 8; ++db) {
        const uint2 lo = lds_read_tr16(vt + v_addr[db] + c * 8192);
        const uint2 hi = lds_read_tr16(vt + v_addr[db] + c * 8192 + 4096);
        vop[db] = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
    }
}

// FP8 tiles keep the codes in LDS: one 128-byte row per key, its eight 16-byte units
// permuted by pf_swz8(key), a bijection of the unit index that changes with key bits 1..4
// and not with key + 32 (so a 32-key chunk's read offsets hold for every chunk).  The K
// operand reads (16 keys of one unit) and the transposed V reads (eight keys, two units)
// then hit distinct banks.
__device__ inline int pf_swz8(int key) { return ((key >> 1) & 7) ^ ((key >> 4) & 1); }

// Transposed 8-bit LDS read: within each group of 16 lanes, if lane m points at eight
// consecutive bytes (row m of a 16 x 8 byte tile), lane i receives byte i % 8 of rows
// 2 j + i / 8, j = 0..7 (measured on the chip with an in-bounds probe).
__device__ inline u32x2 lds_read_tr8(const void* p)
{
    typedef int v2i __attribute__((ext_vector_type(2)));
    const v2i v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) v2i*)(const_cast<void*>(p)));
    return __builtin_bit_cast(u32x2, v);
}

// FP8 tile: the transposed V operand of 32-key chunk c as bf16 (the codes widened exactly).
// v_addr[db] points lane (kslice, m) at key 4 kslice + m / 2 (m / 2 < 4) or
// 16 + 4 kslice + m / 2 - 4 of the chunk, dims 16 db + 8 (m % 2) .. +8, so lane
// (kslice, i) receives dim 16 db + i of the same eight keys the bf16 operand holds; a
// chunk is 4 KiB of codes.
__device__ __forceinline__ void pf_read_v8(const char* vt, const int (&v_addr)[8], int c, bf16x8 (&vop)[8])
{
#pragma unroll
    for (int db = 0; db < 8; ++db)
        vop[db] = __builtin_bit_cast(bf16x8, e4m3x8_to_bf16(lds_read_tr8(vt + v_addr[db] + c * 4096)));
}

template <bool kV8>
__device__ __forceinline__ void pf_read_vx(const char* vt, const int (&v_addr)[8], int c, bf16x8 (&vop)[8])
{
    if constexpr (kV8)
        pf_read_v8(vt, v_addr, c, vop);
    else
        pf_read_v(vt, v_addr, c, vop);
}

// One 64-key half step of a prefill wavefront (two row blocks rb of 16 rows): S^T = K Q^T,
// the online softmax, O^T += V^T P^T.  The running maximum is raised lazily: a lane
// compares its own scores with the row's running maximum plus kRescaleSlack, and only
// when some lane's score passes it does the wavefront take the row maxima across its
// lanes and rescale O and the denominators; otherwise no cross-lane exchange is needed.
//
// Instruction order within the step (fixed with scheduling-group barriers): the S^T
// products go out interleaved with the transposed reads of V's first 32-key chunk; after
// the maxima and the rescale test come the first chunk's exponentials (both row blocks),
// the first chunk's PV products interleaved with the second chunk's V reads and
// exponentials, and the second chunk's PV products with the denominator sums.
// The matrix unit thus stays busy while the wavefront works through the softmax.
// kMask: the step holds keys past some row's position or past kv_hi.
//
// Tile shapes: kRB row blocks of 16 rows per wavefront and kKB key blocks of 16 keys per
// wavefront and step.  The full tile (kRB 2, kKB 4) runs the instruction order above; the
// smaller tiles (kKB 2: one 32-key chunk per wavefront and step) run the same arithmetic
// in program order.
template <int kRB, int kKB, bool kMask, bool kV8 = false>
__device__ __forceinline__ void pf_step(const bf16x8 (&kop)[kKB][4], const char* vt, const int (&v_addr)[8],
                                        const bf16x8 (&qop)[kRB][4], f32x4 (&oacc)[kRB][8], float (&m)[kRB],
                                        float (&lsum)[kRB], int key0, int kslice, const int (&qpos)[kRB], int kv_hi,
                                        float scale_log2)
{
    if constexpr (kKB == 2) {
        bf16x8 v0[8];
        pf_read_vx<kV8>(vt, v_addr, 0, v0);
        f32x4 sacc[kRB][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb) {
                sacc[rb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    sacc[rb][kb] =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[kb][ks], qop[rb][ks], sacc[rb][kb], 0, 0, 0);
            }
        // x[rb][4 kb + e] is the score of key key0 + 16 kb + 4 kslice + e for this lane's row
        float x[kRB][8];
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    x[rb][4 * kb + e] = sacc[rb][kb][e];
        if constexpr (kMask) {
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int key = key0 + 16 * (i >> 2) + 4 * kslice + (i & 3);
                    x[rb][i] = (key > qpos[rb] || key >= kv_hi) ? -INFINITY : x[rb][i];
                }
        }
        float lmax[kRB];
        bool raise = false;
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
            const float a = max3f(x[rb][0], x[rb][1], x[rb][2]);
            const float b = max3f(x[rb][3], x[rb][4], x[rb][5]);
            lmax[rb] = max3f(max3f(a, b, x[rb][6]), x[rb][7], -INFINITY) * scale_log2;
            raise = raise || lmax[rb] > m[rb] + kRescaleSlack;
        }
        if (__any(raise)) {
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb) {
                float t = fmaxf(lmax[rb], shfl_xor(lmax[rb], 16));
                t = fmaxf(t, shfl_xor(t, 32));
                if (t > m[rb] + kRescaleSlack) {
                    const float alpha = (m[rb] == -INFINITY) ? 0.f : fast_exp2(m[rb] - t);
                    m[rb] = t;
                    lsum[rb] *= alpha;
#pragma unroll
                    for (int db = 0; db < 8; ++db)
                        oacc[rb][db] *= alpha;
                }
            }
        }
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
            const float nm = (m[rb] == -INFINITY) ? 0.f : -m[rb];
            bf16x8 pb;
            lsum[rb] += pf_exp8(&x[rb][0], nm, scale_log2, pb);
#pragma unroll
            for (int db = 0; db < 8; ++db)
                oacc[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v0[db], pb, oacc[rb][db], 0, 0, 0);
        }
        return;
    } else {
    static_assert(kRB == 2 && kKB == 4, "the full tile: two row blocks and four key blocks per wavefront");
    bf16x8 v0[8];
    pf_read_vx<kV8>(vt, v_addr, 0, v0);
    // key block by key block, so that each K operand is dead once both row blocks used it
    f32x4 sacc[2][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            sacc[rb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                sacc[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[kb][ks], qop[rb][ks], sacc[rb][kb], 0, 0, 0);
        }
    // x[rb][4 kb + e] is the score of key key0 + 16 kb + 4 kslice + e for this lane's row
    float x[2][16];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                x[rb][4 * kb + e] = sacc[rb][kb][e];
    if constexpr (kMask) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = key0 + 16 * (i >> 2) + 4 * kslice + (i & 3);
                x[rb][i] = (key > qpos[rb] || key >= kv_hi) ? -INFINITY : x[rb][i];
            }
    }
    float lmax[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const float a = max3f(x[rb][0], x[rb][1], x[rb][2]);
        const float b = max3f(x[rb][3], x[rb][4], x[rb][5]);
        const float c = max3f(x[rb][6], x[rb][7], x[rb][8]);
        const float d = max3f(x[rb][9], x[rb][10], x[rb][11]);
        const float e = max3f(x[rb][12], x[rb][13], x[rb][14]);
        lmax[rb] = max3f(max3f(a, b, c), max3f(d, e, x[rb][15]), -INFINITY) * scale_log2;
    }
    const bool raise = lmax[0] > m[0] + kRescaleSlack || lmax[1] > m[1] + kRescaleSlack;
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 16, 0);     // K operand reads
    __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 9, 0);    // next step's copies
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
    if (__any(raise)) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            float t = fmaxf(lmax[rb], shfl_xor(lmax[rb], 16));
            t = fmaxf(t, shfl_xor(t, 32));
            if (t > m[rb] + kRescaleSlack) {
                const float alpha = (m[rb] == -INFINITY) ? 0.f : fast_exp2(m[rb] - t);
                m[rb] = t;
                lsum[rb] *= alpha;
#pragma unroll
                for (int db = 0; db < 8; ++db)
                    oacc[rb][db] *= alpha;
            }
        }
    }
    // with no visible key yet every score is -inf and any finite offset gives 0
    const float nm0 = (m[0] == -INFINITY) ? 0.f : -m[0];
    const float nm1 = (m[1] == -INFINITY) ? 0.f : -m[1];
    bf16x8 p00, p10, p01, p11;                                       // p<rb><chunk>
    float s0 = pf_exp8(&x[0][0], nm0, scale_log2, p00);
    float s1 = pf_exp8(&x[1][0], nm1, scale_log2, p10);
    bf16x8 v1[8];
    pf_read_vx<kV8>(vt, v_addr, 1, v1);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
        oacc[0][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v0[db], p00, oacc[0][db], 0, 0, 0);
        oacc[1][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v0[db], p10, oacc[1][db], 0, 0, 0);
    }
    s0 += pf_exp8(&x[0][8], nm0, scale_log2, p01);
    s1 += pf_exp8(&x[1][8], nm1, scale_log2, p11);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
        oacc[0][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v1[db], p01, oacc[0][db], 0, 0, 0);
        oacc[1][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v1[db], p11, oacc[1][db], 0, 0, 0);
    }
    lsum[0] += s0;
    lsum[1] += s1;
    __builtin_amdgcn_sched_group_barrier(kSchedValu, 24, 0);       // first chunk's exponentials
#pragma unroll
    for (int i = 0; i < 16; ++i) {                                   // with the second chunk's V reads
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, 2, 0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, 1, 0);
    }
    }
}

// The full tile's step in two halves, for the alternating schedule of prefill_body: the
// matrix half (PV of the previous step with its weights pw, then S^T = K Q^T of this step)
// and the vector half (masking, maxima, lazy rescale, exponentials and denominators, which
// leave the next PV's weights in pw).  Per output value the arithmetic and its order are
// those of pf_step: the same products accumulate in the same order and the softmax takes
// the same steps, so both schedules give the same bits.
template <bool kV8 = false>
__device__ __forceinline__ void pf_pv_full(const char* vt, const int (&v_addr)[8], const bf16x8 (&pw)[2][2],
                                           f32x4 (&oacc)[2][8])
{
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        bf16x8 v[8];
        pf_read_vx<kV8>(vt, v_addr, c, v);
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            oacc[0][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v[db], pw[0][c], oacc[0][db], 0, 0, 0);
            oacc[1][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v[db], pw[1][c], oacc[1][db], 0, 0, 0);
        }
    }
}

// k_addr: this lane's K operand offsets (a bf16 tile), or, as [2][4], those of an FP8
// tile's even and odd key blocks, whose codes are widened exactly to bf16 as they are read.
__device__ __forceinline__ bf16x8 pf_k_op(const char* kt, const int (&k_addr)[4], int kb, int ks)
{
    return *reinterpret_cast<const bf16x8*>(kt + k_addr[ks] + kb * 4096);
}
__device__ __forceinline__ bf16x8 pf_k_op(const char* kt, const int (&k_addr8)[2][4], int kb, int ks)
{
    return __builtin_bit_cast(bf16x8,
                              e4m3x8_to_bf16(*reinterpret_cast<const u32x2*>(kt + k_addr8[kb & 1][ks] + kb * 2048)));
}

template <class KAddr>
__device__ __forceinline__ void pf_qk_full(const char* kt, const KAddr& k_addr, const bf16x8 (&qop)[2][4],
                                           f32x4 (&sacc)[2][4])
{
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        bf16x8 kop[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            kop[ks] = pf_k_op(kt, k_addr, kb, ks);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            sacc[rb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                sacc[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[ks], qop[rb][ks], sacc[rb][kb], 0, 0, 0);
        }
    }
}

// Both products of the matrix half in one instruction stream: the 48 LDS operand reads
// (V's two 32-key chunks, then K's four 16-key blocks) go out eight ahead of the 64
// products that use them, one per product, so that few operands are live at a time.
// An FP8 tile (kV8, k_addr as [2][4]) reads half the bytes: 16 V and 16 K operand reads,
// each widened by four conversions, ahead of the 64 products.
template <bool kV8 = false, class KAddr>
__device__ __forceinline__ void pf_matrix_full(const char* vt, const int (&v_addr)[8], const bf16x8 (&pw)[2][2],
                                               f32x4 (&oacc)[2][8], const char* kt, const KAddr& k_addr,
                                               const bf16x8 (&qop)[2][4], f32x4 (&sacc)[2][4])
{
    pf_pv_full<kV8>(vt, v_addr, pw, oacc);
    pf_qk_full(kt, k_addr, qop, sacc);
    if constexpr (kV8) {
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
        for (int i = 0; i < 28; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 36, 0);
    } else {
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8, 0);
#pragma unroll
        for (int i = 0; i < 40; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 24, 0);
    }
}

template <bool kMask>
__device__ __forceinline__ void pf_softmax_full(const f32x4 (&sacc)[2][4], f32x4 (&oacc)[2][8], float (&m)[2],
                                                float (&lsum)[2], bf16x8 (&pw)[2][2], int key0, int kslice,
                                                const int (&qpos)[2], int kv_hi, float scale_log2)
{
    float x[2][16];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                x[rb][4 * kb + e] = sacc[rb][kb][e];
    if constexpr (kMask) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = key0 + 16 * (i >> 2) + 4 * kslice + (i & 3);
                x[rb][i] = (key > qpos[rb] || key >= kv_hi) ? -INFINITY : x[rb][i];
            }
    }
    float lmax[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const float a = max3f(x[rb][0], x[rb][1], x[rb][2]);
        const float b = max3f(x[rb][3], x[rb][4], x[rb][5]);
        const float c = max3f(x[rb][6], x[rb][7], x[rb][8]);
        const float d = max3f(x[rb][9], x[rb][10], x[rb][11]);
        const float e = max3f(x[rb][12], x[rb][13], x[rb][14]);
        lmax[rb] = max3f(max3f(a, b, c), max3f(d, e, x[rb][15]), -INFINITY) * scale_log2;
    }
    const bool raise = lmax[0] > m[0] + kRescaleSlack || lmax[1] > m[1] + kRescaleSlack;
    if (__any(raise)) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            float t = fmaxf(lmax[rb], shfl_xor(lmax[rb], 16));
            t = fmaxf(t, shfl_xor(t, 32));
            if (t > m[rb] + kRescaleSlack) {
                const float alpha = (m[rb] == -INFINITY) ? 0.f : fast_exp2(m[rb] - t);
                m[rb] = t;
                lsum[rb] *= alpha;
#pragma unroll
                for (int db = 0; db < 8; ++db)
                    oacc[rb][db] *= alpha;
            }
        }
    }
    const float nm0 = (m[0] == -INFINITY) ? 0.f : -m[0];
    const float nm1 = (m[1] == -INFINITY) ? 0.f : -m[1];
    float s0 = pf_exp8(&x[0][0], nm0, scale_log2, pw[0][0]);
    float s1 = pf_exp8(&x[1][0], nm1, scale_log2, pw[1][0]);
    s0 += pf_exp8(&x[0][8], nm0, scale_log2, pw[0][1]);
    s1 += pf_exp8(&x[1][8], nm1, scale_log2, pw[1][1]);
    lsum[0] += s0;
    lsum[1] += s1;
}

// Workgroup of eight wavefronts per (prefill row, 32-token query tile, KV head, key split).
// The tile's 128 MFMA rows are (token, head) pairs, row = 4 * token + head, so the four
// query heads of a group share every K / V tile.  Wavefront w owns rows 32 (w % 4) .. +32
// and keys 64 (w / 4) .. +64 of every 128-key step; the two wavefronts that share a SIMD
// hold the same rows.  Their two key halves are merged through LDS at the end, lane by
// lane, by the log-sum-exp rule.
//
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Round two floats to binary16 (nearest even) and pack them, low half first.
__device__ inline uint32_t pack_f16(float a, float b)
{
    f16x2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ f32x4 mfma_f16(const bf16x8& a, const bf16x8& b, const f32x4& c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                  0);
}

// pf_step over a q8_0 pool.  The staged K tile holds the codes as binary16 integers
// (exact), the staged V tile the values code x scale rounded to binary16, Q is binary16,
// and the K scales of the step's keys sit in LDS as floats, [group][key] (ksc).  S^T is
// formed one 32-dim group (one k-slice of the product) at a time: the group's codes times
// Q, exact products summed in fp32, then weighted by each key's scale of that group, so
// the scores carry no rounding of the stored values.  PV takes the softmax weights rounded
// to binary16 against the staged V values, as the bf16 tile takes them in bf16.  The
// softmax statistics are those of pf_step (same lazy rescaling; the denominators are
// summed from the unrounded weights).
template <bool kMask>
__device__ __forceinline__ void pf_step_q8(const bf16x8 (&kop)[4][4], const char* vt, const int (&v_addr)[8],
                                           const float* ksc, const bf16x8 (&qop)[2][4],
                                           f32x4 (&oacc)[2][8], float (&m)[2], float (&lsum)[2], int key0, int kh,
                                           int kslice, const int (&qpos)[2], int kv_hi, float scale_log2)
{
    const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
    // x[rb][4 kb + e] is the score of key key0 + 16 kb + 4 kslice + e for this lane's row
    float x[2][16];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        f32x4 dk[4];
#pragma unroll
        for (int g = 0; g < 4; ++g)
            dk[g] = *reinterpret_cast<const f32x4*>(ksc + g * kPfKeys + 64 * kh + 16 * kb + 4 * kslice);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            f32x4 acc = zero;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 part = mfma_f16(kop[kb][g], qop[rb][g], zero);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[e] = fmaf(part[e], dk[g][e], acc[e]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
                x[rb][4 * kb + e] = acc[e];
        }
    }
    if constexpr (kMask) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = key0 + 16 * (i >> 2) + 4 * kslice + (i & 3);
                x[rb][i] = (key > qpos[rb] || key >= kv_hi) ? -INFINITY : x[rb][i];
            }
    }
    float lmax[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        float t = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            t = fmaxf(t, x[rb][i]);
        lmax[rb] = t * scale_log2;
    }
    const bool raise = lmax[0] > m[0] + kRescaleSlack || lmax[1] > m[1] + kRescaleSlack;
    if (__any(raise)) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            float t = fmaxf(lmax[rb], shfl_xor(lmax[rb], 16));
            t = fmaxf(t, shfl_xor(t, 32));
            if (t > m[rb] + kRescaleSlack) {
                const float alpha = (m[rb] == -INFINITY) ? 0.f : fast_exp2(m[rb] - t);
                m[rb] = t;
                lsum[rb] *= alpha;
#pragma unroll
                for (int db = 0; db < 8; ++db)
                    oacc[rb][db] *= alpha;
            }
        }
    }
    const float nm[2] = {(m[0] == -INFINITY) ? 0.f : -m[0], (m[1] == -INFINITY) ? 0.f : -m[1]};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        bf16x8 vop[8];
        pf_read_v(vt, v_addr, c, vop);
        // this lane's keys of chunk c: 32 c + 4 kslice + 0..3, then 32 c + 16 + 4 kslice + 0..3
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            float pe[8];
            float sum = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                pe[i] = fast_exp2(fmaf(x[rb][8 * c + i], scale_log2, nm[rb]));
                sum += pe[i];
            }
            lsum[rb] += sum;
            const bf16x8 pg = __builtin_bit_cast(bf16x8, u32x4{pack_f16(pe[0], pe[1]), pack_f16(pe[2], pe[3]),
                                                               pack_f16(pe[4], pe[5]), pack_f16(pe[6], pe[7])});
#pragma unroll
            for (int db = 0; db < 8; ++db)
                oacc[rb][db] = mfma_f16(vop[db], pg, oacc[rb][db]);
        }
    }
}

// Key splits: the tile's causal key range, ceil(kv_hi / 128) steps, is cut into `splits`
// contiguous step ranges, one workgroup each.  With one split the workgroup writes the
// output; otherwise each writes its normalised partial and log2-sum-exp to the workspace
// with agent-scope stores and counts itself in, and the last one merges all partials.
//
// K / V staging: all eight wavefronts copy one step's eight blocks (one block each, K and
// V, 8 KiB) straight from the pool into LDS with global_load_lds_dwordx4, double-buffered
// in two named buffer pairs: the copy of step s + 1 is issued right after the K operand
// reads of step s, and since it targets the other pair, the transposed V reads of step s
// need not wait for it.  Slots past kv_len are filled from a valid slot of the same
// block, so every staged value is finite.
//
// MFMA v_mfma_f32_16x16x32_bf16: lane l supplies A[l%16][k-slice l/16] and
// B[k-slice l/16][l%16] (8 bf16 each) and receives D[4*(l/16) + e][l%16], e = 0..3.
//   S^T (keys x rows) = K (keys x dims) . Q^T (dims x rows)          contraction over dims
//   O^T (dims x rows) += V^T (dims x keys) . P^T (keys x rows)       contraction over keys
// Each lane's S^T values all belong to one row, so softmax statistics and the rescaling of
// O^T stay lane-local except for one exchange across the four k-slices.  In PV lane l's
// eight keys of chunk c are {4j..4j+3} and {16+4j..16+4j+3} (j = l/16) of the chunk:
// exactly S^T values it holds; the V^T operand is read with the same key order by two
// transposed LDS reads, and a contraction does not care how its index is permuted.
//
// q8_0 pool (kQ8): the copies go through registers instead.  Lane l of wavefront w loads
// the 32 codes and the scale of group l % 4 of token l / 4 of its block (K and V) when the
// step is staged; right before the next barrier it writes the K codes as binary16 integers
// (exact) and the V values code x scale rounded to binary16 to the same LDS places the
// bf16 copies use, and the K scale as a float to a [group][key] table beside the tiles.
// The products then run on binary16 operands (Q converted once, exact for bf16 values
// inside the binary16 range), see pf_step_q8.
// a or b, chosen at compile time (the two may differ in type)
template <bool kFirst, class A, class B>
__device__ __forceinline__ constexpr const auto& pf_pick(const A& a, const B& b)
{
    if constexpr (kFirst)
        return a;
    else
        return b;
}

template <bool kCascade, bool kFused = false, bool kQ8 = false, int kRG = 4, int kRB = 2, bool kFp8 = false>
__device__ __attribute__((always_inline)) inline void prefill_body(const PrefillParams& p, const DecodeParams& dp,
                                                                   int bid)
{
    static_assert(!(kFp8 && kQ8), "one pool format");
    // Quantised pools: a step's chunk rows are encoded into the pool by a launch of their own
    // first (encoding inside the tile raised its register spills in the step loop).
    static_assert(!(kFused && (kQ8 || kFp8)), "quantised pools: chunk rows are appended before the tiles");
    // Only the one-launch mixed batch fuses the append into its (full) chunk tiles; the
    // separate tile launches read rows appended by a short launch of their own.
    static_assert(!kFused || (kRG == 4 && !kCascade), "fused append: full chunk tiles of the one-launch form");
    // Tile shape: kRG row groups of kRB row blocks (16 MFMA rows each) and kNKP = 8 / kRG
    // key parts of kKPW keys of every 128-key step, one wavefront per (row group, key part).
    static_assert((kRG == 4 && kRB == 2) || (kRG == 2 && (kRB == 2 || kRB == 1)), "tile shapes: 4 x 2, 2 x 2, 2 x 1");
    static_assert(!kQ8 || (kRG == 4 && kRB == 2), "q8_0 pools run the full tile");
    constexpr int kNKP = kPfWaves / kRG;              // key parts
    constexpr int kKPW = kPfKeys / kNKP;              // keys per wavefront and step (64 or 32)
    constexpr int kKB = kKPW / 16;                    // 16-key blocks per wavefront and step
    constexpr int kRows = kRG * 16 * kRB;             // MFMA rows of the tile: 128, 64 or 32
    constexpr int kTileTok = kRows / kGroup;          // chunk tokens of the tile: 32, 16 or 8
    __shared__ __attribute__((aligned(1024))) u32x4 k_tile0[kTileChunks];
    __shared__ __attribute__((aligned(1024))) u32x4 v_tile0[kTileChunks];
    __shared__ __attribute__((aligned(1024))) u32x4 k_tile1[kTileChunks];
    __shared__ __attribute__((aligned(1024))) u32x4 v_tile1[kTileChunks];
    __shared__ int last_lds;
    // q8_0: K scales of the staged keys, [buffer pair][group][key]
    __shared__ __attribute__((aligned(16))) float q8_sc[kQ8 ? 2 * 4 * kPfKeys : 4];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int rg = wave % kRG, kh = wave / kRG;     // row group, key part
    const int vkv = bid % p.num_vheads;
    const int rest = bid / p.num_vheads;
    const int split = rest % p.splits;
    const int tile = rest / p.splits;
    const HeadSlice hs = head_slice(vkv, p.num_q_heads, p.num_kv_heads);
    const int kvh = hs.kvh, head0 = hs.head0;
    int r, qt, q0, qlen, kvlen, ctx, nblk_row, kv_hi;
    bool bad_row;
    int grp_first = 0, grp_count = 0;
    if constexpr (kCascade) {
        // the group's requests are rows r .. r + grp_count - 1, each one decode token; the
        // keys are the first group_blocks blocks of their (shared) tables, all of them
        // before every one of the group's queries
        grp_first = p.group_first[tile];
        grp_count = p.group_count[tile];
        r = grp_first;
        qt = q0 = qlen = ctx = 0;
        nblk_row = p.group_blocks[tile];
        kvlen = nblk_row * kBlock;
        bad_row = nblk_row < 1 || nblk_row > p.max_blocks || grp_count < 1 || grp_count > PA_MAX_PREFIX_GROUP_REQS;
        kv_hi = bad_row ? 0 : kvlen;
    } else {
        int pr = 0;
        while (pr + 1 < p.num_prefill_rows && p.tile_start[pr + 1] <= tile)
            ++pr;
        r = p.prefill_req[pr];
        qt = tile - p.tile_start[pr];
        q0 = p.qo_indptr[r];
        qlen = p.qo_indptr[r + 1] - q0;
        kvlen = p.kv_len[r];
        if (qt * kTileTok >= qlen)              // the same for every split of the tile
            return;
        ctx = kvlen - qlen;                     // tokens before this chunk
        nblk_row = (kvlen + kBlock - 1) / kBlock;
        bad_row = qlen < 2 || ctx < 0 || nblk_row > p.max_blocks;
        // keys any token of this tile can see: 0 .. ctx + last token of the tile
        kv_hi = bad_row ? 0 : min(kvlen, ctx + min(qlen, (qt + 1) * kTileTok));
    }
    // Row groups with no valid row skip the products (their wavefronts still copy their
    // block of every step and meet every barrier).
    const int valid_rows = kCascade ? 4 * grp_count : min(kRows, 4 * (qlen - qt * kTileTok));
    const bool active = 16 * kRB * rg < valid_rows;
    const int nsteps_tile = (kv_hi + kPfKeys - 1) / kPfKeys;
    const int s_begin = split * nsteps_tile / p.splits;
    const int nsteps = (split + 1) * nsteps_tile / p.splits - s_begin;

    const int row16 = lane & 15, kslice = lane >> 4;
    // this lane's rows (row blocks rb = 0 .. kRB - 1)
    int qpos[kRB];
    bf16x8 qop[kRB][4];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
        const int rho = 16 * kRB * rg + 16 * rb + row16;
        int qidx;
        bool ok;
        if constexpr (kCascade) {
            const int slot = rho >> 2;          // the group's request slot
            ok = slot < grp_count;
            qidx = ok ? p.qo_indptr[grp_first + slot] : 0;
            qpos[rb] = INT_MAX;                 // every shared key precedes the query
        } else {
            const int tl = qt * kTileTok + (rho >> 2);
            qpos[rb] = ctx + tl;
            ok = tl < qlen;
            qidx = q0 + tl;
        }
        ok = ok && (rho & 3) < hs.heads;       // empty head slots hold zero queries
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (ok)
                v = *reinterpret_cast<const u32x4*>(
                    p.q + ((int64_t)qidx * p.num_q_heads + head0 + (rho & 3)) * kHeadDim + ks * 32 + kslice * 8);
            if constexpr (kQ8) {
                // toward zero, as the decode rows convert Q: exact inside the binary16
                // range, and a magnitude past 65504 saturates instead of becoming inf
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    v[j] = pack_half_rtz(bf16_lo(v[j]), bf16_hi(v[j]));
            }
            qop[rb][ks] = __builtin_bit_cast(bf16x8, v);
        }
    }

    const int64_t tile_elems = (int64_t)kBlock * kHeadDim;
    const int64_t kvh_off = (int64_t)kvh * tile_elems;
    const int64_t blk_stride = (int64_t)p.num_kv_heads * tile_elems;
    const int32_t* bt = p.block_tables + (int64_t)r * p.max_blocks;
    bool bad = bad_row;

    // Table entry of block `wave` of step s (the row's first block if the step runs past
    // the row).  It is range-checked only where it is used, one step later, so that the
    // load does not hold up the copies issued just before it.
    auto table_entry = [&](int s) __attribute__((always_inline)) {
        const int b = s * (kPfKeys / kBlock) + wave;
        return bt[b < nblk_row ? b : 0];
    };
    auto checked = [&](int id) __attribute__((always_inline)) {
        if (id < 0 || id >= p.num_blocks) {
            bad = true;
            id = 0;
        }
        return id;
    };
    // Wavefront w copies block w of step s: 16 keys = four 1 KiB LDS rows-of-four, for K
    // and V.  Copy i of lane l moves 16 bytes of token 4 i + l / 16 of the block (element
    // offset cp_off[i]); in the row's last step, slots past kv_len take token 0's bytes
    // (cp_tail[i]), so that every staged value is finite.
    int cp_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tok = 4 * i + (lane >> 4);
        const int chunk = (lane & 15) ^ pf_swz(tok);      // pf_swz sees only the key's low four bits
        cp_off[i] = tok * kHeadDim + chunk * 8;            // token 0's offset is cp_off[i] % kHeadDim
    }
    // q8_0 copies in flight: this lane's 32 K and 32 V codes (token q8_tok, group q8_grp of
    // the wavefront's block) and the two scales
    const int q8_tok = lane >> 2, q8_grp = lane & 3;
    u32x4 q8k[2], q8v[2];
    uint32_t q8ks = 0, q8vs = 0;
    // The copies of a 64- / 32-row chunk tile (chosen only when every chunk row fits one
    // tile, so each row's keys are read by its own workgroups and nobody else) carry the
    // nontemporal hint, as the decode kernel's loads do: 16 rows x 8 new tokens at 8,200
    // context took 91 against 102 us with it.  The 128-row tiles of a long chunk share
    // every K / V step with the chunk's other query tiles through L2 and keep the default
    // policy (with the hint the 512-token chunk at 4096 took 60 against 55 us); so do the
    // shared-prefix tiles, read once per KV head as well, which measured slower with the
    // hint for small groups (16 rows sharing 96 blocks: 44 against 30 us).
    auto copy_load = [&](const auto* ptr) __attribute__((always_inline)) {
        if constexpr (kPfCopyAux<kCascade, kRG> != 0)
            return __builtin_nontemporal_load(ptr);
        else
            return *ptr;
    };
    auto stage = [&](auto sel, int s, int id) __attribute__((always_inline)) {
        const int valid = kvlen - (s * kPfKeys + 16 * wave);   // tokens of this block inside the row
        if constexpr (kQ8) {
            // slots past kv_len read token 0 of the block, so that every staged value is finite
            const int t = q8_tok < valid ? q8_tok : 0;
            const uint8_t* kt = reinterpret_cast<const uint8_t*>(p.k_pool) +
                                ((int64_t)id * p.num_kv_heads + kvh) * (2 * pa::kQ8TileBytes);
            const uint8_t* vt = kt + pa::kQ8TileBytes;
            const int co = t * kHeadDim + q8_grp * pa::kQ8Group;
            q8k[0] = copy_load(reinterpret_cast<const u32x4*>(kt + co));
            q8k[1] = copy_load(reinterpret_cast<const u32x4*>(kt + co + 16));
            q8v[0] = copy_load(reinterpret_cast<const u32x4*>(vt + co));
            q8v[1] = copy_load(reinterpret_cast<const u32x4*>(vt + co + 16));
            const int so = pa::kQ8CodeBytes + 2 * (t * (kHeadDim / pa::kQ8Group) + q8_grp);
            q8ks = *reinterpret_cast<const uint16_t*>(kt + so);
            q8vs = *reinterpret_cast<const uint16_t*>(vt + so);
            return;
        }
        if constexpr (kFp8) {
            // the codes go to LDS as they are: wavefront w's block is keys 16 w .. 16 w + 15
            // of the step, two 1 KiB copies per pool; lane l of copy i moves 16 bytes (unit
            // l % 8 of LDS row 16 w + 8 i + l / 8, i.e. unit (l % 8) ^ swz8 of the token's
            // row); slots past kv_len take token 0's bytes
            u32x4* kd = decltype(sel)::value == 0 ? k_tile0 : k_tile1;
            u32x4* vd = decltype(sel)::value == 0 ? v_tile0 : v_tile1;
            const int64_t base = (int64_t)id * blk_stride + kvh_off;   // bytes in an FP8 pool
            const auto kr = pf_rsrc(reinterpret_cast<const uint8_t*>(p.k_pool) + base, kBlock * kHeadDim);
            const auto vr = pf_rsrc(reinterpret_cast<const uint8_t*>(p.v_pool) + base, kBlock * kHeadDim);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int tok = 8 * i + (lane >> 3);
                const int off = (tok < valid ? tok : 0) * kHeadDim + (((lane & 7) ^ pf_swz8(16 * wave + tok)) << 4);
                lds_copy16(kr, off, reinterpret_cast<char*>(kd) + (16 * wave + 8 * i) * kHeadDim, PfCopy<kCascade, kRG>{});
                lds_copy16(vr, off, reinterpret_cast<char*>(vd) + (16 * wave + 8 * i) * kHeadDim, PfCopy<kCascade, kRG>{});
            }
            return;
        }
        u32x4* kd = decltype(sel)::value == 0 ? k_tile0 : k_tile1;
        u32x4* vd = decltype(sel)::value == 0 ? v_tile0 : v_tile1;
        const int64_t base = (int64_t)id * blk_stride + kvh_off;
        if constexpr (kFused) {
            // A block that reaches this chunk takes the chunk's positions from the new rows
            // (past kv_len: the chunk's last token, so that every staged value is finite).
            // The test is the same for the whole wavefront, and other blocks take the plain
            // copies below.
            if (s * kPfKeys + 16 * wave + kBlock > ctx) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int pos = s * kPfKeys + 16 * wave + 4 * i + (lane >> 4);
                    const int off = (4 * i + (lane >> 4)) < valid ? cp_off[i] : (cp_off[i] & (kHeadDim - 1));
                    const int64_t src = ((int64_t)(q0 + min(pos, kvlen - 1) - ctx) * p.num_kv_heads + kvh) * kHeadDim +
                                        (cp_off[i] & (kHeadDim - 1));
                    const uint16_t* ks = pos >= ctx ? p.k_new + src : p.k_pool + base + off;
                    const uint16_t* vs = pos >= ctx ? p.v_new + src : p.v_pool + base + off;
                    lds_copy16(ks, &kd[(16 * wave + 4 * i) * 16], PfCopy<kCascade, kRG>{});
                    lds_copy16(vs, &vd[(16 * wave + 4 * i) * 16], PfCopy<kCascade, kRG>{});
                }
                return;
            }
        }
        const auto kr = pf_rsrc(p.k_pool + base, kBlock * kHeadDim * 2);
        const auto vr = pf_rsrc(p.v_pool + base, kBlock * kHeadDim * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int off = (4 * i + (lane >> 4)) < valid ? cp_off[i] : (cp_off[i] & (kHeadDim - 1));
            lds_copy16(kr, 2 * off, &kd[(16 * wave + 4 * i) * 16], PfCopy<kCascade, kRG>{});
            lds_copy16(vr, 2 * off, &vd[(16 * wave + 4 * i) * 16], PfCopy<kCascade, kRG>{});
        }
    };
    // The copies of one pool (K or V) of step s into buffer `sel` of that pool, as `stage`
    // makes them for both; the alternating schedule stages K one step ahead of V.
    auto stage_pool = [&](auto which, auto sel, int s, int id) __attribute__((always_inline)) {
        constexpr bool kV = decltype(which)::value;
        u32x4* dst = kV ? (decltype(sel)::value == 0 ? v_tile0 : v_tile1)
                        : (decltype(sel)::value == 0 ? k_tile0 : k_tile1);
        if constexpr (kFp8) {
            // the codes of one pool, as `stage` copies them
            const int valid = kvlen - (s * kPfKeys + 16 * wave);
            const int64_t base = (int64_t)id * blk_stride + kvh_off;   // bytes in an FP8 pool
            const auto rs = pf_rsrc(reinterpret_cast<const uint8_t*>(kV ? p.v_pool : p.k_pool) + base, kBlock * kHeadDim);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int tok = 8 * i + (lane >> 3);
                const int off = (tok < valid ? tok : 0) * kHeadDim + (((lane & 7) ^ pf_swz8(16 * wave + tok)) << 4);
                lds_copy16(rs, off, reinterpret_cast<char*>(dst) + (16 * wave + 8 * i) * kHeadDim, PfCopy<kCascade, kRG>{});
            }
            return;
        }
        const uint16_t* pool = kV ? p.v_pool : p.k_pool;
        const int valid = kvlen - (s * kPfKeys + 16 * wave);
        const int64_t base = (int64_t)id * blk_stride + kvh_off;
        if constexpr (kFused) {
            if (s * kPfKeys + 16 * wave + kBlock > ctx) {
                const uint16_t* fresh = kV ? p.v_new : p.k_new;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int pos = s * kPfKeys + 16 * wave + 4 * i + (lane >> 4);
                    const int off = (4 * i + (lane >> 4)) < valid ? cp_off[i] : (cp_off[i] & (kHeadDim - 1));
                    const int64_t src = ((int64_t)(q0 + min(pos, kvlen - 1) - ctx) * p.num_kv_heads + kvh) * kHeadDim +
                                        (cp_off[i] & (kHeadDim - 1));
                    lds_copy16(pos >= ctx ? fresh + src : pool + base + off, &dst[(16 * wave + 4 * i) * 16], PfCopy<kCascade, kRG>{});
                }
                return;
            }
        }
        const auto rs = pf_rsrc(pool + base, kBlock * kHeadDim * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int off = (4 * i + (lane >> 4)) < valid ? cp_off[i] : (cp_off[i] & (kHeadDim - 1));
            lds_copy16(rs, 2 * off, &dst[(16 * wave + 4 * i) * 16], PfCopy<kCascade, kRG>{});
        }
    };
    // q8_0: the copies staged one step ago into buffer pair `sel` (whose previous contents
    // every wavefront finished reading before the last barrier)
    auto finish_q8 = [&](auto sel) __attribute__((always_inline)) {
        if constexpr (kQ8) {
            constexpr int B = decltype(sel)::value;
            u32x4* kd = B == 0 ? k_tile0 : k_tile1;
            u32x4* vd = B == 0 ? v_tile0 : v_tile1;
            wait_vmcnt<0>();
            const f16x2 bias = {(_Float16)kQ8Bias, (_Float16)kQ8Bias};
            // codes 2 i, 2 i + 1 of word w as binary16 integers: (1152 + code) - 1152, exact
            auto code2 = [&](uint32_t w, int i) __attribute__((always_inline)) {
                const uint32_t c = q8_to_half2(w, w, i ? 0x0c030c02u : 0x0c010c00u);
                return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, c) - bias);
            };
            // V values: code x scale, one binary16 product rounded to nearest
            const _Float16 dvh = __builtin_bit_cast(_Float16, (uint16_t)q8vs);
            const f16x2 dv2 = {dvh, dvh};
            auto value2 = [&](uint32_t w, int i) __attribute__((always_inline)) {
                return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, code2(w, i)) * dv2);
            };
            const int row = (16 * wave + q8_tok) * 16;
#pragma unroll
            for (int j = 0; j < 4; ++j) {                  // chunk 4 q8_grp + j: dims 8 j .. 8 j + 7 of the group
                const uint32_t k0 = q8k[j >> 1][2 * (j & 1)], k1 = q8k[j >> 1][2 * (j & 1) + 1];
                const uint32_t v0 = q8v[j >> 1][2 * (j & 1)], v1 = q8v[j >> 1][2 * (j & 1) + 1];
                const int slot = (4 * q8_grp + j) ^ pf_swz(q8_tok);
                kd[row + slot] = u32x4{code2(k0, 0), code2(k0, 1), code2(k1, 0), code2(k1, 1)};
                vd[row + slot] = u32x4{value2(v0, 0), value2(v0, 1), value2(v1, 0), value2(v1, 1)};
            }
            float* sc = q8_sc + B * (4 * kPfKeys) + q8_grp * kPfKeys + 16 * wave + q8_tok;
            sc[0] = (float)__builtin_bit_cast(_Float16, (uint16_t)q8ks);
        }
    };
    // LDS byte offsets of this lane's operand reads within a K or V tile.  K: key
    // kKPW kh + 16 kb + row16, chunk 4 ks + kslice (kb adds 4 KiB).  V: source lane i16 of
    // group kslice points at key 4 kslice + i16/4 (+16) of chunk c, dims 16 db + 4 (i16 % 4)
    // .. +4, and lane (kslice, i16) receives dim 16 db + i16 of keys 4 kslice + 0..3 (+16)
    // (c adds 8 KiB, +16 keys 4 KiB).  kKPW kh is a multiple of 32, so the swizzle, which
    // sees a key's low four bits, is the same for every key part.
    int k_addr[4], v_addr[8];
    int k_addr8[2][4];          // FP8 tiles: K operand offsets for even and odd key blocks kb
    if constexpr (kFp8) {
        // K: key kKPW kh + 16 kb + row16, dims 32 ks + 8 kslice .. +8 = unit 2 ks + kslice / 2,
        // half kslice % 2 of that unit (kb adds 2 KiB; its parity flips the swizzle's bit 4)
#pragma unroll
        for (int par = 0; par < 2; ++par)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                k_addr8[par][ks] = (kKPW * kh + row16) * kHeadDim +
                                   (((2 * ks + (kslice >> 1)) ^ pf_swz8(16 * par + row16)) << 4) + ((kslice & 1) << 3);
        const int mm = lane & 15, j = mm >> 1;
        const int key = kKPW * kh + (j < 4 ? 4 * kslice + j : 16 + 4 * kslice + j - 4);
#pragma unroll
        for (int db = 0; db < 8; ++db)
            v_addr[db] = key * kHeadDim + ((db ^ pf_swz8(key)) << 4) + ((mm & 1) << 3);
    } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            k_addr[ks] = (kKPW * kh + row16) * 256 + (((ks * 4 + kslice) ^ pf_swz(row16)) << 4);
        const int i16 = lane & 15;
        const int k_lo = kKPW * kh + 4 * kslice + (i16 >> 2);
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const int cc = 2 * db + ((i16 & 3) >> 1);
            v_addr[db] = k_lo * 256 + ((cc ^ pf_swz(k_lo)) << 4) + ((i16 & 1) << 3);
        }
    }

    f32x4 oacc[kRB][8];
    float m[kRB], lsum[kRB];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
        m[rb] = -INFINITY;
        lsum[rb] = 0.f;
#pragma unroll
        for (int db = 0; db < 8; ++db)
            oacc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // Step order: the steps no row of the tile needs masked first, rotated so that
    // workgroups of neighbouring query tiles start one step apart (at any time each K / V
    // step is then fetched from memory by one workgroup and found in the XCD's L2 by the
    // others: all tiles of one KV head run on one XCD), then the diagonal and tail steps.
    // smallest query position of the tile (a shared prefix masks only past its end)
    const int qmin = kCascade ? kv_hi - 1 : ctx + qt * kTileTok;
    const int s_masked = max(s_begin, min(s_begin + nsteps, (qmin + 1) / kPfKeys));
    const int n_plain = s_masked - s_begin;
    const int rot = (!kCascade && n_plain > 0) ? qt % n_plain : 0;
    auto step_at = [&](int i) __attribute__((always_inline)) {
        i = min(i, nsteps - 1);
        return i >= n_plain ? s_begin + i : s_begin + (i + rot < n_plain ? i + rot : i + rot - n_plain);
    };
    // The full tile on bf16 and FP8 pools runs the alternating schedule (see below); the
    // other shapes and the q8_0 pool run one step at a time.
    constexpr bool kAlternate = !kQ8 && kRG == 4 && kRB == 2;
    int next_id = 0, cur_id = 0;
    if (nsteps > 0) {
        cur_id = checked(table_entry(step_at(0)));
        if constexpr (kAlternate)
            stage_pool(std::false_type{}, BufSel<0>{}, step_at(0), cur_id);
        else
            stage(BufSel<0>{}, step_at(0), cur_id);
        next_id = table_entry(step_at(1));
    }

    auto do_step = [&](auto sel, auto msk, int it) __attribute__((always_inline)) {
        constexpr int B = decltype(sel)::value;
        const char* kt = reinterpret_cast<const char*>(B == 0 ? k_tile0 : k_tile1);
        const char* vt = reinterpret_cast<const char*>(B == 0 ? v_tile0 : v_tile1);
        const int s = step_at(it);
        finish_q8(sel);
        // This wavefront's copies of this step have landed and its LDS reads of the previous
        // step have returned; after the barrier everyone's have.  The memory clobber keeps
        // the compiler from moving any memory access across; register-only work of the
        // previous step may still drift past it.
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (!active) {
            int id = next_id;
            asm volatile("" : "+v"(id));
            stage(BufSel<B ^ 1>{}, step_at(it + 1), checked(__builtin_amdgcn_readfirstlane(id)));
            next_id = table_entry(step_at(it + 2));
            return;
        }
        bf16x8 kop[kKB][4];
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                if constexpr (kFp8)
                    kop[kb][ks] = __builtin_bit_cast(
                        bf16x8, e4m3x8_to_bf16(*reinterpret_cast<const u32x2*>(kt + k_addr8[kb & 1][ks] + kb * 2048)));
                else
                    kop[kb][ks] = *reinterpret_cast<const bf16x8*>(kt + k_addr[ks] + kb * 4096);
            }
        // Next step's copy (the last step repeats its own; nothing reads that copy) into
        // the other buffer pair, which every wavefront finished reading in the previous
        // step.  Its table entry was loaded one step ago and has landed; the empty asm
        // keeps it in a vector register until here, since moving it to a scalar one at
        // its load would make the load wait for all of this wavefront's copies.
        {
            int id = next_id;
            asm volatile("" : "+v"(id));
            stage(BufSel<B ^ 1>{}, step_at(it + 1), checked(__builtin_amdgcn_readfirstlane(id)));
            next_id = table_entry(step_at(it + 2));
        }
        if constexpr (kQ8) {
            const float* ksc = q8_sc + B * (4 * kPfKeys);
            pf_step_q8<decltype(msk)::value>(kop, vt, v_addr, ksc, qop, oacc, m, lsum,
                                             s * kPfKeys + 64 * kh, kh, kslice, qpos, kv_hi, p.scale_log2);
        } else {
            pf_step<kRB, kKB, decltype(msk)::value, kFp8>(kop, vt, v_addr, qop, oacc, m, lsum, s * kPfKeys + kKPW * kh,
                                                    kslice, qpos, kv_hi, p.scale_log2);
        }
    };
    // Steps alternate between the two buffer pairs; each loop is unrolled by two so that
    // every LDS access names its buffer statically.
    auto run = [&](auto msk, int it, int it_end) __attribute__((always_inline)) {
        if (it < it_end && (it & 1)) {
            do_step(BufSel<1>{}, msk, it);
            ++it;
        }
        for (; it + 1 < it_end; it += 2) {
            do_step(BufSel<0>{}, msk, it);
            do_step(BufSel<1>{}, msk, it + 1);
        }
        if (it < it_end)
            do_step(BufSel<0>{}, msk, it);
    };
    if constexpr (kAlternate) {
        // Alternating schedule.  The two wavefronts of a SIMD (row group rg, key parts 0
        // and 1) take the two halves of each step in opposite order, so that one issues
        // matrix products while the other runs the softmax:
        //   iteration t, first half:   part 0: PV(t - 1), S(t)     part 1: softmax(t - 1)
        //   iteration t, second half:  part 0: softmax(t)          part 1: PV(t - 1), S(t)
        // for t = 0 .. nsteps (PV(-1), S(nsteps) and softmax(-1) are empty).  K of step t
        // sits in K buffer t & 1 and V of step t in V buffer t & 1: iteration t copies
        // K(t + 1) and V(t), which land before its closing barrier, while it reads K(t) and
        // V(t - 1), so V is staged one step after K and no buffer is written while read.
        f32x4 sacc[2][4];
        bf16x8 pw[2][2];
        const auto& k_ops = pf_pick<kFp8>(k_addr8, k_addr);   // the K operand offsets of the format
        auto ktile = [&](auto sel) __attribute__((always_inline)) {
            return reinterpret_cast<const char*>(decltype(sel)::value == 0 ? k_tile0 : k_tile1);
        };
        auto vtile = [&](auto sel) __attribute__((always_inline)) {
            return reinterpret_cast<const char*>(decltype(sel)::value == 0 ? v_tile0 : v_tile1);
        };
        // iteration t's copies: K(t + 1) (past the last step a spare copy of it, which
        // nothing reads) and V(t)
        auto copies = [&](auto sel, int t) __attribute__((always_inline)) {
            constexpr int B = decltype(sel)::value;
            int id = next_id;
            asm volatile("" : "+v"(id));
            const int id1 = checked(__builtin_amdgcn_readfirstlane(id));
            stage_pool(std::false_type{}, BufSel<B ^ 1>{}, step_at(t + 1), id1);
            stage_pool(std::true_type{}, BufSel<B>{}, step_at(t), cur_id);
            cur_id = id1;
            next_id = table_entry(step_at(t + 2));
        };
        auto softmax = [&](auto msk, int t) __attribute__((always_inline)) {
            pf_softmax_full<decltype(msk)::value>(sacc, oacc, m, lsum, pw, step_at(t) * kPfKeys + kKPW * kh, kslice,
                                                  qpos, kv_hi, p.scale_log2);
        };
        auto softmax_any = [&](int t) __attribute__((always_inline)) {
            if (t >= n_plain)
                softmax(std::true_type{}, t);
            else
                softmax(std::false_type{}, t);
        };
        auto sync = [&]() __attribute__((always_inline)) {
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        };
        // keeps the two halves of the key parts aligned (no data passes here)
        auto half_sync = [&]() __attribute__((always_inline)) { asm volatile("s_barrier" ::: "memory"); };
        // iterations t0 .. t1 - 1 of the steady state (both products, one softmax), with the
        // softmax's step masked or not throughout
        auto steady = [&](auto part, auto msk, int t0, int t1) __attribute__((always_inline)) {
            auto body = [&](auto sel, int t) __attribute__((always_inline)) {
                constexpr int B = decltype(sel)::value;
                copies(sel, t);
                if constexpr (decltype(part)::value == 0) {
                    if (active)
                        pf_matrix_full<kFp8>(vtile(BufSel<B ^ 1>{}), v_addr, pw, oacc, ktile(sel), k_ops, qop, sacc);
                    half_sync();
                    if (active)
                        softmax(msk, t);
                } else {
                    if (active)
                        softmax(msk, t - 1);
                    half_sync();
                    if (active)
                        pf_matrix_full<kFp8>(vtile(BufSel<B ^ 1>{}), v_addr, pw, oacc, ktile(sel), k_ops, qop, sacc);
                }
                sync();
            };
            int t = t0;
            if (t < t1 && (t & 1)) {
                body(BufSel<1>{}, t);
                ++t;
            }
            for (; t + 1 < t1; t += 2) {
                body(BufSel<0>{}, t);
                body(BufSel<1>{}, t + 1);
            }
            if (t < t1)
                body(BufSel<0>{}, t);
        };
        auto loop = [&](auto part) __attribute__((always_inline)) {
            constexpr int kPart = decltype(part)::value;
            // t = 0: S(0) (and part 0's softmax of it)
            copies(BufSel<0>{}, 0);
            if constexpr (kPart == 0) {
                if (active)
                    pf_qk_full(ktile(BufSel<0>{}), k_ops, qop, sacc);
                half_sync();
                if (active)
                    softmax_any(0);
            } else {
                half_sync();
                if (active)
                    pf_qk_full(ktile(BufSel<0>{}), k_ops, qop, sacc);
            }
            sync();
            // t = 1 .. nsteps - 1; the softmax of step t (part 0) or t - 1 (part 1) is
            // masked from step n_plain on
            const int edge = min(max(n_plain + kPart, 1), nsteps);
            steady(part, std::false_type{}, 1, edge);
            steady(part, std::true_type{}, edge, nsteps);
            // t = nsteps: the last PV (after part 1's last softmax)
            auto last_pv = [&]() __attribute__((always_inline)) {
                if ((nsteps - 1) & 1)
                    pf_pv_full<kFp8>(vtile(BufSel<1>{}), v_addr, pw, oacc);
                else
                    pf_pv_full<kFp8>(vtile(BufSel<0>{}), v_addr, pw, oacc);
            };
            if constexpr (kPart == 0) {
                if (active)
                    last_pv();
                half_sync();
            } else {
                if (active)
                    softmax_any(nsteps - 1);
                half_sync();
                if (active)
                    last_pv();
            }
            sync();
        };
        if (nsteps > 0) {
            asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");   // K(0)
            if (kh == 0)
                loop(std::integral_constant<int, 0>{});
            else
                loop(std::integral_constant<int, 1>{});
        }
    } else {
        run(std::integral_constant<bool, false>{}, 0, n_plain);
        run(std::integral_constant<bool, true>{}, n_plain, nsteps);
        wait_vmcnt<0>();                       // the last step's spare copy
    }

    // Fused append: split 0 of each (tile, KV head) writes the tile's new tokens of this KV
    // head into their slots (every workgroup of the launch reads new positions from k_new /
    // v_new, see `stage`).  The rows are loaded here and stored after the key-part merge,
    // so that their load latency hides behind it.
    u32x4 new_k = u32x4{0u, 0u, 0u, 0u}, new_v = new_k;
    int64_t new_dst = -1;
    if constexpr (kFused) {
        const int tl = qt * kTileTok + (tid >> 4), c = tid & 15;          // kTileTok tokens x 16 chunks
        if (split == 0 && hs.slice == 0 && !bad_row && (tid >> 4) < kTileTok && tl < qlen) {
            const int pos = ctx + tl;
            const int phys = p.block_tables[(int64_t)r * p.max_blocks + pos / kBlock];
            if (phys >= 0 && phys < p.num_blocks) {
                new_dst = (((int64_t)phys * p.num_kv_heads + kvh) * kBlock + pos % kBlock) * kHeadDim + c * 8;
                const int64_t src = ((int64_t)(q0 + tl) * p.num_kv_heads + kvh) * kHeadDim + c * 8;
                new_k = *reinterpret_cast<const u32x4*>(p.k_new + src);
                new_v = *reinterpret_cast<const u32x4*>(p.v_new + src);
            }
        }
    }

    // Merge the key parts: the wavefronts of key parts 1 .. kNKP - 1 hand (m, lane-partial l,
    // O^T) to the key-part-0 wavefront with the same rows, in the lanes' own layout.  The
    // O^T blocks (kRB x 8 KiB per wavefront) fill the first three tile buffers in (key part,
    // row group) order, the maxima and sums sit in the fourth; every wavefront is past its
    // last LDS read of the tiles and its last copy has landed.
    __syncthreads();
    auto xo_at = [&](int kp) __attribute__((always_inline)) {
        const int e = ((kp - 1) * kRG + rg) * (kRB * 8 * 64);     // 16-byte units
        const int bi = e / kTileChunks;
        u32x4* base = bi == 0 ? k_tile0 : (bi == 1 ? v_tile0 : k_tile1);
        return base + (e - bi * kTileChunks);
    };
    static_assert((kNKP - 1) * kRG * kRB * 8 * 64 <= 3 * kTileChunks, "key-part partials fit three tile buffers");
    float* const xm = reinterpret_cast<float*>(v_tile1);              // [kNKP - 1][kRG][kRB][64]
    float* const xl = xm + 1024;
    static_assert((kNKP - 1) * kRG * kRB * 64 <= 1024, "key-part maxima fit");
    if (kh > 0) {
        u32x4* xo = xo_at(kh);
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
#pragma unroll
            for (int db = 0; db < 8; ++db)
                xo[(rb * 8 + db) * 64 + lane] = __builtin_bit_cast(u32x4, oacc[rb][db]);
            const int mi = (((kh - 1) * kRG + rg) * kRB + rb) * 64 + lane;
            xm[mi] = m[rb];
            xl[mi] = lsum[rb];
        }
    }
    bad = __syncthreads_or(bad);
    if constexpr (kFused) {
        if (new_dst >= 0) {
            *reinterpret_cast<u32x4*>(const_cast<uint16_t*>(p.k_pool) + new_dst) = new_k;
            *reinterpret_cast<u32x4*>(const_cast<uint16_t*>(p.v_pool) + new_dst) = new_v;
        }
    }
    const float nan = __builtin_nanf("");
    float lse2[kRB];                            // log2-sum-exp of this workgroup's keys per row
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
        lse2[rb] = -INFINITY;
    if (kh == 0) {
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
            float mk[kNKP], lk[kNKP], w[kNKP];
            mk[0] = m[rb];
            lk[0] = lsum[rb];
            float M = m[rb];
#pragma unroll
            for (int kp = 1; kp < kNKP; ++kp) {
                const int mi = (((kp - 1) * kRG + rg) * kRB + rb) * 64 + lane;
                mk[kp] = xm[mi];
                lk[kp] = xl[mi];
                M = fmaxf(M, mk[kp]);
            }
#pragma unroll
            for (int kp = 0; kp < kNKP; ++kp)
                w[kp] = (mk[kp] == -INFINITY) ? 0.f : fast_exp2(mk[kp] - M);
            float l = w[0] * lk[0] + w[1] * lk[1];
#pragma unroll
            for (int kp = 2; kp < kNKP; ++kp)
                l += w[kp] * lk[kp];
            l += shfl_xor(l, 16);
            l += shfl_xor(l, 32);
            const float inv = l > 0.f ? p.v_scale / l : 0.f;
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                f32x4 o = w[0] * oacc[rb][db] + w[1] * __builtin_bit_cast(f32x4, xo_at(1)[(rb * 8 + db) * 64 + lane]);
#pragma unroll
                for (int kp = 2; kp < kNKP; ++kp)
                    o += w[kp] * __builtin_bit_cast(f32x4, xo_at(kp)[(rb * 8 + db) * 64 + lane]);
                oacc[rb][db] = o * inv;
            }
            lse2[rb] = bad ? nan : (l > 0.f ? M + fast_log2(l) : -INFINITY);
        }
    }

    if constexpr (kCascade) {
        // this split's normalised partial and log2-sum-exp per (request, query head), in
        // the decode kernel's partial layout, with agent-scope stores: the decode
        // workgroups of the same launch merge them.  The kh = 0 wavefronts first stage
        // their rows in LDS ([row][dim], rows 0..63 in k_tile0, 64..127 in v_tile0, each
        // row's 16-byte chunks XOR-swizzled by the row), so that the workgroup then writes
        // every row as contiguous 256-byte pieces; written straight from the MFMA layout,
        // each store instruction would scatter 16-byte pieces over 16 rows.
        const int nrows_valid = 4 * grp_count;
        auto stage_at = [&](int row, int chunk) __attribute__((always_inline)) {
            u32x4* base = row < 64 ? k_tile0 : v_tile0;
            return base + (row & 63) * (kHeadDim / 4) + (chunk ^ (row & 31));
        };
        __syncthreads();                        // the key-half exchange above is done with k_tile0 / v_tile0
        if (kh == 0) {
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb) {
                const int rho = 16 * kRB * rg + 16 * rb + row16;
#pragma unroll
                for (int db = 0; db < 8; ++db)
                    *stage_at(rho, 4 * db + kslice) = __builtin_bit_cast(u32x4, oacc[rb][db]);
                if (kslice == 0 && rho < nrows_valid) {
                    const int64_t pi =
                        ((int64_t)(grp_first + (rho >> 2)) * p.splits + split) * (p.num_vheads * kGroup) + hs.slot0 +
                        (rho & 3);
                    store_agent(p.px_part_lse + pi, lse2[rb]);
                }
            }
        }
        __syncthreads();
        for (int idx = tid; idx < nrows_valid * kHeadDim; idx += 64 * kPfWaves) {
            const int rho = idx / kHeadDim, d = idx % kHeadDim;
            const int64_t pi =
                ((int64_t)(grp_first + (rho >> 2)) * p.splits + split) * (p.num_vheads * kGroup) + hs.slot0 + (rho & 3);
            const float v = reinterpret_cast<const float*>(stage_at(rho, d >> 2))[d & 3];
            store_agent(p.px_part_o + pi * kHeadDim + d, v);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        // count in for every request of the group, one lane per request so that the
        // atomics travel together; the last arrival of a (request, KV head) -- decode split
        // or prefix split -- merges its result
        if (tid == 0)
            last_lds = 0;
        __syncthreads();
        if (tid < grp_count) {
            const int rr = grp_first + tid;
            const int nsplit = decode_splits_of(dp, rr, prefix_skip_of(dp, rr));
            if (nsplit >= 0) {                  // else the decode side does not count this row either
                uint32_t* counter = dp.counters + (int64_t)rr * dp.num_vheads + vkv;
                const uint32_t done = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (done == (uint32_t)(nsplit + p.splits - 1)) {
                    __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    atomicOr(reinterpret_cast<unsigned int*>(&last_lds), 1u << tid);
                }
            }
        }
        __syncthreads();
        int rows[PA_MAX_PREFIX_GROUP_REQS];
        int nrows = 0;
        for (uint32_t mine = (uint32_t)last_lds; mine; mine &= mine - 1)
            rows[nrows++] = grp_first + __builtin_ctz(mine);
        if (nrows > 0)
            merge_group_rows(dp, rows, nrows, vkv, p.splits);
        return;
    }

    // output: lane l holds O^T[16 db + 4 kslice + e][row row16] of row block rb
    auto write_out = [&](const f32x4 (&o)[kRB][8], const float (&lse_row)[kRB]) __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
            const int rho = 16 * kRB * rg + 16 * rb + row16;
            const int tl = qt * kTileTok + (rho >> 2);
            if (tl >= qlen || (rho & 3) >= hs.heads)
                continue;
            const bool nan_row = lse_row[rb] != lse_row[rb];
            const int64_t orow = ((int64_t)(q0 + tl) * p.num_q_heads + head0 + (rho & 3));
            uint16_t* dst = p.out + orow * kHeadDim + 4 * kslice;
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                const f32x4 v = nan_row ? f32x4{nan, nan, nan, nan} : o[rb][db];
                *reinterpret_cast<u32x2*>(dst + 16 * db) = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
            }
            if (kslice == 0)
                p.lse[orow] = lse_row[rb] * kLn2;
        }
    };

    if (p.splits == 1) {
        if (kh == 0)
            write_out(oacc, lse2);
        return;
    }

    // Partials are written with agent-scope stores (coherent across the XCDs' separate L2
    // caches) and every thread waits until its stores have completed before the
    // workgroup counts itself in; the last split reads them with agent-scope loads.
    const int64_t item0 = ((int64_t)tile * p.num_vheads + vkv) * p.splits;   // split 0 of this (tile, virtual KV head)
    // per (tile, KV head, split): kRG row groups of kRB x 8 f32x4 per lane, and kRB x 64
    // log2-sum-exps per row group, in lane order
    auto part_o_at = [&](int sp) __attribute__((always_inline)) { return p.part_o + ((item0 + sp) * kRG + rg) * (kRB * 8 * 4 * 64); };
    auto part_lse_at = [&](int sp) __attribute__((always_inline)) { return p.part_lse + ((item0 + sp) * kRG + rg) * (kRB * 64); };
    if (kh == 0) {
        float* po = part_o_at(split);
#pragma unroll
        for (int i = 0; i < kRB * 8; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                store_agent(po + (i * 4 + e) * 64 + lane, oacc[i >> 3][i & 7][e]);
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
            store_agent(part_lse_at(split) + rb * 64 + lane, lse2[rb]);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    uint32_t* counter = p.counters + (int64_t)tile * p.num_vheads + vkv;
    if (tid == 0) {
        const uint32_t done = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = done == (uint32_t)(p.splits - 1);
        if (last)
            __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // ready for the next call
        last_lds = last;
    }
    __syncthreads();
    if (!last_lds || kh != 0)
        return;

    if (p.splits == 2) {
        // Two splits, the usual case: the other split's log2-sum-exps and values are loaded
        // together, so that the merge waits for one round trip.  The arithmetic and its order
        // are those of the general merge below.
        const int other = split ^ 1;
        const float* po = part_o_at(other);
        float lo[kRB];
        f32x4 oo[kRB][8];
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
            lo[rb] = load_agent(part_lse_at(other) + rb * 64 + lane);
#pragma unroll
            for (int db = 0; db < 8; ++db)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    oo[rb][db][e] = load_agent(po + ((rb * 8 + db) * 4 + e) * 64 + lane);
        }
        bool any_nan = false;
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
            const float l0 = split == 0 ? lse2[rb] : lo[rb];
            const float l1 = split == 0 ? lo[rb] : lse2[rb];
            any_nan |= l0 != l0;
            any_nan |= l1 != l1;
            const float L = fmaxf(fmaxf(-INFINITY, l0), l1);
            const float w0 = (l0 > -INFINITY) ? fast_exp2(l0 - L) : 0.f;
            const float w1 = (l1 > -INFINITY) ? fast_exp2(l1 - L) : 0.f;
            float wsum = 0.f;
            wsum += w0;
            wsum += w1;
            const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
                o += w0 * (split == 0 ? oacc[rb][db] : oo[rb][db]);
                o += w1 * (split == 0 ? oo[rb][db] : oacc[rb][db]);
                oacc[rb][db] = o * inv;
            }
            lse2[rb] = wsum > 0.f ? L + fast_log2(wsum) : -INFINITY;
        }
        if (any_nan) {
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb)
                lse2[rb] = nan;
        }
    } else {
        // Each row block's 32 values in a lane belong to one row and share its log2-sum-exp,
        // so the merge weights are found once per split: L = max_s l_s, c_s = 2^(l_s - L),
        // then O = sum_s c_s O_s / sum_s c_s and LSE = L + log2 sum_s c_s.  Both row blocks
        // are merged together, the log2-sum-exps loaded eight splits at a time and each
        // split's 64 values at once, so the merge costs about one memory round trip per
        // split.  The splits are taken in index order whichever finished last, so the bits
        // do not depend on timing.
        auto lse_of = [&](int sp, int rb) __attribute__((always_inline)) {
            return sp == split ? lse2[rb] : load_agent(part_lse_at(sp) + rb * 64 + lane);
        };
        float L[kRB];
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
            L[rb] = -INFINITY;
        bool any_nan = false;
        for (int s0 = 0; s0 < p.splits; s0 += 8) {
            float ls[8][kRB];
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int rb = 0; rb < kRB; ++rb)
                    ls[u][rb] = lse_of(min(s0 + u, p.splits - 1), rb);
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int rb = 0; rb < kRB; ++rb)
                    if (s0 + u < p.splits) {
                        any_nan |= ls[u][rb] != ls[u][rb];
                        L[rb] = fmaxf(L[rb], ls[u][rb]);
                    }
        }
        float wsum[kRB];
        f32x4 o[kRB][8];
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
            wsum[rb] = 0.f;
#pragma unroll
            for (int db = 0; db < 8; ++db)
                o[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        for (int sp = 0; sp < p.splits; ++sp) {
            float c[kRB];
            f32x4 os[kRB][8];
            if (sp == split) {
#pragma unroll
                for (int rb = 0; rb < kRB; ++rb) {
                    c[rb] = lse2[rb];
#pragma unroll
                    for (int db = 0; db < 8; ++db)
                        os[rb][db] = oacc[rb][db];
                }
            } else {
                const float* po = part_o_at(sp);
#pragma unroll
                for (int rb = 0; rb < kRB; ++rb) {
                    c[rb] = load_agent(part_lse_at(sp) + rb * 64 + lane);
#pragma unroll
                    for (int db = 0; db < 8; ++db)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            os[rb][db][e] = load_agent(po + ((rb * 8 + db) * 4 + e) * 64 + lane);
                }
            }
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb) {
                const float w = (c[rb] > -INFINITY) ? fast_exp2(c[rb] - L[rb]) : 0.f;
                wsum[rb] += w;
#pragma unroll
                for (int db = 0; db < 8; ++db)
                    o[rb][db] += w * os[rb][db];
            }
        }
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
            const float inv = wsum[rb] > 0.f ? 1.f / wsum[rb] : 0.f;
#pragma unroll
            for (int db = 0; db < 8; ++db)
                oacc[rb][db] = o[rb][db] * inv;
            lse2[rb] = any_nan ? nan : (wsum[rb] > 0.f ? L[rb] + fast_log2(wsum[rb]) : -INFINITY);
        }
    }
    write_out(oacc, lse2);
}
template <bool kFused, bool kQ8, int kRG, int kRB, bool kFp8 = false>
__global__ __launch_bounds__(64 * kPfWaves) void pa_prefill_tile(PrefillParams p)
{
    prefill_body<false, kFused, kQ8, kRG, kRB, kFp8>(p, DecodeParams{}, blockIdx.x);
}

// The chunk rows of a fused step: each row's new K / V rows go into the slots of positions
// kv_len - qo_len .. kv_len - 1 through its table before the tiles read them, as they are
// (bf16 pool) or encoded exactly as pa_append_q8_scatter / pa_append_fp8_scatter encode
// them.  One thread per (token, KV head, piece): 8 values (bf16), a 32-value group (q8_0)
// or 16 values (FP8); blockIdx.y is the prefill row.
enum PoolFmt { kFmtBf16 = 0, kFmtQ8 = 1, kFmtFp8 = 2 };
template <int kFmt>
constexpr int kAppendPieces = kFmt == kFmtBf16 ? kHeadDim / 8 : kFmt == kFmtQ8 ? kHeadDim / pa::kQ8Group : kHeadDim / 16;

// Piece idx of prefill row i's new tokens (idx = (token * num_kv_heads + head) * pieces +
// piece); indices past the row's tokens do nothing.
template <int kFmt>
__device__ inline void append_chunk_piece(const PrefillParams& p, int i, int64_t idx)
{
    constexpr bool kQ8 = kFmt == kFmtQ8;
    constexpr int kPieces = kAppendPieces<kFmt>;
    const int r = p.prefill_req[i];
    const int q0 = p.qo_indptr[r];
    const int qlen = p.qo_indptr[r + 1] - q0;
    const int kvlen = p.kv_len[r];
    const int ctx = kvlen - qlen;
    const int64_t per_token = (int64_t)p.num_kv_heads * kPieces;
    if (qlen < 1 || ctx < 0 || idx >= (int64_t)qlen * per_token)
        return;
    const int t = (int)(idx / per_token);
    const int rem = (int)(idx - (int64_t)t * per_token);
    const int h = rem / kPieces, c = rem % kPieces;
    const int pos = ctx + t;
    if (pos / kBlock >= p.max_blocks)
        return;
    const int phys = p.block_tables[(int64_t)r * p.max_blocks + pos / kBlock];
    if (phys < 0 || phys >= p.num_blocks)
        return;
    const int64_t src = ((int64_t)(q0 + t) * p.num_kv_heads + h) * kHeadDim;
    uint8_t* kpool = reinterpret_cast<uint8_t*>(const_cast<uint16_t*>(p.k_pool));
    uint8_t* vpool = reinterpret_cast<uint8_t*>(const_cast<uint16_t*>(p.v_pool));
    const int64_t dst = (((int64_t)phys * p.num_kv_heads + h) * kBlock + pos % kBlock) * kHeadDim;
    if constexpr (kFmt == kFmtBf16) {
        *reinterpret_cast<u32x4*>(const_cast<uint16_t*>(p.k_pool) + dst + 8 * c) =
            *reinterpret_cast<const u32x4*>(p.k_new + src + 8 * c);
        *reinterpret_cast<u32x4*>(const_cast<uint16_t*>(p.v_pool) + dst + 8 * c) =
            *reinterpret_cast<const u32x4*>(p.v_new + src + 8 * c);
    } else if constexpr (kQ8) {
        q8_append_group(kpool, p.k_new, p.v_new, src, c, phys, pos % kBlock, h, p.num_kv_heads);
    } else {
        fp8_append_chunk(kpool, vpool, p.k_new, p.v_new, src, c, dst, p.k_div, p.v_div);
    }
}

template <int kFmt>
__global__ __launch_bounds__(256) void pa_append_chunk_rows(PrefillParams p)
{
    append_chunk_piece<kFmt>(p, blockIdx.y, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

// A fused step's decode rows (their append inside, as in pa_decode_split) and, in
// workgroups past them, its chunk rows' appends (append_wgs_per_row workgroups of
// 64 * kDecodeWaves threads per prefill row): one launch instead of an append launch
// before the chunk tiles, which the host then launches after this one.
template <bool kQ8, bool kFp8>
__global__ __launch_bounds__(64 * kDecodeWaves) void pa_decode_split_append(DecodeParams dp, PrefillParams pp,
                                                                             int32_t decode_wgs,
                                                                             int32_t append_wgs_per_row)
{
    if ((int32_t)blockIdx.x < decode_wgs) {
        decode_body<kQ8, true, kFp8>(dp, blockIdx.x);
        return;
    }
    constexpr int kFmt = kQ8 ? kFmtQ8 : kFp8 ? kFmtFp8 : kFmtBf16;
    const int e = (int)blockIdx.x - decode_wgs;
    const int i = e / append_wgs_per_row;
    if (i >= pp.num_prefill_rows)
        return;
    append_chunk_piece<kFmt>(pp, i, (int64_t)(e % append_wgs_per_row) * (64 * kDecodeWaves) + threadIdx.x);
}

static_assert(kPfWaves == kDecodeWaves, "the fused shared-prefix launch runs both bodies with one block size");

// A batch with shared-prefix groups in one launch: workgroups 0 .. num_prefix_wgs - 1 read
// each group's shared blocks once per KV head (the prefill body in its shared-prefix
// form), the rest are the decode workgroups.  The prefix workgroups come first in the
// grid and wait for nothing; a (row, KV head) is finished by whichever of its decode
// splits and prefix splits arrives last, so no workgroup ever waits for another.
template <bool kQ8, bool kFused, int kRG, int kRB, bool kFp8 = false>
__global__ __launch_bounds__(64 * kPfWaves) void pa_cascade_decode(PrefillParams pp, DecodeParams dp,
                                                                 int32_t num_prefix_wgs)
{
    if ((int32_t)blockIdx.x < num_prefix_wgs)
        prefill_body<true, false, kQ8, kRG, kRB, kFp8>(pp, dp, blockIdx.x);
    else
        decode_body<kQ8, kFused, kFp8>(dp, blockIdx.x - num_prefix_wgs);
}


// Sets n 32-bit words to zero (a kernel rather than a memset, so that a stream capture
// records an ordinary kernel node).
__global__ __launch_bounds__(256) void pa_zero_words(uint32_t* __restrict__ p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n)
        p[i] = 0u;
}

// A mixed batch (chunk tiles and decode rows) in one launch.  With `interleave` 0 the grid
// holds the chunk-tile workgroups first, then the decode workgroups (which fill CUs as the
// chunk tiles drain).  Otherwise both kinds come in groups of num_vheads, one per virtual
// KV head, and the grid alternates a group of chunk-tile workgroups with a group of decode
// workgroups while both last, then runs the rest of the longer kind; workgroups are dealt
// round-robin to the XCDs, so each KV head keeps one XCD (and its L2) for both kinds.
// Nothing waits for anything else: the two kinds share no outputs, and their split
// counters and partials sit in separate parts of the workspace.
template <bool kFused>
__global__ __launch_bounds__(64 * kPfWaves) void pa_mixed_batch(PrefillParams pp, DecodeParams dp,
                                                                int32_t num_prefill_wgs, int32_t num_decode_wgs,
                                                                int32_t interleave)
{
    const int H = dp.num_vheads;
    const int b = blockIdx.x, grp = b / H, lane = b - grp * H;
    const int pf_groups = num_prefill_wgs / H, dc_groups = num_decode_wgs / H;
    const int both = interleave ? min(pf_groups, dc_groups) : 0;
    bool prefill;
    int idx;
    if (!interleave) {
        prefill = b < num_prefill_wgs;
        idx = prefill ? b : b - num_prefill_wgs;
    } else if (grp < 2 * both) {
        prefill = (grp & 1) == 0;
        idx = (grp >> 1) * H + lane;
    } else {
        prefill = pf_groups > both;
        idx = (grp - both) * H + lane;
    }
    if (prefill)
        prefill_body<false, kFused, false>(pp, dp, idx);
    else
        decode_body<false, kFused>(dp, idx);
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

// ------------------------------------------------------------------------------ C entry points

// With PA_VALIDATE=1 in the environment the entry points also run the content checks of
// pa_validate_batch / pa_validate_append before launching anything: a debugging mode in
// which the index arrays are copied to the host in stream order (so the call waits for
// the stream) and a failed check returns its status with nothing launched.
static bool validate_requested()
{
    const char* v = getenv("PA_VALIDATE");
    return v && v[0] == '1';
}

template <typename T>
static pa_status copy_to_host(std::vector<T>& dst, const T* src, size_t n, hipStream_t st)
{
    dst.resize(n);
    if (n == 0)
        return PA_OK;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cap) != hipSuccess)
        return PA_ERR_HIP;
    if (cap != hipStreamCaptureStatusNone)
        return PA_ERR_UNSUPPORTED;             // the check cannot wait inside a graph capture
    if (hipMemcpyAsync(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost, st) != hipSuccess)
        return PA_ERR_HIP;
    return hipStreamSynchronize(st) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

static pa_status validate_slots(const pa_geometry* g, const int32_t* slot_mapping, int32_t n_tokens, void* stream)
{
    std::vector<int32_t> slots;
    const pa_status st = copy_to_host(slots, slot_mapping, (size_t)n_tokens, as_stream(stream));
    return st != PA_OK ? st : pa_validate_append(g, slots.data(), n_tokens, nullptr);
}

extern "C" pa_status pa_append_kv(const pa_geometry* g, void* k_pool, void* v_pool, const void* k_new,
                                  const void* v_new, const int32_t* slot_mapping, int32_t n_tokens, void* stream)
{
    if (!g)
        return PA_ERR_NULL;
    if (!pa::geometry_supported(g))
        return PA_ERR_UNSUPPORTED;
    if (n_tokens < 0)
        return PA_ERR_SHAPE;
    if (n_tokens == 0)
        return PA_OK;
    if (!k_pool || !v_pool || !k_new || !v_new || !slot_mapping)
        return PA_ERR_NULL;
    if (validate_requested()) {
        const pa_status st = validate_slots(g, slot_mapping, n_tokens, stream);
        if (st != PA_OK)
            return st;
    }
    const int64_t threads = (int64_t)n_tokens * g->num_kv_heads * (kHeadDim * 2 / 16);
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > INT32_MAX)
        return PA_ERR_SHAPE;
    hipLaunchKernelGGL(pa_append_scatter, dim3((uint32_t)blocks), dim3(256), 0, as_stream(stream),
                       static_cast<uint16_t*>(k_pool), static_cast<uint16_t*>(v_pool),
                       static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), slot_mapping,
                       n_tokens, g->num_kv_heads, (int64_t)g->num_blocks * kBlock);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

extern "C" pa_status pa_append_kv_q8(const pa_geometry* g, void* kv_pool_q8, const void* k_new, const void* v_new,
                                     const int32_t* slot_mapping, int32_t n_tokens, void* stream)
{
    if (!g)
        return PA_ERR_NULL;
    if (!pa::geometry_supported(g))
        return PA_ERR_UNSUPPORTED;
    if (n_tokens < 0)
        return PA_ERR_SHAPE;
    if (n_tokens == 0)
        return PA_OK;
    if (!kv_pool_q8 || !k_new || !v_new || !slot_mapping)
        return PA_ERR_NULL;
    if (validate_requested()) {
        const pa_status st = validate_slots(g, slot_mapping, n_tokens, stream);
        if (st != PA_OK)
            return st;
    }
    const int64_t threads = (int64_t)n_tokens * g->num_kv_heads * (kHeadDim / pa::kQ8Group);
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > INT32_MAX)
        return PA_ERR_SHAPE;
    hipLaunchKernelGGL(pa_append_q8_scatter, dim3((uint32_t)blocks), dim3(256), 0, as_stream(stream),
                       static_cast<uint8_t*>(kv_pool_q8), static_cast<const uint16_t*>(k_new),
                       static_cast<const uint16_t*>(v_new), slot_mapping, n_tokens, g->num_kv_heads,
                       (int64_t)g->num_blocks * kBlock);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

extern "C" pa_status pa_append_kv_fp8(const pa_geometry* g, void* k_pool_fp8, void* v_pool_fp8, const void* k_new,
                                      const void* v_new, const int32_t* slot_mapping, int32_t n_tokens, float k_scale,
                                      float v_scale, void* stream)
{
    if (!g)
        return PA_ERR_NULL;
    if (!pa::geometry_supported(g))
        return PA_ERR_UNSUPPORTED;
    if (n_tokens < 0 || !(k_scale > 0.0f) || !(v_scale > 0.0f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
        return PA_ERR_SHAPE;
    if (n_tokens == 0)
        return PA_OK;
    if (!k_pool_fp8 || !v_pool_fp8 || !k_new || !v_new || !slot_mapping)
        return PA_ERR_NULL;
    if (validate_requested()) {
        const pa_status st = validate_slots(g, slot_mapping, n_tokens, stream);
        if (st != PA_OK)
            return st;
    }
    const int64_t threads = (int64_t)n_tokens * g->num_kv_heads * (kHeadDim / 16);
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > INT32_MAX)
        return PA_ERR_SHAPE;
    hipLaunchKernelGGL(pa_append_fp8_scatter, dim3((uint32_t)blocks), dim3(256), 0, as_stream(stream),
                       static_cast<uint8_t*>(k_pool_fp8), static_cast<uint8_t*>(v_pool_fp8),
                       static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), slot_mapping, n_tokens,
                       g->num_kv_heads, (int64_t)g->num_blocks * kBlock, k_scale, v_scale);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

static pa_status copy_blocks(const pa_geometry* g, void* k_pool, void* v_pool, const int32_t* src_blocks,
                             const int32_t* dst_blocks, int32_t n, void* stream, int64_t head_bytes, int32_t npools)
{
    if (!g)
        return PA_ERR_NULL;
    if (!pa::geometry_supported(g))
        return PA_ERR_UNSUPPORTED;
    if (n < 0)
        return PA_ERR_SHAPE;
    if (n == 0)
        return PA_OK;
    if (!k_pool || !v_pool || !src_blocks || !dst_blocks)
        return PA_ERR_NULL;
    const int64_t blk_chunks = (int64_t)g->num_kv_heads * head_bytes / 16;   // one pool's block, all KV heads
    const int64_t threads = (int64_t)n * npools * blk_chunks;
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > INT32_MAX)
        return PA_ERR_SHAPE;
    hipLaunchKernelGGL(pa_copy_scatter, dim3((uint32_t)blocks), dim3(256), 0, as_stream(stream),
                       static_cast<u32x4*>(k_pool), static_cast<u32x4*>(v_pool), src_blocks, dst_blocks, n,
                       g->num_blocks, blk_chunks, npools);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

extern "C" pa_status pa_copy_blocks(const pa_geometry* g, void* k_pool, void* v_pool, const int32_t* src_blocks,
                                    const int32_t* dst_blocks, int32_t n, void* stream)
{
    return copy_blocks(g, k_pool, v_pool, src_blocks, dst_blocks, n, stream, kBlock * kHeadDim * 2, 2);
}

extern "C" pa_status pa_copy_blocks_fp8(const pa_geometry* g, void* k_pool_fp8, void* v_pool_fp8,
                                        const int32_t* src_blocks, const int32_t* dst_blocks, int32_t n, void* stream)
{
    return copy_blocks(g, k_pool_fp8, v_pool_fp8, src_blocks, dst_blocks, n, stream, kBlock * kHeadDim, 2);
}

extern "C" pa_status pa_copy_blocks_q8(const pa_geometry* g, void* kv_pool_q8, const int32_t* src_blocks,
                                       const int32_t* dst_blocks, int32_t n, void* stream)
{
    return copy_blocks(g, kv_pool_q8, kv_pool_q8, src_blocks, dst_blocks, n, stream, 2 * pa::kQ8TileBytes, 1);
}

// Tile shape (row groups, row blocks per wavefront) of a tile of `rows` MFMA rows.
static bool tile_rows_supported(int rows) { return rows == 32 || rows == 64 || rows == 128; }

template <typename... Args>
static void launch(void (*kernel)(Args...), uint32_t grid, hipStream_t st, Args... args)
{
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(64 * kPfWaves), 0, st, args...);
}

static void launch_prefill_tiles(bool q8, bool fp8, int rows, uint32_t grid, hipStream_t st, const PrefillParams& pp)
{
    if (q8)
        launch(pa_prefill_tile<false, true, 4, 2>, grid, st, pp);
    else if (fp8)
        launch(rows == 32   ? pa_prefill_tile<false, false, 2, 1, true>
               : rows == 64 ? pa_prefill_tile<false, false, 2, 2, true>
                            : pa_prefill_tile<false, false, 4, 2, true>,
               grid, st, pp);
    else if (rows == 32)
        launch(pa_prefill_tile<false, false, 2, 1>, grid, st, pp);
    else if (rows == 64)
        launch(pa_prefill_tile<false, false, 2, 2>, grid, st, pp);
    else
        launch(pa_prefill_tile<false, false, 4, 2>, grid, st, pp);
}

static void launch_cascade(bool q8, bool fused, bool fp8, int rows, uint32_t grid, hipStream_t st,
                           const PrefillParams& pp, const DecodeParams& dp, int32_t nprefix)
{
    if (q8)
        launch(fused ? pa_cascade_decode<true, true, 4, 2> : pa_cascade_decode<true, false, 4, 2>, grid, st, pp, dp,
               nprefix);
    else if (fp8 && fused)
        launch(rows == 32   ? pa_cascade_decode<false, true, 2, 1, true>
               : rows == 64 ? pa_cascade_decode<false, true, 2, 2, true>
                            : pa_cascade_decode<false, true, 4, 2, true>,
               grid, st, pp, dp, nprefix);
    else if (fp8)
        launch(rows == 32   ? pa_cascade_decode<false, false, 2, 1, true>
               : rows == 64 ? pa_cascade_decode<false, false, 2, 2, true>
                            : pa_cascade_decode<false, false, 4, 2, true>,
               grid, st, pp, dp, nprefix);
    else if (rows == 32)
        launch(fused ? pa_cascade_decode<false, true, 2, 1> : pa_cascade_decode<false, false, 2, 1>, grid, st, pp, dp,
               nprefix);
    else if (rows == 64)
        launch(fused ? pa_cascade_decode<false, true, 2, 2> : pa_cascade_decode<false, false, 2, 2>, grid, st, pp, dp,
               nprefix);
    else
        launch(fused ? pa_cascade_decode<false, true, 4, 2> : pa_cascade_decode<false, false, 4, 2>, grid, st, pp, dp,
               nprefix);
}

// The plan's view of the rows must be that of the device lengths: the same rows with
// qo_len > 1, in order and with their tile counts, every other row a decode row whose
// splits fit max_splits, and shared-prefix groups made of decode rows with blocks past
// the shared ones.  A row the plan classifies wrongly would otherwise be left unwritten.
static pa_status check_plan_matches(const pa_plan_t* plan, const std::vector<int32_t>& qo,
                                    const std::vector<int32_t>& kvl)
{
    const int32_t R = plan->num_reqs;
    std::vector<int32_t> skip((size_t)R, 0);
    for (int gi = 0; gi < plan->num_prefix_groups; ++gi)
        for (int k = 0; k < plan->prefix_num_reqs[gi]; ++k)
            skip[(size_t)(plan->prefix_first_req[gi] + k)] = plan->prefix_blocks[gi];
    int32_t nd = 0, np = 0;
    for (int32_t r = 0; r < R; ++r) {
        if (qo[r] == 1) {
            ++nd;
            const int32_t nblk = (kvl[r] + kBlock - 1) / kBlock;
            if (plan->split_blocks < 1 || nblk <= skip[r] ||
                (nblk - skip[r] + plan->split_blocks - 1) / plan->split_blocks > plan->max_splits)
                return PA_ERR_SHAPE;
        } else {
            if (np >= plan->num_prefill_rows || plan->prefill_req[np] != r || skip[r] != 0 ||
                plan->prefill_tile_start[np + 1] - plan->prefill_tile_start[np] !=
                    (qo[r] + plan->prefill_tile_tokens - 1) / plan->prefill_tile_tokens)
                return PA_ERR_SHAPE;
            ++np;
        }
    }
    return nd == plan->num_decode_rows && np == plan->num_prefill_rows ? PA_OK : PA_ERR_SHAPE;
}

// FP8 pools pass fp8 = true and their scales (k_scale, v_scale); other pools leave them at 1.
static pa_status attention_batch(bool q8, const pa_geometry* g, const pa_plan_t* plan, const void* q,
                                 const void* k_pool, const void* v_pool, const int32_t* block_tables,
                                 int32_t max_blocks_per_req, const int32_t* qo_indptr, const int32_t* kv_len, void* out,
                                 float* lse, void* workspace, size_t workspace_bytes, void* stream,
                                 const void* k_new = nullptr, const void* v_new = nullptr, bool fp8 = false,
                                 float k_scale = 1.0f, float v_scale = 1.0f)
{
    const bool fused = k_new != nullptr;
    if (!g || !plan)
        return PA_ERR_NULL;
    if (fp8 && (!(k_scale > 0.0f) || !(v_scale > 0.0f) || !std::isfinite(k_scale) || !std::isfinite(v_scale)))
        return PA_ERR_SHAPE;
    if (!pa::geometry_supported(g) || plan->num_q_heads != g->num_q_heads || plan->num_kv_heads != g->num_kv_heads)
        return PA_ERR_UNSUPPORTED;
    if (plan->num_reqs == 0 || plan->total_q == 0)
        return PA_OK;
    if (!q || !k_pool || !v_pool || !block_tables || !qo_indptr || !kv_len || !out || !lse)
        return PA_ERR_NULL;
    if (max_blocks_per_req < 1 || plan->num_prefill_rows > PA_MAX_PREFILL_ROWS)
        return PA_ERR_SHAPE;
    if (plan->prefill_tiles > 0 && (plan->prefill_splits < 1 || plan->prefill_splits > pa::kMaxPrefillSplits ||
                                    !tile_rows_supported(kGroup * plan->prefill_tile_tokens)))
        return PA_ERR_SHAPE;
    const int ngroups = plan->num_prefix_groups;
    if (ngroups < 0 || ngroups > PA_MAX_PREFIX_GROUPS ||
        (ngroups > 0 && (plan->prefix_splits < 1 || plan->prefix_splits > pa::kMaxPrefillSplits)))
        return PA_ERR_SHAPE;
    if (ngroups > 0 && (plan->num_decode_rows < 1 || plan->max_splits < 1 || !tile_rows_supported(plan->prefix_tile_rows)))
        return PA_ERR_SHAPE;
    for (int i = 0; i < ngroups; ++i)
        for (int j = 0; j < i; ++j)          // a row belongs to at most one group
            if (plan->prefix_first_req[i] < plan->prefix_first_req[j] + plan->prefix_num_reqs[j] &&
                plan->prefix_first_req[j] < plan->prefix_first_req[i] + plan->prefix_num_reqs[i])
                return PA_ERR_SHAPE;
    for (int i = 0; i < ngroups; ++i)
        if (plan->prefix_first_req[i] < 0 || plan->prefix_num_reqs[i] < 1 ||
            plan->prefix_num_reqs[i] > PA_MAX_PREFIX_GROUP_REQS ||
            (!q8 && kGroup * plan->prefix_num_reqs[i] > plan->prefix_tile_rows) ||
            plan->prefix_first_req[i] + plan->prefix_num_reqs[i] > plan->num_reqs || plan->prefix_blocks[i] < 1 ||
            plan->prefix_blocks[i] > max_blocks_per_req)
            return PA_ERR_SHAPE;
    const pa::WorkspaceLayout ws =
        pa::workspace_layout(plan->num_reqs, plan->max_splits, g->num_q_heads, g->num_kv_heads, plan->prefill_tiles,
                             plan->prefill_splits, ngroups > 0 ? plan->prefix_splits : 0);
    if (ws.total > 0 && (!workspace || workspace_bytes < ws.total || (reinterpret_cast<uintptr_t>(workspace) & 255)))
        return PA_ERR_WORKSPACE;
    if (ws.counters_used > pa::kMaxCounters)
        return PA_ERR_UNSUPPORTED;
    char* wsp = static_cast<char*>(workspace);
    hipStream_t st = as_stream(stream);
    if (validate_requested()) {
        const int32_t R = plan->num_reqs;
        std::vector<int32_t> indptr, kvl, bt;
        pa_status vs = copy_to_host(indptr, qo_indptr, (size_t)R + 1, st);
        if (vs == PA_OK)
            vs = copy_to_host(kvl, kv_len, (size_t)R, st);
        if (vs == PA_OK)
            vs = copy_to_host(bt, block_tables, (size_t)R * max_blocks_per_req, st);
        if (vs != PA_OK)
            return vs;
        if (indptr[0] != 0 || indptr[R] != plan->total_q)
            return PA_ERR_SHAPE;
        std::vector<int32_t> qo(R);
        for (int32_t r = 0; r < R; ++r)
            qo[r] = indptr[r + 1] - indptr[r];
        vs = pa_validate_batch(g, R, qo.data(), kvl.data(), bt.data(), max_blocks_per_req, nullptr);
        if (vs != PA_OK)
            return vs;
        vs = check_plan_matches(plan, qo, kvl);
        if (vs != PA_OK)
            return vs;
        if (fused) {            // the slots the fused append writes: positions kv_len - qo_len .. kv_len - 1
            std::vector<int32_t> slots;
            slots.reserve((size_t)plan->total_q);
            for (int32_t r = 0; r < R; ++r)
                for (int32_t pos = kvl[r] - qo[r]; pos < kvl[r]; ++pos)
                    slots.push_back(bt[(size_t)r * max_blocks_per_req + pos / kBlock] * kBlock + pos % kBlock);
            vs = pa_validate_append(g, slots.data(), (int32_t)slots.size(), nullptr);
            if (vs != PA_OK)
                return vs;
        }
    }
    const float scale_log2 = g->scale * kLog2e * (fp8 ? k_scale : 1.0f);   // an FP8 pool's K scale folds in
    const float out_v_scale = fp8 ? v_scale : 1.0f;
    const int32_t vheads = pa::num_vheads(g->num_q_heads, g->num_kv_heads);

    auto prefill_params = [&]() {
        PrefillParams pp = {};
        pp.q = static_cast<const uint16_t*>(q);
        pp.k_pool = static_cast<const uint16_t*>(k_pool);
        pp.v_pool = static_cast<const uint16_t*>(v_pool);
        pp.block_tables = block_tables;
        pp.qo_indptr = qo_indptr;
        pp.kv_len = kv_len;
        pp.out = static_cast<uint16_t*>(out);
        pp.lse = lse;
        pp.max_blocks = max_blocks_per_req;
        pp.num_q_heads = g->num_q_heads;
        pp.num_kv_heads = g->num_kv_heads;
        pp.num_vheads = vheads;
        pp.num_blocks = g->num_blocks;
        pp.scale_log2 = scale_log2;
        pp.v_scale = out_v_scale;
        pp.k_div = k_scale;
        pp.v_div = v_scale;
        return pp;
    };

    // chunk tiles and decode rows in one launch (bf16 pool, no shared-prefix group)
    const bool one_launch = plan->one_launch >= 1 && !q8 && !fp8 && ngroups == 0 && plan->prefill_tile_tokens == 32 &&
                            plan->num_prefill_rows > 0 &&
                            plan->prefill_tiles > 0 && plan->num_decode_rows > 0 && plan->max_splits > 0;
    PrefillParams mixed_pp = {};
    int64_t mixed_prefill_wgs = 0;
    // A fused step with decode rows and chunk rows (no shared-prefix group, two launches):
    // the chunk rows' appends ride in extra workgroups of the decode launch, which then
    // goes first, and the chunk tiles follow it (the two kinds share no blocks, outputs or
    // workspace).
    const bool append_in_decode = fused && !one_launch && ngroups == 0 && plan->num_prefill_rows > 0 &&
                                  plan->prefill_tiles > 0 && plan->num_decode_rows > 0 && plan->max_splits > 0;
    PrefillParams later_pp = {};
    int64_t later_grid = 0;
    int32_t append_wgs_per_row = 0;
    if (plan->num_prefill_rows > 0 && plan->prefill_tiles > 0) {
        PrefillParams pp = prefill_params();
        pp.q = static_cast<const uint16_t*>(q);
        pp.k_pool = static_cast<const uint16_t*>(k_pool);
        pp.v_pool = static_cast<const uint16_t*>(v_pool);
        pp.block_tables = block_tables;
        pp.qo_indptr = qo_indptr;
        pp.kv_len = kv_len;
        pp.out = static_cast<uint16_t*>(out);
        pp.lse = lse;
        pp.max_blocks = max_blocks_per_req;
        pp.num_q_heads = g->num_q_heads;
        pp.num_kv_heads = g->num_kv_heads;
        pp.num_vheads = vheads;
        pp.num_blocks = g->num_blocks;
        pp.num_prefill_rows = plan->num_prefill_rows;
        pp.splits = plan->prefill_splits;
        const bool split = plan->prefill_splits > 1;
        pp.counters = split ? reinterpret_cast<uint32_t*>(wsp + ws.counters) + ws.pf_counter_base : nullptr;
        pp.part_o = split ? reinterpret_cast<float*>(wsp + ws.pf_part_o) : nullptr;
        pp.part_lse = split ? reinterpret_cast<float*>(wsp + ws.pf_part_lse) : nullptr;
        pp.scale_log2 = scale_log2;
        pp.v_scale = out_v_scale;
        pp.k_div = k_scale;
        pp.v_div = v_scale;
        for (int i = 0; i < PA_MAX_PREFILL_ROWS; ++i)
            pp.prefill_req[i] = i < plan->num_prefill_rows ? plan->prefill_req[i] : 0;
        for (int i = 0; i <= PA_MAX_PREFILL_ROWS; ++i)
            pp.tile_start[i] = i <= plan->num_prefill_rows ? plan->prefill_tile_start[i] : plan->prefill_tiles;
        const int64_t grid = (int64_t)plan->prefill_tiles * vheads * plan->prefill_splits;
        if (grid > INT32_MAX)
            return PA_ERR_SHAPE;
        pp.k_new = static_cast<const uint16_t*>(k_new);
        pp.v_new = static_cast<const uint16_t*>(v_new);
        if (one_launch) {
            mixed_pp = pp;
            mixed_prefill_wgs = grid;
        } else if (append_in_decode) {
            int32_t most_tiles = 0;
            for (int i = 0; i < plan->num_prefill_rows; ++i)
                most_tiles = std::max(most_tiles, plan->prefill_tile_start[i + 1] - plan->prefill_tile_start[i]);
            const int64_t pieces = (int64_t)most_tiles * plan->prefill_tile_tokens * g->num_kv_heads *
                                   (q8 ? kHeadDim / pa::kQ8Group : fp8 ? kHeadDim / 16 : kHeadDim / 8);
            const int64_t per_row = std::max<int64_t>((pieces + 64 * kDecodeWaves - 1) / (64 * kDecodeWaves), 1);
            if (per_row * plan->num_prefill_rows > INT32_MAX / 2)
                return PA_ERR_SHAPE;
            append_wgs_per_row = (int32_t)per_row;
            later_pp = pp;
            later_grid = grid;
        } else {
            if (fused) {
                // the chunk rows' new tokens go into the pool first (encoded on a quantised
                // pool), then the tiles read them there; the decode rows keep the fused append
                int32_t most_tiles = 0;
                for (int i = 0; i < plan->num_prefill_rows; ++i)
                    most_tiles = std::max(most_tiles, plan->prefill_tile_start[i + 1] - plan->prefill_tile_start[i]);
                const int64_t pieces = (int64_t)most_tiles * plan->prefill_tile_tokens * g->num_kv_heads *
                                       (q8 ? kHeadDim / pa::kQ8Group : fp8 ? kHeadDim / 16 : kHeadDim / 8);
                const int64_t bx = (pieces + 255) / 256;
                if (bx > INT32_MAX)
                    return PA_ERR_SHAPE;
                const dim3 agrid((uint32_t)std::max<int64_t>(bx, 1), (uint32_t)plan->num_prefill_rows);
                if (q8)
                    hipLaunchKernelGGL(pa_append_chunk_rows<kFmtQ8>, agrid, dim3(256), 0, st, pp);
                else if (fp8)
                    hipLaunchKernelGGL(pa_append_chunk_rows<kFmtFp8>, agrid, dim3(256), 0, st, pp);
                else
                    hipLaunchKernelGGL(pa_append_chunk_rows<kFmtBf16>, agrid, dim3(256), 0, st, pp);
            }
            launch_prefill_tiles(q8, fp8, q8 ? 128 : kGroup * plan->prefill_tile_tokens, (uint32_t)grid, st, pp);
        }
        if (!one_launch && hipGetLastError() != hipSuccess)
            return PA_ERR_HIP;
    }
    if (plan->num_decode_rows > 0 && plan->max_splits > 0) {
        DecodeParams dp;
        dp.q = static_cast<const uint16_t*>(q);
        dp.k_pool = static_cast<const uint16_t*>(k_pool);
        dp.v_pool = static_cast<const uint16_t*>(v_pool);
        dp.block_tables = block_tables;
        dp.qo_indptr = qo_indptr;
        dp.kv_len = kv_len;
        dp.out = static_cast<uint16_t*>(out);
        dp.lse = lse;
        const bool partials = plan->max_splits > 1 || ngroups > 0;
        dp.counters = partials ? reinterpret_cast<uint32_t*>(wsp + ws.counters) : nullptr;
        dp.part_o = partials ? reinterpret_cast<float*>(wsp + ws.part_o) : nullptr;
        dp.part_lse = partials ? reinterpret_cast<float*>(wsp + ws.part_lse) : nullptr;
        dp.max_blocks = max_blocks_per_req;
        dp.num_reqs = plan->num_reqs;
        dp.num_q_heads = g->num_q_heads;
        dp.num_kv_heads = g->num_kv_heads;
        dp.num_vheads = vheads;
        dp.num_blocks = g->num_blocks;
        dp.split_blocks = plan->split_blocks;
        dp.max_splits = plan->max_splits;
        dp.scale_log2 = scale_log2;
        dp.v_scale = out_v_scale;
        dp.k_div = k_scale;
        dp.v_div = v_scale;
        dp.num_prefix_groups = ngroups;
        dp.prefix_splits = ngroups > 0 ? plan->prefix_splits : 0;
        for (int i = 0; i < PA_MAX_PREFIX_GROUPS; ++i) {
            dp.prefix_first[i] = i < ngroups ? plan->prefix_first_req[i] : 0;
            dp.prefix_count[i] = i < ngroups ? plan->prefix_num_reqs[i] : 0;
            dp.prefix_blocks[i] = i < ngroups ? plan->prefix_blocks[i] : 0;
        }
        dp.px_part_o = ngroups > 0 ? reinterpret_cast<float*>(wsp + ws.px_part_o) : nullptr;
        dp.px_part_lse = ngroups > 0 ? reinterpret_cast<float*>(wsp + ws.px_part_lse) : nullptr;
        dp.k_new = static_cast<const uint16_t*>(k_new);
        dp.v_new = static_cast<const uint16_t*>(v_new);
        const int64_t grid = (int64_t)plan->max_splits * plan->num_reqs * vheads;
        if (ngroups > 0) {
            // each group's shared blocks, once per KV head, for all of its query rows, in
            // the same launch as the decode workgroups
            PrefillParams pp = prefill_params();
            pp.splits = plan->prefix_splits;
            for (int i = 0; i < ngroups; ++i) {
                pp.group_first[i] = plan->prefix_first_req[i];
                pp.group_count[i] = plan->prefix_num_reqs[i];
                pp.group_blocks[i] = plan->prefix_blocks[i];
            }
            pp.px_part_o = reinterpret_cast<float*>(wsp + ws.px_part_o);
            pp.px_part_lse = reinterpret_cast<float*>(wsp + ws.px_part_lse);
            const int64_t nprefix = (int64_t)ngroups * vheads * plan->prefix_splits;
            if (grid + nprefix > INT32_MAX)
                return PA_ERR_SHAPE;
            launch_cascade(q8, fused, fp8, q8 ? 128 : plan->prefix_tile_rows, (uint32_t)(grid + nprefix), st, pp, dp,
                           (int32_t)nprefix);
        } else if (one_launch) {
            if (grid + mixed_prefill_wgs > INT32_MAX)
                return PA_ERR_SHAPE;
            const dim3 blocks((uint32_t)(grid + mixed_prefill_wgs));
            if (fused)
                hipLaunchKernelGGL((pa_mixed_batch<true>), blocks, dim3(64 * kPfWaves), 0, st, mixed_pp, dp,
                                   (int32_t)mixed_prefill_wgs, (int32_t)grid, (int32_t)(plan->one_launch == 2));
            else
                hipLaunchKernelGGL((pa_mixed_batch<false>), blocks, dim3(64 * kPfWaves), 0, st, mixed_pp, dp,
                                   (int32_t)mixed_prefill_wgs, (int32_t)grid, (int32_t)(plan->one_launch == 2));
        } else if (append_in_decode) {
            const int64_t total = grid + (int64_t)append_wgs_per_row * plan->num_prefill_rows;
            if (total > INT32_MAX)
                return PA_ERR_SHAPE;
            if (q8)
                hipLaunchKernelGGL((pa_decode_split_append<true, false>), dim3((uint32_t)total), dim3(64 * kDecodeWaves),
                                   0, st, dp, later_pp, (int32_t)grid, append_wgs_per_row);
            else if (fp8)
                hipLaunchKernelGGL((pa_decode_split_append<false, true>), dim3((uint32_t)total), dim3(64 * kDecodeWaves),
                                   0, st, dp, later_pp, (int32_t)grid, append_wgs_per_row);
            else
                hipLaunchKernelGGL((pa_decode_split_append<false, false>), dim3((uint32_t)total),
                                   dim3(64 * kDecodeWaves), 0, st, dp, later_pp, (int32_t)grid, append_wgs_per_row);
            if (hipGetLastError() != hipSuccess)
                return PA_ERR_HIP;
            launch_prefill_tiles(q8, fp8, q8 ? 128 : kGroup * plan->prefill_tile_tokens, (uint32_t)later_grid, st,
                                 later_pp);
        } else {
            if (grid > INT32_MAX)
                return PA_ERR_SHAPE;
            if (q8)
                hipLaunchKernelGGL((fused ? pa_decode_split<true, true> : pa_decode_split<true, false>),
                                   dim3((uint32_t)grid), dim3(64 * kDecodeWaves), 0, st, dp);
            else if (fp8)
                hipLaunchKernelGGL((fused ? pa_decode_split<false, true, true> : pa_decode_split<false, false, true>),
                                   dim3((uint32_t)grid), dim3(64 * kDecodeWaves), 0, st, dp);
            else if (fused)
                hipLaunchKernelGGL((pa_decode_split<false, true>), dim3((uint32_t)grid), dim3(64 * kDecodeWaves), 0, st,
                                   dp);
            else
                hipLaunchKernelGGL((pa_decode_split<false, false>), dim3((uint32_t)grid), dim3(64 * kDecodeWaves), 0, st,
                                   dp);
        }
        if (hipGetLastError() != hipSuccess)
            return PA_ERR_HIP;
    }
    return PA_OK;
}

extern "C" pa_status pa_attention_batch(const pa_geometry* g, const pa_plan_t* plan, const void* q,
                                        const void* k_pool, const void* v_pool, const int32_t* block_tables,
                                        int32_t max_blocks_per_req, const int32_t* qo_indptr, const int32_t* kv_len,
                                        void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream)
{
    return attention_batch(false, g, plan, q, k_pool, v_pool, block_tables, max_blocks_per_req, qo_indptr, kv_len,
                           out, lse, workspace, workspace_bytes, stream);
}

extern "C" pa_status pa_decode_step(const pa_geometry* g, const pa_plan_t* plan, const void* q, void* k_pool,
                                    void* v_pool, const void* k_new, const void* v_new, const int32_t* block_tables,
                                    int32_t max_blocks_per_req, const int32_t* qo_indptr, const int32_t* kv_len,
                                    void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream)
{
    if (!g || !plan)
        return PA_ERR_NULL;
    if (plan->num_prefill_rows > 0 || plan->prefill_tiles > 0)
        return PA_ERR_UNSUPPORTED;                 // decode rows only
    if (plan->num_reqs > 0 && plan->total_q > 0 && (!k_new || !v_new))
        return PA_ERR_NULL;
    return attention_batch(false, g, plan, q, k_pool, v_pool, block_tables, max_blocks_per_req, qo_indptr, kv_len,
                           out, lse, workspace, workspace_bytes, stream, k_new, v_new);
}

extern "C" pa_status pa_attention_step(const pa_geometry* g, const pa_plan_t* plan, const void* q, void* k_pool,
                                       void* v_pool, const void* k_new, const void* v_new, const int32_t* block_tables,
                                       int32_t max_blocks_per_req, const int32_t* qo_indptr, const int32_t* kv_len,
                                       void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream)
{
    if (!g || !plan)
        return PA_ERR_NULL;
    if (plan->num_reqs > 0 && plan->total_q > 0 && (!k_new || !v_new))
        return PA_ERR_NULL;
    return attention_batch(false, g, plan, q, k_pool, v_pool, block_tables, max_blocks_per_req, qo_indptr, kv_len,
                           out, lse, workspace, workspace_bytes, stream, k_new, v_new);
}

extern "C" pa_status pa_attention_batch_q8(const pa_geometry* g, const pa_plan_t* plan, const void* q,
                                           const void* kv_pool_q8, const int32_t* block_tables,
                                           int32_t max_blocks_per_req, const int32_t* qo_indptr, const int32_t* kv_len,
                                           void* out, float* lse, void* workspace, size_t workspace_bytes,
                                           void* stream)
{
    return attention_batch(true, g, plan, q, kv_pool_q8, kv_pool_q8, block_tables, max_blocks_per_req, qo_indptr,
                           kv_len, out, lse, workspace, workspace_bytes, stream);
}

extern "C" pa_status pa_attention_batch_fp8(const pa_geometry* g, const pa_plan_t* plan, const void* q,
                                            const void* k_pool_fp8, const void* v_pool_fp8, const int32_t* block_tables,
                                            int32_t max_blocks_per_req, const int32_t* qo_indptr, const int32_t* kv_len,
                                            void* out, float* lse, void* workspace, size_t workspace_bytes,
                                            float k_scale, float v_scale, void* stream)
{
    return attention_batch(false, g, plan, q, k_pool_fp8, v_pool_fp8, block_tables, max_blocks_per_req, qo_indptr,
                           kv_len, out, lse, workspace, workspace_bytes, stream, nullptr, nullptr, true, k_scale,
                           v_scale);
}

extern "C" pa_status pa_decode_step_q8(const pa_geometry* g, const pa_plan_t* plan, const void* q, void* kv_pool_q8,
                                       const void* k_new, const void* v_new, const int32_t* block_tables,
                                       int32_t max_blocks_per_req, const int32_t* qo_indptr, const int32_t* kv_len,
                                       void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream)
{
    if (!g || !plan)
        return PA_ERR_NULL;
    if (plan->num_prefill_rows > 0 || plan->prefill_tiles > 0)
        return PA_ERR_UNSUPPORTED;                 // decode rows only
    if (plan->num_reqs > 0 && plan->total_q > 0 && (!k_new || !v_new))
        return PA_ERR_NULL;
    return attention_batch(true, g, plan, q, kv_pool_q8, kv_pool_q8, block_tables, max_blocks_per_req, qo_indptr,
                           kv_len, out, lse, workspace, workspace_bytes, stream, k_new, v_new);
}

extern "C" pa_status pa_attention_step_q8(const pa_geometry* g, const pa_plan_t* plan, const void* q, void* kv_pool_q8,
                                          const void* k_new, const void* v_new, const int32_t* block_tables,
                                          int32_t max_blocks_per_req, const int32_t* qo_indptr, const int32_t* kv_len,
                                          void* out, float* lse, void* workspace, size_t workspace_bytes,
                                          void* stream)
{
    if (!g || !plan)
        return PA_ERR_NULL;
    if (plan->num_reqs > 0 && plan->total_q > 0 && (!k_new || !v_new))
        return PA_ERR_NULL;
    return attention_batch(true, g, plan, q, kv_pool_q8, kv_pool_q8, block_tables, max_blocks_per_req, qo_indptr,
                           kv_len, out, lse, workspace, workspace_bytes, stream, k_new, v_new);
}

extern "C" pa_status pa_decode_step_fp8(const pa_geometry* g, const pa_plan_t* plan, const void* q, void* k_pool_fp8,
                                        void* v_pool_fp8, const void* k_new, const void* v_new,
                                        const int32_t* block_tables, int32_t max_blocks_per_req,
                                        const int32_t* qo_indptr, const int32_t* kv_len, void* out, float* lse,
                                        void* workspace, size_t workspace_bytes, float k_scale, float v_scale,
                                        void* stream)
{
    if (!g || !plan)
        return PA_ERR_NULL;
    if (plan->num_prefill_rows > 0 || plan->prefill_tiles > 0)
        return PA_ERR_UNSUPPORTED;                 // decode rows only
    if (plan->num_reqs > 0 && plan->total_q > 0 && (!k_new || !v_new))
        return PA_ERR_NULL;
    return attention_batch(false, g, plan, q, k_pool_fp8, v_pool_fp8, block_tables, max_blocks_per_req, qo_indptr,
                           kv_len, out, lse, workspace, workspace_bytes, stream, k_new, v_new, true, k_scale, v_scale);
}

extern "C" pa_status pa_attention_step_fp8(const pa_geometry* g, const pa_plan_t* plan, const void* q,
                                           void* k_pool_fp8, void* v_pool_fp8, const void* k_new, const void* v_new,
                                           const int32_t* block_tables, int32_t max_blocks_per_req,
                                           const int32_t* qo_indptr, const int32_t* kv_len, void* out, float* lse,
                                           void* workspace, size_t workspace_bytes, float k_scale, float v_scale,
                                           void* stream)
{
    if (!g || !plan)
        return PA_ERR_NULL;
    if (plan->num_reqs > 0 && plan->total_q > 0 && (!k_new || !v_new))
        return PA_ERR_NULL;
    return attention_batch(false, g, plan, q, k_pool_fp8, v_pool_fp8, block_tables, max_blocks_per_req, qo_indptr,
                           kv_len, out, lse, workspace, workspace_bytes, stream, k_new, v_new, true, k_scale, v_scale);
}

extern "C" pa_status pa_query_num_cus(int32_t device, int32_t* num_cus)
{
    if (!num_cus)
        return PA_ERR_NULL;
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
        return PA_ERR_HIP;
    *num_cus = v;
    return PA_OK;
}

// ------------------------------------------------------------------------------ allocation-free entry

// Scratch memory of pa_attention_batch_noalloc: the completion counters and split
// partials that pa_attention_batch keeps in the caller's workspace, in a fixed array that
// every device holds from the moment the library's code is loaded on it until the process
// ends.  Host code must never use the array's name as an address (it names a host-side
// stand-in); it uses the device address that hipGetSymbolAddress returns for the current
// device, kept in g_scratch below.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxScratchDevices] = {};

// This device's copy of `scratch`, looked up once per device.  The first call on a device
// also zeroes the completion counters on `stream` (the array starts zeroed when it is
// loaded; every call leaves the counters zero again).
pa_status scratch_for_device(int device, hipStream_t stream, void** out)
{
    if (device < 0 || device >= kMaxScratchDevices)
        return PA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch[device]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
            return PA_ERR_HIP;
        constexpr int64_t words = pa::kCounterBytes / sizeof(uint32_t);
        hipLaunchKernelGGL(pa_zero_words, dim3((uint32_t)((words + 255) / 256)), dim3(256), 0, stream,
                           static_cast<uint32_t*>(ptr), words);
        if (hipGetLastError() != hipSuccess)
            return PA_ERR_HIP;
        g_scratch[device] = ptr;
    }
    *out = g_scratch[device];
    return PA_OK;
}

}  // namespace

extern "C" pa_status pa_attention_batch_noalloc(const pa_geometry* g, const pa_plan_t* plan, const void* q,
                                                const void* k_pool, const void* v_pool, const int32_t* block_tables,
                                                int32_t max_blocks_per_req, const int32_t* qo_indptr,
                                                const int32_t* kv_len, void* out, float* lse, void* stream)
{
    if (!g || !plan)
        return PA_ERR_NULL;
    if (plan->workspace_bytes > PA_NOALLOC_SCRATCH_BYTES)
        return PA_ERR_WORKSPACE;
    void* ws = nullptr;
    if (plan->workspace_bytes > 0) {
        // the scratch copy must be that of the device the stream runs on
        int current = -1;
        hipDevice_t stream_device = -1;
        if (hipGetDevice(&current) != hipSuccess)
            return PA_ERR_HIP;
        if (stream && hipStreamGetDevice(as_stream(stream), &stream_device) != hipSuccess)
            return PA_ERR_HIP;
        if (stream && stream_device != current)
            return PA_ERR_UNSUPPORTED;
        const pa_status st = scratch_for_device(current, as_stream(stream), &ws);
        if (st != PA_OK)
            return st;
    }
    return attention_batch(false, g, plan, q, k_pool, v_pool, block_tables, max_blocks_per_req, qo_indptr, kv_len,
                           out, lse, ws, ws ? (size_t)PA_NOALLOC_SCRATCH_BYTES : 0, stream);
}

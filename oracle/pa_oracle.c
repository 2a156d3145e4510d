/*
 * Plain CPU oracle for paged-KV attention over a mixed decode / chunked-prefill
 * batch.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU baseline call it; the product library never does.  It shares
 * no code, header or table with the GPU library.
 *
 * It is the plain definition, written out slowly in double precision:
 *
 *   append     For every new token t with slot s = slot_mapping[t] >= 0, copy its
 *              K and V rows for every KV head into pool[s / B][head][s % B][:].
 *              Blocks of B tokens, a per-request block table from logical to
 *              physical block, and new tokens written into the slot that the
 *              table gives (AI-infra book ch. 8 "Inference optimisation",
 *              section 8.3.1 and fig. 8-10; the Perplexity blog on prefill /
 *              decode disaggregation orders the per-layer append before attention).
 *
 *   attention  For request r, new token i in [0, qo_len) and query head h:
 *                p    = kv_len - qo_len + i        (absolute position of the token)
 *                kvh  = h / (Hq / Hkv)             (grouped-query attention: each KV
 *                                                   head serves a contiguous group)
 *                s_j  = scale * sum_c q[c] * K_j[c]   for j = 0..p, K_j read through the
 *                                                   block table: K_pool[bt[r][j/B]][kvh][j%B]
 *                LSE  = ln sum_j exp(s_j)          (natural log)
 *                o[c] = sum_j exp(s_j - LSE) * V_j[c]
 *              The i-th new token of a chunk at context h sees h + i + 1 keys, i.e.
 *              itself and everything before it (book section 8.2.3, the N_pair sum
 *              and figs. 8-8 / 8-9).  The output is rounded to bf16 (nearest even),
 *              the LSE is stored as float.
 *
 * Everything is accumulated in double; the scores are kept and exponentiated
 * in a second pass (max subtracted first), which is mathematically the same
 * as any one-pass or split form of softmax.
 *
 *   q8_0 pool  (book section 8.4.2 and fig. 8-23: every 32 values share one 2-byte
 *              scale and are stored as 8-bit codes, 34 bytes instead of 64.)  A group
 *              is 32 consecutive dims of one token's row for one KV head.  The K (or
 *              V) tile of one (block, KV head) holds the codes of its B tokens, [B][D]
 *              int8, followed by their scales, [B][D / 32] IEEE binary16; the pool
 *              keeps each (block, KV head)'s K tile and V tile side by side,
 *              [num_blocks][Hkv][2][tile bytes].  The pages fix
 *              neither the scale's type nor the rounding; the readings taken here:
 *                d    = binary16(min(amax / 127, 65504)), amax = max |x| of the group,
 *                       the division in binary32, the conversion to nearest (ties even)
 *                code = clamp(rint(x / d), -127, 127) with x / d in binary32 and rint
 *                       to nearest, ties even; code = 0 when d = 0
 *                value represented = code * d
 *              Append quantises each new row this way; attention is the definition
 *              above applied to the represented values.
 *
 *   FP8 pool   (book section 8.4.4: KV stored in FP8 while Q stays BF16, figs. 8-27 and
 *              8-28; section 8.4.2's cost model ΔT = ΔD/β − T_c with the H100 BF16 and FP8
 *              slopes.)  The pages fix neither the FP8 encoding nor the scale's
 *              granularity; the readings taken here: OCP FP8 E4M3 (1 sign bit, 4
 *              exponent bits with bias 7, 3 fraction bits, no infinities, S.1111.111 =
 *              NaN, largest magnitude 448), one binary32 scale per pool (k_scale for K,
 *              v_scale for V), the bf16 pool's layout with one byte per value, and
 *                code = e4m3(y), y = x / scale in binary32, to nearest with ties to
 *                       even, magnitudes above 448 (infinities too) saturating to 448,
 *                       and a NaN stored as the NaN code 0x7F
 *                value represented = decode(code) * scale
 *              Append stores each new value this way; attention is the definition
 *              above applied to the represented values.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_BAD_BLOCK 2
#define ORACLE_NO_MEMORY 3

static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bf16 value, ties to even, in one rounding step.
 * bf16 keeps 8 significant bits; a finite x with |x| = m * 2^e (m in [0.5, 1))
 * lies between two neighbours that are multiples of 2^(e-8) (normal range) or
 * of 2^-133 (subnormal range). */
uint16_t oracle_double_to_bf16(double x)
{
    if (isnan(x))
        return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isinf(a))
        return sign | 0x7F80;
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);
    int qexp = (e > -125 ? e : -125) - 8;
    double quantum = ldexp(1.0, qexp);
    double lo = floor(a / quantum);        /* exact: a / quantum scales by a power of two */
    double below = lo * quantum, above = (lo + 1.0) * quantum;
    double dlo = a - below, dhi = above - a;
    double r;
    if (dlo < dhi)
        r = below;
    else if (dhi < dlo)
        r = above;
    else
        r = (fmod(lo, 2.0) == 0.0) ? below : above;
    /* largest finite bf16 is (2 - 2^-7) * 2^127; anything that rounds past it is infinite */
    if (r >= ldexp(1.0, 128))
        return sign | 0x7F80;
    float f = (float)r;                    /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)((u >> 16) & 0x7FFF);
}

double oracle_bf16_to_double(uint16_t b) { return bf16_to_double(b); }

/* Pool slot of logical position pos of one request: bt_row[pos / B] * B + pos % B. */
int64_t oracle_slot(const int32_t* bt_row, int64_t pos, int32_t block_size)
{
    return (int64_t)bt_row[pos / block_size] * block_size + pos % block_size;
}

/* IEEE binary16 -> double: sign, 5-bit exponent (bias 15), 10-bit fraction. */
static double half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1, e = (h >> 10) & 31, f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                     /* zero and subnormals: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp(1.0 + f / 1024.0, e - 15);
    return sign ? -v : v;
}

double oracle_half_to_double(uint16_t h) { return half_to_double(h); }

/* binary32 -> binary16, to nearest with ties to even.  Normal results keep 11
 * significant bits (quantum 2^(E-10) for |x| in [2^E, 2^(E+1))); below 2^-14 the
 * quantum is 2^-24.  Everything is done in double, where these scalings are exact. */
uint16_t oracle_float_to_half(float x)
{
    if (isnan(x))
        return 0x7E00;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs((double)x);
    if (isinf(a))
        return sign | 0x7C00;
    int e;
    frexp(a, &e);                                  /* a = m * 2^e, m in [0.5, 1) */
    int E = e - 1;                                 /* a in [2^E, 2^(E+1)) */
    int qexp = (E < -14 ? -14 : E) - 10;
    double units = nearbyint(a / ldexp(1.0, qexp));   /* default rounding: nearest, ties even */
    double r = units * ldexp(1.0, qexp);
    if (r > 65504.0)                               /* past the largest finite binary16 */
        return sign | 0x7C00;
    if (r < ldexp(1.0, -14))                       /* subnormal (or zero): fraction = r / 2^-24 */
        return sign | (uint16_t)nearbyint(r / ldexp(1.0, -24));
    int er;
    frexp(r, &er);
    int Er = er - 1;
    uint16_t frac = (uint16_t)nearbyint((r / ldexp(1.0, Er) - 1.0) * 1024.0);
    return sign | (uint16_t)((Er + 15) << 10) | frac;
}

/* OCP FP8 E4M3 code -> double: (-1)^s * 2^(e-7) * (1 + f/8) for e >= 1, (-1)^s * 2^-6 *
 * (f/8) for e = 0, NaN for e = 15 and f = 7 (the format has no infinities). */
static double e4m3_to_double(uint8_t c)
{
    const double sign = (c & 0x80) ? -1.0 : 1.0;
    const int e = (c >> 3) & 15, f = c & 7;
    if (e == 15 && f == 7)
        return NAN;
    if (e == 0)
        return sign * ldexp((double)f, -9);
    return sign * ldexp(8.0 + f, e - 10);
}

double oracle_e4m3_to_double(uint8_t c) { return e4m3_to_double(c); }

/* double -> E4M3 code, to nearest with ties to even; magnitudes above 448 become 448,
 * a NaN becomes 0x7F.  Below 2^-6 the quantum is 2^-9 (subnormal codes 0..7; a rounded
 * count of 8 is the smallest normal, code 8); in [2^E, 2^(E+1)) it is 2^(E-3). */
uint8_t oracle_double_to_e4m3(double x)
{
    if (isnan(x))
        return 0x7F;
    const uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs(x);
    if (a > 448.0)
        a = 448.0;
    if (a < 0.015625) {
        const double k = nearbyint(ldexp(a, 9));          /* 0 .. 8, ties to even */
        return (uint8_t)(sign | (uint8_t)k);
    }
    int E;
    const double m = frexp(a, &E);                         /* a = m * 2^E, m in [0.5, 1) */
    int e = E - 1;                                         /* a in [2^e, 2^(e+1)) */
    double f = nearbyint(ldexp(m, 4) - 8.0);               /* (a / 2^e - 1) * 8, ties to even */
    if (f == 8.0) {
        f = 0.0;
        ++e;
    }
    return (uint8_t)(sign | (uint8_t)(((e + 7) << 3) | (int)f));
}

/* One q8_0 group of 32 bf16 values -> 32 codes and the scale's binary16 bits. */
static void quantize_q8_group(const uint16_t* x, int8_t* codes, uint16_t* scale)
{
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) {
        float v = fabsf((float)bf16_to_double(x[i]));
        if (v > amax)
            amax = v;
    }
    float d = amax / 127.0f;
    if (d > 65504.0f)
        d = 65504.0f;
    *scale = oracle_float_to_half(d);
    float dw = (float)half_to_double(*scale);
    for (int i = 0; i < 32; ++i) {
        float c = 0.0f;
        if (dw != 0.0f) {
            c = rintf((float)bf16_to_double(x[i]) / dw);
            if (c > 127.0f)
                c = 127.0f;
            if (c < -127.0f)
                c = -127.0f;
        }
        codes[i] = (int8_t)c;
    }
}

/* q8_0 of n rows of head_dim bf16 values: codes [n][D], scales [n][D / 32]. */
int oracle_quantize_q8_rows(const uint16_t* x, int64_t n, int32_t head_dim, int8_t* codes, uint16_t* scales)
{
    if (!x || !codes || !scales || head_dim % 32 != 0 || n < 0)
        return ORACLE_BAD_ARG;
    for (int64_t r = 0; r < n; ++r)
        for (int32_t g = 0; g < head_dim / 32; ++g)
            quantize_q8_group(x + r * head_dim + g * 32, codes + r * head_dim + g * 32,
                              scales + r * (head_dim / 32) + g);
    return ORACLE_OK;
}

/* Bytes of one q8_0 (block, KV head) tile. */
int64_t oracle_q8_tile_bytes(int32_t head_dim, int32_t block_size)
{
    return (int64_t)block_size * head_dim + (int64_t)block_size * (head_dim / 32) * 2;
}

/* append into a q8_0 pool [num_blocks][Hkv][2][tile bytes] (K tile, then V tile);
 * k_new / v_new are bf16 [n][Hkv][D]. */
int oracle_append_q8(uint8_t* kv_pool, const uint16_t* k_new, const uint16_t* v_new, const int32_t* slot_mapping,
                     int32_t n_tokens, int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks)
{
    if (!kv_pool || !k_new || !v_new || (!slot_mapping && n_tokens > 0) || n_tokens < 0 || head_dim % 32 != 0)
        return ORACLE_BAD_ARG;
    const int64_t tile = oracle_q8_tile_bytes(head_dim, block_size);
    const int32_t groups = head_dim / 32;
    for (int32_t t = 0; t < n_tokens; ++t) {
        int64_t s = slot_mapping[t];
        if (s < 0)
            continue;
        int64_t blk = s / block_size, off = s % block_size;
        if (blk >= num_blocks)
            return ORACLE_BAD_BLOCK;
        for (int32_t h = 0; h < num_kv_heads; ++h) {
            size_t src = ((size_t)t * num_kv_heads + h) * head_dim;
            for (int which = 0; which < 2; ++which) {
                uint8_t* base = kv_pool + (((size_t)blk * num_kv_heads + h) * 2 + which) * tile;
                const uint16_t* row = (which ? v_new : k_new) + src;
                for (int32_t g = 0; g < groups; ++g) {
                    uint16_t sc;
                    quantize_q8_group(row + g * 32, (int8_t*)(base + off * head_dim + g * 32), &sc);
                    memcpy(base + (size_t)block_size * head_dim + ((size_t)off * groups + g) * 2, &sc, 2);
                }
            }
        }
    }
    return ORACLE_OK;
}

/* append: pools are [num_blocks][Hkv][B][D] bf16; k_new / v_new are [n][Hkv][D]. */
int oracle_append(uint16_t* k_pool, uint16_t* v_pool, const uint16_t* k_new, const uint16_t* v_new,
                  const int32_t* slot_mapping, int32_t n_tokens, int32_t num_kv_heads, int32_t head_dim,
                  int32_t block_size, int32_t num_blocks)
{
    if (!k_pool || !v_pool || !k_new || !v_new || (!slot_mapping && n_tokens > 0) || n_tokens < 0)
        return ORACLE_BAD_ARG;
    for (int32_t t = 0; t < n_tokens; ++t) {
        int64_t s = slot_mapping[t];
        if (s < 0)
            continue;                      /* negative slot: token not cached */
        int64_t blk = s / block_size, off = s % block_size;
        if (blk >= num_blocks)
            return ORACLE_BAD_BLOCK;
        for (int32_t h = 0; h < num_kv_heads; ++h) {
            size_t dst = (((size_t)blk * num_kv_heads + h) * block_size + off) * head_dim;
            size_t src = ((size_t)t * num_kv_heads + h) * head_dim;
            memcpy(k_pool + dst, k_new + src, sizeof(uint16_t) * head_dim);
            memcpy(v_pool + dst, v_new + src, sizeof(uint16_t) * head_dim);
        }
    }
    return ORACLE_OK;
}

/* append into FP8 pools [num_blocks][Hkv][B][D] (one E4M3 code per value): each new bf16
 * value x is stored as e4m3(x / scale), the division in binary32 (k_scale for K rows,
 * v_scale for V rows); k_new / v_new are bf16 [n][Hkv][D]. */
int oracle_append_fp8(uint8_t* k_pool, uint8_t* v_pool, const uint16_t* k_new, const uint16_t* v_new,
                      const int32_t* slot_mapping, int32_t n, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t num_blocks, float k_scale, float v_scale)
{
    if (!k_pool || !v_pool || (n > 0 && (!k_new || !v_new || !slot_mapping)) || n < 0 || !(k_scale > 0.0f) ||
        !(v_scale > 0.0f))
        return ORACLE_BAD_ARG;
    const int64_t num_slots = (int64_t)num_blocks * block_size;
    for (int32_t t = 0; t < n; ++t) {
        const int64_t slot = slot_mapping[t];
        if (slot < 0)
            continue;
        if (slot >= num_slots)
            return ORACLE_BAD_BLOCK;
        const int64_t blk = slot / block_size, off = slot % block_size;
        for (int32_t h = 0; h < num_kv_heads; ++h) {
            const size_t dst = (((size_t)blk * num_kv_heads + h) * block_size + (size_t)off) * head_dim;
            const size_t src = ((size_t)t * num_kv_heads + h) * head_dim;
            for (int32_t c = 0; c < head_dim; ++c) {
                const float ky = (float)bf16_to_double(k_new[src + c]) / k_scale;
                const float vy = (float)bf16_to_double(v_new[src + c]) / v_scale;
                k_pool[dst + c] = oracle_double_to_e4m3((double)ky);
                v_pool[dst + c] = oracle_double_to_e4m3((double)vy);
            }
        }
    }
    return ORACLE_OK;
}

/*
 * block copy (book section 8.3.2, copy-on-write: the writer gets a private copy of a
 * shared block): block src[i]'s tiles of every KV head, K and V, become block dst[i]'s.
 * The pairs are applied in order; a valid list never writes a block it later reads.
 */
static int copy_blocks_bytes(uint8_t* k_pool, uint8_t* v_pool, const int32_t* src, const int32_t* dst, int32_t n,
                             size_t block_bytes, int32_t num_blocks)
{
    if (!k_pool || !v_pool || (n > 0 && (!src || !dst)) || n < 0)
        return ORACLE_BAD_ARG;
    for (int32_t i = 0; i < n; ++i) {
        if (src[i] < 0 || src[i] >= num_blocks || dst[i] < 0 || dst[i] >= num_blocks)
            continue;                      /* out-of-range pair: skipped */
        memcpy(k_pool + (size_t)dst[i] * block_bytes, k_pool + (size_t)src[i] * block_bytes, block_bytes);
        memcpy(v_pool + (size_t)dst[i] * block_bytes, v_pool + (size_t)src[i] * block_bytes, block_bytes);
    }
    return ORACLE_OK;
}

int oracle_copy_blocks(uint16_t* k_pool, uint16_t* v_pool, const int32_t* src, const int32_t* dst, int32_t n,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks)
{
    return copy_blocks_bytes((uint8_t*)k_pool, (uint8_t*)v_pool, src, dst, n,
                             sizeof(uint16_t) * (size_t)num_kv_heads * block_size * head_dim, num_blocks);
}

/* block copy for FP8 pools (one byte per value). */
int oracle_copy_blocks_fp8(uint8_t* k_pool, uint8_t* v_pool, const int32_t* src, const int32_t* dst, int32_t n,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks)
{
    return copy_blocks_bytes(k_pool, v_pool, src, dst, n, (size_t)num_kv_heads * block_size * head_dim, num_blocks);
}

/*
 * attention.  q: [total_q][Hq][D] bf16 with rows of request r at qo_indptr[r]..;
 * out: same shape bf16; lse: [total_q][Hq] float.  block_tables: [R][max_blocks].
 * row_select (may be NULL): if given, only requests with row_select[r] != 0 are
 * computed and the other rows of the outputs are left untouched.  out_f64 / lse_f64
 * (may be NULL) receive the same results before rounding, for tests that need more
 * than bf16 resolution.  pair_count (may be NULL) receives the number of
 * (query, key) pairs visited for one head, summed over the computed rows: an
 * instrument for the causal mask.
 */
enum { FMT_BF16 = 0, FMT_Q8_0 = 1, FMT_FP8 = 2 };

/* The values of token `tok` of physical block `phys`, KV head kvh, as doubles.  q8_0:
 * `pool` points at the K or the V tile of (block 0, KV head 0), and the tiles of
 * consecutive (block, KV head) pairs lie two tiles apart. */
static void load_row(int fmt, const void* pool, int32_t phys, int32_t kvh, int32_t tok, int32_t num_kv_heads,
                     int32_t head_dim, int32_t block_size, double pool_scale, double* dst)
{
    if (fmt == FMT_FP8) {
        const uint8_t* src = (const uint8_t*)pool +
                             (((size_t)phys * num_kv_heads + kvh) * block_size + (size_t)tok) * head_dim;
        for (int32_t c = 0; c < head_dim; ++c)
            dst[c] = e4m3_to_double(src[c]) * pool_scale;
    } else if (fmt == FMT_BF16) {
        const uint16_t* src = (const uint16_t*)pool +
                              (((size_t)phys * num_kv_heads + kvh) * block_size + (size_t)tok) * head_dim;
        for (int32_t c = 0; c < head_dim; ++c)
            dst[c] = bf16_to_double(src[c]);
    } else {
        const uint8_t* tile = (const uint8_t*)pool +
                              ((size_t)phys * num_kv_heads + kvh) * 2 * (size_t)oracle_q8_tile_bytes(head_dim, block_size);
        const int8_t* codes = (const int8_t*)tile + (size_t)tok * head_dim;
        const uint8_t* sc = tile + (size_t)block_size * head_dim + (size_t)tok * (head_dim / 32) * 2;
        for (int32_t c = 0; c < head_dim; ++c) {
            uint16_t h;
            memcpy(&h, sc + (c / 32) * 2, 2);
            dst[c] = (double)codes[c] * half_to_double(h);
        }
    }
}

static int attention_impl(int fmt, const uint16_t* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_tables, int32_t max_blocks, const int32_t* qo_len,
                          const int32_t* kv_len, int32_t num_reqs, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t num_blocks, double scale,
                          double k_scale, double v_scale, const uint8_t* row_select, uint16_t* out, float* lse,
                          double* out_f64, double* lse_f64, int64_t* pair_count)
{
    if (!q || !k_pool || !v_pool || !block_tables || !qo_len || !kv_len)
        return ORACLE_BAD_ARG;
    if (num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 || head_dim <= 0 || block_size <= 0)
        return ORACLE_BAD_ARG;
    if (fmt == FMT_Q8_0 && head_dim % 32 != 0)
        return ORACLE_BAD_ARG;
    const int32_t group = num_q_heads / num_kv_heads;

    /* Row r's first query row is the sum of the earlier qo_len. */
    int64_t* first_row = (int64_t*)malloc(sizeof(int64_t) * (size_t)(num_reqs + 1));
    if (!first_row)
        return ORACLE_NO_MEMORY;
    first_row[0] = 0;
    for (int32_t r = 0; r < num_reqs; ++r) {
        if (qo_len[r] < 1 || kv_len[r] < qo_len[r] || (kv_len[r] + block_size - 1) / block_size > max_blocks) {
            free(first_row);
            return ORACLE_BAD_ARG;
        }
        first_row[r + 1] = first_row[r] + qo_len[r];
    }
    /* Every table entry that a row reads must name a pool block. */
    for (int32_t r = 0; r < num_reqs; ++r) {
        int32_t nb = (kv_len[r] + block_size - 1) / block_size;
        for (int32_t b = 0; b < nb; ++b) {
            int32_t phys = block_tables[(size_t)r * max_blocks + b];
            if (phys < 0 || phys >= num_blocks) {
                free(first_row);
                return ORACLE_BAD_BLOCK;
            }
        }
    }

    /* Work items: (request, new token, query head). */
    int64_t total = first_row[num_reqs] * num_q_heads;
    int64_t pairs = 0;
    int status = ORACLE_OK;

#pragma omp parallel reduction(+ : pairs)
    {
        int32_t max_kv = 0;
        for (int32_t r = 0; r < num_reqs; ++r)
            if (kv_len[r] > max_kv)
                max_kv = kv_len[r];
        double* s = (double*)malloc(sizeof(double) * (size_t)(max_kv > 0 ? max_kv : 1));
        double* acc = (double*)malloc(sizeof(double) * (size_t)head_dim);
        double* qd = (double*)malloc(sizeof(double) * (size_t)head_dim);
        double* kvrow = (double*)malloc(sizeof(double) * (size_t)head_dim);
        if (!s || !acc || !qd || !kvrow) {
#pragma omp atomic write
            status = ORACLE_NO_MEMORY;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t w = 0; w < total; ++w) {
                int64_t row = w / num_q_heads;
                int32_t h = (int32_t)(w % num_q_heads);
                int32_t r = 0;                         /* request owning this query row */
                while (first_row[r + 1] <= row)
                    ++r;
                if (row_select && !row_select[r])
                    continue;
                int32_t i = (int32_t)(row - first_row[r]);
                int32_t kvh = h / group;
                int64_t p = (int64_t)kv_len[r] - qo_len[r] + i;   /* keys 0..p are visible */
                const int32_t* bt = block_tables + (size_t)r * max_blocks;
                const uint16_t* qrow = q + ((size_t)row * num_q_heads + h) * head_dim;
                for (int32_t c = 0; c < head_dim; ++c)
                    qd[c] = bf16_to_double(qrow[c]);

                double m = -INFINITY;
                for (int64_t j = 0; j <= p; ++j) {
                    load_row(fmt, k_pool, bt[j / block_size], kvh, (int32_t)(j % block_size), num_kv_heads,
                             head_dim, block_size, k_scale, kvrow);
                    double dot = 0.0;
                    for (int32_t c = 0; c < head_dim; ++c)
                        dot += qd[c] * kvrow[c];
                    s[j] = scale * dot;
                    if (s[j] > m)
                        m = s[j];
                }
                pairs += p + 1;

                double l = 0.0;
                for (int32_t c = 0; c < head_dim; ++c)
                    acc[c] = 0.0;
                for (int64_t j = 0; j <= p; ++j) {
                    double e = exp(s[j] - m);
                    l += e;
                    load_row(fmt, v_pool, bt[j / block_size], kvh, (int32_t)(j % block_size), num_kv_heads,
                             head_dim, block_size, v_scale, kvrow);
                    for (int32_t c = 0; c < head_dim; ++c)
                        acc[c] += e * kvrow[c];
                }
                size_t orow = ((size_t)row * num_q_heads + h) * head_dim;
                for (int32_t c = 0; c < head_dim; ++c) {
                    if (out)
                        out[orow + c] = oracle_double_to_bf16(acc[c] / l);
                    if (out_f64)
                        out_f64[orow + c] = acc[c] / l;
                }
                if (lse)
                    lse[(size_t)row * num_q_heads + h] = (float)(m + log(l));
                if (lse_f64)
                    lse_f64[(size_t)row * num_q_heads + h] = m + log(l);
            }
        }
        free(s);
        free(acc);
        free(qd);
        free(kvrow);
    }
    free(first_row);
    if (pair_count)
        *pair_count = pairs / num_q_heads;
    return status;
}

int oracle_attention(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                     const int32_t* block_tables, int32_t max_blocks, const int32_t* qo_len,
                     const int32_t* kv_len, int32_t num_reqs, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t block_size, int32_t num_blocks, double scale,
                     const uint8_t* row_select, uint16_t* out, float* lse, double* out_f64,
                     double* lse_f64, int64_t* pair_count)
{
    return attention_impl(FMT_BF16, q, k_pool, v_pool, block_tables, max_blocks, qo_len, kv_len, num_reqs,
                          num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, 1.0, 1.0, row_select,
                          out, lse, out_f64, lse_f64, pair_count);
}

/* attention over FP8 pools [num_blocks][Hkv][B][D] (E4M3 codes) with scales k_scale / v_scale. */
int oracle_attention_fp8(const uint16_t* q, const uint8_t* k_pool, const uint8_t* v_pool,
                         const int32_t* block_tables, int32_t max_blocks, const int32_t* qo_len,
                         const int32_t* kv_len, int32_t num_reqs, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t num_blocks, double scale, double k_scale,
                         double v_scale, const uint8_t* row_select, uint16_t* out, float* lse, double* out_f64,
                         double* lse_f64, int64_t* pair_count)
{
    return attention_impl(FMT_FP8, q, k_pool, v_pool, block_tables, max_blocks, qo_len, kv_len, num_reqs,
                          num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, k_scale, v_scale,
                          row_select, out, lse, out_f64, lse_f64, pair_count);
}

/* attention over a q8_0 pool [num_blocks][Hkv][2][tile bytes]; everything else as above. */
int oracle_attention_q8(const uint16_t* q, const uint8_t* kv_pool, const int32_t* block_tables, int32_t max_blocks, const int32_t* qo_len,
                        const int32_t* kv_len, int32_t num_reqs, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size, int32_t num_blocks, double scale,
                        const uint8_t* row_select, uint16_t* out, float* lse, double* out_f64,
                        double* lse_f64, int64_t* pair_count)
{
    if (!kv_pool || head_dim <= 0 || block_size <= 0)
        return ORACLE_BAD_ARG;
    return attention_impl(FMT_Q8_0, q, kv_pool, kv_pool + oracle_q8_tile_bytes(head_dim, block_size), block_tables,
                          max_blocks, qo_len, kv_len, num_reqs,
                          num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, 1.0, 1.0, row_select,
                          out, lse, out_f64, lse_f64, pair_count);
}

/* Element-wise E4M3 encode / decode over arrays (for the format tests). */
void oracle_encode_e4m3_array(const double* x, uint8_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_double_to_e4m3(x[i]);
}

void oracle_decode_e4m3_array(const uint8_t* c, double* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = e4m3_to_double(c[i]);
}

/* Element-wise oracle_double_to_bf16 over an array (for the rounding tests). */
void oracle_round_bf16_array(const double* x, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_double_to_bf16(x[i]);
}

/* Threads the attention loop may use (OpenMP's current maximum; 1 without OpenMP), and
 * a setter for it (timing runs on one thread and on all host threads). */
#ifdef _OPENMP
#include <omp.h>
int oracle_num_threads(void) { return omp_get_max_threads(); }
void oracle_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
#else
int oracle_num_threads(void) { return 1; }
void oracle_set_num_threads(int n) { (void)n; }
#endif

/*
 * The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer: small random
 * batches (decode rows, chunk rows, shared prefixes, unused table entries of -1,
 * skipped slots) through append, attention, the q8_0 append and attention, the row
 * quantiser and the block copy.  Every call must return 0 and touch only its own
 * buffers.  Built with gcc, without OpenMP, by tests/test_host_sanitizers.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_append(uint16_t* k_pool, uint16_t* v_pool, const uint16_t* k_new, const uint16_t* v_new,
                  const int32_t* slot_mapping, int32_t n_tokens, int32_t num_kv_heads, int32_t head_dim,
                  int32_t block_size, int32_t num_blocks);
int oracle_append_q8(uint8_t* kv_pool, const uint16_t* k_new, const uint16_t* v_new, const int32_t* slot_mapping,
                     int32_t n_tokens, int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks);
int oracle_copy_blocks(uint16_t* k_pool, uint16_t* v_pool, const int32_t* src, const int32_t* dst, int32_t n,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks);
int oracle_quantize_q8_rows(const uint16_t* x, int64_t n, int32_t head_dim, int8_t* codes, uint16_t* scales);
int64_t oracle_q8_tile_bytes(int32_t head_dim, int32_t block_size);
int oracle_attention(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool, const int32_t* block_tables,
                     int32_t max_blocks, const int32_t* qo_len, const int32_t* kv_len, int32_t num_reqs,
                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t num_blocks, double scale, const uint8_t* row_select, uint16_t* out, float* lse,
                     double* out_f64, double* lse_f64, int64_t* pair_count);
int oracle_attention_q8(const uint16_t* q, const uint8_t* kv_pool, const int32_t* block_tables, int32_t max_blocks,
                        const int32_t* qo_len, const int32_t* kv_len, int32_t num_reqs, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, double scale,
                        const uint8_t* row_select, uint16_t* out, float* lse, double* out_f64, double* lse_f64,
                        int64_t* pair_count);

static uint32_t rng_state;
static uint32_t rnd(void)
{
    rng_state = rng_state * 1664525u + 1013904223u;
    return rng_state >> 8;
}
/* a bf16 bit pattern of a value in (-4, 4) */
static uint16_t rnd_bf16(void)
{
    const float x = ((float)(rnd() % 20001) - 10000.f) / 2500.f;
    uint32_t u;
    memcpy(&u, &x, 4);
    return (uint16_t)(u >> 16);
}

#define CHECK(c)                                                                  \
    do {                                                                          \
        if (!(c)) {                                                               \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);       \
            exit(1);                                                              \
        }                                                                         \
    } while (0)

static void one_batch(uint32_t seed)
{
    rng_state = seed;
    const int32_t D = 128, B = 16, Hkv = 1 + (int32_t)(rnd() % 2), Hq = 4 * Hkv;
    const int32_t R = 1 + (int32_t)(rnd() % 4);
    int32_t qo[4], kv[4], mb = 1, total_q = 0, need = 0;
    for (int32_t r = 0; r < R; ++r) {
        qo[r] = rnd() % 2 ? 1 : 1 + (int32_t)(rnd() % 40);
        kv[r] = qo[r] + (int32_t)(rnd() % 200);
        const int32_t nb = (kv[r] + B - 1) / B;
        mb = nb > mb ? nb : mb;
        need += nb;
        total_q += qo[r];
    }
    const int32_t NB = need + 2;
    const size_t pool = (size_t)NB * Hkv * B * D;
    uint16_t* kp = malloc(pool * 2);
    uint16_t* vp = malloc(pool * 2);
    for (size_t i = 0; i < pool; ++i) {
        kp[i] = rnd_bf16();
        vp[i] = rnd_bf16();
    }
    int32_t* bt = malloc(sizeof(int32_t) * (size_t)R * (mb + 1));
    int32_t next = 0;
    for (int32_t r = 0; r < R; ++r)
        for (int32_t b = 0; b < mb + 1; ++b)
            bt[r * (mb + 1) + b] = b < (kv[r] + B - 1) / B ? next++ : -1;   /* unused entries -1 */
    const size_t rowe = (size_t)total_q * Hkv * D;
    uint16_t* kn = malloc(rowe * 2);
    uint16_t* vn = malloc(rowe * 2);
    uint16_t* q = malloc((size_t)total_q * Hq * D * 2);
    for (size_t i = 0; i < rowe; ++i) {
        kn[i] = rnd_bf16();
        vn[i] = rnd_bf16();
    }
    for (size_t i = 0; i < (size_t)total_q * Hq * D; ++i)
        q[i] = rnd_bf16();
    int32_t* slots = malloc(sizeof(int32_t) * total_q);
    int32_t t = 0;
    for (int32_t r = 0; r < R; ++r)
        for (int32_t i = 0; i < qo[r]; ++i, ++t) {
            const int32_t pos = kv[r] - qo[r] + i;
            slots[t] = (rnd() % 9 == 0) ? -1 : bt[r * (mb + 1) + pos / B] * B + pos % B;   /* some skipped */
        }
    CHECK(oracle_append(kp, vp, kn, vn, slots, total_q, Hkv, D, B, NB) == 0);
    uint16_t* out = malloc((size_t)total_q * Hq * D * 2);
    float* lse = malloc(sizeof(float) * total_q * Hq);
    double* o64 = malloc(sizeof(double) * total_q * Hq * D);
    double* l64 = malloc(sizeof(double) * total_q * Hq);
    int64_t pairs = 0;
    CHECK(oracle_attention(q, kp, vp, bt, mb + 1, qo, kv, R, Hq, Hkv, D, B, NB, 1.0 / sqrt(128.0), NULL, out, lse, o64,
                           l64, &pairs) == 0);
    for (int32_t i = 0; i < total_q * Hq; ++i)
        CHECK(isfinite(lse[i]));
    /* q8_0 pool */
    const int64_t tile = oracle_q8_tile_bytes(D, B);
    uint8_t* kvq = malloc((size_t)NB * Hkv * 2 * tile);
    memset(kvq, 0, (size_t)NB * Hkv * 2 * tile);
    CHECK(oracle_append_q8(kvq, kn, vn, slots, total_q, Hkv, D, B, NB) == 0);
    CHECK(oracle_attention_q8(q, kvq, bt, mb + 1, qo, kv, R, Hq, Hkv, D, B, NB, 1.0 / sqrt(128.0), NULL, out, lse,
                              NULL, NULL, &pairs) == 0);
    int8_t* codes = malloc(rowe);
    uint16_t* scales = malloc(2 * rowe / 32);
    CHECK(oracle_quantize_q8_rows(kn, (int64_t)total_q * Hkv, D, codes, scales) == 0);
    int32_t src[2] = {0, NB - 1}, dst[2] = {NB - 2, 1};
    if (NB > 3)
        CHECK(oracle_copy_blocks(kp, vp, src, dst, 2, Hkv, D, B, NB) == 0);
    free(kp); free(vp); free(bt); free(kn); free(vn); free(q); free(slots); free(out); free(lse); free(o64); free(l64);
    free(kvq); free(codes); free(scales);
}

int main(void)
{
    for (uint32_t s = 0; s < 60; ++s)
        one_batch(77 + s);
    printf("oracle checks ok\n");
    return 0;
}

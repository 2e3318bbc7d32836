/*
 * Self-test driver of the oracle (test infrastructure): exercises every entry
 * point on small inputs so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer can check the oracle's memory accesses and
 * arithmetic.  It also checks two identities on the way: the folded attention
 * equals the plain one, and a re-append leaves the pool unchanged.  Exit
 * status 0 on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int64_t kvqo_region_bytes(int kbits, int vbits);
int kvqo_quantize_append_paged(int kbits, int vbits, int page_tokens, const uint16_t *key, const uint16_t *value,
                               int64_t key_token_stride, int64_t value_token_stride, const int64_t *slot_mapping,
                               int64_t num_tokens, int32_t num_kv_heads, uint8_t *pool, int64_t num_pages);
int kvqo_decode_attention_paged(int kbits, int vbits, int page_tokens, const uint8_t *pool, int64_t num_pages,
                                int32_t num_kv_heads, const int32_t *block_tables, int32_t max_pages_per_seq,
                                const int32_t *seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                const uint16_t *query, double scale, const uint8_t *head_mask, double *out);
int kvqo_decode_attention_mq_paged(int kbits, int vbits, int page_tokens, const uint8_t *pool, int64_t num_pages,
                                   int32_t num_kv_heads, const int32_t *block_tables, int32_t max_pages_per_seq,
                                   const int32_t *seq_lens, int32_t num_seqs, int32_t q_len, int32_t num_q_heads,
                                   const uint16_t *query, double scale, double *out);
int kvqo_decode_attention_folded_fmt(int kbits, int vbits, const uint8_t *pool, int64_t num_pages,
                                     int32_t num_kv_heads, const int32_t *block_tables,
                                     int32_t max_pages_per_seq, const int32_t *seq_lens, int32_t num_seqs,
                                     int32_t num_q_heads, const uint16_t *query, double scale, double *out);
void kvqo_attention_f16(const uint16_t *k, const uint16_t *v, int64_t n, const uint16_t *q, int32_t G,
                        double scale, double *out);
int kvqo_block_variant(const uint16_t *x, const uint8_t *present, int T, int bits, int iters,
                       uint8_t *codes_out, uint16_t *s_out, uint16_t *z_out, int *e_out, double *out);
int kvqo_quantize_append_pb(const uint16_t *key, const uint16_t *value, int64_t key_token_stride,
                            int64_t value_token_stride, const int64_t *slot_mapping, int64_t num_tokens,
                            int32_t num_kv_heads, uint8_t *pool, int64_t num_pages);
int kvqo_decode_attention_pb(const uint8_t *pool, int64_t num_pages, int32_t num_kv_heads,
                             const int32_t *block_tables, int32_t max_pages_per_seq, const int32_t *seq_lens,
                             int32_t num_seqs, int32_t num_q_heads, const uint16_t *query, double scale,
                             const uint8_t *head_mask, double *out);
uint16_t kvqo_float_to_half(float f);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static double uniform(void)
{
    state ^= state << 13; state ^= state >> 7; state ^= state << 17;
    return (double)(state >> 11) * 0x1p-53;
}
static uint16_t rand_half(double scale)
{
    double u1 = uniform() + 1e-12, u2 = uniform();
    return kvqo_float_to_half((float)(scale * sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2)));
}

static int check_format(int kbits, int vbits, int page_tokens)
{
    enum { B = 2, HKV = 2, HQ = 4, D = 128 };
    const int lens[B] = {page_tokens * 2 + 3, 5};
    const int max_pages = 3;
    const int64_t num_pages = B * max_pages;
    const int64_t page_bytes = kvqo_region_bytes(kbits, vbits) * (page_tokens / 16);
    int32_t bt[B * max_pages];
    for (int i = 0; i < B * max_pages; i++) bt[i] = (int32_t)((i * 5 + 1) % num_pages);   /* a permutation */
    uint8_t *pool = calloc((size_t)(num_pages * HKV * page_bytes), 1);
    uint8_t *copy = malloc((size_t)(num_pages * HKV * page_bytes));
    const int n_max = lens[0];
    uint16_t *k = malloc(sizeof(uint16_t) * n_max * HKV * D), *v = malloc(sizeof(uint16_t) * n_max * HKV * D);
    int64_t *slots = malloc(sizeof(int64_t) * n_max);
    if (!pool || !copy || !k || !v || !slots) return 1;
    for (int b = 0; b < B; b++) {
        for (int i = 0; i < lens[b] * HKV * D; i++) {
            k[i] = rand_half(b ? 300.0 : 1.0);
            v[i] = rand_half(b ? 1e-5 : 1.0);
        }
        for (int t = 0; t < lens[b]; t++)
            slots[t] = (int64_t)bt[b * max_pages + t / page_tokens] * page_tokens + t % page_tokens;
        if (kvqo_quantize_append_paged(kbits, vbits, page_tokens, k, v, HKV * D, HKV * D, slots, lens[b], HKV, pool,
                                       num_pages) != 0)
            return 2;
    }
    /* re-append of the last sequence leaves the pool unchanged */
    memcpy(copy, pool, (size_t)(num_pages * HKV * page_bytes));
    if (kvqo_quantize_append_paged(kbits, vbits, page_tokens, k, v, HKV * D, HKV * D, slots, lens[1], HKV, pool,
                                   num_pages) != 0 ||
        memcmp(copy, pool, (size_t)(num_pages * HKV * page_bytes)) != 0)
        return 3;
    uint16_t q[B * 3 * HQ * D];
    for (int i = 0; i < B * 3 * HQ * D; i++) q[i] = rand_half(1.0);
    double out[B * 3 * HQ * D], folded[B * HQ * D];
    const double scale = 1.0 / sqrt(128.0);
    if (kvqo_decode_attention_paged(kbits, vbits, page_tokens, pool, num_pages, HKV, bt, max_pages, lens, B, HQ, q,
                                    scale, NULL, out) != 0)
        return 4;
    if (page_tokens == 16) {
        if (kvqo_decode_attention_folded_fmt(kbits, vbits, pool, num_pages, HKV, bt, max_pages, lens, B, HQ, q, scale,
                                             folded) != 0)
            return 5;
        for (int i = 0; i < B * HQ * D; i++)
            if (!(fabs(out[i] - folded[i]) <= 1e-9)) return 6;
    }
    if (kvqo_decode_attention_mq_paged(kbits, vbits, page_tokens, pool, num_pages, HKV, bt, max_pages, lens, B, 3,
                                       HQ, q, scale, out) != 0)
        return 7;
    for (int i = 0; i < B * 3 * HQ * D; i++)
        if (!isfinite(out[i])) return 8;
    free(pool); free(copy); free(k); free(v); free(slots);
    return 0;
}

int main(void)
{
    const int fmts[5][2] = {{4, 2}, {4, 4}, {8, 2}, {8, 4}, {3, 3}};
    const int pages[4] = {16, 32, 64, 128};
    for (int f = 0; f < 5; f++)
        for (int p = 0; p < 4; p++) {
            int rc = check_format(fmts[f][0], fmts[f][1], pages[p]);
            if (rc) {
                fprintf(stderr, "selftest: k%dv%d page %d failed (%d)\n", fmts[f][0], fmts[f][1], pages[p], rc);
                return rc;
            }
        }
    /* uncompressed attention and the variance-normalisation variants */
    uint16_t kx[64 * 128], vx[64 * 128], qx[3 * 128];
    for (int i = 0; i < 64 * 128; i++) { kx[i] = rand_half(2.0); vx[i] = rand_half(1.0); }
    for (int i = 0; i < 3 * 128; i++) qx[i] = rand_half(1.0);
    double o[3 * 128], rec[16 * 128];
    uint8_t codes[16 * 128];
    kvqo_attention_f16(kx, vx, 64, qx, 3, 0.088, o);
    kvqo_attention_f16(kx, vx, 0, qx, 3, 0.088, o);
    uint16_t ss[16], zz[16];
    int ee[128];
    uint8_t pres[16];
    for (int t = 0; t < 16; t++) pres[t] = (uint8_t)(t % 5 != 3);
    for (int bits = 2; bits <= 8; bits *= 2)
        for (int it = 0; it < 3; it++) {
            if (kvqo_block_variant(kx, NULL, 16, bits, it, codes, ss, zz, ee, rec)) return 20;
            if (kvqo_block_variant(kx, pres, 11, bits, it, codes, NULL, NULL, ee, rec)) return 21;
        }
    /* page-balanced keys: 2 pages (the second partial, with a hole) of 2 KV
     * heads in a pool of 3, then a decode (30 tokens x 2 heads x 128 <= kx) */
    {
        const int64_t ntok = 30;
        int64_t slots[30];
        for (int t = 0; t < 30; t++) slots[t] = 16 * (t / 16 == 0 ? 2 : 0) + t % 16;
        slots[20] = -1;
        uint8_t *pool = calloc(3 * 2 * 1792, 1);
        if (!pool) return 22;
        if (kvqo_quantize_append_pb(kx, vx, 2 * 128, 2 * 128, slots, ntok, 2, pool, 3)) return 23;
        const int32_t bt[3] = {2, 0, 1}, lens[1] = {30};
        uint16_t q8[4 * 128];
        for (int i = 0; i < 4 * 128; i++) q8[i] = rand_half(1.0);
        double out8[4 * 128];
        if (kvqo_decode_attention_pb(pool, 3, 2, bt, 3, lens, 1, 4, q8, 0.088, NULL, out8)) return 24;
        free(pool);
    }
    printf("selftest: ok\n");
    return 0;
}

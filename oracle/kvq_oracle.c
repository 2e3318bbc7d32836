/*
 * kvq oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded CPU statement of what the K4V2 group-128
 * quantized KV cache computes.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library) shares no code, header, table or helper with this file.
 *
 * Sources (web pages; cited by tag):
 *   [KVARN-HN]  beyondheadline.xyz, "Huawei's KV-cache trick: FP16 accuracy, a
 *               four-times-larger cache and higher throughput at once" -- the
 *               lede and the section "The claim that breaks the usual
 *               trade-off" (4-bit keys, 2-bit values, Hadamard rotation,
 *               variance normalisation, asymmetric low-bit quantisation of cache
 *               blocks, preset kvarn_k4v2_g128).
 *   [KVARN-P]   dothoosh.com, "KVarN vs TurboQuant: 5x more context with higher
 *               accuracy" -- the four-stage pipeline list: (1) Hadamard
 *               rotation, (2) variance normalisation, (3) asymmetric
 *               round-to-nearest quantisation, (4) scale folding on read-back.
 *   [KV-INFRA]  encorp.ai, "KV cache compression is an infrastructure decision,
 *               not a model debate" -- section on decode being bound by HBM,
 *               not FLOPs.
 *
 * The pages give no formulas.  The readings fixed here (one 128-channel group
 * per token per KV head, unnormalised Sylvester Hadamard in natural order,
 * per-group RMS as the variance normalisation, min/max asymmetric RTN with
 * ties to even, fp16 scale/zero, 16-token pages and the byte layout) are the
 * format "kvq-k4v2-g128 v1"; each is listed with its reason in the design
 * notes of the repository.
 *
 * Precision: the encoder decides integer codes, so it runs in IEEE fp32 with
 * round-to-nearest-even, no fused multiply-add (build with -ffp-contract=off)
 * and denormals kept -- the precision the GPU encoder uses.  Attention is
 * computed in fp64 from its plain definition.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define KVQO_D 128          /* head_dim == group size                     */
#define KVQO_PAGE 16        /* tokens per page                            */
#define KVQO_REGION 1664    /* bytes per (page, kv head), 4-bit K / 2-bit V */

/* Bit widths.  The pages name the KVarN preset with 4-bit keys and 2-bit
 * values, and report presets of other widths (8-bit keys with 4-bit values,
 * 4-bit both) as nearly lossless next to fp16, and 3-bit codes as
 * noticeably worse (dzen.ru summary of the vLLM TurboQuant post, the sections
 * on accuracy and on memory).  The same KVarN pipeline is applied at those
 * widths: keys take kbits in {4, 8}, values vbits in {2, 4}, and 3 bits for
 * both (kbits = vbits = 3).  A (page, KV head) region then holds, in this
 * order:
 *   key codes    16 tokens x 16*kbits bytes   at 0
 *   value codes  16 tokens x 16*vbits bytes   at 256*kbits
 *   key (s, z)   16 tokens x 4 bytes          at 256*(kbits+vbits)
 *   value (s, mu) 16 tokens x 4 bytes         at 256*(kbits+vbits) + 64
 * i.e. 256*(kbits+vbits) + 128 bytes (1664 at 4/2, a multiple of 128). */
static int fmt_ok(int kbits, int vbits)
{
    return ((kbits == 4 || kbits == 8) && (vbits == 2 || vbits == 4)) || (kbits == 3 && vbits == 3);
}

/* Little-endian u32 at p. */
static void put_u32(uint8_t *p, uint32_t w)
{
    p[0] = (uint8_t)w; p[1] = (uint8_t)(w >> 8); p[2] = (uint8_t)(w >> 16); p[3] = (uint8_t)(w >> 24);
}

static uint32_t get_u32(const uint8_t *p)
{
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

/* 3-bit codes are stored as bit planes: bit p (0, 1, 2) of every code of a
 * set of channels in one word per plane.  Token slot i of a quad of 4 takes
 * byte K3V3_SLOT_BYTE[i] of a value plane word. */
static const int K3V3_SLOT_BYTE[4] = {0, 2, 1, 3};

int64_t kvqo_region_bytes(int kbits, int vbits)
{
    return fmt_ok(kbits, vbits) ? 256 * (kbits + vbits) + 128 : -1;
}

void kvqo_attention_f64(const double *k, const double *v, int64_t n, const uint16_t *q, int32_t G,
                        double scale, double *out);

/* Page size.  The pages promise a variable page size [KVARN-P, closing list];
 * read here as pages of page_tokens = 16 * S tokens (S = 1, 2, 4, 8), each
 * (page, KV head) holding S consecutive 16-token regions of the layout above:
 * the pool is u8 [num_pages][num_kv_heads][S][region].  Token r (0 <=
 * r < page_tokens) of a page sits in region r / 16, slot r % 16. */
static int page_ok(int page_tokens)
{
    return page_tokens == 16 || page_tokens == 32 || page_tokens == 64 || page_tokens == 128;
}

/* The 16-token region holding token r of page `page`, KV head h. */
static const uint8_t *token_region(const uint8_t *pool, int64_t page, int h, int num_kv_heads, int r,
                                   int page_tokens, int64_t region_bytes)
{
    const int subs = page_tokens / KVQO_PAGE;
    return pool + ((page * num_kv_heads + h) * subs + r / KVQO_PAGE) * region_bytes;
}

/* ------------------------------------------------------------------------ */
/* IEEE binary16 <-> binary32/64, written from the format definition.        */
/* ------------------------------------------------------------------------ */

/* binary16 bits -> exact real value (every binary16 is exact in double). */
double kvqo_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* zero / subnormal */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);     /* (1 + m/1024) 2^(e-15) */
    return sign ? -v : v;
}

static float kvqo_half_to_float(uint16_t h) { return (float)kvqo_half_to_double(h); }

/* Nearest binary16 to a binary32 value, ties to even.  |f| is scaled by the
 * binary16 unit in the last place of its binade (a power of two, so exact in
 * double) and rounded to an integer with the default rounding mode
 * (nearest-even).  A carry out of the significand lands in the exponent field
 * by itself, and a result beyond the largest finite value becomes infinity. */
uint16_t kvqo_float_to_half(float f)
{
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    double a = fabs((double)f);
    if (isnan(f)) return (uint16_t)(sign | 0x7e00);
    if (isinf(f)) return (uint16_t)(sign | 0x7c00);
    if (a < 0x1p-14) {                             /* subnormal binade */
        double n = nearbyint(a * 0x1p24);          /* units of 2^-24 */
        return (uint16_t)(sign | (uint16_t)n);     /* n == 1024 is the min normal */
    }
    int ex;
    frexp(a, &ex);                                 /* a = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1;                                /* a in [2^e, 2^(e+1)) */
    double n = nearbyint(ldexp(a, 10 - e));        /* in [1024, 2048] */
    long bits = ((long)(e + 15) << 10) + ((long)n - 1024);
    if (bits >= 0x7c00) return (uint16_t)(sign | 0x7c00);
    return (uint16_t)(sign | (uint16_t)bits);
}

/* ------------------------------------------------------------------------ */
/* Hadamard matrix of order 128 (Sylvester construction, natural order).     */
/* ------------------------------------------------------------------------ */

/* Entry (i, j) of the unnormalised Sylvester Hadamard matrix: (-1)^popcount(i&j). */
int kvqo_hadamard_entry(int i, int j)
{
    return (__builtin_popcount((unsigned)(i & j)) & 1) ? -1 : 1;
}

/* Fast Walsh-Hadamard transform in fp32, in place, no scaling.  Butterfly
 * stages h = 1, 2, 4, ..., 64; each butterfly replaces (a, b) = (y[i], y[i+h])
 * with (a + b, a - b).  This stage order is part of the format: it fixes the
 * fp32 rounding of the rotated values that the codes are taken from. */
void kvqo_fwht_f32(float *y)
{
    for (int h = 1; h < KVQO_D; h <<= 1)
        for (int i = 0; i < KVQO_D; i++)
            if ((i & h) == 0) {
                float a = y[i], b = y[i + h];
                y[i] = a + b;
                y[i + h] = a - b;
            }
}

/* y = H x in fp64 as a dense matrix-vector product (used where rounding order
 * does not matter: un-rotating the cache for attention). */
void kvqo_hadamard_matvec_f64(const double *x, double *y)
{
    for (int i = 0; i < KVQO_D; i++) {
        double acc = 0.0;
        for (int j = 0; j < KVQO_D; j++)
            acc += kvqo_hadamard_entry(i, j) * x[j];
        y[i] = acc;
    }
}

/* ------------------------------------------------------------------------ */
/* Encoder: one group = the 128 channels of one token of one KV head.        */
/* ------------------------------------------------------------------------ */

/*
 * Quantise one group of 128 fp16 values to `bits`-bit codes (4 for keys, 2
 * for values) with an fp16 scale s and an fp16 offset, following the pipeline
 * order of [KVARN-P] (stages 1-3) and [KVARN-HN]:
 *
 *   1. Hadamard rotation [KVARN-P stage 1]: y = H x by the fp32 FWHT above.
 *   2. Variance normalisation [KVARN-P stage 2, KVARN-HN]: read here as the
 *      group's RMS.  p_i = y_i^2, summed by the fixed pairwise tree
 *      (h = 64, 32, ..., 1: p[i] += p[i+h] for i < h); sigma =
 *      sqrt(ss / 128); r = 1 / sigma; yh_i = y_i * r.  An all-zero group
 *      encodes as codes 0, s = 0, z = 0.
 *   3. Asymmetric round-to-nearest [KVARN-P stage 3]: m = min yh, M = max yh,
 *      L = 2^bits - 1.  If M == m every code is 0 and the step is 0.
 *      Otherwise delta = (M - m) / L, inv = L / (M - m) and
 *      c_i = min(L, rint((yh_i - m) * inv)), ties to even.
 *   4. The normalisation is folded back into the stored metadata, s =
 *      fp16(delta * sigma), and one offset:
 *        keys   (offset_mode 0): the zero z = fp16(m * sigma); the rotated
 *               value is s * c + z;
 *        values (offset_mode 1): the group mean mu = fp16(sigma * (m + delta
 *               * C / 128)), C = sum of the 128 codes (the fp32 product delta*C
 *               is scaled by the exact 2^-7, then m is added); the rotated
 *               value is s * c + (mu - s * C / 128).
 *      mu is the dequantised group's mean in the rotated domain, which is
 *      the dequantised original channel 0 (H 1 = 128 e_0); storing it
 *      instead of z keeps channel 0 free of the cancellation between s*C and
 *      128*z.  A zero offset is stored as +0.
 */
void kvqo_quantize_group_mode(const uint16_t *x, int bits, int offset_mode, uint8_t *codes,
                              uint16_t *s_out, uint16_t *z_out)
{
    float y[KVQO_D], p[KVQO_D];
    for (int i = 0; i < KVQO_D; i++)
        y[i] = kvqo_half_to_float(x[i]);

    /* 1. Hadamard rotation */
    kvqo_fwht_f32(y);

    /* 2. variance normalisation */
    for (int i = 0; i < KVQO_D; i++)
        p[i] = y[i] * y[i];
    for (int h = KVQO_D / 2; h >= 1; h >>= 1)
        for (int i = 0; i < h; i++)
            p[i] = p[i] + p[i + h];
    float ss = p[0];
    if (ss == 0.0f) {
        memset(codes, 0, KVQO_D);
        *s_out = 0;
        *z_out = 0;
        return;
    }
    float sigma = sqrtf(ss * 0x1p-7f);
    float r = 1.0f / sigma;
    float yh[KVQO_D];
    for (int i = 0; i < KVQO_D; i++)
        yh[i] = y[i] * r;

    /* 3. asymmetric round-to-nearest */
    float m = yh[0], M = yh[0];
    for (int i = 1; i < KVQO_D; i++) {
        if (yh[i] < m) m = yh[i];
        if (yh[i] > M) M = yh[i];
    }
    const int L = (1 << bits) - 1;
    float delta;
    if (M == m) {
        delta = 0.0f;
        memset(codes, 0, KVQO_D);
    } else {
        delta = (M - m) / (float)L;
        float inv = (float)L / (M - m);
        for (int i = 0; i < KVQO_D; i++) {
            float c = rintf((yh[i] - m) * inv);
            codes[i] = (uint8_t)(c > (float)L ? L : (int)c);
        }
    }

    /* 4. metadata */
    *s_out = kvqo_float_to_half(delta * sigma);
    uint16_t z;
    if (offset_mode == 0) {
        z = kvqo_float_to_half(m * sigma);
    } else {
        int csum = 0;
        for (int i = 0; i < KVQO_D; i++) csum += codes[i];
        float t = delta * (float)csum;
        t = t * 0x1p-7f;
        t = m + t;
        z = kvqo_float_to_half(t * sigma);
    }
    *z_out = (z == 0x8000) ? 0 : z;
}

/* ------------------------------------------------------------------------ */
/* Byte layout of one (page, KV head) region.                                */
/* ------------------------------------------------------------------------ */

/* Write token slot `off` (0..15) of a region: 128 key codes (0..2^kbits-1),
 * 128 value codes (0..2^vbits-1) and the two (s, offset) pairs.
 *   key codes:   the token's row of 16*kbits bytes at 16*kbits*off holds the
 *                code of channel c at bits kbits*c .. kbits*c+kbits-1 of the
 *                row, least significant bit first (4 bits: byte b = code[2b]
 *                | code[2b+1] << 4; 8 bits: byte c = code[c]).
 *     3 bits (bit planes): for G = 0..3 and p = 0..2 the little-endian u32
 *                at 12G + 4p of the 48-byte row holds, at bit x, bit p of
 *                the code of channel 32G + x.
 *   value codes, for quad g = off/4, slot i = off%4 and channel c = 16j + m:
 *     2 bits: the 16-bit little-endian word at vbase + 128g + 8m + 2i holds
 *             the code of channel 16j + m in bits 2j..2j+1 (j = 0..7);
 *     4 bits: with j = 4h + k (h = 0, 1; k = 0..3), the 16-bit word at
 *             vbase + 256g + 16m + 8(i/2) + 4h + 2(i%2) holds the code of
 *             channel 16j + m in bits 4k..4k+3;
 *     3 bits (bit planes): byte K3V3_SLOT_BYTE[i] of the little-endian u32 at
 *             vbase + 12(16g + m) + 4p holds, at bit j, bit p of the code of
 *             channel 16j + m.
 *   metadata:    fp16 s then fp16 offset, little-endian, 4 bytes per token at
 *                kmeta + 4*off (keys) and kmeta + 64 + 4*off (values).
 * (vbase = 256*kbits, kmeta = 256*(kbits+vbits).) */
void kvqo_store_token_fmt(int kbits, int vbits, uint8_t *region, int off,
                          const uint8_t *kc, uint16_t ks, uint16_t kz,
                          const uint8_t *vc, uint16_t vs, uint16_t vz)
{
    const int vbase = 256 * kbits, kmeta = 256 * (kbits + vbits);
    const unsigned kmask = (1u << kbits) - 1, vmask = (1u << vbits) - 1;

    uint8_t *kb = region + 16 * kbits * off;
    memset(kb, 0, (size_t)(16 * kbits));
    if (kbits == 3) {
        for (int G = 0; G < 4; G++)
            for (int p = 0; p < 3; p++) {
                uint32_t w = 0;
                for (int x = 0; x < 32; x++)
                    w |= (uint32_t)((kc[32 * G + x] >> p) & 1u) << x;
                put_u32(kb + 12 * G + 4 * p, w);
            }
    } else {
        for (int c = 0; c < KVQO_D; c++) {
            int bit = kbits * c;
            kb[bit / 8] |= (uint8_t)((kc[c] & kmask) << (bit % 8));
        }
    }

    int g = off / 4, i = off % 4;
    if (vbits == 3) {
        for (int m = 0; m < 16; m++)
            for (int p = 0; p < 3; p++) {
                unsigned b = 0;
                for (int j = 0; j < 8; j++)
                    b |= ((vc[16 * j + m] >> p) & 1u) << j;
                region[vbase + 12 * (16 * g + m) + 4 * p + K3V3_SLOT_BYTE[i]] = (uint8_t)b;
            }
    } else if (vbits == 2) {
        for (int m = 0; m < 16; m++) {
            unsigned w = 0;
            for (int j = 0; j < 8; j++)
                w |= (unsigned)(vc[16 * j + m] & vmask) << (2 * j);
            uint8_t *vb = region + vbase + 128 * g + 8 * m + 2 * i;
            vb[0] = (uint8_t)(w & 0xff);
            vb[1] = (uint8_t)(w >> 8);
        }
    } else {
        for (int m = 0; m < 16; m++)
            for (int h = 0; h < 2; h++) {
                unsigned w = 0;
                for (int k = 0; k < 4; k++)
                    w |= (unsigned)(vc[16 * (4 * h + k) + m] & vmask) << (4 * k);
                uint8_t *vb = region + vbase + 256 * g + 16 * m + 8 * (i / 2) + 4 * h + 2 * (i % 2);
                vb[0] = (uint8_t)(w & 0xff);
                vb[1] = (uint8_t)(w >> 8);
            }
    }

    uint8_t *km = region + kmeta + 4 * off;
    km[0] = (uint8_t)(ks & 0xff); km[1] = (uint8_t)(ks >> 8);
    km[2] = (uint8_t)(kz & 0xff); km[3] = (uint8_t)(kz >> 8);
    uint8_t *vm = region + kmeta + 64 + 4 * off;
    vm[0] = (uint8_t)(vs & 0xff); vm[1] = (uint8_t)(vs >> 8);
    vm[2] = (uint8_t)(vz & 0xff); vm[3] = (uint8_t)(vz >> 8);
}

/* Inverse of kvqo_store_token_fmt. */
void kvqo_load_token_fmt(int kbits, int vbits, const uint8_t *region, int off,
                         uint8_t *kc, uint16_t *ks, uint16_t *kz,
                         uint8_t *vc, uint16_t *vs, uint16_t *vz)
{
    const int vbase = 256 * kbits, kmeta = 256 * (kbits + vbits);
    const unsigned kmask = (1u << kbits) - 1, vmask = (1u << vbits) - 1;

    const uint8_t *kb = region + 16 * kbits * off;
    if (kbits == 3) {
        for (int G = 0; G < 4; G++)
            for (int x = 0; x < 32; x++) {
                unsigned c = 0;
                for (int p = 0; p < 3; p++)
                    c |= ((get_u32(kb + 12 * G + 4 * p) >> x) & 1u) << p;
                kc[32 * G + x] = (uint8_t)c;
            }
    } else {
        for (int c = 0; c < KVQO_D; c++) {
            int bit = kbits * c;
            kc[c] = (uint8_t)((kb[bit / 8] >> (bit % 8)) & kmask);
        }
    }
    int g = off / 4, i = off % 4;
    if (vbits == 3) {
        for (int m = 0; m < 16; m++)
            for (int j = 0; j < 8; j++) {
                unsigned c = 0;
                for (int p = 0; p < 3; p++)
                    c |= ((region[vbase + 12 * (16 * g + m) + 4 * p + K3V3_SLOT_BYTE[i]] >> j) & 1u) << p;
                vc[16 * j + m] = (uint8_t)c;
            }
    } else if (vbits == 2) {
        for (int m = 0; m < 16; m++) {
            const uint8_t *vb = region + vbase + 128 * g + 8 * m + 2 * i;
            unsigned w = (unsigned)vb[0] | ((unsigned)vb[1] << 8);
            for (int j = 0; j < 8; j++)
                vc[16 * j + m] = (uint8_t)((w >> (2 * j)) & vmask);
        }
    } else {
        for (int m = 0; m < 16; m++)
            for (int h = 0; h < 2; h++) {
                const uint8_t *vb = region + vbase + 256 * g + 16 * m + 8 * (i / 2) + 4 * h + 2 * (i % 2);
                unsigned w = (unsigned)vb[0] | ((unsigned)vb[1] << 8);
                for (int k = 0; k < 4; k++)
                    vc[16 * (4 * h + k) + m] = (uint8_t)((w >> (4 * k)) & vmask);
            }
    }
    const uint8_t *km = region + kmeta + 4 * off;
    *ks = (uint16_t)(km[0] | (km[1] << 8));
    *kz = (uint16_t)(km[2] | (km[3] << 8));
    const uint8_t *vm = region + kmeta + 64 + 4 * off;
    *vs = (uint16_t)(vm[0] | (vm[1] << 8));
    *vz = (uint16_t)(vm[2] | (vm[3] << 8));
}

/* The 4-bit key / 2-bit value layout (KVarN's preset). */

/* ------------------------------------------------------------------------ */
/* Quantise-on-write of cache blocks [KVARN-HN].                             */
/* ------------------------------------------------------------------------ */

/*
 * key/value: fp16 [num_tokens][num_kv_heads][128] with the given token
 * strides (in elements; the head stride is 128).  slot_mapping[t] = page*16 +
 * offset, or < 0 to skip the token.  pool: u8 [num_pages][num_kv_heads][1664].
 * Returns 0, or -1 on a slot outside the pool (nothing is written for it).
 */
int kvqo_quantize_append_paged(int kbits, int vbits, int page_tokens, const uint16_t *key, const uint16_t *value,
                               int64_t key_token_stride, int64_t value_token_stride,
                               const int64_t *slot_mapping, int64_t num_tokens,
                               int32_t num_kv_heads, uint8_t *pool, int64_t num_pages)
{
    if (!fmt_ok(kbits, vbits) || !page_ok(page_tokens)) return -1;
    const int64_t region_bytes = kvqo_region_bytes(kbits, vbits);
    int rc = 0;
    uint8_t kc[KVQO_D], vc[KVQO_D];
    for (int64_t t = 0; t < num_tokens; t++) {
        int64_t slot = slot_mapping[t];
        if (slot < 0) continue;
        int64_t page = slot / page_tokens;
        int r = (int)(slot % page_tokens);
        if (page >= num_pages) { rc = -1; continue; }
        for (int h = 0; h < num_kv_heads; h++) {
            uint16_t ks, kz, vs, vz;
            kvqo_quantize_group_mode(key + t * key_token_stride + (int64_t)h * KVQO_D, kbits, 0, kc, &ks, &kz);
            kvqo_quantize_group_mode(value + t * value_token_stride + (int64_t)h * KVQO_D, vbits, 1, vc, &vs, &vz);
            uint8_t *region = (uint8_t *)token_region(pool, page, h, num_kv_heads, r, page_tokens, region_bytes);
            kvqo_store_token_fmt(kbits, vbits, region, r % KVQO_PAGE, kc, ks, kz, vc, vs, vz);
        }
    }
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Decode attention over the quantised paged cache.                          */
/* ------------------------------------------------------------------------ */

/* Zero-point of a group in the rotated domain: z itself for keys; for values
 * z = mu - s * C / 128 (exact in double: C <= 128 * 15). */
static double group_zero(const uint8_t *codes, uint16_t s16, uint16_t off16, int is_value)
{
    double off = kvqo_half_to_double(off16);
    if (!is_value) return off;
    int csum = 0;
    for (int i = 0; i < KVQO_D; i++) csum += codes[i];
    return off - kvqo_half_to_double(s16) * csum / 128.0;
}

/* Dequantise one cached token back to the original (un-rotated) domain:
 * rotated value yt_i = s*c_i + z; original value = H yt / 128 (H H = 128 I). */
static void dequant_unrotate(const uint8_t *codes, uint16_t s16, uint16_t z16, int is_value, double *out)
{
    double yt[KVQO_D];
    double s = kvqo_half_to_double(s16), z = group_zero(codes, s16, z16, is_value);
    for (int i = 0; i < KVQO_D; i++)
        yt[i] = s * codes[i] + z;
    kvqo_hadamard_matvec_f64(yt, out);
    for (int i = 0; i < KVQO_D; i++)
        out[i] /= 128.0;
}

/* Dequantised, un-rotated key and value of one slot (kbits, vbits layout). */
void kvqo_dequant_slot_fmt(int kbits, int vbits, const uint8_t *region, int off, double *k_out, double *v_out)
{
    uint8_t kc[KVQO_D], vc[KVQO_D];
    uint16_t ks, kz, vs, vz;
    kvqo_load_token_fmt(kbits, vbits, region, off, kc, &ks, &kz, vc, &vs, &vz);
    dequant_unrotate(kc, ks, kz, 0, k_out);
    dequant_unrotate(vc, vs, vz, 1, v_out);
}

/* Rotated-domain dequantised values of one slot (s*c + z per channel). */
void kvqo_dequant_slot_rotated_fmt(int kbits, int vbits, const uint8_t *region, int off, double *k_out,
                                   double *v_out)
{
    uint8_t kc[KVQO_D], vc[KVQO_D];
    uint16_t ks, kz, vs, vz;
    kvqo_load_token_fmt(kbits, vbits, region, off, kc, &ks, &kz, vc, &vs, &vz);
    double kzero = group_zero(kc, ks, kz, 0), vzero = group_zero(vc, vs, vz, 1);
    for (int i = 0; i < KVQO_D; i++) {
        k_out[i] = kvqo_half_to_double(ks) * kc[i] + kzero;
        v_out[i] = kvqo_half_to_double(vs) * vc[i] + vzero;
    }
}

/*
 * Plain definition of one decode step.  For sequence b, query head hq and its
 * KV head kvh = hq / (num_q_heads / num_kv_heads), with n = seq_lens[b]
 * cached tokens (token t lives in page block_tables[b][t / 16], slot t % 16):
 *     k_t, v_t = dequantised, un-rotated key and value of token t
 *     l_t      = scale * (q . k_t)
 *     out      = sum_t softmax(l)_t v_t
 * in fp64.  query: fp16 [num_seqs][num_q_heads][128].  out: fp64, same shape.
 * head_mask (optional, [num_seqs][num_q_heads]): only heads with a non-zero
 * entry are computed; the rest of `out` is left untouched.
 * Returns 0, or -1 on an invalid shape or page id.
 */
int kvqo_decode_attention_paged(int kbits, int vbits, int page_tokens, const uint8_t *pool, int64_t num_pages,
                                int32_t num_kv_heads, const int32_t *block_tables, int32_t max_pages_per_seq,
                                const int32_t *seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                const uint16_t *query, double scale,
                                const uint8_t *head_mask, double *out)
{
    if (!fmt_ok(kbits, vbits) || !page_ok(page_tokens)) return -1;
    const int64_t region_bytes = kvqo_region_bytes(kbits, vbits);
    if (num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return -1;
    const int G = num_q_heads / num_kv_heads;
    for (int b = 0; b < num_seqs; b++) {
        const int64_t n = seq_lens[b];
        if (n < 0 || n > (int64_t)max_pages_per_seq * page_tokens) return -1;
        for (int kvh = 0; kvh < num_kv_heads; kvh++) {
            int any = 0;
            for (int g = 0; g < G; g++)
                if (!head_mask || head_mask[b * num_q_heads + kvh * G + g]) any = 1;
            if (!any || n == 0) continue;
            double *K = malloc(sizeof(double) * KVQO_D * n);
            double *V = malloc(sizeof(double) * KVQO_D * n);
            double *lg = malloc(sizeof(double) * n);
            if (!K || !V || !lg) { free(K); free(V); free(lg); return -1; }
            for (int64_t t = 0; t < n; t++) {
                int32_t page = block_tables[(int64_t)b * max_pages_per_seq + t / page_tokens];
                if (page < 0 || page >= num_pages) { free(K); free(V); free(lg); return -1; }
                const int r = (int)(t % page_tokens);
                const uint8_t *region = token_region(pool, page, kvh, num_kv_heads, r, page_tokens, region_bytes);
                kvqo_dequant_slot_fmt(kbits, vbits, region, r % KVQO_PAGE, K + t * KVQO_D, V + t * KVQO_D);
            }
            for (int g = 0; g < G; g++) {
                int hq = kvh * G + g;
                if (head_mask && !head_mask[b * num_q_heads + hq]) continue;
                const uint16_t *q16 = query + ((int64_t)b * num_q_heads + hq) * KVQO_D;
                double q[KVQO_D];
                for (int i = 0; i < KVQO_D; i++) q[i] = kvqo_half_to_double(q16[i]);
                double mx = -INFINITY;
                for (int64_t t = 0; t < n; t++) {
                    double d = 0.0;
                    for (int i = 0; i < KVQO_D; i++) d += q[i] * K[t * KVQO_D + i];
                    lg[t] = scale * d;
                    if (lg[t] > mx) mx = lg[t];
                }
                double den = 0.0, o[KVQO_D] = {0};
                for (int64_t t = 0; t < n; t++) {
                    double e = exp(lg[t] - mx);
                    den += e;
                    for (int i = 0; i < KVQO_D; i++) o[i] += e * V[t * KVQO_D + i];
                }
                double *dst = out + ((int64_t)b * num_q_heads + hq) * KVQO_D;
                for (int i = 0; i < KVQO_D; i++) dst[i] = o[i] / den;
            }
            free(K); free(V); free(lg);
        }
    }
    return 0;
}

/*
 * Several query rows per sequence (the tokens of a speculative-decoding draft
 * or a prefill chunk): q_len rows, the last q_len tokens of the sequence, all
 * already in the cache.  Row m of sequence b sits at position n - q_len + m
 * (n = seq_lens[b]) and attends causally, to tokens 0 .. n - q_len + m:
 *     out[b][m][hq] = sum_{t <= n - q_len + m} softmax(scale * q.k_t) v_t
 * with k_t, v_t as in kvqo_decode_attention_fmt, in fp64.  query, out:
 * [num_seqs][q_len][num_q_heads][128] (fp16 in, fp64 out).  A row that sees
 * no token (n - q_len + m < 0) is zero.  Returns 0, or -1 on an invalid shape
 * or page id.
 */
int kvqo_decode_attention_mq_paged(int kbits, int vbits, int page_tokens, const uint8_t *pool, int64_t num_pages,
                                   int32_t num_kv_heads, const int32_t *block_tables, int32_t max_pages_per_seq,
                                   const int32_t *seq_lens, int32_t num_seqs, int32_t q_len, int32_t num_q_heads,
                                   const uint16_t *query, double scale, double *out)
{
    if (!fmt_ok(kbits, vbits) || !page_ok(page_tokens) || q_len <= 0) return -1;
    const int64_t region_bytes = kvqo_region_bytes(kbits, vbits);
    if (num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return -1;
    const int G = num_q_heads / num_kv_heads;
    for (int b = 0; b < num_seqs; b++) {
        const int64_t n = seq_lens[b];
        if (n < 0 || n > (int64_t)max_pages_per_seq * page_tokens) return -1;
        for (int kvh = 0; kvh < num_kv_heads; kvh++) {
            double *K = malloc(sizeof(double) * KVQO_D * (n > 0 ? n : 1));
            double *V = malloc(sizeof(double) * KVQO_D * (n > 0 ? n : 1));
            if (!K || !V) { free(K); free(V); return -1; }
            for (int64_t t = 0; t < n; t++) {
                int32_t page = block_tables[(int64_t)b * max_pages_per_seq + t / page_tokens];
                if (page < 0 || page >= num_pages) { free(K); free(V); return -1; }
                const int r = (int)(t % page_tokens);
                const uint8_t *region = token_region(pool, page, kvh, num_kv_heads, r, page_tokens, region_bytes);
                kvqo_dequant_slot_fmt(kbits, vbits, region, r % KVQO_PAGE, K + t * KVQO_D, V + t * KVQO_D);
            }
            for (int m = 0; m < q_len; m++) {
                const int64_t visible = n - q_len + m + 1;        /* tokens 0 .. n - q_len + m */
                for (int g = 0; g < G; g++) {
                    const int hq = kvh * G + g;
                    const int64_t row = ((int64_t)b * q_len + m) * num_q_heads + hq;
                    kvqo_attention_f64(K, V, visible > 0 ? visible : 0, query + row * KVQO_D, 1, scale,
                                       out + row * KVQO_D);
                }
            }
            free(K); free(V);
        }
    }
    return 0;
}

/*
 * The same step reached by scale folding on read-back [KVARN-P stage 4], in
 * fp64: never materialise k_t or v_t.  With q' = H q (H symmetric):
 *     q . k_t   = (q' . (s c_t + z 1)) / 128 = (s (q' . c_t) + z sum(q')) / 128
 *     sum_t p_t v_t = H (acc + zv 1) / 128,  acc = sum_t p_t s_t c_t,
 *                                          zv = sum_t p_t z_t,
 *     and H 1 = 128 e_0, so the value zero-points reach output channel 0
 *     only; there (H acc)_0 + 128 zv = 128 sum_t p_t mu_t, the stored means.
 * Exists to pin this algebra against the plain definition above.
 */
int kvqo_decode_attention_folded_fmt(int kbits, int vbits, const uint8_t *pool, int64_t num_pages,
                                     int32_t num_kv_heads, const int32_t *block_tables,
                                     int32_t max_pages_per_seq, const int32_t *seq_lens, int32_t num_seqs,
                                     int32_t num_q_heads, const uint16_t *query, double scale, double *out)
{
    if (!fmt_ok(kbits, vbits)) return -1;
    const int64_t region_bytes = kvqo_region_bytes(kbits, vbits);
    if (num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return -1;
    const int G = num_q_heads / num_kv_heads;
    uint8_t kc[KVQO_D], vc[KVQO_D];
    for (int b = 0; b < num_seqs; b++) {
        const int64_t n = seq_lens[b];
        if (n <= 0 || n > (int64_t)max_pages_per_seq * KVQO_PAGE) return -1;
        double *lg = malloc(sizeof(double) * n);
        if (!lg) return -1;
        for (int hq = 0; hq < num_q_heads; hq++) {
            int kvh = hq / G;
            const uint16_t *q16 = query + ((int64_t)b * num_q_heads + hq) * KVQO_D;
            double q[KVQO_D], qr[KVQO_D], qsum = 0.0;
            for (int i = 0; i < KVQO_D; i++) q[i] = kvqo_half_to_double(q16[i]);
            kvqo_hadamard_matvec_f64(q, qr);
            for (int i = 0; i < KVQO_D; i++) qsum += qr[i];
            double mx = -INFINITY;
            for (int64_t t = 0; t < n; t++) {
                int32_t page = block_tables[(int64_t)b * max_pages_per_seq + t / KVQO_PAGE];
                if (page < 0 || page >= num_pages) { free(lg); return -1; }
                const uint8_t *region = pool + ((int64_t)page * num_kv_heads + kvh) * region_bytes;
                uint16_t ks, kz, vs, vz;
                kvqo_load_token_fmt(kbits, vbits, region, (int)(t % KVQO_PAGE), kc, &ks, &kz, vc, &vs, &vz);
                double dot = 0.0;
                for (int i = 0; i < KVQO_D; i++) dot += qr[i] * kc[i];
                lg[t] = scale * (kvqo_half_to_double(ks) * dot + kvqo_half_to_double(kz) * qsum) / 128.0;
                if (lg[t] > mx) mx = lg[t];
            }
            double l = 0.0, zacc = 0.0, acc[KVQO_D] = {0};
            for (int64_t t = 0; t < n; t++) {
                int32_t page = block_tables[(int64_t)b * max_pages_per_seq + t / KVQO_PAGE];
                const uint8_t *region = pool + ((int64_t)page * num_kv_heads + kvh) * region_bytes;
                uint16_t ks, kz, vs, vz;
                kvqo_load_token_fmt(kbits, vbits, region, (int)(t % KVQO_PAGE), kc, &ks, &kz, vc, &vs, &vz);
                double p = exp(lg[t] - mx);
                double sv = kvqo_half_to_double(vs);
                l += p;
                zacc += p * kvqo_half_to_double(vz);      /* value mean mu */
                for (int i = 0; i < KVQO_D; i++) acc[i] += p * sv * vc[i];
            }
            double o[KVQO_D];
            kvqo_hadamard_matvec_f64(acc, o);
            double *dst = out + ((int64_t)b * num_q_heads + hq) * KVQO_D;
            for (int i = 0; i < KVQO_D; i++) dst[i] = o[i] / (128.0 * l);
            /* channel 0: (H acc)_0 + 128 sum p z = sum p (s C + 128 (mu - s C/128)) */
            dst[0] = zacc / l;
        }
        free(lg);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Uncompressed reference: attention over fp16 keys and values.              */
/* ------------------------------------------------------------------------ */

/* Plain decode attention of G query heads over n tokens of one KV head, in
 * fp64: out[g] = sum_t softmax_t(scale * q_g . k_t) v_t.  k, v: [n][128]
 * (fp64); q: fp16 [G][128]; out: [G][128].  n == 0 gives zero rows. */
void kvqo_attention_f64(const double *k, const double *v, int64_t n, const uint16_t *q, int32_t G,
                        double scale, double *out)
{
    double *lg = n > 0 ? malloc(sizeof(double) * n) : NULL;
    for (int g = 0; g < G; g++) {
        double *dst = out + (int64_t)g * KVQO_D;
        for (int i = 0; i < KVQO_D; i++) dst[i] = 0.0;
        if (n <= 0 || !lg) continue;
        double qd[KVQO_D];
        for (int i = 0; i < KVQO_D; i++) qd[i] = kvqo_half_to_double(q[(int64_t)g * KVQO_D + i]);
        double mx = -INFINITY;
        for (int64_t t = 0; t < n; t++) {
            double d = 0.0;
            for (int i = 0; i < KVQO_D; i++) d += qd[i] * k[t * KVQO_D + i];
            lg[t] = scale * d;
            if (lg[t] > mx) mx = lg[t];
        }
        double den = 0.0;
        for (int64_t t = 0; t < n; t++) {
            double e = exp(lg[t] - mx);
            den += e;
            for (int i = 0; i < KVQO_D; i++) dst[i] += e * v[t * KVQO_D + i];
        }
        for (int i = 0; i < KVQO_D; i++) dst[i] /= den;
    }
    free(lg);
}

/* The same over fp16 tokens: the uncompressed cache the K4V2 format is
 * measured against [KVARN-HN: fp16 as the accuracy and capacity reference].
 * k, v: fp16 [n][128]. */
void kvqo_attention_f16(const uint16_t *k, const uint16_t *v, int64_t n, const uint16_t *q,
                        int32_t G, double scale, double *out)
{
    double *kd = n > 0 ? malloc(sizeof(double) * KVQO_D * n) : NULL;
    double *vd = n > 0 ? malloc(sizeof(double) * KVQO_D * n) : NULL;
    if (n > 0 && (!kd || !vd)) {
        free(kd); free(vd);
        for (int64_t i = 0; i < (int64_t)G * KVQO_D; i++) out[i] = NAN;
        return;
    }
    for (int64_t i = 0; i < n * KVQO_D; i++) {
        kd[i] = kvqo_half_to_double(k[i]);
        vd[i] = kvqo_half_to_double(v[i]);
    }
    kvqo_attention_f64(kd, vd, n, q, G, scale, out);
    free(kd);
    free(vd);
}

/* ------------------------------------------------------------------------ */
/* Page-balanced keys: an active variance normalisation.                     */
/* ------------------------------------------------------------------------ */

/*
 * The pages name variance normalisation as stage 2 of the pipeline [KVARN-P
 * stage 2; KVARN-HN] without a formula.  The Persian page's wording reads as
 * an iterative ("repeated") normalisation of the variance, and its closing
 * paragraph credits the method with removing fluctuations in logarithmic
 * space.  The per-group reading of the v1 format (divide each group by its
 * RMS) is inert in exact arithmetic, since min/max RTN is scale-equivariant.
 * This reading acts on a block -- one page of one KV head, up to 16 tokens --
 * and does change the codes:
 *
 *   Y_t = FWHT(x_t) for the present rows (fp32, the encoder's rotation);
 *   absent rows are zero.  Row exponents f_t = 0.  For pass p = 1 .. iters:
 *     column pass: ss_j = sum over the 16 row slots of (Y_tj 2^-f_t)^2 in
 *       fp32, summed by the fixed tree h = 8, 4, 2, 1 (a[t] += a[t + h] for
 *       t < h); e_j = floor(F_j / 2), where ss_j = m 2^F_j with m in [0.5, 1)
 *       -- the nearest integer to log2 of the column's root mean square up
 *       to a constant, halves rounded up; a zero column has no exponent;
 *     row pass (between column passes only): ss_t = sum_j (Y_tj 2^-e_j)^2
 *       by the encoder's tree (h = 64 .. 1), f_t = floor(F_t / 2) likewise
 *       (0 for a zero row).
 *   (Sinkhorn-style balancing of the block's second moments, with every
 *   scale kept as a power of two: the log-space reading.)  The final column
 *   exponents come from the last column pass's sums ss_j = m_j 2^F_j, in
 *   integers: over the n non-zero columns, with S = sum of their F_j and
 *   d_j = n F_j - S (n times the column's offset from the mean, in
 *   half-octaves of its RMS),
 *     e_j = 0                         if |d_j| < 2n  (within an octave),
 *     e_j = floor((d_j + n) / (2n))   otherwise      (nearest octave),
 *   clamped to [-6, 6]; a zero column takes -6.  A block whose columns the
 *   rotation has already evened out thus keeps every e_j = 0 and is encoded
 *   as the per-token encoder would; a column an octave or more louder than
 *   the typical one is shrunk by 2^-e_j before RTN (and restored on read),
 *   a quieter one amplified, so the rows' ranges stop being set by a few
 *   columns.
 *   Each present row of Yhat_tj = Y_tj 2^-e_j -- exact in fp32, since the
 *   scales are powers of two -- goes through the encoder's own steps 2-4
 *   (RMS, min/max, RTN with ties to even, fp16 s_t and z_t); the rotated
 *   reconstruction is 2^e_j (s_t c_tj + z_t) and the original H (that)/128.
 *
 * iters = 0 leaves every e_j = 0: the per-token encoder, bit for bit.
 *
 * x: fp16 [T][128], T <= 16; present (optional, [T]): rows with 0 are
 * absent (no codes, no metadata, zero in the sums).  Outputs (each optional):
 * codes u8 [T][128], s, z fp16 bits [T], e int [128], out fp64 [T][128] (the
 * original-domain reconstruction; absent rows zero).  Returns 0, or -1 when T
 * is out of range.
 */
static int floor_div(int a, int b) { return a >= 0 ? a / b : -((b - 1 - a) / b); }   /* b > 0 */
static int floor_half(int f) { return floor_div(f, 2); }
#define KVQO_PB_EMAX 6

int kvqo_block_variant(const uint16_t *x, const uint8_t *present, int T, int bits, int iters,
                       uint8_t *codes_out, uint16_t *s_out, uint16_t *z_out, int *e_out, double *out)
{
    if (T < 0 || T > KVQO_PAGE || (bits != 2 && bits != 3 && bits != 4 && bits != 8) || iters < 0) return -1;
    const int L = (1 << bits) - 1;
    float Y[KVQO_PAGE][KVQO_D];
    int f[KVQO_PAGE], e[KVQO_D], has[KVQO_D];
    memset(Y, 0, sizeof(Y));
    for (int t = 0; t < T; t++) {
        if (present && !present[t]) continue;
        for (int j = 0; j < KVQO_D; j++) Y[t][j] = kvqo_half_to_float(x[t * KVQO_D + j]);
        kvqo_fwht_f32(Y[t]);
    }
    for (int t = 0; t < KVQO_PAGE; t++) f[t] = 0;
    for (int j = 0; j < KVQO_D; j++) { e[j] = 0; has[j] = 1; }
    float css[KVQO_D];          /* the last column pass's sums */
    for (int pass = 1; pass <= iters; pass++) {
        for (int j = 0; j < KVQO_D; j++) {
            float a[KVQO_PAGE];
            for (int t = 0; t < KVQO_PAGE; t++) {
                float u = ldexpf(Y[t][j], -f[t]);
                a[t] = u * u;
            }
            for (int h = KVQO_PAGE / 2; h >= 1; h >>= 1)
                for (int t = 0; t < h; t++) a[t] = a[t] + a[t + h];
            int F;
            css[j] = a[0];
            has[j] = a[0] != 0.0f;
            (void)frexpf(a[0], &F);
            e[j] = has[j] ? floor_half(F) : 0;
        }
        if (pass == iters) break;
        for (int t = 0; t < KVQO_PAGE; t++) {
            float a[KVQO_D];
            for (int j = 0; j < KVQO_D; j++) {
                float u = ldexpf(Y[t][j], -e[j]);
                a[j] = u * u;
            }
            for (int h = KVQO_D / 2; h >= 1; h >>= 1)
                for (int j = 0; j < h; j++) a[j] = a[j] + a[j + h];
            int F;
            (void)frexpf(a[0], &F);
            f[t] = a[0] != 0.0f ? floor_half(F) : 0;
        }
    }
    if (iters > 0) {
        int n = 0, S = 0, F[KVQO_D];
        for (int j = 0; j < KVQO_D; j++) {
            (void)frexpf(css[j], &F[j]);
            if (has[j]) { n++; S += F[j]; }
        }
        for (int j = 0; j < KVQO_D; j++) {
            if (!has[j]) { e[j] = -KVQO_PB_EMAX; continue; }
            const int d = n * F[j] - S;
            int r = (d < 2 * n && d > -2 * n) ? 0 : floor_div(d + n, 2 * n);
            e[j] = r < -KVQO_PB_EMAX ? -KVQO_PB_EMAX : r > KVQO_PB_EMAX ? KVQO_PB_EMAX : r;
        }
    }
    for (int t = 0; t < T; t++) {
        if (present && !present[t]) {
            if (out) memset(out + (int64_t)t * KVQO_D, 0, sizeof(double) * KVQO_D);
            continue;
        }
        float y[KVQO_D], p[KVQO_D];
        for (int j = 0; j < KVQO_D; j++) y[j] = ldexpf(Y[t][j], -e[j]);
        /* the encoder's steps 2-4 on the scaled rotated row (zero offset) */
        for (int j = 0; j < KVQO_D; j++) p[j] = y[j] * y[j];
        for (int h = KVQO_D / 2; h >= 1; h >>= 1)
            for (int j = 0; j < h; j++) p[j] = p[j] + p[j + h];
        uint8_t code[KVQO_D];
        memset(code, 0, sizeof(code));
        float sm = 0.0f, zm = 0.0f;
        if (p[0] != 0.0f) {
            float sigma = sqrtf(p[0] * 0x1p-7f);
            float rcp = 1.0f / sigma;
            float yh[KVQO_D];
            for (int j = 0; j < KVQO_D; j++) yh[j] = y[j] * rcp;
            float m = yh[0], M = yh[0];
            for (int j = 1; j < KVQO_D; j++) { if (yh[j] < m) m = yh[j]; if (yh[j] > M) M = yh[j]; }
            float delta = 0.0f;
            if (M != m) {
                delta = (M - m) / (float)L;
                float inv = (float)L / (M - m);
                for (int j = 0; j < KVQO_D; j++) {
                    float cc = rintf((yh[j] - m) * inv);
                    code[j] = (uint8_t)(cc > (float)L ? L : (int)cc);
                }
            }
            sm = delta * sigma;
            zm = m * sigma;
        }
        uint16_t s16 = kvqo_float_to_half(sm);
        uint16_t z16 = kvqo_float_to_half(zm);
        if (z16 == 0x8000) z16 = 0;
        if (codes_out) memcpy(codes_out + (int64_t)t * KVQO_D, code, KVQO_D);
        if (s_out) s_out[t] = s16;
        if (z_out) z_out[t] = z16;
        if (out) {
            double yt[KVQO_D];
            for (int j = 0; j < KVQO_D; j++)
                yt[j] = ldexp(kvqo_half_to_double(s16) * code[j] + kvqo_half_to_double(z16), e[j]);
            kvqo_hadamard_matvec_f64(yt, out + (int64_t)t * KVQO_D);
            for (int j = 0; j < KVQO_D; j++) out[(int64_t)t * KVQO_D + j] /= 128.0;
        }
    }
    if (e_out) memcpy(e_out, e, sizeof(e));
    return 0;
}

/*
 * The page-balanced key preset: the K4V2 layout of a 16-token region (1664
 * bytes) followed by the keys' 128 column scales, one byte each: byte j at
 * 1664 + j is the high byte of the fp16 bit pattern of 2^e_j (e_j in
 * [-6, 6]; the low byte of a power of two is zero), i.e. (e_j + 15) * 4.
 * 1792 bytes per (page, KV head), 112 per token.  Keys are balanced per page
 * with KVQO_PB_ITERS column passes (kvqo_block_variant, 4 bits, zero offset);
 * values are the v1 per-token groups (2 bits, group mean).
 */
#define KVQO_PB_REGION 1792
#define KVQO_PB_ITERS 2

int kvqo_pb_region_bytes(void) { return KVQO_PB_REGION; }
int kvqo_pb_iters(void) { return KVQO_PB_ITERS; }

/*
 * Append whole pages.  Call tokens 16b .. 16b + 15 form block b: with
 * base = slot_mapping[16b], the block fills page base / 16 from slot 0 and
 * token 16b + r belongs to it iff 16b + r < num_tokens and slot_mapping[16b +
 * r] == base + r (others are not written).  A block whose base is negative
 * or not a multiple of 16 is skipped; one whose page is >= num_pages is
 * skipped and makes the call return -1.  Slots of a page that no token of the
 * block fills keep their bytes; the page's column scales are rewritten.
 */
int kvqo_quantize_append_pb(const uint16_t *key, const uint16_t *value, int64_t key_token_stride,
                            int64_t value_token_stride, const int64_t *slot_mapping, int64_t num_tokens,
                            int32_t num_kv_heads, uint8_t *pool, int64_t num_pages)
{
    int rc = 0;
    for (int64_t b0 = 0; b0 < num_tokens; b0 += KVQO_PAGE) {
        const int64_t base = slot_mapping[b0];
        if (base < 0 || base % KVQO_PAGE) continue;
        const int64_t page = base / KVQO_PAGE;
        if (page >= num_pages) { rc = -1; continue; }
        uint8_t present[KVQO_PAGE];
        int T = 0;
        for (int r = 0; r < KVQO_PAGE; r++) {
            present[r] = b0 + r < num_tokens && slot_mapping[b0 + r] == base + r;
            if (b0 + r < num_tokens) T = r + 1;
        }
        for (int h = 0; h < num_kv_heads; h++) {
            uint16_t kx[KVQO_PAGE * KVQO_D];
            memset(kx, 0, sizeof(kx));
            for (int r = 0; r < T; r++)
                if (present[r])
                    memcpy(kx + r * KVQO_D, key + (b0 + r) * key_token_stride + (int64_t)h * KVQO_D,
                           sizeof(uint16_t) * KVQO_D);
            uint8_t kc[KVQO_PAGE * KVQO_D];
            uint16_t ks[KVQO_PAGE], kz[KVQO_PAGE];
            int e[KVQO_D];
            kvqo_block_variant(kx, present, T, 4, KVQO_PB_ITERS, kc, ks, kz, e, NULL);
            uint8_t *region = pool + (page * num_kv_heads + h) * KVQO_PB_REGION;
            for (int r = 0; r < T; r++) {
                if (!present[r]) continue;
                uint8_t vc[KVQO_D];
                uint16_t vs, vz;
                kvqo_quantize_group_mode(value + (b0 + r) * value_token_stride + (int64_t)h * KVQO_D, 2, 1,
                                         vc, &vs, &vz);
                kvqo_store_token_fmt(4, 2, region, r, kc + r * KVQO_D, ks[r], kz[r], vc, vs, vz);
            }
            for (int j = 0; j < KVQO_D; j++) region[KVQO_REGION + j] = (uint8_t)((e[j] + 15) * 4);
        }
    }
    return rc;
}

/* Dequantised, un-rotated key and value of token slot `off` of a
 * page-balanced region: key 2^e_j (s c_j + z) (e_j from the column-scale
 * byte), value as in v1; both through H / 128. */
void kvqo_dequant_slot_pb(const uint8_t *region, int off, double *k_out, double *v_out)
{
    uint8_t kc[KVQO_D], vc[KVQO_D];
    uint16_t ks, kz, vs, vz;
    kvqo_load_token_fmt(4, 2, region, off, kc, &ks, &kz, vc, &vs, &vz);
    double yt[KVQO_D];
    for (int j = 0; j < KVQO_D; j++) {
        const int e = region[KVQO_REGION + j] / 4 - 15;
        yt[j] = ldexp(kvqo_half_to_double(ks) * kc[j] + kvqo_half_to_double(kz), e);
    }
    kvqo_hadamard_matvec_f64(yt, k_out);
    for (int j = 0; j < KVQO_D; j++) k_out[j] /= 128.0;
    dequant_unrotate(vc, vs, vz, 1, v_out);
}

/* Plain definition of a decode step over a page-balanced cache (16-token
 * pages, u8 [num_pages][num_kv_heads][1792]): as kvqo_decode_attention, with
 * the keys dequantised by kvqo_dequant_slot_pb.  Returns 0, or -1 on an
 * invalid shape or page id. */
int kvqo_decode_attention_pb(const uint8_t *pool, int64_t num_pages, int32_t num_kv_heads,
                             const int32_t *block_tables, int32_t max_pages_per_seq, const int32_t *seq_lens,
                             int32_t num_seqs, int32_t num_q_heads, const uint16_t *query, double scale,
                             const uint8_t *head_mask, double *out)
{
    if (num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return -1;
    const int G = num_q_heads / num_kv_heads;
    for (int b = 0; b < num_seqs; b++) {
        const int64_t n = seq_lens[b];
        if (n < 0 || n > (int64_t)max_pages_per_seq * KVQO_PAGE) return -1;
        for (int kvh = 0; kvh < num_kv_heads; kvh++) {
            int any = 0;
            for (int g = 0; g < G; g++)
                if (!head_mask || head_mask[b * num_q_heads + kvh * G + g]) any = 1;
            if (!any) continue;
            double *K = malloc(sizeof(double) * KVQO_D * (n > 0 ? n : 1));
            double *V = malloc(sizeof(double) * KVQO_D * (n > 0 ? n : 1));
            if (!K || !V) { free(K); free(V); return -1; }
            for (int64_t t = 0; t < n; t++) {
                int32_t page = block_tables[(int64_t)b * max_pages_per_seq + t / KVQO_PAGE];
                if (page < 0 || page >= num_pages) { free(K); free(V); return -1; }
                kvqo_dequant_slot_pb(pool + ((int64_t)page * num_kv_heads + kvh) * KVQO_PB_REGION,
                                     (int)(t % KVQO_PAGE), K + t * KVQO_D, V + t * KVQO_D);
            }
            for (int g = 0; g < G; g++) {
                const int hq = kvh * G + g;
                if (head_mask && !head_mask[b * num_q_heads + hq]) continue;
                kvqo_attention_f64(K, V, n, query + ((int64_t)b * num_q_heads + hq) * KVQO_D, 1, scale,
                                   out + ((int64_t)b * num_q_heads + hq) * KVQO_D);
            }
            free(K); free(V);
        }
    }
    return 0;
}

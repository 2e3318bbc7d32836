/*
 * kvq.h -- C ABI of libkvq: K4V2 group-128 quantised paged KV cache (and the
 * same pipeline at 4/8-bit keys with 2/4-bit values, and at 3 bits both) for
 * AMD Instinct MI355X (gfx950).
 *
 * Two operations on a paged KV cache:
 *   kvq_quantize_append   quantise-on-write of new key/value tokens
 *   kvq_decode_attention  one decode step of attention over the packed cache
 *
 * The method is the KVarN write/read path described on these web pages:
 *   [KVARN-HN] beyondheadline.xyz, "Huawei's KV-cache trick: FP16 accuracy, a
 *              four-times-larger cache and higher throughput at once" -- lede
 *              and section "The claim that breaks the usual trade-off"
 *              (4-bit keys, 2-bit values, Hadamard rotation, variance
 *              normalisation, asymmetric low-bit quantisation of cache blocks;
 *              one preset flag, kvarn_k4v2_g128; no calibration, no model
 *              edits).
 *   [KVARN-P]  dothoosh.com, "KVarN vs TurboQuant: 5x more context with higher
 *              accuracy" -- the four-stage pipeline list (Hadamard rotation;
 *              variance normalisation; asymmetric round-to-nearest; scale
 *              folding on read-back) and the preset kv_cache_dtype string.
 *   [TQ]       dzen.ru summary of the vLLM TurboQuant post -- sections on
 *              accuracy and on memory (8-bit keys with 4-bit values, and 4-bit
 *              both, nearly lossless; 3-bit noticeably worse).
 *   [KV-INFRA] encorp.ai, "KV cache compression is an infrastructure decision,
 *              not a model debate" -- decode bound by HBM traffic; the section
 *              on OSCAR (sink and recent tokens kept in BF16).
 *
 * Cache format "kvq-k4v2-g128 v1" (the pages fix no numbers; this library
 * fixes them):
 *   - head_dim = group = 128: one group per token per KV head;
 *   - rotation: unnormalised Sylvester Hadamard H (H_ij = (-1)^popcount(i&j)),
 *     computed as an fp32 fast Walsh-Hadamard transform with butterfly stages
 *     h = 1, 2, ..., 64;
 *   - variance normalisation: divide by the group RMS sigma = sqrt(sum y^2 /
 *     128) (pairwise sum, fixed tree), folded back into the stored metadata;
 *   - asymmetric round-to-nearest-even on the group's [min m, max M]: keys
 *     to 4 bits (0..15), values to 2 bits (0..3), step delta = (M - m) / L;
 *     fp16 scale s = delta * sigma and one fp16 offset per group: keys store
 *     the zero z = m * sigma, values the group mean mu = sigma * (m + delta *
 *     C / 128) with C the sum of the group's codes (z = mu - s * C / 128).
 *     A rotated value is s * code + z and the original is H (s c + z) / 128;
 *     mu is the dequantised original channel 0 (H 1 = 128 e_0);
 *   - pages of 16 tokens; the pool is u8 [num_pages][num_kv_heads][1664],
 *     one 1664-byte region per (page, KV head):
 *       [0, 1024)     key codes, token o at 64*o, byte b = c[2b] | c[2b+1] << 4
 *       [1024, 1536)  value codes, token o (quad g = o/4, slot i = o%4): for
 *                     m = 0..15 the little-endian u16 at 1024 + 128g + 8m + 2i
 *                     holds the code of channel 16j + m in bits 2j..2j+1
 *       [1536, 1600)  key (s, z) fp16 pairs, token o at 1536 + 4*o
 *       [1600, 1664)  value (s, mu) fp16 pairs, token o at 1600 + 4*o
 *     104 bytes per token per KV head (fp16: 512 bytes).
 *
 * Other bit widths (k_bits in {4, 8}, v_bits in {2, 4}; presets "k4v4_g128",
 * "k8v2_g128", "k8v4_g128", also with the "kvarn_" prefix): the same pipeline
 * with L = 2^bits - 1, at the widths whose accuracy the pages compare (8-bit
 * keys with 4-bit values and 4-bit both reported as nearly lossless:
 * [TQ] dzen.ru summary of the vLLM TurboQuant post, sections on accuracy and
 * memory).  Values still store the group mean.  Region of
 * 256 * (k_bits + v_bits) + 128 bytes (2176, 2688, 3200), in this order:
 *       key codes     16 tokens x 16*k_bits bytes, token-major; the code of
 *                     channel c at bits k_bits*c.. of the token's row, least
 *                     significant first (8 bits: byte c)
 *       value codes   16 tokens x 16*v_bits bytes at 256*k_bits; 2 bits: as
 *                     above (u16 at base + 128g + 8m + 2i); 4 bits: with
 *                     j = 4h + k, the u16 at base + 256g + 16m + 8(i/2) + 4h +
 *                     2(i%2) holds the code of channel 16j + m in bits
 *                     4k..4k+3
 *       key (s, z)    16 x 4 bytes at 256*(k_bits + v_bits)
 *       value (s, mu) 16 x 4 bytes after them
 * 3 bits both ("k3v3_g128", also "kvarn_k3v3_g128"; the pages rank 3-bit codes
 * as noticeably less accurate than the widths above [TQ]): L = 7, codes
 * stored as bit planes, again 1664 bytes per region in the same order:
 *       key codes     the token's 48-byte row at 48*o: for G = 0..3 and
 *                     p = 0..2 the little-endian u32 at 12G + 4p holds, at
 *                     bit x, bit p of the code of channel 32G + x
 *       value codes   at 768: for quad g = o/4, slot i = o%4, channel
 *                     16j + m, byte (0, 2, 1, 3)[i] of the little-endian u32
 *                     at 768 + 12(16g + m) + 4p holds, at bit j, bit p of the
 *                     code
 *       key (s, z)    at 1536 + 4*o; value (s, mu) at 1600 + 4*o
 *
 * Page-balanced keys ("k4v2_g128_pb", also "kvarn_k4v2_g128_pb"; key_norm =
 * KVQ_KEY_NORM_PAGE): an active reading of the variance normalisation
 * [KVARN-P stage 2, worded there as repeated; its closing paragraph on
 * removing fluctuations in log space].  The rotated keys of one page of one
 * KV head (up to 16 tokens) are balanced as a block: two column passes of
 * second-moment balancing with a row pass between them, every scale a power
 * of two, give each channel j an exponent e_j in [-6, 6] (a channel within an
 * octave of the block's typical RMS keeps e_j = 0, a zero channel takes -6);
 * each token's scaled row Y_tj 2^-e_j is then encoded by the K4V2 steps
 * (RMS, asymmetric 4-bit round-to-nearest, fp16 s and z), and the rotated key
 * is 2^e_j (s c_j + z).  Values are the K4V2 per-token groups.  Region of
 * 1792 bytes: the K4V2 region (1664 bytes, same offsets) followed by 128
 * bytes, byte j at 1664 + j the high byte of the fp16 bit pattern of 2^e_j,
 * i.e. (e_j + 15) * 4; 112 bytes per token per KV head.  Pages of 16 tokens
 * only.  The block is a whole page, so kvq_quantize_append writes whole pages
 * (see there), and the fused append-and-decode and multi-row decode calls
 * return KVQ_ERR_UNSUPPORTED; the recent, partly filled page belongs in an
 * fp16 window merged by the mixed-cache calls below.
 *
 * Baseline format "fp16" (k_bits = v_bits = 16): the uncompressed cache the
 * K4V2 format is measured against (the pages compare KVarN with fp16 on
 * accuracy, capacity and throughput [KVARN-HN lede; KVARN-P results]).  The
 * same calls accept it, except the fused append-and-decode (KVQ_ERR_
 * UNSUPPORTED).  One 8192-byte region per (page, KV head), fp16 elements:
 *       [0, 4096)     keys: token n, channel c = 32d + 8g + e at element
 *                     n*128 + 32g + 8d + e
 *       [4096, 8192)  values: token t (q = t/4, i = t%4), channel c = 16j + m
 *                     at element 2048 + ((16q + m)*8 + j)*4 + i
 *     512 bytes per token per KV head.  kvq_quantize_append copies the rows
 *     (no quantisation); decode computes softmax(scale * q.k) v in fp32 with
 *     the same split-K structure, at most 256 pages per split.
 *
 * Conventions for every call:
 *   - All buffers are owned by the caller.  The library never allocates,
 *     frees or synchronises device memory.  Its only global mutable state is
 *     a thread-local last HIP error and, per device, the number of decode
 *     work-groups the device holds at once (queried on first use, stored
 *     atomically; concurrent first calls from several threads store the same
 *     value).  The measurement aids declared in kvq_measure.h add one more:
 *     a thread-local pair of timing events.
 *   - Pointers marked (device) are device pointers; (host) are host pointers.
 *     fp16 values are passed as their uint16_t bit patterns.
 *   - `stream` is a hipStream_t (NULL: the default stream).  Work is enqueued
 *     and the call returns without waiting.
 *   - Host-visible arguments are validated before anything is launched; a
 *     failed check returns a status and launches nothing.  Device-resident
 *     data (slot mappings, block tables, sequence lengths) are preconditions
 *     the host cannot read.  The kernels never access memory outside the
 *     buffers for any such value: append skips slots outside the pool, decode
 *     reads a page id outside the pool as page 0 and clamps sequence lengths
 *     to [0, max_seq_len]; the results under such violations are unspecified.
 *   - A launch failure returns KVQ_ERR_HIP; kvq_last_hip_error() gives the
 *     hipError_t code.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvq_status {
    KVQ_OK = 0,
    KVQ_ERR_NULL = 1,         /* a required pointer is NULL                    */
    KVQ_ERR_SHAPE = 2,        /* a size is out of range or inconsistent        */
    KVQ_ERR_UNSUPPORTED = 3,  /* unknown format, or a call the format lacks     */
    KVQ_ERR_ALIGN = 4,        /* a device pointer is not suitably aligned      */
    KVQ_ERR_WORKSPACE = 5,    /* workspace missing or smaller than required    */
    KVQ_ERR_HIP = 6           /* the HIP runtime reported an error             */
} kvq_status;

/* Format descriptor: {128, 128, k_bits, v_bits, block_size, key_norm} with
 * k_bits in {4, 8} and v_bits in {2, 4}, or k_bits = v_bits = 3, and
 * block_size in {16, 32, 64, 128} tokens per page ({128, 128, 4, 2, 16, 0}
 * is K4V2 v1), or {128, 128, 16, 16, 16, 0} (the fp16 baseline), or
 * {128, 128, 4, 2, 16, KVQ_KEY_NORM_PAGE} (page-balanced keys).  A page of
 * block_size tokens holds, per KV head, block_size / 16 consecutive 16-token
 * regions of the layout above: the pool is u8
 * [num_pages][num_kv_heads][block_size / 16][region], and token r of a page
 * (slot = page * block_size + r) sits in region r / 16, slot r % 16 (the
 * variable page size [KVARN-P] announces, read this way).  Block tables index
 * pages of block_size tokens.  key_norm is KVQ_KEY_NORM_GROUP (0: each
 * token's key group normalised on its own) unless set; an initialiser that
 * names only the first five fields leaves it 0. */
#define KVQ_KEY_NORM_GROUP 0
#define KVQ_KEY_NORM_PAGE 1

typedef struct kvq_format {
    int32_t head_dim;    /* channels per head                    */
    int32_t group_size;  /* channels per quantisation group      */
    int32_t k_bits;      /* key code width                       */
    int32_t v_bits;      /* value code width                     */
    int32_t block_size;  /* tokens per page                      */
    int32_t key_norm;    /* KVQ_KEY_NORM_GROUP or KVQ_KEY_NORM_PAGE */
} kvq_format;

typedef enum kvq_out_dtype { KVQ_OUT_F16 = 0, KVQ_OUT_F32 = 1 } kvq_out_dtype;

/* Parse a preset name ([KVARN-HN] flag value; [KVARN-P] kv_cache_dtype string).
 * Accepts "k4v2_g128" and "kvarn_k4v2_g128" ({128, 128, 4, 2, 16, 0}); "k4v4_g128",
 * "k8v2_g128", "k8v4_g128" and "k3v3_g128" (each with or without the "kvarn_"
 * prefix); "k4v2_g128_pb" and "kvarn_k4v2_g128_pb" (page-balanced keys,
 * {128, 128, 4, 2, 16, KVQ_KEY_NORM_PAGE}); and the baseline "fp16"
 * ({128, 128, 16, 16, 16, 0}).  Every preset has 16-token pages; set
 * block_size afterwards for larger ones (not with page-balanced keys).
 * preset, out: (host).
 * Returns KVQ_ERR_NULL, KVQ_ERR_UNSUPPORTED for any other name, else KVQ_OK. */
kvq_status kvq_format_from_string(const char *preset, kvq_format *out);

/* Bytes of one (page, KV head): block_size / 16 regions of 256 * (k_bits +
 * v_bits) + 128 bytes for a quantised format (1664 for K4V2 v1), 1792 with
 * page-balanced keys, 8192 for fp16; 0 for an unsupported format or NULL. */
size_t kvq_page_bytes(const kvq_format *fmt);

/* Bytes of a pool of num_pages pages and num_kv_heads heads; 0 on invalid input. */
size_t kvq_cache_bytes(const kvq_format *fmt, int64_t num_pages, int32_t num_kv_heads);

/*
 * Quantise-on-write [KVARN-HN; KVARN-P stages 1-3].
 *   key, value        (device) fp16 [num_tokens][num_kv_heads][128]; token
 *                     strides in elements (>= num_kv_heads*128), head stride
 *                     128; 16-byte aligned; token strides multiples of 8.
 *   slot_mapping      (device) int64 [num_tokens]; slot = page*block_size +
 *                     offset (offset < block_size).
 *                     A negative slot skips the token; a slot whose page is
 *                     >= num_pages is skipped.  Slots must be distinct.
 *   cache             (device) u8 pool [num_pages][num_kv_heads][page bytes]
 *                     (kvq_page_bytes(fmt): 1664 for K4V2), 16-byte aligned.
 *                     Only the addressed token slots change.
 * The codes depend only on the token's own 128 values (no calibration), so
 * appends are order-independent and idempotent.
 * Page-balanced keys encode whole pages instead: call tokens 16b .. 16b + 15
 * form block b, which fills page p = slot_mapping[16b] / 16 from its slot 0;
 * token 16b + r belongs to it iff 16b + r < num_tokens and
 * slot_mapping[16b + r] == 16p + r.  A block whose first slot is negative or
 * not a multiple of 16, or whose page is >= num_pages, is skipped.  The
 * block's tokens are balanced together (absent rows count as zeros); the
 * page's slots that no token of the block fills keep their bytes, and its
 * 128 column-scale bytes are rewritten.  Blocks must name distinct pages.
 * num_tokens == 0 is a no-op returning KVQ_OK.
 */
kvq_status kvq_quantize_append(const kvq_format *fmt,
                               const uint16_t *key, const uint16_t *value,
                               int64_t key_token_stride, int64_t value_token_stride,
                               const int64_t *slot_mapping, int64_t num_tokens,
                               int32_t num_kv_heads, uint8_t *cache, int64_t num_pages,
                               void *stream);

/* Workspace bytes the decode calls need for these sizes (0 on invalid
 * input).  The split plan depends on the KV-head count (it sets the number of
 * (sequence, KV head) work units that share the device) and on the split
 * size, so both are arguments: pages_per_split = 0 selects the library's
 * split heuristic; a positive value forces that many pages per split (see _ex
 * below).  The workspace holds the split partials, fp32
 * [num_seqs][num_q_heads][splits][132] with splits = ceil(ceil(max_seq_len /
 * 16) / pages_per_split). */
size_t kvq_decode_workspace_bytes(const kvq_format *fmt, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t max_seq_len, int32_t pages_per_split);

/*
 * One decode step of attention over the quantised cache, read with scale
 * folding [KVARN-P stage 4]: the key rotation is moved onto the query
 * (H is symmetric), (s, z) are applied inside the dot products, the softmax
 * runs online in fp32 in base 2, and a single Hadamard transform restores the
 * output.  Mathematically equal to
 *     out[b][hq] = sum_t softmax_t(softmax_scale * q . k_t) v_t,
 * with k_t, v_t the dequantised, un-rotated cache entries of tokens
 * t < seq_lens[b] and KV head hq / (num_q_heads / num_kv_heads).
 *   out             (device) [num_seqs][num_q_heads][128], fp16 or fp32.
 *   query           (device) fp16 [num_seqs][num_q_heads][128], contiguous.
 *   cache           (device) pool as above.
 *   block_tables    (device) int32 [num_seqs][max_pages_per_seq]; entry i of
 *                   row b is the page holding tokens 16i..16i+15 of sequence b.
 *                   Only entries i < ceil(seq_lens[b]/16) are read.
 *   seq_lens        (device) int32 [num_seqs], each in [1, max_seq_len]
 *                   (a zero length yields a zero output row).
 *   max_seq_len     host-side bound on seq_lens, <= max_pages_per_seq*16.
 *   workspace       (device) >= kvq_decode_workspace_bytes(...) bytes,
 *                   16-byte aligned, any contents (split partials are written
 *                   before they are read).  Calls that share a workspace must
 *                   not overlap in time.
 * Launches two kernels on `stream` (the split kernel, then the split combine
 * with the Hadamard epilogue) unless every sequence fits one split.
 * Returns KVQ_ERR_SHAPE when num_q_heads % num_kv_heads != 0 or a size is
 * non-positive, KVQ_ERR_WORKSPACE when workspace_bytes is too small.
 */
kvq_status kvq_decode_attention(const kvq_format *fmt, void *out, kvq_out_dtype out_dtype,
                                const uint16_t *query, const uint8_t *cache, int64_t num_pages,
                                const int32_t *block_tables, int32_t max_pages_per_seq,
                                const int32_t *seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t max_seq_len, float softmax_scale,
                                void *workspace, size_t workspace_bytes, void *stream);

/* As kvq_decode_attention, with the split-K granularity forced to
 * pages_per_split pages (a multiple of 2 in [2, 512]; else KVQ_ERR_SHAPE) per
 * work-group instead of the heuristic (which also stays within 512).  The
 * workspace must be sized with the same pages_per_split. */
kvq_status kvq_decode_attention_ex(const kvq_format *fmt, void *out, kvq_out_dtype out_dtype,
                                   const uint16_t *query, const uint8_t *cache, int64_t num_pages,
                                   const int32_t *block_tables, int32_t max_pages_per_seq,
                                   const int32_t *seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t max_seq_len, float softmax_scale,
                                   void *workspace, size_t workspace_bytes,
                                   int32_t pages_per_split, void *stream);

/*
 * The two phases of kvq_decode_attention_ex as separate calls, for callers
 * that time or place them separately, or that merge partials computed over
 * disjoint page sets of one sequence (each set's partials are combined by the
 * same log-sum-exp rule; the combine needs them in one workspace).
 *
 * kvq_decode_partials: the split phase [KVARN-P stage 4].  Same arguments
 * and preconditions as kvq_decode_attention_ex without the output.  For every
 * (sequence b, query head h) and split i < ceil(ceil(len_b / 16) /
 * pages_per_split), writes the partial of tokens [16 i pps, 16 (i+1) pps) at
 * float offset ((b * num_q_heads + h) * splits + i) * 132 of the workspace:
 *   [0] m     reference level of the base-2 logits scale * log2(e) * q.k
 *             (at most 8 below their maximum over the split's tokens),
 *   [1] l     sum of exp2(logit - m - 8) over the split's tokens,
 *   [2] zacc  the same weights times the value mean of each token,
 *   [3]       unused,
 *   [4..131]  acc, the weights times the rotated, scaled value codes
 *             s * c (Hadamard domain, not yet transformed back).
 * Split slots past a sequence's end (and every slot of an empty sequence)
 * receive an empty partial: m = -inf, l = zacc = 0, acc = 0.
 *
 * kvq_decode_combine: merges the partials of each (sequence, query head) and
 * applies the inverse rotation: after rescaling every split by
 * exp2(m_i - max_i m_i) and summing, out_j = (H acc)_j / (128 l) for j >= 1
 * and out_0 = zacc / l.  A sequence of
 * length 0 gets a zero row.  max_seq_len and pages_per_split must be those of
 * the kvq_decode_partials call that filled the workspace (0 selects the same
 * heuristic again), since they fix the number of split slots; seq_lens is
 * validated but not read (every slot holds a partial).  The call must follow
 * the partials call on the same stream or after a synchronisation.
 */
kvq_status kvq_decode_partials(const kvq_format *fmt, const uint16_t *query, const uint8_t *cache,
                               int64_t num_pages, const int32_t *block_tables, int32_t max_pages_per_seq,
                               const int32_t *seq_lens, int32_t num_seqs, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t max_seq_len, float softmax_scale,
                               void *workspace, size_t workspace_bytes, int32_t pages_per_split,
                               void *stream);

kvq_status kvq_decode_combine(const kvq_format *fmt, void *out, kvq_out_dtype out_dtype,
                              const int32_t *seq_lens, int32_t num_seqs, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t max_seq_len, const void *workspace,
                              size_t workspace_bytes, int32_t pages_per_split, void *stream);

/*
 * A decode step that first appends the step's new token: for every sequence
 * b with seq_lens[b] >= 1, the key and value rows new_key[b], new_value[b]
 * (fp16 [num_seqs][num_kv_heads][128], token strides in elements, >=
 * num_kv_heads * 128 and multiples of 8, 16-byte aligned) are quantised into
 * token seq_lens[b] - 1 (page block_tables[b][(seq_lens[b] - 1) / 16], slot
 * (seq_lens[b] - 1) % 16) exactly as kvq_quantize_append would store them
 * [KVARN-HN; KVARN-P stages 1-3], and the attention then covers seq_lens[b]
 * tokens including it [KVARN-P stage 4].  The encoding runs inside the decode
 * kernel, in the work-group that reads that page, so the step is one launch
 * fewer than kvq_quantize_append followed by kvq_decode_attention_ex, with
 * identical cache bytes and output.  A page id outside the pool is not
 * written (and is read as page 0, as in every decode call).  The cache is
 * written, so it is not const here, and must be 128-byte aligned (else
 * KVQ_ERR_ALIGN); sequences must not share the page that receives their new
 * token.
 *
 * kvq_append_decode_attention: both phases (as kvq_decode_attention_ex).
 * kvq_append_decode_partials: the split phase only (as kvq_decode_partials);
 * kvq_decode_combine finishes it.
 */
kvq_status kvq_append_decode_attention(const kvq_format *fmt, void *out, kvq_out_dtype out_dtype,
                                       const uint16_t *new_key, const uint16_t *new_value,
                                       int64_t key_token_stride, int64_t value_token_stride,
                                       const uint16_t *query, uint8_t *cache, int64_t num_pages,
                                       const int32_t *block_tables, int32_t max_pages_per_seq,
                                       const int32_t *seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t max_seq_len, float softmax_scale,
                                       void *workspace, size_t workspace_bytes, int32_t pages_per_split,
                                       void *stream);

kvq_status kvq_append_decode_partials(const kvq_format *fmt, const uint16_t *new_key, const uint16_t *new_value,
                                      int64_t key_token_stride, int64_t value_token_stride,
                                      const uint16_t *query, uint8_t *cache, int64_t num_pages,
                                      const int32_t *block_tables, int32_t max_pages_per_seq,
                                      const int32_t *seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t max_seq_len, float softmax_scale,
                                      void *workspace, size_t workspace_bytes, int32_t pages_per_split,
                                      void *stream);

/*
 * The decode step of kvq_append_decode_attention without a caller-supplied
 * workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 * The split partials go to a fixed array of KVQ_NOALLOC_SCRATCH_BYTES in
 * the library's device code, one per device, resolved on the first call on
 * each device (with that device current) and held until the process ends.
 * The call allocates nothing, on the host or the device.
 *   Arguments, layouts, checks and results: as kvq_append_decode_attention
 *   with workspace and workspace_bytes left out.
 *   Errors: KVQ_ERR_WORKSPACE, before anything touches the device, when the
 *   partials of these sizes (kvq_decode_workspace_bytes(fmt, num_seqs,
 *   num_q_heads, num_kv_heads, max_seq_len, pages_per_split)) exceed
 *   KVQ_NOALLOC_SCRATCH_BYTES; KVQ_ERR_UNSUPPORTED on a device index >= 64;
 *   KVQ_ERR_HIP if the array's address cannot be resolved; otherwise the
 *   statuses of kvq_append_decode_attention (invalid sizes included).
 * Every call on a device shares that device's array, and it keeps the last
 * call's contents (the partials are written before they are read, so
 * nothing needs clearing).  Calls that overlap in time on one device --
 * concurrent streams, or several host threads -- race on it: serialise
 * them, e.g. on one stream.
 */
#define KVQ_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

kvq_status kvq_append_decode_attention_noalloc(const kvq_format *fmt, void *out, kvq_out_dtype out_dtype,
                                               const uint16_t *new_key, const uint16_t *new_value,
                                               int64_t key_token_stride, int64_t value_token_stride,
                                               const uint16_t *query, uint8_t *cache, int64_t num_pages,
                                               const int32_t *block_tables, int32_t max_pages_per_seq,
                                               const int32_t *seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                               int32_t num_kv_heads, int32_t max_seq_len, float softmax_scale,
                                               int32_t pages_per_split, void *stream);

/*
 * Several query rows per sequence: the q_len newest tokens of every sequence
 * (a speculative-decoding draft being verified, or a chunk of a prefill),
 * already appended to the cache, attend at once.  Row m of sequence b sits at
 * position seq_lens[b] - q_len + m and attends causally to tokens
 * 0 .. seq_lens[b] - q_len + m (a row that sees no token is zero).  The page
 * stream is read once for all rows: each (row, head) pair takes a column of
 * the decode kernel's MFMA tiles, so q_len * G columns per KV head fill the
 * tiles that a small GQA group leaves empty.
 *   query      (device) fp16 [num_seqs][q_len][num_q_heads][128], contiguous
 *   out        (device) fp16|fp32 [num_seqs][q_len][num_q_heads][128]
 *   q_len      1 .. 16; q_len * num_q_heads <= 65535
 *   workspace  kvq_decode_workspace_bytes_mq(...) bytes (the workspace of a
 *              decode with q_len * num_q_heads query heads)
 * Quantised formats only for q_len > 1 (fp16: KVQ_ERR_UNSUPPORTED).  Other
 * arguments, checks and ownership as kvq_decode_attention_ex; q_len = 1 is
 * that call.  Precondition: seq_lens[b] >= q_len.
 */
size_t kvq_decode_workspace_bytes_mq(const kvq_format *fmt, int32_t num_seqs, int32_t q_len,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t max_seq_len,
                                     int32_t pages_per_split);

kvq_status kvq_decode_attention_mq(const kvq_format *fmt, void *out, kvq_out_dtype out_dtype,
                                   const uint16_t *query, int32_t q_len, const uint8_t *cache, int64_t num_pages,
                                   const int32_t *block_tables, int32_t max_pages_per_seq,
                                   const int32_t *seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t max_seq_len, float softmax_scale,
                                   void *workspace, size_t workspace_bytes, int32_t pages_per_split,
                                   void *stream);

/*
 * Mixed caches: the partials of several caches merged by one combine.  A
 * decode step may read its tokens from more than one cache -- e.g. the first
 * (sink) and the most recent tokens kept uncompressed in an fp16 cache beside
 * the K4V2 history, as deployed low-bit caches do ([KV-INFRA] section on
 * OSCAR: sink and recent tokens in BF16, the history compressed) -- and the
 * attention over the union of their tokens is the log-sum-exp merge of each
 * cache's split partials.  Both formats produce partials in the same base-2
 * logit units.
 *
 * kvq_decode_split_slots: number of partial slots (splits) a partials call
 * over one cache with these sizes uses; 0 on invalid input.
 *
 * kvq_decode_partials_slots: as kvq_decode_partials, but the partial of split
 * i goes to slot slot_offset + i of rows holding total_slots slots each: the
 * workspace holds fp32 [num_seqs][num_q_heads][total_slots][132], at least
 * num_seqs * num_q_heads * total_slots * 528 bytes, 16-byte aligned.
 * rotated = 1 stores the partial in the Hadamard domain of the quantised
 * caches (acc' = H acc, zacc = acc_0), as their partials always are (0 is
 * rejected for them); set it for an fp16 cache whose partials are merged with
 * quantised-cache ones.  slot_offset + the call's split count must not exceed
 * total_slots (else KVQ_ERR_SHAPE).  Caches of different quantised widths
 * may also share one workspace row.
 *
 * kvq_decode_combine_slots: merges all total_slots slots of every (sequence,
 * query head) row and writes out (fp16 or fp32 [num_seqs][num_q_heads][128]).
 * rotated = 1 applies the quantised-cache epilogue (any mix holding their
 * partials or rotated fp16 ones), 0 the plain one (unrotated fp16 partials
 * only).  Every slot must have been written by a partials call for this step.
 */
int32_t kvq_decode_split_slots(const kvq_format *fmt, int32_t num_seqs, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t max_seq_len, int32_t pages_per_split);

kvq_status kvq_decode_partials_slots(const kvq_format *fmt, const uint16_t *query, const uint8_t *cache,
                                     int64_t num_pages, const int32_t *block_tables, int32_t max_pages_per_seq,
                                     const int32_t *seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t max_seq_len, float softmax_scale,
                                     void *workspace, size_t workspace_bytes, int32_t pages_per_split,
                                     int32_t slot_offset, int32_t total_slots, int32_t rotated, void *stream);

kvq_status kvq_decode_combine_slots(void *out, kvq_out_dtype out_dtype, int32_t num_seqs, int32_t num_q_heads,
                                    const void *workspace, size_t workspace_bytes, int32_t total_slots,
                                    int32_t rotated, void *stream);

/* Pages per split the heuristic picks for these sizes with the K4V2 format
 * (0 on invalid input).  The heuristic plans one round of work-groups: the
 * device's compute units times the work-groups per unit that fit (at most
 * two), divided among the (sequence, KV head, head group) units, rounded up
 * to whole page pairs and capped at 512 pages.  The other formats' choice
 * shows in kvq_decode_split_slots and kvq_decode_workspace_bytes. */
int32_t kvq_decode_pages_per_split(int32_t num_seqs, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t max_seq_len);

/* Static description of a status code (never NULL). */
const char *kvq_status_string(kvq_status status);

/* hipError_t of the last KVQ_ERR_HIP returned on this thread (0 if none). */
int kvq_last_hip_error(void);

/* Library version string, e.g. "kvq 1.0 (kvq-k4v2-g128 v1, gfx950)". */
const char *kvq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */

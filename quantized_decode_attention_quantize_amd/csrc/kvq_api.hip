// C ABI of libkvq: argument validation, sizing and dispatch to the kernels.
// The declarations, argument meanings, layouts and error behaviour are in
// include/kvq.h.
#include <string.h>

#include <mutex>

#include "../../include/kvq.h"
#include "../../include/kvq_measure.h"
#include "kvq_device.h"
#include "kvq_probe.h"

namespace {

thread_local int g_last_hip_error = 0;
thread_local kvq::LaunchEvents g_split_events;

bool is_g128(const kvq_format *f) { return f && f->head_dim == 128 && f->group_size == 128; }

// log2 of the 16-token regions per page: pages of 16, 32, 64 or 128 tokens
int page_log2s(const kvq_format *f) {
    switch (f->block_size) {
    case 16: return 0;
    case 32: return 1;
    case 64: return 2;
    case 128: return 3;
    default: return -1;
    }
}

// Page-balanced keys: K4V2 with 16-token pages and per-page column scales.
bool is_pb(const kvq_format *f) {
    return is_g128(f) && f->key_norm == KVQ_KEY_NORM_PAGE && f->k_bits == 4 && f->v_bits == 2 &&
           f->block_size == 16;
}

// A quantised cache: 4- or 8-bit keys with 2- or 4-bit values (4/2 is
// KVarN's), or 3 bits both; pages of 16 to 128 tokens; or page-balanced keys.
bool is_quant(const kvq_format *f) {
    return (is_g128(f) && f->key_norm == KVQ_KEY_NORM_GROUP &&
            (((f->k_bits == 4 || f->k_bits == 8) && (f->v_bits == 2 || f->v_bits == 4)) ||
             (f->k_bits == 3 && f->v_bits == 3)) &&
            page_log2s(f) >= 0) ||
           is_pb(f);
}

// The uncompressed fp16 baseline cache (16-token pages).
bool is_fp16(const kvq_format *f) {
    return is_g128(f) && f->key_norm == KVQ_KEY_NORM_GROUP && f->k_bits == 16 && f->v_bits == 16 &&
           f->block_size == 16;
}

bool is_known(const kvq_format *f) { return is_quant(f) || is_fp16(f); }

// Bytes of one (page, KV head): its 16-token regions.
size_t region_bytes(const kvq_format *f) {
    return is_pb(f) ? (size_t)kvq::kRegionPB
                    : is_quant(f) ? (size_t)(256 * (f->k_bits + f->v_bits) + 128) << page_log2s(f)
                                  : is_fp16(f) ? (size_t)kvq::kRegionF16 : 0;
}

int32_t max_pps(bool fp16) { return fp16 ? kvq::kMaxPagesPerSplitF16 : kvq::kMaxPagesPerSplit; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

kvq_status hip_status(hipError_t e) {
    if (e == hipSuccess) return KVQ_OK;
    g_last_hip_error = (int)e;
    return KVQ_ERR_HIP;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Split partials of kvq_append_decode_attention_noalloc, for callers that
// cannot allocate: one fixed array per device, held until the process ends.
// Host code never passes the array's name to a kernel (on the host it is a
// stand-in, not a device address): the device address is resolved once per
// device with hipGetSymbolAddress and kept in g_scratch_ptr.
constexpr size_t kScratchBytes = (size_t)16 << 20;
static_assert(kScratchBytes == KVQ_NOALLOC_SCRATCH_BYTES, "the header states the scratch size");
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[64];    // per device: the address of `scratch` there, once resolved

// Device address of `scratch` on the current device (resolved on the first
// call on each device, with that device current).
kvq_status scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= 64) return KVQ_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e);
        if (!p) return KVQ_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return KVQ_OK;
}

int32_t head_groups(int32_t gqa) { return (int32_t)ceil_div(gqa, kvq::kHeadsPerGroup); }

// Split heuristic: one round of resident work-groups.  A (sequence, KV head,
// work-group of head groups) unit is cut into S = max(1, resident / units) splits of equal
// page count (rounded up to a page pair), so every work-group starts at once,
// carries the same work, and pays its fixed cost (query rotation, wave merge,
// partial write) once.
int32_t heuristic_pps(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t max_seq_len,
                      int32_t k_bits = 4, int32_t v_bits = 2, bool page_balanced = false) {
    const bool fp16 = k_bits == 16;
    // work-groups per (sequence, KV head): the quantised kernel takes two head
    // groups per work-group when there are several; the fp16 kernel one
    const int64_t hgs = head_groups(num_q_heads / num_kv_heads);
    const int64_t wgs = fp16 || hgs < 2 ? hgs : (hgs + 1) / 2;
    const int64_t units = (int64_t)num_seqs * num_kv_heads * wgs;
    const int64_t max_pages = ceil_div(max_seq_len, kvq::kPage);
    const int64_t resident = fp16 ? kvq::decode_fp16_resident_workgroups()
                                  : kvq::decode_resident_workgroups(k_bits, v_bits, page_balanced);
    int64_t splits = resident / units;
    if (splits < 1) splits = 1;
    int64_t pps = ceil_div(max_pages, splits);
    pps = ceil_div(pps, 2) * 2;
    if (pps < 2) pps = 2;
    if (pps > max_pps(fp16)) pps = max_pps(fp16);
    return (int32_t)pps;
}

bool decode_sizes_ok(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t max_seq_len) {
    return num_seqs > 0 && num_q_heads > 0 && num_kv_heads > 0 && max_seq_len > 0 &&
           num_q_heads % num_kv_heads == 0 && num_seqs <= 65535 &&
           (int64_t)num_kv_heads * head_groups(num_q_heads / num_kv_heads) <= 65535;
}

struct WorkspaceLayout {
    int32_t splits;
    size_t total;
};

WorkspaceLayout layout(int32_t num_seqs, int32_t num_q_heads, int32_t max_seq_len, int32_t pps) {
    WorkspaceLayout w;
    const int64_t max_pages = ceil_div(max_seq_len, kvq::kPage);
    w.splits = (int32_t)ceil_div(max_pages, pps);
    const size_t partial_bytes = (size_t)num_seqs * num_q_heads * w.splits * kvq::kPartialFloats * sizeof(float);
    w.total = ((partial_bytes + 255) & ~(size_t)255) + 256;
    return w;
}

// Checks shared by the decode entry points; fills the sizes, the split
// decomposition and the workspace of `a`.  max_pages_per_seq < 0: no block
// table (the combine).
kvq_status decode_common(const kvq_format *fmt, const int32_t *seq_lens, int32_t num_seqs,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t max_seq_len,
                         int32_t max_pages_per_seq, void *workspace, size_t workspace_bytes,
                         int32_t pages_per_split, kvq::DecodeArgs &a) {
    if (!fmt) return KVQ_ERR_NULL;
    if (!is_known(fmt)) return KVQ_ERR_UNSUPPORTED;
    if (!seq_lens) return KVQ_ERR_NULL;
    const bool fp16 = is_fp16(fmt);
    if (!decode_sizes_ok(num_seqs, num_q_heads, num_kv_heads, max_seq_len) || pages_per_split < 0 ||
        (pages_per_split % 2) || pages_per_split > max_pps(fp16))
        return KVQ_ERR_SHAPE;
    if (max_pages_per_seq >= 0 &&
        (max_pages_per_seq == 0 || (int64_t)max_seq_len > (int64_t)max_pages_per_seq * fmt->block_size))
        return KVQ_ERR_SHAPE;
    if ((uintptr_t)seq_lens & 3u) return KVQ_ERR_ALIGN;
    const int32_t pps = pages_per_split ? pages_per_split
                                        : heuristic_pps(num_seqs, num_q_heads, num_kv_heads, max_seq_len,
                                                        fmt->k_bits, fmt->v_bits, is_pb(fmt));
    const WorkspaceLayout w = layout(num_seqs, num_q_heads, max_seq_len, pps);
    if (!workspace || workspace_bytes < w.total) return KVQ_ERR_WORKSPACE;
    if (!aligned16(workspace)) return KVQ_ERR_ALIGN;
    if (w.splits > 65535) return KVQ_ERR_SHAPE;
    memset(&a, 0, sizeof(a));
    a.q_len = 1;
    a.rotated = fp16 ? 0 : 1;
    a.k_bits = fmt->k_bits;
    a.v_bits = fmt->v_bits;
    a.key_norm = is_pb(fmt) ? 1 : 0;
    a.page_log2s = fp16 ? 0 : page_log2s(fmt);
    a.max_seq_len = max_seq_len;
    a.seq_lens = seq_lens;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.gqa = num_q_heads / num_kv_heads;
    a.head_groups = head_groups(a.gqa);
    a.splits = w.splits;
    a.slot_offset = 0;
    a.slot_stride = w.splits;
    a.pages_per_split = pps;
    a.partials = static_cast<float *>(workspace);
    return KVQ_OK;
}

kvq_status decode_inputs(const uint16_t *query, const uint8_t *cache, int64_t num_pages,
                         const int32_t *block_tables, int32_t max_pages_per_seq, float softmax_scale,
                         kvq::DecodeArgs &a) {
    if (!query || !cache || !block_tables) return KVQ_ERR_NULL;
    if (num_pages <= 0) return KVQ_ERR_SHAPE;
    if (!(softmax_scale == softmax_scale)) return KVQ_ERR_SHAPE;
    if (!aligned16(query) || !aligned16(cache) || ((uintptr_t)block_tables & 3u)) return KVQ_ERR_ALIGN;
    a.query = query;
    a.cache = cache;
    a.num_pages = num_pages;
    a.block_tables = block_tables;
    a.bt_stride = max_pages_per_seq;
    // quantised-cache scores carry the 128 of H H = 128 I; fp16 scores do not
    a.alpha = a.rotated ? softmax_scale * 1.4426950408889634f / 128.0f : softmax_scale * 1.4426950408889634f;
    return KVQ_OK;
}

kvq_status append_inputs(const uint16_t *new_key, const uint16_t *new_value, int64_t key_token_stride,
                         int64_t value_token_stride, kvq::DecodeArgs &a) {
    // the fused append exists for quantised caches with per-token key groups
    // only (page-balanced keys are encoded a whole page at a time)
    if (!a.rotated || a.key_norm) return KVQ_ERR_UNSUPPORTED;
    if (!new_key || !new_value) return KVQ_ERR_NULL;
    const int64_t row = (int64_t)a.num_kv_heads * kvq::kHeadDim;
    if (key_token_stride < row || value_token_stride < row) return KVQ_ERR_SHAPE;
    if (!aligned16(new_key) || !aligned16(new_value) || (key_token_stride % 8) || (value_token_stride % 8) ||
        ((uintptr_t)a.cache & 127u))
        return KVQ_ERR_ALIGN;
    a.append = 1;
    a.new_key = new_key;
    a.new_value = new_value;
    a.new_key_stride = key_token_stride;
    a.new_value_stride = value_token_stride;
    return KVQ_OK;
}

kvq_status decode_output(void *out, kvq_out_dtype out_dtype, kvq::DecodeArgs &a) {
    if (out_dtype != KVQ_OUT_F16 && out_dtype != KVQ_OUT_F32) return KVQ_ERR_UNSUPPORTED;
    if (!out) return KVQ_ERR_NULL;
    if (!aligned16(out)) return KVQ_ERR_ALIGN;
    a.out = out;
    a.out_f32 = out_dtype == KVQ_OUT_F32;
    return KVQ_OK;
}

hipError_t launch_split(const kvq::DecodeArgs &a, hipStream_t stream) {
    return a.rotated ? kvq::launch_decode_split(a, stream, g_split_events)
                     : kvq::launch_fp16_decode_split(a, stream, g_split_events);
}

// Split kernel, then the combine unless every sequence fits one split.
hipError_t launch_both(const kvq::DecodeArgs &a, hipStream_t stream) {
    const hipError_t e = launch_split(a, stream);
    if (e != hipSuccess || (a.splits <= 1 && !a.partials_only)) return e;
    return kvq::launch_decode_combine(a, stream);
}

}  // namespace

extern "C" {

kvq_status kvq_format_from_string(const char *preset, kvq_format *out) {
    if (!preset || !out) return KVQ_ERR_NULL;
    static const struct {
        const char *name;
        int32_t k_bits, v_bits, key_norm;
    } presets[] = {
        {"k4v2_g128", 4, 2, 0}, {"kvarn_k4v2_g128", 4, 2, 0}, {"k4v4_g128", 4, 4, 0}, {"kvarn_k4v4_g128", 4, 4, 0},
        {"k8v2_g128", 8, 2, 0}, {"kvarn_k8v2_g128", 8, 2, 0}, {"k8v4_g128", 8, 4, 0}, {"kvarn_k8v4_g128", 8, 4, 0},
        {"k3v3_g128", 3, 3, 0}, {"kvarn_k3v3_g128", 3, 3, 0},
        {"k4v2_g128_pb", 4, 2, KVQ_KEY_NORM_PAGE}, {"kvarn_k4v2_g128_pb", 4, 2, KVQ_KEY_NORM_PAGE},
        {"fp16", 16, 16, 0},
    };
    for (const auto &p : presets) {
        if (strcmp(preset, p.name) == 0) {
            out->head_dim = 128;
            out->group_size = 128;
            out->k_bits = p.k_bits;
            out->v_bits = p.v_bits;
            out->block_size = 16;
            out->key_norm = p.key_norm;
            return KVQ_OK;
        }
    }
    return KVQ_ERR_UNSUPPORTED;
}

size_t kvq_page_bytes(const kvq_format *fmt) { return region_bytes(fmt); }

size_t kvq_cache_bytes(const kvq_format *fmt, int64_t num_pages, int32_t num_kv_heads) {
    if (!is_known(fmt) || num_pages < 0 || num_kv_heads <= 0) return 0;
    return (size_t)num_pages * (size_t)num_kv_heads * region_bytes(fmt);
}

kvq_status kvq_quantize_append(const kvq_format *fmt, const uint16_t *key, const uint16_t *value,
                               int64_t key_token_stride, int64_t value_token_stride,
                               const int64_t *slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                               uint8_t *cache, int64_t num_pages, void *stream) {
    if (!fmt) return KVQ_ERR_NULL;
    if (!is_known(fmt)) return KVQ_ERR_UNSUPPORTED;
    if (num_tokens < 0 || num_kv_heads <= 0 || num_pages < 0) return KVQ_ERR_SHAPE;
    if (num_tokens == 0) return KVQ_OK;
    if (!key || !value || !slot_mapping || !cache) return KVQ_ERR_NULL;
    const int64_t row = (int64_t)num_kv_heads * kvq::kHeadDim;
    if (key_token_stride < row || value_token_stride < row) return KVQ_ERR_SHAPE;
    if (num_tokens > ((int64_t)1 << 40) / num_kv_heads) return KVQ_ERR_SHAPE;
    if (!aligned16(key) || !aligned16(value) || !aligned16(cache) || ((uintptr_t)slot_mapping & 7u) ||
        (key_token_stride % 8) || (value_token_stride % 8))
        return KVQ_ERR_ALIGN;
    kvq::AppendArgs a;
    a.key = key;
    a.value = value;
    a.key_stride = key_token_stride;
    a.value_stride = value_token_stride;
    a.slots = slot_mapping;
    a.num_tokens = num_tokens;
    a.num_kv_heads = num_kv_heads;
    a.cache = cache;
    a.num_pages = num_pages;
    a.k_bits = fmt->k_bits;
    a.v_bits = fmt->v_bits;
    a.page_log2s = is_fp16(fmt) ? 0 : page_log2s(fmt);
    if (is_pb(fmt)) {
        if (num_kv_heads > 65535) return KVQ_ERR_SHAPE;
        return hip_status(kvq::launch_balance_append(a, (hipStream_t)stream));
    }
    return hip_status(is_fp16(fmt) ? kvq::launch_fp16_append(a, (hipStream_t)stream)
                                   : kvq::launch_append(a, (hipStream_t)stream));
}

int32_t kvq_decode_pages_per_split(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t max_seq_len) {
    if (!decode_sizes_ok(num_seqs, num_q_heads, num_kv_heads, max_seq_len)) return 0;
    return heuristic_pps(num_seqs, num_q_heads, num_kv_heads, max_seq_len);
}

size_t kvq_decode_workspace_bytes(const kvq_format *fmt, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t max_seq_len, int32_t pages_per_split) {
    if (!is_known(fmt) || !decode_sizes_ok(num_seqs, num_q_heads, num_kv_heads, max_seq_len)) return 0;
    const bool fp16 = is_fp16(fmt);
    if (pages_per_split < 0 || (pages_per_split % 2) || pages_per_split > max_pps(fp16)) return 0;
    const int32_t pps = pages_per_split ? pages_per_split
                                        : heuristic_pps(num_seqs, num_q_heads, num_kv_heads, max_seq_len, fmt->k_bits, fmt->v_bits,
                                                        is_pb(fmt));
    return layout(num_seqs, num_q_heads, max_seq_len, pps).total;
}

kvq_status kvq_decode_attention_ex(const kvq_format *fmt, void *out, kvq_out_dtype out_dtype,
                                   const uint16_t *query, const uint8_t *cache, int64_t num_pages,
                                   const int32_t *block_tables, int32_t max_pages_per_seq,
                                   const int32_t *seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t max_seq_len, float softmax_scale,
                                   void *workspace, size_t workspace_bytes, int32_t pages_per_split,
                                   void *stream) {
    kvq::DecodeArgs a;
    kvq_status st = decode_common(fmt, seq_lens, num_seqs, num_q_heads, num_kv_heads, max_seq_len,
                                  max_pages_per_seq, workspace, workspace_bytes, pages_per_split, a);
    if (st == KVQ_OK) st = decode_output(out, out_dtype, a);
    if (st == KVQ_OK) st = decode_inputs(query, cache, num_pages, block_tables, max_pages_per_seq, softmax_scale, a);
    if (st != KVQ_OK) return st;
    return hip_status(launch_both(a, (hipStream_t)stream));
}

kvq_status kvq_decode_partials(const kvq_format *fmt, const uint16_t *query, const uint8_t *cache,
                               int64_t num_pages, const int32_t *block_tables, int32_t max_pages_per_seq,
                               const int32_t *seq_lens, int32_t num_seqs, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t max_seq_len, float softmax_scale,
                               void *workspace, size_t workspace_bytes, int32_t pages_per_split,
                               void *stream) {
    kvq::DecodeArgs a;
    kvq_status st = decode_common(fmt, seq_lens, num_seqs, num_q_heads, num_kv_heads, max_seq_len,
                                  max_pages_per_seq, workspace, workspace_bytes, pages_per_split, a);
    if (st == KVQ_OK) st = decode_inputs(query, cache, num_pages, block_tables, max_pages_per_seq, softmax_scale, a);
    if (st != KVQ_OK) return st;
    a.partials_only = 1;
    return hip_status(launch_split(a, (hipStream_t)stream));
}

kvq_status kvq_append_decode_partials(const kvq_format *fmt, const uint16_t *new_key, const uint16_t *new_value,
                                      int64_t key_token_stride, int64_t value_token_stride,
                                      const uint16_t *query, uint8_t *cache, int64_t num_pages,
                                      const int32_t *block_tables, int32_t max_pages_per_seq,
                                      const int32_t *seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t max_seq_len, float softmax_scale,
                                      void *workspace, size_t workspace_bytes, int32_t pages_per_split,
                                      void *stream) {
    kvq::DecodeArgs a;
    kvq_status st = decode_common(fmt, seq_lens, num_seqs, num_q_heads, num_kv_heads, max_seq_len,
                                  max_pages_per_seq, workspace, workspace_bytes, pages_per_split, a);
    if (st == KVQ_OK) st = decode_inputs(query, cache, num_pages, block_tables, max_pages_per_seq, softmax_scale, a);
    if (st == KVQ_OK) st = append_inputs(new_key, new_value, key_token_stride, value_token_stride, a);
    if (st != KVQ_OK) return st;
    a.partials_only = 1;
    return hip_status(launch_split(a, (hipStream_t)stream));
}

kvq_status kvq_append_decode_attention(const kvq_format *fmt, void *out, kvq_out_dtype out_dtype,
                                       const uint16_t *new_key, const uint16_t *new_value,
                                       int64_t key_token_stride, int64_t value_token_stride,
                                       const uint16_t *query, uint8_t *cache, int64_t num_pages,
                                       const int32_t *block_tables, int32_t max_pages_per_seq,
                                       const int32_t *seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t max_seq_len, float softmax_scale,
                                       void *workspace, size_t workspace_bytes, int32_t pages_per_split,
                                       void *stream) {
    kvq::DecodeArgs a;
    kvq_status st = decode_common(fmt, seq_lens, num_seqs, num_q_heads, num_kv_heads, max_seq_len,
                                  max_pages_per_seq, workspace, workspace_bytes, pages_per_split, a);
    if (st == KVQ_OK) st = decode_output(out, out_dtype, a);
    if (st == KVQ_OK) st = decode_inputs(query, cache, num_pages, block_tables, max_pages_per_seq, softmax_scale, a);
    if (st == KVQ_OK) st = append_inputs(new_key, new_value, key_token_stride, value_token_stride, a);
    if (st != KVQ_OK) return st;
    return hip_status(launch_both(a, (hipStream_t)stream));
}

kvq_status kvq_append_decode_attention_noalloc(const kvq_format *fmt, void *out, kvq_out_dtype out_dtype,
                                               const uint16_t *new_key, const uint16_t *new_value,
                                               int64_t key_token_stride, int64_t value_token_stride,
                                               const uint16_t *query, uint8_t *cache, int64_t num_pages,
                                               const int32_t *block_tables, int32_t max_pages_per_seq,
                                               const int32_t *seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                               int32_t num_kv_heads, int32_t max_seq_len, float softmax_scale,
                                               int32_t pages_per_split, void *stream) {
    // the partials this call needs must fit the fixed array (checked before
    // the device is touched); sizes the workspace query rejects are rejected
    // the same way as by kvq_append_decode_attention, and so are the formats
    // without a fused append (the fp16 baseline, page-balanced keys)
    if (!fmt) return KVQ_ERR_NULL;
    if (!is_quant(fmt) || is_pb(fmt)) return KVQ_ERR_UNSUPPORTED;
    const size_t need = kvq_decode_workspace_bytes(fmt, num_seqs, num_q_heads, num_kv_heads, max_seq_len,
                                                   pages_per_split);
    if (need > kScratchBytes) return KVQ_ERR_WORKSPACE;
    void *ws = nullptr;
    if (need > 0) {
        const kvq_status st = scratch_address(&ws);
        if (st != KVQ_OK) return st;
    }
    return kvq_append_decode_attention(fmt, out, out_dtype, new_key, new_value, key_token_stride,
                                       value_token_stride, query, cache, num_pages, block_tables,
                                       max_pages_per_seq, seq_lens, num_seqs, num_q_heads, num_kv_heads,
                                       max_seq_len, softmax_scale, ws, need ? kScratchBytes : 0,
                                       pages_per_split, stream);
}

int32_t kvq_decode_split_slots(const kvq_format *fmt, int32_t num_seqs, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t max_seq_len, int32_t pages_per_split) {
    if (!is_known(fmt) || !decode_sizes_ok(num_seqs, num_q_heads, num_kv_heads, max_seq_len)) return 0;
    const bool fp16 = is_fp16(fmt);
    if (pages_per_split < 0 || (pages_per_split % 2) || pages_per_split > max_pps(fp16)) return 0;
    const int32_t pps = pages_per_split ? pages_per_split
                                        : heuristic_pps(num_seqs, num_q_heads, num_kv_heads, max_seq_len, fmt->k_bits, fmt->v_bits,
                                                        is_pb(fmt));
    const WorkspaceLayout w = layout(num_seqs, num_q_heads, max_seq_len, pps);
    return w.splits > 65535 ? 0 : w.splits;
}

kvq_status kvq_decode_partials_slots(const kvq_format *fmt, const uint16_t *query, const uint8_t *cache,
                                     int64_t num_pages, const int32_t *block_tables, int32_t max_pages_per_seq,
                                     const int32_t *seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t max_seq_len, float softmax_scale,
                                     void *workspace, size_t workspace_bytes, int32_t pages_per_split,
                                     int32_t slot_offset, int32_t total_slots, int32_t rotated, void *stream) {
    if (!fmt) return KVQ_ERR_NULL;
    if (!is_known(fmt)) return KVQ_ERR_UNSUPPORTED;
    if (rotated != 0 && rotated != 1) return KVQ_ERR_SHAPE;
    if (is_quant(fmt) && !rotated) return KVQ_ERR_UNSUPPORTED;   // quantised-cache partials are always rotated
    if (total_slots <= 0 || total_slots > 65535 || slot_offset < 0) return KVQ_ERR_SHAPE;
    if (!decode_sizes_ok(num_seqs, num_q_heads, num_kv_heads, max_seq_len)) return KVQ_ERR_SHAPE;
    // the slotted workspace: [num_seqs][num_q_heads][total_slots] partials
    const size_t need = (size_t)num_seqs * num_q_heads * total_slots * kvq::kPartialFloats * sizeof(float);
    kvq::DecodeArgs a;
    kvq_status st = decode_common(fmt, seq_lens, num_seqs, num_q_heads, num_kv_heads, max_seq_len,
                                  max_pages_per_seq, workspace, (size_t)-1, pages_per_split, a);
    if (st == KVQ_OK) st = decode_inputs(query, cache, num_pages, block_tables, max_pages_per_seq, softmax_scale, a);
    if (st != KVQ_OK) return st;
    if (workspace_bytes < need) return KVQ_ERR_WORKSPACE;
    if ((int64_t)slot_offset + a.splits > total_slots) return KVQ_ERR_SHAPE;
    a.slot_offset = slot_offset;
    a.slot_stride = total_slots;
    a.partials_only = 1;
    a.rotate_partials = is_fp16(fmt) ? rotated : 0;
    return hip_status(launch_split(a, (hipStream_t)stream));
}

kvq_status kvq_decode_combine_slots(void *out, kvq_out_dtype out_dtype, int32_t num_seqs, int32_t num_q_heads,
                                    const void *workspace, size_t workspace_bytes, int32_t total_slots,
                                    int32_t rotated, void *stream) {
    if (rotated != 0 && rotated != 1) return KVQ_ERR_SHAPE;
    if (num_seqs <= 0 || num_q_heads <= 0 || total_slots <= 0 || total_slots > 65535) return KVQ_ERR_SHAPE;
    if (!workspace) return KVQ_ERR_WORKSPACE;
    const size_t need = (size_t)num_seqs * num_q_heads * total_slots * kvq::kPartialFloats * sizeof(float);
    if (workspace_bytes < need) return KVQ_ERR_WORKSPACE;
    if (!aligned16(workspace)) return KVQ_ERR_ALIGN;
    kvq::DecodeArgs a;
    memset(&a, 0, sizeof(a));
    kvq_status st = decode_output(out, out_dtype, a);
    if (st != KVQ_OK) return st;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.splits = total_slots;
    a.slot_stride = total_slots;
    a.rotated = rotated;
    a.partials_only = 1;
    a.partials = static_cast<float *>(const_cast<void *>(workspace));
    return hip_status(kvq::launch_decode_combine(a, (hipStream_t)stream));
}

kvq_status kvq_decode_combine(const kvq_format *fmt, void *out, kvq_out_dtype out_dtype,
                              const int32_t *seq_lens, int32_t num_seqs, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t max_seq_len, const void *workspace,
                              size_t workspace_bytes, int32_t pages_per_split, void *stream) {
    kvq::DecodeArgs a;
    kvq_status st = decode_common(fmt, seq_lens, num_seqs, num_q_heads, num_kv_heads, max_seq_len, -1,
                                  const_cast<void *>(workspace), workspace_bytes, pages_per_split, a);
    if (st == KVQ_OK) st = decode_output(out, out_dtype, a);
    if (st != KVQ_OK) return st;
    a.partials_only = 1;
    return hip_status(kvq::launch_decode_combine(a, (hipStream_t)stream));
}

size_t kvq_decode_workspace_bytes_mq(const kvq_format *fmt, int32_t num_seqs, int32_t q_len,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t max_seq_len,
                                     int32_t pages_per_split) {
    if (q_len < 1 || q_len > 16 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads)
        return 0;
    if ((int64_t)num_q_heads * q_len > 65535) return 0;
    return kvq_decode_workspace_bytes(fmt, num_seqs, num_q_heads * q_len, num_kv_heads, max_seq_len,
                                      pages_per_split);
}

kvq_status kvq_decode_attention_mq(const kvq_format *fmt, void *out, kvq_out_dtype out_dtype,
                                   const uint16_t *query, int32_t q_len, const uint8_t *cache, int64_t num_pages,
                                   const int32_t *block_tables, int32_t max_pages_per_seq,
                                   const int32_t *seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t max_seq_len, float softmax_scale,
                                   void *workspace, size_t workspace_bytes, int32_t pages_per_split,
                                   void *stream) {
    if (!fmt) return KVQ_ERR_NULL;
    if (!is_known(fmt)) return KVQ_ERR_UNSUPPORTED;
    if (q_len < 1 || q_len > 16 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads ||
        (int64_t)num_q_heads * q_len > 65535)
        return KVQ_ERR_SHAPE;
    // the fp16 baseline and page-balanced keys decode one row
    if (q_len > 1 && (!is_quant(fmt) || is_pb(fmt))) return KVQ_ERR_UNSUPPORTED;
    // (row, head) pairs take the place of query heads: q_len * num_q_heads of them
    kvq::DecodeArgs a;
    kvq_status st = decode_common(fmt, seq_lens, num_seqs, q_len * num_q_heads, num_kv_heads, max_seq_len,
                                  max_pages_per_seq, workspace, workspace_bytes, pages_per_split, a);
    if (st == KVQ_OK) st = decode_output(out, out_dtype, a);
    if (st == KVQ_OK) st = decode_inputs(query, cache, num_pages, block_tables, max_pages_per_seq, softmax_scale, a);
    if (st != KVQ_OK) return st;
    a.q_len = q_len;
    return hip_status(launch_both(a, (hipStream_t)stream));
}

kvq_status kvq_decode_attention(const kvq_format *fmt, void *out, kvq_out_dtype out_dtype,
                                const uint16_t *query, const uint8_t *cache, int64_t num_pages,
                                const int32_t *block_tables, int32_t max_pages_per_seq,
                                const int32_t *seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t max_seq_len, float softmax_scale,
                                void *workspace, size_t workspace_bytes, void *stream) {
    return kvq_decode_attention_ex(fmt, out, out_dtype, query, cache, num_pages, block_tables,
                                   max_pages_per_seq, seq_lens, num_seqs, num_q_heads, num_kv_heads,
                                   max_seq_len, softmax_scale, workspace, workspace_bytes, 0, stream);
}

kvq_status kvq_page_walk_probe(const kvq_format *fmt, const uint8_t *cache, int64_t num_pages,
                               const int32_t *block_tables, int32_t max_pages_per_seq, const int32_t *seq_lens,
                               int32_t num_seqs, int32_t num_kv_heads, int32_t max_seq_len,
                               int32_t pages_per_split, uint32_t *sink, void *stream) {
    if (!fmt) return KVQ_ERR_NULL;
    if (!is_quant(fmt) || fmt->block_size != 16) return KVQ_ERR_UNSUPPORTED;
    if (!cache || !block_tables || !seq_lens || !sink) return KVQ_ERR_NULL;
    if (num_pages <= 0 || num_seqs <= 0 || num_seqs > 65535 || num_kv_heads <= 0 || num_kv_heads > 65535 ||
        max_seq_len <= 0 || max_pages_per_seq <= 0 ||
        (int64_t)max_seq_len > (int64_t)max_pages_per_seq * fmt->block_size || pages_per_split < 2 ||
        (pages_per_split % 2) || pages_per_split > kvq::kMaxPagesPerSplit)
        return KVQ_ERR_SHAPE;
    if (!aligned16(cache) || ((uintptr_t)block_tables & 3u) || ((uintptr_t)seq_lens & 3u) ||
        ((uintptr_t)sink & 3u))
        return KVQ_ERR_ALIGN;
    const int64_t splits = ceil_div(ceil_div(max_seq_len, kvq::kPage), pages_per_split);
    if (splits > 65535) return KVQ_ERR_SHAPE;
    kvq::PageWalkArgs a;
    a.cache = cache;
    a.num_pages = num_pages;
    a.region16 = (int32_t)(region_bytes(fmt) / 16);
    a.num_kv_heads = num_kv_heads;
    a.block_tables = block_tables;
    a.bt_stride = max_pages_per_seq;
    a.seq_lens = seq_lens;
    a.max_seq_len = max_seq_len;
    a.pages_per_split = pages_per_split;
    a.sink = sink;
    return hip_status(kvq::launch_page_walk(a, (int32_t)splits, num_seqs, (hipStream_t)stream));
}

kvq_status kvq_stream_read_probe(const void *buffer, size_t bytes, uint32_t *sink, void *stream) {
    if (!buffer || !sink) return KVQ_ERR_NULL;
    if (bytes == 0 || (bytes % 16) || bytes > ((size_t)1 << 40)) return KVQ_ERR_SHAPE;
    if (!aligned16(buffer) || ((uintptr_t)sink & 3u)) return KVQ_ERR_ALIGN;
    return hip_status(kvq::launch_stream_read(buffer, (int64_t)bytes, sink, (hipStream_t)stream));
}

kvq_status kvq_set_split_kernel_events(void *start_event, void *stop_event) {
    g_split_events.start = static_cast<hipEvent_t>(start_event);
    g_split_events.stop = static_cast<hipEvent_t>(stop_event);
    return KVQ_OK;
}

const char *kvq_status_string(kvq_status status) {
    switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_NULL: return "null pointer";
    case KVQ_ERR_SHAPE: return "invalid size or shape";
    case KVQ_ERR_UNSUPPORTED: return "unsupported format";
    case KVQ_ERR_ALIGN: return "misaligned pointer or stride";
    case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
    case KVQ_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

int kvq_last_hip_error(void) { return g_last_hip_error; }

const char *kvq_version(void) { return "kvq 1.0 (kvq-k4v2-g128 v1, gfx950)"; }

}  // extern "C"

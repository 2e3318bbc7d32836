// Uncompressed fp16 paged cache: the baseline the K4V2 format is measured
// against.  The pages compare KVarN's packed cache with fp16 on accuracy,
// capacity and throughput (beyondheadline.xyz, "Huawei's KV-cache trick",
// lede; dothoosh.com, "KVarN vs TurboQuant", results paragraph); decode over
// either cache streams every cached byte through HBM once per token
// (encorp.ai, "KV cache compression is an infrastructure decision, not a model
// debate", section on the HBM ceiling), so this cache moves 512 bytes per token
// per KV head where K4V2 moves 104.
//
// Region of one (page, KV head), 8192 bytes, laid out so that every lane's
// MFMA fragments are 64 contiguous bytes:
//   keys   [0, 4096):    token n, channel c = 32d + 8g + e at element
//                        n*128 + 32g + 8d + e     (lane (n, g) reads 64 B)
//   values [4096, 8192): token t (quad q = t/4, i = t%4), channel c = 16j + m
//                        at element ((16q + m)*8 + j)*4 + i  (lane (m, g = q))
//
// Decode uses the K4V2 kernel's work decomposition (split-K, 4 waves, page ids
// in lanes, triple-buffered prefetch, lazy base-2 softmax, wave merge) with
// single pages as the unit: scores are v_mfma_f32_16x16x32_f16 of the fp16
// keys with the fp16 query (its products are exact, so one term suffices;
// columns 8-15 repeat heads 0-7 so that both lanes of a column pair hold the
// same scores), and P.V is v_mfma_f32_16x16x16_f16 of the values with the
// weights split into fp16 and residual columns, as in the K4V2 kernel.
#include <hip/hip_ext.h>

#include <atomic>
#include <math.h>

#include "kvq_decode_common.h"
#include "kvq_device.h"

namespace kvq {
namespace {

typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Append: one thread per 8 channels of one (token, KV head, key|value) row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fp16_append_kernel(AppendArgs a) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t rows = a.num_tokens * a.num_kv_heads;
    if (gid >= rows * 32) return;
    const int chunk = (int)(gid & 15);               // 8-channel chunk k: channels 8k .. 8k+7
    const int is_v = (int)((gid >> 4) & 1);
    const int64_t rowi = gid >> 5;
    const int64_t tok = rowi / a.num_kv_heads;
    const int head = (int)(rowi % a.num_kv_heads);
    const int64_t slot = a.slots[tok];
    if (slot < 0) return;
    const int64_t page = slot / kPage;
    const int off = (int)(slot % kPage);
    if (page >= a.num_pages) return;
    const uint16_t *src = is_v ? a.value + tok * a.value_stride + (int64_t)head * kHeadDim
                               : a.key + tok * a.key_stride + (int64_t)head * kHeadDim;
    const uint4 raw = *reinterpret_cast<const uint4 *>(src + 8 * chunk);
    uint16_t *region = reinterpret_cast<uint16_t *>(a.cache + (page * a.num_kv_heads + head) * (int64_t)kRegionF16);
    if (!is_v) {
        const int d = chunk >> 2, g = chunk & 3;      // c = 32d + 8g + e
        *reinterpret_cast<uint4 *>(region + off * 128 + 32 * g + 8 * d) = raw;
    } else {
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
        const int q = off >> 2, i = off & 3, j = chunk >> 1;
        uint16_t *vb = region + kVCodesF16 / 2;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const int m = 8 * (chunk & 1) + e;        // c = 16j + m
            vb[((16 * q + m) * 8 + j) * 4 + i] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        }
    }
}

// ---------------------------------------------------------------------------
// Decode split kernel.
// ---------------------------------------------------------------------------
struct Page16 {
    uint4 k[4];   // keys: token (lane & 15), channels 32d + 8g .. +7 in k[d]
    uint4 v[4];   // values: channel 16j + (lane & 15), tokens 4g .. 4g+3 of block j in v[j/2]
};

__device__ __forceinline__ void load_page16(const uint8_t *region, uint32_t koff, uint32_t voff, Page16 &r) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(region), (short)0, kRegionF16, 0x00020000);
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const v4u k = __builtin_amdgcn_raw_buffer_load_b128(rs, koff + 16 * q, 0, 0);
        const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16 * q, 0, 0);
        r.k[q] = make_uint4(k.x, k.y, k.z, k.w);
        r.v[q] = make_uint4(v.x, v.y, v.z, v.w);
    }
}

// One page.  kMasked: tokens at or beyond n_tokens (the page starts at token
// tok0) take no weight, and their values are read as zero (an unwritten slot
// may hold any bits, and NaN times a zero weight would poison the sums).
// kFirst: the wave's first page, which sets the running maximum.  Scores are
// formed relative to the reference mref = m + 8, as in the K4V2 kernel.
template <bool kMasked, bool kFirst>
__device__ __forceinline__ void process_page16(const Page16 &P, int tok0, int n_tokens, const v8h (&bq)[4],
                                               float c1, float res_k, int g, State &st) {
    const float mref = kFirst ? 0.0f : st.m + kLazyThreshold;
    v4f d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int q = 0; q < 4; q++) d = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, P.k[q]), bq[q], d, 0, 0, 0);
    float lg[4];
    bool valid[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        lg[i] = __builtin_fmaf(d[i], c1, -mref);
        valid[i] = !kMasked || tok0 + 4 * g + i < n_tokens;
        if (kMasked) lg[i] = valid[i] ? lg[i] : -INFINITY;
    }
    const float lmax = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
    if (kFirst || __any(lmax > 0.0f)) {
        float cm = fmaxf(lmax, xor_lane(lmax, 16));
        cm = fmaxf(cm, xor_lane(cm, 32));
        const float m_new = kFirst ? cm : fmaxf(st.m, cm + mref);
        const float f = kFirst ? 0.0f : fast_exp2(st.m - m_new);
        st.l *= f;
#pragma unroll
        for (int j = 0; j < 8; j++) st.acc[j] *= f;
        st.m = m_new;
        const float shift = (m_new + kLazyThreshold) - mref;
#pragma unroll
        for (int i = 0; i < 4; i++) lg[i] -= shift;
    }
    v4h bw;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const float p = fast_exp2(lg[i]);    // exp2(-inf) = 0 for masked tokens
        st.l += p;
        // columns n < 8 take fp16(p), columns n >= 8 the residual p - fp16(p)
        const _Float16 hi = (_Float16)p;
        bw[i] = (_Float16)fmaf((float)hi, res_k, p);
    }
    uint32_t vmask0 = 0xffffffffu, vmask1 = 0xffffffffu;   // tokens 4g+0,1 and 4g+2,3
    if (kMasked) {
        vmask0 = (valid[0] ? 0x0000ffffu : 0u) | (valid[1] ? 0xffff0000u : 0u);
        vmask1 = (valid[2] ? 0x0000ffffu : 0u) | (valid[3] ? 0xffff0000u : 0u);
    }
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const uint4 &v = P.v[j >> 1];
        uint2 u = (j & 1) ? make_uint2(v.z, v.w) : make_uint2(v.x, v.y);
        if (kMasked) {
            u.x &= vmask0;
            u.y &= vmask1;
        }
        st.acc[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(v4h, u), bw, st.acc[j], 0, 0, 0);
    }
}

__global__ __launch_bounds__(256) void decode_fp16_kernel(DecodeArgs a) {
    const int split = blockIdx.x;
    const int kvh = blockIdx.y / a.head_groups;
    const int hg = blockIdx.y % a.head_groups;
    const int b = blockIdx.z;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // Page ids of this wave's pages, one per lane: lane j holds page
    // k = wave + 4j of the split (at most 256 pages per split: j < 64).
    const int32_t *bt = a.block_tables + (int64_t)b * a.bt_stride;
    int32_t bt_p;
    {
        const int last = a.bt_stride - 1;
        const int p = split * a.pages_per_split + wave + kWaves * lane;
        bt_p = bt[p < last ? p : last];
    }

    const int max_len = a.max_seq_len;
    int n_tokens = a.seq_lens[b];
    n_tokens = n_tokens < 0 ? 0 : (n_tokens > max_len ? max_len : n_tokens);
    const int npages = (n_tokens + kPage - 1) / kPage;
    const int pps = a.pages_per_split;
    const int p_begin = split * pps;
    const int hq0 = kvh * a.gqa + hg * kHeadsPerGroup;
    const int nh = min(kHeadsPerGroup, a.gqa - hg * kHeadsPerGroup);
    if (p_begin >= npages) {         // an empty sequence, or a split past its end
        write_empty(a, tid, b, kvh, hg * kHeadsPerGroup, nh, split);
        return;
    }
    const int p_end = min(p_begin + pps, npages);

    __shared__ _Float16 s_q[kHeadsPerGroup][kHeadDim];
    __shared__ MergeLds s_merge;

    const int64_t head_off = (int64_t)kvh * kRegionF16;
    const int64_t page_stride = (int64_t)a.num_kv_heads * kRegionF16;
    const uint32_t num_pages32 = a.num_pages < 0x7fffffff ? (uint32_t)a.num_pages : 0x7fffffffu;
    auto region_of = [&](int32_t page_id) -> const uint8_t * {
        uint32_t id = (uint32_t)page_id;
        if (id >= num_pages32) id = 0;           // a page id outside the pool is read as page 0
        return a.cache + (int64_t)id * page_stride + head_off;
    };
    const uint32_t koff = (uint32_t)((lane & 15) * 256 + (lane >> 4) * 64);
    const uint32_t voff = (uint32_t)(kVCodesF16 + ((lane >> 4) * 16 + (lane & 15)) * 64);

    // Pages of the split: all but possibly the sequence's last are full.  Wave
    // w takes pages w, w + 4, ...; full pages run through a triple-buffered
    // loop (loads always issued; past the end they repeat the wave's last
    // page); a partial last page is processed afterwards with masking.
    const int np = p_end - p_begin;
    const bool last_partial = p_end == npages && (n_tokens % kPage) != 0;
    const int nfull = np - (last_partial ? 1 : 0);
    const int nk = nfull > wave ? (nfull - wave + kWaves - 1) / kWaves : 0;
    auto issue = [&](Page16 &A, int i) {
        const int j = i < nk ? i : nk - 1;
        load_page16(region_of(__builtin_amdgcn_readlane(bt_p, j)), koff, voff, A);
        __builtin_amdgcn_sched_barrier(0);
    };
    // The query slice is requested before any page: loads return in issue
    // order, so a later query load would wait for the first pages.
    const int hh_q = 2 * wave + (lane >> 5);
    const int c0_q = 4 * (lane & 31);
    uint2 qraw = make_uint2(0, 0);
    if (hh_q < nh)
        qraw = *reinterpret_cast<const uint2 *>(a.query + ((int64_t)b * a.num_q_heads + hq0 + hh_q) * kHeadDim + c0_q);
    asm volatile("" ::"v"(bt_p));
    Page16 r0, r1, r2;
    if (nk > 0) {
        issue(r0, 0);
        issue(r1, 1);
    }

    // ---- query: wave w copies heads 2w and 2w + 1 to LDS (zero past nh) ----
    *reinterpret_cast<uint2 *>(&s_q[hh_q][c0_q]) = qraw;
    __syncthreads();
    const int n16 = lane & 15;
    const int g = lane >> 4;
    v8h bq[4];
#pragma unroll
    for (int q = 0; q < 4; q++) bq[q] = *reinterpret_cast<const v8h *>(&s_q[n16 & 7][32 * q + 8 * g]);
    const float c1 = a.alpha;                 // softmax_scale * log2(e)
    const float res_k = n16 < 8 ? 0.0f : -1.0f;

    State st;
    st.m = -INFINITY;
    st.l = 0.0f;
    st.z = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; j++) st.acc[j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    if (nk > 0) {
        issue(r2, 2);
        process_page16<false, true>(r0, 0, 0, bq, c1, res_k, g, st);
        if (nk > 1) {
            for (int i = 1;; i += 3) {
                issue(r0, i + 2);
                process_page16<false, false>(r1, 0, 0, bq, c1, res_k, g, st);
                if (i + 1 >= nk) break;
                issue(r1, i + 3);
                process_page16<false, false>(r2, 0, 0, bq, c1, res_k, g, st);
                if (i + 2 >= nk) break;
                issue(r2, i + 4);
                process_page16<false, false>(r0, 0, 0, bq, c1, res_k, g, st);
                if (i + 3 >= nk) break;
            }
        }
    }
    if (last_partial && wave == nfull % kWaves) {
        Page16 t;
        const int j = nfull / kWaves;             // this wave's slot of page nfull
        load_page16(region_of(__builtin_amdgcn_readlane(bt_p, j)), koff, voff, t);
        const int tok0 = (p_begin + nfull) * kPage;
        if (nk == 0)
            process_page16<true, true>(t, tok0, n_tokens, bq, c1, res_k, g, st);
        else
            process_page16<true, false>(t, tok0, n_tokens, bq, c1, res_k, g, st);
    }

    merge_and_store(st, s_merge, a, 0, [](int) { return 1.0f; }, wave, tid, b, kvh, hg * kHeadsPerGroup, nh, split, a.rotate_partials);
}

}  // namespace

int decode_fp16_resident_workgroups() {
    // one entry per device; several host threads may fill an entry at once,
    // and they all store the same value
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 512;
    }
    const int known = cached[dev].load(std::memory_order_relaxed);
    if (known > 0) return known;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_fp16_kernel, 256, 0) != hipSuccess ||
        cus <= 0 || per_cu <= 0) {
        (void)hipGetLastError();
        return 512;
    }
    cached[dev].store(cus * per_cu, std::memory_order_relaxed);
    return cus * per_cu;
}

hipError_t launch_fp16_append(const AppendArgs &a, hipStream_t stream) {
    const int64_t threads = a.num_tokens * a.num_kv_heads * 32;
    const int64_t blocks = (threads + 255) / 256;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fp16_append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_fp16_decode_split(const DecodeArgs &a, hipStream_t stream, const LaunchEvents &ev) {
    const dim3 grid((unsigned)a.splits, (unsigned)(a.num_kv_heads * a.head_groups), (unsigned)a.num_seqs);
    if (ev.start || ev.stop)
        hipExtLaunchKernelGGL(decode_fp16_kernel, grid, dim3(256), 0, stream, ev.start, ev.stop, 0, a);
    else
        hipLaunchKernelGGL(decode_fp16_kernel, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kvq

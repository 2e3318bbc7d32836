// Quantise-on-write of new key/value tokens into the g128 paged cache (4/8-bit
// keys with 2/4-bit values, or 3 bits both; the KVarN preset is 4-bit keys
// and 2-bit values): Hadamard rotation, variance normalisation, asymmetric
// round-to-nearest (dothoosh.com, "KVarN vs TurboQuant: 5x more context with
// higher accuracy", pipeline list stages 1-3).
//
// Three kernels encode the same bytes:
//   quantize_append_kernel   one 16-lane row per group = (token, KV head,
//                            key|value), via encode_group (kvq_quant.h); low
//                            latency for a handful of tokens;
//   quantize_append_staged   one lane per group (encode_row), the rows staged
//                            in LDS by coalesced direct-to-LDS loads while the
//                            previous batch is encoded; bulk appends with a
//                            power-of-two number of KV heads;
//   quantize_append_lanes    one lane per group, each lane loading its own
//                            row; bulk appends otherwise.
// All follow the format's definition operation for operation (fp32, no
// contraction, round-to-nearest-even, denormals kept), so their codes and
// metadata are bit-identical.  The bulk kernels are bound by the vector ALU
// (about 2100 instructions per group, 896 of them the FWHT's butterflies), so
// the one-lane-per-group encoder is written for the fewest instructions that
// keep every rounding of the definition.
#pragma clang fp contract(off)

#include <atomic>

#include "kvq_quant.h"

namespace kvq {
namespace {

constexpr int kRowsPerBlock = 16;   // 256 threads, 16 groups
// (token, KV head) rows from which the one-lane-per-group kernel is used: a
// wave per SIMD (1024 SIMDs x 64 lanes) and more
constexpr int64_t kLaneKernelMinRows = 65536;

template <int KB, int VB>
__global__ __launch_bounds__(256) void quantize_append_kernel(AppendArgs a) {
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;                                  // lane within the row
    const int64_t group = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 4);
    const int64_t total = a.num_tokens * a.num_kv_heads * 2;
    if (group >= total) return;                               // row-uniform
    const int is_v = (int)(group & 1);
    const int64_t th = group >> 1;
    const int head = (int)(th % a.num_kv_heads);
    const int64_t tok = th / a.num_kv_heads;

    const int64_t slot = a.slots[tok];
    if (slot < 0) return;
    const int64_t page = slot >> (4 + a.page_log2s);                 // slot = page * page_tokens + t
    const int t = (int)(slot & ((16 << a.page_log2s) - 1));
    if (page >= a.num_pages) return;

    const uint16_t *src = is_v ? a.value + tok * a.value_stride + (int64_t)head * kHeadDim
                               : a.key + tok * a.key_stride + (int64_t)head * kHeadDim;
    // region t / 16 of the (page, head) run
    uint8_t *region = a.cache + (((page * a.num_kv_heads + head) << a.page_log2s) + (t >> 4)) *
                                    (int64_t)Layout<KB, VB>::kBytes;
    encode_group_fmt<KB, VB>(src, is_v, r, region, t & 15);
}

// Groups per lane-kernel work-group: waves 0 and 1 encode the keys of 128
// consecutive (token, KV head) rows, waves 2 and 3 their values.
constexpr int kLaneRows = 128;

// Stage h = 1 of the FWHT straight from one dword of two fp16 inputs (lo =
// channel 2e, hi = channel 2e + 1): v_fma_mix_f32 computes fma(lo, 1.0, +-hi)
// on the fp16 halves with one fp32 rounding of the exact result, which is
// fp32(lo) +- fp32(hi) since both conversions to fp32 are exact -- the stage's
// a + b and a - b, without the two conversions.  (Checked on the device
// against fp32 a + b and a - b for every finite fp16 a against 40 b patterns
// including subnormals and the extremes: no differences.)
__device__ __forceinline__ void fwht_pair_f16(uint32_t w, float &sum, float &diff) {
    asm("v_fma_mix_f32 %0, %1, 1.0, %1 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "=v"(sum) : "v"(w));
    asm("v_fma_mix_f32 %0, %1, 1.0, -%1 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "=v"(diff) : "v"(w));
}

// A code is rint(t) for 0 <= t <= L (t = (yh - m) * inv never exceeds L: the
// product of the rounded range and its rounded reciprocal stays within two
// ulps of L, so the clamp of the definition never acts).  Adding 2^23 rounds t
// to an integer with ties to even -- rint's rounding -- and leaves the bit
// pattern 0x4B000000 + code, so a code is one add, and packing shifts and adds
// those patterns; the sum of the shifted 0x4B000000 terms is subtracted once
// per word (all modulo 2^32).
constexpr uint32_t kRoundBits = 0x4B000000u;    // bit pattern of 2^23
__device__ __forceinline__ uint32_t code_bits(float t) { return __builtin_bit_cast(uint32_t, t + 0x1p23f); }
__device__ __forceinline__ constexpr uint32_t round_bits_sum(int n, int step) {
    uint32_t s = 0;
    for (int k = 0; k < n; k++) s += kRoundBits << (step * k);
    return s;
}

// One group per lane: encode the 128 fp16 values of a row (chunk(c) returns
// its 16-byte chunk c, channels 8c..8c+7) and store token slot `off` of
// `region` (KB-bit key / VB-bit value layout).  kValue selects the value
// encoding.  Each chunk is converted as it is fetched, so that the raw
// halves and the 128 fp32 values are not all live at once.
//   after_fetch() runs once every chunk has been fetched (the staged kernel
// starts its next batch's loads there).
template <int KB, int VB, bool kValue, typename Chunk, typename AfterFetch>
__device__ __forceinline__ void encode_row(const Chunk &chunk, const AfterFetch &after_fetch, uint8_t *region,
                                           int off, bool store = true) {
    using Lay = Layout<KB, VB>;
    float y[kHeadDim];
    // 1. Hadamard rotation, butterfly stages h = 1, 2, ..., 64; stage 1 from
    // the fp16 pairs as they are fetched (fwht_pair_f16)
#pragma unroll
    for (int c = 0; c < kHeadDim / 8; c++) {
        const uint4 raw = chunk(c);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 4; e++) fwht_pair_f16(w[e], y[8 * c + 2 * e], y[8 * c + 2 * e + 1]);
    }
    after_fetch();
#pragma unroll
    for (int h = 2; h < kHeadDim; h <<= 1) {
#pragma unroll
        for (int i = 0; i < kHeadDim; i++) {
            if ((i & h) == 0) {
                const float p = y[i], q = y[i + h];
                y[i] = p + q;
                y[i + h] = p - q;
            }
        }
    }
    // 2. variance normalisation: squares, then the tree h = 64, 32, ..., 1
    float ss;
    {
        float p[kHeadDim / 2];
#pragma unroll
        for (int i = 0; i < kHeadDim / 2; i++) {
            const float a0 = y[i] * y[i];
            const float a1 = y[i + kHeadDim / 2] * y[i + kHeadDim / 2];
            p[i] = a0 + a1;
        }
#pragma unroll
        for (int h = kHeadDim / 4; h >= 1; h >>= 1) {
#pragma unroll
            for (int i = 0; i < h; i++) p[i] = p[i] + p[i + h];
        }
        ss = p[0];
    }
    constexpr int L = kValue ? Lay::kVL : Lay::kKL;
    // keys: the token's code row as dwords (16 of nibbles, 32 of bytes, or
    // 12 bit-plane words); values: the 16-bit words of the layout (16 of
    // crumbs or 32 of nibbles), or 48 bit-plane bytes (3 per m)
    constexpr int kWords = kValue ? (VB == 2 ? 16 : VB == 3 ? 48 : 32) : (KB == 4 ? 16 : KB == 3 ? 12 : 32);
    uint32_t packed[kWords];
#pragma unroll
    for (int d = 0; d < kWords; d++) packed[d] = 0;
    float sm = 0.0f, zm = 0.0f;
    if (ss != 0.0f) {
        const float sigma = sqrtf(ss * 0x1p-7f);
        const float rcp = 1.0f / sigma;
        float lo = y[0] * rcp, hi = lo;
#pragma unroll
        for (int i = 0; i < kHeadDim; i++) {
            y[i] = y[i] * rcp;
            lo = fminf(lo, y[i]);
            hi = fmaxf(hi, y[i]);
        }
        // 3. asymmetric round-to-nearest (ties to even) in [0, L]
        float delta = 0.0f;
        uint32_t csum = 0;
        if (hi != lo) {
            const float range = hi - lo;
            delta = range / (float)L;
            const float inv = (float)L / range;
#pragma unroll
            for (int i = 0; i < kHeadDim; i++) {
                const uint32_t cb = code_bits((y[i] - lo) * inv);     // 0x4B000000 + code
                if (kValue) {
                    csum += cb;
                    if (VB == 2) {
                        packed[i & 15] += cb << (2 * (i >> 4));        // word m: channel 16j + m at bits 2j
                    } else if (VB == 3) {
                        // byte 3m + p: bit p of channel 16j + m's code at bit j
#pragma unroll
                        for (int p = 0; p < 3; p++) packed[3 * (i & 15) + p] |= ((cb >> p) & 1u) << (i >> 4);
                    } else {   // word 2m + h: channel 16(4h + k) + m at bits 4k
                        packed[2 * (i & 15) + (i >> 6)] += cb << (4 * ((i >> 4) & 3));
                    }
                } else if (KB == 3) {
                    // plane word 3G + p (G = i / 32): bit p of the code at bit i % 32
#pragma unroll
                    for (int p = 0; p < 3; p++) packed[3 * (i >> 5) + p] |= ((cb >> p) & 1u) << (i & 31);
                } else if (KB == 4) {
                    packed[i >> 3] += cb << (4 * (i & 7));         // byte b = c[2b] | c[2b+1] << 4
                } else {
                    packed[i >> 2] += cb << (8 * (i & 3));         // byte c = c[c]
                }
            }
            // remove the 0x4B000000 of every code
            constexpr uint32_t kCorr = kValue ? (VB == 2 ? round_bits_sum(8, 2) : VB == 4 ? round_bits_sum(4, 4) : 0u)
                                              : (KB == 4 ? round_bits_sum(8, 4) : KB == 8 ? round_bits_sum(4, 8) : 0u);
            if (kCorr != 0u) {
#pragma unroll
                for (int d = 0; d < kWords; d++) packed[d] -= kCorr;
            }
            csum -= kRoundBits * (uint32_t)kHeadDim;
        }
        sm = delta * sigma;
        if (!kValue) {
            zm = lo * sigma;
        } else {
            float t = delta * (float)csum;
            t = t * 0x1p-7f;
            t = lo + t;
            zm = t * sigma;
        }
    }
    const uint32_t s16 = float_to_half_bits(materialize(sm));
    uint32_t z16 = float_to_half_bits(materialize(zm));
    if (z16 == 0x8000u) z16 = 0;         // a zero offset is stored as +0
    if (!store) return;
    if (!kValue) {
        uint4 *dst = reinterpret_cast<uint4 *>(region + Lay::kKCodes + 16 * KB * off);
#pragma unroll
        for (int q = 0; q < kWords / 4; q++)
            dst[q] = make_uint4(packed[4 * q], packed[4 * q + 1], packed[4 * q + 2], packed[4 * q + 3]);
        *reinterpret_cast<uint32_t *>(region + Lay::kKMeta + 4 * off) = s16 | (z16 << 16);
    } else if (VB == 3) {
        // byte (0, 2, 1, 3)[i] of plane word p at 12 (16g + m) + 4p
        const int i = off & 3;
        uint8_t *vb = region + Lay::kVCodes + 192 * (off >> 2) + (((i & 1) << 1) | (i >> 1));
#pragma unroll
        for (int m = 0; m < 16; m++)
#pragma unroll
            for (int p = 0; p < 3; p++) vb[12 * m + 4 * p] = (uint8_t)packed[3 * m + p];
        *reinterpret_cast<uint32_t *>(region + Lay::kVMeta + 4 * off) = s16 | (z16 << 16);
    } else if (VB == 2) {
        uint8_t *vb = region + Lay::kVCodes + 128 * (off >> 2) + 2 * (off & 3);
#pragma unroll
        for (int m = 0; m < 16; m++) *reinterpret_cast<uint16_t *>(vb + 8 * m) = (uint16_t)packed[m];
        *reinterpret_cast<uint32_t *>(region + Lay::kVMeta + 4 * off) = s16 | (z16 << 16);
    } else {
        const int i = off & 3;
        uint8_t *vb = region + Lay::kVCodes + 256 * (off >> 2) + 8 * (i >> 1) + 2 * (i & 1);
#pragma unroll
        for (int m = 0; m < 16; m++) {
            *reinterpret_cast<uint16_t *>(vb + 16 * m) = (uint16_t)packed[2 * m];
            *reinterpret_cast<uint16_t *>(vb + 16 * m + 4) = (uint16_t)packed[2 * m + 1];
        }
        *reinterpret_cast<uint32_t *>(region + Lay::kVMeta + 4 * off) = s16 | (z16 << 16);
    }
}

// The 16-token region holding slot `slot`, or nullptr for a skipped slot.
template <int KB, int VB>
__device__ __forceinline__ uint8_t *slot_region(const AppendArgs &a, int64_t slot, int head, int &off) {
    if (slot < 0) return nullptr;
    const int64_t page = slot >> (4 + a.page_log2s);
    const int t = (int)(slot & ((16 << a.page_log2s) - 1));
    if (page >= a.num_pages) return nullptr;
    off = t & 15;
    return a.cache + (((page * a.num_kv_heads + head) << a.page_log2s) + (t >> 4)) * (int64_t)Layout<KB, VB>::kBytes;
}

// Bulk append for any number of KV heads: each lane loads its own row.
template <int KB, int VB>
__global__ __launch_bounds__(256) void quantize_append_lanes(AppendArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int64_t rowi = (int64_t)blockIdx.x * kLaneRows + (wave & 1) * 64 + lane;
    if (rowi >= a.num_tokens * a.num_kv_heads) return;
    const int64_t tok = rowi / a.num_kv_heads;
    const int head = (int)(rowi % a.num_kv_heads);
    int off = 0;
    uint8_t *region = slot_region<KB, VB>(a, a.slots[tok], head, off);
    if (!region) return;
    if (wave >> 1) {
        const uint4 *src = reinterpret_cast<const uint4 *>(a.value + tok * a.value_stride + (int64_t)head * kHeadDim);
        encode_row<KB, VB, true>([&](int c) { return src[c]; }, [] {}, region, off);
    } else {
        const uint4 *src = reinterpret_cast<const uint4 *>(a.key + tok * a.key_stride + (int64_t)head * kHeadDim);
        encode_row<KB, VB, false>([&](int c) { return src[c]; }, [] {}, region, off);
    }
}

// Bulk append with coalesced loads staged in LDS, for a power-of-two number
// of KV heads.  A work-group takes batches of 128 consecutive (token, KV head)
// rows (grid-stride): waves 0 and 1 encode the keys of rows 0-63 and 64-127,
// waves 2 and 3 their values.  Each wave owns a 16 KB LDS tile of its 64
// rows.  The rows arrive by direct-to-LDS buffer loads (no registers hold
// loads in flight): load j brings rows 4j..4j+3, each a contiguous 256 bytes,
// so every load reads whole rows (not one 16-byte piece of each of 64 rows,
// as lane-per-row loads do).  Row r's chunk c is stored at slot c ^ (r & 15)
// of the row, so that when lane r reads its row back (chunk c from slot c ^
// (r & 15)), 16 consecutive lanes hit 16 different bank groups.  The next
// batch's loads are issued as soon as the tile has been read and run while
// the current batch is encoded.
//
// Addresses: the batch's 64 rows start at row R0 (a multiple of 64, hence of
// the head count when that is at most 64, and of 64 heads otherwise), so load
// j of lane (rho0 = lane / 16, kappa = lane % 16) reads row R0 + 4j + rho0 at
// byte offset U_j + V_(j % 4) from row R0: U_j is wave-uniform (the scalar
// offset) and V_q = lane_base + 16 (kappa ^ (4q + rho0)) one of four per-lane
// values.  The buffer resource ends with the last row of the input, so rows
// past it read as zeros (and are not stored).
constexpr int kStagedRows = 128;

// The batch loop of one wave: keys (kValue = false) or values.
template <int KB, int VB, bool kValue>
__device__ __forceinline__ void staged_rows(const AppendArgs &a, int64_t nbatch, uint4 *tile, int lane,
                                            int64_t half0) {
    const int hs = __builtin_ctz((unsigned)a.num_kv_heads);          // power of two
    const int hmask = a.num_kv_heads - 1;
    const int64_t rows = a.num_tokens << hs;
    const uint16_t *src = kValue ? a.value : a.key;
    const int64_t stride = kValue ? a.value_stride : a.key_stride;   // elements
    const uint32_t sb = (uint32_t)(stride * 2);                       // bytes per token (checked by the launcher)
    // one past the last row's bytes
    const int64_t end_bytes = ((a.num_tokens - 1) * stride + (int64_t)a.num_kv_heads * kHeadDim) * 2;
    const int rho0 = lane >> 4, kappa = lane & 15;
    const uint32_t lane_base = hs >= 2 ? (uint32_t)rho0 * 256u
                                       : (uint32_t)(rho0 >> hs) * sb + (uint32_t)(rho0 & hmask) * 256u;
    uint32_t vq[4];
#pragma unroll
    for (int q = 0; q < 4; q++) vq[q] = lane_base + 16u * (uint32_t)(kappa ^ (4 * q + rho0));
    // token and head steps of load j: rows 4j + rho0 lie (4j) >> hs tokens
    // after row R0 (heads below 4 per token) or in token (4j) >> hs, head (4j) &
    // hmask + rho0 (4 heads or more)
    const int ts = hs >= 2 ? (hs - 2 < 4 ? hs - 2 : 4) : 0;

    // live = false: a resource of no bytes, every load out of range (the
    // loads past the last batch stay in the instruction stream, so the loop
    // has one path)
    auto issue = [&](int64_t g, bool live) {
        const int64_t r0 = g * kStagedRows + half0;
        const int64_t base = ((r0 >> hs) * stride + (r0 & hmask) * kHeadDim) * 2;     // bytes
        const int64_t left = end_bytes - base;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t *>(reinterpret_cast<const uint8_t *>(src) + base), (short)0,
            live ? (left < 0x7fffffff ? (int)left : 0x7fffffff) : 0, 0x00020000);
#pragma unroll
        for (int j = 0; j < 16; j++) {
            const uint32_t u = hs >= 2 ? (uint32_t)(j >> ts) * sb + (uint32_t)(j & ((1 << ts) - 1)) * 1024u
                                       : (uint32_t)((4 * j) >> hs) * sb;
            // the whole offset in the per-lane operand: the range check covers it
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, tile + 64 * j, 16, vq[j & 3] + u, 0, 0, 0);
        }
    };

    int64_t g = blockIdx.x;
    issue(g, true);
#pragma clang loop unroll(disable)
    for (;;) {
        const int64_t row = g * kStagedRows + half0 + lane;
        const bool live = row < rows;
        const int64_t tok = (live ? row : rows - 1) >> hs;
        const int head = (int)(row & hmask);
        const int64_t slot = a.slots[tok];
        const int64_t gn = g + gridDim.x;
        // the tile's loads (and the slot) have landed
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        int off = 0;
        uint8_t *region = live ? slot_region<KB, VB>(a, slot, head, off) : nullptr;
        // the row's 16 chunks, all requested at once (one LDS round trip)
        const int sw = lane & 15;
        uint4 raw[kHeadDim / 8];
#pragma unroll
        for (int c = 0; c < kHeadDim / 8; c++) raw[c] = tile[16 * lane + (c ^ sw)];
        // every lane has read its row before the next batch overwrites the tile
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        issue(gn < nbatch ? gn : g, gn < nbatch);
        encode_row<KB, VB, kValue>([&](int c) { return raw[c]; }, [] {}, region ? region : a.cache, off,
                                   region != nullptr);
        if (gn >= nbatch) break;
        g = gn;
    }
    // the empty loads of the last issue have completed before the wave ends
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int KB, int VB>
__global__ __launch_bounds__(256, 2) void quantize_append_staged(AppendArgs a, int64_t nbatch) {
    __shared__ uint4 s_tile[4][64 * 16];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if ((int64_t)blockIdx.x >= nbatch) return;
    const int lane = threadIdx.x & 63;
    const int64_t half0 = (int64_t)(wave & 1) * 64;
    if (wave >> 1)
        staged_rows<KB, VB, true>(a, nbatch, s_tile[wave], lane, half0);
    else
        staged_rows<KB, VB, false>(a, nbatch, s_tile[wave], lane, half0);
}

// Work-groups of quantize_append_staged<KB, VB> the current device holds at
// once (compute units x occupancy), queried once per device; 512 without one.
template <int KB, int VB>
int64_t staged_resident_workgroups() {
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
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, quantize_append_staged<KB, VB>, 256, 0) != hipSuccess ||
        cus <= 0 || per_cu <= 0) {
        (void)hipGetLastError();
        return 512;
    }
    cached[dev].store(cus * per_cu, std::memory_order_relaxed);
    return cus * per_cu;
}

template <int KB, int VB>
hipError_t launch_append_fmt(const AppendArgs &a, hipStream_t stream) {
    const int64_t rows = a.num_tokens * a.num_kv_heads;
    // the staged kernel: a power-of-two head count, and 64 tokens' rows within
    // 31-bit byte offsets of each other (3-bit codes keep the lane kernel: their
    // bit-plane packing does not fit the staged kernel's registers)
    const int64_t max_stride = a.key_stride > a.value_stride ? a.key_stride : a.value_stride;
    if constexpr (KB != 3) {
        if (rows >= kLaneKernelMinRows && (a.num_kv_heads & (a.num_kv_heads - 1)) == 0 &&
            max_stride * 2 * 64 < ((int64_t)1 << 31)) {
            const int64_t nbatch = (rows + kStagedRows - 1) / kStagedRows;
            const int64_t resident = staged_resident_workgroups<KB, VB>();
            const int64_t blocks = nbatch < resident ? nbatch : resident;
            hipLaunchKernelGGL(HIP_KERNEL_NAME(quantize_append_staged<KB, VB>), dim3((unsigned)blocks), dim3(256),
                               0, stream, a, nbatch);
            return hipGetLastError();
        }
    }
    if (rows >= kLaneKernelMinRows) {
        const int64_t blocks = (rows + kLaneRows - 1) / kLaneRows;
        if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
        hipLaunchKernelGGL(HIP_KERNEL_NAME(quantize_append_lanes<KB, VB>), dim3((unsigned)blocks), dim3(256), 0,
                           stream, a);
        return hipGetLastError();
    }
    const int64_t groups = a.num_tokens * a.num_kv_heads * 2;
    const int64_t blocks = (groups + kRowsPerBlock - 1) / kRowsPerBlock;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(HIP_KERNEL_NAME(quantize_append_kernel<KB, VB>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const AppendArgs &a, hipStream_t stream) {
    if (a.k_bits == 4 && a.v_bits == 2) return launch_append_fmt<4, 2>(a, stream);
    if (a.k_bits == 4 && a.v_bits == 4) return launch_append_fmt<4, 4>(a, stream);
    if (a.k_bits == 8 && a.v_bits == 2) return launch_append_fmt<8, 2>(a, stream);
    if (a.k_bits == 8 && a.v_bits == 4) return launch_append_fmt<8, 4>(a, stream);
    if (a.k_bits == 3 && a.v_bits == 3) return launch_append_fmt<3, 3>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace kvq

// Quantise-on-write of new key/value tokens into the g128 paged cache (4/8-bit
// keys with 2/4-bit values, or 3 bits both; the KVarN preset is 4-bit keys
// and 2-bit values).
//
// Two kernels encode the same bytes:
//   quantize_append_kernel   one 16-lane row per group = (token, KV head,
//                            key|value), via encode_group (kvq_quant.h); low
//                            latency for a handful of tokens;
//   quantize_append_lanes    one lane per group, all 128 values in that lane's
//                            registers; no cross-lane traffic and no repeated
//                            per-group scalar work, about 3x fewer issued
//                            instructions per group; used for bulk appends.
// Both follow the format's definition operation for operation (fp32, no
// contraction, round-to-nearest-even, denormals kept), so their codes and
// metadata are bit-identical.
#pragma clang fp contract(off)

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

// One group per lane: encode the 128 fp16 values at `src` and store token
// slot `off` of `region` (KB-bit key / VB-bit value layout).  kValue selects
// the value encoding.
template <int KB, int VB, bool kValue>
__device__ __forceinline__ void encode_lane(const uint16_t *src, uint8_t *region, int off) {
    using Lay = Layout<KB, VB>;
    float y[kHeadDim];
#pragma unroll
    for (int c = 0; c < kHeadDim / 8; c++) {
        const uint4 raw = reinterpret_cast<const uint4 *>(src)[c];
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
            y[8 * c + 2 * e] = half_bits_to_float(w[e] & 0xffffu);
            y[8 * c + 2 * e + 1] = half_bits_to_float(w[e] >> 16);
        }
    }
    // 1. Hadamard rotation, butterfly stages h = 1, 2, ..., 64
#pragma unroll
    for (int h = 1; h < kHeadDim; h <<= 1) {
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
        // 3. asymmetric round-to-nearest (ties to even), clamp to [0, L]
        float delta = 0.0f;
        uint32_t csum = 0;
        if (hi != lo) {
            const float range = hi - lo;
            delta = range / (float)L;
            const float inv = (float)L / range;
#pragma unroll
            for (int i = 0; i < kHeadDim; i++) {
                const uint32_t code = (uint32_t)fminf(rintf((y[i] - lo) * inv), (float)L);
                if (kValue) {
                    csum += code;
                    if (VB == 2) {
                        packed[i & 15] |= code << (2 * (i >> 4));     // word m: channel 16j + m at bits 2j
                    } else if (VB == 3) {
                        // byte 3m + p: bit p of channel 16j + m's code at bit j
#pragma unroll
                        for (int p = 0; p < 3; p++) packed[3 * (i & 15) + p] |= ((code >> p) & 1u) << (i >> 4);
                    } else {   // word 2m + h: channel 16(4h + k) + m at bits 4k
                        packed[2 * (i & 15) + (i >> 6)] |= code << (4 * ((i >> 4) & 3));
                    }
                } else if (KB == 3) {
                    // plane word 3G + p (G = i / 32): bit p of the code at bit i % 32
#pragma unroll
                    for (int p = 0; p < 3; p++) packed[3 * (i >> 5) + p] |= ((code >> p) & 1u) << (i & 31);
                } else if (KB == 4) {
                    packed[i >> 3] |= code << (4 * (i & 7));      // byte b = c[2b] | c[2b+1] << 4
                } else {
                    packed[i >> 2] |= code << (8 * (i & 3));      // byte c = c[c]
                }
            }
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

template <int KB, int VB>
__global__ __launch_bounds__(256) void quantize_append_lanes(AppendArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int64_t rowi = (int64_t)blockIdx.x * kLaneRows + (wave & 1) * 64 + lane;
    if (rowi >= a.num_tokens * a.num_kv_heads) return;
    const int64_t tok = rowi / a.num_kv_heads;
    const int head = (int)(rowi % a.num_kv_heads);
    const int64_t slot = a.slots[tok];
    if (slot < 0) return;
    const int64_t page = slot >> (4 + a.page_log2s);
    const int t = (int)(slot & ((16 << a.page_log2s) - 1));
    const int off = t & 15;
    if (page >= a.num_pages) return;
    uint8_t *region = a.cache + (((page * a.num_kv_heads + head) << a.page_log2s) + (t >> 4)) *
                                    (int64_t)Layout<KB, VB>::kBytes;
    if (wave >> 1)
        encode_lane<KB, VB, true>(a.value + tok * a.value_stride + (int64_t)head * kHeadDim, region, off);
    else
        encode_lane<KB, VB, false>(a.key + tok * a.key_stride + (int64_t)head * kHeadDim, region, off);
}

template <int KB, int VB>
hipError_t launch_append_fmt(const AppendArgs &a, hipStream_t stream) {
    const int64_t rows = a.num_tokens * a.num_kv_heads;
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

// Encoder of one g128 group (one token of one KV head, keys or values) at
// 4/8-bit keys and 2/4-bit values, or 3 bits both, shared by the
// quantise-append kernel and the fused append-and-decode path.
//
// Method: the KVarN write path -- Hadamard rotation, variance normalisation,
// asymmetric round-to-nearest to 4-bit keys / 2-bit values (dothoosh.com,
// "KVarN vs TurboQuant: 5x more context with higher accuracy", pipeline list
// stages 1-3; beyondheadline.xyz, "Huawei's KV-cache trick", section "The
// claim that breaks the usual trade-off").
//
// Mapping: one 16-lane row of a wave encodes one group; lane r of the row
// holds channels 8r..8r+7 in registers.  The FWHT runs stages h = 1, 2, 4
// inside a lane and h = 8, 16, 32, 64 across lanes r^1, r^2, r^4, r^8, so
// every butterfly is the same fp32 a+b / a-b, in the same stage order, as the
// format's definition.  Partners 1, 2 and 8 lanes apart are read with DPP
// moves, 4 apart through the LDS crossbar (the values are the same either
// way); a row is always active or inactive as a whole, so every partner
// lane is active.  The sum of squares uses the format's fixed pairwise
// tree (lanes ^8, ^4, ^2, ^1, then in-lane 4, 2, 1); IEEE addition is
// commutative, so both lanes of a pair hold identical bits.  Codes are
// therefore bit-identical to any correct implementation of the format.  No
// fused multiply-add may be formed here: contraction is switched off inside
// the function body, which holds wherever it is inlined.
//
// Metadata per group: fp16 scale s = delta * sigma and one fp16 offset: the
// zero m * sigma for keys, the group mean sigma * (m + delta * C / 128) for
// values (C = sum of the codes), which is the dequantised original channel 0.
#pragma once

#include "kvq_device.h"

namespace kvq {

// The metadata is defined as an fp32 product rounded to fp16.  Left alone, the
// compiler fuses "fp32 multiply, convert to fp16" into one mixed-precision FMA
// that rounds only once, which differs from the definition at fp16 ties (and
// rotated values of subnormal inputs land on such ties often).  An empty asm
// statement pins the fp32 product in a register before the conversion.
__device__ __forceinline__ float materialize(float x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Step 1, the Hadamard rotation, of the group whose channels 8r..8r+7 are
// the four words of `raw` (fp16 pairs, low half first), on the 16 lanes of
// one row (r = lane within the row; all 16 must be active): y[e] receives
// rotated channel 8r + e in fp32.
__device__ __forceinline__ void rotate_row(const uint4 raw, int r, float (&y)[8]) {
#pragma clang fp contract(off)
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 4; e++) {
        y[2 * e] = half_bits_to_float(w[e] & 0xffffu);
        y[2 * e + 1] = half_bits_to_float(w[e] >> 16);
    }
    // in-lane stages h = 1, 2, 4 ...
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
        for (int e = 0; e < 8; e++) {
            if ((e & h) == 0) {
                const float p = y[e], q = y[e + h];
                y[e] = p + q;
                y[e + h] = p - q;
            }
        }
    }
    // ... cross-lane stages h = 8, 16, 32, 64 (lane r ^ (h / 8))
#pragma unroll
    for (int x = 1; x < 16; x <<= 1) {
        const bool upper = (r & x) != 0;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const float other = xor_lane_dpp(y[e], x);
            y[e] = upper ? (other - y[e]) : (y[e] + other);
        }
    }
}

// Sum of squares of the row's 128 values (y[e] = channel 8r + e, 16 lanes)
// by the format's fixed pairwise tree; every lane of the row gets the sum.
__device__ __forceinline__ float row_sum_squares(const float (&y)[8]) {
#pragma clang fp contract(off)
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; e++) p[e] = y[e] * y[e];
#pragma unroll
    for (int x = 8; x >= 1; x >>= 1) {
#pragma unroll
        for (int e = 0; e < 8; e++) p[e] = p[e] + xor_lane_dpp(p[e], x);
    }
    p[0] = p[0] + p[4]; p[1] = p[1] + p[5]; p[2] = p[2] + p[6]; p[3] = p[3] + p[7];
    p[0] = p[0] + p[2]; p[1] = p[1] + p[3];
    return p[0] + p[1];
}

// Steps 2-4 of the group held rotated in y (channel 8r + e in y[e], 16 lanes
// of one row, all active, sharing the arguments), and the store of its codes
// and metadata in token slot `off` (0..15) of the (page, KV head) region
// `region` of the KB-bit key / VB-bit value layout.
template <int KB, int VB>
__device__ __forceinline__ void encode_rotated_fmt(float (&y)[8], int is_v, int r, uint8_t *region, int off) {
#pragma clang fp contract(off)
    using Lay = Layout<KB, VB>;
    // 2. Variance normalisation: RMS over the group, fixed pairwise tree.
    const float ss = row_sum_squares(y);

    const int L = is_v ? Lay::kVL : Lay::kKL;
    uint32_t code[8];
    float sm = 0.0f, zm = 0.0f;   // metadata before fp16 rounding
    if (ss == 0.0f) {
#pragma unroll
        for (int e = 0; e < 8; e++) code[e] = 0;
    } else {
        const float sigma = sqrtf(ss * 0x1p-7f);
        const float rcp = 1.0f / sigma;
        float lo, hi;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            y[e] = y[e] * rcp;
            lo = e ? fminf(lo, y[e]) : y[e];
            hi = e ? fmaxf(hi, y[e]) : y[e];
        }
#pragma unroll
        for (int x = 1; x < 16; x <<= 1) {
            lo = fminf(lo, xor_lane_dpp(lo, x));
            hi = fmaxf(hi, xor_lane_dpp(hi, x));
        }
        // 3. Asymmetric round-to-nearest (ties to even), clamp to [0, L].
        float delta = 0.0f;
        if (hi == lo) {
#pragma unroll
            for (int e = 0; e < 8; e++) code[e] = 0;
        } else {
            const float range = hi - lo;
            delta = range / (float)L;
            const float inv = (float)L / range;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const float c = rintf((y[e] - lo) * inv);
                code[e] = c > (float)L ? (uint32_t)L : (uint32_t)c;
            }
        }
        sm = delta * sigma;
        if (!is_v) {
            zm = lo * sigma;                       // keys: the zero
        } else {
            // values: the group mean sigma * (m + delta * C / 128), C = sum of codes
            uint32_t csum = 0;
#pragma unroll
            for (int e = 0; e < 8; e++) csum += code[e];
#pragma unroll
            for (int x = 1; x < 16; x <<= 1) csum += xor_lane_u_dpp(csum, x);
            float t = delta * (float)csum;
            t = t * 0x1p-7f;
            t = lo + t;
            zm = t * sigma;
        }
    }
    const uint32_t s16 = float_to_half_bits(materialize(sm));
    uint32_t z16 = float_to_half_bits(materialize(zm));
    if (z16 == 0x8000u) z16 = 0;   // a zero offset is stored as +0

    if (!is_v) {
        if (KB == 3) {
            // keys as bit planes: lane r holds channels 32G + x, G = r / 4,
            // x = 8 (r % 4) + e, so byte r % 4 of plane word (G, p) at
            // 12G + 4p of the token's 48-byte row is this lane's bit p of
            // codes e = 0..7
            uint8_t *row = region + Lay::kKCodes + 48 * off + 12 * (r >> 2) + (r & 3);
#pragma unroll
            for (int p = 0; p < 3; p++) {
                uint32_t b = 0;
#pragma unroll
                for (int e = 0; e < 8; e++) b |= ((code[e] >> p) & 1u) << e;
                row[4 * p] = (uint8_t)b;
            }
        } else if (KB == 4) {
            // keys: byte b of the token's 64 = code[2b] | code[2b+1] << 4
            uint32_t packed = 0;
#pragma unroll
            for (int e = 0; e < 8; e++) packed |= code[e] << (4 * e);
            *reinterpret_cast<uint32_t *>(region + Lay::kKCodes + 64 * off + 4 * r) = packed;
        } else {
            // keys: byte c of the token's 128 = code[c]
            const uint32_t lo = code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
            const uint32_t hi = code[4] | (code[5] << 8) | (code[6] << 16) | (code[7] << 24);
            *reinterpret_cast<uint2 *>(region + Lay::kKCodes + 128 * off + 8 * r) = make_uint2(lo, hi);
        }
        if (r == 0)
            *reinterpret_cast<uint32_t *>(region + Lay::kKMeta + 4 * off) = s16 | (z16 << 16);
    } else if (VB == 3) {
        // values as bit planes: for channel 16j + m, byte p of the word for
        // m collects bit p of the code at bit j.  Lane r has channels
        // 8r..8r+7, i.e. j = r/2 and m = 8(r&1) + e; the 8 lanes that share
        // r&1 are OR-reduced with the transpose used for 2-bit values, which
        // leaves each lane the word of one m.  Its byte p goes to byte
        // (0, 2, 1, 3)[i] of plane word p at 12 (16g + m) + 4p.
        const int j = r >> 1;
        uint32_t v8[8];
#pragma unroll
        for (int e = 0; e < 8; e++)
            v8[e] = ((code[e] & 1u) << j) | (((code[e] >> 1) & 1u) << (8 + j)) | (((code[e] >> 2) & 1u) << (16 + j));
        const bool b1 = (r & 2) != 0, b2 = (r & 4) != 0, b3 = (r & 8) != 0;
        uint32_t v4[4];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const uint32_t send = b1 ? v8[k] : v8[4 + k];
            const uint32_t keep = b1 ? v8[4 + k] : v8[k];
            v4[k] = keep | xor_lane_u_dpp(send, 2);
        }
        uint32_t v2[2];
#pragma unroll
        for (int k = 0; k < 2; k++) {
            const uint32_t send = b2 ? v4[k] : v4[2 + k];
            const uint32_t keep = b2 ? v4[2 + k] : v4[k];
            v2[k] = keep | xor_lane_u_dpp(send, 4);
        }
        const uint32_t send = b3 ? v2[0] : v2[1];
        const uint32_t keep = b3 ? v2[1] : v2[0];
        const uint32_t word = keep | xor_lane_u_dpp(send, 8);
        const int m = 8 * (r & 1) + 4 * (int)b1 + 2 * (int)b2 + (int)b3;
        const int g = off >> 2, i = off & 3;
        uint8_t *vb = region + Lay::kVCodes + 12 * (16 * g + m) + (((i & 1) << 1) | (i >> 1));
#pragma unroll
        for (int p = 0; p < 3; p++) vb[4 * p] = (uint8_t)(word >> (8 * p));
        if (r == 0)
            *reinterpret_cast<uint32_t *>(region + Lay::kVMeta + 4 * off) = s16 | (z16 << 16);
    } else if (VB == 4) {
        // values: with channel 16j + m and j = 4h + k, the u16 word for
        // (m, h) holds code(16j + m) << 4k, k = 0..3.  Lane r has channels
        // 8r..8r+7: j = r/2 (h = r/8, k = (r/2) & 3) and m = 8(r&1) + e.  The
        // 4 lanes that differ in bits 1 and 2 of r fill the same 8 words;
        // a transpose-OR over lanes ^2, ^4 leaves each lane 2 whole words.
        uint32_t v8[8];
#pragma unroll
        for (int e = 0; e < 8; e++) v8[e] = code[e] << (4 * ((r >> 1) & 3));
        const bool b1 = (r & 2) != 0, b2 = (r & 4) != 0;
        uint32_t v4[4];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const uint32_t send = b1 ? v8[k] : v8[4 + k];
            const uint32_t keep = b1 ? v8[4 + k] : v8[k];
            v4[k] = keep | xor_lane_u_dpp(send, 2);
        }
        const int g = off >> 2, i = off & 3, h = r >> 3;
        uint8_t *base = region + Lay::kVCodes + 256 * g + 8 * (i >> 1) + 4 * h + 2 * (i & 1);
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const uint32_t send = b2 ? v4[u] : v4[2 + u];
            const uint32_t keep = b2 ? v4[2 + u] : v4[u];
            const uint32_t word = keep | xor_lane_u_dpp(send, 4);
            const int m = 8 * (r & 1) + 4 * (int)b1 + 2 * (int)b2 + u;
            *reinterpret_cast<uint16_t *>(base + 16 * m) = (uint16_t)word;
        }
        if (r == 0)
            *reinterpret_cast<uint32_t *>(region + Lay::kVMeta + 4 * off) = s16 | (z16 << 16);
    } else {
        // values: u16 word for m holds code(16j + m) << 2j, j = 0..7.  Lane r
        // has channels 8r..8r+7, i.e. j = r/2 and m = 8(r&1) + e.  Reduce the
        // 8 lanes that share r&1 with a transpose-OR over lanes ^2, ^4, ^8:
        // each step keeps half of the words and ORs in the partner's half.
        uint32_t v8[8];
#pragma unroll
        for (int e = 0; e < 8; e++) v8[e] = code[e] << (2 * (r >> 1));
        const bool b1 = (r & 2) != 0, b2 = (r & 4) != 0, b3 = (r & 8) != 0;
        uint32_t v4[4];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const uint32_t send = b1 ? v8[k] : v8[4 + k];
            const uint32_t keep = b1 ? v8[4 + k] : v8[k];
            v4[k] = keep | xor_lane_u_dpp(send, 2);
        }
        uint32_t v2[2];
#pragma unroll
        for (int k = 0; k < 2; k++) {
            const uint32_t send = b2 ? v4[k] : v4[2 + k];
            const uint32_t keep = b2 ? v4[2 + k] : v4[k];
            v2[k] = keep | xor_lane_u_dpp(send, 4);
        }
        const uint32_t send = b3 ? v2[0] : v2[1];
        const uint32_t keep = b3 ? v2[1] : v2[0];
        const uint32_t word = keep | xor_lane_u_dpp(send, 8);
        const int m = 8 * (r & 1) + 4 * (int)b1 + 2 * (int)b2 + (int)b3;
        const int g = off >> 2, i = off & 3;
        *reinterpret_cast<uint16_t *>(region + Lay::kVCodes + 128 * g + 8 * m + 2 * i) = (uint16_t)word;
        if (r == 0)
            *reinterpret_cast<uint32_t *>(region + Lay::kVMeta + 4 * off) = s16 | (z16 << 16);
    }
}

// Encode the 128 fp16 values at `src` (16-byte aligned) with the 16 lanes of
// one row (r = lane within the row; all 16 lanes must be active and share the
// arguments) and store codes and metadata of token slot `off` (0..15) in the
// (page, KV head) region `region` of the KB-bit key / VB-bit value layout.
template <int KB, int VB>
__device__ __forceinline__ void encode_group_fmt(const uint16_t *src, int is_v, int r, uint8_t *region,
                                                 int off) {
    float y[8];
    rotate_row(*reinterpret_cast<const uint4 *>(src + 8 * r), r, y);
    encode_rotated_fmt<KB, VB>(y, is_v, r, region, off);
}

// The K4V2 layout.
__device__ __forceinline__ void encode_group(const uint16_t *src, int is_v, int r, uint8_t *region, int off) {
    encode_group_fmt<4, 2>(src, is_v, r, region, off);
}

}  // namespace kvq

// Device pieces shared by the decode split kernels (K4V2 and the fp16
// baseline) and the split combine: the per-lane softmax state, the merge of
// the 4 waves of a work-group, the partial write, and the output epilogue.
#pragma once

#include <math.h>

#include "kvq_device.h"

namespace kvq {

constexpr float kLazyThreshold = 8.0f;   // log2 of the largest unnormalised weight

struct State {
    float m;        // running max (base 2) of this lane's column
    float l;        // partial sum of weights over this lane's tokens
    float z;        // partial sum of weight * value mean (quantised caches)
    v4f acc[8];     // value accumulators, channel 16j + 4g + i, column n
};

// In-place unnormalised Hadamard transform of one head's 128 values held by
// 32 lanes (lane32 = lane & 31), 4 channels each: 2 stages in-lane, 5 across
// (partners 1, 2 and 8 lanes apart by DPP moves, 4 and 16 by permutes).
__device__ __forceinline__ void hadamard_128(float (&y)[4], int lane32) {
    {
        float p = y[0], q = y[1]; y[0] = p + q; y[1] = p - q;
        p = y[2]; q = y[3]; y[2] = p + q; y[3] = p - q;
        p = y[0]; q = y[2]; y[0] = p + q; y[2] = p - q;
        p = y[1]; q = y[3]; y[1] = p + q; y[3] = p - q;
    }
#pragma unroll
    for (int x = 1; x < 32; x <<= 1) {
        const bool upper = (lane32 & x) != 0;
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const float other = xor_lane_dpp(y[e], x);
            y[e] = upper ? (other - y[e]) : (y[e] + other);
        }
    }
}

// Output of one head from merged sums: 32 lanes (lane32 = lane & 31) hold
// channels 4*lane32 .. +3.  rotated (the K4V2 path): o_j = (H acc)_j / (128 l)
// for j >= 1 and o_0 = z / l (the FWHT runs 2 stages in-lane and 5 across);
// otherwise o = acc / l.  l = 0 gives a zero row.
__device__ __forceinline__ void finalize_head(const float (&acc)[4], float l, float z, int lane32,
                                              void *out, int out_f32, int64_t row, int rotated) {
    float y[4] = {acc[0], acc[1], acc[2], acc[3]};
    const float inv_l = l > 0.0f ? 1.0f / l : 0.0f;
    float o[4];
    if (rotated) {
        hadamard_128(y, lane32);
        const float sc = inv_l * (1.0f / 128.0f);
#pragma unroll
        for (int e = 0; e < 4; e++) o[e] = y[e] * sc;
        if (lane32 == 0) o[0] = z * inv_l;   // channel 0 is the weighted mean of the stored value means
    } else {
#pragma unroll
        for (int e = 0; e < 4; e++) o[e] = y[e] * inv_l;
    }
    const int64_t base = row * kHeadDim + 4 * lane32;
    if (out_f32) {
        *reinterpret_cast<float4 *>(static_cast<float *>(out) + base) = make_float4(o[0], o[1], o[2], o[3]);
    } else {
        const uint32_t lo = (uint32_t)float_to_half_bits(o[0]) | ((uint32_t)float_to_half_bits(o[1]) << 16);
        const uint32_t hi = (uint32_t)float_to_half_bits(o[2]) | ((uint32_t)float_to_half_bits(o[3]) << 16);
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + base) = make_uint2(lo, hi);
    }
}

// Query / output row of head index v (0 <= v < a.gqa) of KV head kvh of
// sequence b.  One query row per sequence: row b * Hq + kvh * G + v.  With
// q_len rows, v = m * G + g is head kvh * G + g of row m, and rows are laid
// out [num_seqs][q_len][Hq].  kMQ = false: one query row (q_len is not read).
template <bool kMQ>
__device__ __forceinline__ int64_t io_row(const DecodeArgs &a, int b, int kvh, int v) {
    if (!kMQ || a.q_len <= 1) return (int64_t)b * a.num_q_heads + kvh * a.gqa + v;
    const int G = a.gqa / a.q_len;
    const int m = v / G;
    return ((int64_t)b * a.q_len + m) * (a.num_q_heads / a.q_len) + kvh * G + (v - m * G);
}

// LDS of the merge of the W waves of a work-group.
template <int W>
struct MergeLdsT {
    float m[W][kHeadsPerGroup];
    float l[W][kHeadsPerGroup];
    float z[W][kHeadsPerGroup];
    float acc[W][kHeadsPerGroup][kHeadDim];
};
using MergeLds = MergeLdsT<kWaves>;

// Merge the W waves' states of a work-group (head indices v0 .. v0 + nh - 1
// of KV head kvh of sequence b) and write the split's partial, or the output
// when the launch has a single split (then no combine runs).  unscale(j) is
// the factor of channel block j.  Every thread of the work-group must call it;
// the first 256 (32 per head) merge and store.
// (rotate_out: the partial is stored in the K4V2 Hadamard domain, acc' = H acc
// and zacc = acc_0, so that it merges with K4V2 partials in one combine:
// (H acc')_j / 128 = acc_j for j >= 1 and channel 0 comes from zacc.)
template <bool kMQ = false, int W, typename Unscale>
__device__ __forceinline__ void merge_and_store(State &st, MergeLdsT<W> &s, const DecodeArgs &a, int rotated,
                                                Unscale unscale, int wave, int tid, int b, int kvh, int v0,
                                                int nh, int split, int rotate_out = 0) {
    const int hq0 = kvh * a.gqa + v0;
    const int lane = tid & 63;
    const int n16 = lane & 15;
    const int g = lane >> 4;
    float lsum = st.l + xor_lane(st.l, 16);
    lsum += xor_lane(lsum, 32);
    float zsum = st.z + xor_lane(st.z, 16);
    zsum += xor_lane(zsum, 32);
    // value sums: column n holds the fp16 part, column n + 8 the residual
#pragma unroll
    for (int j = 0; j < 8; j++)
#pragma unroll
        for (int i = 0; i < 4; i++) st.acc[j][i] += row_swap8(st.acc[j][i]);
    if (n16 < kHeadsPerGroup) {
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const float u = unscale(j);
#pragma unroll
            for (int i = 0; i < 4; i++) s.acc[wave][n16][16 * j + 4 * g + i] = st.acc[j][i] * u;
        }
        if (g == 0) {
            s.m[wave][n16] = st.m;
            s.l[wave][n16] = lsum;
            s.z[wave][n16] = zsum;
        }
    }
    __syncthreads();

    const int hh = tid >> 5;          // head of this thread in the merge
    if (hh >= kHeadsPerGroup) return;
    const int l32 = tid & 31;
    const int c0 = 4 * l32;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; w++) M = fmaxf(M, s.m[w][hh]);
    float lt = 0.0f, zt = 0.0f, acc4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int w = 0; w < W; w++) {
        const float mw = s.m[w][hh];
        const float f = (mw == -INFINITY) ? 0.0f : fast_exp2(mw - M);
        lt += f * s.l[w][hh];
        zt += f * s.z[w][hh];
#pragma unroll
        for (int e = 0; e < 4; e++) acc4[e] += f * s.acc[w][hh][c0 + e];
    }

    const int64_t row = (int64_t)b * a.num_q_heads + hq0 + hh;
    if (a.splits == 1 && !a.partials_only) {
        if (hh < nh)
            finalize_head(acc4, lt, zt, l32, a.out, a.out_f32, io_row<kMQ>(a, b, kvh, v0 + hh), rotated);
        return;
    }
    if (rotate_out) {
        zt = __shfl(acc4[0], tid & 32, 64);   // channel 0 of this head, from its lane 0
        hadamard_128(acc4, l32);
    }
    float *mine = a.partials + (row * a.slot_stride + a.slot_offset + split) * kPartialFloats;
    if (hh < nh) {
        if (l32 == 0) {
            mine[0] = M;
            mine[1] = lt;
            mine[2] = zt;
        }
        *reinterpret_cast<float4 *>(mine + 4 + c0) = make_float4(acc4[0], acc4[1], acc4[2], acc4[3]);
    }
}

// A work-group with no tokens (an empty sequence, or a split past the
// sequence's end).  With a single split and no combine to follow it writes
// zero output rows; otherwise it writes empty partials (m = -inf, l = zacc =
// acc = 0), so that the combine can merge every split slot of every row
// without knowing the sequence lengths.
template <bool kMQ = false>
__device__ __forceinline__ void write_empty(const DecodeArgs &a, int tid, int b, int kvh, int v0, int nh,
                                            int split) {
    const int hq0 = kvh * a.gqa + v0;
    if (a.splits == 1 && !a.partials_only) {
        if ((tid >> 5) < nh) {
            const int64_t base = io_row<kMQ>(a, b, kvh, v0 + (tid >> 5)) * kHeadDim + 4 * (tid & 31);
            if (a.out_f32) *reinterpret_cast<float4 *>(static_cast<float *>(a.out) + base) = make_float4(0, 0, 0, 0);
            else *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + base) = make_uint2(0, 0);
        }
        return;
    }
    constexpr int kQuads = kPartialFloats / 4;   // 33 float4 per partial
    for (int i = tid; i < nh * kQuads; i += (int)blockDim.x) {
        const int hh = i / kQuads, qd = i % kQuads;
        const int64_t row = (int64_t)b * a.num_q_heads + hq0 + hh;
        float *mine = a.partials + (row * a.slot_stride + a.slot_offset + split) * kPartialFloats;
        *reinterpret_cast<float4 *>(mine + 4 * qd) = qd == 0 ? make_float4(-INFINITY, 0, 0, 0) : make_float4(0, 0, 0, 0);
    }
}

}  // namespace kvq

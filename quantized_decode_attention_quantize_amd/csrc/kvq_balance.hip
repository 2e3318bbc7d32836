// Quantise-on-write with page-balanced keys: an active reading of the
// variance normalisation, stage 2 of the KVarN pipeline (dothoosh.com, "KVarN
// vs TurboQuant: 5x more context with higher accuracy", pipeline list stage 2,
// which words the normalisation as repeated, and its closing paragraph on
// removing fluctuations in logarithmic space; beyondheadline.xyz, "Huawei's
// KV-cache trick", section "The claim that breaks the usual trade-off": cache
// blocks normalised before low-bit quantisation).
//
// A block is one 16-token page of one KV head.  Its rotated keys Y (16 rows x
// 128 channels, absent rows zero) are balanced in second moment with every
// scale a power of two:
//   column pass: ss_j = sum_t (Y_tj 2^-f_t)^2 by the pairwise tree over the
//     16 row slots (h = 8, 4, 2, 1), e_j = floor(F_j / 2) for ss_j = m 2^F_j,
//     m in [0.5, 1) (0 for a zero column);
//   row pass (between column passes): ss_t = sum_j (Y_tj 2^-e_j)^2 by the
//     encoder's tree, f_t = floor(F_t / 2) likewise (0 for a zero row);
// two column passes with one row pass between them.  The stored exponents
// come from the last column pass in integers: over the n non-zero columns,
// with S the sum of their F_j and d_j = n F_j - S, e_j = 0 when |d_j| < 2n,
// else floor((d_j + n) / (2n)), clamped to [-6, 6]; a zero column takes -6.
// Each present row of Y_tj 2^-e_j (exact: the scales are powers of two) then
// goes through the K4V2 encoder's steps 2-4, and byte j of the region's
// scale block holds the high byte of fp16 2^e_j.  Values are the K4V2
// per-token groups.
//
// Mapping: one work-group of 256 lanes per (page, KV head); row t of the
// block is lanes 16t .. 16t + 15 (lane r holds channels 8r .. 8r + 7, as in
// the per-token encoder, whose rotation, sum-of-squares tree and steps 2-4
// run unchanged).  Column sums go through LDS: 128 lanes each add one
// column's 16 squares by the block tree.  Every operation is the plain fp32
// one with contraction off, so the bytes equal any correct implementation of
// this definition.
#include "kvq_device.h"
#include "kvq_quant.h"

namespace kvq {
namespace {

constexpr int kColumnPasses = 2;   // column passes; a row pass between consecutive ones
constexpr int kScaleExpMax = 6;    // column exponents lie in [-6, 6]

__device__ __forceinline__ int floor_div(int a, int b) { return a >= 0 ? a / b : -((b - 1 - a) / b); }   // b > 0
__device__ __forceinline__ int floor_half(int f) { return floor_div(f, 2); }
__device__ __forceinline__ int frexp_exponent(float x) {
    int e = 0;
    (void)frexpf(x, &e);
    return e;
}

// Sum of the 64 lanes' values of one wave.
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int x = 1; x < 64; x <<= 1) v += (int)xor_lane_u_dpp((uint32_t)v, x);
    return v;
}

__global__ __launch_bounds__(256) void balance_append_kernel(AppendArgs a) {
#pragma clang fp contract(off)
    const int64_t b0 = (int64_t)blockIdx.x * kPage;   // call tokens b0 .. b0 + 15
    const int head = blockIdx.y;
    const int tid = threadIdx.x;
    const int t = tid >> 4;                            // row (token slot of the page)
    const int r = tid & 15;                            // lane of the row: channels 8r .. 8r + 7
    const int64_t base = a.slots[b0];
    // the whole work-group takes the same branch
    if (base < 0 || (base % kPage) != 0 || base / kPage >= a.num_pages) return;
    const int64_t page = base / kPage;
    const int64_t tok = b0 + t;
    const bool present = tok < a.num_tokens && a.slots[tok] == base + t;
    uint8_t *region = a.cache + (page * a.num_kv_heads + head) * kRegionPB;

    __shared__ float s_sq[kPage][kHeadDim];   // squares of the scaled block
    __shared__ int s_e[kHeadDim];             // column exponents
    __shared__ int s_red[2][2];               // (non-zero columns, sum of their F) per wave

    // the row's key and value words, both requested before any arithmetic
    uint4 raw = make_uint4(0u, 0u, 0u, 0u), raw_v = make_uint4(0u, 0u, 0u, 0u);
    if (present) {
        raw = *reinterpret_cast<const uint4 *>(a.key + tok * a.key_stride + (int64_t)head * kHeadDim + 8 * r);
        raw_v = *reinterpret_cast<const uint4 *>(a.value + tok * a.value_stride + (int64_t)head * kHeadDim + 8 * r);
    }
    float y[8];
    rotate_row(raw, r, y);                     // an absent row stays zero

    int f = 0;                 // this row's exponent f_t
    float css = 0.0f;          // lanes < 128: the last column pass's sum of column tid
    for (int pass = 1; pass <= kColumnPasses; pass++) {
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const float u = __builtin_ldexpf(y[e], -f);
            s_sq[t][8 * r + e] = u * u;
        }
        __syncthreads();
        if (tid < kHeadDim) {
            float c[kPage];
#pragma unroll
            for (int i = 0; i < kPage; i++) c[i] = s_sq[i][tid];
#pragma unroll
            for (int h = kPage / 2; h >= 1; h >>= 1)
#pragma unroll
                for (int i = 0; i < h; i++) c[i] = c[i] + c[i + h];
            css = c[0];
            s_e[tid] = css != 0.0f ? floor_half(frexp_exponent(css)) : 0;
        }
        __syncthreads();
        if (pass == kColumnPasses) break;
        // row pass (the next column pass rewrites s_e only after its barrier)
        float u[8];
#pragma unroll
        for (int e = 0; e < 8; e++) u[e] = __builtin_ldexpf(y[e], -s_e[8 * r + e]);
        const float ss = row_sum_squares(u);
        f = ss != 0.0f ? floor_half(frexp_exponent(ss)) : 0;
    }

    // the stored exponents, from the last column pass
    const bool has = tid < kHeadDim && css != 0.0f;
    const int F = has ? frexp_exponent(css) : 0;
    if (tid < kHeadDim) {
        const int cnt = wave_sum(has ? 1 : 0);
        const int sum = wave_sum(F);
        if ((tid & 63) == 0) {
            s_red[tid >> 6][0] = cnt;
            s_red[tid >> 6][1] = sum;
        }
    }
    __syncthreads();
    if (tid < kHeadDim) {
        const int n = s_red[0][0] + s_red[1][0];
        const int S = s_red[0][1] + s_red[1][1];
        int e = -kScaleExpMax;
        if (has) {
            const int d = n * F - S;
            const int q = (d < 2 * n && d > -2 * n) ? 0 : floor_div(d + n, 2 * n);
            e = q < -kScaleExpMax ? -kScaleExpMax : (q > kScaleExpMax ? kScaleExpMax : q);
        }
        s_e[tid] = e;
        region[kScalesPB + tid] = (uint8_t)((e + 15) * 4);
    }
    __syncthreads();

    if (present) {
        float ys[8];
#pragma unroll
        for (int e = 0; e < 8; e++) ys[e] = __builtin_ldexpf(y[e], -s_e[8 * r + e]);
        encode_rotated_fmt<4, 2>(ys, 0, r, region, t);
        float yv[8];
        rotate_row(raw_v, r, yv);
        encode_rotated_fmt<4, 2>(yv, 1, r, region, t);
    }
}

}  // namespace

hipError_t launch_balance_append(const AppendArgs &a, hipStream_t stream) {
    const int64_t blocks = (a.num_tokens + kPage - 1) / kPage;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL || a.num_kv_heads > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL(balance_append_kernel, dim3((unsigned)blocks, (unsigned)a.num_kv_heads), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace kvq

// Split-K decode attention over the K4V2 g128 paged cache, read with scale
// folding (dothoosh.com, "KVarN vs TurboQuant: 5x more context with higher
// accuracy", pipeline list stage 4).  Decode streams the whole cache through
// HBM once per token (encorp.ai, "KV cache compression is an infrastructure
// decision, not a model debate", section on the HBM ceiling), so the kernel is
// built to move 104 bytes per cached token per KV head and nothing more, and
// never materialises dequantised keys or values (vLLM's TurboQuant test lost
// 10-70% throughput to exactly that conversion: dzen.ru summary of the vLLM
// TurboQuant post, section "Performance").
//
// Algebra (H = H^T, H H = 128 I, H 1 = 128 e_0; cached rotated value s c + z):
//   q . k_t  = (s_t (q'.c_t) + z_t sum(q')) / 128,          q' = H q
//   sum_t p_t v_t = (H acc + 128 zv e_0) / 128,  acc = sum p_t s_t c_t,
//                                                zv = sum p_t z_t,
// and since the value metadata stores the group mean mu_t = s_t C_t / 128 +
// z_t (C_t = code sum), output channel 0 is simply sum p_t mu_t / sum p_t:
// the large, nearly cancelling terms s_t C_t and 128 z_t never meet in fp32.
//
// Work decomposition.  Grid (split, KV head x work-group of head groups,
// sequence); a work-group of 4 waves owns `pages_per_split` consecutive pages
// of one (sequence, KV head) and up to 8 query heads of that KV head (one
// head group), or 16 (two groups sharing the page unpack) when the KV head
// has more.  Each wave takes page pairs w, w+4, ... of the split.
//
// Per page pair, per wave (64 lanes; n = lane & 15, g = lane >> 4):
//   Scores: v_mfma_f32_16x16x32_f16 x 4, A = key codes (row = token n, the
//     16 bytes of the token's 64-byte code row at 16g, each nibble an fp16
//     subnormal), B = the rotated query in fp16 with 16 columns: columns 0-7
//     q_hi of heads 0-7, columns 8-15 the residual q_lo = q' - q_hi (the
//     two-term query of the BitDecoding digest: rit.work, "BitDecoding-FP4
//     ...", second paragraph).  Output lane (n, g) holds tokens 4g..4g+3 of
//     column n; a DPP row rotation by 8 adds the partner column.
//   Softmax: base 2, fp32, running max per head, rescaled lazily (only when a
//     page's score exceeds the running max by more than 8, i.e. p <= 256).
//     The per-token work (fold, exp, weight, sums) is split between the two
//     lanes of a column pair: lane n < 8 takes page A's 4 tokens, lane n + 8
//     page B's, and one bank-masked DPP move per dword hands each lane the
//     weight half it lacks.
//   Values: v_mfma_f32_16x16x32_f16, A = value codes (row = channel 16j + m,
//     k = 8 tokens: 4 of each page), B = w = p * s_v (k = the same 8 tokens):
//     column n < 8 holds fp16(w) of head n, column n + 8 the residual
//     w - fp16(w), so the two columns together carry w to ~2^-22 and the
//     rounding cannot break the cancellation between s_v * sum(c) and the
//     zero-point sum in output channel 0.  A 2-bit code at bits 2j'..2j'+1 of a 16-bit
//     word is, bit for bit, the fp16 subnormal c * 2^(2j' - 24); MFMA takes
//     fp16 subnormals exactly, so the value codes need one AND per pair of
//     tokens (and a shared shift) and no conversion.  The power of two is
//     removed per channel block in the epilogue.
// Epilogue: merge the 4 waves in LDS and write one partial (m, l, zacc, acc)
// per head (zacc = sum p mu); a sequence that fits one split is finished in
// place.  combine_kernel, launched next on the same stream, merges the
// partials (LSE) and writes o_j = (H acc)_j / (128 l) for j >= 1 and
// o_0 = zacc / l.  (A last-work-group-merges scheme inside one kernel needs a
// device-scope release and acquire per work-group, i.e. a write-back and an
// invalidate of the XCD's L2 each time; measured, that cost several times
// the whole page stream.)
//
// Variants, all instantiations of the same kernel template: 8-bit keys and
// 4-bit values (KB, VB: other key-operand and value-operand unpacking, the
// same algebra); several causal query rows per sequence (kMQ: (row, head)
// pairs take the MFMA columns, per-lane token limits in the masked tail
// pairs, an XCD-aware grid); pages of 32-128 tokens (kPaged: a block-table
// entry covers several 16-token regions).  The K4V2 single-row 16-token
// instantiation is the hot path above.
#include <hip/hip_ext.h>

#include <atomic>
#include <math.h>
#include <type_traits>

#include "kvq_decode_common.h"
#include "kvq_device.h"
#include "kvq_quant.h"

namespace kvq {
namespace {

constexpr int kDecodeWaves = 4;    // waves per work-group of decode_kernel


// One page of one lane, for KB-bit keys and VB-bit values.
template <int KB, int VB>
struct PageRegs {
    uint32_t k[KB];   // key codes: token (lane & 15), channels 32g..32g+31 (g = lane >> 4),
                      // the 4*KB bytes at 4*KB*g of the token's code row (3 bits: the
                      // three bit-plane words of those channels)
    uint32_t v[VB];   // value codes: the 4*VB bytes at 4*VB*lane (quad g, channel lane & 15;
                      // 3 bits: the three bit-plane words)
    uint4 km;         // key (s, z) of tokens 4g..4g+3
    uint4 vm;         // value (s, mu) of tokens 4g..4g+3
};

// Byte offsets of a lane's loads inside a page region (loop invariant).
template <int KB, int VB>
struct LaneOffsets {
    uint32_t k, v, km, vm;
    __device__ explicit LaneOffsets(int lane)
        : k(Layout<KB, VB>::kKCodes + (uint32_t)(lane & 15) * (16u * KB) + (uint32_t)(lane >> 4) * (4u * KB)),
          v(Layout<KB, VB>::kVCodes + (uint32_t)lane * (4u * VB)),
          km(Layout<KB, VB>::kKMeta + (uint32_t)(lane >> 4) * 16u),
          vm(Layout<KB, VB>::kVMeta + (uint32_t)(lane >> 4) * 16u) {}
};

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v3u __attribute__((ext_vector_type(3)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

// `region` is wave-uniform: it becomes a buffer resource in scalar registers
// (the region's byte range, so the hardware bounds-checks every access) and
// the per-lane 32-bit offsets are loop invariant, so a page costs four to six
// buffer loads and no vector address arithmetic.  live = false gives the
// resource no bytes: every load is out of range and returns zeros without a
// memory access (the prefetch past a wave's last pair).
template <int KB, int VB>
__device__ __forceinline__ void load_page(const uint8_t *region, const LaneOffsets<KB, VB> &o,
                                          PageRegs<KB, VB> &r, bool live = true) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(region), (short)0, live ? Layout<KB, VB>::kBytes : 0, 0x00020000);
    if constexpr (KB == 3) {
        const v3u k = __builtin_amdgcn_raw_buffer_load_b96(rs, o.k, 0, 0);
        r.k[0] = k.x; r.k[1] = k.y; r.k[2] = k.z;
    } else {
#pragma unroll
        for (int h = 0; h < KB / 4; h++) {
            const v4u k = __builtin_amdgcn_raw_buffer_load_b128(rs, o.k + 16 * h, 0, 0);
            r.k[4 * h] = k.x; r.k[4 * h + 1] = k.y; r.k[4 * h + 2] = k.z; r.k[4 * h + 3] = k.w;
        }
    }
    if constexpr (VB == 2) {
        const v2u v = __builtin_amdgcn_raw_buffer_load_b64(rs, o.v, 0, 0);
        r.v[0] = v.x; r.v[1] = v.y;
    } else if constexpr (VB == 3) {
        const v3u v = __builtin_amdgcn_raw_buffer_load_b96(rs, o.v, 0, 0);
        r.v[0] = v.x; r.v[1] = v.y; r.v[2] = v.z;
    } else {
        const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rs, o.v, 0, 0);
        r.v[0] = v.x; r.v[1] = v.y; r.v[2] = v.z; r.v[3] = v.w;
    }
    const v4u km = __builtin_amdgcn_raw_buffer_load_b128(rs, o.km, 0, 0);
    const v4u vm = __builtin_amdgcn_raw_buffer_load_b128(rs, o.vm, 0, 0);
    r.km = make_uint4(km.x, km.y, km.z, km.w);
    r.vm = make_uint4(vm.x, vm.y, vm.z, vm.w);
}

// Key-code A operand of one 8-channel dword w (channels 8d..8d+7 of the 32
// this lane-group owns): four dwords of fp16 pairs.  A 4-bit code at bits
// 4r'..4r'+3 of a 16-bit half is, bit for bit, the fp16 subnormal
// c * 2^(4r' - 24); with r' in {0, 1} every code needs one AND per pair of
// channels.  Slot e of the 8 holds channel perm[e] = {0,4,1,5,2,6,3,7}[e],
// scaled by 2^-24 (e & 2 == 0) or 2^-20 (e & 2 != 0); the query operand
// carries the matching channel order and the inverse 2^-4.
__device__ __forceinline__ v8h key_codes(uint32_t w) {
    const uint32_t t = w >> 8;
    const uint4 u = {w & 0x000F000Fu, w & 0x00F000F0u, t & 0x000F000Fu, t & 0x00F000F0u};
    return __builtin_bit_cast(v8h, u);
}

// 8-bit keys: the A operand of the 8 channels in dwords w0, w1 (bytes =
// channels 8d..8d+7 of the lane-group's 32).  A byte at bits 0-7 of a 16-bit
// half is the fp16 subnormal c * 2^-24, so one AND (and one shift) per pair of
// channels; slot e holds channel {0,2,1,3,4,6,5,7}[e], all scaled by 2^-24.
__device__ __forceinline__ v8h key_codes8(uint32_t w0, uint32_t w1) {
    const uint4 u = {w0 & 0x00FF00FFu, (w0 >> 8) & 0x00FF00FFu, w1 & 0x00FF00FFu, (w1 >> 8) & 0x00FF00FFu};
    return __builtin_bit_cast(v8h, u);
}

// 3-bit keys: the A operand of k-step d (0..3) from the lane's three
// bit-plane words (bit x of word p = bit p of the code of channel 32g + x).
// Dword k holds channel x = 8 (d >> 1) + j, j = 4 (d & 1) + k, in its low
// half and channel x + 16 in its high half, each code at mantissa bits
// j..j+2: the fp16 subnormal c * 2^(j - 24).  Planes 1 and 2 are shifted up
// by 1 and 2 first, so a code takes one AND and two AND-ORs per pair of
// channels.  The query operand carries the matching order and 2^-j.
__device__ __forceinline__ v8h key_codes3(const uint32_t (&pl)[3], int d) {
    const int sh = 8 * (d >> 1);
    const uint32_t a = pl[0] >> sh, b = (pl[1] >> sh) << 1, c = (pl[2] >> sh) << 2;
    uint32_t u[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const int j = 4 * (d & 1) + k;
        const uint32_t m = (1u << j) | (1u << (16 + j));
        u[k] = (a & m) | (b & (m << 1)) | (c & (m << 2));
    }
    return __builtin_bit_cast(v8h, make_uint4(u[0], u[1], u[2], u[3]));
}

// Key-code A operand of k-step q (32 channels) of one page.
template <int KB, int VB>
__device__ __forceinline__ v8h key_operand(const PageRegs<KB, VB> &r, int q) {
    if (KB == 3) {
        const uint32_t pl[3] = {r.k[0], r.k[1 % KB], r.k[2 % KB]};
        return key_codes3(pl, q);
    }
    return KB == 4 ? key_codes(r.k[q]) : key_codes8(r.k[(2 * q) % KB], r.k[(2 * q + 1) % KB]);
}

// Code-domain dot products of the lane's 4 tokens (4g..4g+3) of one page:
// v_mfma_f32_16x16x32_f16 x 4 (32 channels per instruction and lane-group),
// columns n < 8 the fp16 query q_hi of head n, columns n >= 8 its residual
// q_lo = q' - q_hi.  Adding the partner column (lane n ^ 8, one DPP move)
// gives the full dot q' . c of head n & 7.
template <int KB, int VB>
__device__ __forceinline__ v4f page_dots(const PageRegs<KB, VB> &r, const v8h (&bq)[4]) {
    v4f d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int q = 0; q < 4; q++) d = __builtin_amdgcn_mfma_f32_16x16x32_f16(key_operand<KB, VB>(r, q), bq[q], d, 0, 0, 0);
    return d;
}

// Value-code A operands of one page for one lane: u = two 16-bit words
// (token slots 4g+i, 4g+i+1 for i = 0 or 2), crumb j of a word at bits
// 2j..2j+1.  Each output dword is a pair of fp16 subnormals holding crumb j
// of both words at mantissa bits 4-5 (value c * 2^-20: j = 2, 5), 6-7
// (c * 2^-18: j = 0, 3, 6) or 8-9 (c * 2^-16: j = 1, 4, 7); crumbs 3 and 4
// are in place, and one shift each way (<< 6, >> 6) serves the other six.
// The codes sit that high because the MFMA accumulates very small products
// with less than fp32 precision (codes at bits 0-1 lost up to ~3e-5
// relative, biased towards zero; at bits 4-9 the output error stays below
// 3e-5 absolute at 16K tokens).  The left shift only spills low-word bits
// into bits 16-21 and the right shift high-word bits into bits 10-15; both
// lie outside the masks.
__device__ __forceinline__ uint32_t value_code(uint32_t u, int j) {
    constexpr uint32_t kBits45 = 0x00300030u, kBits67 = 0x00C000C0u, kBits89 = 0x03000300u;
    switch (j) {
    case 0: return (u << 6) & kBits67;
    case 1: return (u << 6) & kBits89;
    case 2: return u & kBits45;
    case 3: return u & kBits67;
    case 4: return u & kBits89;
    case 5: return (u >> 6) & kBits45;
    case 6: return (u >> 6) & kBits67;
    default: return (u >> 6) & kBits89;
    }
}

// log2 of the factor that removes the code scaling of channel block j
__device__ __forceinline__ constexpr int value_unscale_log2(int j) {
    return (j == 2 || j == 5) ? 20 : (j == 0 || j == 3 || j == 6) ? 18 : 16;
}

// 4-bit values: u = one 32-bit word of the layout, the 16-bit word of the
// lane's channel m for token slots (i, i + 1) of a quad (low, high half), each
// holding the codes of channel blocks 4h..4h+3 in nibbles k = 0..3.  Returns
// nibble k of both halves at mantissa bits 4-7: the fp16 subnormals
// c * 2^-20.  Shifted-in bits of the other half fall outside the mask.
__device__ __forceinline__ uint32_t value_code4(uint32_t u, int k) {
    constexpr uint32_t kBits47 = 0x00F000F0u;
    switch (k) {
    case 0: return (u << 4) & kBits47;
    case 1: return u & kBits47;
    case 2: return (u >> 4) & kBits47;
    default: return (u >> 8) & kBits47;
    }
}

// 3-bit values: the three bit-plane words of one page for one lane (quad g,
// channel m; byte (0, 2, 1, 3)[i] of word p holds bit p of the codes of
// token slot i, channel block j at bit j).  Returns the dword of channel
// block j for token slots 0, 1 (hi = 0) or 2, 3 (hi = 1), each code at
// mantissa bits pos..pos+2 with pos = 4 + (j & 3): the fp16 subnormal
// c * 2^(pos - 24).  Each plane is shifted so that block j's bit of both
// slots lands at pos + p and pos + p + 16; then one AND and two AND-ORs.
__device__ __forceinline__ uint32_t value_code3(const uint32_t (&w)[3], int j, int hi) {
    const int pos = 4 + (j & 3);
    uint32_t x[3];
#pragma unroll
    for (int p = 0; p < 3; p++) {
        // the slot's byte (0 or 2 for slots 0/1, 1 or 3 for slots 2/3) has
        // block j at bit j (+ 8 for slots 2/3); move it to pos + p
        const int from = j + (hi ? 8 : 0);
        const int to = pos + p;
        x[p] = to >= from ? (w[p] << (to - from)) : (w[p] >> (from - to));
    }
    const uint32_t m = (1u << pos) | (1u << (16 + pos));
    return (x[0] & m) | (x[1] & (m << 1)) | (x[2] & (m << 2));
}

// log2 of the factor that removes the code scaling of channel block j (3 bits)
__device__ __forceinline__ constexpr int value3_unscale_log2(int j) { return 20 - (j & 3); }

struct LaneConsts {
    float c1, c2;          // folded score constants of head n & 7
    bool hb;               // lane n >= 8 (weights page B's tokens; n < 8: page A's)
};

// Value-code A operand of channel block j for the page pair: tokens 4g,
// 4g+1 | 4g+2, 4g+3 of page A, then of page B.
template <int KB, int VB>
__device__ __forceinline__ v8h value_operand(const PageRegs<KB, VB> &A, const PageRegs<KB, VB> &B, int j) {
    uint4 packed;
    if (VB == 2) {
        packed = {value_code(A.v[0], j), value_code(A.v[1], j), value_code(B.v[0], j), value_code(B.v[1], j)};
    } else if (VB == 3) {
        const uint32_t wa[3] = {A.v[0], A.v[1 % VB], A.v[2 % VB]};
        const uint32_t wb[3] = {B.v[0], B.v[1 % VB], B.v[2 % VB]};
        packed = {value_code3(wa, j, 0), value_code3(wa, j, 1), value_code3(wb, j, 0), value_code3(wb, j, 1)};
    } else {
        const int h = j >> 2, k = j & 3;
        packed = {value_code4(A.v[h], k), value_code4(A.v[(2 + h) % VB], k), value_code4(B.v[h], k),
                  value_code4(B.v[(2 + h) % VB], k)};
    }
    return __builtin_bit_cast(v8h, packed);
}

// Softmax weights of one page pair for one head group, from the code-domain
// dot products dA, dB of its pages.  kMasked: tokens at or beyond this lane's limit `lim` (the
// tokens its query row sees; page A starts at token tokA, page B at tokB;
// tokB >= every limit marks an absent page B) take no weight, whatever their
// (possibly never written) slots hold.  kFirst: the wave's first pair, which
// always sets the running maximum (-inf for a column that sees none of its
// tokens, which is then also the wave's last pair).
//
// Scores are formed relative to the reference mref = m + 8 (m the running
// maximum; 0 before the first pair), so the weights are exp2 of them
// directly.  When a score exceeds the reference (some logit beats m by more
// than 8), the state is rescaled and the scores shifted to the new reference.
//
// Lanes n and n ^ 8 hold the same tokens of the same head (the query's two
// fp16 terms sit in their columns), so the per-token softmax work is split
// between them: lane n < 8 folds, weights and sums page A's 4 tokens, lane
// n + 8 page B's.  Each lane turns its weights w into w_hi = fp16(w) and
// w_lo = fp16(w - w_hi); one bank-masked DPP move per dword then hands the
// partner the half it lacks, so that column n < 8 again holds w_hi and
// column n + 8 w_lo for all 8 tokens.  l and zacc are per-lane halves,
// added across the pair before the merge.
template <int KB, int VB, bool kMasked, bool kFirst>
__device__ __forceinline__ v8h pair_weights(const PageRegs<KB, VB> &A, const PageRegs<KB, VB> &B, const v4f &dA,
                                            const v4f &dB, int tokA, int tokB, int lim, const LaneConsts &lc, float c2,
                                            float woff, int g, State &st) {
    constexpr bool first = kFirst;
    const bool hb = lc.hb;
    const float mref = first ? 0.0f : st.m + kLazyThreshold;
    const uint32_t kmA[4] = {A.km.x, A.km.y, A.km.z, A.km.w}, kmB[4] = {B.km.x, B.km.y, B.km.z, B.km.w};
    const uint32_t vmA[4] = {A.vm.x, A.vm.y, A.vm.z, A.vm.w}, vmB[4] = {B.vm.x, B.vm.y, B.vm.z, B.vm.w};
    float lg[4];
    bool valid[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const float sA = dA[i] + row_swap8(dA[i]);     // q_hi . c + q_lo . c
        const float sB = dB[i] + row_swap8(dB[i]);
        const float dot = (hb ? sB : sA) - woff;
        const uint32_t km = hb ? kmB[i] : kmA[i];
        const float ks = half_bits_to_float(km & 0xffffu);
        const float kz = half_bits_to_float(km >> 16);
        lg[i] = __builtin_fmaf(dot * lc.c1, ks, __builtin_fmaf(c2, kz, -mref));
        if (kMasked) {
            valid[i] = (hb ? tokB : tokA) + 4 * g + i < lim;
            lg[i] = valid[i] ? lg[i] : -INFINITY;
        }
    }
    float lmax = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
    if (first || __any(lmax > 0.0f)) {
        float cm = fmaxf(lmax, row_swap8(lmax));
        cm = fmaxf(cm, xor_lane(cm, 16));
        cm = fmaxf(cm, xor_lane(cm, 32));
        const float m_new = first ? cm : fmaxf(st.m, cm + mref);
        const float f = first ? 0.0f : fast_exp2(st.m - m_new);
        st.l *= f;
        st.z *= f;
#pragma unroll
        for (int j = 0; j < 8; j++) st.acc[j] *= f;
        st.m = m_new;
        const float shift = (kMasked && first && m_new == -INFINITY) ? 0.0f : (m_new + kLazyThreshold) - mref;
#pragma unroll
        for (int i = 0; i < 4; i++) lg[i] -= shift;
    }
    // Weights are exp2(l - m - 8) <= 1 (the lazy threshold is folded into the
    // exponent), so w = p * s_v <= s_v stays inside fp16 for any value scale
    // the format can store; l and zacc carry the same factor, which cancels.
    _Float16 wh[4], wl[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const float p = fast_exp2(lg[i]);
        const uint32_t vm = hb ? vmB[i] : vmA[i];
        const float vs = half_bits_to_float(vm & 0xffffu);
        const float vz = half_bits_to_float(vm >> 16);
        st.l += p;
        // w = p s_v as fp16 plus the residual fl(p s_v - fp16(w)): the value
        // sum is carried to ~2^-22
        _Float16 h = (_Float16)__builtin_fmaf(p, vs, 0.0f);
        _Float16 r = (_Float16)__builtin_fmaf(p, vs, -(float)h);
        if (kMasked) {
            st.z += valid[i] ? p * vz : 0.0f;
            h = valid[i] ? h : (_Float16)0.0f;
            r = valid[i] ? r : (_Float16)0.0f;
        } else {
            st.z = __builtin_fmaf(p, vz, st.z);
        }
        wh[i] = h;
        wl[i] = r;
    }
    const int own_hi[2] = {__builtin_bit_cast(int, v2h{wh[0], wh[1]}), __builtin_bit_cast(int, v2h{wh[2], wh[3]})};
    const int own_lo[2] = {__builtin_bit_cast(int, v2h{wl[0], wl[1]}), __builtin_bit_cast(int, v2h{wl[2], wl[3]})};
    // page A's dwords: lanes n + 8 (banks 2, 3 of a row) take w_lo from lane
    // n; page B's: lanes n < 8 (banks 0, 1) take w_hi from lane n + 8
    uint4 bwu;
    bwu.x = (uint32_t)__builtin_amdgcn_update_dpp(own_hi[0], own_lo[0], 0x128, 0xF, 0xC, false);
    bwu.y = (uint32_t)__builtin_amdgcn_update_dpp(own_hi[1], own_lo[1], 0x128, 0xF, 0xC, false);
    bwu.z = (uint32_t)__builtin_amdgcn_update_dpp(own_lo[0], own_hi[0], 0x128, 0xF, 0x3, false);
    bwu.w = (uint32_t)__builtin_amdgcn_update_dpp(own_lo[1], own_hi[1], 0x128, 0xF, 0x3, false);
    return __builtin_bit_cast(v8h, bwu);
}

// Code-domain dot products of one page pair for kG head groups: the score
// MFMAs (4 per page and group).  With kG = 2 each k-step's key operands feed
// both groups' MFMAs as they are unpacked, so that only one operand per page
// is live at a time.
template <int KB, int VB, int kG>
__device__ __forceinline__ void pair_dots(const PageRegs<KB, VB> &A, const PageRegs<KB, VB> &B,
                                          const v8h (&bq)[kG][4], v4f (&dA)[kG], v4f (&dB)[kG]) {
    if constexpr (kG == 1) {
        dA[0] = page_dots<KB, VB>(A, bq[0]);
        dB[0] = page_dots<KB, VB>(B, bq[0]);
    } else {
#pragma unroll
        for (int h = 0; h < kG; h++) dA[h] = dB[h] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const v8h ka = key_operand<KB, VB>(A, q);
            const v8h kb = key_operand<KB, VB>(B, q);
#pragma unroll
            for (int h = 0; h < kG; h++) {
                dA[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, bq[h][q], dA[h], 0, 0, 0);
                dB[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kb, bq[h][q], dB[h], 0, 0, 0);
            }
        }
    }
}

// The rest of a page pair once its dot products dA, dB are known: softmax
// weights, then the P.V MFMAs (8 per group); the value operands are unpacked
// once and feed every group.  Each group keeps its own softmax state.
// lim[h]: group h's token limit (kMasked).
// c2[h]: the coefficient of the key offset z in group h's scores for this
// lane's page (the query sum times the score scale); woff[h]: subtracted
// from the lane's dot products first (0 but for page-balanced keys).
template <int KB, int VB, int kG, bool kMasked, bool kFirst>
__device__ __forceinline__ void pair_finish(const PageRegs<KB, VB> &A, const PageRegs<KB, VB> &B,
                                            const v4f (&dA)[kG], const v4f (&dB)[kG], int tokA, int tokB,
                                            const int (&lim)[kG], const LaneConsts (&lc)[kG], const float (&c2)[kG],
                                            const float (&woff)[kG], int g, State (&st)[kG]) {
    v8h bw[kG];
#pragma unroll
    for (int h = 0; h < kG; h++)
        bw[h] = pair_weights<KB, VB, kMasked, kFirst>(A, B, dA[h], dB[h], tokA, tokB, lim[h], lc[h], c2[h], woff[h],
                                                      g, st[h]);
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const v8h av = value_operand<KB, VB>(A, B, j);
#pragma unroll
        for (int h = 0; h < kG; h++)
            st[h].acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bw[h], st[h].acc[j], 0, 0, 0);
    }
}

// One page pair for kG head groups of 8 query heads (kG = 2: 16 heads, when
// a KV head has more than 8 query heads or query rows): the key and value
// operands are unpacked once and feed every group's MFMAs.
template <int KB, int VB, int kG, bool kMasked, bool kFirst>
__device__ __forceinline__ void process_pair(const PageRegs<KB, VB> &A, const PageRegs<KB, VB> &B, int tokA,
                                             int tokB, const int (&lim)[kG], const v8h (&bq)[kG][4],
                                             const LaneConsts (&lc)[kG], int g, State (&st)[kG]) {
    v4f dA[kG], dB[kG];
    pair_dots<KB, VB, kG>(A, B, bq, dA, dB);
    float c2[kG], woff[kG];
#pragma unroll
    for (int h = 0; h < kG; h++) {
        c2[h] = lc[h].c2;
        woff[h] = 0.0f;
    }
    pair_finish<KB, VB, kG, kMasked, kFirst>(A, B, dA, dB, tokA, tokB, lim, lc, c2, woff, g, st);
}

// ---- page-balanced keys ----
// A page's key channel j carries the column scale 2^e_j, stored as the high
// byte of its fp16 bit pattern at 1664 + j.  The key operand carries it: the
// A element of (token t, channel j) is the fp16 number 2^e_j (1 + c_tj / 16),
// its bits the scale's bits OR the code at mantissa bits 6-9 (one shift and
// one AND-OR per pair of channels, as many instructions as key_codes).  With
// D'_t = sum_j a_tj q''_j and W = sum_j 2^e_j q''_j (the same MFMA against the
// scales alone), sum_j q''_j 2^e_j c_tj = 16 (D'_t - W): the score of token t
// is c1 (s_t (D'_t - W) + z_t W / 16), c1 = alpha 2^(4 - shift).  The products
// are normal fp16 products, so the MFMA keeps the precision of the per-token
// format (an earlier form that scaled the query by 2^e_j per page and kept the
// codes as subnormals lost up to 40x more against the fp64 definition: the
// MFMA keeps fewer bits of very small products), and the query needs no
// per-page scaling.

// The 32 scale bytes of lane group g (channels 32g .. 32g + 31), as loaded.
struct PageScales {
    uint32_t w[8];
};
struct NoScales {};

__device__ __forceinline__ void load_scales(const uint8_t *region, int g, PageScales &s, bool live) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(region), (short)0, live ? kRegionPB : 0, 0x00020000);
    const v4u lo = __builtin_amdgcn_raw_buffer_load_b128(rs, kScalesPB + 32 * g, 0, 0);
    const v4u hi = __builtin_amdgcn_raw_buffer_load_b128(rs, kScalesPB + 32 * g + 16, 0, 0);
    s.w[0] = lo.x; s.w[1] = lo.y; s.w[2] = lo.z; s.w[3] = lo.w;
    s.w[4] = hi.x; s.w[5] = hi.y; s.w[6] = hi.z; s.w[7] = hi.w;
}

// The scales 2^e as fp16 in the key operand's slot order: slot pair k of
// k-step d (k = 0..3) holds channels 8d + k and 8d + 4 + k (see key_codes),
// i.e. byte k of dword 2d and of dword 2d + 1 of the scale bytes, each moved
// to the high byte of its half by one byte permute.
__device__ __forceinline__ uint4 scale_words(const PageScales &s, int d) {
    const uint32_t lo = s.w[2 * d], hi = s.w[2 * d + 1];
    return uint4{__builtin_amdgcn_perm(hi, lo, 0x040c000cu), __builtin_amdgcn_perm(hi, lo, 0x050c010cu),
                 __builtin_amdgcn_perm(hi, lo, 0x060c020cu), __builtin_amdgcn_perm(hi, lo, 0x070c030cu)};
}

// D' (rows: tokens 4g..4g+3 of column n) and W (of column n's head, both
// query terms) of one page for kG head groups.
template <int kG>
__device__ __forceinline__ void page_dots_pb(const PageRegs<4, 2> &r, const PageScales &sc, const v8h (&bq)[kG][4],
                                             v4f (&d)[kG], float (&w)[kG]) {
    constexpr uint32_t kBits69 = 0x03C003C0u;
    v4f wv[kG];
#pragma unroll
    for (int h = 0; h < kG; h++) d[h] = wv[h] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const uint4 m = scale_words(sc, q);
        const uint32_t x = r.k[q];
        const uint4 a = {((x << 6) & kBits69) | m.x, ((x << 2) & kBits69) | m.y, ((x >> 2) & kBits69) | m.z,
                         ((x >> 6) & kBits69) | m.w};
#pragma unroll
        for (int h = 0; h < kG; h++) {
            d[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a), bq[h][q], d[h], 0, 0, 0);
            wv[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, m), bq[h][q], wv[h], 0, 0, 0);
        }
    }
#pragma unroll
    for (int h = 0; h < kG; h++) w[h] = wv[h][0] + row_swap8(wv[h][0]);   // every row holds W
}

// One page pair with page-balanced keys (K4V2).
template <int kG, bool kMasked, bool kFirst>
__device__ __forceinline__ void process_pair_pb(const PageRegs<4, 2> &A, const PageRegs<4, 2> &B,
                                                const PageScales &SA, const PageScales &SB, int tokA, int tokB,
                                                const int (&lim)[kG], const v8h (&bq)[kG][4],
                                                const LaneConsts (&lc)[kG], int g, State (&st)[kG]) {
    v4f dA[kG], dB[kG];
    float wa[kG], wb[kG], c2[kG], woff[kG];
    page_dots_pb<kG>(A, SA, bq, dA, wa);
    page_dots_pb<kG>(B, SB, bq, dB, wb);
#pragma unroll
    for (int h = 0; h < kG; h++) {
        woff[h] = lc[h].hb ? wb[h] : wa[h];
        c2[h] = lc[h].c1 * 0.0625f * woff[h];
    }
    pair_finish<4, 2, kG, kMasked, kFirst>(A, B, dA, dB, tokA, tokB, lim, lc, c2, woff, g, st);
}

// One page pair of either key normalisation (Scales: PageScales with
// page-balanced keys, else NoScales, unused).
template <int KB, int VB, int kG, bool kMasked, bool kFirst, bool kPB, typename Scales>
__device__ __forceinline__ void run_pair(const PageRegs<KB, VB> &A, const PageRegs<KB, VB> &B, const Scales &SA,
                                         const Scales &SB, int tokA, int tokB, const int (&lim)[kG],
                                         const v8h (&bq)[kG][4], const LaneConsts (&lc)[kG], int g,
                                         State (&st)[kG]) {
    if constexpr (kPB)
        process_pair_pb<kG, kMasked, kFirst>(A, B, SA, SB, tokA, tokB, lim, bq, lc, g, st);
    else
        process_pair<KB, VB, kG, kMasked, kFirst>(A, B, tokA, tokB, lim, bq, lc, g, st);
}

// Issue priority of this wave from the page pairs it has left (wave-uniform):
// two waves of different work-groups share each SIMD, and the older one wins
// the issue arbitration by default, so that it finishes first and the other
// runs its last pairs alone (per-wave timestamps showed one work-group of
// every compute unit ending ~4 us after the other).  With the priority
// falling over a wave's last three pairs, the wave with more work left is
// issued first and the two finish together (measured: 2-3% less time per
// launch).
__device__ __forceinline__ void set_priority(int left) {
    if (left >= 3) __builtin_amdgcn_s_setprio(3);
    else if (left == 2) __builtin_amdgcn_s_setprio(2);
    else if (left == 1) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
}

// kG: head groups (of 8 query heads, or (row, head) pairs) per work-group;
// 2 when a KV head has more than 8, so that they share the page unpack.
// kPB: page-balanced keys (K4V2, one query row, 16-token pages; 1792-byte
// regions whose column scales are folded into the query per page).
template <int KB, int VB, bool kMQ, bool kPaged, int kG, bool kPB = false>
__global__ __launch_bounds__(64 * kDecodeWaves, 2) void decode_kernel(DecodeArgs a) {
    static_assert(!kPB || (KB == 4 && VB == 2 && !kMQ && !kPaged), "page-balanced keys: K4V2, one row, 16-token pages");
    using Lay = Layout<KB, VB>;
    using Scales = typename std::conditional<kPB, PageScales, NoScales>::type;
    constexpr int kRegion = kPB ? kRegionPB : Lay::kBytes;   // bytes of one (16-token page, KV head)
    const int sgroups = (a.head_groups + kG - 1) / kG;   // work-groups per (split, KV head, sequence)
    int split, kvh, sg, b;
    if (!kMQ) {
        split = blockIdx.x;
        kvh = blockIdx.y / sgroups;
        sg = blockIdx.y % sgroups;
        b = blockIdx.z;
    } else {
        // One-dimensional grid, XCD-aware: work-groups are dispatched to the 8
        // XCDs in turn, so block L runs on XCD L % 8.  The work-groups of one
        // (split, sequence, KV head) take consecutive blocks of one XCD and
        // read the same pages at about the same time: the later reads are
        // served by that XCD's L2.  Blocks past the work (the grid is padded
        // to whole rounds) exit at once.
        const int L = blockIdx.x;
        sg = (L >> 3) % sgroups;
        const int64_t w = (int64_t)((L >> 3) / sgroups) * 8 + (L & 7);
        const int64_t units = (int64_t)a.splits * a.num_kv_heads * a.num_seqs;
        if (w >= units) return;
        split = (int)(w % a.splits);
        kvh = (int)((w / a.splits) % a.num_kv_heads);
        b = (int)(w / ((int64_t)a.splits * a.num_kv_heads));
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // Page ids of this wave's page pairs, one pair per lane: lane j holds the
    // block-table entries of pages 2k and 2k + 1 of the split, k = wave + W j
    // with W = kDecodeWaves (a split has at most 512 pages, so j < 64 for
    // W >= 4; indices are clamped into the
    // row, and entries past the split or the sequence are never used).  One
    // vector load at the start replaces a scalar load and wait per pair; the
    // pair loop reads the ids with v_readlane.
    const int32_t *bt = a.block_tables + (int64_t)b * a.bt_stride;
    int32_t bt_a, bt_b;
    {
        const int last = a.bt_stride - 1;
        const int pa = split * a.pages_per_split + 2 * (wave + kDecodeWaves * lane);
        // with pages of several 16-token regions, entry pa >> log2s holds region pa
        const int ea = kPaged ? pa >> a.page_log2s : pa;
        const int eb = kPaged ? (pa + 1) >> a.page_log2s : pa + 1;
        bt_a = bt[ea < last ? ea : last];
        bt_b = bt[eb < last ? eb : last];
    }
    // This lane's slice of the query (head 2 wave + lane / 32 of the head
    // group, channels 4 (lane % 32) ..+3) is requested with the page ids,
    // before any page: loads return in issue order, so a query load issued
    // after the first pages would hold the query prologue until those pages
    // had arrived (measured: the prologue then ended ~4.4 us after the wave
    // started, against ~1 us for the page ids).
    const int hg0 = sg * kG;                 // first head group of this work-group
    int nh[kG];                              // heads of each group (0: a padding group)
    uint2 qraw[kG];
#pragma unroll
    for (int h = 0; h < kG; h++) {
        nh[h] = max(0, min(kHeadsPerGroup, a.gqa - (hg0 + h) * kHeadsPerGroup));
        qraw[h] = make_uint2(0u, 0u);
        const int hh = 2 * wave + (lane >> 5);
        if (hh < nh[h])
            qraw[h] = *reinterpret_cast<const uint2 *>(
                a.query + io_row<kMQ>(a, b, kvh, (hg0 + h) * kHeadsPerGroup + hh) * kHeadDim + 4 * (lane & 31));
    }

    const int max_len = a.max_seq_len;
    int n_tokens = a.seq_lens[b];
    n_tokens = n_tokens < 0 ? 0 : (n_tokens > max_len ? max_len : n_tokens);
    // query rows per sequence (kMQ; at most 16); row m sees tokens below
    // n_tokens - (M - 1 - m), so every row sees the first n_min (at least one
    // token when there is one)
    const int M = kMQ ? a.q_len : 1;
    const int n_min = kMQ ? max(min(n_tokens, 1), n_tokens - (M - 1)) : n_tokens;
    const int npages = (n_tokens + kPage - 1) / kPage;
    const int pps = a.pages_per_split;
    const int p_begin = split * pps;

    if (p_begin >= npages) {         // an empty sequence, or a split past its end
#pragma unroll
        for (int h = 0; h < kG; h++)
            if (nh[h] > 0) write_empty<kMQ>(a, tid, b, kvh, (hg0 + h) * kHeadsPerGroup, nh[h], split);
        return;
    }
    const int p_end = min(p_begin + pps, npages);

    __shared__ _Float16 s_qb[kG][16][kHeadDim];   // [group][column][slot], slot = 32g + 8d + e
    __shared__ float s_c1[kG][kHeadsPerGroup], s_c2[kG][kHeadsPerGroup];
    __shared__ MergeLdsT<kDecodeWaves> s_merge;

    // ---- page-pair loop ----
    const int npairs = (p_end - p_begin + 1) >> 1;
    const int log2s = kPaged ? a.page_log2s : 0;
    const int64_t head_off = ((int64_t)kvh * kRegion) << log2s;
    const int64_t page_stride = ((int64_t)a.num_kv_heads * kRegion) << log2s;
    const int sub_mask = (1 << log2s) - 1;

    // A page id outside the pool is read as page 0: never an out-of-bounds
    // access (the output is unspecified under that precondition violation).
    const LaneOffsets<KB, VB> lo(lane);
    const uint32_t num_pages32 = a.num_pages < 0x7fffffff ? (uint32_t)a.num_pages : 0x7fffffffu;
    // region of 16-token page pa (of the sequence) in block-table page page_id
    auto region_of = [&](int32_t page_id, int pa) -> const uint8_t * {
        uint32_t id = (uint32_t)page_id;
        if (id >= num_pages32) id = 0;           // also catches negative ids
        const uint8_t *r = a.cache + (int64_t)id * page_stride + head_off;
        return kPaged ? r + (int64_t)(pa & sub_mask) * Lay::kBytes : r;
    };

    // Pairs of this split: the leading ones are full (both pages inside the
    // split, every token seen by every query row), the rest -- the last one
    // or two (query rows span at most 16 tokens) -- are masked.  Wave w takes
    // pairs w, w + 4, ...; full pairs run through a triple-buffered loop whose
    // loads are always issued (past the end as loads that read nothing), so
    // two pairs are in flight while one is computed.  A masked pair is
    // loaded and processed afterwards with per-token masking.
    const int full_end = min(p_end, n_min / kPage);       // pages below: full
    const int nfull = full_end > p_begin ? (full_end - p_begin) >> 1 : 0;
    const int nk = nfull > wave ? (nfull - wave + kDecodeWaves - 1) / kDecodeWaves : 0;

    // The scheduling barrier keeps the compiler from sinking the prefetch
    // loads into the next pair's arithmetic (which it otherwise does to save
    // registers, leaving the current pair's loads as the newest in flight).
    // Past the wave's last pair the loads stay in the instruction stream (so
    // that every wait count in the loop is the same on every path) but read
    // nothing: measured, 0.2 us per launch at 16K against re-reading the
    // last pair, and ~14 MB less cache traffic per launch.
    auto issue = [&](PageRegs<KB, VB> &A, PageRegs<KB, VB> &B, Scales &SA, Scales &SB, int i) {
        const int j = i < nk ? i : nk - 1;      // the wave's j-th pair: lane j of bt_a / bt_b
        const int pa = kPaged ? p_begin + 2 * (wave + kDecodeWaves * j) : 0;
        const bool live = i < nk;
        const uint8_t *ra = region_of(__builtin_amdgcn_readlane(bt_a, j), pa);
        const uint8_t *rb = region_of(__builtin_amdgcn_readlane(bt_b, j), pa + 1);
        load_page(ra, lo, A, live);
        load_page(rb, lo, B, live);
        if constexpr (kPB) {
            load_scales(ra, lane >> 4, SA, live);
            load_scales(rb, lane >> 4, SB, live);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // Fused append: a work-group whose split holds the sequence's last token
    // encodes that token (the key and the value group of its KV head) into
    // the cache before any of its waves reads the page.  With more than one
    // head group per KV head, every such work-group stores the same bytes; each
    // reads the page only after its own stores have completed.
    if (!kPB && a.append) {             // (no fused append with page-balanced keys)
        const int pos = n_tokens - 1;
        const int pnew = pos / kPage;
        if (pnew >= p_begin && pnew < p_end) {
            if (wave == 0 && lane < 32) {
                const uint32_t id = (uint32_t)bt[kPaged ? pnew >> log2s : pnew];
                if (id < num_pages32) {
                    const int is_v = lane >> 4;
                    const uint16_t *src = is_v
                        ? a.new_value + (int64_t)b * a.new_value_stride + (int64_t)kvh * kHeadDim
                        : a.new_key + (int64_t)b * a.new_key_stride + (int64_t)kvh * kHeadDim;
                    uint8_t *region = const_cast<uint8_t *>(region_of((int32_t)id, pnew));
                    encode_group_fmt<KB, VB>(src, is_v, lane & 15, region, pos % kPage);
                }
            }
            // the stores have reached L2 before any wave of the group loads
            // the page (regions are 128-byte aligned, so no other work-group
            // holds one of their cache lines)
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            __syncthreads();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        }
    }

    // The first three pairs (all three buffers) are requested before the
    // query prologue so that their HBM latency overlaps it (measured: 0.2-0.4
    // us less per launch than issuing the third after the prologue).  The
    // empty asm consumes the page ids on every path, so the wait for their
    // load is placed here and not repeated (as a wait for all loads in
    // flight) inside the pair loop.
    asm volatile("" ::"v"(bt_a), "v"(bt_b));
    PageRegs<KB, VB> r0A, r0B, r1A, r1B, r2A, r2B;
    Scales s0A, s0B, s1A, s1B, s2A, s2B;
    if (nk > 0) {
        issue(r0A, r0B, s0A, s0B, 0);
        issue(r1A, r1B, s1A, s1B, 1);
        issue(r2A, r2B, s2A, s2B, 2);
    }

    // ---- query prologue: wave w rotates and splits heads 2w and 2w+1 of each group ----
    // q' = H q in fp32, scaled by a power of two so that max |q'| lies in
    // [2^13, 2^14), then written as q_hi = fp16(q'), q_lo = fp16(q' - q_hi):
    // the two-term query carries q' to about 2^-22 of each element.  (Waves
    // past the fourth have no heads to rotate.)
#pragma unroll
    for (int hq = 0; hq < kG && 2 * wave < kHeadsPerGroup; hq++) {
        const int hh = 2 * wave + (lane >> 5);
        const int l32 = lane & 31;
        const int c0 = 4 * l32;
        float q[4];
        q[0] = half_bits_to_float(qraw[hq].x & 0xffffu);   // zero for heads past the group
        q[1] = half_bits_to_float(qraw[hq].x >> 16);
        q[2] = half_bits_to_float(qraw[hq].y & 0xffffu);
        q[3] = half_bits_to_float(qraw[hq].y >> 16);
        {
            float p = q[0], r = q[1]; q[0] = p + r; q[1] = p - r;
            p = q[2]; r = q[3]; q[2] = p + r; q[3] = p - r;
            p = q[0]; r = q[2]; q[0] = p + r; q[2] = p - r;
            p = q[1]; r = q[3]; q[1] = p + r; q[3] = p - r;
        }
#pragma unroll
        for (int x = 1; x < 32; x <<= 1) {
            const bool upper = (l32 & x) != 0;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const float other = xor_lane_dpp(q[e], x);
                q[e] = upper ? (other - q[e]) : (q[e] + other);
            }
        }
        float am = fmaxf(fmaxf(fabsf(q[0]), fabsf(q[1])), fmaxf(fabsf(q[2]), fabsf(q[3])));
        float qs = q[0] + q[1] + q[2] + q[3];
#pragma unroll
        for (int x = 1; x < 32; x <<= 1) {
            am = fmaxf(am, xor_lane_dpp(am, x));
            qs += xor_lane_dpp(qs, x);
        }
        int ex = 0;
        if (am > 0.0f) (void)frexpf(am, &ex);          // am in [2^(ex-1), 2^ex)
        const int shift = 14 - ex;                       // q' * 2^shift: max in [2^13, 2^14)
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int ch = c0 + e;
            const int r8 = ch & 7;
            // slot of channel ch in the key operand's order (see key_codes,
            // key_codes8, key_codes3) and log2 of the code scaling it
            // carries: 4-bit keys in slots 2, 3, 6, 7 carry 2^-20 (down = 4);
            // a 3-bit key at mantissa bits j..j+2 carries 2^(j - 24)
            int slot, down = 0;
            if (KB == 4) {
                slot = (ch & ~7) + (r8 < 4 ? 2 * r8 : 2 * (r8 - 4) + 1);
                down = kPB ? 0 : 4 * ((slot >> 1) & 1);   // (page-balanced keys: normal fp16 operands)
            } else if (KB == 3) {
                const int x = ch & 31, r16 = x & 15;   // channel 32g + x; x = 16 hi + r16
                slot = (ch & ~31) + 8 * (2 * (r16 >> 3) + ((r16 >> 2) & 1)) + 2 * (r16 & 3) + (x >> 4);
                down = r16 & 7;
            } else {
                slot = (ch & ~7) + ((r8 & 4) | ((r8 & 1) << 1) | ((r8 >> 1) & 1));
            }
            const float v = __builtin_ldexpf(q[e], shift - down);
            const _Float16 vh = (_Float16)v;
            s_qb[hq][hh][slot] = vh;
            s_qb[hq][8 + hh][slot] = (_Float16)(v - (float)vh);
        }
        if (l32 == 0) {
            // dot(q', c) = D * 2^(24 - shift), D the MFMA sum with codes c * 2^-24;
            // page-balanced keys: 16 (D' - W) 2^-shift (see page_dots_pb)
            s_c1[hq][hh] = a.alpha * __builtin_ldexpf(1.0f, (kPB ? 4 : 24) - shift);
            s_c2[hq][hh] = a.alpha * qs;
        }
    }
    __syncthreads();

    const int n16 = lane & 15;
    const int g = lane >> 4;
    v8h bq[kG][4];
    LaneConsts lc[kG];
    State st[kG];
    const int lim0[kG] = {};                 // unused by unmasked pairs
#pragma unroll
    for (int h = 0; h < kG; h++) {
#pragma unroll
        for (int d = 0; d < 4; d++) bq[h][d] = *reinterpret_cast<const v8h *>(&s_qb[h][n16][32 * g + 8 * d]);
        lc[h].c1 = s_c1[h][n16 & 7];
        lc[h].c2 = s_c2[h][n16 & 7];
        lc[h].hb = n16 >= 8;
        st[h].m = -INFINITY;
        st[h].l = 0.0f;
        st[h].z = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; j++) st[h].acc[j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }

    if (nk > 0) {
        // The wave's first pair sets the running maximum; the loop then
        // rotates the three buffers (pair i in r1, i + 1 in r2, i + 2 in r0).
        // Three is the measured best depth: two left the arithmetic waiting
        // for loads, four made the split kernel slower (more random reads in
        // flight lower the HBM's efficiency on 1664-byte regions; the
        // page-walk probe alone slows the same way with depth), and so did a
        // four-buffer variant that issued each pair's score MFMAs one pair
        // ahead of its softmax.
        set_priority(nk);
        run_pair<KB, VB, kG, false, true, kPB>(r0A, r0B, s0A, s0B, 0, 0, lim0, bq, lc, g, st);
        int i = 1;
        // Whole rounds of three pairs whose loads all read live pages, with
        // no exit test between the pairs (measured: 2-3% less time per
        // launch than the guarded loop below alone; with two head groups the
        // unguarded body needs more registers than the file holds, so they
        // take the guarded loop throughout).
        if constexpr (kG == 1) {
            for (; i + 4 < nk; i += 3) {
                issue(r0A, r0B, s0A, s0B, i + 2);
                run_pair<KB, VB, kG, false, false, kPB>(r1A, r1B, s1A, s1B, 0, 0, lim0, bq, lc, g, st);
                issue(r1A, r1B, s1A, s1B, i + 3);
                run_pair<KB, VB, kG, false, false, kPB>(r2A, r2B, s2A, s2B, 0, 0, lim0, bq, lc, g, st);
                issue(r2A, r2B, s2A, s2B, i + 4);
                run_pair<KB, VB, kG, false, false, kPB>(r0A, r0B, s0A, s0B, 0, 0, lim0, bq, lc, g, st);
            }
        }
        // the last pairs (and every pair with two head groups)
        for (; i < nk; i += 3) {
            set_priority(nk - i);
            issue(r0A, r0B, s0A, s0B, i + 2);
            run_pair<KB, VB, kG, false, false, kPB>(r1A, r1B, s1A, s1B, 0, 0, lim0, bq, lc, g, st);
            if (i + 1 >= nk) break;
            set_priority(nk - i - 1);
            issue(r1A, r1B, s1A, s1B, i + 3);
            run_pair<KB, VB, kG, false, false, kPB>(r2A, r2B, s2A, s2B, 0, 0, lim0, bq, lc, g, st);
            if (i + 2 >= nk) break;
            set_priority(nk - i - 2);
            issue(r2A, r2B, s2A, s2B, i + 4);
            run_pair<KB, VB, kG, false, false, kPB>(r0A, r0B, s0A, s0B, 0, 0, lim0, bq, lc, g, st);
        }
        set_priority(0);
    }
    // Masked pairs: the last pair, and with several query rows possibly the
    // one before it (each the last pair of its wave).
    auto masked_pair = [&](int i) {
        int lim[kG];                            // the tokens this lane's query row sees, per group
#pragma unroll
        for (int h = 0; h < kG; h++) {
            lim[h] = n_tokens;
            if (kMQ) {
                const int G = a.gqa / M;
                const int mrow = min(((hg0 + h) * kHeadsPerGroup + (n16 & 7)) / G, M - 1);
                lim[h] = n_tokens - (M - 1 - mrow);
            }
        }
        PageRegs<KB, VB> tA, tB;
        Scales tsA, tsB;
        const int pa = p_begin + 2 * i;
        const bool has_b = pa + 1 < p_end;
        const int j = i / kDecodeWaves;         // the pair's lane in bt_a / bt_b
        const int32_t id_a = __builtin_amdgcn_readlane(bt_a, j);
        const uint8_t *ra = region_of(id_a, pa);
        const uint8_t *rb = has_b ? region_of(__builtin_amdgcn_readlane(bt_b, j), pa + 1) : ra;
        load_page(ra, lo, tA);
        load_page(rb, lo, tB);
        if constexpr (kPB) {
            load_scales(ra, g, tsA, true);
            load_scales(rb, g, tsB, true);
        }
        const int tok_b = has_b ? (pa + 1) * kPage : n_tokens;
        if (nk == 0)
            run_pair<KB, VB, kG, true, true, kPB>(tA, tB, tsA, tsB, pa * kPage, tok_b, lim, bq, lc, g, st);
        else
            run_pair<KB, VB, kG, true, false, kPB>(tA, tB, tsA, tsB, pa * kPage, tok_b, lim, bq, lc, g, st);
    };
    if (nfull < npairs && wave == (npairs - 1) % kDecodeWaves) masked_pair(npairs - 1);
    if (kMQ && nfull + 1 < npairs && wave == (npairs - 2) % kDecodeWaves) masked_pair(npairs - 2);

    // ---- merge the 4 waves; write the partial (or the output) ----
#pragma unroll
    for (int h = 0; h < kG; h++) {
        st[h].l += row_swap8(st[h].l);     // the two halves of the lane pair's tokens
        st[h].z += row_swap8(st[h].z);
        if (h > 0) __syncthreads();        // the previous group's merge has read s_merge
        merge_and_store<kMQ>(st[h], s_merge, a, 1,
                        [](int j) {
                            return __builtin_ldexpf(1.0f, VB == 2 ? value_unscale_log2(j) : VB == 3 ? value3_unscale_log2(j) : 20);
                        },
                        wave, tid, b, kvh, (hg0 + h) * kHeadsPerGroup, nh[h], split);
    }
}

// Merge the split partials of each (sequence, query head) and apply the
// Hadamard epilogue.  Runs after decode_kernel on the same stream (the kernel
// boundary makes every partial visible).  Each wave handles two rows, 32
// lanes per row, 4 channels per lane.  The kernel is latency-bound, so every
// lane requests the (m, l, zacc) words and its 4 channels of up to 8 splits
// at once (one memory round trip) and merges them in-lane; longer rows take
// further groups of 8 with a running maximum.  A work-group is one wave, so
// that the rows spread over as many compute units as possible (measured:
// 0.6 us less per decode step than 4-wave work-groups on the 512 rows of the
// 16K, 64-head workload).
__global__ __launch_bounds__(64) void combine_kernel(DecodeArgs a) {
    constexpr int kChunk = 8;
    const int lane = threadIdx.x & 63;
    const int l32 = lane & 31;
    const int64_t row = (int64_t)blockIdx.x * 2 + (lane >> 5);
    if (row >= (int64_t)a.num_seqs * a.num_q_heads) return;
    // Every split slot of every row holds a partial (empty ones: m = -inf,
    // l = 0), so the merge needs no sequence lengths; a row with no tokens
    // ends with l = 0 and a zero output.
    const int nsplit = a.slot_stride;
    const float *base = a.partials + row * a.slot_stride * kPartialFloats;
    const int c0 = 4 * l32;
    float M = -INFINITY, l = 0.0f, z = 0.0f;
    float o4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = 0; s0 < nsplit; s0 += kChunk) {
        float4 meta[kChunk], v[kChunk];
#pragma unroll
        for (int u = 0; u < kChunk; u++) {
            const int sp = s0 + u < nsplit ? s0 + u : nsplit - 1;   // in range; duplicates get weight 0
            meta[u] = *reinterpret_cast<const float4 *>(base + sp * kPartialFloats);
            v[u] = *reinterpret_cast<const float4 *>(base + sp * kPartialFloats + 4 + c0);
        }
        float mc = M;
#pragma unroll
        for (int u = 0; u < kChunk; u++) mc = s0 + u < nsplit ? fmaxf(mc, meta[u].x) : mc;
        if (mc != M) {                   // rescale what earlier groups accumulated
            const float f = M == -INFINITY ? 0.0f : fast_exp2(M - mc);
            l *= f;
            z *= f;
#pragma unroll
            for (int e = 0; e < 4; e++) o4[e] *= f;
            M = mc;
        }
#pragma unroll
        for (int u = 0; u < kChunk; u++) {
            const bool live = s0 + u < nsplit && meta[u].x != -INFINITY;
            const float f = live ? fast_exp2(meta[u].x - M) : 0.0f;
            l += f * meta[u].y;
            z += f * meta[u].z;
            o4[0] += f * v[u].x;
            o4[1] += f * v[u].y;
            o4[2] += f * v[u].z;
            o4[3] += f * v[u].w;
        }
    }
    // output row: with several query rows per sequence, the combine's rows
    // are (sequence, KV head, row-head pair) and the output is [B][q_len][Hq]
    int64_t orow = row;
    if (a.q_len > 1) {
        const int bb = (int)(row / a.num_q_heads), v = (int)(row % a.num_q_heads);
        orow = io_row<true>(a, bb, v / a.gqa, v % a.gqa);
    }
    finalize_head(o4, l, z, l32, a.out, a.out_f32, orow, a.rotated);
}

// The combine for rows of many split slots (more than 8): one work-group per
// row; thread (g, c) with split group g = tid / 32 and channel quad c merges
// splits g, g + 8, g + 16, ... (issuing every load at once: one memory round
// trip, where the row-per-32-lanes kernel above takes one per 8 splits), then
// the 8 split groups merge in LDS and group 0 applies the epilogue.
constexpr int kWideGroups = 8;
constexpr int kWideMaxPerGroup = 8;   // up to 64 slots in one round

__global__ __launch_bounds__(256) void combine_wide_kernel(DecodeArgs a) {
    const int tid = threadIdx.x;
    const int l32 = tid & 31;
    const int grp = tid >> 5;
    const int64_t row = blockIdx.x;
    const int nsplit = a.slot_stride;
    const float *base = a.partials + row * a.slot_stride * kPartialFloats;
    const int c0 = 4 * l32;
    float M = -INFINITY, l = 0.0f, z = 0.0f;
    float o4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = grp; s0 < nsplit; s0 += kWideGroups * kWideMaxPerGroup) {
        float4 meta[kWideMaxPerGroup], v[kWideMaxPerGroup];
#pragma unroll
        for (int u = 0; u < kWideMaxPerGroup; u++) {
            const int sp0 = s0 + u * kWideGroups;
            const int sp = sp0 < nsplit ? sp0 : grp;    // in range; duplicates get weight 0
            meta[u] = *reinterpret_cast<const float4 *>(base + sp * kPartialFloats);
            v[u] = *reinterpret_cast<const float4 *>(base + sp * kPartialFloats + 4 + c0);
        }
        float mc = M;
#pragma unroll
        for (int u = 0; u < kWideMaxPerGroup; u++)
            mc = s0 + u * kWideGroups < nsplit ? fmaxf(mc, meta[u].x) : mc;
        if (mc != M) {
            const float f = M == -INFINITY ? 0.0f : fast_exp2(M - mc);
            l *= f;
            z *= f;
#pragma unroll
            for (int e = 0; e < 4; e++) o4[e] *= f;
            M = mc;
        }
#pragma unroll
        for (int u = 0; u < kWideMaxPerGroup; u++) {
            const bool live = s0 + u * kWideGroups < nsplit && meta[u].x != -INFINITY;
            const float f = live ? fast_exp2(meta[u].x - M) : 0.0f;
            l += f * meta[u].y;
            z += f * meta[u].z;
            o4[0] += f * v[u].x;
            o4[1] += f * v[u].y;
            o4[2] += f * v[u].z;
            o4[3] += f * v[u].w;
        }
    }
    __shared__ float s_m[kWideGroups], s_l[kWideGroups], s_z[kWideGroups];
    __shared__ float s_acc[kWideGroups][kHeadDim];
    if (l32 == 0) {
        s_m[grp] = M;
        s_l[grp] = l;
        s_z[grp] = z;
    }
    *reinterpret_cast<float4 *>(&s_acc[grp][c0]) = make_float4(o4[0], o4[1], o4[2], o4[3]);
    __syncthreads();
    if (grp != 0) return;
    float Mt = -INFINITY;
#pragma unroll
    for (int g2 = 0; g2 < kWideGroups; g2++) Mt = fmaxf(Mt, s_m[g2]);
    float lt = 0.0f, zt = 0.0f, acc4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int g2 = 0; g2 < kWideGroups; g2++) {
        const float mw = s_m[g2];
        const float f = mw == -INFINITY ? 0.0f : fast_exp2(mw - Mt);
        lt += f * s_l[g2];
        zt += f * s_z[g2];
#pragma unroll
        for (int e = 0; e < 4; e++) acc4[e] += f * s_acc[g2][c0 + e];
    }
    int64_t orow = row;
    if (a.q_len > 1) {
        const int bb = (int)(row / a.num_q_heads), vv = (int)(row % a.num_q_heads);
        orow = io_row<true>(a, bb, vv / a.gqa, vv % a.gqa);
    }
    finalize_head(acc4, lt, zt, l32, a.out, a.out_f32, orow, a.rotated);
}

// Work-groups of decode_kernel<KB, VB> the current device holds at once
// (compute units x occupancy), queried once per device; 512 without a device.
template <int KB, int VB, bool kPB = false>
int resident_workgroups() {
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
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_kernel<KB, VB, false, false, 1, kPB>, 64 * kDecodeWaves, 0) != hipSuccess ||
        cus <= 0 || per_cu <= 0) {
        (void)hipGetLastError();
        return 512;
    }
    // Plan for two work-groups per CU even where three would fit (k4v2 at
    // 166 VGPRs): measured at 16K and 128K, three per CU made the split
    // kernel ~1.2 us slower, and the extra splits push the combine onto its
    // wide path.
    if (per_cu > 2) per_cu = 2;
    cached[dev].store(cus * per_cu, std::memory_order_relaxed);
    return cus * per_cu;
}

template <int KB, int VB, bool kMQ, bool kPaged, int kG, bool kPB = false>
hipError_t launch_split_kernel(const DecodeArgs &a, hipStream_t stream, const LaunchEvents &ev) {
    const int sgroups = (a.head_groups + kG - 1) / kG;
    dim3 grid((unsigned)a.splits, (unsigned)(a.num_kv_heads * sgroups), (unsigned)a.num_seqs);
    if (kMQ) {
        // one dimension: rounds of 8 (split, sequence, KV head) units x work-groups per unit
        const int64_t units = (int64_t)a.splits * a.num_kv_heads * a.num_seqs;
        const int64_t blocks = (units + 7) / 8 * 8 * sgroups;
        if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
        grid = dim3((unsigned)blocks, 1, 1);
    }
    if (ev.start || ev.stop)
        hipExtLaunchKernelGGL(HIP_KERNEL_NAME(decode_kernel<KB, VB, kMQ, kPaged, kG, kPB>), grid, dim3(64 * kDecodeWaves), 0, stream, ev.start,
                              ev.stop, 0, a);
    else
        hipLaunchKernelGGL(HIP_KERNEL_NAME(decode_kernel<KB, VB, kMQ, kPaged, kG, kPB>), grid, dim3(64 * kDecodeWaves), 0, stream, a);
    return hipGetLastError();
}

// One query row per sequence, or several (causal among them).
template <int KB, int VB, int kG>
hipError_t launch_split_groups(const DecodeArgs &a, hipStream_t stream, const LaunchEvents &ev) {
    if (a.page_log2s > 0)
        return a.q_len > 1 ? launch_split_kernel<KB, VB, true, true, kG>(a, stream, ev)
                           : launch_split_kernel<KB, VB, false, true, kG>(a, stream, ev);
    return a.q_len > 1 ? launch_split_kernel<KB, VB, true, false, kG>(a, stream, ev)
                       : launch_split_kernel<KB, VB, false, false, kG>(a, stream, ev);
}

// Two head groups per work-group whenever a KV head has more than one (the
// split heuristic of the C ABI counts work-groups the same way).
template <int KB, int VB>
hipError_t launch_split_fmt(const DecodeArgs &a, hipStream_t stream, const LaunchEvents &ev) {
    return a.head_groups >= 2 ? launch_split_groups<KB, VB, 2>(a, stream, ev)
                              : launch_split_groups<KB, VB, 1>(a, stream, ev);
}

}  // namespace

int decode_resident_workgroups(int k_bits, int v_bits, bool page_balanced) {
    if (page_balanced) return k_bits == 4 && v_bits == 2 ? resident_workgroups<4, 2, true>() : 512;
    if (k_bits == 4 && v_bits == 2) return resident_workgroups<4, 2>();
    if (k_bits == 4 && v_bits == 4) return resident_workgroups<4, 4>();
    if (k_bits == 8 && v_bits == 2) return resident_workgroups<8, 2>();
    if (k_bits == 8 && v_bits == 4) return resident_workgroups<8, 4>();
    if (k_bits == 3 && v_bits == 3) return resident_workgroups<3, 3>();
    return 512;
}

hipError_t launch_decode_split(const DecodeArgs &a, hipStream_t stream, const LaunchEvents &ev) {
    if (a.key_norm) {          // page-balanced keys: K4V2, one query row, 16-token pages
        if (a.k_bits != 4 || a.v_bits != 2 || a.q_len > 1 || a.page_log2s != 0 || a.append)
            return hipErrorInvalidValue;
        return a.head_groups >= 2 ? launch_split_kernel<4, 2, false, false, 2, true>(a, stream, ev)
                                  : launch_split_kernel<4, 2, false, false, 1, true>(a, stream, ev);
    }
    if (a.k_bits == 4 && a.v_bits == 2) return launch_split_fmt<4, 2>(a, stream, ev);
    if (a.k_bits == 4 && a.v_bits == 4) return launch_split_fmt<4, 4>(a, stream, ev);
    if (a.k_bits == 8 && a.v_bits == 2) return launch_split_fmt<8, 2>(a, stream, ev);
    if (a.k_bits == 8 && a.v_bits == 4) return launch_split_fmt<8, 4>(a, stream, ev);
    if (a.k_bits == 3 && a.v_bits == 3) return launch_split_fmt<3, 3>(a, stream, ev);
    return hipErrorInvalidValue;
}

hipError_t launch_decode_combine(const DecodeArgs &a, hipStream_t stream) {
    const int64_t rows = (int64_t)a.num_seqs * a.num_q_heads;
    if (a.slot_stride > 8) {     // many slots per row: one work-group per row, one round of loads
        if (rows > 0x7fffffffLL) return hipErrorInvalidValue;
        hipLaunchKernelGGL(combine_wide_kernel, dim3((unsigned)rows), dim3(256), 0, stream, a);
        return hipGetLastError();
    }
    const int64_t blocks = (rows + 1) / 2;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(64), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream, const LaunchEvents &ev) {
    const hipError_t e = launch_decode_split(a, stream, ev);
    if (e != hipSuccess || (a.splits <= 1 && !a.partials_only)) return e;
    return launch_decode_combine(a, stream);
}

}  // namespace kvq

// Internal definitions of libkvq (gfx950).  Not part of the public ABI.
//
// Cache format "kvq-k4v2-g128 v1": one 1664-byte region per 16 tokens of one
// KV head; 128 channels per head; see include/kvq.h for the layout.  The same
// layout family holds 8-bit keys and 4-bit values (Layout below).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int kHeadDim = 128;
constexpr int kPage = 16;

// Region of KB-bit keys (4 or 8) and VB-bit values (2 or 4), or 3-bit keys
// and values (bit planes): key codes (16 tokens x 16 KB bytes, token-major),
// value codes (16 x 16 VB bytes), key and value metadata (16 x 4 bytes each).
// Layout<4, 2> and Layout<3, 3> are 1664-byte regions.
template <int KB, int VB>
struct Layout {
    static_assert(((KB == 4 || KB == 8) && (VB == 2 || VB == 4)) || (KB == 3 && VB == 3), "unsupported bit widths");
    static constexpr int kKCodes = 0;
    static constexpr int kVCodes = 256 * KB;
    static constexpr int kKMeta = 256 * (KB + VB);
    static constexpr int kVMeta = kKMeta + 64;
    static constexpr int kBytes = kKMeta + 128;
    static constexpr int kKL = (1 << KB) - 1;   // largest key code
    static constexpr int kVL = (1 << VB) - 1;   // largest value code
};
// K4V2: key codes [0, 1024) (token o at 64 o), value codes [1024, 1536) (the
// u16 of quad g, channel m, slot i at 1024 + 128 g + 8 m + 2 i), key (s, z)
// at 1536 + 4 o, value (s, mu) at 1600 + 4 o.
static_assert(Layout<4, 2>::kVCodes == 1024 && Layout<4, 2>::kKMeta == 1536 && Layout<4, 2>::kVMeta == 1600 &&
                  Layout<4, 2>::kBytes == 1664,
              "the K4V2 region");

// Page-balanced keys: the K4V2 region followed by 128 column-scale bytes
// (byte j = the high byte of fp16 2^e_j), 1792 bytes per (page, KV head).
constexpr int kScalesPB = 1664;
constexpr int kRegionPB = 1792;

// Decode work decomposition.
constexpr int kWaves = 4;           // waves per work-group
constexpr int kHeadsPerGroup = 8;   // query heads per MFMA column block (hi + lo = 16 columns)
constexpr int kPartialFloats = 132; // m, l, zacc, pad, acc[128]
constexpr int kMaxPagesPerSplit = 512;  // 64 page pairs per wave (one per lane)

// Uncompressed fp16 baseline cache: one 8192-byte region per (page, KV head).
constexpr int kRegionF16 = 8192;
constexpr int kVCodesF16 = 4096;           // values after the 4096 bytes of keys
constexpr int kMaxPagesPerSplitF16 = 256;  // 64 pages per wave (one per lane)

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

__device__ __forceinline__ uint16_t float_to_half_bits(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);   // v_cvt_f16_f32, nearest-even
}

// Lane exchange within a wave (ds_bpermute); `mask` < 64.
__device__ __forceinline__ float xor_lane(float v, int mask) {
    return __shfl_xor(v, mask, 64);
}
__device__ __forceinline__ uint32_t xor_lane_u(uint32_t v, int mask) {
    return (uint32_t)__shfl_xor((int)v, mask, 64);
}

// Value of lane (l ^ 8) within each row of 16 lanes, as one DPP move
// (row_ror:8 rotates a row by half its width).
__device__ __forceinline__ float row_swap8(float v) {
    return __builtin_bit_cast(float,
        __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
}

// Value of lane l ^ x for a constant x (the loops that call it are
// unrolled): one DPP move for x = 1, 2 (quad permutes) and 8 (row rotation
// by 8), a cross-lane permute through the LDS crossbar otherwise.  The
// values are the same as xor_lane's; only the transport differs.
__device__ __forceinline__ float xor_lane_dpp(float v, int x) {
    const int b = __builtin_bit_cast(int, v);
    return x == 1   ? __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, b, 0xB1, 0xF, 0xF, false))
           : x == 2 ? __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, b, 0x4E, 0xF, 0xF, false))
           : x == 8 ? __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, b, 0x128, 0xF, 0xF, false))
                    : xor_lane(v, x);
}

// The same for 32-bit integers.
__device__ __forceinline__ uint32_t xor_lane_u_dpp(uint32_t v, int x) {
    const int b = (int)v;
    return x == 1   ? (uint32_t)__builtin_amdgcn_update_dpp(0, b, 0xB1, 0xF, 0xF, false)
           : x == 2 ? (uint32_t)__builtin_amdgcn_update_dpp(0, b, 0x4E, 0xF, 0xF, false)
           : x == 8 ? (uint32_t)__builtin_amdgcn_update_dpp(0, b, 0x128, 0xF, 0xF, false)
                    : xor_lane_u(v, x);
}

__device__ __forceinline__ float fast_exp2(float x) {
    return __builtin_amdgcn_exp2f(x);   // v_exp_f32; exp2(-inf) = 0
}

}  // namespace kvq

// Launchers (host side), implemented next to their kernels.
namespace kvq {

struct AppendArgs {
    const uint16_t *key;
    const uint16_t *value;
    int64_t key_stride;
    int64_t value_stride;
    const int64_t *slots;
    int64_t num_tokens;
    int32_t num_kv_heads;
    uint8_t *cache;
    int64_t num_pages;
    int32_t k_bits;    // 4 or 8 (3 with v_bits 3)
    int32_t v_bits;    // 2 or 4 (3 with k_bits 3)
    int32_t page_log2s;   // pages of 16 << page_log2s tokens: 2^page_log2s 16-token regions each
};

hipError_t launch_append(const AppendArgs &a, hipStream_t stream);
// Page-balanced keys (K4V2, 16-token pages): whole-page blocks of 16 call tokens.
hipError_t launch_balance_append(const AppendArgs &a, hipStream_t stream);

struct DecodeArgs {
    void *out;
    int out_f32;
    const uint16_t *query;
    const uint8_t *cache;
    int64_t num_pages;
    const int32_t *block_tables;
    int32_t bt_stride;        // entries per block-table row (max_pages_per_seq)
    int32_t max_seq_len;      // sequences are clamped to this many tokens
    const int32_t *seq_lens;
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t gqa;              // num_q_heads / num_kv_heads
    int32_t head_groups;      // ceil(gqa / 8)
    // Query rows per sequence (1: plain decode).  With q_len > 1, num_q_heads
    // and gqa count (row, head) pairs: q_len * Hq and q_len * G, the pair
    // (m, g) being index m * G + g of its KV head; query and output rows are
    // [num_seqs][q_len][Hq], and row m attends to tokens 0 .. n - q_len + m.
    int32_t q_len;
    int32_t splits;           // work-groups per (seq, kv head, head group)
    int32_t pages_per_split;
    float alpha;              // softmax_scale * log2(e) / 128
    float *partials;          // [num_seqs][num_q_heads][splits][132]
    int32_t k_bits, v_bits;   // quantised cache: 4|8, 2|4 (16, 16: fp16 baseline)
    int32_t page_log2s;       // block-table pages of 16 << page_log2s tokens, each a run of
                              // 2^page_log2s 16-token regions per KV head (0: 16-token pages)
    int32_t rotated;          // 1: quantised (Hadamard epilogue); 0: fp16 baseline
    int32_t key_norm;         // 1: page-balanced keys (K4V2, 16-token pages, 1792-byte regions)
    int32_t slot_offset;      // partial of split s goes to slot slot_offset + s ...
    int32_t slot_stride;      // ... of rows holding slot_stride slots each
    int32_t rotate_partials;  // fp16: store partials in the Hadamard domain
    int32_t partials_only;    // 1: the split kernel writes a partial for every
                              // split it runs (also the only one) and leaves
                              // every output row to the combine kernel
    // Fused append (append != 0): token seq_lens[b] - 1 of every sequence is
    // encoded from new_key / new_value [num_seqs][num_kv_heads][128] (token
    // strides in elements) before it is attended to.
    int32_t append;
    const uint16_t *new_key;
    const uint16_t *new_value;
    int64_t new_key_stride;
    int64_t new_value_stride;
};

// Start/stop events the split kernel records at its own start and end
// (hipExtLaunchKernel's kernel events); NULL for none.
struct LaunchEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

// Split kernel then, if any sequence spans more than one split, the combine.
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream, const LaunchEvents &ev);
// The two phases on their own (a.partials_only = 1 for both).
hipError_t launch_decode_split(const DecodeArgs &a, hipStream_t stream, const LaunchEvents &ev);
hipError_t launch_decode_combine(const DecodeArgs &a, hipStream_t stream);

// Work-groups of the decode kernel for these bit widths that the current
// device runs at once.
int decode_resident_workgroups(int k_bits, int v_bits, bool page_balanced = false);

// fp16 baseline cache: append, decode split kernel (the combine is shared,
// with a.rotated = 0), resident work-groups of its split kernel.
hipError_t launch_fp16_append(const AppendArgs &a, hipStream_t stream);
hipError_t launch_fp16_decode_split(const DecodeArgs &a, hipStream_t stream, const LaunchEvents &ev);
int decode_fp16_resident_workgroups();

}  // namespace kvq

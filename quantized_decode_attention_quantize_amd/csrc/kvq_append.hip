// Quantise-on-write of new key/value tokens into the K4V2 g128 paged cache:
// one 16-lane row per group = (token, KV head, key|value), encoded by
// encode_group (kvq_quant.h).
#pragma clang fp contract(off)

#include "kvq_quant.h"

namespace kvq {
namespace {

constexpr int kRowsPerBlock = 16;   // 256 threads, 16 groups

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
    const int64_t page = slot / kPage;
    const int off = (int)(slot % kPage);
    if (page >= a.num_pages) return;

    const uint16_t *src = is_v ? a.value + tok * a.value_stride + (int64_t)head * kHeadDim
                               : a.key + tok * a.key_stride + (int64_t)head * kHeadDim;
    uint8_t *region = a.cache + (page * a.num_kv_heads + head) * (int64_t)kRegion;
    encode_group(src, is_v, r, region, off);
}

}  // namespace

hipError_t launch_append(const AppendArgs &a, hipStream_t stream) {
    const int64_t groups = a.num_tokens * a.num_kv_heads * 2;
    const int64_t blocks = (groups + kRowsPerBlock - 1) / kRowsPerBlock;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(quantize_append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kvq

// Read probes (measurement aids beside the decode path).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

// Reads `bytes` (a multiple of 16) from src in one launch.
hipError_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t stream);

// The page walk of a decode split kernel (validated by the caller).
struct PageWalkArgs {
    const uint8_t *cache;
    int64_t num_pages;
    int32_t region16;          // 16-byte words of one (16-token page, KV head) region
    int32_t num_kv_heads;
    const int32_t *block_tables;
    int32_t bt_stride;         // max_pages_per_seq
    const int32_t *seq_lens;
    int32_t max_seq_len;
    int32_t pages_per_split;   // even
    uint32_t *sink;
};

hipError_t launch_page_walk(const PageWalkArgs &a, int32_t splits, int32_t num_seqs, hipStream_t stream);

}  // namespace kvq

// Streaming-read probe (a measurement aid beside the decode path).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

// Reads `bytes` (a multiple of 16) from src in one launch.
hipError_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t stream);

}  // namespace kvq

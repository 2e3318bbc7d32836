// Streaming-read probe: the device's plain sequential-read rate, measured on
// the same hardware as the decode kernel, to set its HBM figure against a
// ceiling that this machine reaches and not only against the vendor peak
// (decode streams the whole cache through HBM once per token: encorp.ai,
// "KV cache compression is an infrastructure decision, not a model debate",
// section on the HBM ceiling).  Not part of the decode path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_probe.h"

namespace kvq {
namespace {

constexpr int kProbeUnroll = 4;   // 16-byte loads in flight per lane per step

// Grid-stride read of n16 16-byte words: each lane keeps kProbeUnroll loads
// in flight and folds them into an XOR, stored only if it equals a value no
// real data is expected to give, so that the loads stay live without output
// traffic.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *src, int64_t n16, uint32_t *sink) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
        uint4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; u++) v[u] = src[i + u * stride];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = src[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t stream) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    // two work-groups of 256 lanes per compute unit: the fastest plain-read
    // shape measured on this part (more lanes per unit lowered the rate)
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)(2 * cus)), dim3(256), 0, stream,
                       static_cast<const uint4 *>(src), bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace kvq

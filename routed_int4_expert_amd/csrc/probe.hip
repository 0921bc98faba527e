// probe.hip -- measurement only: a streaming-read probe that gives the practical HBM
// read ceiling the expert kernels are compared with.  It reads a device buffer once
// with 16-byte loads (eight in flight per thread, consecutive lanes on consecutive
// 16-byte words, so every wave load is 1 KB contiguous) from a grid of many resident
// workgroups, and folds the words into an XOR that is stored only if it equals a
// caller-given key, so the loads cannot be removed while nothing is written in
// practice.  Not a step of the layer.
#include <hip/hip_runtime.h>

#include "moe.h"
#include "moe_internal.h"

namespace moe {

constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(256) void read_probe_kernel(const uint4 *p, size_t n16, uint32_t key,
                                                         uint32_t *sink) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
        uint4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; u++) v[u] = p[i + u * stride];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == key) sink[0] = acc;
}

}  // namespace moe

using namespace moe;

extern "C" int moe_probe_read(const void *buf, size_t bytes, uint32_t key, uint32_t *sink,
                              int32_t blocks, void *stream) {
    if (!buf || !sink || bytes == 0 || bytes % 16 || ((uintptr_t)buf & 15u) || blocks <= 0 ||
        blocks > (1 << 20))
        return MOE_EINVAL;
    if (device_ok()) return MOE_EDEVICE;
    ProfScope prof("probe_read", (hipStream_t)stream);
    read_probe_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>(static_cast<const uint4 *>(buf), bytes / 16,
                                                                key, sink);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EDEVICE;
}

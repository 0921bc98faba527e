// glue.hip -- residual add and RMSNorm between stacked MoE layers (unit gain).
// Not a step of the MoE layer: the stacked-layer workload normalises each
// layer's input and adds each layer's output back to the residual stream.
//
// One workgroup per token row; each thread owns float4 columns; the sum of
// squares is reduced by a butterfly in each wave and the wave sums are added in
// wave order, so the result is deterministic.
#include <math.h>

#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(256) void residual_rmsnorm_kernel(GlueArgs a) {
    __shared__ float part[256 / kWave];
    const int t = blockIdx.x;
    const int n4 = a.H / 4;
    const float4 *h4 = reinterpret_cast<const float4 *>(a.h + (size_t)t * a.H);
    const float4 *d4 = a.delta ? reinterpret_cast<const float4 *>(a.delta + (size_t)t * a.H) : nullptr;
    float4 *ho4 = reinterpret_cast<float4 *>(a.h_out + (size_t)t * a.H);
    float4 *xo4 = reinterpret_cast<float4 *>(a.x_out + (size_t)t * a.H);
    float ss = 0.f;
    for (int j = threadIdx.x; j < n4; j += blockDim.x) {
        float4 v = h4[j];
        if (d4) {
            const float4 d = d4[j];
            v.x += d.x; v.y += d.y; v.z += d.z; v.w += d.w;
        }
        ho4[j] = v;
        ss = fmaf(v.x, v.x, ss);
        ss = fmaf(v.y, v.y, ss);
        ss = fmaf(v.z, v.z, ss);
        ss = fmaf(v.w, v.w, ss);
    }
#pragma unroll
    for (int m = kWave / 2; m > 0; m >>= 1) ss += __shfl_xor(ss, m, kWave);
    if (threadIdx.x % kWave == 0) part[threadIdx.x / kWave] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < 256 / kWave; w++) tot += part[w];
    const float r = 1.0f / sqrtf(tot / (float)a.H + a.eps);
    // each thread rescales the columns it wrote itself (same thread, program order)
    for (int j = threadIdx.x; j < n4; j += blockDim.x) {
        float4 v = ho4[j];
        v.x *= r; v.y *= r; v.z *= r; v.w *= r;
        xo4[j] = v;
    }
}

hipError_t launch_residual_rmsnorm(const GlueArgs &a, hipStream_t st) {
    ProfScope prof("residual_rmsnorm", st);
    residual_rmsnorm_kernel<<<a.T, 256, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace moe

// combine.hip -- step 5 of the MoE layer on gfx950: the gate-weighted sum of the
// expert outputs of each token plus the always-on shared expert
// ("MoE 路由与专家流式加载" §1 and §1.4).
//
// Each thread owns four consecutive outputs of one token (combine4 in combine.h).
// No atomics: the order is fixed, so the result is deterministic.
#include "combine.h"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
    const int t = blockIdx.y;
    const int n = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (n >= a.H) return;
    combine4(a, t, n);
}

hipError_t launch_combine(const CombineArgs &a, hipStream_t st) {
    dim3 grid((a.H / 4 + 255) / 256, a.T);
    ProfScope prof("combine", st);
    combine_kernel<<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace moe

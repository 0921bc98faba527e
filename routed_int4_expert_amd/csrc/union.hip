// union.hip -- step 3 of the MoE layer on gfx950: the batch union of the kept
// experts and the token permutation ("MoE 路由与专家流式加载" §1.3, batch-union:
// every distinct expert of the batch is read once and applied to all positions
// routed to it).
//
// One workgroup of 1024 threads.  A per-expert token bitmap in LDS is filled
// with LDS atomicOr (the result does not depend on their order); counts are
// popcounts, the offsets an exclusive wave scan.  The rows of an expert are
// then produced in token order by one wave per expert: a wave scan of the
// per-word popcounts gives each set bit its rank, so no atomics touch the
// outputs and the result is deterministic.
#include "select_union.h"

namespace moe {

__global__ __launch_bounds__(1024) void union_kernel(UnionArgs a) {
    extern __shared__ uint32_t lds[];
    union_block(a, a.ids, a.keff, lds);
}

hipError_t launch_union(const UnionArgs &a, hipStream_t st) {
    const size_t lds = union_lds_words(a.E, a.T) * sizeof(uint32_t);
    if (lds > 64 * 1024) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&union_kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        (void)hipGetLastError();
    }
    ProfScope prof("union", st);
    union_kernel<<<1, 1024, lds, st>>>(a);
    return hipGetLastError();
}

}  // namespace moe

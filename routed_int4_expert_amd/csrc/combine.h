// combine.h -- step 5 of the MoE layer ("MoE 路由与专家流式加载" §1 and §1.4): the
// gate-weighted sum of a token's expert outputs plus the always-on shared expert,
// for four consecutive outputs.  Used by the combine kernel and by the down launch
// that fuses it, so both add in the same order: slot order in fp32 (fmaf), then
// the shared expert's output with weight 1.  The bf16 output is the
// round-to-nearest-even of that fp32.
#pragma once

#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ uint16_t bf16_rne(float v) {
    const uint32_t b = __float_as_uint(v);
    return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

// outputs n .. n+3 of token t (n a multiple of 4, H a multiple of 64)
__device__ __forceinline__ void combine4(const CombineArgs &a, int t, int n) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    const int ke = min(max(a.keff[t], 0), a.k);
    for (int j = 0; j < ke; j++) {
        const int r = a.pick_row[(size_t)t * a.k + j];
        if (r < 0) continue;
        const float wj = a.w[(size_t)t * a.k + j];
        const float4 y = *reinterpret_cast<const float4 *>(a.y_routed + (size_t)r * a.H + n);
        acc.x = fmaf(wj, y.x, acc.x);
        acc.y = fmaf(wj, y.y, acc.y);
        acc.z = fmaf(wj, y.z, acc.z);
        acc.w = fmaf(wj, y.w, acc.w);
    }
    if (a.y_shared) {
        const float4 y = *reinterpret_cast<const float4 *>(a.y_shared + (size_t)t * a.H + n);
        acc.x += y.x;
        acc.y += y.y;
        acc.z += y.z;
        acc.w += y.w;
    }
    if (a.out_bf16) {
        uint16_t *o = reinterpret_cast<uint16_t *>(a.out) + (size_t)t * a.H + n;
        const uint2 packed = make_uint2((uint32_t)bf16_rne(acc.x) | ((uint32_t)bf16_rne(acc.y) << 16),
                                        (uint32_t)bf16_rne(acc.z) | ((uint32_t)bf16_rne(acc.w) << 16));
        *reinterpret_cast<uint2 *>(o) = packed;
    } else {
        *reinterpret_cast<float4 *>(reinterpret_cast<float *>(a.out) + (size_t)t * a.H + n) = acc;
    }
}

}  // namespace moe

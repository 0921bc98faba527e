// combine.h -- step 5 of the MoE layer ("MoE 路由与专家流式加载" §1 and §1.4): the
// gate-weighted sum of a token's expert outputs plus the always-on shared expert,
// for four consecutive outputs, as the combine kernel computes it: slot order in fp32
// (fmaf), then the shared expert's output with weight 1.  The bf16 output is the
// round-to-nearest-even of that fp32.
#pragma once

#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ uint16_t bf16_rne(float v) {
    const uint32_t b = __float_as_uint(v);
    return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

// four outputs n .. n+3 of token t, as fp32 or as their bf16 round-to-nearest-even
__device__ __forceinline__ void store4(const CombineArgs &a, int t, int n, float4 acc) {
    if (a.out_bf16) {
        uint16_t *o = reinterpret_cast<uint16_t *>(a.out) + (size_t)t * a.H + n;
        const uint2 packed = make_uint2((uint32_t)bf16_rne(acc.x) | ((uint32_t)bf16_rne(acc.y) << 16),
                                        (uint32_t)bf16_rne(acc.z) | ((uint32_t)bf16_rne(acc.w) << 16));
        *reinterpret_cast<uint2 *>(o) = packed;
    } else {
        *reinterpret_cast<float4 *>(reinterpret_cast<float *>(a.out) + (size_t)t * a.H + n) = acc;
    }
}

// outputs n .. n+3 of token t (n a multiple of 4, H a multiple of 64).  The slots'
// rows and weights are read first, then all the rows' values, so the loads take two
// round trips whatever k is; the sum runs in slot order.
__device__ __forceinline__ void combine4(const CombineArgs &a, int t, int n) {
    if (a.k == 0) {  // no routed experts: the always-on FFN's output alone
        store4(a, t, n, *reinterpret_cast<const float4 *>(a.y_shared + (size_t)t * a.H + n));
        return;
    }
    const int ke = min(max(a.keff[t], 0), a.k);
    // loads are unconditional (clamped slot, row 0 for an empty slot), so they are all
    // in flight together; empty slots are masked out of the sum
    int rj[MOE_MAX_TOPK];
    float wj[MOE_MAX_TOPK];
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; j++) {
        const size_t sj = (size_t)t * a.k + min(j, a.k - 1);
        rj[j] = a.pick_row[sj];
        wj[j] = a.w[sj];
    }
    float4 yj[MOE_MAX_TOPK];
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; j++)
        yj[j] = *reinterpret_cast<const float4 *>(a.y_routed + (size_t)max(rj[j], 0) * a.H + n);
    float4 ys = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.y_shared) ys = *reinterpret_cast<const float4 *>(a.y_shared + (size_t)t * a.H + n);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; j++) {
        const bool live = j < ke && rj[j] >= 0;
        const float w = live ? wj[j] : 0.f;
        if (live) {
            acc.x = fmaf(w, yj[j].x, acc.x);
            acc.y = fmaf(w, yj[j].y, acc.y);
            acc.z = fmaf(w, yj[j].z, acc.z);
            acc.w = fmaf(w, yj[j].w, acc.w);
        }
    }
    if (a.y_shared) {
        acc.x += ys.x;
        acc.y += ys.y;
        acc.z += ys.z;
        acc.w += ys.w;
    }
    store4(a, t, n, acc);
}

}  // namespace moe

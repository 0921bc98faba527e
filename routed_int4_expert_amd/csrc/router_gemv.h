// router_gemv.h -- step 1 of the MoE layer ("MoE 路由与专家流式加载" §1.1) for a
// few tokens: the logits of one expert, logit[t][e] = Wr[e]·x[t], by one workgroup.
// Its four waves split H, every lane issues all its float4 loads of the router row
// before using any, the row is applied to every token with exact fp32 products summed in
// fp64, and the four wave sums are added in a fixed order.  Complete logits, a
// single slice (S = 1); with `sig` set, also each logit's sigmoid gate and choice key.
#pragma once

#include "moe_internal.h"
#include "select_union.h"

namespace moe {

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xF, 0xF, false);
    return __hiloint2double(hi, lo);
}

__device__ __forceinline__ double readlane_lane_f64(double v, int lane) {
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), lane),
                            __builtin_amdgcn_readlane(__double2loint(v), lane));
}

// Sum over the 64 lanes of a wave (all active), in a fixed order: rows of 16 lanes by
// DPP moves (swap neighbours, swap pairs, rotate by 4, rotate by 8), then the four
// row sums from lanes 0, 16, 32 and 48, wave-uniform.
__device__ __forceinline__ double router_wave_sum_f64(double v) {
    v += dpp_f64<0xB1>(v);
    v += dpp_f64<0x4E>(v);
    v += dpp_f64<0x124>(v);
    v += dpp_f64<0x128>(v);
    return (readlane_lane_f64(v, 0) + readlane_lane_f64(v, 16)) +
           (readlane_lane_f64(v, 32) + readlane_lane_f64(v, 48));
}

template <int TT>
__device__ __forceinline__ void router_gemv_body(const LogitsArgs &a, int e) {
    // float4 loads of the router row per lane issued before the first is used (all of
    // a row of up to 8192 values); indices past the row re-read its last float4 and
    // are not accumulated, so no load waits behind a branch
    constexpr int U = 8;
    __shared__ double red[4][TT];
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
    const int n4 = a.H / 4;
    const float4 *w4 = reinterpret_cast<const float4 *>(a.wr + (size_t)e * a.H);
    const float4 *x4 = reinterpret_cast<const float4 *>(a.x);
    double acc[TT];
#pragma unroll
    for (int t = 0; t < TT; t++) acc[t] = 0.0;
    for (int j0 = threadIdx.x; j0 < n4; j0 += 256 * U) {
        float4 w[U];
#pragma unroll
        for (int u = 0; u < U; u++) w[u] = w4[min(j0 + 256 * u, n4 - 1)];
#pragma unroll
        for (int t = 0; t < TT; t++) {
            const float4 *xt = x4 + (size_t)min(t, a.T - 1) * n4;  // rows past T: not written
            float4 v[U];
#pragma unroll
            for (int u = 0; u < U; u++) v[u] = xt[min(j0 + 256 * u, n4 - 1)];
#pragma unroll
            for (int u = 0; u < U; u++) {
                if (j0 + 256 * u < n4) {
                    acc[t] = fma((double)v[u].x, (double)w[u].x, acc[t]);
                    acc[t] = fma((double)v[u].y, (double)w[u].y, acc[t]);
                    acc[t] = fma((double)v[u].z, (double)w[u].z, acc[t]);
                    acc[t] = fma((double)v[u].w, (double)w[u].w, acc[t]);
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < TT; t++) {
        acc[t] = router_wave_sum_f64(acc[t]);
        if (lane == 0) red[wv][t] = acc[t];
    }
    __syncthreads();
    if (threadIdx.x < TT && (int)threadIdx.x < a.T) {
        const int t = threadIdx.x;
        const double l = ((red[0][t] + red[1][t]) + red[2][t]) + red[3][t];
        a.part[(size_t)t * a.E + e] = l;
        if (a.sig) {  // the logit is complete: its gate and choice key too
            double sg;
            unsigned long long ky;
            gate_and_key(l, a.bias, e, sg, ky);
            a.sig[(size_t)t * a.E + e] = sg;
            a.key[(size_t)t * a.E + e] = ky;
        }
    }
}

}  // namespace moe

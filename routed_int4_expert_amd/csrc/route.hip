// route.hip -- steps 1 and 2 of the MoE layer on gfx950: router logits and
// noaux_tc sigmoid selection ("MoE 路由与专家流式加载" §1.1, §1.2).
//
// Logits, few tokens (T <= 8): one workgroup per expert streams the expert's router
// row once (four waves across H) and applies it to every token, accumulating in fp64
// (fp32 x fp32 products are exact in fp64); the logits are complete, so it also
// writes each one's sigmoid gate and choice key for the selection.
// Logits, more tokens: each workgroup owns a 64-token x 64-expert tile and one
// slice of H; fp32 tiles of x and Wr are staged through LDS and the fp64 matrix
// cores accumulate their exact products.  The per-slice partial sums go to the
// workspace and are added, in slice order, by the selection kernel, so the result
// does not depend on scheduling.
//
// Selection: one wave per token (select_token in select_union.h).  Each lane holds
// up to four experts' sigmoid gate and biased choice score in fp64, the choice as a
// monotone 64-bit key.  The k-th largest key is found by a bitwise threshold search
// (one ballot count per candidate bit, starting below the bits all live keys share).
// If exactly k keys reach it, those are the picks; otherwise every key above it is
// picked and the keys equal to it fill the remaining slots in increasing expert id
// (the result of k rounds of argmax with ties to the lower id).  The picks are then
// ranked (choice descending, lower id first) by DPP rotations within one row of 16
// lanes and moved to their slots with ds_permute.  Top-p, renormalisation and
// scaling work on the at most 16 picks in lanes 0..k-1.
#include <math.h>

#include "router_gemv.h"
#include "select_union.h"

namespace moe {

RouterSplit router_split(int T, int E, int H) {
    if (T <= kRouterGemvTokens) {  // one wave per expert, whole H: no split
        RouterSplit r;
        r.S = 1;
        r.kslice = H;
        return r;
    }
    const int tiles = ((T + kRouterTile - 1) / kRouterTile) * ((E + kRouterTile - 1) / kRouterTile);
    const int chunks = H / kRouterKC;
    // enough H slices that the launch has about one workgroup per CU (the slices'
    // partial logits are summed in slice order by the selection)
    int S = (256 + tiles - 1) / tiles;
    if (S > 64) S = 64;
    if (S > chunks) S = chunks;
    if (S < 1) S = 1;
    const int per = (chunks + S - 1) / S;
    RouterSplit r;
    r.kslice = per * kRouterKC;
    r.S = (H + r.kslice - 1) / r.kslice;
    return r;
}

// ------------------------------------------------------------------ logits
// More tokens: each workgroup owns a 64-token x 64-expert tile and one slice of H.
// fp32 tiles of x and Wr (64 H values per step) are staged through two LDS buffers:
// the next step's loads are issued before the current step's products, and one
// barrier per step hands a buffer over.  The fp64 matrix cores
// (v_mfma_f64_16x16x4_f64) take the values converted to fp64 (exact) and accumulate
// their exact products in fp64.
// Wave w owns tokens 16w .. 16w+15 of the tile and all 64 experts (four 16x16 blocks).
// Operand layouts: A (tokens x K) lane l holds [l % 16][l / 16], B (K x experts) lane
// l holds [l / 16][l % 16]; register v of lane l holds the result's row l / 16 + 4v,
// column l % 16 (rows interleaved across the lane groups, unlike the fp32 16x16 layouts).
typedef double f64x4_t __attribute__((ext_vector_type(4)));

// loader mapping: 64 rows x 64 columns = 1024 float4 per operand, 4 per thread
constexpr int kRouterLoads = kRouterTile * kRouterKC / 4 / 256;

struct RouterStage {
    float4 x[kRouterLoads], w[kRouterLoads];
};

__device__ __forceinline__ void router_stage_load(const LogitsArgs &a, int t0, int e0, int h0,
                                                  RouterStage &r) {
#pragma unroll
    for (int rep = 0; rep < kRouterLoads; rep++) {
        const int idx = threadIdx.x + rep * 256;
        const int row = idx / (kRouterKC / 4), c4 = (idx % (kRouterKC / 4)) * 4;
        const int t = t0 + row, e = e0 + row;
        r.x[rep] = make_float4(0.f, 0.f, 0.f, 0.f);
        r.w[rep] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (t < a.T) r.x[rep] = *reinterpret_cast<const float4 *>(a.x + (size_t)t * a.H + h0 + c4);
        if (e < a.E) r.w[rep] = *reinterpret_cast<const float4 *>(a.wr + (size_t)e * a.H + h0 + c4);
    }
}

__device__ __forceinline__ void router_stage_store(const RouterStage &r,
                                                   float (*xs)[kRouterTile + 1],
                                                   float (*wsh)[kRouterTile + 1]) {
#pragma unroll
    for (int rep = 0; rep < kRouterLoads; rep++) {
        const int idx = threadIdx.x + rep * 256;
        const int row = idx / (kRouterKC / 4), c4 = (idx % (kRouterKC / 4)) * 4;
        xs[c4 + 0][row] = r.x[rep].x; xs[c4 + 1][row] = r.x[rep].y;
        xs[c4 + 2][row] = r.x[rep].z; xs[c4 + 3][row] = r.x[rep].w;
        wsh[c4 + 0][row] = r.w[rep].x; wsh[c4 + 1][row] = r.w[rep].y;
        wsh[c4 + 2][row] = r.w[rep].z; wsh[c4 + 3][row] = r.w[rep].w;
    }
}

__global__ __launch_bounds__(256) void router_logits_mfma_kernel(LogitsArgs a) {
    __shared__ float xs[2][kRouterKC][kRouterTile + 1];
    __shared__ float wsh[2][kRouterKC][kRouterTile + 1];
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
    const int t0 = blockIdx.x * kRouterTile;
    const int e0 = blockIdx.y * kRouterTile;
    const int s = blockIdx.z;
    const int h_begin = s * a.kslice;
    const int h_end = min(a.H, h_begin + a.kslice);
    f64x4_t acc[4];
#pragma unroll
    for (int b = 0; b < 4; b++) acc[b] = f64x4_t{0.0, 0.0, 0.0, 0.0};
    RouterStage r;
    router_stage_load(a, t0, e0, h_begin, r);
    router_stage_store(r, xs[0], wsh[0]);
    __syncthreads();
    int cur = 0;
    for (int h0 = h_begin; h0 < h_end; h0 += kRouterKC) {
        const bool more = h0 + kRouterKC < h_end;
        if (more) router_stage_load(a, t0, e0, h0 + kRouterKC, r);
#pragma unroll
        for (int kk = 0; kk < kRouterKC; kk += 4) {
            const int k = kk + lane / 16, i = lane % 16;
            const double av = (double)xs[cur][k][16 * wv + i];
            double bv[4];
#pragma unroll
            for (int b = 0; b < 4; b++) bv[b] = (double)wsh[cur][k][16 * b + i];
#pragma unroll
            for (int b = 0; b < 4; b++) acc[b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv[b], acc[b], 0, 0, 0);
        }
        // the other buffer was last read before the previous barrier
        if (more) router_stage_store(r, xs[cur ^ 1], wsh[cur ^ 1]);
        __syncthreads();
        cur ^= 1;
    }
#pragma unroll
    for (int b = 0; b < 4; b++) {
        const int e = e0 + 16 * b + lane % 16;
        if (e >= a.E) continue;
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const int t = t0 + 16 * wv + (lane / 16) + 4 * v;
            if (t < a.T) a.part[((size_t)s * a.T + t) * a.E + e] = acc[b][v];
        }
    }
}

// Few tokens: one workgroup per expert (router_gemv.h).
template <int TT>
__global__ __launch_bounds__(256) void router_gemv_kernel(LogitsArgs a) {
    router_gemv_body<TT>(a, blockIdx.x);
}

hipError_t launch_router_logits(const LogitsArgs &a, int S, hipStream_t st) {
    ProfScope prof("router_logits", st);
    if (S == 1 && a.T <= kRouterGemvTokens) {
        const int blocks = a.E;
        if (a.T == 1) router_gemv_kernel<1><<<blocks, 256, 0, st>>>(a);
        else if (a.T <= 2) router_gemv_kernel<2><<<blocks, 256, 0, st>>>(a);
        else if (a.T <= 4) router_gemv_kernel<4><<<blocks, 256, 0, st>>>(a);
        else router_gemv_kernel<kRouterGemvTokens><<<blocks, 256, 0, st>>>(a);
        return hipGetLastError();
    }
    dim3 grid((a.T + kRouterTile - 1) / kRouterTile, (a.E + kRouterTile - 1) / kRouterTile, S);
    router_logits_mfma_kernel<<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
}

// ------------------------------------------------------------------ selection
// One workgroup per token: each thread sums one expert's logit over the router's
// slices (coalesced over experts), then one wave selects from LDS.
__global__ __launch_bounds__(256) void route_select_kernel(SelectArgs a) {
    __shared__ PickScratch ps;
    __shared__ double lg[MOE_MAX_EXPERTS];
    const int t = blockIdx.x;
    if (!a.key_in) {
        for (int e = threadIdx.x; e < a.E; e += blockDim.x) lg[e] = sum_partials(a, t, e);
        __syncthreads();
    }
    if (threadIdx.x >= kWave) return;
    select_token(a, t, threadIdx.x, a.ids + (size_t)t * a.k, a.w + (size_t)t * a.k, a.keff + t,
                 nullptr, nullptr, &ps, lg);
}

hipError_t launch_route_select(const SelectArgs &a, hipStream_t st) {
    ProfScope prof("route_select", st);
    route_select_kernel<<<a.T, 256, 0, st>>>(a);
    return hipGetLastError();
}

// Small batches: one workgroup selects every token (a wave each) and builds the
// union from the picks it keeps in LDS, saving a launch and a round trip.
__global__ __launch_bounds__(1024) void select_union_kernel(SelectArgs s, UnionArgs u) {
    __shared__ PickScratch ps[kSelectUnionTokens];
    extern __shared__ double lds_d[];
    double *lg = lds_d;  // [T][E] logits, summed over the router's slices by all threads
    int32_t *ids_l = reinterpret_cast<int32_t *>(lg + (size_t)s.T * s.E);
    int32_t *keff_l = ids_l + s.T * s.k;
    uint32_t *scratch = reinterpret_cast<uint32_t *>(keff_l + s.T);
    if (!s.key_in) {
        for (int i = threadIdx.x; i < s.T * s.E; i += blockDim.x) lg[i] = sum_partials(s, i / s.E, i % s.E);
        __syncthreads();
    }
    const int lane = threadIdx.x % kWave;
    const int t = threadIdx.x / kWave;
    if (t < s.T)
        select_token(s, t, lane, s.ids + (size_t)t * s.k, s.w + (size_t)t * s.k, s.keff + t,
                     ids_l + t * s.k, keff_l + t, &ps[t], lg + (size_t)t * s.E);
    __syncthreads();
    union_block(u, ids_l, keff_l, scratch);
}

hipError_t launch_select_union(const SelectArgs &s, const UnionArgs &u, hipStream_t st) {
    const size_t lds = (size_t)s.T * s.E * sizeof(double) +
                       ((size_t)s.T * s.k + s.T + union_lds_words(u.E, u.T)) * sizeof(uint32_t);
    ProfScope prof("select_union", st);
    // a wave per token, at least four waves for the union
    const int threads = max(256, kWave * s.T);
    select_union_kernel<<<1, threads, lds, st>>>(s, u);
    return hipGetLastError();
}

}  // namespace moe

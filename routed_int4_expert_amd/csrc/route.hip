// route.hip -- steps 1 and 2 of the MoE layer on gfx950: router logits and
// noaux_tc sigmoid selection ("MoE 路由与专家流式加载" §1.1, §1.2).
//
// Logits: each workgroup owns a 64-token x 64-expert tile and one slice of H.
// fp32 tiles of x and Wr are staged through LDS; every thread accumulates a 4x4
// register micro-tile in fp64 (fp32 x fp32 products are exact in fp64).  The
// per-slice partial sums go to the workspace and are added, in slice order, by
// the selection kernel, so the result does not depend on scheduling.
//
// Selection: one wave per token.  Each lane holds up to four experts' sigmoid
// and biased choice score in fp64; the k picks are k wave-wide argmax
// reductions (butterfly over the 64 lanes, ties to the lower expert id).  The
// top-p cut, renormalisation and scaling work on at most 16 picks held
// identically in every lane.
#include <math.h>

#include "moe_internal.h"

namespace moe {

RouterSplit router_split(int T, int E, int H) {
    const int tiles = ((T + kRouterTile - 1) / kRouterTile) * ((E + kRouterTile - 1) / kRouterTile);
    const int chunks = H / kRouterKC;
    int S = (256 + tiles - 1) / tiles;
    if (S > 32) S = 32;
    if (S > chunks) S = chunks;
    if (S < 1) S = 1;
    const int per = (chunks + S - 1) / S;
    RouterSplit r;
    r.kslice = per * kRouterKC;
    r.S = (H + r.kslice - 1) / r.kslice;
    return r;
}

// ------------------------------------------------------------------ logits
__global__ __launch_bounds__(256) void router_logits_kernel(LogitsArgs a) {
    __shared__ float xs[kRouterKC][kRouterTile + 1];
    __shared__ float wsh[kRouterKC][kRouterTile + 1];
    const int tid = threadIdx.x;
    const int t0 = blockIdx.x * kRouterTile;
    const int e0 = blockIdx.y * kRouterTile;
    const int s = blockIdx.z;
    const int h_begin = s * a.kslice;
    const int h_end = min(a.H, h_begin + a.kslice);
    const int ty = tid / 16, tx = tid % 16;

    double acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = 0.0;

    // loader mapping: 64 rows x 32 columns = 512 float4 per operand, 2 per thread
    for (int h0 = h_begin; h0 < h_end; h0 += kRouterKC) {
#pragma unroll
        for (int rep = 0; rep < 2; rep++) {
            const int idx = tid + rep * 256;   // 0..511
            const int row = idx / 8;            // tile row 0..63
            const int c4 = (idx % 8) * 4;       // column 0,4,...,28
            float4 vx = make_float4(0.f, 0.f, 0.f, 0.f);
            float4 vw = make_float4(0.f, 0.f, 0.f, 0.f);
            const int t = t0 + row, e = e0 + row;
            if (t < a.T) vx = *reinterpret_cast<const float4 *>(a.x + (size_t)t * a.H + h0 + c4);
            if (e < a.E) vw = *reinterpret_cast<const float4 *>(a.wr + (size_t)e * a.H + h0 + c4);
            xs[c4 + 0][row] = vx.x; xs[c4 + 1][row] = vx.y; xs[c4 + 2][row] = vx.z; xs[c4 + 3][row] = vx.w;
            wsh[c4 + 0][row] = vw.x; wsh[c4 + 1][row] = vw.y; wsh[c4 + 2][row] = vw.z; wsh[c4 + 3][row] = vw.w;
        }
        __syncthreads();
#pragma unroll 4
        for (int kk = 0; kk < kRouterKC; kk++) {
            double xv[4], wv[4];
#pragma unroll
            for (int i = 0; i < 4; i++) xv[i] = (double)xs[kk][ty + 16 * i];
#pragma unroll
            for (int j = 0; j < 4; j++) wv[j] = (double)wsh[kk][tx + 16 * j];
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++) acc[i][j] = fma(xv[i], wv[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int t = t0 + ty + 16 * i;
        if (t >= a.T) continue;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int e = e0 + tx + 16 * j;
            if (e < a.E) a.part[((size_t)s * a.T + t) * a.E + e] = acc[i][j];
        }
    }
}

hipError_t launch_router_logits(const LogitsArgs &a, int S, hipStream_t st) {
    dim3 grid((a.T + kRouterTile - 1) / kRouterTile, (a.E + kRouterTile - 1) / kRouterTile, S);
    ProfScope prof("router_logits", st);
    router_logits_kernel<<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
}

// ------------------------------------------------------------------ selection
__device__ __forceinline__ double shfl_xor_f64(double v, int m) {
    const int lo = __shfl_xor(__double2loint(v), m, kWave);
    const int hi = __shfl_xor(__double2hiint(v), m, kWave);
    return __hiloint2double(hi, lo);
}

__device__ __forceinline__ double shfl_f64(double v, int src) {
    const int lo = __shfl(__double2loint(v), src, kWave);
    const int hi = __shfl(__double2hiint(v), src, kWave);
    return __hiloint2double(hi, lo);
}

__global__ __launch_bounds__(256) void route_select_kernel(SelectArgs a) {
    const int lane = threadIdx.x % kWave;
    const int t = blockIdx.x * 4 + threadIdx.x / kWave;
    if (t >= a.T) return;  // whole wave leaves together

    constexpr int EPL = MOE_MAX_EXPERTS / kWave;  // experts per lane (4)
    double sig[EPL], ch[EPL];
    bool live[EPL];
#pragma unroll
    for (int i = 0; i < EPL; i++) {
        const int e = lane + kWave * i;
        live[i] = e < a.E;
        sig[i] = 0.0;
        ch[i] = -INFINITY;
        if (live[i]) {
            double l = 0.0;
            for (int s = 0; s < a.S; s++) l += a.part[((size_t)s * a.T + t) * a.E + e];
            sig[i] = 1.0 / (1.0 + exp(-l));
            const double b = a.bias ? (double)a.bias[e] : 0.0;
            const double c = sig[i] + b;
            ch[i] = isnan(c) ? -INFINITY : c;
        }
    }

    // k picks, identical in every lane after each reduction
    int pid[MOE_MAX_TOPK];
    double psig[MOE_MAX_TOPK];
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; j++) {
        pid[j] = -1;
        psig[j] = 0.0;
        if (j >= a.k) continue;
        double bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < EPL; i++) {
            if (!live[i]) continue;
            if (bi == 0x7fffffff || ch[i] > bv) {  // e grows with i: strict > keeps the lower id
                bv = ch[i];
                bi = lane + kWave * i;
            }
        }
#pragma unroll
        for (int m = kWave / 2; m > 0; m >>= 1) {
            const double ov = shfl_xor_f64(bv, m);
            const int oi = __shfl_xor(bi, m, kWave);
            if (oi != 0x7fffffff && (bi == 0x7fffffff || ov > bv || (ov == bv && oi < bi))) {
                bv = ov;
                bi = oi;
            }
        }
        const int owner = bi % kWave, slot = bi / kWave;
        double mysig = 0.0;
#pragma unroll
        for (int i = 0; i < EPL; i++)
            if (i == slot) mysig = sig[i];
        psig[j] = shfl_f64(mysig, owner);
        pid[j] = bi;
        if (lane == owner) {
#pragma unroll
            for (int i = 0; i < EPL; i++)
                if (i == slot) live[i] = false;
        }
    }

    // adaptive top-p: rank of each pick by sig descending, equal sigs in slot order
    bool keep[MOE_MAX_TOPK];
    int keff = a.k;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; j++) keep[j] = j < a.k;
    if (a.top_p > 0.0f && a.top_p < 1.0f) {
        int rank[MOE_MAX_TOPK];
#pragma unroll
        for (int j = 0; j < MOE_MAX_TOPK; j++) {
            int r = 0;
#pragma unroll
            for (int i = 0; i < MOE_MAX_TOPK; i++)
                if (i < a.k && j < a.k && (psig[i] > psig[j] || (psig[i] == psig[j] && i < j))) r++;
            rank[j] = r;
        }
        // total and running sums in rank order
        double tot = 0.0;
#pragma unroll
        for (int r = 0; r < MOE_MAX_TOPK; r++)
#pragma unroll
            for (int j = 0; j < MOE_MAX_TOPK; j++)
                if (j < a.k && r < a.k && rank[j] == r) tot += psig[j];
        const double thr = (double)a.top_p * tot;
        double cum = 0.0;
        int m = a.k;
        bool done = false;
#pragma unroll
        for (int r = 0; r < MOE_MAX_TOPK; r++)
#pragma unroll
            for (int j = 0; j < MOE_MAX_TOPK; j++)
                if (!done && j < a.k && r < a.k && rank[j] == r) {
                    cum += psig[j];
                    if (cum >= thr) {
                        m = r + 1;
                        done = true;
                    }
                }
        keff = m;
#pragma unroll
        for (int j = 0; j < MOE_MAX_TOPK; j++) keep[j] = j < a.k && rank[j] < m;
    }

    double denom = 0.0;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; j++)
        if (keep[j]) denom += psig[j];

    // lane j writes the output slot of pick j (kept picks compacted in slot order)
    int pos = 0;
    bool mine_kept = false;
    double g = 0.0;
    int gid = -1;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; j++) {
        if (j == lane && keep[j]) {
            mine_kept = true;
            g = psig[j];
            gid = pid[j];
        }
        if (j < lane && keep[j]) pos++;
    }
    int32_t *ids = a.ids + (size_t)t * a.k;
    float *w = a.w + (size_t)t * a.k;
    if (lane < a.k && mine_kept) {
        if (a.norm_topk) g = g / denom;
        g = g * (double)a.routed_scale;
        ids[pos] = gid;
        w[pos] = (float)g;
    }
    if (lane >= keff && lane < a.k) {
        ids[lane] = -1;
        w[lane] = 0.0f;
    }
    if (lane == 0) a.keff[t] = keff;
}

hipError_t launch_route_select(const SelectArgs &a, hipStream_t st) {
    ProfScope prof("route_select", st);
    route_select_kernel<<<(a.T + 3) / 4, 256, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace moe

// select_union.h -- device building blocks of steps 2 and 3 of the MoE layer
// ("MoE 路由与专家流式加载" §1.1-§1.3): one token's noaux_tc selection by one
// wave, and the batch union of a block.  Included by route.hip and union.hip.
#pragma once

#include <math.h>

#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ double shfl_xor_f64(double v, int m) {
    const int lo = __shfl_xor(__double2loint(v), m, kWave);
    const int hi = __shfl_xor(__double2hiint(v), m, kWave);
    return __hiloint2double(hi, lo);
}

// value of lane `src` (wave-uniform) to every lane, through scalar registers
__device__ __forceinline__ double readlane_f64(double v, int src) {
    const int s = __builtin_amdgcn_readfirstlane(src);
    const int lo = __builtin_amdgcn_readlane(__double2loint(v), s);
    const int hi = __builtin_amdgcn_readlane(__double2hiint(v), s);
    return __hiloint2double(hi, lo);
}

// One token, one wave.  [R] §1.1: sig = sigmoid(logit) and choice = sig + bias,
// in fp64; [R] §1.2: k rounds of argmax over choice excluding taken experts
// (equal scores: lower id), adaptive top-p over the k gates, norm_topk, scale.
// Lane j < k holds pick j.  Writes ids/w (this token's k slots) and *keff; when
// ids_copy/keff_copy are given, the ids and keff are written there too.
__device__ __forceinline__ void select_token(const SelectArgs &a, int t, int lane, int32_t *ids,
                                             float *w, int32_t *keff_out, int32_t *ids_copy,
                                             int32_t *keff_copy) {
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
            // slice partials added in slice order; loads issued eight at a time
            double l = 0.0;
            int s = 0;
            for (; s + 8 <= a.S; s += 8) {
                double v[8];
#pragma unroll
                for (int u = 0; u < 8; u++) v[u] = a.part[((size_t)(s + u) * a.T + t) * a.E + e];
#pragma unroll
                for (int u = 0; u < 8; u++) l += v[u];
            }
            for (; s < a.S; s++) l += a.part[((size_t)s * a.T + t) * a.E + e];
            sig[i] = 1.0 / (1.0 + exp(-l));
            const double b = a.bias ? (double)a.bias[e] : 0.0;
            const double c = sig[i] + b;
            ch[i] = isnan(c) ? -INFINITY : c;
        }
    }

    int my_id = -1;
    double my_sig = 0.0;
    for (int j = 0; j < a.k; j++) {
        double bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < EPL; i++) {
            if (live[i] && (bi == 0x7fffffff || ch[i] > bv)) {  // e grows with i: strict > keeps the lower id
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
        bi = __builtin_amdgcn_readfirstlane(bi);  // identical in every lane
        const int owner = bi % kWave, slot = bi / kWave;
        double s_own = sig[0];
#pragma unroll
        for (int i = 1; i < EPL; i++)
            if (i == slot) s_own = sig[i];
        const double ps = readlane_f64(s_own, owner);
        if (lane == owner) {
#pragma unroll
            for (int i = 0; i < EPL; i++)
                if (i == slot) live[i] = false;
        }
        if (lane == j) {
            my_id = bi;
            my_sig = ps;
        }
    }

    // adaptive top-p: rank of each pick by sig descending (equal sigs in slot order);
    // total and running sum in rank order; keep the shortest prefix reaching p * total
    const bool act = lane < a.k;
    int keff = a.k;
    bool keep = act;
    if (a.top_p > 0.0f && a.top_p < 1.0f) {
        int rank = 0;
        for (int i = 0; i < a.k; i++) {
            const double si = readlane_f64(my_sig, i);
            if (act && (si > my_sig || (si == my_sig && i < lane))) rank++;
        }
        double tot = 0.0;
        for (int r = 0; r < a.k; r++) {
            const unsigned long long m = __ballot(act && rank == r);
            tot += readlane_f64(my_sig, __ffsll((long long)m) - 1);
        }
        const double thr = (double)a.top_p * tot;
        double cum = 0.0;
        int kept = a.k;
        for (int r = 0; r < a.k; r++) {
            const unsigned long long m = __ballot(act && rank == r);
            cum += readlane_f64(my_sig, __ffsll((long long)m) - 1);
            if (cum >= thr) {
                kept = r + 1;
                break;
            }
        }
        keff = kept;
        keep = act && rank < kept;
    }

    // kept gates renormalised in slot order, then scaled; kept picks compacted
    const unsigned long long km = __ballot(keep);
    double denom = 0.0;
    for (int j = 0; j < a.k; j++)
        if ((km >> j) & 1ull) denom += readlane_f64(my_sig, j);
    const int pos = __popcll(km & ((1ull << lane) - 1ull));
    if (keep) {
        double g = my_sig;
        if (a.norm_topk) g = g / denom;
        g = g * (double)a.routed_scale;
        ids[pos] = my_id;
        w[pos] = (float)g;
        if (ids_copy) ids_copy[pos] = my_id;
    }
    if (act && lane >= keff) {
        ids[lane] = -1;
        w[lane] = 0.0f;
        if (ids_copy) ids_copy[lane] = -1;
    }
    if (lane == 0) {
        *keff_out = keff;
        if (keff_copy) *keff_copy = keff;
    }
}

// LDS words union_block needs for E experts and T tokens.
__host__ __device__ inline size_t union_lds_words(int E, int T) {
    const int W = (T + 31) / 32;
    return (size_t)E * W + 2 * (size_t)E + 1;
}

// The batch union ([R] §1.3), by a whole block: every kept (token, expert) pick
// sets a bit in a per-expert token bitmap (LDS atomicOr: the result does not
// depend on their order); counts are popcounts, offsets and the distinct-expert
// list exclusive scans by one wave; each expert's rows are then emitted in token
// order by one wave (a scan of per-word popcounts ranks every set bit), so the
// outputs need no atomics and are deterministic.  ids/keff may live in LDS or
// global memory.
__device__ __forceinline__ void union_block(const UnionArgs &a, const int32_t *ids,
                                            const int32_t *keff, uint32_t *lds) {
    const int E = a.E, T = a.T, k = a.k;
    const int W = (T + 31) / 32;
    uint32_t *hit = lds;                                              // [E][W]
    int32_t *cnt = reinterpret_cast<int32_t *>(hit + (size_t)E * W);  // [E]
    int32_t *offs = cnt + E;                                          // [E+1]
    const int tid = threadIdx.x;
    const int lane = tid % kWave, wave = tid / kWave, nwaves = blockDim.x / kWave;

    for (int i = tid; i < E * W; i += blockDim.x) hit[i] = 0u;
    __syncthreads();
    for (int p = tid; p < T * k; p += blockDim.x) {
        const int t = p / k, j = p % k;
        const int ke = min(max(keff[t], 0), k);
        const int e = ids[p];
        if (j < ke && e >= 0 && e < E) atomicOr(&hit[e * W + t / 32], 1u << (t % 32));
    }
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x) {
        int c = 0;
        for (int w = 0; w < W; w++) c += __popc(hit[e * W + w]);
        cnt[e] = c;
    }
    __syncthreads();

    // exclusive scans of counts and of (count > 0) by wave 0; E <= 256 = 4 per lane
    if (wave == 0) {
        int c[4], f[4], cs = 0, fs = 0;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int e = lane * 4 + i;
            c[i] = e < E ? cnt[e] : 0;
            f[i] = c[i] > 0 ? 1 : 0;
            cs += c[i];
            fs += f[i];
        }
        int ci = cs, fi = fs;  // inclusive scans over lanes
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int oc = __shfl_up(ci, d, kWave), of = __shfl_up(fi, d, kWave);
            if (lane >= d) {
                ci += oc;
                fi += of;
            }
        }
        int run = ci - cs, frun = fi - fs;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int e = lane * 4 + i;
            if (e < E) {
                offs[e] = run;
                a.off[e] = run;
                if (f[i]) a.uniq[frun] = e;
            }
            run += c[i];
            frun += f[i];
        }
        const int total = __shfl(ci, kWave - 1, kWave);
        const int nu = __shfl(fi, kWave - 1, kWave);
        if (lane == 0) {
            offs[E] = total;
            a.off[E] = total;
            a.n_uniq[0] = nu;
        }
        for (int i = nu + lane; i < E; i += kWave) a.uniq[i] = -1;
    }
    __syncthreads();

    const int rows = offs[E];
    for (int r = rows + tid; r < T * k; r += blockDim.x) a.row_tok[r] = -1;
    for (int p = tid; p < T * k; p += blockDim.x) {
        const int t = p / k, j = p % k;
        const int ke = min(max(keff[t], 0), k);
        const int e = ids[p];
        if (!(j < ke && e >= 0 && e < E)) a.pick_row[p] = -1;
    }

    // rows of each expert in token order
    for (int e = wave; e < E; e += nwaves) {
        if (cnt[e] == 0) continue;
        int run = offs[e];
        for (int w0 = 0; w0 < W; w0 += kWave) {
            const int w = w0 + lane;
            uint32_t bits = w < W ? hit[e * W + w] : 0u;
            const int pc = __popc(bits);
            int inc = pc;
#pragma unroll
            for (int d = 1; d < kWave; d <<= 1) {
                const int o = __shfl_up(inc, d, kWave);
                if (lane >= d) inc += o;
            }
            int r = run + inc - pc;
            while (bits) {
                const int b = __ffs(bits) - 1;
                bits &= bits - 1;
                const int t = w * 32 + b;
                a.row_tok[r] = t;
                const int ke = min(max(keff[t], 0), k);
                for (int j = 0; j < ke; j++)
                    if (ids[(size_t)t * k + j] == e) a.pick_row[(size_t)t * k + j] = r;
                r++;
            }
            run += __shfl(inc, kWave - 1, kWave);
        }
    }
}

}  // namespace moe

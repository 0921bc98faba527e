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

// Larger double -> larger unsigned key (finite values and -inf; NaN excluded).
__device__ __forceinline__ unsigned long long mono_key(double v) {
    const unsigned long long b = (unsigned long long)__double_as_longlong(v);
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// The sigmoid gate of a logit and the monotone key of its choice score ([R] §1.1:
// sig = 1 / (1 + exp(-logit)), choice = sig + bias), fp64.
__device__ __forceinline__ void gate_and_key(double l, const float *bias, int e, double &sig,
                                             unsigned long long &key) {
    sig = 1.0 / (1.0 + exp(-l));
    const double b = bias ? (double)bias[e] : 0.0;
    const double c = sig + b;
    key = mono_key(isnan(c) ? -INFINITY : c);
}

// Per-wave LDS scratch of select_token: the k picks, compacted (expert order), and the
// token's choice scores for the group scores of group-limited routing.
struct PickScratch {
    unsigned long long key[MOE_MAX_TOPK];
    double sig[MOE_MAX_TOPK];
    int id[MOE_MAX_TOPK];
    double choice[MOE_MAX_EXPERTS];
};

// The choice score a monotone key came from (mono_key inverted).
__device__ __forceinline__ double key_value(unsigned long long k) {
    const unsigned long long b = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
    return __longlong_as_double((long long)b);
}

// AND and OR of a 64-bit value over a whole wave (all 64 lanes active), as
// wave-uniform values: within each row of 16 lanes by DPP moves (swap neighbours,
// swap pairs, rotate by 4, rotate by 8), then the four rows' results read from lanes
// 0, 16, 32 and 48.  No LDS round trip; the results live in scalar registers.
__device__ __forceinline__ uint32_t row_reduce_and(uint32_t v) {
    v &= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
    v &= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
    v &= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, false);  // row_ror 4
    v &= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);  // row_ror 8
    return v;
}

__device__ __forceinline__ uint32_t row_reduce_or(uint32_t v) {
    v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
    v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
    v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, false);
    v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);
    return v;
}

__device__ __forceinline__ uint32_t rows_and(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 0) & (uint32_t)__builtin_amdgcn_readlane((int)v, 16) &
           (uint32_t)__builtin_amdgcn_readlane((int)v, 32) & (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
}

__device__ __forceinline__ uint32_t rows_or(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 0) | (uint32_t)__builtin_amdgcn_readlane((int)v, 16) |
           (uint32_t)__builtin_amdgcn_readlane((int)v, 32) | (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
}

__device__ __forceinline__ unsigned long long wave_and_u64(unsigned long long v) {
    const uint32_t lo = rows_and(row_reduce_and((uint32_t)v)), hi = rows_and(row_reduce_and((uint32_t)(v >> 32)));
    return ((unsigned long long)hi << 32) | lo;
}

__device__ __forceinline__ unsigned long long wave_or_u64(unsigned long long v) {
    const uint32_t lo = rows_or(row_reduce_or((uint32_t)v)), hi = rows_or(row_reduce_or((uint32_t)(v >> 32)));
    return ((unsigned long long)hi << 32) | lo;
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// One token, one wave.  [R] §1.1: sig = sigmoid(logit) and choice = sig + bias,
// in fp64; [R] §1.2: the k experts with the largest choice (the same set and order
// as k rounds of argmax excluding taken experts, equal scores going to the lower
// id), adaptive top-p over the k gates, norm_topk, routed scale.
// The k-th largest choice is found exactly by a bitwise search on monotone 64-bit
// keys (each step counts keys >= a candidate with one ballot per slot, stopping
// once exactly k keys qualify); the picks are then compacted and ranked (choice
// descending, lower id first).
// Lane j < k ends up holding pick j.  Writes ids/w (this token's k slots) and
// *keff; when ids_copy/keff_copy are given, the ids and keff are written there too.
// The logit of (t, e): the router's slice partials added in slice order.
__device__ __forceinline__ double sum_partials(const SelectArgs &a, int t, int e) {
    double l = 0.0;
    int s = 0;
    for (; s + 8 <= a.S; s += 8) {  // loads issued eight at a time
        double v[8];
#pragma unroll
        for (int u = 0; u < 8; u++) v[u] = a.part[((size_t)(s + u) * a.T + t) * a.E + e];
#pragma unroll
        for (int u = 0; u < 8; u++) l += v[u];
    }
    for (; s < a.S; s++) l += a.part[((size_t)s * a.T + t) * a.E + e];
    return l;
}

// lg: this token's E logits already summed (in LDS), or null to sum them here; both
// unused when the router gave the gates and keys.
// GROUPED: group-limited routing (a.n_group > 1), a separate instantiation so that the
// one-group selection on the decode critical path carries none of its code.
template <bool GROUPED>
__device__ __forceinline__ void select_token_impl(const SelectArgs &a, int t, int lane, int32_t *ids,
                                                  float *w, int32_t *keff_out, int32_t *ids_copy,
                                                  int32_t *keff_copy, PickScratch *ps,
                                                  const double *lg) {
    constexpr int EPL = MOE_MAX_EXPERTS / kWave;  // experts per lane (4)
    double sig[EPL];
    unsigned long long key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; i++) {
        const int e = lane + kWave * i;
        sig[i] = 0.0;
        key[i] = 0ull;  // below every live key
        if (e < a.E) {
            if (a.key_in) {  // computed by the router
                sig[i] = a.sig_in[(size_t)t * a.E + e];
                key[i] = a.key_in[(size_t)t * a.E + e];
            } else {
                gate_and_key(lg ? lg[e] : sum_partials(a, t, e), a.bias, e, sig[i], key[i]);
            }
        }
    }

    // Group-limited routing (n_group > 1; DeepSeek-V3's noaux_tc, [R] §1.2 has one group):
    // group g = experts [g*gs, (g+1)*gs); its score is the sum of its two largest choices;
    // the topk_group best groups (equal scores: lower id) stay, the other experts' keys
    // become 0, below every live key, so they are never picked.
    if constexpr (GROUPED) {
#pragma unroll
        for (int i = 0; i < EPL; i++) {
            const int e = lane + kWave * i;
            if (e < a.E) ps->choice[e] = key_value(key[i]);
        }
        wave_lds_sync();
        const int gs = a.E / a.n_group;
        double gscore = -INFINITY;
        if (lane < a.n_group) {
            double m1 = -INFINITY, m2 = -INFINITY;
            for (int j = 0; j < gs; j++) {
                const double c = ps->choice[lane * gs + j];
                if (c > m1) {
                    m2 = m1;
                    m1 = c;
                } else if (c > m2) {
                    m2 = c;
                }
            }
            gscore = m1 + m2;
        }
        int grank = 0;
        for (int g = 0; g < a.n_group; g++) {
            const double sg = readlane_f64(gscore, g);
            grank += (sg > gscore || (sg == gscore && g < lane)) ? 1 : 0;
        }
        const unsigned long long gkeep = __ballot(lane < a.n_group && grank < a.topk_group);
#pragma unroll
        for (int i = 0; i < EPL; i++) {
            const int e = lane + kWave * i;
            if (e < a.E && !((gkeep >> (e / gs)) & 1ull)) key[i] = 0ull;
        }
        wave_lds_sync();  // the choice scratch is read by every lane before it is reused
    }

    // thr = the k-th largest key: the largest value with at least k keys >= it, built
    // bit by bit.  As soon as exactly k keys are >= a candidate, those k are the picks
    // (no key equal to the k-th is left out), which ends the search early.  Bits above
    // the highest one in which the live keys differ are the same in all of them, so
    // thr starts with them and the search starts below (there are at least k live keys).
    // live keys: experts below E (and, grouped, in a kept group); every live key is nonzero
    auto live = [&](int i) __attribute__((always_inline)) {
        return GROUPED ? key[i] != 0ull : (lane + kWave * i) < a.E;
    };
    unsigned long long kand = ~0ull, kor = 0ull;
#pragma unroll
    for (int i = 0; i < EPL; i++)
        if (live(i)) {
            kand &= key[i];
            kor |= key[i];
        }
    kand = wave_and_u64(kand);
    kor = wave_or_u64(kor);
    const unsigned long long diff = kand ^ kor;
    const int top = diff ? 63 - __clzll((long long)diff) : -1;  // highest differing bit
    // All live keys equal (diff == 0, e.g. a zero token without bias): thr is that key
    // and there is nothing to search; the equal-key branch below takes the k lowest ids.
    unsigned long long thr = diff == 0 ? kor : (top >= 63 ? 0ull : kor & ~((2ull << top) - 1ull));
    bool exact = false;
    for (int bit = top; bit >= 0; bit--) {
        const unsigned long long cand = thr | (1ull << bit);
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < EPL; i++) cnt += __popcll(__ballot(key[i] >= cand));
        if (cnt >= a.k) thr = cand;
        if (cnt == a.k) {
            exact = true;
            break;
        }
    }
    // every key above thr is picked; among keys equal to thr the lowest ids fill up to k
    const unsigned long long below = (1ull << lane) - 1ull;
    bool sel[EPL];
    if (exact) {
#pragma unroll
        for (int i = 0; i < EPL; i++) sel[i] = key[i] >= thr;
    } else {
        int cgt = 0;
#pragma unroll
        for (int i = 0; i < EPL; i++) cgt += __popcll(__ballot(key[i] > thr));
        const int need = a.k - cgt;
        int eq_before = 0;
#pragma unroll
        for (int i = 0; i < EPL; i++) {
            const unsigned long long eqm = __ballot(key[i] == thr && live(i));
            const int r = eq_before + __popcll(eqm & below);
            sel[i] = key[i] > thr || (((eqm >> lane) & 1ull) && r < need);
            eq_before += __popcll(eqm);
        }
    }
    // compact the k picks into LDS (expert order): lane j < k then holds pick j.  Exactly
    // k experts are selected above; the bound keeps every store inside the k-entry scratch
    // whatever the keys are.
    int base = 0;
#pragma unroll
    for (int i = 0; i < EPL; i++) {
        const unsigned long long sm = __ballot(sel[i]);
        const int pos = base + (int)__popcll(sm & below);
        if (sel[i] && pos < a.k) {
            ps->key[pos] = key[i];
            ps->sig[pos] = sig[i];
            ps->id[pos] = lane + kWave * i;
        }
        base += (int)__popcll(sm);
    }
    wave_lds_sync();
    // rank of pick j (choice descending, equal choices by lower id): the k <= 16 picks
    // sit in lanes 0-15 (the rest padded with key 0 and the largest id, which no pick
    // ranks below), and each lane compares its pick with the other 15 lanes of that
    // row, rotated past it
    unsigned long long mk = 0ull;
    int mid = 0x7fffffff;
    double msig = 0.0;
    if (lane < a.k) {
        mk = ps->key[lane];
        mid = ps->id[lane];
        msig = ps->sig[lane];
    }
    const int mk_lo = (int)(uint32_t)mk, mk_hi = (int)(uint32_t)(mk >> 32);
    int rank = 0;
    // DPP row_ror:r (control 0x120 + r) gives each lane the value of lane (l + r) mod 16
    // of its row
#define MOE_RANK_STEP(r)                                                                \
    {                                                                                   \
        const uint32_t olo = (uint32_t)__builtin_amdgcn_mov_dpp(mk_lo, 0x120 + (r), 0xF, 0xF, false); \
        const uint32_t ohi = (uint32_t)__builtin_amdgcn_mov_dpp(mk_hi, 0x120 + (r), 0xF, 0xF, false); \
        const int oid = __builtin_amdgcn_mov_dpp(mid, 0x120 + (r), 0xF, 0xF, false);  \
        const unsigned long long ok = ((unsigned long long)ohi << 32) | olo;            \
        rank += (ok > mk || (ok == mk && oid < mid)) ? 1 : 0;                           \
    }
    MOE_RANK_STEP(1) MOE_RANK_STEP(2) MOE_RANK_STEP(3) MOE_RANK_STEP(4) MOE_RANK_STEP(5)
    MOE_RANK_STEP(6) MOE_RANK_STEP(7) MOE_RANK_STEP(8) MOE_RANK_STEP(9) MOE_RANK_STEP(10)
    MOE_RANK_STEP(11) MOE_RANK_STEP(12) MOE_RANK_STEP(13) MOE_RANK_STEP(14) MOE_RANK_STEP(15)
#undef MOE_RANK_STEP
    // slot r takes the pick of rank r: each pick is pushed to lane `rank`
    const int dst = lane < a.k ? rank : lane;
    const int my_id_p = __builtin_amdgcn_ds_permute(4 * dst, mid);
    const int sg_lo = __builtin_amdgcn_ds_permute(4 * dst, __double2loint(msig));
    const int sg_hi = __builtin_amdgcn_ds_permute(4 * dst, __double2hiint(msig));
    int my_id = -1;
    double my_sig = 0.0;
    if (lane < a.k) {
        my_id = my_id_p;
        my_sig = __hiloint2double(sg_hi, sg_lo);
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
        const double thr_p = (double)a.top_p * tot;
        double cum = 0.0;
        int kept = a.k;
        for (int r = 0; r < a.k; r++) {
            const unsigned long long m = __ballot(act && rank == r);
            cum += readlane_f64(my_sig, __ffsll((long long)m) - 1);
            if (cum >= thr_p) {
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
    const int pos = __popcll(km & below);
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

__device__ __forceinline__ void select_token(const SelectArgs &a, int t, int lane, int32_t *ids,
                                             float *w, int32_t *keff_out, int32_t *ids_copy,
                                             int32_t *keff_copy, PickScratch *ps,
                                             const double *lg = nullptr) {
    if (a.n_group > 1)
        select_token_impl<true>(a, t, lane, ids, w, keff_out, ids_copy, keff_copy, ps, lg);
    else
        select_token_impl<false>(a, t, lane, ids, w, keff_out, ids_copy, keff_copy, ps, lg);
}

// LDS words union_block needs for E experts and T tokens.
__host__ __device__ inline size_t union_lds_words(int E, int T) {
    const int W = (T + 31) / 32;
    const int W8 = (W + 7) / 8;
    return (size_t)E * W + (size_t)E * W8 + 2 * (size_t)E + 1;
}

// The batch union ([R] §1.3), by a whole block: every kept (token, expert) pick
// sets a bit in a per-expert token bitmap (LDS atomicOr: the result does not
// depend on their order); counts are popcounts, offsets and the distinct-expert
// list exclusive scans by one wave.  A pick's row is its expert's offset plus the
// number of earlier tokens of that expert -- a per-8-word prefix count plus at
// most eight popcounts -- so every pick is placed independently, without atomics,
// and the result is deterministic.  ids/keff may live in LDS or global memory.
__device__ __forceinline__ void union_block(const UnionArgs &a, const int32_t *ids,
                                            const int32_t *keff, uint32_t *lds) {
    const int E = a.E, T = a.T, k = a.k;
    const int W = (T + 31) / 32;
    const int W8 = (W + 7) / 8;
    uint32_t *hit = lds;                                              // [E][W]
    int32_t *pre8 = reinterpret_cast<int32_t *>(hit + (size_t)E * W); // [E][W8]
    int32_t *cnt = pre8 + (size_t)E * W8;                             // [E]
    int32_t *offs = cnt + E;                                          // [E+1]
    const int tid = threadIdx.x;
    const int lane = tid % kWave, wave = tid / kWave;

    for (int i = tid; i < E * W; i += blockDim.x) hit[i] = 0u;
    __syncthreads();
    for (int p = tid; p < T * k; p += blockDim.x) {
        const int t = p / k, j = p % k;
        const int ke = min(max(keff[t], 0), k);
        const int e = ids[p];
        if (j < ke && e >= 0 && e < E) atomicOr(&hit[e * W + t / 32], 1u << (t % 32));
    }
    __syncthreads();
    // per expert: running popcount, recorded every 8 words, and the total
    for (int e = tid; e < E; e += blockDim.x) {
        int c = 0;
        for (int w = 0; w < W; w++) {
            if (w % 8 == 0) pre8[e * W8 + w / 8] = c;
            c += __popc(hit[e * W + w]);
        }
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
    // every pick: row = off[e] + (tokens before t routed to e); rows run (expert, token)
    for (int p = tid; p < T * k; p += blockDim.x) {
        const int t = p / k, j = p % k;
        const int ke = min(max(keff[t], 0), k);
        const int e = ids[p];
        if (!(j < ke && e >= 0 && e < E)) {
            a.pick_row[p] = -1;
            continue;
        }
        const int w = t / 32;
        const uint32_t *he = hit + (size_t)e * W;
        int rank = pre8[e * W8 + w / 8];
        for (int v = (w / 8) * 8; v < w; v++) rank += __popc(he[v]);
        rank += __popc(he[w] & ((1u << (t % 32)) - 1u));
        const int r = offs[e] + rank;
        a.pick_row[p] = r;
        a.row_tok[r] = t;
    }
}

}  // namespace moe

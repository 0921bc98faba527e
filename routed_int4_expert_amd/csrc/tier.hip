// tier.hip -- the expert residency tier on gfx950: HBM slots as a per-layer cache over
// an expert bank in pinned host memory ("MoE 路由与专家流式加载" §1.3 cache resolution,
// §3 multi-level expert cache, §4 tier repin, §5 router-lookahead prefetch;
// "colibri 开发演进实录" §2.1 VRAM expert tier).
//
// Everything is decided on the device, right after the batch union, so a forward never
// waits for the host:
//  - resolve (one workgroup): every union expert, in ascending id order, is a hit (its
//    slot is stamped with the step) or a miss; misses take the slots that are neither
//    pinned nor holding an expert of this union, least recently used first (empty
//    slots, then the smallest stamp, then the lower slot index: one bitonic sort of
//    (stamp, slot) keys), and are listed for copying.  Heat and usage grow by each
//    union expert's row count.  The table of slot pointers the expert FFNs read is
//    written for every union expert;
//  - copy (many workgroups): each listed expert's six tensors are read from host memory
//    with 16-byte loads (several in flight per thread) and written into its slot;
//  - repin (one workgroup): the coldest pinned expert gives way to the hottest unpinned
//    one when the heat difference passes the 25 % + 4 hysteresis, at most four times a
//    pass, then every heat is halved;
//  - init (one workgroup): all slots empty, then the caller's pins in the first slots.
// A slot's layout is TierLayout: gate codes, gate scales, up codes, up scales, down
// codes, down scales, each 256-byte aligned.
#include "moe_internal.h"

namespace moe {

struct TierView {
    int32_t *hdr, *slot_expert, *slot_pinned, *slot_used, *expert_slot, *copies;
    uint32_t *heat, *usage;
    moe_q4 *tab;
};

__device__ __forceinline__ TierView tier_view(const TierArgs &a) {
    TierView v;
    uint8_t *b = a.state;
    v.hdr = reinterpret_cast<int32_t *>(b + a.lay.hdr);
    v.slot_expert = reinterpret_cast<int32_t *>(b + a.lay.slot_expert);
    v.slot_pinned = reinterpret_cast<int32_t *>(b + a.lay.slot_pinned);
    v.slot_used = reinterpret_cast<int32_t *>(b + a.lay.slot_used);
    v.expert_slot = reinterpret_cast<int32_t *>(b + a.lay.expert_slot);
    v.heat = reinterpret_cast<uint32_t *>(b + a.lay.heat);
    v.usage = reinterpret_cast<uint32_t *>(b + a.lay.usage);
    v.copies = reinterpret_cast<int32_t *>(b + a.lay.copies);
    v.tab = reinterpret_cast<moe_q4 *>(b + a.lay.tab);
    return v;
}

// expert e's three matrices in slot s
__device__ __forceinline__ void tier_point(const TierArgs &a, const TierView &v, int e, int s) {
    uint8_t *sl = a.slots + (size_t)s * a.lay.slot;
    v.tab[3 * e + 0].q = sl + a.lay.gq;
    v.tab[3 * e + 0].s = sl + a.lay.gs;
    v.tab[3 * e + 1].q = sl + a.lay.uq;
    v.tab[3 * e + 1].s = sl + a.lay.us;
    v.tab[3 * e + 2].q = sl + a.lay.dq;
    v.tab[3 * e + 2].s = sl + a.lay.ds;
}

// expert e's matrices in the backing store (read over the host link; used only when no
// slot is free, which the host-side checks rule out)
__device__ __forceinline__ void tier_point_backing(const TierArgs &a, const TierView &v, int e) {
    v.tab[3 * e + 0] = fmt_stack_at(a.gate, a.fmt, e, a.F, a.H);
    v.tab[3 * e + 1] = fmt_stack_at(a.up, a.fmt, e, a.F, a.H);
    v.tab[3 * e + 2] = fmt_stack_at(a.down, a.fmt, e, a.H, a.F);
}

// ------------------------------------------------------------------ init
__global__ __launch_bounds__(1024) void tier_init_kernel(TierArgs a, TierPins pins, int n_pin) {
    const TierView v = tier_view(a);
    const int S = a.lay.S, E = a.lay.E;
    for (int i = threadIdx.x; i < 16; i += blockDim.x) v.hdr[i] = 0;
    for (int s = threadIdx.x; s < S; s += blockDim.x) {
        v.slot_expert[s] = -1;
        v.slot_pinned[s] = 0;
        v.slot_used[s] = -1;
    }
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        v.expert_slot[e] = -1;
        v.heat[e] = 0u;
        v.usage[e] = 0u;
    }
    __syncthreads();
    for (int s = threadIdx.x; s < n_pin; s += blockDim.x) {
        const int e = pins.id[s];
        v.slot_expert[s] = e;
        v.slot_pinned[s] = 1;
        v.slot_used[s] = 0;
        v.expert_slot[e] = s;
        v.copies[2 * s] = e;
        v.copies[2 * s + 1] = s;
        tier_point(a, v, e, s);
    }
    if (threadIdx.x == 0) {
        v.hdr[1] = n_pin;
        v.hdr[6] = S;
        v.hdr[7] = E;
    }
}

// ------------------------------------------------------------------ resolve
// One workgroup of 1024 threads (E <= 256 union experts, S <= 1024 slots).
__global__ __launch_bounds__(1024) void tier_resolve_kernel(TierArgs a, TierResolveIn in) {
    __shared__ int ue[MOE_MAX_EXPERTS];         // union experts, ascending
    __shared__ int ucnt[MOE_MAX_EXPERTS];       // their row counts (forward)
    __shared__ int umiss[MOE_MAX_EXPERTS];      // miss rank, or -1 for a hit
    __shared__ int flag[MOE_MAX_EXPERTS];
    __shared__ int inuse[kTierMaxSlots];
    __shared__ unsigned long long key[kTierMaxSlots];
    __shared__ int s_nu, s_ncand;
    const TierView v = tier_view(a);
    const int S = a.lay.S, E = a.lay.E;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;

    // ---- the experts to resolve, ascending
    for (int s = tid; s < S; s += blockDim.x) inuse[s] = 0;
    if (in.prefetch) {
        for (int e = tid; e < E; e += blockDim.x) flag[e] = 0;
        __syncthreads();
        for (int p = tid; p < in.T * in.k; p += blockDim.x) {
            const int t = p / in.k, j = p % in.k;
            const int ke = min(max(in.keff[t], 0), in.k);
            const int e = in.ids[p];
            if (j < ke && e >= 0 && e < E) flag[e] = 1;
        }
        __syncthreads();
        if (wave == 0) {  // ascending compaction: E <= 256, four experts per lane
            int f[4], c = 0;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int e = 4 * lane + i;
                f[i] = e < E ? flag[e] : 0;
                c += f[i];
            }
            int inc = c;
#pragma unroll
            for (int d = 1; d < kWave; d <<= 1) {
                const int o = __shfl_up(inc, d, kWave);
                if (lane >= d) inc += o;
            }
            int pos = inc - c;
#pragma unroll
            for (int i = 0; i < 4; i++)
                if (f[i]) {
                    ue[pos] = 4 * lane + i;
                    ucnt[pos] = 0;
                    pos++;
                }
            if (lane == kWave - 1) s_nu = inc;
        }
    } else {
        if (tid == 0) s_nu = min(max(in.n_uniq[0], 0), E);
        __syncthreads();
        for (int i = tid; i < s_nu; i += blockDim.x) {
            const int e = in.uniq[i];
            ue[i] = e;
            ucnt[i] = in.off[e + 1] - in.off[e];
        }
    }
    __syncthreads();
    const int nu = s_nu;
    const int step = v.hdr[0] + (in.prefetch ? 0 : 1);

    // ---- hits are stamped; the union's slots are off limits as victims
    for (int i = tid; i < nu; i += blockDim.x) {
        const int e = ue[i];
        const int s = v.expert_slot[e];
        if (!in.prefetch) {
            v.heat[e] += (uint32_t)ucnt[i];
            v.usage[e] += (uint32_t)ucnt[i];
        }
        umiss[i] = s >= 0 ? -1 : 0;
        if (s >= 0) {
            inuse[s] = 1;
            v.slot_used[s] = step;
        }
    }
    __syncthreads();
    // miss ranks in union order (wave 0: four entries per lane)
    if (wave == 0) {
        int m[4], c = 0;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int u = 4 * lane + i;
            m[i] = (u < nu && umiss[u] == 0) ? 1 : 0;
            c += m[i];
        }
        int inc = c;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int o = __shfl_up(inc, d, kWave);
            if (lane >= d) inc += o;
        }
        int r = inc - c;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int u = 4 * lane + i;
            if (u < nu) umiss[u] = m[i] ? r : -1;
            r += m[i];
        }
    }
    // ---- victims: slots neither pinned nor in use, (stamp, slot) ascending
    int P = 1;
    while (P < S) P <<= 1;
    if (tid == 0) s_ncand = 0;
    __syncthreads();
    int my_cand = 0;
    for (int s = tid; s < P; s += blockDim.x) {
        const bool cand = s < S && !v.slot_pinned[s] && !inuse[s];
        key[s] = cand ? ((unsigned long long)(uint32_t)(v.slot_used[s] + 1) << 32) | (uint32_t)s : ~0ull;
        my_cand += cand ? 1 : 0;
    }
    if (my_cand) atomicAdd(&s_ncand, my_cand);
    __syncthreads();
    for (int kk = 2; kk <= P; kk <<= 1) {
        for (int j = kk >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < P; i += blockDim.x) {
                const int ixj = i ^ j;
                if (ixj > i) {
                    const unsigned long long x = key[i], y = key[ixj];
                    const bool up = (i & kk) == 0;
                    if ((x > y) == up) {
                        key[i] = y;
                        key[ixj] = x;
                    }
                }
            }
            __syncthreads();
        }
    }
    const int ncand = s_ncand;

    // ---- misses take their victims; every union expert's table entry
    int hits = 0, miss = 0;
    for (int i = tid; i < nu; i += blockDim.x) {
        const int e = ue[i];
        const int r = umiss[i];
        if (r < 0) {
            tier_point(a, v, e, v.expert_slot[e]);
            hits++;
            continue;
        }
        miss++;
        if (r < ncand) {
            const int s = (int)(uint32_t)key[r];
            const int old = v.slot_expert[s];
            if (old >= 0) v.expert_slot[old] = -1;
            v.expert_slot[e] = s;
            v.slot_expert[s] = e;
            v.slot_used[s] = step;
            v.copies[2 * r] = e;
            v.copies[2 * r + 1] = s;
            tier_point(a, v, e, s);
        } else {
            tier_point_backing(a, v, e);
        }
    }
    // totals by LDS atomics
    __shared__ int s_hit, s_miss;
    if (tid == 0) {
        s_hit = 0;
        s_miss = 0;
    }
    __syncthreads();
    if (hits) atomicAdd(&s_hit, hits);
    if (miss) atomicAdd(&s_miss, miss);
    __syncthreads();
    if (tid == 0) {
        const int copies = min(s_miss, ncand);
        v.hdr[1] = copies;
        if (in.prefetch) {
            v.hdr[5] += copies;
        } else {
            v.hdr[0] = step;
            v.hdr[2] += s_hit;
            v.hdr[3] += s_miss;
        }
    }
}

// ------------------------------------------------------------------ repin
// One workgroup of 256 threads.  [R] §4: tier_pick_swap with the 25 % + 4 hysteresis,
// at most max_swaps exchanges, then tier_decay (heat >>= 1).
__global__ __launch_bounds__(256) void tier_repin_kernel(TierArgs a, int max_swaps) {
    __shared__ unsigned long long red[256 / kWave];
    __shared__ int s_go, s_nc;
    const TierView v = tier_view(a);
    const int S = a.lay.S, E = a.lay.E;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    if (tid == 0) s_nc = 0;
    auto block_min = [&](unsigned long long x) {
        for (int m = kWave / 2; m > 0; m >>= 1) {
            const unsigned long long o = __shfl_xor(x, m, kWave);
            x = o < x ? o : x;
        }
        __syncthreads();
        if (lane == 0) red[wave] = x;
        __syncthreads();
        unsigned long long r = red[0];
        for (int w = 1; w < (int)(blockDim.x / kWave); w++) r = red[w] < r ? red[w] : r;
        return r;
    };
    for (int it = 0; it < max_swaps; it++) {
        // coldest pinned expert: smallest (heat, id)
        unsigned long long kc = ~0ull;
        for (int s = tid; s < S; s += blockDim.x)
            if (v.slot_pinned[s]) {
                const int e = v.slot_expert[s];
                const unsigned long long k = ((unsigned long long)v.heat[e] << 32) | (uint32_t)e;
                kc = k < kc ? k : kc;
            }
        kc = block_min(kc);
        // hottest unpinned expert: largest heat, then smallest id; as a minimum of
        // (~heat, id)
        unsigned long long kh = ~0ull;
        for (int e = tid; e < E; e += blockDim.x) {
            const int s = v.expert_slot[e];
            if (s >= 0 && v.slot_pinned[s]) continue;
            const unsigned long long k = ((unsigned long long)(~v.heat[e]) << 32) | (uint32_t)e;
            kh = k < kh ? k : kh;
        }
        kh = block_min(kh);
        if (tid == 0) {
            s_go = 0;
            if (kc != ~0ull && kh != ~0ull) {
                const int fc = (int)(uint32_t)kc, fh = (int)(uint32_t)kh;
                const unsigned long long hc = v.heat[fc], hh = v.heat[fh];
                if (hh > hc + hc / 4 + 4) {
                    const int sc = v.expert_slot[fc], s2 = v.expert_slot[fh];
                    if (s2 >= 0) {  // fh is cached: it takes over the pinned flag
                        v.slot_pinned[s2] = 1;
                        v.slot_pinned[sc] = 0;
                    } else {        // fh is copied into fc's slot; fc leaves HBM
                        v.expert_slot[fc] = -1;
                        v.expert_slot[fh] = sc;
                        v.slot_expert[sc] = fh;
                        v.slot_used[sc] = v.hdr[0];
                        v.copies[2 * s_nc] = fh;
                        v.copies[2 * s_nc + 1] = sc;
                        tier_point(a, v, fh, sc);
                        s_nc++;
                    }
                    v.hdr[4] += 1;
                    s_go = 1;
                }
            }
        }
        __syncthreads();
        if (!s_go) break;
    }
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x) v.heat[e] >>= 1;
    if (tid == 0) v.hdr[1] = s_nc;
}

// ------------------------------------------------------------------ copy
// Grid (blocks per job, jobs).  Job j < hdr[1] copies expert copies[2j] from the
// backing store into slot copies[2j+1]: six tensors, each strided over the job's
// workgroups with four 16-byte loads in flight per thread before the stores.
__global__ __launch_bounds__(256) void tier_copy_kernel(TierArgs a) {
    const TierView v = tier_view(a);
    const int job = blockIdx.y;
    if (job >= v.hdr[1]) return;
    const int e = v.copies[2 * job], s = v.copies[2 * job + 1];
    uint8_t *sl = a.slots + (size_t)s * a.lay.slot;
    // every matrix of the three takes F * code bytes(H) and F * scale bytes(H), multiples of 16
    const size_t nq = (size_t)a.F * fmt_code_bytes(a.fmt, a.H) / 16, ns = (size_t)a.F * fmt_scale_bytes(a.fmt, a.H) / 16;
    const moe_q4 g = fmt_stack_at(a.gate, a.fmt, e, a.F, a.H), u = fmt_stack_at(a.up, a.fmt, e, a.F, a.H),
                 d = fmt_stack_at(a.down, a.fmt, e, a.H, a.F);
    const uint4 *src[6] = {
        reinterpret_cast<const uint4 *>(g.q), static_cast<const uint4 *>(g.s),
        reinterpret_cast<const uint4 *>(u.q), static_cast<const uint4 *>(u.s),
        reinterpret_cast<const uint4 *>(d.q), static_cast<const uint4 *>(d.s)};
    const size_t dst_off[6] = {a.lay.gq, a.lay.gs, a.lay.uq, a.lay.us, a.lay.dq, a.lay.ds};
    const size_t n16[6] = {nq, ns, nq, ns, nq, ns};
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (int m = 0; m < 6; m++) {
        const uint4 *sp = src[m];
        uint4 *dp = reinterpret_cast<uint4 *>(sl + dst_off[m]);
        size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
        for (; i + 3 * stride < n16[m]; i += 4 * stride) {
            uint4 w[4];
#pragma unroll
            for (int u = 0; u < 4; u++) w[u] = sp[i + u * stride];
#pragma unroll
            for (int u = 0; u < 4; u++) dp[i + u * stride] = w[u];
        }
        for (; i < n16[m]; i += stride) dp[i] = sp[i];
    }
}

hipError_t launch_tier_init(const TierArgs &a, const TierPins &pins, int n_pin, hipStream_t st) {
    ProfScope prof("tier_init", st);
    tier_init_kernel<<<1, 1024, 0, st>>>(a, pins, n_pin);
    return hipGetLastError();
}

hipError_t launch_tier_resolve(const TierArgs &a, const TierResolveIn &in, hipStream_t st) {
    ProfScope prof(in.prefetch ? "tier_prefetch_resolve" : "tier_resolve", st);
    tier_resolve_kernel<<<1, 1024, 0, st>>>(a, in);
    return hipGetLastError();
}

hipError_t launch_tier_repin(const TierArgs &a, int max_swaps, hipStream_t st) {
    ProfScope prof("tier_repin", st);
    tier_repin_kernel<<<1, 256, 0, st>>>(a, max_swaps);
    return hipGetLastError();
}

hipError_t launch_tier_copy(const TierArgs &a, int max_jobs, hipStream_t st) {
    if (max_jobs <= 0) return hipSuccess;
    // about 256 KB of an expert per workgroup, at most 256 workgroups per job
    const size_t per = a.lay.slot / (256u << 10);
    const int bpj = (int)(per < 1 ? 1 : (per > 256 ? 256 : per));
    ProfScope prof("tier_copy", st);
    tier_copy_kernel<<<dim3(bpj, max_jobs), 256, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace moe

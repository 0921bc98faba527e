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
#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(1024) void union_kernel(UnionArgs a) {
    extern __shared__ uint32_t lds[];
    const int E = a.E, T = a.T, k = a.k;
    const int W = (T + 31) / 32;
    uint32_t *hit = lds;                               // [E][W]
    int32_t *cnt = reinterpret_cast<int32_t *>(hit + (size_t)E * W);  // [E]
    int32_t *offs = cnt + E;                           // [E+1]
    const int tid = threadIdx.x;
    const int lane = tid % kWave, wave = tid / kWave, nwaves = blockDim.x / kWave;

    for (int i = tid; i < E * W; i += blockDim.x) hit[i] = 0u;
    __syncthreads();
    for (int p = tid; p < T * k; p += blockDim.x) {
        const int t = p / k, j = p % k;
        const int ke = min(max(a.keff[t], 0), k);
        const int e = a.ids[p];
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
        const int ke = min(max(a.keff[t], 0), k);
        const int e = a.ids[p];
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
                const int ke = min(max(a.keff[t], 0), k);
                for (int j = 0; j < ke; j++)
                    if (a.ids[(size_t)t * k + j] == e) a.pick_row[(size_t)t * k + j] = r;
                r++;
            }
            run += __shfl(inc, kWave - 1, kWave);
        }
    }
}

size_t union_lds_bytes(int E, int T) {
    const int W = (T + 31) / 32;
    return sizeof(uint32_t) * (size_t)E * W + sizeof(int32_t) * (2 * (size_t)E + 1);
}

hipError_t launch_union(const UnionArgs &a, hipStream_t st) {
    const size_t lds = union_lds_bytes(a.E, a.T);
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

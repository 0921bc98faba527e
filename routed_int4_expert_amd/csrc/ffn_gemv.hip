// ffn_gemv.hip -- step 4 of the MoE layer on gfx950 for small row counts: the
// int4-gs64 SwiGLU expert FFN as grouped dequantising GEMVs
// ("MoE 路由与专家流式加载" §1.3: gate, up, SiLU, down per union expert; §1.4: the
// shared expert on every token).
//
// Work unit = (expert of the union or the shared expert, block of output rows).
// The unit's token rows (at most RM at a time) are staged once per workgroup in
// LDS as fp32; each weight row is streamed from HBM exactly once per RM rows,
// with LPR lanes per row each issuing coalesced 16-byte loads of 32 codes, so a
// wave's load covers LPR*16 contiguous bytes of one row.
//
// Codes: a byte holds elements 2j (low nibble) and 2j+1 (high nibble) as
// two's-complement int4 ("colibrì 深度拆解" §5.2).  XOR with 0x8 turns a code q
// into u = q + 8 in [0, 15], so a 32-element partial dot is
//   sum(q x) = sum(u x) - 8 sum(x)
// (the unsigned-offset identity of "colibri 开发演进实录" §2.2, K1), with u
// converted by the byte-to-float instruction and sum(x) precomputed per 32
// elements while staging.  The fp32 gs64 scale multiplies each 32-element
// partial (two per 64-group), all in fp32.
//
// The gate/up kernel finishes with the fused SiLU(g) * u epilogue and writes
// h [rows][F]; the down kernel writes the unweighted y [rows][H].  Each output
// is reduced inside one lane group in a fixed order (deterministic).
#include <math.h>

#include "moe_internal.h"

namespace moe {

// LDS row layout: 32-float chunks padded to 36 floats (the pad slot 32 holds the
// chunk's sum), so the 16-byte reads of 8 consecutive lanes hit distinct banks.
constexpr int kChunkPitch = 36;

__device__ __forceinline__ float dot32_offset(const uint4 q, const float4 *xv) {
    const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int d = 0; d < 4; d++) {
        const uint32_t u = wd[d] ^ 0x88888888u;
        const uint32_t lo = u & 0x0F0F0F0Fu;          // elements 0,2,4,6 of this word
        const uint32_t hi = (u >> 4) & 0x0F0F0F0Fu;   // elements 1,3,5,7
        const float4 a = xv[2 * d], b = xv[2 * d + 1];
        s0 = fmaf((float)(lo & 0xFFu), a.x, s0);
        s1 = fmaf((float)(hi & 0xFFu), a.y, s1);
        s0 = fmaf((float)((lo >> 8) & 0xFFu), a.z, s0);
        s1 = fmaf((float)((hi >> 8) & 0xFFu), a.w, s1);
        s0 = fmaf((float)((lo >> 16) & 0xFFu), b.x, s0);
        s1 = fmaf((float)((hi >> 16) & 0xFFu), b.y, s1);
        s0 = fmaf((float)(lo >> 24), b.z, s0);
        s1 = fmaf((float)(hi >> 24), b.w, s1);
    }
    return s0 + s1;
}

template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int m = LPR / 2; m > 0; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

// Outputs per lane group per pass: enough rows in flight for ~8 loads per lane.
template <int LPR, bool GU>
struct GemvShape {
    static constexpr int G = kWave / LPR;                     // lane groups per wave
    static constexpr int NF = (LPR >= 16 ? LPR / 16 : 1) * (GU ? 1 : 2);
    static constexpr int NM = GU ? 2 : 1;                     // matrices per output
    static constexpr int WF = G * NF;                         // outputs per wave
    static constexpr int BF = 4 * WF;                         // outputs per workgroup
};

template <int LPR, int RM, bool GU>
__global__ __launch_bounds__(256) void q4_gemv_kernel(FfnArgs a) {
    using S = GemvShape<LPR, GU>;
    extern __shared__ float xs[];  // [RM][C * kChunkPitch]
    const int unit = blockIdx.y;
    const int H = a.H;

    // ---- the unit: a routed expert of the union, or the shared expert
    int nrows, Fu;
    const int32_t *rt;
    moe_q4 m0, m1;
    const float *xin;   // row source for K
    float *out;         // output rows
    size_t out_row0;    // first output row index
    if (unit < a.max_units) {
        if (!a.with_routed || unit >= a.n_uniq[0]) return;
        const int e = a.uniq[unit];
        const int r0 = a.off[e];
        nrows = a.off[e + 1] - r0;
        Fu = a.F;
        if (GU) {
            const size_t gq = (size_t)e * Fu * (H / 2), gs = (size_t)e * Fu * (H / 64);
            m0.q = a.gate.q + gq; m0.s = a.gate.s + gs;
            m1.q = a.up.q + gq;   m1.s = a.up.s + gs;
            rt = a.row_tok + r0;
            xin = a.x;
            out = a.h_routed;
        } else {
            const size_t dq = (size_t)e * H * (Fu / 2), ds = (size_t)e * H * (Fu / 64);
            m0.q = a.down.q + dq; m0.s = a.down.s + ds;
            m1 = m0;
            rt = nullptr;
            xin = a.h_routed + (size_t)r0 * Fu;
            out = a.y_routed;
        }
        out_row0 = (size_t)r0;
    } else {
        if (!a.with_shared) return;
        nrows = a.T;
        Fu = a.Fs;
        if (GU) {
            m0 = a.sh_gate; m1 = a.sh_up;
            xin = a.x;
            out = a.h_shared;
        } else {
            m0 = a.sh_down; m1 = m0;
            xin = a.h_shared;
            out = a.y_shared;
        }
        rt = nullptr;
        out_row0 = 0;
    }
    const int K = GU ? H : Fu;      // reduction length
    const int N = GU ? Fu : H;      // outputs of this unit
    const int C = K / 32;           // 32-element chunks per row
    const int nb0 = blockIdx.x * S::BF;
    if (nb0 >= N) return;

    const int tid = threadIdx.x;
    const int lane = tid % kWave, wv = tid / kWave;
    const int sub = lane % LPR, grp = lane / LPR;
    const int rowpitch = C * kChunkPitch;

    for (int rc = 0; rc < nrows; rc += RM) {
        const int R = min(RM, nrows - rc);
        __syncthreads();  // previous rows fully consumed
        // stage R input rows (fp32) into the padded LDS layout
        for (int i = tid; i < R * (K / 4); i += blockDim.x) {
            const int r = i / (K / 4), c4 = i % (K / 4);
            const int src = rt ? rt[rc + r] : rc + r;
            const float4 v = *reinterpret_cast<const float4 *>(xin + (size_t)src * K + 4 * c4);
            *reinterpret_cast<float4 *>(xs + r * rowpitch + (c4 / 8) * kChunkPitch + (c4 % 8) * 4) = v;
        }
        __syncthreads();
        for (int i = tid; i < R * C; i += blockDim.x) {
            const int r = i / C, c = i % C;
            const float *p = xs + r * rowpitch + c * kChunkPitch;
            // even and odd elements summed in the order dot32_offset accumulates them, so a
            // group of zero codes (u = 8 everywhere) cancels to exactly 0
            float se = 0.f, so = 0.f;
#pragma unroll
            for (int q = 0; q < 32; q += 2) {
                se += p[q];
                so += p[q + 1];
            }
            xs[r * rowpitch + c * kChunkPitch + 32] = se + so;
        }
        __syncthreads();

        float acc[S::NF][S::NM][RM];
#pragma unroll
        for (int f = 0; f < S::NF; f++)
#pragma unroll
            for (int m = 0; m < S::NM; m++)
#pragma unroll
                for (int r = 0; r < RM; r++) acc[f][m][r] = 0.f;

        int nidx[S::NF];
#pragma unroll
        for (int f = 0; f < S::NF; f++) nidx[f] = nb0 + wv * S::WF + f * S::G + grp;

        for (int c = sub; c < C; c += LPR) {
            uint4 q[S::NF][S::NM];
            float sc[S::NF][S::NM];
#pragma unroll
            for (int f = 0; f < S::NF; f++) {
                const int n = min(nidx[f], N - 1);  // rows past N compute garbage, never stored
#pragma unroll
                for (int m = 0; m < S::NM; m++) {
                    const moe_q4 &mm = m == 0 ? m0 : m1;
                    q[f][m] = *reinterpret_cast<const uint4 *>(mm.q + (size_t)n * (K / 2) + 16 * c);
                    sc[f][m] = mm.s[(size_t)n * (K / 64) + (c >> 1)];
                }
            }
#pragma unroll
            for (int r = 0; r < RM; r++) {
                if (r < R) {
                    const float *p = xs + r * rowpitch + c * kChunkPitch;
                    float4 xv[8];
#pragma unroll
                    for (int v = 0; v < 8; v++) xv[v] = *reinterpret_cast<const float4 *>(p + 4 * v);
                    const float sx8 = 8.0f * p[32];
#pragma unroll
                    for (int f = 0; f < S::NF; f++)
#pragma unroll
                        for (int m = 0; m < S::NM; m++)
                            acc[f][m][r] = fmaf(sc[f][m], dot32_offset(q[f][m], xv) - sx8, acc[f][m][r]);
                }
            }
        }
#pragma unroll
        for (int f = 0; f < S::NF; f++)
#pragma unroll
            for (int m = 0; m < S::NM; m++)
#pragma unroll
                for (int r = 0; r < RM; r++) acc[f][m][r] = group_sum<LPR>(acc[f][m][r]);

        if (sub == 0) {
#pragma unroll
            for (int f = 0; f < S::NF; f++) {
                const int n = nidx[f];
                if (n >= N) continue;
#pragma unroll
                for (int r = 0; r < RM; r++) {
                    if (r >= R) continue;
                    float v;
                    if (GU) {
                        const float g = acc[f][0][r], u = acc[f][S::NM - 1][r];
                        v = g / (1.0f + expf(-g)) * u;
                    } else {
                        v = acc[f][0][r];
                    }
                    out[(out_row0 + rc + r) * (size_t)N + n] = v;
                }
            }
        }
    }
}

static int lanes_per_row(int K) {
    const int C = K / 32;
    int l = 64;
    while (l > 2 && l > C) l >>= 1;
    return l;
}

static int rows_per_pass(int T, int K) {
    const size_t row_bytes = (size_t)(K / 32) * kChunkPitch * sizeof(float);
    int rm = T >= 3 ? 4 : (T == 2 ? 2 : 1);
    while (rm > 1 && (size_t)rm * row_bytes > 160 * 1024) rm >>= 1;
    return rm;
}

template <int LPR, int RM, bool GU>
static hipError_t launch_one(const FfnArgs &a, int N, int K, hipStream_t st) {
    using S = GemvShape<LPR, GU>;
    const size_t lds = (size_t)RM * (K / 32) * kChunkPitch * sizeof(float);
    if (lds > 64 * 1024) {
        // raise the dynamic-LDS cap for this kernel; the launch itself reports a real failure
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&q4_gemv_kernel<LPR, RM, GU>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        (void)hipGetLastError();
    }
    dim3 grid((N + S::BF - 1) / S::BF, a.max_units + 1);
    ProfScope prof(GU ? "ffn_gateup" : "ffn_down", st);
    q4_gemv_kernel<LPR, RM, GU><<<grid, 256, lds, st>>>(a);
    return hipGetLastError();
}

template <bool GU>
static hipError_t dispatch(const FfnArgs &a, int N, int K, int rm, hipStream_t st) {
    const int lpr = lanes_per_row(K);
#define MOE_GEMV_CASE(L)                                                  \
    if (lpr == L) {                                                       \
        if (rm == 1) return launch_one<L, 1, GU>(a, N, K, st);            \
        if (rm == 2) return launch_one<L, 2, GU>(a, N, K, st);            \
        return launch_one<L, 4, GU>(a, N, K, st);                         \
    }
    MOE_GEMV_CASE(64)
    MOE_GEMV_CASE(32)
    MOE_GEMV_CASE(16)
    MOE_GEMV_CASE(8)
    MOE_GEMV_CASE(4)
    MOE_GEMV_CASE(2)
#undef MOE_GEMV_CASE
    return hipErrorInvalidValue;
}

// Gate/up then down.  Routed and shared units share a launch when their
// reduction lengths give the same lane split; otherwise each has its own.
hipError_t launch_ffn_gemv(const FfnArgs &a, hipStream_t st) {
    hipError_t e;
    const bool same_down = !a.with_shared || !a.with_routed ||
                           lanes_per_row(a.F) == lanes_per_row(a.Fs);
    const int nmax = a.with_shared ? (a.with_routed ? max(a.F, a.Fs) : a.Fs) : a.F;
    e = dispatch<true>(a, nmax, a.H, rows_per_pass(a.T, a.H), st);
    if (e != hipSuccess) return e;
    if (same_down) {
        // one launch; the LDS is sized for the longer of the two reductions
        const int K = a.with_routed ? a.F : a.Fs;
        const int kmax = a.with_shared && a.with_routed ? max(a.F, a.Fs) : K;
        return dispatch<false>(a, a.H, kmax, rows_per_pass(a.T, kmax), st);
    }
    FfnArgs r = a;
    r.with_shared = 0;
    e = dispatch<false>(r, a.H, a.F, rows_per_pass(a.T, a.F), st);
    if (e != hipSuccess) return e;
    FfnArgs s = a;
    s.with_routed = 0;
    return dispatch<false>(s, a.H, a.Fs, rows_per_pass(a.T, a.Fs), st);
}

}  // namespace moe

// ffn_mfma.hip -- step 4 of the MoE layer on gfx950 for larger row counts: the
// int4-gs64 SwiGLU expert FFN as an LDS-tiled grouped GEMM on the matrix cores
// ("MoE 路由与专家流式加载" §1.3: gate, up, SiLU, down for every union expert,
// each expert's weights read once for all rows routed to it; §1.4: the shared
// expert on every token).
//
// D[rows][outputs] = X[rows][K] * W[outputs][K]^T with v_mfma_f32_32x32x16_bf16:
//  - B (weights): a lane's 16-byte load holds 32 consecutive codes of one
//    output row; each 32-bit word of 8 codes becomes 4 bf16 pairs of (136 + q)
//    by one bit operation each (0x4300 is 128.0; q XOR 8 = q + 8), so the codes
//    enter the matrix core exactly ("colibrì 深度拆解" §5.2 packing);
//  - A (activations): prepared once as bf16 hi + lo (16 significant bits), laid
//    out in the same in-group element order as the codes; two MFMAs per step;
//  - per 64-group ("colibri 开发演进实录" §2.1 gs64) the group accumulator starts
//    at -136 * sum(x) (the unsigned-offset identity of §2.2, K1), and its result
//    is scaled by the fp32 group scale into the fp32 running sum.
// A workgroup owns 32 rows x 128 outputs (4 waves x 32); K is staged through
// LDS eight groups at a time with asynchronous global-to-LDS loads, while the
// chunk's weight codes are already in flight into registers.  Outputs of a row
// have one owner: deterministic.
#include <math.h>

#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr uint32_t kPairOffset = 0x43084308u;   // bf16 pair (136 + q) from a code pair
constexpr float kMfmaCodeOffset = 136.0f;
constexpr int kGroupBytes = 256;                // one row's 64-element group in fragment order
constexpr int kChunkGroups = 8;                 // groups staged per LDS step
constexpr int kTileRows = 32;
constexpr int kTileOut = 128;                   // outputs per workgroup (4 waves x 32)
constexpr int kRowPitch = kChunkGroups * kGroupBytes + 16;  // LDS bytes per row (+16: bank stagger)

__device__ __forceinline__ uint32_t bf16_rne_u(float f) {
    const uint32_t b = __float_as_uint(f);
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// ------------------------------------------------------------------ prep
// Rows of K fp32 values -> per 64-group 256 bytes: for half kg (32 elements) and
// block j (8 elements): 8 bf16 hi then 8 bf16 lo, elements in the order
// 0,4,1,5,2,6,3,7 of the block; and sx[row][group] = sum of (hi + lo).
// One thread per 8-element block; the 8 blocks of a group are 8 adjacent lanes.
__global__ __launch_bounds__(256) void prep_frag_kernel(const float *src, int rows, int K,
                                                       uint8_t *frag, float *sx) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;  // 8-element block index
    const long nblk = (long)rows * (K / 8);
    const bool live = i < nblk;
    const long ii = live ? i : nblk - 1;
    const int row = (int)(ii / (K / 8)), b = (int)(ii % (K / 8));
    const float4 *p = reinterpret_cast<const float4 *>(src + (size_t)row * K + 8 * b);
    const float4 v0 = p[0], v1 = p[1];
    const float e[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    const int ord[8] = {0, 4, 1, 5, 2, 6, 3, 7};
    uint32_t hb[8], lb[8];
    float part = 0.f;
#pragma unroll
    for (int s = 0; s < 8; s++) {
        const float x = e[ord[s]];
        hb[s] = bf16_rne_u(x);
        const float hi = __uint_as_float(hb[s] << 16);
        lb[s] = bf16_rne_u(x - hi);
        part += hi + __uint_as_float(lb[s] << 16);
    }
    const int G = b / 8, kg = (b % 8) / 4, j = b % 4;
    uint4 *dst = reinterpret_cast<uint4 *>(frag + (size_t)row * (K / 64) * kGroupBytes +
                                           (size_t)G * kGroupBytes + kg * 128 + j * 32);
    if (live) {
        dst[0] = make_uint4(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16), hb[4] | (hb[5] << 16),
                            hb[6] | (hb[7] << 16));
        dst[1] = make_uint4(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16), lb[4] | (lb[5] << 16),
                            lb[6] | (lb[7] << 16));
    }
    // group sum over the 8 blocks = 8 adjacent lanes (K is a multiple of 64)
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) part += __shfl_xor(part, m, kWave);
    if (live && b % 8 == 0) sx[(size_t)row * (K / 64) + G] = part;
}

hipError_t launch_prep_frag(const float *src, int rows, int K, uint8_t *frag, float *sx,
                            hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    const long nblk = (long)rows * (K / 8);
    ProfScope prof("prep_frag", st);
    prep_frag_kernel<<<(unsigned)((nblk + 255) / 256), 256, 0, st>>>(src, rows, K, frag, sx);
    return hipGetLastError();
}

// ------------------------------------------------------------------ grouped GEMM
__device__ __forceinline__ bf16x8_t code_pairs(uint32_t w) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 v;
    v.x = (w & 0x000F000Fu) ^ kPairOffset;
    v.y = ((w >> 4) & 0x000F000Fu) ^ kPairOffset;
    v.z = ((w >> 8) & 0x000F000Fu) ^ kPairOffset;
    v.w = ((w >> 12) & 0x000F000Fu) ^ kPairOffset;
    return __builtin_bit_cast(bf16x8_t, v);
}

template <bool GU>
__global__ __launch_bounds__(256, 2) void q4_mfma_kernel(MfmaArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t atile[kTileRows * kRowPitch];
    __shared__ __attribute__((aligned(16))) float sxt[kChunkGroups][kTileRows];
    const int unit = blockIdx.y;
    const int H = a.H;

    int nrows, Fu;
    const int32_t *rt;     // token of each row (GU routed), else rows are contiguous
    moe_q4 m0, m1;
    const uint8_t *afrag;  // fragment rows
    const float *asx;
    float *out;
    size_t out_row0;
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
            afrag = a.x_frag;
            asx = a.x_sx;
            out = a.h_routed;
        } else {
            const size_t dq = (size_t)e * H * (Fu / 2), ds = (size_t)e * H * (Fu / 64);
            m0.q = a.down.q + dq; m0.s = a.down.s + ds;
            m1 = m0;
            rt = nullptr;
            afrag = a.hr_frag + (size_t)r0 * (Fu / 64) * kGroupBytes;
            asx = a.hr_sx + (size_t)r0 * (Fu / 64);
            out = a.y_routed;
        }
        out_row0 = (size_t)r0;
    } else {
        if (!a.with_shared) return;
        nrows = a.T;
        Fu = a.Fs;
        rt = nullptr;
        if (GU) {
            m0 = a.sh_gate; m1 = a.sh_up;
            afrag = a.x_frag;
            asx = a.x_sx;
            out = a.h_shared;
        } else {
            m0 = a.sh_down; m1 = m0;
            afrag = a.hs_frag;
            asx = a.hs_sx;
            out = a.y_shared;
        }
        out_row0 = 0;
    }
    const int K = GU ? H : Fu;
    const int N = GU ? Fu : H;
    const int NG = K / 64;
    const int nb0 = blockIdx.x * kTileOut;
    if (nb0 >= N) return;

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int ln = lane % 32, kg = lane / 32;
    const int n0 = nb0 + wv * 32;
    const int nrow = min(n0 + ln, N - 1);  // weight row of this lane (clamped: never stored)
    const uint8_t *q0 = m0.q + (size_t)nrow * (K / 2) + 16 * kg;
    const uint8_t *q1 = m1.q + (size_t)nrow * (K / 2) + 16 * kg;
    const float *s0 = m0.s + (size_t)nrow * NG;
    const float *s1 = m1.s + (size_t)nrow * NG;

    for (int rc = 0; rc < nrows; rc += kTileRows) {
        const int R = min(kTileRows, nrows - rc);
        f32x16_t acc0 = {}, acc1 = {};
        for (int g0 = 0; g0 < NG; g0 += kChunkGroups) {
            const int ng = min(kChunkGroups, NG - g0);
            // this chunk's codes and scales first: their latency overlaps the staging below
            uint4 cq0[kChunkGroups], cq1[kChunkGroups];
            float cs0[kChunkGroups], cs1[kChunkGroups];
#pragma unroll
            for (int g = 0; g < kChunkGroups; g++) {
                const int G = g0 + min(g, ng - 1);  // past the end: re-read the last group
                cq0[g] = *reinterpret_cast<const uint4 *>(q0 + 32 * G);
                cs0[g] = s0[G];
                if (GU) {
                    cq1[g] = *reinterpret_cast<const uint4 *>(q1 + 32 * G);
                    cs1[g] = s1[G];
                }
            }
            __syncthreads();  // previous chunk consumed
            // stage rows [rc, rc+R) x groups [g0, g0+ng) straight into LDS: a row's chunk is
            // at most 2 KB, copied as 1-KB pieces, one asynchronous wave instruction each
            // (lane L moves bytes 16L..16L+15); lanes past the chunk re-read its start and
            // land in the row's unused tail
            const int bytes = ng * kGroupBytes;
            const int pieces = (bytes + 1023) / 1024;
            for (int pc = wv; pc < R * pieces; pc += 256 / kWave) {
                const int r = pc / pieces, h = pc % pieces;
                const int src = rt ? rt[rc + r] : rc + r;
                int off = h * 1024 + lane * 16;
                if (off >= bytes) off = 0;
                __builtin_amdgcn_global_load_lds(afrag + ((size_t)src * NG + g0) * kGroupBytes + off,
                                                 atile + r * kRowPitch + h * 1024, 16, 0, 0);
            }
            for (int i = tid; i < kTileRows * ng; i += blockDim.x) {
                const int r = i % kTileRows, g = i / kTileRows;
                float v = 0.f;
                if (r < R) {
                    const int src = rt ? rt[rc + r] : rc + r;
                    v = asx[(size_t)src * NG + g0 + g];
                }
                sxt[g][r] = v;
            }
            __syncthreads();
#pragma unroll
            for (int g = 0; g < kChunkGroups; g++) {
                if (g >= ng) break;
                // group accumulators start at -136 * sum(x) of their row
                f32x16_t ga;
#pragma unroll
                for (int q4 = 0; q4 < 4; q4++) {
                    const float4 sv = *reinterpret_cast<const float4 *>(&sxt[g][8 * q4 + 4 * kg]);
                    ga[4 * q4 + 0] = -kMfmaCodeOffset * sv.x;
                    ga[4 * q4 + 1] = -kMfmaCodeOffset * sv.y;
                    ga[4 * q4 + 2] = -kMfmaCodeOffset * sv.z;
                    ga[4 * q4 + 3] = -kMfmaCodeOffset * sv.w;
                }
                f32x16_t g0acc = ga, g1acc = ga;
                const uint32_t w0[4] = {cq0[g].x, cq0[g].y, cq0[g].z, cq0[g].w};
                const uint32_t w1[4] = {cq1[g].x, cq1[g].y, cq1[g].z, cq1[g].w};
                const uint8_t *arow = atile + ln * kRowPitch + g * kGroupBytes + kg * 128;
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const bf16x8_t ahi = *reinterpret_cast<const bf16x8_t *>(arow + 32 * j);
                    const bf16x8_t alo = *reinterpret_cast<const bf16x8_t *>(arow + 32 * j + 16);
                    const bf16x8_t b0 = code_pairs(w0[j]);
                    g0acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, b0, g0acc, 0, 0, 0);
                    g0acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, b0, g0acc, 0, 0, 0);
                    if (GU) {
                        const bf16x8_t b1 = code_pairs(w1[j]);
                        g1acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, b1, g1acc, 0, 0, 0);
                        g1acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, b1, g1acc, 0, 0, 0);
                    }
                }
#pragma unroll
                for (int v = 0; v < 16; v++) {
                    acc0[v] = fmaf(cs0[g], g0acc[v], acc0[v]);
                    if (GU) acc1[v] = fmaf(cs1[g], g1acc[v], acc1[v]);
                }
            }
        }
        // D layout: register v of lane (ln, kg) is row 8*(v/4) + 4*kg + v%4, column ln
        const int n = n0 + ln;
        if (n < N) {
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int r = 8 * (v / 4) + 4 * kg + (v % 4);
                if (r < R) {
                    float val;
                    if (GU) {
                        const float gg = acc0[v], uu = acc1[v];
                        val = gg / (1.0f + expf(-gg)) * uu;
                    } else {
                        val = acc0[v];
                    }
                    out[(out_row0 + rc + r) * (size_t)N + n] = val;
                }
            }
        }
    }
}

// Gate/up for every unit (x prepared once), then h prepared, then down.
hipError_t launch_ffn_mfma(const MfmaArgs &a, hipStream_t st) {
    hipError_t e;
    // activations of every token, once
    e = launch_prep_frag(a.x, a.T, a.H, a.x_frag, a.x_sx, st);
    if (e != hipSuccess) return e;
    const int nmax = a.with_shared ? (a.with_routed ? max(a.F, a.Fs) : a.Fs) : a.F;
    {
        dim3 grid((nmax + kTileOut - 1) / kTileOut, a.max_units + 1);
        ProfScope prof("ffn_gateup_mfma", st);
        q4_mfma_kernel<true><<<grid, 256, 0, st>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // h rows in fragment order: the routed rows (as many as the largest union can
    // have) and the shared rows
    if (a.with_routed) {
        e = launch_prep_frag(a.h_routed, a.max_rows, a.F, a.hr_frag, a.hr_sx, st);
        if (e != hipSuccess) return e;
    }
    if (a.with_shared) {
        e = launch_prep_frag(a.h_shared, a.T, a.Fs, a.hs_frag, a.hs_sx, st);
        if (e != hipSuccess) return e;
    }
    {
        dim3 grid((a.H + kTileOut - 1) / kTileOut, a.max_units + 1);
        ProfScope prof("ffn_down_mfma", st);
        q4_mfma_kernel<false><<<grid, 256, 0, st>>>(a);
        return hipGetLastError();
    }
}

}  // namespace moe

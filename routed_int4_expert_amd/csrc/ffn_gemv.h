// ffn_gemv.h -- step 4 of the MoE layer on gfx950 for small row counts: the
// int4-gs64 SwiGLU expert FFN as grouped dequantising GEMVs
// ("MoE 路由与专家流式加载" §1.3: gate, up, SiLU, down per union expert; §1.4: the
// shared expert on every token).
//
// Work unit = (expert of the union or the shared expert, block of output rows).
// The unit's token rows (at most RM at a time) are staged once per workgroup in
// LDS (16-bit fixed point, below); each weight row is streamed from HBM exactly once
// per RM rows, with LPR lanes per row each issuing coalesced 16-byte loads of 32
// codes, so a wave's load covers LPR*16 contiguous bytes of one row.
//
// Codes: a byte holds elements 2j (low nibble) and 2j+1 (high nibble) as
// two's-complement int4 ("colibrì 深度拆解" §5.2).  XOR with 8 in every nibble turns
// code q into u = q + 8 in [0, 15]; masking a 32-bit word of 8 codes with 0x0F0F0F0F
// (and the word shifted right by 4) gives the even (odd) elements as four unsigned
// bytes, three bit operations for eight codes.  Activations are staged per 32-element
// chunk in 16-bit fixed point: x16 = rint(x * 2^n) with the power-of-two step 2^-n
// that maps max|x| to at most 32639 (act_shift), split into two signed bytes
// x16 = 256 hi + lo; v_dot4_i32_i8 accumulates u * hi and u * lo exactly in int32,
// and per chunk
//   sum(q x16) = 256 sum(u hi) + sum(u lo) - 8 sum(x16)
// (the unsigned-offset identity of "colibri 开发演进实录" §2.2, K1), times the chunk's
// step and the fp32 gs64 scale (two chunks per 64-group).  The only rounding before
// the fp32 accumulation is x16: less than max|x| / 32639 per element, none for values
// with at most 15 significant bits relative to the chunk's largest.
//
// int3-g64 codes (moe.h bit planes): a lane's 32-element chunk is two words of the
// low-bit plane and one word of the sign plane; shift and mask give the unsigned
// u = c + 4 in [0, 7] of four elements of one parity per step, in the element order
// above, and sum(c x16) = 256 sum(u hi) + sum(u lo) - 4 sum(x16).
// MXFP4 codes: a lane's 16-byte load is one 32-element block with one UE8M0 exponent,
// matching the 32-element activation chunk.  Every E2M1 value doubled is an integer
// 2v in [-12, 12]: two byte permutes (a table of the magnitudes, one of their
// negatives) indexed by the code's low three bits, and a select on its sign bit, give
// 2v as four signed bytes of one parity per word; sum(2v x16) is an exact int32 sum,
// times the chunk's step, the block's 2^(e - 127) and 1/2.
//
// The gate/up kernel finishes with the fused SiLU(g) * u epilogue and writes
// h [rows][F]; the down kernel writes the unweighted y [rows][H].  Each output
// is reduced inside one lane group in a fixed order (deterministic).
#pragma once

#include <math.h>

#include "moe_internal.h"
#include "select_union.h"

namespace moe {

// LDS row layout: per 32-element chunk 20 dwords -- for each 8-element group d four
// dwords of signed bytes (hi of elements 8d+0,2,4,6; hi of 8d+1,3,5,7; lo of the
// even ones; lo of the odd ones), the chunk's step 2^-n (fp32) at dword 16
// and 8 sum(x16) (int32) at dword 17, then padding: the 16-byte reads of 8
// consecutive lanes (80 bytes apart) hit distinct banks.
constexpr int kChunkPitch = 20;
constexpr float kX16Max = 32639.0f;  // 127 * 256 + 127: both bytes of x16 stay in [-128, 127]

// the value of each lane's DPP source lane (CTRL: a quad_perm or row_ror control, for
// which every source lane is in the same row)
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// sum over 32 codes of (q_i + 8) * x16_i, the chunk staged as 4 uint4 of byte limbs
__device__ __forceinline__ int dot32_i8(const uint4 q, const uint4 *xv) {
    const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
    int ah = 0, al = 0;
#pragma unroll
    for (int d = 0; d < 4; d++) {
        const uint32_t ev = (wd[d] ^ 0x08080808u) & 0x0F0F0F0Fu;         // u of elements 0,2,4,6
        const uint32_t od = ((wd[d] >> 4) ^ 0x08080808u) & 0x0F0F0F0Fu;  // u of elements 1,3,5,7
        const uint4 x = xv[d];
        ah = __builtin_amdgcn_sdot4((int)ev, (int)x.x, ah, false);
        ah = __builtin_amdgcn_sdot4((int)od, (int)x.y, ah, false);
        al = __builtin_amdgcn_sdot4((int)ev, (int)x.z, al, false);
        al = __builtin_amdgcn_sdot4((int)od, (int)x.w, al, false);
    }
    return (ah << 8) + al;  // |.| < 2^25: 32 products of at most 15 * 32639
}

// sum over 32 int3 codes of (c_i + 4) * x16_i: q.x, q.y the chunk's two low-plane words,
// q.z its sign-plane word.  Word dd of the low plane holds 8-element groups 2dd and
// 2dd+1; its bit pair s (0..3) gives the even elements of group 2dd, the odd ones, then
// the same of group 2dd+1, matching sign bit 4dd + s of every byte of q.z.
__device__ __forceinline__ int dot32_i3(const uint4 q, const uint4 *xv) {
    const uint32_t pos = ~q.z;  // bit 2 of u = c + 4 is the inverted sign bit
    int ah = 0, al = 0;
#pragma unroll
    for (int dd = 0; dd < 2; dd++) {
        const uint32_t A = dd ? q.y : q.x;
#pragma unroll
        for (int s = 0; s < 4; s++) {
            const uint32_t u = ((A >> (2 * s)) & 0x03030303u) | (((pos >> (4 * dd + s)) & 0x01010101u) << 2);
            const uint4 x = xv[2 * dd + s / 2];
            ah = __builtin_amdgcn_sdot4((int)u, (int)((s & 1) ? x.y : x.x), ah, false);
            al = __builtin_amdgcn_sdot4((int)u, (int)((s & 1) ? x.w : x.z), al, false);
        }
    }
    return (ah << 8) + al;  // |.| < 2^23: 32 products of at most 7 * 32639
}

// sum over the 32 E2M1 codes of one block of 2v_i * x16_i (2v the doubled value, an
// integer in [-12, 12]), the chunk staged as 4 uint4 of byte limbs.  Per word: the low
// three bits of each code select its doubled magnitude from {0, 1, 2, 3, 4, 6, 8, 12}
// (one byte permute) and its negative (another); the sign bit, spread to a byte mask by a
// shift and a multiply by 255, picks one of the two (bit select).
__device__ __forceinline__ int dot32_f4(const uint4 q, const uint4 *xv) {
    constexpr uint32_t kPosLo = 0x03020100u, kPosHi = 0x0C080604u;  // 0, 1, 2, 3 | 4, 6, 8, 12
    constexpr uint32_t kNegLo = 0xFDFEFF00u, kNegHi = 0xF4F8FAFCu;  // their negatives
    const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
    int ah = 0, al = 0;
#pragma unroll
    for (int d = 0; d < 4; d++) {
        const uint32_t se = wd[d] & 0x07070707u, so = (wd[d] >> 4) & 0x07070707u;
        const uint32_t me = ((wd[d] >> 3) & 0x01010101u) * 0xFFu, mo = ((wd[d] >> 7) & 0x01010101u) * 0xFFu;
        const uint32_t pe = __builtin_amdgcn_perm(kPosHi, kPosLo, se), ne = __builtin_amdgcn_perm(kNegHi, kNegLo, se);
        const uint32_t po = __builtin_amdgcn_perm(kPosHi, kPosLo, so), no = __builtin_amdgcn_perm(kNegHi, kNegLo, so);
        const uint32_t ve = (ne & me) | (pe & ~me);  // elements 8d, 8d+2, 8d+4, 8d+6
        const uint32_t vo = (no & mo) | (po & ~mo);  // elements 8d+1, 8d+3, 8d+5, 8d+7
        const uint4 x = xv[d];
        ah = __builtin_amdgcn_sdot4((int)ve, (int)x.x, ah, false);
        ah = __builtin_amdgcn_sdot4((int)vo, (int)x.y, ah, false);
        al = __builtin_amdgcn_sdot4((int)ve, (int)x.z, al, false);
        al = __builtin_amdgcn_sdot4((int)vo, (int)x.w, al, false);
    }
    return (ah << 8) + al;  // |.| < 2^24: 32 products of at most 12 * 32639
}

// Sum over each group of LPR lanes, in a fixed order (deterministic); the group's
// first lane holds the total.  A whole wave (LPR = 64, all lanes active): each row
// of 16 lanes by DPP moves (swap neighbours, swap pairs, rotate by 4, rotate by 8),
// then the four row sums read from lanes 0, 16, 32 and 48 -- no LDS round trip.
// Narrower groups: butterfly shuffles.
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (LPR == kWave) {
        v += dpp_f32<0xB1>(v);   // quad_perm 1,0,3,2
        v += dpp_f32<0x4E>(v);   // quad_perm 2,3,0,1
        v += dpp_f32<0x124>(v);  // row_ror 4
        v += dpp_f32<0x128>(v);  // row_ror 8
        const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
        const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
        const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
        const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
        return (r0 + r1) + (r2 + r3);
    } else {
#pragma unroll
        for (int m = LPR / 2; m > 0; m >>= 1) v += __shfl_xor(v, m, kWave);
        return v;
    }
}

// Selection and union of a one-token decode step, by wave 0 into LDS ([R] §1.1-§1.3;
// select_token as in the selection kernels).  One token picks an expert at most once,
// so the union is its kept picks in increasing expert order, one row each, and needs
// no block-wide passes.  LDS layout (the general one at T = 1):
// ids[k] w[k] keff[1] n_uniq[1] uniq[E] off[E+1] row_tok[k] pick_row[k].
// With `writer` the wave also writes them to global memory for the later launches.
__device__ __forceinline__ void select_union_one(const FfnArgs &a, int32_t *lds, bool writer) {
    __shared__ PickScratch ps_sel;
    const int k = a.sel.k, E = a.sel.E;
    const int lane = threadIdx.x % kWave;
    int32_t *ids_l = lds;
    float *w_l = reinterpret_cast<float *>(ids_l + k);
    int32_t *keff_l = reinterpret_cast<int32_t *>(w_l + k);
    int32_t *nu_l = keff_l + 1;
    int32_t *uniq_l = nu_l + 1;
    int32_t *off_l = uniq_l + E;
    int32_t *rt_l = off_l + E + 1;
    int32_t *pick_l = rt_l + k;
    // byte flags of the kept experts (in the pick scratch's place: the selection is done)
    uint8_t *flag = reinterpret_cast<uint8_t *>(&ps_sel);
    static_assert(sizeof(PickScratch) >= MOE_MAX_EXPERTS, "flag bytes fit the scratch");
    // The selection is on the critical path of every routed workgroup and shares its
    // SIMD with older workgroups' streaming waves, which the arbiter would favour:
    // the selecting wave runs at raised issue priority until the union is built.
    __builtin_amdgcn_s_setprio(3);
    // (one group: the host sends group-limited layers to the selection kernels)
    select_token_impl<false>(a.sel, 0, lane, ids_l, w_l, keff_l, nullptr, nullptr, &ps_sel, nullptr);
    wave_lds_sync();
    const int keff = *keff_l;
    const int my = lane < keff ? ids_l[lane] : -1;
    reinterpret_cast<uint32_t *>(flag)[lane] = 0u;  // 256 bytes
    wave_lds_sync();
    if (my >= 0) flag[my] = 1;
    wave_lds_sync();
    // lane l owns experts 4l .. 4l+3: off[e] = kept experts below e, from the flags'
    // ballots (flags of expert 4l + m are bit l of ballot m)
    const uint32_t f4 = reinterpret_cast<const uint32_t *>(flag)[lane];
    unsigned long long bm[4];
    int before = 0;  // kept experts in lanes below this one
#pragma unroll
    for (int m = 0; m < 4; m++) {
        bm[m] = __ballot((f4 >> (8 * m)) & 1u);
        before += __popcll(bm[m] & ((1ull << lane) - 1ull));
    }
    int run = before;
#pragma unroll
    for (int m = 0; m < 4; m++) {
        const int e = 4 * lane + m;
        const bool kept = (f4 >> (8 * m)) & 1u;
        if (e < E) {
            off_l[e] = run;
            if (kept) uniq_l[run] = e;
        }
        run += kept ? 1 : 0;
    }
    for (int i = keff + lane; i < E; i += kWave) uniq_l[i] = -1;
    if (lane == 0) {
        off_l[E] = keff;
        nu_l[0] = keff;
    }
    wave_lds_sync();
    if (lane < k) {  // a kept pick's row: its expert's offset
        pick_l[lane] = my >= 0 ? off_l[my] : -1;
        rt_l[lane] = my >= 0 ? 0 : -1;
    }
    wave_lds_sync();
    __builtin_amdgcn_s_setprio(0);
    if (writer) {
        for (int i = lane; i < k; i += kWave) {
            a.sel.ids[i] = ids_l[i];
            a.sel.w[i] = w_l[i];
            a.uni.row_tok[i] = rt_l[i];
            a.uni.pick_row[i] = pick_l[i];
        }
        for (int i = lane; i < E; i += kWave) a.uni.uniq[i] = uniq_l[i];
        for (int i = lane; i <= E; i += kWave) a.uni.off[i] = off_l[i];
        if (lane == 0) {
            a.sel.keff[0] = keff;
            a.uni.n_uniq[0] = keff;
        }
    }
}

// Stages R input rows in the 16-bit fixed-point chunk format above, by nt threads of
// the block (nt a multiple of 4; thread number i of them starts at item i): a thread
// per 8 elements, in batches of four items per thread whose loads are all issued
// (stage_issue) before any is converted and stored (stage_commit).  The 4 threads of
// a chunk form an aligned quad of lanes and combine their max|x| and sum(x16) with
// two DPP moves each.
constexpr int kStageBatch = 4;
struct StageBatch {
    float4 v[kStageBatch][2];
};

__device__ __forceinline__ void stage_issue(StageBatch &sb, const float *xin, const int32_t *rt, int rc,
                                            int K, int n8, int i0, int nt) {
#pragma unroll
    for (int b = 0; b < kStageBatch; b++) {
        const int i = i0 + b * nt;
        if (i < n8) {
            const int r = i / (K / 8), g = i % (K / 8);
            const int src = rt ? rt[rc + r] : rc + r;
            const float4 *px = reinterpret_cast<const float4 *>(xin + (size_t)src * K + 8 * g);
            sb.v[b][0] = px[0];
            sb.v[b][1] = px[1];
        }
    }
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

// four signed bytes (a, b, c, d) as one word, a in the low byte
__device__ __forceinline__ uint32_t pack_i8x4(int a, int b, int c, int d) {
    return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) | ((uint32_t)(c & 0xFF) << 16) |
           ((uint32_t)d << 24);
}

__device__ __forceinline__ void stage_commit(const StageBatch &sb, float *xs, int rowpitch, int K, int n8,
                                             int i0, int nt) {
    uint32_t *xw = reinterpret_cast<uint32_t *>(xs);
#pragma unroll
    for (int b = 0; b < kStageBatch; b++) {
        const int i = i0 + b * nt;
        if (i >= n8) continue;  // the same for the 4 lanes of a chunk
        const int r = i / (K / 8), g = i % (K / 8);
        const float xe[8] = {sb.v[b][0].x, sb.v[b][0].y, sb.v[b][0].z, sb.v[b][0].w,
                             sb.v[b][1].x, sb.v[b][1].y, sb.v[b][1].z, sb.v[b][1].w};
        // chunk max of |x| as an unsigned bit pattern (NaN and infinity order above
        // every finite value, so they are not lost)
        uint32_t mb = 0;
#pragma unroll
        for (int e = 0; e < 8; e++) mb = max(mb, __float_as_uint(xe[e]) & 0x7FFFFFFFu);
        mb = max(mb, dpp_u32<0xB1>(mb));
        mb = max(mb, dpp_u32<0x4E>(mb));
        const bool finite = mb < 0x7F800000u;
        const bool live = finite && mb != 0u;
        constexpr ActRule rule = act_rule(0);
        const int n = live ? act_shift(mb, rule) : 0;
        constexpr float lim = rule.lim;
        int x16[8], hi[8], lo[8];
        int ps = 0;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            x16[e] = live ? (int)fminf(fmaxf(rintf(ldexpf(xe[e], n)), -lim), lim) : 0;
            hi[e] = (x16[e] + 128) >> 8;
            lo[e] = x16[e] - (hi[e] << 8);
            ps += x16[e];
        }
        uint4 w;  // hi of the even and odd elements, lo of the even and odd elements
        w.x = pack_i8x4(hi[0], hi[2], hi[4], hi[6]);
        w.y = pack_i8x4(hi[1], hi[3], hi[5], hi[7]);
        w.z = pack_i8x4(lo[0], lo[2], lo[4], lo[6]);
        w.w = pack_i8x4(lo[1], lo[3], lo[5], lo[7]);
        uint32_t *chunk = xw + r * rowpitch + (g / 4) * kChunkPitch;
        *reinterpret_cast<uint4 *>(chunk + (g % 4) * 4) = w;
        ps += (int)dpp_u32<0xB1>((uint32_t)ps);
        ps += (int)dpp_u32<0x4E>((uint32_t)ps);
        if (g % 4 == 0) {
            // step of x16 (a NaN step carries a non-finite input into every product)
            chunk[16] = finite ? (live ? __float_as_uint(ldexpf(1.0f, -n)) : 0u) : 0x7FC00000u;
            chunk[17] = (uint32_t)(8 * ps);
        }
    }
}

// The thread's batches from item `first` on (its number among the nt threads, for a
// whole staging).
__device__ __forceinline__ void stage_rows(float *xs, int rowpitch, const float *xin,
                                           const int32_t *rt, int rc, int R, int K, int first, int nt) {
    const int n8 = R * (K / 8);
    for (int i0 = first; i0 < n8; i0 += kStageBatch * nt) {
        StageBatch sb;
        stage_issue(sb, xin, rt, rc, K, n8, i0, nt);
        stage_commit(sb, xs, rowpitch, K, n8, i0, nt);
    }
}

// Outputs per lane group per pass: four weight rows per step at one token (the
// next step's rows are loaded while the current ones are computed), fewer with
// more tokens so the accumulators fit in registers.
template <int LPR, int RM, bool GU>
struct GemvShape {
    static constexpr int G = kWave / LPR;                     // lane groups per wave
    static constexpr int NFB = (LPR >= 32 ? LPR / 32 : 1) * (GU ? 1 : 2);
    static constexpr int NF = NFB / RM > 0 ? NFB / RM : 1;    // outputs per lane group per pass
    static constexpr int NM = GU ? 2 : 1;                     // matrices per output
    static constexpr int WF = G * NF;                         // outputs per wave per pass
    static constexpr int BF = 4 * WF;                         // outputs per workgroup per pass
};

// The work of workgroup bx of one unit (the kernels below map it from blockIdx).
template <int LPR, int RM, bool GU, int FMT>
__device__ __forceinline__ void gemv_body(const FfnArgs &a, int passes, int unit, int bx) {
    using S = GemvShape<LPR, RM, GU>;
    constexpr int kPitch = kChunkPitch;
    extern __shared__ float xs[];  // [RM][C * kPitch] (+ selection and union, when fused)
    const int H = a.H;

    // ---- the union: from global memory, or, for one token, selected here ([R] §1.1-§1.3)
    // into LDS by wave 0 while the other waves stage the token's row
    const int32_t *n_uniq_p = a.n_uniq, *uniq_p = a.uniq, *off_p = a.off, *row_tok_p = a.row_tok;
    bool staged = false;
    if constexpr (GU && RM == 1) if (a.fuse_select && unit < a.max_units && a.with_routed) {
        int32_t *lds = reinterpret_cast<int32_t *>(xs + (size_t)(H / 32) * kPitch);
        if (threadIdx.x < kWave)
            select_union_one(a, lds, bx == 0 && unit == 0);
        else
            stage_rows(xs, (H / 32) * kPitch, a.x, nullptr, 0, 1, H, (int)threadIdx.x - kWave,
                            blockDim.x - kWave);
        __syncthreads();
        const int k = a.sel.k, E = a.sel.E;
        n_uniq_p = lds + 2 * k + 1;
        uniq_p = n_uniq_p + 1;
        off_p = uniq_p + E;
        row_tok_p = off_p + E + 1;
        staged = true;
    }

    // ---- the unit: a routed expert of the union, or the shared expert
    int nrows, Fu;
    const int32_t *rt;
    moe_q4 m0, m1;
    const float *xin;   // row source for K
    float *out;         // output rows
    size_t out_row0;    // first output row index
    if (unit < a.max_units) {
        if (!a.with_routed) return;
        // both loads at once: uniq holds max_units <= E entries, -1 past the union
        const int nu = n_uniq_p[0];
        const int e = uniq_p[unit];
        if ((unit >= nu) | (e < 0)) return;  // (either test alone suffices; both keep the loads together)
        // one token: each union expert has one row, in union order, so unit u is row u
        // (no offset lookup, one round trip less before the first weight load)
        const int r0 = a.T == 1 ? unit : off_p[e];
        nrows = a.T == 1 ? 1 : off_p[e + 1] - r0;
        Fu = a.F;
        if (GU) {
            if (a.tab) {  // the residency tier's slots
                m0 = a.tab[3 * e];
                m1 = a.tab[3 * e + 1];
            } else {
                m0 = fmt_stack_at(a.gate, FMT, e, Fu, H);
                m1 = fmt_stack_at(a.up, FMT, e, Fu, H);
            }
            rt = row_tok_p + r0;
            xin = a.x;
            out = a.h_routed;
        } else {
            if (a.tab) {
                m0 = a.tab[3 * e + 2];
            } else {
                m0 = fmt_stack_at(a.down, FMT, e, H, Fu);
            }
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
    const int nbw = bx * S::BF * passes;  // first output of this workgroup
    if (nbw >= N) return;

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
    const int sub = lane % LPR;
    const int grp = LPR == kWave ? 0 : lane / LPR;  // with 64 lanes per row the row is wave-uniform
    const int rowpitch = C * kPitch;

    // Steps = (pass, chunk iteration), flattened so the codes and scales of the
    // next step are in flight while the current one is computed.
    const int nit = (C + LPR - 1) / LPR;
    const int nsteps = passes * nit;
    uint4 q[S::NF][S::NM], qn[S::NF][S::NM];
    float sc[S::NF][S::NM], scn[S::NF][S::NM];
    float acc[S::NF][S::NM][RM];
    auto load_step = [&](int step, uint4 (&qq)[S::NF][S::NM], float (&ss)[S::NF][S::NM]) {
        const int p = step / nit, c = sub + (step % nit) * LPR;
        const int cc = c < C ? c : C - 1;  // lanes past the row's end re-read its last chunk
#pragma unroll
        for (int f = 0; f < S::NF; f++) {
            const int n = min(nbw + p * S::BF + wv * S::WF + f * S::G + grp, N - 1);
#pragma unroll
            for (int m = 0; m < S::NM; m++) {
                // row base (wave-uniform when LPR == 64) plus a 32-bit lane offset
                const uint8_t *rq = (m == 0 ? m0.q : m1.q) + (size_t)n * fmt_code_bytes(FMT, K);
                const uint8_t *rs = static_cast<const uint8_t *>(m == 0 ? m0.s : m1.s) +
                                    (size_t)n * fmt_scale_bytes(FMT, K);
                if constexpr (FMT == kFmtI3) {
                    // two low-plane words and the sign-plane word of chunk cc
                    const uint2 lw = *reinterpret_cast<const uint2 *>(rq + (uint32_t)(8 * cc));
                    const uint32_t sw = *reinterpret_cast<const uint32_t *>(rq + (uint32_t)(K / 4 + 4 * cc));
                    qq[f][m] = make_uint4(lw.x, lw.y, sw, 0u);
                } else {
                    qq[f][m] = *reinterpret_cast<const uint4 *>(rq + (uint32_t)(16 * cc));
                }
                if constexpr (FMT == kFmtF4)  // the block's exponent byte, kept as raw bits
                    ss[f][m] = __uint_as_float((uint32_t)rs[(uint32_t)cc]);
                else
                    ss[f][m] = reinterpret_cast<const float *>(rs)[(uint32_t)(cc >> 1)];
            }
        }
    };
    // The first batch of the first rows' activation loads goes out first, then the first
    // step's codes (independent of the staged rows), so the rows are converted while the
    // codes are in flight.
    if (staged) {
        load_step(0, q, sc);
    } else {
        const int n80 = min(RM, nrows) * (K / 8);
        StageBatch sb0;
        stage_issue(sb0, xin, rt, 0, K, n80, tid, blockDim.x);
        load_step(0, q, sc);
        stage_commit(sb0, xs, rowpitch, K, n80, tid, blockDim.x);
        stage_rows(xs, rowpitch, xin, rt, 0, min(RM, nrows), K, tid + kStageBatch * blockDim.x, blockDim.x);
        __syncthreads();
    }

    for (int rc = 0; rc < nrows; rc += RM) {
        const int R = min(RM, nrows - rc);
        if (rc > 0) {
            __syncthreads();  // previous rows fully consumed
            stage_rows(xs, rowpitch, xin, rt, rc, R, K, tid, blockDim.x);
            __syncthreads();
        }

        if (rc > 0) load_step(0, q, sc);  // rows beyond the first RM restart the weight stream
        // one step: prefetch the next step's rows into (qn, scn), compute with (qc, scc)
        auto do_step = [&](int step, uint4 (&qc)[S::NF][S::NM], float (&scc)[S::NF][S::NM],
                           uint4 (&qnx)[S::NF][S::NM], float (&scnx)[S::NF][S::NM]) {
            const int p = step / nit, it = step % nit;
            const int nb0 = nbw + p * S::BF;
            // unconditional, so the wait before the compute below only covers this step's
            // loads (the last step re-fetches itself, which the cache serves)
            load_step(step + 1 < nsteps ? step + 1 : step, qnx, scnx);
            if (it == 0) {
#pragma unroll
                for (int f = 0; f < S::NF; f++)
#pragma unroll
                    for (int m = 0; m < S::NM; m++)
#pragma unroll
                        for (int r = 0; r < RM; r++) acc[f][m][r] = 0.f;
            }
            const int c = sub + it * LPR;
            if (c < C) {
#pragma unroll
                for (int r = 0; r < RM; r++) {
                    if (r < R) {
                        const float *px = xs + r * rowpitch + c * kPitch;
                        {
                            uint4 xv[4];
#pragma unroll
                            for (int v = 0; v < 4; v++) xv[v] = *reinterpret_cast<const uint4 *>(px + 4 * v);
                            const float2 sc2 = *reinterpret_cast<const float2 *>(px + 16);
                            const float sx = sc2.x;                    // step of x16
                            const int c8 = __float_as_int(sc2.y);     // 8 sum(x16)
#pragma unroll
                            for (int f = 0; f < S::NF; f++)
#pragma unroll
                                for (int m = 0; m < S::NM; m++) {
                                    // sum(q x16), exact (int3: sum((c + 4) x16) - 4 sum(x16); MXFP4:
                                    // sum(2v x16), the block scale halved)
                                    if constexpr (FMT == kFmtF4) {
                                        const float blk = ue8m0_f32(__float_as_uint(scc[f][m])) * 0.5f;
                                        acc[f][m][r] = fmaf(blk * sx, (float)dot32_f4(qc[f][m], xv), acc[f][m][r]);
                                    } else {
                                        const int iv = FMT == kFmtI3 ? dot32_i3(qc[f][m], xv) - (c8 >> 1)
                                                                     : dot32_i8(qc[f][m], xv) - c8;
                                        acc[f][m][r] = fmaf(scc[f][m] * sx, (float)iv, acc[f][m][r]);
                                    }
                                    // one row at a time: keeps the unpacked codes of a single row live
                                    __builtin_amdgcn_sched_barrier(0);
                                }
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);  // one token's activations live at a time
                }
            }
            if (it == nit - 1) {
#pragma unroll
                for (int f = 0; f < S::NF; f++)
#pragma unroll
                    for (int m = 0; m < S::NM; m++)
#pragma unroll
                        for (int r = 0; r < RM; r++) acc[f][m][r] = group_sum<LPR>(acc[f][m][r]);
                if (sub == 0) {
#pragma unroll
                    for (int f = 0; f < S::NF; f++) {
                        const int n = nb0 + wv * S::WF + f * S::G + grp;
                        if (n >= N) continue;
#pragma unroll
                        for (int r = 0; r < RM; r++) {
                            if (r >= R) continue;
                            float v;
                            if (GU) {
                                v = gate_up_out(a.gu_out, acc[f][0][r], acc[f][S::NM - 1][r]);
                            } else {
                                v = acc[f][0][r];
                            }
                            out[(out_row0 + rc + r) * (size_t)N + n] = v;
                        }
                    }
                }
            }
        };
        if (RM == 1) {
            // ping-pong between the two register buffers, two steps per iteration
            for (int step = 0; step < nsteps; step += 2) {
                do_step(step, q, sc, qn, scn);
                if (step + 1 < nsteps) do_step(step + 1, qn, scn, q, sc);
            }
        } else {
            // more tokens per row: more arithmetic per byte; one body keeps registers in check
            for (int step = 0; step < nsteps; step++) {
                do_step(step, q, sc, qn, scn);
#pragma unroll
                for (int f = 0; f < S::NF; f++)
#pragma unroll
                    for (int m = 0; m < S::NM; m++) {
                        q[f][m] = qn[f][m];
                        sc[f][m] = scn[f][m];
                    }
            }
        }
    }
}

// One-dimensional grid: workgroups [0, nsh) take the shared expert with passes_sh
// passes each, the rest the routed units, gx workgroups of `passes` passes per unit.
// The counts are chosen on the host so the grid fits in one round of resident
// workgroups.
template <int LPR, int RM, bool GU, int FMT>
__global__ __launch_bounds__(256, 4) void q4_gemv_kernel(FfnArgs a, int passes, int passes_sh, int nsh,
                                                         int gx) {
    const int w = blockIdx.x;
    if (w < nsh) {
        gemv_body<LPR, RM, GU, FMT>(a, passes_sh, a.max_units, w);
    } else {
        const int r = w - nsh;
        gemv_body<LPR, RM, GU, FMT>(a, passes, r / gx, r % gx);
    }
}

static int lanes_per_row(int K) {
    const int C = K / 32;
    int l = 64;
    while (l > 2 && l > C) l >>= 1;
    return l;
}


static int device_cus() {
    static int cus = 0;
    if (cus == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            cus = n;
        else
            cus = 256;
        (void)hipGetLastError();
    }
    return cus;
}

template <int LPR, int RM, bool GU, int FMT>
static hipError_t launch_one(const FfnArgs &a, int N, int K, hipStream_t st) {
    using S = GemvShape<LPR, RM, GU>;
    size_t lds = (size_t)RM * (K / 32) * kChunkPitch * sizeof(float);
    if (GU && RM == 1 && a.fuse_select) lds += select_lds_words(a.sel.E, a.sel.T, a.sel.k) * sizeof(uint32_t);
    if (lds > 64 * 1024) {
        // raise the dynamic-LDS cap for this kernel; the launch itself reports a real failure
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&q4_gemv_kernel<LPR, RM, GU, FMT>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        (void)hipGetLastError();
    }
    // resident workgroups per CU (4 waves each): registers allow 4, LDS may allow fewer
    int per_cu = 4;
    const size_t lds_static = (GU && RM == 1) ? sizeof(PickScratch) + 256 : 256;
    while (per_cu > 1 && (size_t)per_cu * (lds + lds_static) > 160 * 1024) per_cu--;
    const long cap = (long)device_cus() * per_cu;
    const int blocks1 = (N + S::BF - 1) / S::BF;  // workgroups per unit at one pass each
    int passes = 1, passes_sh = 1, nsh = 0, gx;
    if (GU && RM == 1 && a.fuse_select && a.with_shared) {
        // One token: the routed units cannot start before the selection, the shared
        // expert can; it gets one-pass workgroups, so its weights stream during the
        // selection.  The routed grid is sized so that, with them, every CU holds
        // at most three workgroups: a fourth workgroup on some CUs starts its
        // selection later and streams slower than the rest, and sets the end.
        const int sh1 = (a.Fs + S::BF - 1) / S::BF;
        const long cap3 = (long)device_cus() * 3;
        while ((long)((blocks1 + passes - 1) / passes) * a.max_units + sh1 > cap3 && passes < blocks1) passes++;
        gx = (blocks1 + passes - 1) / passes;
        const long left = cap - (long)gx * a.max_units;
        while ((long)((sh1 + passes_sh - 1) / passes_sh) > left && passes_sh < sh1) passes_sh++;
        nsh = (sh1 + passes_sh - 1) / passes_sh;
    } else {
        const int units = a.max_units + 1;
        while ((long)((blocks1 + passes - 1) / passes) * units > cap && passes < blocks1) passes++;
        gx = (blocks1 + passes - 1) / passes;
        passes_sh = passes;
        nsh = a.with_shared ? gx : 0;
    }
    const long blocks = nsh + (long)gx * a.max_units;
    ProfScope prof(GU ? "ffn_gateup" : "ffn_down", st);
    q4_gemv_kernel<LPR, RM, GU, FMT><<<(unsigned)blocks, 256, lds, st>>>(a, passes, passes_sh, nsh, gx);
    return hipGetLastError();
}

template <bool GU, int FMT>
static hipError_t dispatch_fmt(const FfnArgs &a, int N, int K, int rm, hipStream_t st) {
    const int lpr = lanes_per_row(K);
#define MOE_GEMV_CASE(L)                                                  \
    if (lpr == L) {                                                       \
        if (rm == 1) return launch_one<L, 1, GU, FMT>(a, N, K, st);       \
        if (rm == 2) return launch_one<L, 2, GU, FMT>(a, N, K, st);       \
        return launch_one<L, 4, GU, FMT>(a, N, K, st);                    \
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

// The gate/up (GU) or down kernels of one expert format; each format's kernels are
// instantiated in a translation unit of their own (ffn_gemv.hip, ffn_gemv_i3.hip,
// ffn_gemv_f4.hip).
template <int FMT>
hipError_t gemv_dispatch(bool GU, const FfnArgs &a, int N, int K, int rm, hipStream_t st) {
    return GU ? dispatch_fmt<true, FMT>(a, N, K, rm, st) : dispatch_fmt<false, FMT>(a, N, K, rm, st);
}
extern template hipError_t gemv_dispatch<kFmtI4>(bool, const FfnArgs &, int, int, int, hipStream_t);
extern template hipError_t gemv_dispatch<kFmtI3>(bool, const FfnArgs &, int, int, int, hipStream_t);
extern template hipError_t gemv_dispatch<kFmtF4>(bool, const FfnArgs &, int, int, int, hipStream_t);

int rows_per_pass(int T, int K, int fmt);

}  // namespace moe

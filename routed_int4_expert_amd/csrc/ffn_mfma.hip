// ffn_mfma.hip -- step 4 of the MoE layer on gfx950 for larger row counts: the
// int4-gs64 SwiGLU expert FFN as a grouped GEMM on the matrix cores
// ("MoE 路由与专家流式加载" §1.3: gate, up, SiLU, down for every union expert,
// each expert's weights read once for all rows routed to it; §1.4: the shared
// expert on every token).
//
// D[rows][outputs] = X[rows][K] * W[outputs][K]^T with v_mfma_f32_16x16x32_bf16.
//  - B (weights): for one 64-group of one output row, lane (column j, part p)
//    holds words 2p and 2p+1 (8 bytes, 16 codes).  Each 32-bit word of 8 codes
//    becomes 4 bf16 pairs of (136 + q) by one bit operation per pair (0x4300 is
//    128.0; q XOR 8 = q + 8), so the codes enter the matrix core exactly
//    ("colibrì 深度拆解" §5.2 packing).  Word 2p+ks feeds K-step ks.
//  - A (activations): prepared once as bf16 hi + lo (16 significant bits) in
//    the codes' element order (per word: elements 0,4,1,5,2,6,3,7), 256 bytes
//    per row and group; hi and lo are two MFMAs on the same B.
//  - per 64-group ("colibri 开发演进实录" §2.1 gs64) the group accumulator
//    starts at -136 * sum(x) (the unsigned-offset identity of §2.2, K1) and its
//    result is scaled by the fp32 group scale into the fp32 running sum.
//
// Work item = up to 16 rows of one expert (one 16-row MFMA block) x a block
// of outputs: 4 waves x 32 outputs (gate and up for the same columns) or
// 4 waves x 64 outputs (down).  Experts with more rows, and the shared expert,
// span several items.  K advances in chunks of 4 groups.  The weight stream is
// kept in flight by a ring of three register slots (the chunk being computed
// and the next two).  Activation chunks are loaded into registers two steps
// ahead and written to the other of two LDS buffers after each compute; the
// barrier between steps waits only for those LDS writes, and loads are issued
// in an order where no wait for one covers data needed later (completions are
// counted in issue order), so the weight loads stay in flight across steps.  Every output has one owner:
// the result is deterministic.
#include <math.h>

#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr uint32_t kPairOffset = 0x43084308u;   // bf16 pair (136 + q) from a code pair
constexpr float kMfmaCodeOffset = 136.0f;
constexpr int kGroupBytes = 256;                // one row's 64-group: 8 x 16 B hi, then 8 x 16 B lo
constexpr int kCG = 4;                          // groups per K chunk
constexpr int kChunkBytes = kCG * kGroupBytes;  // a row's chunk: 1 KB, one wave-wide LDS copy
constexpr int kRowPitch = kChunkBytes + 16;     // +16: rows start in distinct LDS banks
constexpr int kTileBytes = kMfmaItemRows * kRowPitch;
// a wave's weight codes of one chunk, regrouped through LDS: 4 B blocks x 16 rows x
// 128 B, rows 144 B apart so the 8-byte operand reads of 16 rows hit distinct banks
constexpr int kCodePitch = 144;
constexpr int kCodeBytes = 4 * 16 * kCodePitch;

__device__ __forceinline__ uint32_t bf16_rne_u(float f) {
    const uint32_t b = __float_as_uint(f);
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// ------------------------------------------------------------------ prep
// Rows of K fp32 values -> per 64-group G: 256 bytes, word w (elements
// 64G + 8w .. +7) as 8 bf16 hi at 16w and 8 bf16 lo at 128 + 16w, elements in
// the order 0,4,1,5,2,6,3,7; and nsx[row][G] = -136 * sum of (hi + lo) over the
// group.  Rows are NGp groups long (whole chunks).  One thread per word; the 8
// words of a group are 8 adjacent lanes.
struct PrepJob {
    const float *src;
    int rows, K;
    uint8_t *frag;
    float *nsx;
    int blocks;  // workgroups of 256 threads this job takes
};

__device__ __forceinline__ void prep_frag_body(const PrepJob &j, int blk) {
    const float *src = j.src;
    const int rows = j.rows, K = j.K;
    const long i = (long)blk * blockDim.x + threadIdx.x;  // word index
    const long nwd = (long)rows * (K / 8);
    const bool live = i < nwd;
    const long ii = live ? i : nwd - 1;
    const int row = (int)(ii / (K / 8)), b = (int)(ii % (K / 8));
    const int NGp = mfma_groups_padded(K);
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
    const int G = b / 8, w = b % 8;
    uint8_t *grp = j.frag + ((size_t)row * NGp + G) * kGroupBytes;
    if (live) {
        *reinterpret_cast<uint4 *>(grp + 16 * w) =
            make_uint4(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16), hb[4] | (hb[5] << 16),
                       hb[6] | (hb[7] << 16));
        *reinterpret_cast<uint4 *>(grp + 128 + 16 * w) =
            make_uint4(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16), lb[4] | (lb[5] << 16),
                       lb[6] | (lb[7] << 16));
    }
    // group sum over the 8 words = 8 adjacent lanes (K is a multiple of 64)
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) part += __shfl_xor(part, m, kWave);
    if (live && w == 0) j.nsx[(size_t)row * NGp + G] = -kMfmaCodeOffset * part;
}

static PrepJob prep_job(const float *src, int rows, int K, uint8_t *frag, float *nsx) {
    PrepJob j;
    j.src = src;
    j.rows = rows;
    j.K = K;
    j.frag = frag;
    j.nsx = nsx;
    const long nwd = rows > 0 ? (long)rows * (K / 8) : 0;
    j.blocks = (int)((nwd + 255) / 256);
    return j;
}

// ------------------------------------------------------------------ work list
// Items in union order: expert uniq[u] with c rows gets ceil(c / 16) items of
// consecutive rows.  One workgroup of 256 threads, one thread per union slot
// (E <= 256); an exclusive scan of the item counts places each expert's items.
__device__ __forceinline__ void mfma_items_body(const int32_t *n_uniq, const int32_t *uniq,
                                                const int32_t *off, int E, int32_t *items,
                                                int32_t *n_items) {
    __shared__ int wsum[256 / kWave];
    const int u = threadIdx.x, lane = u % kWave, wv = u / kWave;
    const int nu = n_uniq[0];
    int e = -1, cnt = 0;
    if (u < nu && u < E) {
        e = uniq[u];
        cnt = off[e + 1] - off[e];
    }
    const int ni = (cnt + kMfmaItemRows - 1) / kMfmaItemRows;
    int inc = ni;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(inc, d, kWave);
        if (lane >= d) inc += o;
    }
    if (lane == kWave - 1) wsum[wv] = inc;
    __syncthreads();
    int base = inc - ni;
    for (int v = 0; v < wv; v++) base += wsum[v];
    for (int i = 0; i < ni; i++) {
        int32_t *it = items + 4 * (base + i);
        it[0] = e;
        it[1] = off[e] + kMfmaItemRows * i;
        it[2] = min(kMfmaItemRows, cnt - kMfmaItemRows * i);
        it[3] = 0;
    }
    if (u == blockDim.x - 1) n_items[0] = base + ni;
}

// Up to two fragment preparations and, optionally, the work list, in one launch:
// workgroups [0, j0.blocks) prepare job 0, the next j1.blocks job 1, and one more
// builds the work list when `items` is set.
struct ItemsJob {
    const int32_t *n_uniq, *uniq, *off;
    int E;
    int32_t *items, *n_items;
};

__global__ __launch_bounds__(256) void prep_kernel(PrepJob j0, PrepJob j1, ItemsJob it) {
    const int b = blockIdx.x;
    if (b < j0.blocks)
        prep_frag_body(j0, b);
    else if (b < j0.blocks + j1.blocks)
        prep_frag_body(j1, b - j0.blocks);
    else if (it.items)
        mfma_items_body(it.n_uniq, it.uniq, it.off, it.E, it.items, it.n_items);
}

static hipError_t launch_prep(const PrepJob &j0, const PrepJob &j1, const ItemsJob &it,
                              const char *name, hipStream_t st) {
    const int blocks = j0.blocks + j1.blocks + (it.items ? 1 : 0);
    if (blocks == 0) return hipSuccess;
    ProfScope prof(name, st);
    prep_kernel<<<blocks, 256, 0, st>>>(j0, j1, it);
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

// The LDS writes of this wave are done; meet the other waves.  Written out so
// that no wait for the weight loads in flight is added.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <bool GU>
__global__ __launch_bounds__(256, 2) void q4_mfma_kernel(MfmaArgs a) {
    // activation chunks, double-buffered: [row][1 KB + 16] and [row][4 groups]
    __shared__ __attribute__((aligned(16))) uint8_t at0[kTileBytes];
    __shared__ __attribute__((aligned(16))) uint8_t at1[kTileBytes];
    __shared__ __attribute__((aligned(16))) float ns0[kMfmaItemRows * 4];  // -136*sum(x)
    __shared__ __attribute__((aligned(16))) float ns1[kMfmaItemRows * 4];
    __shared__ __attribute__((aligned(16))) uint8_t cbuf[4][kCodeBytes];  // per wave

    // ---- the item: rows [row0, row0 + R) of a routed expert e, or of the shared expert (e < 0)
    const int item = blockIdx.y;
    int e, row0, R;
    if (item < a.max_items) {
        if (!a.with_routed || item >= a.n_items[0]) return;
        e = a.items[4 * item];
        row0 = a.items[4 * item + 1];
        R = a.items[4 * item + 2];
    } else {
        if (!a.with_shared) return;
        e = -1;
        row0 = (item - a.max_items) * kMfmaItemRows;
        R = min(kMfmaItemRows, a.T - row0);
        if (R <= 0) return;
    }
    const int H = a.H;
    const int Fu = e >= 0 ? a.F : a.Fs;
    const int K = GU ? H : Fu;
    const int N = GU ? Fu : H;
    const int NG = K / 64;
    const int NGp = mfma_groups_padded(K);
    constexpr int kWaveOut = GU ? 32 : 64;
    const int nb0 = blockIdx.x * (4 * kWaveOut);
    if (nb0 >= N) return;

    moe_q4 m0, m1;
    const int32_t *rt = nullptr;  // token of each row (routed gate/up), else rows are contiguous
    const uint8_t *afrag;
    const float *ansx;
    float *out;
    if (e >= 0) {
        if (GU) {
            const size_t gq = (size_t)e * Fu * (H / 2), gs = (size_t)e * Fu * (H / 64);
            m0.q = a.gate.q + gq; m0.s = a.gate.s + gs;
            m1.q = a.up.q + gq;   m1.s = a.up.s + gs;
            rt = a.row_tok + row0;
            afrag = a.x_frag;
            ansx = a.x_nsx;
            out = a.h_routed + (size_t)row0 * N;
        } else {
            const size_t dq = (size_t)e * H * (Fu / 2), ds = (size_t)e * H * (Fu / 64);
            m0.q = a.down.q + dq; m0.s = a.down.s + ds;
            m1 = m0;
            afrag = a.hr_frag + (size_t)row0 * NGp * kGroupBytes;
            ansx = a.hr_nsx + (size_t)row0 * NGp;
            out = a.y_routed + (size_t)row0 * N;
        }
    } else {
        if (GU) {
            m0 = a.sh_gate; m1 = a.sh_up;
            afrag = a.x_frag + (size_t)row0 * NGp * kGroupBytes;
            ansx = a.x_nsx + (size_t)row0 * NGp;
            out = a.h_shared + (size_t)row0 * N;
        } else {
            m0 = a.sh_down; m1 = m0;
            afrag = a.hs_frag + (size_t)row0 * NGp * kGroupBytes;
            ansx = a.hs_nsx + (size_t)row0 * NGp;
            out = a.y_shared + (size_t)row0 * N;
        }
    }

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int j = lane % 16, p = lane / 16;
    const int nchunks = (NG + kCG - 1) / kCG;

    // ---- B blocks: GU -> (gate, cols 0-15), (gate, 16-31), (up, 0-15), (up, 16-31) of the
    // wave's 32 outputs; down -> 4 x 16 of its 64 outputs.  A lane's column, clamped for
    // loads (never stored past N).
    int ncol[4];
    uint32_t soff[4];
#pragma unroll
    for (int b = 0; b < 4; b++) {
        const int cb = GU ? b % 2 : b;
        ncol[b] = nb0 + wv * kWaveOut + cb * 16 + j;
        soff[b] = (uint32_t)min(ncol[b], N - 1) * (uint32_t)NG;
    }
    // code loads are coalesced: for a block of 16 rows, load i (0, 1) gives lane l row
    // 8i + l/8 and bytes 16 (l % 8) of the row's 128-byte chunk (4 groups); rows past N
    // re-read row N-1 (never stored)
    constexpr int kColBlocks = GU ? 2 : 4;
    uint32_t qrow[kColBlocks][2];
#pragma unroll
    for (int cb = 0; cb < kColBlocks; cb++)
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int n = min(nb0 + wv * kWaveOut + cb * 16 + 8 * i + lane / 8, N - 1);
            qrow[cb][i] = (uint32_t)n * (uint32_t)(K / 2);
        }
    const uint32_t qlast = (uint32_t)(K / 2 - 16);  // last 16-byte piece of a row
    auto qbase = [&](int b) { return (GU && b >= 2) ? m1.q : m0.q; };
    auto sbase = [&](int b) { return (GU && b >= 2) ? m1.s : m0.s; };

    // ---- activation staging: wave wv moves rows wv + 4i (16 bytes per lane of each
    // row's 1-KB chunk), lanes 0-15 the group sums of rows 0-15.  Rows past R repeat
    // row R-1 (cached, finite; their outputs are never stored), so staging has no branches.
    constexpr int kRowsPerWave = kMfmaItemRows / 4;
    int srow[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; i++) {
        const int r = min(wv + 4 * i, R - 1);
        srow[i] = rt ? rt[r] : r;
    }
    const int lr = min(lane % kMfmaItemRows, R - 1);
    const int nsrow = rt ? rt[lr] : lr;
    struct Staged {
        uint4 a[kRowsPerWave];
        uint4 n;
    };
    // values are returned, not kept in a captured array, so they stay in registers
    auto stage_load = [&](int c) __attribute__((always_inline)) {
        const int g0 = c * kCG;
        Staged v;
#pragma unroll
        for (int i = 0; i < kRowsPerWave; i++)
            v.a[i] = *reinterpret_cast<const uint4 *>(
                afrag + ((size_t)srow[i] * NGp + g0) * kGroupBytes + 16 * lane);
        v.n = *reinterpret_cast<const uint4 *>(ansx + (size_t)nsrow * NGp + g0);
        return v;
    };
    auto stage_store = [&](const Staged &v, uint8_t *tile, float *nst) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kRowsPerWave; i++)
            *reinterpret_cast<uint4 *>(tile + (wv + 4 * i) * kRowPitch + 16 * lane) = v.a[i];
        if (wv == 0 && lane < kMfmaItemRows) *reinterpret_cast<uint4 *>(nst + 4 * lane) = v.n;
    };

    u32x4_t cq[3][4][2];
    float cs[3][4];
    auto fetch = [&](int c, u32x4_t (&q)[4][2], float (&s)[4]) __attribute__((always_inline)) {
        const int g0 = min(c, nchunks - 1) * kCG;  // past the end: re-fetch the last chunk
        // past the row's end (a last chunk of fewer than 4 groups): re-read its last piece
        const uint32_t off = min((uint32_t)(32 * g0 + 16 * (lane % 8)), qlast);
#pragma unroll
        for (int b = 0; b < 4; b++)
#pragma unroll
            for (int i = 0; i < 2; i++)
                q[b][i] = *reinterpret_cast<const u32x4_t *>(qbase(b) + (qrow[GU ? b % 2 : b][i] + off));
        // lane (j, p) fetches its column's scale of group g0 + p
#pragma unroll
        for (int b = 0; b < 4; b++) s[b] = sbase(b)[soff[b] + (uint32_t)min(g0 + p, NG - 1)];
    };

    f32x4_t acc[4];
#pragma unroll
    for (int b = 0; b < 4; b++) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    uint8_t *cw = cbuf[wv];
    auto compute = [&](int c, const uint8_t *tile, const float *nst, const u32x4_t (&q)[4][2],
                       const float (&s)[4]) __attribute__((always_inline)) {
        const int ng = min(kCG, NG - c * kCG);
        // regroup the chunk's codes: row-major into this wave's LDS area, then each lane
        // reads its column's words 2p, 2p+1 of every group
#pragma unroll
        for (int b = 0; b < 4; b++)
#pragma unroll
            for (int i = 0; i < 2; i++)
                *reinterpret_cast<u32x4_t *>(cw + (16 * b + 8 * i + lane / 8) * kCodePitch + 16 * (lane % 8)) = q[b][i];
#pragma unroll
        for (int gi = 0; gi < kCG; gi++) {
            if (gi >= ng) break;
            // the column's group scale sits in lane j + 16 gi
            float sg[4];
#pragma unroll
            for (int b = 0; b < 4; b++) sg[b] = __shfl(s[b], j + 16 * gi, kWave);
            // group accumulators start at -136 * sum(x) of rows 4p .. 4p+3
            f32x4_t ga;
#pragma unroll
            for (int v = 0; v < 4; v++) ga[v] = nst[(4 * p + v) * 4 + gi];
            f32x4_t g[4];
#pragma unroll
            for (int b = 0; b < 4; b++) g[b] = ga;
            uint2 w[4];
#pragma unroll
            for (int b = 0; b < 4; b++)
                w[b] = *reinterpret_cast<const uint2 *>(cw + (16 * b + j) * kCodePitch + 32 * gi + 8 * p);
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                const uint8_t *ar = tile + j * kRowPitch + gi * kGroupBytes + 16 * (2 * p + ks);
                const bf16x8_t ah = *reinterpret_cast<const bf16x8_t *>(ar);
                const bf16x8_t al = *reinterpret_cast<const bf16x8_t *>(ar + 128);
                bf16x8_t bo[4];
#pragma unroll
                for (int b = 0; b < 4; b++) bo[b] = code_pairs(ks ? w[b].y : w[b].x);
#pragma unroll
                for (int b = 0; b < 4; b++) g[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bo[b], g[b], 0, 0, 0);
#pragma unroll
                for (int b = 0; b < 4; b++) g[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bo[b], g[b], 0, 0, 0);
            }
#pragma unroll
            for (int b = 0; b < 4; b++)
#pragma unroll
                for (int v = 0; v < 4; v++) acc[b][v] = fmaf(sg[b], g[b][v], acc[b][v]);
        }
    };

    // One chunk step.  Loads are issued so that no wait covers data needed later:
    // the activations of chunk c+2 (before the codes of c+2, so writing them to LDS two
    // steps later never waits for codes that are still ahead of use), then the codes
    // of c+2 into the slot just freed.  The activations of c+1, loaded a step ago, go to
    // the other LDS buffer after the compute.  Staging register sets alternate.
    Staged stg0, stg1;
    auto step = [&](int c, int slot, Staged &ld, const Staged &st) __attribute__((always_inline)) {
        const bool odd = c & 1;
        lds_barrier();
        ld = stage_load(min(c + 2, nchunks - 1));  // past the end: re-load the last chunk (not stored)
        fetch(c + 2, cq[(slot + 2) % 3], cs[(slot + 2) % 3]);
        compute(c, odd ? at1 : at0, odd ? ns1 : ns0, cq[slot], cs[slot]);
        if (c + 1 < nchunks) stage_store(st, odd ? at0 : at1, odd ? ns0 : ns1);
    };

    {
        const Staged first = stage_load(0);
        fetch(0, cq[0], cs[0]);
        stg1 = stage_load(min(1, nchunks - 1));
        fetch(1, cq[1], cs[1]);
        stage_store(first, at0, ns0);
    }
    // whole turns of both rings (codes: 3 slots, staging: 2 sets) without branches
    // inside, then the rest
    int c = 0;
    for (; c + 6 <= nchunks; c += 6) {
        step(c, 0, stg0, stg1);
        step(c + 1, 1, stg1, stg0);
        step(c + 2, 2, stg0, stg1);
        step(c + 3, 0, stg1, stg0);
        step(c + 4, 1, stg0, stg1);
        step(c + 5, 2, stg1, stg0);
    }
    if (c < nchunks) step(c, 0, stg0, stg1);
    if (c + 1 < nchunks) step(c + 1, 1, stg1, stg0);
    if (c + 2 < nchunks) step(c + 2, 2, stg0, stg1);
    if (c + 3 < nchunks) step(c + 3, 0, stg1, stg0);
    if (c + 4 < nchunks) step(c + 4, 1, stg0, stg1);

    // ---- epilogue.  D layout: register v of lane (j, p) is row 4p + v, column j of the block
#pragma unroll
    for (int b = 0; b < (GU ? 2 : 4); b++) {
        const int n = ncol[b];
        if (n >= N) continue;
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const int r = 4 * p + v;
            if (r >= R) continue;
            float val;
            if (GU) {
                const float gg = acc[b][v], uu = acc[b + 2][v];
                val = gg / (1.0f + expf(-gg)) * uu;
            } else {
                val = acc[b][v];
            }
            out[(size_t)r * N + n] = val;
        }
    }
}

// x prepared once with the work list; gate/up for every item; the routed and shared
// h prepared together; down.
hipError_t launch_ffn_mfma(const MfmaArgs &a, hipStream_t st) {
    hipError_t e;
    const PrepJob none = prep_job(nullptr, 0, 64, nullptr, nullptr);
    ItemsJob it;
    it.n_uniq = a.n_uniq;
    it.uniq = a.uniq;
    it.off = a.off;
    it.E = a.E;
    it.items = a.with_routed ? a.items : nullptr;
    it.n_items = a.n_items;
    e = launch_prep(prep_job(a.x, a.T, a.H, a.x_frag, a.x_nsx), none, it, "prep_x+items", st);
    if (e != hipSuccess) return e;
    const int shared_items = a.with_shared ? (a.T + kMfmaItemRows - 1) / kMfmaItemRows : 0;
    const int nmax = a.with_shared ? (a.with_routed ? max(a.F, a.Fs) : a.Fs) : a.F;
    {
        dim3 grid((nmax + 127) / 128, a.max_items + shared_items);
        ProfScope prof("ffn_gateup_mfma", st);
        q4_mfma_kernel<true><<<grid, 256, 0, st>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // h rows in fragment order: the routed rows (as many as the largest union can
    // have) and the shared rows
    ItemsJob no_items = it;
    no_items.items = nullptr;
    e = launch_prep(a.with_routed ? prep_job(a.h_routed, a.max_rows, a.F, a.hr_frag, a.hr_nsx) : none,
                    a.with_shared ? prep_job(a.h_shared, a.T, a.Fs, a.hs_frag, a.hs_nsx) : none,
                    no_items, "prep_h", st);
    if (e != hipSuccess) return e;
    {
        dim3 grid((a.H + 255) / 256, a.max_items + shared_items);
        ProfScope prof("ffn_down_mfma", st);
        q4_mfma_kernel<false><<<grid, 256, 0, st>>>(a);
        return hipGetLastError();
    }
}

}  // namespace moe

// ffn_mfma.hip -- step 4 of the MoE layer on gfx950 for larger row counts: the
// int4-gs64 SwiGLU expert FFN as a grouped GEMM on the matrix cores
// ("MoE 路由与专家流式加载" §1.3: gate, up, SiLU, down for every union expert,
// each expert's weights read once for all rows routed to it; §1.4: the shared
// expert on every token).
//
// D[rows][outputs] = X[rows][K] * W[outputs][K]^T with v_mfma_i32_16x16x64_i8.
//  - B (weights): for one 64-group of one output row, lane (column j, part p)
//    holds words 2p and 2p+1 (8 bytes, 16 codes).  A code nibble masked in the
//    high half of its byte is 16 q as a signed byte: the odd elements of a word
//    are w AND 0xF0F0F0F0, the even ones (w << 4) AND 0xF0F0F0F0, so the codes
//    enter the matrix core exactly ("colibrì 深度拆解" §5.2 packing).
//  - A (activations): prepared once per row and 256-element K chunk as 16-bit
//    fixed point, x16 = rint(x * 2^n) with the power-of-two step 2^-n that maps
//    max|x| to at most 32639 (act_shift), split into signed bytes
//    x16 = 256 hi + lo (the unsigned-offset and split identities of
//    "colibri 开发演进实录" §2.2, K1, with the offset removed by the sign-carrying
//    codes), in the codes' element order (per word: 0,2,4,6 then 1,3,5,7),
//    128 bytes per row and group; hi and lo are two MFMAs on the same B, each an
//    exact int32 sum.
//  - per 64-group ("colibri 开发演进实录" §2.1 gs64) 256 hi + lo is converted to
//    fp32 and scaled by the group scale into the chunk's sum, which the row's
//    chunk step (over 16 for the codes' factor) scales into the fp32 running sum.
//    The one rounding of x is x16 itself.
//
// int3-g64 codes (moe.h bit planes) take the same path: a lane's operand is one word of
// the low-bit plane (16 codes in the int4 order above) and its 16 sign bits, placed
// as 32 c in the top three bits of each byte (the chunk's sums then carry a factor
// 32 instead of 16).
// MXFP4 codes are turned into their exact bf16 values (E2M1 times the block's power of
// two, by the hardware's scaled fp4 -> bf16 conversion) and multiply bf16 activations
// on v_mfma_f32_16x16x32_bf16, one 32-element block (one scale) per product; each
// activation enters as two bf16 terms hi = bf16(x), lo = bf16(x - hi), 256 bytes per
// row and 64-group (hi of the group's two blocks, then lo), and the products
// accumulate in the fp32 accumulators across the whole reduction.
//
// Work item = up to 16 or, for batches with many rows per expert, 32 rows of one
// expert (one or two 16-row MFMA blocks) x a block of outputs: 4 column sets x 32
// outputs (gate and up for the same columns) or 4 x 64 outputs (down).  Experts with more rows, and the shared expert, span several
// items.  The kernel is persistent (one workgroup of 12 waves per CU, looping over
// (item, output block) pairs) and splits loading from computing: 4 loader waves keep
// two 4-group K chunks in flight in registers and place each one in one of two LDS
// buffers (codes regrouped for the operand reads, scales, the activation tile and the
// rows' chunk steps); 8 compute waves, two per column set, run the MFMAs on the
// other buffer, issuing a group's MFMAs before converting the next group's codes; the
// converted codes serve both row blocks of an item.  One barrier per chunk.  Every
// output has one owner: the result is deterministic.

#include <math.h>

#include <type_traits>

#include "moe_internal.h"
#include "select_union.h"

namespace moe {

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr uint32_t kHighNibbles = 0xF0F0F0F0u;  // 16 q per byte
constexpr int kCG = 4;                          // groups per K chunk
// one row's 64-group of prepared activations: 4 x 16 B hi, then 4 x 16 B lo (int8
// limbs), or 2 x 64 B hi, then 2 x 64 B lo (bf16 terms, MXFP4)
template <int FMT>
constexpr int group_bytes() { return FMT == kFmtF4 ? 256 : 128; }
template <int FMT>
constexpr int chunk_bytes() { return kCG * group_bytes<FMT>(); }  // a row's chunk: 512 or 1024 B
template <int FMT>
constexpr int row_pitch() { return chunk_bytes<FMT>() + 16; }     // +16: rows start in distinct LDS banks
// a column set's weight codes of one chunk in LDS: 4 B blocks x 16 rows x 128 B, rows
// 144 B apart so the 8-byte operand reads of 16 rows hit distinct banks
constexpr int kCodePitch = 144;

// ------------------------------------------------------------------ prep
// Rows of K fp32 values -> per 256-element chunk c: step[row][c] = 2^-act_shift(max|x|)
// (NaN if the chunk holds a non-finite value, 0 if it is all zero) and, per 64-group
// G, 128 bytes: for word w (elements 64G + 8w .. +7) the hi bytes of its even
// elements (0,2,4,6) and of its odd ones at 8w, the lo bytes likewise at 64 + 8w.
// Rows are NGp groups long (whole chunks).  One thread per word, the 32 words of a
// chunk in 32 adjacent lanes (threads of words past K write nothing).
struct PrepJob {
    const float *src;
    int rows, K;
    uint8_t *frag;
    float *step;
    int blocks;  // workgroups of 256 threads this job takes
    int act8;    // the opt-in 8-bit codes (hi bytes 0, lo bytes the code)
    int bf16;    // the MXFP4 path's two bf16 terms per value instead (no steps)
    // the rows in use, or nullptr for all: the routed h rows stop at the union's row count
    // off[E] (top-p may keep fewer than T*k picks); no work item reads a row past it
    const int32_t *live_rows;
};

__device__ __forceinline__ uint16_t bf16_bits_rne(float v) {
    const uint32_t b = __float_as_uint(v);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((b >> 16) | 0x40u);  // NaN stays NaN
    return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ uint32_t pack_bytes(int a, int b, int c, int d) {
    return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) | ((uint32_t)(c & 0xFF) << 16) |
           ((uint32_t)d << 24);
}

__device__ __forceinline__ void prep_frag_body(const PrepJob &j, int blk) {
    const int rows = j.rows, K = j.K;
    const int NGp = mfma_groups_padded(K), NC = NGp / kCG;
    const long i = (long)blk * blockDim.x + threadIdx.x;  // (row, chunk, word of the chunk)
    const long n = (long)rows * NC * 32;
    const long ii = i < n ? i : n - 1;
    const int row = (int)(ii / (NC * 32)), c = (int)(ii / 32 % NC), w = (int)(ii % 32);
    // (uniform over a chunk's 32 lanes, which all hold the same row)
    const bool in_rows = i < n && (!j.live_rows || row < j.live_rows[0]);
    const int b = 32 * c + w;  // word of the row
    const bool live = in_rows && b < K / 8;
    float e[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (live) {
        const float4 *p = reinterpret_cast<const float4 *>(j.src + (size_t)row * K + 8 * b);
        const float4 v0 = p[0], v1 = p[1];
        e[0] = v0.x; e[1] = v0.y; e[2] = v0.z; e[3] = v0.w;
        e[4] = v1.x; e[5] = v1.y; e[6] = v1.z; e[7] = v1.w;
    }
    if (j.bf16) {
        // hi = bf16(x), lo = bf16(x - hi) (x - hi is exact in fp32), in element order:
        // word b of the row is block (b % 8) / 4 of group b / 8, 16 bytes at (b % 4) * 16
        if (live) {
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int s = 0; s < 4; s++) {
                const uint16_t h0 = bf16_bits_rne(e[2 * s]), h1 = bf16_bits_rne(e[2 * s + 1]);
                const float r0 = e[2 * s] - __uint_as_float((uint32_t)h0 << 16);
                const float r1 = e[2 * s + 1] - __uint_as_float((uint32_t)h1 << 16);
                hw[s] = (uint32_t)h0 | ((uint32_t)h1 << 16);
                lw[s] = (uint32_t)bf16_bits_rne(r0) | ((uint32_t)bf16_bits_rne(r1) << 16);
            }
            const int G = b / 8, wg = b % 8;
            uint8_t *grp = j.frag + ((size_t)row * NGp + G) * group_bytes<kFmtF4>() + (wg / 4) * 64 + (wg % 4) * 16;
            *reinterpret_cast<uint4 *>(grp) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
            *reinterpret_cast<uint4 *>(grp + 128) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        }
        return;
    }
    // the chunk's largest magnitude as bits (an integer max, so NaN and Inf count)
    uint32_t mb = 0;
#pragma unroll
    for (int s = 0; s < 8; s++) mb = max(mb, __float_as_uint(e[s]) & 0x7FFFFFFFu);
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) mb = max(mb, (uint32_t)__shfl_xor((int)mb, m, kWave));
    const bool finite = mb < 0x7F800000u;
    const bool nz = finite && mb != 0u;
    const ActRule rule = act_rule(j.act8);
    const int sh = nz ? act_shift(mb, rule) : 0;
    const float lim = rule.lim;
    int hi[8], lo[8];
#pragma unroll
    for (int s = 0; s < 8; s++) {
        const int x16 = nz ? (int)fminf(fmaxf(rintf(ldexpf(e[s], sh)), -lim), lim) : 0;
        hi[s] = (x16 + 128) >> 8;
        lo[s] = x16 - 256 * hi[s];
    }
    if (live) {
        const int G = b / 8, wg = b % 8;
        uint8_t *grp = j.frag + ((size_t)row * NGp + G) * group_bytes<kFmtI4>();
        *reinterpret_cast<uint2 *>(grp + 8 * wg) =
            make_uint2(pack_bytes(hi[0], hi[2], hi[4], hi[6]), pack_bytes(hi[1], hi[3], hi[5], hi[7]));
        *reinterpret_cast<uint2 *>(grp + 64 + 8 * wg) =
            make_uint2(pack_bytes(lo[0], lo[2], lo[4], lo[6]), pack_bytes(lo[1], lo[3], lo[5], lo[7]));
    }
    if (in_rows && w == 0) j.step[(size_t)row * NC + c] = finite ? (nz ? ldexpf(1.0f, -sh) : 0.0f) : __builtin_nanf("");
}

static PrepJob prep_job(const float *src, int rows, int K, uint8_t *frag, float *step, int act8 = 0,
                        int bf16 = 0, const int32_t *live_rows = nullptr) {
    PrepJob j;
    j.act8 = act8;
    j.bf16 = bf16;
    j.live_rows = live_rows;
    j.src = src;
    j.rows = rows;
    j.K = K;
    j.frag = frag;
    j.step = step;
    const long nwd = rows > 0 ? (long)rows * (mfma_groups_padded(K) / kCG) * 32 : 0;
    j.blocks = (int)((nwd + 255) / 256);
    return j;
}

// ------------------------------------------------------------------ work list
// Work items: expert e with c rows gets ceil(c / IR) items of consecutive rows.  The
// items of experts with more than 16 rows (items of two MFMA row blocks, about 1.5 times
// the work of one, or several items) come first, then the single items of the others;
// each class in union order, and an expert's items stay together, so that the pairs
// that read its weights run side by side and share them in L2.  The kernel deals its
// (item, output block) pairs to the workgroups in turn, so the longer pairs go out
// first and the shorter ones even out the end.  One workgroup of 256 threads, one
// thread per union slot (E <= 256); exclusive scans of the two item counts place each
// expert's items.
__device__ __forceinline__ int block_exclusive_scan(int v, int *total) {
    __shared__ int wsum[256 / kWave];
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
    int inc = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(inc, d, kWave);
        if (lane >= d) inc += o;
    }
    if (lane == kWave - 1) wsum[wv] = inc;
    __syncthreads();
    int base = inc - v;
    for (int w = 0; w < wv; w++) base += wsum[w];
    *total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();  // wsum is reused by the next scan
    return base;
}

__device__ __forceinline__ void place_items(int e, int c, int row_base, int IR, int32_t *items,
                                            int32_t *n_items) {
    const int ni = (c + IR - 1) / IR;
    const int nbig = c > 16 ? ni : 0;
    int big_total, small_total;
    const int big_base = block_exclusive_scan(nbig, &big_total);
    const int small_base = block_exclusive_scan(ni - nbig, &small_total);
    for (int i = 0; i < ni; i++) {
        const int pos = i < nbig ? big_base + i : big_total + small_base + (i - nbig);
        int32_t *it = items + 4 * pos;
        it[0] = e;
        it[1] = row_base + IR * i;
        it[2] = min(IR, c - IR * i);
        it[3] = 0;
    }
    if (threadIdx.x == 0) n_items[0] = big_total + small_total;
}

__device__ __forceinline__ void mfma_items_body(const int32_t *n_uniq, const int32_t *uniq,
                                                const int32_t *off, int E, int IR, int32_t *items,
                                                int32_t *n_items) {
    const int u = threadIdx.x;
    const int nu = n_uniq[0];
    int e = -1, cnt = 0, r0 = 0;
    if (u < nu && u < E) {
        e = uniq[u];
        cnt = off[e + 1] - off[e];
        r0 = off[e];
    }
    place_items(e, cnt, r0, IR, items, n_items);
}

// Up to two fragment preparations and, optionally, the work list, in one launch:
// workgroups [0, j0.blocks) prepare job 0, the next j1.blocks job 1, and one more
// builds the work list when `items` is set.
struct ItemsJob {
    const int32_t *n_uniq, *uniq, *off;
    int E;
    int item_rows;  // IR: rows per item
    int32_t *items, *n_items;
    int with_union;  // build the union first (uni), in this workgroup
    UnionArgs uni;
};

// The work list from the union's per-expert counts and offsets in LDS (union_block's
// layout): the same items, in the same order, as mfma_items_body.
__device__ __forceinline__ void mfma_items_from_counts(const int32_t *cnt, const int32_t *offs, int E,
                                                       int IR, int32_t *items, int32_t *n_items) {
    const int u = threadIdx.x;
    place_items(u, u < E ? cnt[u] : 0, u < E ? offs[u] : 0, IR, items, n_items);
}

__global__ __launch_bounds__(256) void prep_kernel(PrepJob j0, PrepJob j1, ItemsJob it) {
    extern __shared__ uint32_t prep_lds[];
    const int b = blockIdx.x;
    if (b < j0.blocks) {
        prep_frag_body(j0, b);
    } else if (b < j0.blocks + j1.blocks) {
        prep_frag_body(j1, b - j0.blocks);
    } else if (it.items) {
        if (it.with_union) {
            // the union ([R] §1.3), then the work list from its counts in LDS
            union_block(it.uni, it.uni.ids, it.uni.keff, prep_lds);
            __syncthreads();
            const int E = it.uni.E, W = (it.uni.T + 31) / 32, W8 = (W + 7) / 8;
            const int32_t *cnt = reinterpret_cast<const int32_t *>(prep_lds + (size_t)E * W + (size_t)E * W8);
            mfma_items_from_counts(cnt, cnt + E, E, it.item_rows, it.items, it.n_items);
        } else {
            mfma_items_body(it.n_uniq, it.uniq, it.off, it.E, it.item_rows, it.items, it.n_items);
        }
    }
}

// (a 256-thread workgroup places at most about four picks per thread; larger batches keep
// the union's own 1024-thread launch)
bool union_in_prep_fits(int E, int T, int k) {
    return (long)T * k <= 1024 && union_lds_words(E, T) * sizeof(uint32_t) <= 64 * 1024;
}

static hipError_t launch_prep(const PrepJob &j0, const PrepJob &j1, const ItemsJob &it,
                              const char *name, hipStream_t st) {
    const int blocks = j0.blocks + j1.blocks + (it.items ? 1 : 0);
    if (blocks == 0) return hipSuccess;
    const size_t lds = it.items && it.with_union ? union_lds_words(it.uni.E, it.uni.T) * sizeof(uint32_t) : 0;
    ProfScope prof(name, st);
    prep_kernel<<<blocks, 256, lds, st>>>(j0, j1, it);
    return hipGetLastError();
}

// ------------------------------------------------------------------ grouped GEMM
// 16 codes (two words) of one output row -> the 16 signed bytes 16 q of a B operand:
// per word its even elements, then its odd ones.
__device__ __forceinline__ i32x4_t code_bytes(uint2 w) {
    i32x4_t v;
    v.x = (int)((w.x << 4) & kHighNibbles);
    v.y = (int)(w.x & kHighNibbles);
    v.z = (int)((w.y << 4) & kHighNibbles);
    v.w = (int)(w.y & kHighNibbles);
    return v;
}

// The LDS writes of this wave are done; meet the other waves.  Written out so
// that no wait for the weight loads in flight is added.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Persistent grouped GEMM.  A workgroup of twelve waves runs per CU and loops over work
// items (item, output block) wi = blockIdx.x + k * gridDim.x.  Waves 0-7 compute,
// waves 8-11 load.  For each 4-group K chunk the loaders place, in one of two LDS
// buffers, the chunk's weight codes (regrouped so that a compute lane's operand words
// are one 8-byte read), its group scales and its activation tile; the compute waves
// work on the other buffer.  Compute waves 2c and 2c + 1 take the outputs of column
// set c.  The loaders keep the next two chunks in flight in a pair of register sets,
// across work-item boundaries; one barrier per chunk.
constexpr int kColSets = 4;
constexpr int kLoadWaves = 4;
constexpr int kLoadThreads = kWave * kLoadWaves;                // 256: one per weight row of a chunk
constexpr int kCW = 2;                                          // compute waves per column set
constexpr int kCompWaves = kColSets * kCW;
constexpr int kMfmaThreads = kWave * (kCompWaves + kLoadWaves);  // 768
constexpr int kNBL = 4 / kCW;                                   // 16-column blocks per compute wave
constexpr int kBufCodes = kColSets * 64 * kCodePitch;          // [column set][64 rows][144 B]
constexpr int kMaxWorkPerWg = 64;

// An LDS chunk buffer for items of IRB 16-row blocks: codes, scales ([256 columns]
// [4 groups] fp32, or for MXFP4 [256 columns][4 groups][2 blocks] fp32 powers of two),
// the activation tile [16 IRB rows][528 or 1040 B] and the rows' fp32 chunk steps.
template <int IRB, int FMT>
struct MfmaBuf {
    static constexpr int kScales = kColSets * 64 * 4 * 4 * (FMT == kFmtF4 ? 2 : 1);
    static constexpr int kRows = 16 * IRB;
    static constexpr int kAct = kRows * row_pitch<FMT>();
    static constexpr int kNs = kRows * 4;
    static constexpr int kBytes = kBufCodes + kScales + kAct + kNs;
    static constexpr int kActPerRow = chunk_bytes<FMT>() / 16 / 16;  // 16-byte loads per row and thread
    static constexpr int kActLoads = IRB * kActPerRow;              // per thread
    static_assert(kRows * chunk_bytes<FMT>() / 16 / kLoadThreads == kActLoads, "activation loads");
};

template <int IR>
struct WorkDesc {
    int e;      // expert, -1: shared
    int nb0;    // first output of the block
    int nch;    // K chunks (0: the block lies past this unit's outputs)
    int R;      // rows
    int row0;   // first row: union row (routed) or token (shared)
    int srow[IR];  // activation source row of each row (rows past R repeat R-1)
};


// the weight row (output) and matrix of loader row r (0..255) of a chunk
template <bool GU>
__device__ __forceinline__ int load_row_output(int r, int nb0, bool &second) {
    const int wv = r / 64, lr = r % 64, bb = lr / 16, jj = lr % 16;
    second = GU && bb >= 2;
    return GU ? nb0 + 32 * wv + (bb % 2) * 16 + jj : nb0 + 64 * wv + 16 * bb + jj;
}

template <int NA>
struct ChunkRegs {
    u32x4_t q[8];
    float s[4];
    uint4 a[NA];
    float n;
};

// 16 int3 codes of one output row (a low-plane word and the 16 sign bits at bits
// 4(p % 2) .. 4(p % 2) + 3 of each byte of the sign word) -> the 16 signed bytes 32 c:
// per bit pair s the four elements the int4 order puts in dword s.
__device__ __forceinline__ i32x4_t code_bytes_i3(uint32_t lw, uint32_t sw) {
    i32x4_t v;
    v.x = (int)(((lw << 5) & 0x60606060u) | ((sw << 7) & 0x80808080u));
    v.y = (int)(((lw << 3) & 0x60606060u) | ((sw << 6) & 0x80808080u));
    v.z = (int)(((lw << 1) & 0x60606060u) | ((sw << 5) & 0x80808080u));
    v.w = (int)(((lw >> 1) & 0x60606060u) | ((sw << 4) & 0x80808080u));
    return v;
}

// 8 E2M1 codes (one word, elements 2j in the low nibble of byte j) times the block's
// power of two -> the 8 exact bf16 values of a B operand, in element order.
__device__ __forceinline__ bf16x8_t code_bf16_f4(uint32_t w, float scale) {
    const bf16x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
    const bf16x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
    const bf16x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
    const bf16x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
    return bf16x8_t{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
}

// IRB: 16-row blocks per work item (items hold at most 16 IRB rows; with IRB = 2 an
// item of at most 16 rows computes one block).  Twelve waves: two compute waves per
// column set, each taking two of the set's four 16-column blocks (gate/up: a gate block
// and its up block), and four loaders, three waves per SIMD.  A wave's own MFMAs and
// VALU instructions do not overlap; with two compute waves per SIMD one wave's VALU
// work runs while the other's MFMAs execute.  The register budget of three waves per
// SIMD leaves the loaders two chunks in flight.
// A8: the opt-in 8-bit activations, whose hi bytes are zero: one MFMA per group (the lo
// bytes) and no shift-add.  TAB: routed experts read through the residency tier's
// pointer table (a separate instantiation: the table lookups would otherwise add
// register pressure to the default kernel).
template <bool GU, int IRB, bool A8, bool TAB, int FMT>
__global__ __launch_bounds__(kMfmaThreads, 1) void q4_mfma_kernel(MfmaArgs a) {
    constexpr int kThreads = kMfmaThreads, NBL = kNBL;
    using Buf = MfmaBuf<IRB, FMT>;
    constexpr int IR = Buf::kRows, kBufBytes = Buf::kBytes, kBufAct = Buf::kAct;
    constexpr int kActLoads = Buf::kActLoads, kRowBlocks = IRB, kActPerRow = Buf::kActPerRow;
    constexpr int kBufScales = Buf::kScales;
    constexpr int kGroupBytes = group_bytes<FMT>(), kChunkBytes = chunk_bytes<FMT>();
    constexpr int kRowPitch = row_pitch<FMT>();
    static_assert(!(A8 && FMT == kFmtF4), "the MXFP4 path has no 8-bit activations");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    WorkDesc<IR> *work = reinterpret_cast<WorkDesc<IR> *>(lds + 2 * kBufBytes);
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    constexpr int kBlk = GU ? 128 : 256;  // outputs per work item

    // ---- this workgroup's work items, described in LDS
    const int n_routed = a.with_routed ? a.n_items[0] : 0;
    const int n_sh = a.with_shared ? (a.T + IR - 1) / IR : 0;
    const int nmax = GU ? (a.with_shared ? (a.with_routed ? max(a.F, a.Fs) : a.Fs) : a.F) : a.H;
    const int nb = (nmax + kBlk - 1) / kBlk;
    const int total = (n_routed + n_sh) * nb;
    const int G = gridDim.x, g = blockIdx.x;
    const int nwi = g < total ? min((total - g + G - 1) / G, kMaxWorkPerWg) : 0;
    for (int idx = tid; idx < nwi * IR; idx += kThreads) {
        const int k = idx / IR, r = idx % IR;
        const int wi = g + k * G, y = wi / nb, b = wi % nb;
        int e, row0, R;
        if (y < n_sh) {  // the shared expert's items first (full-size but the last)
            e = -1;
            row0 = y * IR;
            R = min(IR, a.T - row0);
        } else {
            const int32_t *it = a.items + 4 * (y - n_sh);
            e = it[0];
            row0 = it[1];
            R = it[2];
        }
        const int N = GU ? (e >= 0 ? a.F : a.Fs) : a.H;
        const int K = GU ? a.H : (e >= 0 ? a.F : a.Fs);
        const int rr = min(r, R - 1);
        work[k].srow[r] = (GU && e >= 0) ? a.row_tok[row0 + rr] : row0 + rr;
        if (r == 0) {
            work[k].e = e;
            work[k].nb0 = b * kBlk;
            work[k].nch = b * kBlk < N ? (K / 64 + kCG - 1) / kCG : 0;
            work[k].R = R;
            work[k].row0 = row0;
        }
    }
    __syncthreads();
    int S = 0;  // chunks of all the work items, in order
    for (int k = 0; k < nwi; k++) S += work[k].nch;

    if (wv >= kCompWaves) {
        // ================= loader waves
        const int t = tid - kCompWaves * kWave;  // 0..255
        int lk = 0, lc = 0;                      // the next chunk to load: (work item, chunk)
        while (lk < nwi && work[lk].nch == 0) lk++;
        // this lane's row offsets in the current work item (set when the item changes),
        // from wave-uniform matrix bases.  Code row t/8 + 32i is a gate row for even i and
        // an up row for odd i (gate/up), whatever the lane; so is scale column sc_col(i).
        int pk = -1;
        const uint8_t *qb0 = nullptr, *qb1 = nullptr, *abase = nullptr;
        const uint8_t *sb0 = nullptr, *sb1 = nullptr;  // scales, as bytes
        const float *nbase = nullptr;                  // chunk steps
        uint32_t qo[8], so[4], no = 0;
        const uint8_t *arow[kRowBlocks] = {};  // 64-bit: union rows x fragment bytes can pass 2^32
        bool two = false;                       // the item has a second row block
        uint32_t qlast = 0;
        int NG = 1;
        auto sc_col = [&](int i) __attribute__((always_inline)) {
            const int q = t / 4;
            return (q % 32) + 32 * (i & 1) + 64 * ((q / 32) + 2 * (i >> 1));
        };
        auto rows_of = [&](int k) __attribute__((always_inline)) {
            const WorkDesc<IR> &d = work[k];
            const int e = __builtin_amdgcn_readfirstlane(d.e);
            const int nb0 = __builtin_amdgcn_readfirstlane(d.nb0);
            int K, N;
            if (GU) {
                K = a.H;
                N = e >= 0 ? a.F : a.Fs;
                if (TAB && e >= 0) {  // the residency tier's slots
                    qb0 = a.tab[3 * e].q;     sb0 = static_cast<const uint8_t *>(a.tab[3 * e].s);
                    qb1 = a.tab[3 * e + 1].q; sb1 = static_cast<const uint8_t *>(a.tab[3 * e + 1].s);
                } else if (e >= 0) {
                    const size_t gq = (size_t)e * a.F * fmt_code_bytes(FMT, a.H), gs = (size_t)e * a.F * fmt_scale_bytes(FMT, a.H);
                    qb0 = a.gate.q + gq; sb0 = static_cast<const uint8_t *>(a.gate.s) + gs;
                    qb1 = a.up.q + gq;   sb1 = static_cast<const uint8_t *>(a.up.s) + gs;
                } else {
                    qb0 = a.sh_gate.q; sb0 = static_cast<const uint8_t *>(a.sh_gate.s);
                    qb1 = a.sh_up.q;   sb1 = static_cast<const uint8_t *>(a.sh_up.s);
                }
                abase = a.x_frag;
                nbase = a.x_step;
            } else {
                K = e >= 0 ? a.F : a.Fs;
                N = a.H;
                if (e >= 0) {
                    if constexpr (TAB) {
                        qb0 = a.tab[3 * e + 2].q; sb0 = static_cast<const uint8_t *>(a.tab[3 * e + 2].s);
                    } else {
                        const size_t dq = (size_t)e * a.H * fmt_code_bytes(FMT, a.F), ds = (size_t)e * a.H * fmt_scale_bytes(FMT, a.F);
                        qb0 = a.down.q + dq; sb0 = static_cast<const uint8_t *>(a.down.s) + ds;
                    }
                    abase = a.hr_frag;
                    nbase = a.hr_step;
                } else {
                    qb0 = a.sh_down.q; sb0 = static_cast<const uint8_t *>(a.sh_down.s);
                    abase = a.hs_frag;
                    nbase = a.hs_step;
                }
                qb1 = qb0;
                sb1 = sb0;
            }
            NG = K / 64;
            const int NGp = mfma_groups_padded(K);
            qlast = (uint32_t)(K / 2 - 16);
            const uint32_t rowq = (uint32_t)fmt_code_bytes(FMT, K), rows_ = FMT == kFmtF4 ? (uint32_t)(K / 32) : (uint32_t)NG;
            if constexpr (FMT == kFmtI3) {
                // code lane t % 8: the low plane of group 4c + t % 8 (16 B, lanes 0-3) or the
                // sign plane of group 4c + t % 8 - 4 (8 B, lanes 4-7); qlast: plane start
                qlast = (t % 8) < 4 ? 0u : (uint32_t)(K / 4);
            }
#pragma unroll
            for (int i = 0; i < 8; i++) {
                bool second;
                const int n = min(load_row_output<GU>(t / 8 + 32 * i, nb0, second), N - 1);
                qo[i] = (uint32_t)n * rowq;
            }
#pragma unroll
            for (int i = 0; i < 4; i++) {
                bool second;
                const int n = min(load_row_output<GU>(sc_col(i), nb0, second), N - 1);
                so[i] = (uint32_t)n * rows_;
            }
#pragma unroll
            for (int rb = 0; rb < kRowBlocks; rb++)
                arow[rb] = abase + (size_t)d.srow[16 * rb + t / 16] * NGp * kGroupBytes + 16 * (t % 16);
            two = IRB > 1 && __builtin_amdgcn_readfirstlane(d.R) > 16;
            no = (uint32_t)d.srow[t % IR] * (uint32_t)(NGp / kCG);  // (only lanes t < IR store it)
            pk = k;
        };
        auto load = [&](ChunkRegs<kActLoads> &v) __attribute__((always_inline)) {
            const int k = lk, c = lc;  // always a chunk that exists
            if (k != pk) rows_of(k);
            if constexpr (FMT == kFmtI3) {
                const int t8 = t % 8;
                const uint32_t g = (uint32_t)min(kCG * c + (t8 & 3), NG - 1);  // always a group of the row
                if (t8 < 4) {
                    // (two 8-byte loads: int3 rows are 3K/8 bytes long, so only 8-byte aligned)
#pragma unroll
                    for (int i = 0; i < 8; i++) {
                        const uint2 *src = reinterpret_cast<const uint2 *>(((i & 1) ? qb1 : qb0) + (qo[i] + 16 * g));
                        const uint2 w0 = src[0], w1 = src[1];
                        v.q[i] = u32x4_t{w0.x, w0.y, w1.x, w1.y};
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 8; i++) {
                        const uint2 w = *reinterpret_cast<const uint2 *>(((i & 1) ? qb1 : qb0) + (qo[i] + qlast + 8 * g));
                        v.q[i] = u32x4_t{w.x, w.y, 0u, 0u};
                    }
                }
            } else {
                const uint32_t off = min((uint32_t)(128 * c + 16 * (t % 8)), qlast);
#pragma unroll
                for (int i = 0; i < 8; i++) v.q[i] = *reinterpret_cast<const u32x4_t *>(((i & 1) ? qb1 : qb0) + (qo[i] + off));
            }
            const uint32_t sg = (uint32_t)min(kCG * c + t % 4, NG - 1);
            if constexpr (FMT == kFmtF4) {  // the group's two exponent bytes, as raw bits
#pragma unroll
                for (int i = 0; i < 4; i++)
                    v.s[i] = __uint_as_float((uint32_t) * reinterpret_cast<const uint16_t *>(((i & 1) ? sb1 : sb0) + so[i] + 2 * sg));
            } else {
#pragma unroll
                for (int i = 0; i < 4; i++)
                    v.s[i] = reinterpret_cast<const float *>((i & 1) ? sb1 : sb0)[so[i] + sg];
            }
            // the second row block's rows only if the item has them (else the registers
            // keep older values, which no compute wave reads)
#pragma unroll
            for (int i = 0; i < kActLoads; i++)
                if (i < kActPerRow || two)
                    v.a[i] = *reinterpret_cast<const uint4 *>(arow[i / kActPerRow] +
                                                              (uint32_t)(c * kChunkBytes + 256 * (i % kActPerRow)));
            if constexpr (FMT != kFmtF4) v.n = nbase[no + c];
            // advance; past the last chunk the head stays there (that chunk is loaded again)
            int nk = lk, nc = lc + 1;
            if (nc >= work[nk].nch) {
                nc = 0;
                nk++;
                while (nk < nwi && work[nk].nch == 0) nk++;
            }
            if (nk < nwi) {
                lk = nk;
                lc = nc;
            }
        };
        auto store = [&](const ChunkRegs<kActLoads> &v, int buf) __attribute__((always_inline)) {
            uint8_t *B = lds + (size_t)buf * kBufBytes;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int r = t / 8 + 32 * i;
                uint8_t *row = B + (r / 64) * 64 * kCodePitch + (r % 64) * kCodePitch;
                if constexpr (FMT == kFmtI3) {
                    // a row's chunk: low planes of its 4 groups (64 B), then their sign planes (32 B)
                    const int t8 = t % 8;
                    if (t8 < 4) *reinterpret_cast<u32x4_t *>(row + 16 * t8) = v.q[i];
                    else *reinterpret_cast<uint2 *>(row + 64 + 8 * (t8 - 4)) = make_uint2(v.q[i].x, v.q[i].y);
                } else {
                    *reinterpret_cast<u32x4_t *>(row + 16 * (t % 8)) = v.q[i];
                }
            }
            if constexpr (FMT == kFmtF4) {
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const uint32_t eb = __float_as_uint(v.s[i]);
                    *reinterpret_cast<float2 *>(reinterpret_cast<float *>(B + kBufCodes) + 8 * sc_col(i) + 2 * (t % 4)) =
                        make_float2(ue8m0_f32(eb & 0xFFu), ue8m0_f32(eb >> 8));
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; i++) reinterpret_cast<float *>(B + kBufCodes)[4 * sc_col(i) + t % 4] = v.s[i];
            }
#pragma unroll
            for (int i = 0; i < kActLoads; i++) {
                const int ar = 16 * (i / kActPerRow) + t / 16;
                *reinterpret_cast<uint4 *>(B + kBufCodes + kBufScales + ar * kRowPitch + 16 * (t % 16 + 16 * (i % kActPerRow))) = v.a[i];
            }
            if constexpr (FMT != kFmtF4)
                if (t < IR)  // a lane's four rows' steps are one read
                    reinterpret_cast<float *>(B + kBufCodes + kBufScales + kBufAct)[t] = v.n;
        };
        ChunkRegs<kActLoads> r0, r1;
#pragma unroll
        for (int i = 0; i < kActLoads; i++) r0.a[i] = r1.a[i] = make_uint4(0, 0, 0, 0);
        if (S > 0) {
            load(r0);
            load(r1);
            store(r0, 0);
        }
        lds_barrier();
        // chunk m sits in register set m % 2 and LDS buffer m % 2; at step s the set of
        // chunk s (already stored) takes chunk s + 2, and chunk s + 1 is stored
        int s = 0;
        for (; s + 2 <= S; s += 2) {
            load(r0); store(r1, 1); lds_barrier();
            load(r1); store(r0, 0); lds_barrier();
        }
        if (s < S) { load(r0); store(r1, 1); lds_barrier(); }
    } else {
        // ================= compute waves
        const int j = lane % 16, p = lane / 16;
        const int cs = wv / kCW, half = wv % kCW;
        // the 16-column block of the set that local block lb is
        auto gblk = [&](int lb) __attribute__((always_inline)) { return half + 2 * lb; };
        f32x4_t acc[kRowBlocks][NBL];  // [row block][local output block]
        int ck = 0, cc = 0;          // the chunk being computed
        while (ck < nwi && work[ck].nch == 0) ck++;
        // outputs of work item k
        auto epilogue = [&](int k) __attribute__((always_inline)) {
            const WorkDesc<IR> &d = work[k];
            const int e = d.e, R = d.R, row0 = d.row0;
            const int N = GU ? (e >= 0 ? a.F : a.Fs) : a.H;
            float *out = GU ? (e >= 0 ? a.h_routed : a.h_shared) : (e >= 0 ? a.y_routed : a.y_shared);
            out += (size_t)row0 * N;
            // D layout: register v of lane (j, p) is row 4p + v of the row block, column j
#pragma unroll
            for (int rb = 0; rb < kRowBlocks; rb++) {
                if (16 * rb >= R) break;
#pragma unroll
                for (int b = 0; b < (GU ? NBL / 2 : NBL); b++) {
                    // gate/up: local block b is a gate block, b + NBL/2 its up block
                    const int n = GU ? d.nb0 + 32 * cs + gblk(b) * 16 + j : d.nb0 + 64 * cs + 16 * gblk(b) + j;
                    if (n >= N) continue;
#pragma unroll
                    for (int v = 0; v < 4; v++) {
                        const int r = 16 * rb + 4 * p + v;
                        if (r >= R) continue;
                        float val;
                        if (GU) {
                            val = gate_up_out(a.gu_out, acc[rb][b][v], acc[rb][b + NBL / 2][v]);
                        } else {
                            val = acc[rb][b][v];
                        }
                        out[(size_t)r * N + n] = val;
                    }
                }
            }
        };
        // One chunk of RB row blocks: the chunk's group scales of this lane's four
        // columns and the steps of its rows; then the groups, with the next group's code
        // words and A fragments read before this group's products.  Per group: issue its
        // 8 RB MFMAs, then (while they run) read and convert the next group's operands,
        // then scale-accumulate this group's results.  Scheduling barriers keep that
        // order, so the conversion overlaps the matrix pipe.  The code conversion is
        // shared by the row blocks.
        auto run_chunk = [&](const uint8_t *B, int ng, auto rbc) __attribute__((always_inline)) {
            constexpr int RB = decltype(rbc)::value;
            const uint8_t *cw = B + cs * 64 * kCodePitch;
            const float *scl = reinterpret_cast<const float *>(B + kBufCodes);
            const uint8_t *tile = B + kBufCodes + kBufScales;
            const float *stp = reinterpret_cast<const float *>(B + kBufCodes + kBufScales + kBufAct);
            f32x4_t sc4[NBL], csum[RB][NBL], st4[RB];
#pragma unroll
            for (int b = 0; b < NBL; b++) sc4[b] = *reinterpret_cast<const f32x4_t *>(scl + 4 * (cs * 64 + 16 * gblk(b) + j));
#pragma unroll
            for (int rb = 0; rb < RB; rb++) {
                st4[rb] = *reinterpret_cast<const f32x4_t *>(stp + 16 * rb + 4 * p);
#pragma unroll
                for (int b = 0; b < NBL; b++) csum[rb][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
            struct Opnd {
                i32x4_t bo[NBL];    // [local block] 16 q bytes
                i32x4_t a[RB][2];   // [row block][hi, lo]
            };
            auto read_group = [&](int gi) __attribute__((always_inline)) {
                Opnd o;
                uint2 w[NBL];
#pragma unroll
                for (int b = 0; b < NBL; b++) {
                    const uint8_t *cr = cw + (16 * gblk(b) + j) * kCodePitch;
                    if constexpr (FMT == kFmtI3)  // low-plane word p, the sign word of p / 2
                        w[b] = make_uint2(*reinterpret_cast<const uint32_t *>(cr + 16 * gi + 4 * p),
                                          *reinterpret_cast<const uint32_t *>(cr + 64 + 8 * gi + 4 * (p / 2)) >> (4 * (p % 2)));
                    else
                        w[b] = *reinterpret_cast<const uint2 *>(cr + 32 * gi + 8 * p);
                }
#pragma unroll
                for (int rb = 0; rb < RB; rb++) {
                    const uint8_t *ar = tile + (16 * rb + j) * kRowPitch + gi * kGroupBytes + 16 * p;
                    if constexpr (!A8) o.a[rb][0] = *reinterpret_cast<const i32x4_t *>(ar);
                    o.a[rb][1] = *reinterpret_cast<const i32x4_t *>(ar + 64);
                }
#pragma unroll
                for (int b = 0; b < NBL; b++) {
                    if constexpr (FMT == kFmtI3) o.bo[b] = code_bytes_i3(w[b].x, w[b].y);
                    else o.bo[b] = code_bytes(w[b]);
                }
                return o;
            };
            const i32x4_t zero = {0, 0, 0, 0};
            Opnd cur = read_group(0);
#pragma unroll
            for (int gi = 0; gi < kCG; gi++) {
                if (gi >= ng) break;
                i32x4_t gh[RB][NBL], gl[RB][NBL];
#pragma unroll
                for (int rb = 0; rb < RB; rb++) {
                    if constexpr (!A8) {
#pragma unroll
                        for (int b = 0; b < NBL; b++)
                            gh[rb][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(cur.a[rb][0], cur.bo[b], zero, 0, 0, 0);
                    }
#pragma unroll
                    for (int b = 0; b < NBL; b++)
                        gl[rb][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(cur.a[rb][1], cur.bo[b], zero, 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                Opnd nxt;
                if (gi + 1 < kCG) nxt = read_group(min(gi + 1, ng - 1));
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int rb = 0; rb < RB; rb++)
#pragma unroll
                    for (int b = 0; b < NBL; b++)
#pragma unroll
                        for (int v = 0; v < 4; v++) {
                            if constexpr (A8)
                                csum[rb][b][v] = fmaf(sc4[b][gi], (float)gl[rb][b][v], csum[rb][b][v]);
                            else
                                csum[rb][b][v] = fmaf(sc4[b][gi], (float)(gh[rb][b][v] * 256 + gl[rb][b][v]), csum[rb][b][v]);
                        }
                if (gi + 1 < kCG) cur = nxt;
            }
            // the chunk's sums times the row steps (over 16: the codes entered as 16 q; int3:
            // over 32)
            constexpr float kUnit = FMT == kFmtI3 ? 0.03125f : 0.0625f;
#pragma unroll
            for (int rb = 0; rb < RB; rb++)
#pragma unroll
                for (int b = 0; b < NBL; b++)
#pragma unroll
                    for (int v = 0; v < 4; v++)
                        acc[rb][b][v] = fmaf(csum[rb][b][v], st4[rb][v] * kUnit, acc[rb][b][v]);
        };
        // MXFP4: per group and 32-element block, the B operands of this lane's columns (8
        // E2M1 codes times the block's power of two, as bf16) and the rows' hi and lo
        // bf16 terms; two bf16 products per block accumulate straight into acc.
        auto run_chunk_f4 = [&](const uint8_t *B, int ng, auto rbc) __attribute__((always_inline)) {
            constexpr int RB = decltype(rbc)::value;
            const uint8_t *cw = B + cs * 64 * kCodePitch;
            const float *scl = reinterpret_cast<const float *>(B + kBufCodes);
            const uint8_t *tile = B + kBufCodes + kBufScales;
#pragma unroll
            for (int gi = 0; gi < kCG; gi++) {
                if (gi >= ng) break;
#pragma unroll
                for (int blk = 0; blk < 2; blk++) {
                    bf16x8_t bo[NBL], ah[RB], al[RB];
#pragma unroll
                    for (int b = 0; b < NBL; b++) {
                        const int col = 16 * gblk(b) + j;
                        const uint32_t w = *reinterpret_cast<const uint32_t *>(cw + col * kCodePitch + 32 * gi + 16 * blk + 4 * p);
                        bo[b] = code_bf16_f4(w, scl[8 * (cs * 64 + col) + 2 * gi + blk]);
                    }
#pragma unroll
                    for (int rb = 0; rb < RB; rb++) {
                        const uint8_t *ar = tile + (16 * rb + j) * kRowPitch + gi * kGroupBytes + 64 * blk + 16 * p;
                        ah[rb] = *reinterpret_cast<const bf16x8_t *>(ar);
                        al[rb] = *reinterpret_cast<const bf16x8_t *>(ar + 128);
                    }
#pragma unroll
                    for (int rb = 0; rb < RB; rb++)
#pragma unroll
                        for (int b = 0; b < NBL; b++) {
                            acc[rb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[rb], bo[b], acc[rb][b], 0, 0, 0);
                            acc[rb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[rb], bo[b], acc[rb][b], 0, 0, 0);
                        }
                }
            }
        };
        lds_barrier();
        for (int s = 0; s < S; s++) {
            const uint8_t *B = lds + (size_t)(s & 1) * kBufBytes;
            const WorkDesc<IR> &d = work[ck];
            const int K = GU ? a.H : (d.e >= 0 ? a.F : a.Fs);
            const int NG = K / 64;
            const int ng = min(kCG, NG - kCG * cc);
            if (cc == 0) {
#pragma unroll
                for (int rb = 0; rb < kRowBlocks; rb++)
#pragma unroll
                    for (int b = 0; b < NBL; b++) acc[rb][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
            if constexpr (FMT == kFmtF4) {
                static_assert(IRB == 1, "MXFP4 items hold at most 16 rows");
                run_chunk_f4(B, ng, std::integral_constant<int, 1>());
            } else if constexpr (IRB == 2) {
                if (d.R > 16) run_chunk(B, ng, std::integral_constant<int, 2>());
                else run_chunk(B, ng, std::integral_constant<int, 1>());
            } else {
                run_chunk(B, ng, std::integral_constant<int, 1>());
            }
            if (++cc >= d.nch) {
                epilogue(ck);
                cc = 0;
                ck++;
                while (ck < nwi && work[ck].nch == 0) ck++;
            }
            lds_barrier();
        }
    }
}

static int mfma_cus() {
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

template <bool GU, int IRB, bool A8, bool TAB, int FMT>
static hipError_t launch_gemm_rb(const MfmaArgs &a, int shared_items, const char *name, hipStream_t st) {
    const int nmax = GU ? (a.with_shared ? (a.with_routed ? max(a.F, a.Fs) : a.Fs) : a.F) : a.H;
    const int nb = (nmax + (GU ? 127 : 255)) / (GU ? 128 : 256);
    const long total_max = (long)((a.with_routed ? a.max_items : 0) + shared_items) * nb;
    if (total_max == 0) return hipSuccess;
    // one workgroup per CU, more if a workgroup's table would overflow
    long G = mfma_cus();
    if ((total_max + G - 1) / G > kMaxWorkPerWg) G = (total_max + kMaxWorkPerWg - 1) / kMaxWorkPerWg;
    const size_t lds = 2 * (size_t)MfmaBuf<IRB, FMT>::kBytes + kMaxWorkPerWg * sizeof(WorkDesc<16 * IRB>);
    static_assert(2 * (size_t)MfmaBuf<IRB, FMT>::kBytes + kMaxWorkPerWg * sizeof(WorkDesc<16 * IRB>) <= 160 * 1024,
                  "the chunk buffers fit the CU's LDS");
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&q4_mfma_kernel<GU, IRB, A8, TAB, FMT>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    (void)hipGetLastError();
    ProfScope prof(name, st);
    q4_mfma_kernel<GU, IRB, A8, TAB, FMT><<<(int)G, kMfmaThreads, lds, st>>>(a);
    return hipGetLastError();
}

// the work items' row count (16 or 32) selects the kernel; MXFP4 items have at most 16
template <bool GU>
static hipError_t launch_gemm(const MfmaArgs &a, int shared_items, const char *name, hipStream_t st) {
#define MOE_GEMM_CASE(A8, TAB, FMT)                                                                       \
    if (!!a.act8 == A8 && (a.tab != nullptr) == TAB && a.fmt == FMT)                                      \
        return a.item_rows > 16 ? launch_gemm_rb<GU, 2, A8, TAB, FMT>(a, shared_items, name, st)          \
                                : launch_gemm_rb<GU, 1, A8, TAB, FMT>(a, shared_items, name, st);
    MOE_GEMM_CASE(false, false, kFmtI4)
    MOE_GEMM_CASE(true, false, kFmtI4)
    MOE_GEMM_CASE(false, true, kFmtI4)
    MOE_GEMM_CASE(true, true, kFmtI4)
    MOE_GEMM_CASE(false, false, kFmtI3)
    MOE_GEMM_CASE(true, false, kFmtI3)
    MOE_GEMM_CASE(false, true, kFmtI3)
    MOE_GEMM_CASE(true, true, kFmtI3)
#undef MOE_GEMM_CASE
    if (a.fmt == kFmtF4 && !a.act8 && a.item_rows <= 16)
        return a.tab ? launch_gemm_rb<GU, 1, false, true, kFmtF4>(a, shared_items, name, st)
                     : launch_gemm_rb<GU, 1, false, false, kFmtF4>(a, shared_items, name, st);
    return hipErrorInvalidValue;
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
    it.item_rows = a.item_rows;
    it.items = a.with_routed ? a.items : nullptr;
    it.n_items = a.n_items;
    it.with_union = a.union_in_prep;
    it.uni = a.uni;
    const int bf = a.fmt == kFmtF4;
    e = launch_prep(prep_job(a.x, a.T, a.H, a.x_frag, a.x_step, a.act8, bf), none, it, "prep_x+items", st);
    if (e != hipSuccess) return e;
    const int shared_items = a.with_shared ? (a.T + a.item_rows - 1) / a.item_rows : 0;
    if ((e = launch_gemm<true>(a, shared_items, "ffn_gateup_mfma", st)) != hipSuccess) return e;
    // h rows in fragment order: the routed rows (the grid covers the largest union, the
    // workgroups past the union's row count off[E] do nothing) and the shared rows
    ItemsJob no_items = it;
    no_items.items = nullptr;
    no_items.with_union = 0;
    e = launch_prep(a.with_routed ? prep_job(a.h_routed, a.max_rows, a.F, a.hr_frag, a.hr_step, a.act8, bf,
                                             a.off + a.E)
                                  : none,
                    a.with_shared ? prep_job(a.h_shared, a.T, a.Fs, a.hs_frag, a.hs_step, a.act8, bf) : none,
                    no_items, "prep_h", st);
    if (e != hipSuccess) return e;
    return launch_gemm<false>(a, shared_items, "ffn_down_mfma", st);
}

}  // namespace moe

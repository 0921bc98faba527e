// moe_internal.h -- shared declarations of the gfx950 MoE library (host + device).
//
// Only the library's own translation units include this file.  It holds the
// workspace plan, the kernel argument blocks and the device helpers used by
// more than one kernel file.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;

// What the gate/up step writes as h: SiLU(g) * u (the layer), or, for the test entry
// point moe_expert_ffn_probe, the gate or the up pre-activation.
constexpr int kGuSwiglu = MOE_GU_SWIGLU, kGuGate = MOE_GU_GATE, kGuUp = MOE_GU_UP;
__device__ __forceinline__ float gate_up_out(int mode, float g, float u) {
    return mode == kGuSwiglu ? g / (1.0f + expf(-g)) * u : (mode == kGuGate ? g : u);
}

// ---------------------------------------------------------------- expert formats
// The stored layout of one N x K matrix (moe.h): code bytes and scale bytes per row.
constexpr int kFmtI4 = MOE_FMT_INT4_G64, kFmtF4 = MOE_FMT_MXFP4, kFmtI3 = MOE_FMT_INT3_G64;
__host__ __device__ constexpr size_t fmt_code_bytes(int fmt, size_t K) {
    return fmt == kFmtI3 ? 3 * K / 8 : K / 2;
}
__host__ __device__ constexpr size_t fmt_scale_bytes(int fmt, size_t K) {
    return fmt == kFmtF4 ? K / 32 : 4 * (K / 64);
}
// matrix e of a stack of N x K matrices
__host__ __device__ inline moe_q4 fmt_stack_at(const moe_q4 &m, int fmt, int e, size_t N, size_t K) {
    moe_q4 r;
    r.q = m.q + (size_t)e * N * fmt_code_bytes(fmt, K);
    r.s = static_cast<const uint8_t *>(m.s) + (size_t)e * N * fmt_scale_bytes(fmt, K);
    return r;
}
// A UE8M0 exponent byte as the fp32 value 2^(e - 127): the bits e << 23, plus bit 22 for
// e = 0 (2^-127 is the subnormal 0x00400000) and for e = 255 (NaN 0x7FC00000 instead of
// infinity).  Integer operations only, no branch.
__device__ __forceinline__ float ue8m0_f32(uint32_t e) {
    const uint32_t edge = ((e + 1u) & 0xFFu) <= 1u ? 1u : 0u;  // e is 0 or 255
    return __uint_as_float((e << 23) | (edge << 22));
}

// ---------------------------------------------------------------- activation blocks
// Both expert-FFN paths take activations as fixed point per block: x16 = rint(x * 2^n)
// with n the largest integer for which max|x| * 2^n <= 32639 = 127 * 256 + 127 (so
// hi = (x16 + 128) >> 8 and lo = x16 - 256 hi are signed bytes), and step 2^-n; or, on
// the opt-in 8-bit path, the same with 127 as the limit (hi is then 0 and lo the code).
// A power-of-two step scales exactly: values with at most 15 (7) significant bits
// relative to the block's largest are represented exactly.  Subnormal maxima are first
// scaled by 2^64 (exactly); n is at most 149, so the step 2^-n stays representable.
// The activation rule as wave-uniform constants: the largest mantissa (bits) for which
// the larger shift applies, that shift, and the code limit (16-bit: 8,322,560, 14, 32639;
// 8-bit: 8,257,536, 6, 127), so one staging path serves both with no per-element select.
struct ActRule {
    uint32_t thr;
    int khi;
    float lim;
};
__host__ __device__ constexpr ActRule act_rule(int act8) {
    return ActRule{act8 ? 8257536u : 8322560u, act8 ? 6 : 14, act8 ? 127.0f : 32639.0f};
}
// n for the bit pattern mb of max|x| (finite, nonzero): 1.f * 2^khi <= limit iff the
// mantissa bits are at most thr
__device__ __forceinline__ int act_shift(uint32_t mb, const ActRule &r) {
    int bias = 0;
    if (mb < 0x00800000u) {
        mb = __float_as_uint(__uint_as_float(mb) * 18446744073709551616.0f);
        bias = 64;
    }
    const int ef = (int)(mb >> 23);
    const int k = (mb & 0x7FFFFFu) <= r.thr ? r.khi : r.khi - 1;
    return min(k + 127 - ef + bias, 149);
}

// ---------------------------------------------------------------- router tiling
// Router logits are a [T][E] x [E][H]^T product in fp64, tiled 64 tokens x 64
// experts per workgroup with a split over H so small batches still cover the chip.
constexpr int kRouterTile = 64;
constexpr int kRouterKC = 64;  // H elements staged per LDS step
constexpr int kRouterGemvTokens = 8;  // at most this many tokens: one workgroup per expert instead

struct RouterSplit {
    int S;       // number of H slices
    int kslice;  // H elements per slice (multiple of kRouterKC)
};
RouterSplit router_split(int T, int E, int H);

// ---------------------------------------------------------------- workspace plan
struct Plan {
    int T;
    RouterSplit rs;
    int max_units;   // routed units a launch must cover: min(E, T*k)
    size_t part;     // fp64 [S][T][E] router partial logits
    size_t sig, key; // fp64 / u64 [T][E] gates and choice keys (router of a few tokens), or 0
    size_t ids, w, keff;                           // routing, when the caller gives none
    size_t n_uniq, uniq, off, row_tok, pick_row;   // union, when the caller gives none
    size_t h_routed;  // fp32 [T*k][F]  SiLU(gate) * up per routed row
    size_t h_shared;  // fp32 [T][Fs]
    size_t y_routed;  // fp32 [T*k][H]  unweighted expert outputs per routed row
    size_t y_shared;  // fp32 [T][H]
    size_t xq;        // fp32 [T][H] x in 8-bit blocks (opt-in 8-bit path, T <= kGemvMaxTokens), or 0
    size_t x_frag, x_step, hr_frag, hr_step, hs_frag, hs_step;  // matrix-core path (T > kGemvMaxTokens)
    size_t items, n_items;  // matrix-core work list
    int max_items;
    size_t total;
};
Plan make_plan(const moe_layer &L, int T);

// ---------------------------------------------------------------- kernel arguments
struct LogitsArgs {
    const float *x;       // [T][H]
    const float *wr;      // [E][H]
    double *part;         // [S][T][E]
    // complete logits only (S = 1): the sigmoid gate and choice key of every (t, e),
    // or nullptr
    const float *bias;    // [E] or nullptr
    double *sig;          // [T][E]
    unsigned long long *key;  // [T][E]
    int T, E, H, kslice;
};

struct SelectArgs {
    const double *part;   // [S][T][E]
    const float *bias;    // [E] or nullptr
    const double *sig_in;  // [T][E] gates and choice keys from the router, or nullptr
    const unsigned long long *key_in;
    int32_t *ids;         // [T][k]
    float *w;             // [T][k]
    int32_t *keff;        // [T]
    int S, T, E, k;
    float top_p, routed_scale;
    int norm_topk;
    int n_group, topk_group;  // group-limited routing when n_group > 1
};

struct UnionArgs {
    const int32_t *ids, *keff;
    int32_t *n_uniq, *uniq, *off, *row_tok, *pick_row;
    int T, E, k;
};

// One "unit" of expert work: a routed expert of the union (unit < max_units),
// or the shared expert (unit == max_units, rows = all T tokens).
struct CombineArgs {
    const float *w;         // [T][k]
    const int32_t *keff;    // [T]
    const int32_t *pick_row;// [T][k]
    const float *y_routed;  // [rows][H]
    const float *y_shared;  // [T][H] or nullptr
    void *out;              // [T][H] fp32 or bf16
    int T, H, k, out_bf16;  // k == 0: no routed terms (a dense layer's output conversion)
};

struct FfnArgs {
    const float *x;                  // [T][H] tokens
    const int32_t *n_uniq, *uniq, *off, *row_tok;
    moe_q4 gate, up, down;           // routed, stacked
    moe_q4 sh_gate, sh_up, sh_down;  // shared
    float *h_routed;                 // [rows][F]
    float *h_shared;                 // [T][Fs]
    float *y_routed;                 // [rows][H]
    float *y_shared;                 // [T][H]
    int T, H, F, Fs, max_units;
    int with_routed, with_shared;
    int gu_out;  // what the gate/up step writes as h: kGuSwiglu, kGuGate or kGuUp
    // routed expert e's gate, up and down matrices: tab[3e], tab[3e+1], tab[3e+2] (the
    // residency tier's slots), or, when null, the stacked gate/up/down above
    const moe_q4 *tab;
    int act8;  // opt-in 8-bit activation blocks (moe_layer::act_bits == 8)
    int fmt;   // expert weight format (kFmt*)
    float *xq;     // T <= kGemvMaxTokens with act8: x in 8-bit blocks (workspace [T][H])
    int rows_max;  // routed rows the batch can have (T * k)
    // Selection and union inside the gate/up launch (one token): every routed
    // workgroup selects and builds the union in LDS from the router logits; the
    // first routed workgroup also writes them out through sel (ids, w, keff) and uni
    // (union arrays).
    int fuse_select;
    SelectArgs sel;
    UnionArgs uni;
    // Matrix-core path: the union (uni) built by the work-list workgroup of the first
    // preparation launch instead of a launch of its own (union_in_prep_fits).
    int union_in_prep;
};

// LDS words of the in-launch selection and union for T tokens of top-k over E experts.
__host__ __device__ inline size_t select_lds_words(int E, int T, int k) {
    const int W = (T + 31) / 32, W8 = (W + 7) / 8;
    return 4 * (size_t)T * k + T + 1 + E + (E + 1) + (size_t)E * W + (size_t)E * W8 + 2 * (size_t)E + 1;
}

// The matrix-core path (more than kGemvMaxTokens tokens): FfnArgs plus the
// activations prepared in MFMA fragment order (16-bit fixed point as hi and lo
// signed bytes, 128 bytes per row and 64-group) with one step per row and
// 4-group chunk.
constexpr int kGemvMaxTokens = 4;

struct MfmaArgs {
    const float *x;                  // [T][H]
    uint8_t *x_frag;                 // [T][NGp(H)][128]
    float *x_step;                   // [T][NGp(H) / 4]  power-of-two step per chunk
    const int32_t *n_uniq, *uniq, *off, *row_tok;
    int32_t *items;                  // [max_items][4]: expert, first row, rows, 0
    int32_t *n_items;
    moe_q4 gate, up, down;
    moe_q4 sh_gate, sh_up, sh_down;
    float *h_routed, *h_shared;      // [rows][F], [T][Fs]
    uint8_t *hr_frag, *hs_frag;      // h in fragment order
    float *hr_step, *hs_step;
    float *y_routed, *y_shared;      // [rows][H], [T][H]
    int T, H, F, Fs, E, max_units, max_rows, max_items;
    int item_rows;  // rows per work item: 16 or kMfmaItemRows
    int gu_out;     // as FfnArgs::gu_out
    const moe_q4 *tab;  // as FfnArgs::tab
    int act8;           // as FfnArgs::act8
    int fmt;            // as FfnArgs::fmt
    int with_routed, with_shared;
    int union_in_prep;  // build the union (uni) before the work list, in the same workgroup
    UnionArgs uni;
};

// Matrix-core work items: at most this many rows of one expert (two 16-row MFMA
// blocks; an item of at most 16 rows computes one).  Batches with few rows per expert
// cut items at 16 rows (mfma_item_rows).
constexpr int kMfmaItemRows = 32;
inline int mfma_item_rows(int rows, int E) { return rows >= 8 * E ? kMfmaItemRows : 16; }
// Fragment rows hold a whole number of 4-group K chunks.
__host__ __device__ inline int mfma_groups_padded(int K) { return (K / 64 + 3) / 4 * 4; }
// Upper bound of the work items of a batch: sum over experts of ceil(rows / 16).
inline int mfma_max_items(int max_units, int max_rows) {
    return max_units + (max_rows + 15) / 16;
}

hipError_t launch_ffn_mfma(const MfmaArgs &a, hipStream_t st);
// Whether the union of T tokens (top-k) is built by the work-list workgroup: few picks,
// and its LDS fits what that workgroup may take.
bool union_in_prep_fits(int E, int T, int k);


// moe_layer_forward in two parts: host-only argument checks (no HIP call) and, for a
// validated call with T > 0 and a large enough workspace on a checked device, the
// launch sequence.  device_ok: the lazy once-per-device gfx950 check.
int layer_forward_validate(const moe_layer *L, const float *x, int32_t T, const void *out,
                           int32_t out_dtype);
struct TierArgs;
int layer_forward_run(const moe_layer *L, const float *x, int32_t T, void *out, int32_t out_dtype,
                      const moe_route_out *dbg, void *ws, hipStream_t st, const TierArgs *tier);
int device_ok();

// ---------------------------------------------------------------- residency tier
// Byte layout of a tier slot (one expert) and of the tier state (see moe.h).
constexpr int kTierMaxSlots = 1024;
constexpr int kTierMaxPins = 256;

struct TierLayout {
    size_t gq, gs, uq, us, dq, ds, slot;                        // within a slot; slot bytes
    size_t hdr, slot_expert, slot_pinned, slot_used, expert_slot, heat, usage, copies, tab, total;
    int S, E, max_copies;
};

__host__ __device__ inline size_t tier_align(size_t v, size_t a) { return (v + a - 1) / a * a; }

__host__ __device__ inline TierLayout tier_layout(int H, int F, int E, int S, int fmt) {
    TierLayout t;
    size_t o = 0;
    // one matrix's codes and scales (gate/up [F][H] and down [H][F] take the same bytes)
    const size_t wq = (size_t)F * fmt_code_bytes(fmt, H), ws = (size_t)F * fmt_scale_bytes(fmt, H);
    t.gq = o; o = tier_align(o + wq, 256);
    t.gs = o; o = tier_align(o + ws, 256);
    t.uq = o; o = tier_align(o + wq, 256);
    t.us = o; o = tier_align(o + ws, 256);
    t.dq = o; o = tier_align(o + wq, 256);
    t.ds = o; o = tier_align(o + ws, 256);
    t.slot = o;
    t.S = S;
    t.E = E;
    t.max_copies = E < S ? E : S;
    if (t.max_copies < 4) t.max_copies = 4;  // a repin pass copies up to four experts
    o = 0;
    t.hdr = o; o += 16 * 4;
    t.slot_expert = o; o += (size_t)S * 4;
    t.slot_pinned = o; o += (size_t)S * 4;
    t.slot_used = o; o += (size_t)S * 4;
    t.expert_slot = o; o += (size_t)E * 4;
    t.heat = o; o += (size_t)E * 4;
    t.usage = o; o += (size_t)E * 4;
    t.copies = o; o += (size_t)2 * t.max_copies * 4;
    o = tier_align(o, 16);
    t.tab = o; o += (size_t)3 * E * sizeof(moe_q4);
    t.total = tier_align(o, 256);
    return t;
}

struct TierArgs {
    TierLayout lay;
    uint8_t *slots;
    uint8_t *state;
    moe_q4 gate, up, down;  // the host backing store, stacked by expert id
    int H, F, n_pinned;
    int fmt;                // expert weight format
};

struct TierPins {
    int32_t id[kTierMaxPins];
};

// Resolution of a forward's union (n_uniq/uniq/off) or, for a prefetch, of the distinct
// experts of predicted picks (ids/keff).
struct TierResolveIn {
    const int32_t *n_uniq, *uniq, *off;
    const int32_t *ids, *keff;
    int T, k, prefetch;
};

hipError_t launch_tier_init(const TierArgs &a, const TierPins &pins, int n_pin, hipStream_t st);
hipError_t launch_tier_resolve(const TierArgs &a, const TierResolveIn &in, hipStream_t st);
hipError_t launch_tier_repin(const TierArgs &a, int max_swaps, hipStream_t st);
// copies the state's copy list (at most max_jobs entries) from the backing store into slots
hipError_t launch_tier_copy(const TierArgs &a, int max_jobs, hipStream_t st);
int tier_jobs(const moe_layer &L, const TierArgs &t, int T);

// Bracketing HIP events around one kernel launch while moe_prof_begin() is active.
struct ProfScope {
    ProfScope(const char *name, hipStream_t st);
    ~ProfScope();
    int slot;
    hipStream_t st;
};

struct GlueArgs {
    const float *h, *delta;  // [T][H], delta may be null
    float *h_out, *x_out;    // [T][H]
    int T, H;
    float eps;
};

hipError_t launch_residual_rmsnorm(const GlueArgs &a, hipStream_t st);
hipError_t launch_router_logits(const LogitsArgs &a, int S, hipStream_t st);
hipError_t launch_route_select(const SelectArgs &a, hipStream_t st);
hipError_t launch_union(const UnionArgs &a, hipStream_t st);
// selection and union in one workgroup, for T <= kSelectUnionTokens
constexpr int kSelectUnionTokens = 16;
hipError_t launch_select_union(const SelectArgs &s, const UnionArgs &u, hipStream_t st);
hipError_t launch_ffn_gemv(const FfnArgs &a, hipStream_t st);
hipError_t launch_combine(const CombineArgs &a, hipStream_t st);

}  // namespace moe

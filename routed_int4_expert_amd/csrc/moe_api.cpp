// moe_api.cpp -- host side of the C ABI declared in include/moe.h: argument
// validation, the workspace plan and the launch sequence of the MoE layer
// forward ("MoE 路由与专家流式加载" §1: route, select, union, expert FFN, shared
// expert and combine).
//
// Validation is pure host code and runs before any HIP call, so every error
// path is reachable without a device.  The calls never synchronise and never
// copy device data to the host: the union size stays on the device and the
// expert kernels are launched for the largest possible union, their surplus
// workgroups returning at once.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "moe.h"
#include "moe_internal.h"

namespace moe {

static inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// -------------------------------------------------------------- validation
static int check_dims(const moe_layer *L) {
    if (!L) return MOE_EINVAL;
    if (L->hidden <= 0 || L->hidden % 64 || L->ffn <= 0 || L->ffn % 64) return MOE_EINVAL;
    if (L->shared_ffn < 0 || L->shared_ffn % 64) return MOE_EINVAL;
    if (L->n_experts <= 0 || L->top_k <= 0 || L->top_k > L->n_experts) return MOE_EINVAL;
    if (!(L->top_p >= 0.0f && L->top_p <= 1.0f)) return MOE_EINVAL;  // also rejects NaN
    if (!isfinite(L->routed_scale)) return MOE_EINVAL;
    if (L->n_experts > MOE_MAX_EXPERTS || L->top_k > MOE_MAX_TOPK) return MOE_EUNSUPPORTED;
    if (L->act_bits != 0 && L->act_bits != 16 && L->act_bits != 8) return MOE_EINVAL;
    if (L->expert_fmt != MOE_FMT_INT4_G64 && L->expert_fmt != MOE_FMT_MXFP4 && L->expert_fmt != MOE_FMT_INT3_G64)
        return MOE_EINVAL;
    if (L->expert_fmt == MOE_FMT_MXFP4 && L->act_bits == 8) return MOE_EUNSUPPORTED;
    if (L->n_group < 0) return MOE_EINVAL;
    if (L->n_group > 1) {
        if (L->n_group > 64 || L->n_experts % L->n_group || L->n_experts / L->n_group < 2) return MOE_EINVAL;
        if (L->topk_group < 1 || L->topk_group > L->n_group) return MOE_EINVAL;
        if ((long)L->topk_group * (L->n_experts / L->n_group) < L->top_k) return MOE_EINVAL;
    }
    if (L->hidden > MOE_MAX_DIM || L->ffn > MOE_MAX_DIM || L->shared_ffn > MOE_MAX_DIM)
        return MOE_EUNSUPPORTED;
    return MOE_OK;
}

static int check_q4(const moe_q4 &m) {
    if (!m.q || !m.s) return MOE_EINVAL;
    if (!aligned16(m.q) || !aligned16(m.s)) return MOE_EALIGN;
    return MOE_OK;
}

static int check_router(const moe_layer *L) {
    if (!L->router_w) return MOE_EINVAL;
    if (!aligned16(L->router_w)) return MOE_EALIGN;
    if (L->router_bias && ((uintptr_t)L->router_bias & 3u)) return MOE_EALIGN;
    return MOE_OK;
}

static int check_experts(const moe_layer *L, bool routed, bool shared) {
    int rc;
    if (routed) {
        if ((rc = check_q4(L->gate)) || (rc = check_q4(L->up)) || (rc = check_q4(L->down))) return rc;
    }
    if (shared && L->shared_ffn > 0) {
        if ((rc = check_q4(L->sh_gate)) || (rc = check_q4(L->sh_up)) || (rc = check_q4(L->sh_down)))
            return rc;
    }
    return MOE_OK;
}

static int check_T(int32_t T) {
    if (T < 0) return MOE_EINVAL;
    if (T > MOE_MAX_TOKENS) return MOE_EUNSUPPORTED;
    return MOE_OK;
}

static int check_ws(const moe_layer *L, int32_t T, const void *ws, size_t ws_bytes) {
    const size_t need = moe_workspace_bytes(L, T);
    if (need == 0) return MOE_EINVAL;
    if (!ws || ws_bytes < need) return MOE_EWORKSPACE;
    if (!aligned16(ws)) return MOE_EALIGN;
    return MOE_OK;
}

// gfx950 check, once per device (lazy; the only HIP query before launching)
static std::atomic<int> g_dev_ok[64];

static int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return MOE_EDEVICE;
    }
    if (dev < 64) {
        const int c = g_dev_ok[dev].load(std::memory_order_relaxed);
        if (c != 0) return c > 0 ? MOE_OK : MOE_EDEVICE;
    }
    hipDeviceProp_t prop;
    int ok = 0;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess) ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    else (void)hipGetLastError();
    if (dev < 64) g_dev_ok[dev].store(ok ? 1 : -1, std::memory_order_relaxed);
    return ok ? MOE_OK : MOE_EDEVICE;
}

static int launched(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EDEVICE; }

// -------------------------------------------------------------- workspace plan
static size_t router_part_bytes(const moe_layer &L, int T) {
    // largest S(T') * T' over T' <= T, so the plan grows monotonically with T
    size_t best = 0;
    for (int t = 1; t <= T; t++) {
        const RouterSplit rs = router_split(t, L.n_experts, L.hidden);
        const size_t b = (size_t)rs.S * t * L.n_experts * sizeof(double);
        if (b > best) best = b;
    }
    return best;
}

Plan make_plan(const moe_layer &L, int T) {
    Plan p;
    memset(&p, 0, sizeof(p));
    const size_t E = L.n_experts, k = L.top_k, H = L.hidden, F = L.ffn, Fs = L.shared_ffn;
    const size_t Tz = T > 0 ? (size_t)T : 1;
    p.T = T;
    p.rs = router_split((int)Tz, L.n_experts, L.hidden);
    p.max_units = (int)(Tz * k < E ? Tz * k : E);
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = align_up(o + bytes, 256);
        return at;
    };
    p.part = take(router_part_bytes(L, (int)Tz));
    if (Tz <= (size_t)kRouterGemvTokens) {  // the one-slice router also gives gates and keys
        p.sig = take(Tz * E * 8);
        p.key = take(Tz * E * 8);
    }
    p.ids = take(Tz * k * 4);
    p.w = take(Tz * k * 4);
    p.keff = take(Tz * 4);
    p.n_uniq = take(4);
    p.uniq = take(E * 4);
    p.off = take((E + 1) * 4);
    p.row_tok = take(Tz * k * 4);
    p.pick_row = take(Tz * k * 4);
    p.h_routed = take(Tz * k * F * 4);
    p.h_shared = take(Tz * Fs * 4);
    p.y_routed = take(Tz * k * H * 4);
    p.y_shared = take(Tz * H * 4);
    if (L.act_bits == 8 && Tz <= (size_t)kGemvMaxTokens) p.xq = take(Tz * H * 4);
    if (Tz > (size_t)kGemvMaxTokens) {
        // fragment rows padded to whole 4-group chunks
        const size_t gh = mfma_groups_padded((int)H), gf = mfma_groups_padded((int)F),
                     gs = Fs ? mfma_groups_padded((int)Fs) : 0;
        // (128 bytes per row and group, 256 for the MXFP4 path's bf16 terms; one fp32
        // step per row and 4-group chunk)
        const size_t gb = L.expert_fmt == MOE_FMT_MXFP4 ? 256 : 128;
        p.x_frag = take(Tz * gh * gb);
        p.x_step = take(Tz * gh);
        p.hr_frag = take(Tz * k * gf * gb);
        p.hr_step = take(Tz * k * gf);
        p.hs_frag = take(Tz * gs * gb);
        p.hs_step = take(Tz * gs);
        p.max_items = mfma_max_items(p.max_units, (int)(Tz * k));
        p.items = take((size_t)p.max_items * 16);
        p.n_items = take(4);
    }
    p.total = o;
    return p;
}

template <typename P>
static P *at(void *ws, size_t off) {
    return reinterpret_cast<P *>(reinterpret_cast<char *>(ws) + off);
}

// -------------------------------------------------------------- launch pieces
static SelectArgs select_args(const moe_layer &L, const Plan &p, int T, int32_t *ids, float *w,
                              int32_t *keff, void *ws) {
    SelectArgs sa;
    sa.part = at<double>(ws, p.part);
    sa.bias = L.router_bias;
    sa.sig_in = p.sig ? at<double>(ws, p.sig) : nullptr;
    sa.key_in = p.sig ? at<unsigned long long>(ws, p.key) : nullptr;
    sa.ids = ids;
    sa.w = w;
    sa.keff = keff;
    sa.S = p.rs.S;
    sa.T = T;
    sa.E = L.n_experts;
    sa.k = L.top_k;
    sa.top_p = L.top_p;
    sa.routed_scale = L.routed_scale;
    sa.norm_topk = L.norm_topk ? 1 : 0;
    sa.n_group = L.n_group > 1 ? L.n_group : 1;
    sa.topk_group = L.n_group > 1 ? L.topk_group : 1;
    return sa;
}

static UnionArgs union_args(const moe_layer &L, const int32_t *ids, const int32_t *keff, int T,
                            int32_t *n_uniq, int32_t *uniq, int32_t *off, int32_t *row_tok,
                            int32_t *pick_row) {
    UnionArgs ua;
    ua.ids = ids;
    ua.keff = keff;
    ua.n_uniq = n_uniq;
    ua.uniq = uniq;
    ua.off = off;
    ua.row_tok = row_tok;
    ua.pick_row = pick_row;
    ua.T = T;
    ua.E = L.n_experts;
    ua.k = L.top_k;
    return ua;
}

static hipError_t run_logits(const moe_layer &L, const Plan &p, const float *x, int T, void *ws,
                             hipStream_t st) {
    LogitsArgs la;
    la.x = x;
    la.wr = L.router_w;
    la.part = at<double>(ws, p.part);
    la.bias = L.router_bias;
    la.sig = p.sig ? at<double>(ws, p.sig) : nullptr;
    la.key = p.sig ? at<unsigned long long>(ws, p.key) : nullptr;
    la.T = T;
    la.E = L.n_experts;
    la.H = L.hidden;
    la.kslice = p.rs.kslice;
    return launch_router_logits(la, p.rs.S, st);
}

static hipError_t run_route(const moe_layer &L, const Plan &p, const float *x, int T, int32_t *ids,
                            float *w, int32_t *keff, void *ws, hipStream_t st) {
    hipError_t e = run_logits(L, p, x, T, ws, st);
    if (e != hipSuccess) return e;
    return launch_route_select(select_args(L, p, T, ids, w, keff, ws), st);
}

static hipError_t run_union(const moe_layer &L, const int32_t *ids, const int32_t *keff, int T,
                            int32_t *n_uniq, int32_t *uniq, int32_t *off, int32_t *row_tok,
                            int32_t *pick_row, hipStream_t st) {
    return launch_union(union_args(L, ids, keff, T, n_uniq, uniq, off, row_tok, pick_row), st);
}

static MfmaArgs mfma_args(const FfnArgs &f, const Plan &p, int E, int k, void *ws) {
    MfmaArgs m;
    m.gu_out = f.gu_out;
    m.tab = f.tab;
    m.act8 = f.act8;
    m.fmt = f.fmt;
    m.x = f.x;
    m.x_frag = at<uint8_t>(ws, p.x_frag);
    m.x_step = at<float>(ws, p.x_step);
    m.items = at<int32_t>(ws, p.items);
    m.n_items = at<int32_t>(ws, p.n_items);
    m.n_uniq = f.n_uniq;
    m.uniq = f.uniq;
    m.off = f.off;
    m.row_tok = f.row_tok;
    m.gate = f.gate;
    m.up = f.up;
    m.down = f.down;
    m.sh_gate = f.sh_gate;
    m.sh_up = f.sh_up;
    m.sh_down = f.sh_down;
    m.h_routed = f.h_routed;
    m.h_shared = f.h_shared;
    m.hr_frag = at<uint8_t>(ws, p.hr_frag);
    m.hs_frag = at<uint8_t>(ws, p.hs_frag);
    m.hr_step = at<float>(ws, p.hr_step);
    m.hs_step = at<float>(ws, p.hs_step);
    m.y_routed = f.y_routed;
    m.y_shared = f.y_shared;
    m.T = f.T;
    m.H = f.H;
    m.F = f.F;
    m.Fs = f.Fs;
    m.E = E;
    m.max_units = f.max_units;
    m.max_rows = f.T * k;
    // (MXFP4 items hold at most 16 rows: the bf16 activation tile of 32 would not fit the LDS)
    m.item_rows = f.fmt == kFmtF4 ? 16 : mfma_item_rows(m.max_rows, E);
    m.max_items = p.max_items;
    m.with_routed = f.with_routed;
    m.with_shared = f.with_shared;
    m.union_in_prep = f.union_in_prep;
    m.uni = f.uni;
    return m;
}

// grouped GEMVs for a handful of tokens, the matrix-core grouped GEMM above that
static hipError_t run_ffn(const FfnArgs &f, const Plan &p, int E, int k, void *ws,
                          hipStream_t st) {
    if (f.T <= kGemvMaxTokens) return launch_ffn_gemv(f, st);
    return launch_ffn_mfma(mfma_args(f, p, E, k, ws), st);
}

static FfnArgs ffn_args(const moe_layer &L, const Plan &p, const float *x, int T,
                        const int32_t *n_uniq, const int32_t *uniq, const int32_t *off,
                        const int32_t *row_tok, float *y_routed, void *ws,
                        int gu_out = kGuSwiglu) {
    FfnArgs a;
    a.gu_out = gu_out;
    a.tab = nullptr;
    a.act8 = L.act_bits == 8 ? 1 : 0;
    a.fmt = L.expert_fmt;
    a.xq = p.xq ? at<float>(ws, p.xq) : nullptr;
    a.rows_max = T * L.top_k;
    a.x = x;
    a.n_uniq = n_uniq;
    a.uniq = uniq;
    a.off = off;
    a.row_tok = row_tok;
    a.gate = L.gate;
    a.up = L.up;
    a.down = L.down;
    a.sh_gate = L.sh_gate;
    a.sh_up = L.sh_up;
    a.sh_down = L.sh_down;
    a.h_routed = at<float>(ws, p.h_routed);
    a.h_shared = at<float>(ws, p.h_shared);
    a.y_routed = y_routed;
    a.y_shared = at<float>(ws, p.y_shared);
    a.T = T;
    a.H = L.hidden;
    a.F = L.ffn;
    a.Fs = L.shared_ffn;
    a.max_units = p.max_units;
    a.with_routed = 1;
    a.with_shared = L.shared_ffn > 0 ? 1 : 0;
    a.fuse_select = 0;
    a.union_in_prep = 0;
    memset(&a.sel, 0, sizeof(a.sel));
    memset(&a.uni, 0, sizeof(a.uni));
    return a;
}


// ---------------------------------------------------------------- residency tier
static int check_tier(const moe_tier *t) {
    if (!t) return MOE_EINVAL;
    if (t->n_slots < 1 || t->n_pinned < 0 || t->n_pinned > t->n_slots) return MOE_EINVAL;
    if (t->n_slots > kTierMaxSlots || t->n_pinned > kTierMaxPins) return MOE_EUNSUPPORTED;
    if (!t->slots || !t->state) return MOE_EINVAL;
    if (((uintptr_t)t->slots & 255u) || ((uintptr_t)t->state & 255u)) return MOE_EALIGN;
    return MOE_OK;
}

static TierArgs tier_args(const moe_layer &L, const moe_tier &t) {
    TierArgs a;
    a.lay = tier_layout(L.hidden, L.ffn, L.n_experts, t.n_slots, L.expert_fmt);
    a.fmt = L.expert_fmt;
    a.slots = static_cast<uint8_t *>(t.slots);
    a.state = static_cast<uint8_t *>(t.state);
    a.gate = L.gate;
    a.up = L.up;
    a.down = L.down;
    a.H = L.hidden;
    a.F = L.ffn;
    a.n_pinned = t.n_pinned;
    return a;
}

// copies a resolution of T tokens can need: one per union expert, at most one per free slot
int tier_jobs(const moe_layer &L, const TierArgs &t, int T) {
    const long u = min((long)L.n_experts, (long)T * L.top_k);
    const long free_slots = (long)t.lay.S - t.n_pinned;
    return (int)min(u, free_slots);
}

// the unpinned slots hold a whole union of T tokens
static bool tier_fits(const moe_layer &L, const moe_tier &t, int T) {
    return (long)t.n_slots - t.n_pinned >= min((long)L.n_experts, (long)T * L.top_k);
}

// moe_layer_forward's host-only argument checks (no HIP call): MOE_OK or the error code.
int layer_forward_validate(const moe_layer *L, const float *x, int32_t T, const void *out,
                           int32_t out_dtype) {
    int rc;
    if ((rc = check_dims(L)) || (rc = check_T(T))) return rc;
    if (out_dtype != MOE_F32 && out_dtype != MOE_BF16) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if ((rc = check_router(L)) || (rc = check_experts(L, true, true))) return rc;
    if (!x || !out) return MOE_EINVAL;
    if (!aligned16(x) || ((uintptr_t)out & 7u)) return MOE_EALIGN;
    return MOE_OK;
}

int device_ok() { return check_device(); }

// The launch sequence of the layer on a validated call (T > 0, ws large enough for T).
int layer_forward_run(const moe_layer *L, const float *x, int32_t T, void *out, int32_t out_dtype,
                      const moe_route_out *dbg, void *ws, hipStream_t st, const TierArgs *tier) {
    const Plan p = make_plan(*L, T);
    moe_route_out d;
    memset(&d, 0, sizeof(d));
    if (dbg) d = *dbg;
    int32_t *ids = d.ids ? d.ids : at<int32_t>(ws, p.ids);
    float *w = d.w ? d.w : at<float>(ws, p.w);
    int32_t *keff = d.keff ? d.keff : at<int32_t>(ws, p.keff);
    int32_t *n_uniq = d.n_uniq ? d.n_uniq : at<int32_t>(ws, p.n_uniq);
    int32_t *uniq = d.uniq ? d.uniq : at<int32_t>(ws, p.uniq);
    int32_t *off = d.off ? d.off : at<int32_t>(ws, p.off);
    int32_t *row_tok = d.row_tok ? d.row_tok : at<int32_t>(ws, p.row_tok);
    int32_t *pick_row = d.pick_row ? d.pick_row : at<int32_t>(ws, p.pick_row);

    hipError_t e;
    // one token: selection and union run inside the gate/up launch (not with a residency
    // tier, which resolves the union before the expert FFNs start, nor with group-limited
    // routing, which the in-launch selection leaves to the selection kernels)
    const bool sel_in_ffn = T == 1 && !tier && L->n_group <= 1;
    float *y_routed = at<float>(ws, p.y_routed);
    FfnArgs a = ffn_args(*L, p, x, T, n_uniq, uniq, off, row_tok, y_routed, ws);
    if (sel_in_ffn) {
        e = run_logits(*L, p, x, T, ws, st);
    } else if (T <= kSelectUnionTokens && T <= kRouterGemvTokens) {
        // small batch: selection and union in one workgroup, from the gates and keys the
        // one-slice router wrote (with a sliced router, one workgroup summing every
        // token's partial logits would take longer than per-token selection workgroups)
        e = run_logits(*L, p, x, T, ws, st);
        if (e == hipSuccess)
            e = launch_select_union(select_args(*L, p, T, ids, w, keff, ws),
                                    union_args(*L, ids, keff, T, n_uniq, uniq, off, row_tok, pick_row), st);
    } else {
        e = run_route(*L, p, x, T, ids, w, keff, ws, st);
        // the union inside the first matrix-core preparation launch when it fits there
        if (!tier && union_in_prep_fits(L->n_experts, T, L->top_k)) {
            a.union_in_prep = 1;
            a.uni = union_args(*L, ids, keff, T, n_uniq, uniq, off, row_tok, pick_row);
        } else if (e == hipSuccess) {
            e = run_union(*L, ids, keff, T, n_uniq, uniq, off, row_tok, pick_row, st);
        }
    }
    CombineArgs c;
    c.w = w;
    c.keff = keff;
    c.pick_row = pick_row;
    c.y_routed = y_routed;
    c.y_shared = L->shared_ffn > 0 ? at<float>(ws, p.y_shared) : nullptr;
    c.out = out;
    c.T = T;
    c.H = L->hidden;
    c.k = L->top_k;
    c.out_bf16 = out_dtype == MOE_BF16;
    if (e == hipSuccess && tier) {
        // residency tier: every union expert resident (copies from the backing store for
        // the misses); the expert FFNs read them through the tier's table
        TierResolveIn in;
        memset(&in, 0, sizeof(in));
        in.n_uniq = n_uniq;
        in.uniq = uniq;
        in.off = off;
        e = launch_tier_resolve(*tier, in, st);
        if (e == hipSuccess) e = launch_tier_copy(*tier, tier_jobs(*L, *tier, T), st);
        a.tab = reinterpret_cast<const moe_q4 *>(tier->state + tier->lay.tab);
    }
    if (e == hipSuccess) {
        if (sel_in_ffn) {
            a.fuse_select = 1;
            a.sel = select_args(*L, p, T, ids, w, keff, ws);
            a.uni = union_args(*L, ids, keff, T, n_uniq, uniq, off, row_tok, pick_row);
        }
        e = run_ffn(a, p, L->n_experts, L->top_k, ws, st);
    }
    if (e == hipSuccess) e = launch_combine(c, st);
    return launched(e);
}



// ---------------------------------------------------------------- first-dense layers
// A dense layer runs the expert-FFN kernels with no routed unit and the MLP as the
// always-on unit for every token (the shared-expert role).  Its plan holds that unit's
// buffers only: h [T][F], y [T][H] (bf16 output: the fp32 rows before conversion; fp32
// output goes straight to out) and, above the GEMV range, the activation fragments.
static int check_dense(const moe_dense *D) {
    if (!D) return MOE_EINVAL;
    if (D->hidden <= 0 || D->hidden % 64 || D->ffn <= 0 || D->ffn % 64) return MOE_EINVAL;
    if (D->hidden > MOE_MAX_DIM || D->ffn > MOE_MAX_DIM) return MOE_EUNSUPPORTED;
    return MOE_OK;
}

static moe_layer dense_as_layer(const moe_dense &D) {
    moe_layer L;
    memset(&L, 0, sizeof(L));
    L.hidden = D.hidden;
    L.n_experts = 1;
    L.ffn = 64;
    L.shared_ffn = D.ffn;
    L.top_k = 1;
    L.routed_scale = 1.0f;
    L.sh_gate = D.gate;
    L.sh_up = D.up;
    L.sh_down = D.down;
    return L;
}

struct DensePlan {
    size_t h, y, x_frag, x_step, hs_frag, hs_step, total;
};

static DensePlan make_dense_plan(const moe_dense &D, int T) {
    DensePlan p;
    memset(&p, 0, sizeof(p));
    const size_t Tz = T > 0 ? (size_t)T : 1, H = D.hidden, F = D.ffn;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = align_up(o + bytes, 256);
        return at;
    };
    p.h = take(Tz * F * 4);
    p.y = take(Tz * H * 4);
    if (Tz > (size_t)kGemvMaxTokens) {
        const size_t gh = mfma_groups_padded((int)H), gf = mfma_groups_padded((int)F);
        p.x_frag = take(Tz * gh * 128);
        p.x_step = take(Tz * gh);
        p.hs_frag = take(Tz * gf * 128);
        p.hs_step = take(Tz * gf);
    }
    p.total = o;
    return p;
}

}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_workspace_bytes(const moe_layer *L, int32_t max_tokens) {
    if (check_dims(L) != MOE_OK || max_tokens < 0 || max_tokens > MOE_MAX_TOKENS) return 0;
    return make_plan(*L, max_tokens).total;
}

int moe_route(const moe_layer *L, const float *x, int32_t T, int32_t *ids, float *w,
              int32_t *keff, void *ws, size_t ws_bytes, void *stream) {
    int rc;
    if ((rc = check_dims(L)) || (rc = check_T(T))) return rc;
    if (T == 0) return MOE_OK;
    if ((rc = check_router(L))) return rc;
    if (!x || !ids || !w || !keff) return MOE_EINVAL;
    if (!aligned16(x)) return MOE_EALIGN;
    if ((rc = check_ws(L, T, ws, ws_bytes))) return rc;
    if ((rc = check_device())) return rc;
    const Plan p = make_plan(*L, T);
    return launched(run_route(*L, p, x, T, ids, w, keff, ws, (hipStream_t)stream));
}

int moe_union(const moe_layer *L, const int32_t *ids, const int32_t *keff, int32_t T,
              int32_t *n_uniq, int32_t *uniq, int32_t *off, int32_t *row_tok, int32_t *pick_row,
              void *ws, size_t ws_bytes, void *stream) {
    int rc;
    if ((rc = check_dims(L)) || (rc = check_T(T))) return rc;
    if (T == 0) return MOE_OK;
    if (!ids || !keff || !n_uniq || !uniq || !off || !row_tok || !pick_row) return MOE_EINVAL;
    if ((rc = check_ws(L, T, ws, ws_bytes))) return rc;
    if ((rc = check_device())) return rc;
    return launched(run_union(*L, ids, keff, T, n_uniq, uniq, off, row_tok, pick_row,
                              (hipStream_t)stream));
}

static int expert_ffn_call(const moe_layer *L, const float *x, int32_t T, const int32_t *n_uniq,
                           const int32_t *uniq, const int32_t *off, const int32_t *row_tok,
                           int gu_out, float *y_rows, void *ws, size_t ws_bytes, void *stream) {
    int rc;
    if ((rc = check_dims(L)) || (rc = check_T(T))) return rc;
    if (gu_out != kGuSwiglu && gu_out != kGuGate && gu_out != kGuUp) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if ((rc = check_experts(L, true, false))) return rc;
    if (!x || !n_uniq || !uniq || !off || !row_tok || !y_rows) return MOE_EINVAL;
    if (!aligned16(x) || !aligned16(y_rows)) return MOE_EALIGN;
    if ((rc = check_ws(L, T, ws, ws_bytes))) return rc;
    if ((rc = check_device())) return rc;
    const Plan p = make_plan(*L, T);
    FfnArgs a = ffn_args(*L, p, x, T, n_uniq, uniq, off, row_tok, y_rows, ws, gu_out);
    a.with_shared = 0;
    return launched(run_ffn(a, p, L->n_experts, L->top_k, ws, (hipStream_t)stream));
}

int moe_expert_ffn(const moe_layer *L, const float *x, int32_t T, const int32_t *n_uniq,
                   const int32_t *uniq, const int32_t *off, const int32_t *row_tok, float *y_rows,
                   void *ws, size_t ws_bytes, void *stream) {
    return expert_ffn_call(L, x, T, n_uniq, uniq, off, row_tok, kGuSwiglu, y_rows, ws, ws_bytes,
                           stream);
}

int moe_expert_ffn_probe(const moe_layer *L, const float *x, int32_t T, const int32_t *n_uniq,
                         const int32_t *uniq, const int32_t *off, const int32_t *row_tok,
                         int32_t gate_up_output, float *y_rows, void *ws, size_t ws_bytes,
                         void *stream) {
    return expert_ffn_call(L, x, T, n_uniq, uniq, off, row_tok, gate_up_output, y_rows, ws,
                           ws_bytes, stream);
}

int moe_layer_forward(const moe_layer *L, const float *x, int32_t T, void *out, int32_t out_dtype,
                      const moe_route_out *dbg, void *ws, size_t ws_bytes, void *stream) {
    int rc;
    if ((rc = layer_forward_validate(L, x, T, out, out_dtype))) return rc;
    if (T == 0) return MOE_OK;
    if ((rc = check_ws(L, T, ws, ws_bytes))) return rc;
    if ((rc = check_device())) return rc;
    return layer_forward_run(L, x, T, out, out_dtype, dbg, ws, (hipStream_t)stream, nullptr);
}

size_t moe_tier_slot_bytes(const moe_layer *L) {
    if (check_dims(L) != MOE_OK) return 0;
    return tier_layout(L->hidden, L->ffn, L->n_experts, 1, L->expert_fmt).slot;
}

size_t moe_tier_state_bytes(const moe_layer *L, int32_t n_slots) {
    if (check_dims(L) != MOE_OK || n_slots < 1 || n_slots > kTierMaxSlots) return 0;
    return tier_layout(L->hidden, L->ffn, L->n_experts, n_slots, L->expert_fmt).total;
}

int moe_tier_init(const moe_layer *L, const moe_tier *tier, const int32_t *pins, int32_t n_pin,
                  void *stream) {
    int rc;
    if ((rc = check_dims(L)) || (rc = check_tier(tier))) return rc;
    if (n_pin != tier->n_pinned || (n_pin > 0 && !pins)) return MOE_EINVAL;
    TierPins tp;
    memset(&tp, 0, sizeof(tp));
    unsigned char seen[MOE_MAX_EXPERTS];
    memset(seen, 0, sizeof(seen));
    for (int i = 0; i < n_pin; i++) {
        if (pins[i] < 0 || pins[i] >= L->n_experts || seen[pins[i]]) return MOE_EINVAL;
        seen[pins[i]] = 1;
        tp.id[i] = pins[i];
    }
    if ((rc = check_experts(L, true, false))) return rc;
    if ((rc = check_device())) return rc;
    const TierArgs a = tier_args(*L, *tier);
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = launch_tier_init(a, tp, n_pin, st);
    if (e == hipSuccess) e = launch_tier_copy(a, n_pin, st);
    return launched(e);
}

int moe_tier_layer_forward(const moe_layer *L, const moe_tier *tier, const float *x, int32_t T,
                           void *out, int32_t out_dtype, const moe_route_out *dbg, void *ws,
                           size_t ws_bytes, void *stream) {
    int rc;
    if ((rc = layer_forward_validate(L, x, T, out, out_dtype))) return rc;
    if ((rc = check_tier(tier))) return rc;
    if (T == 0) return MOE_OK;
    if (!tier_fits(*L, *tier, T)) return MOE_EUNSUPPORTED;
    if ((rc = check_ws(L, T, ws, ws_bytes))) return rc;
    if ((rc = check_device())) return rc;
    const TierArgs a = tier_args(*L, *tier);
    return layer_forward_run(L, x, T, out, out_dtype, dbg, ws, (hipStream_t)stream, &a);
}

int moe_tier_prefetch(const moe_layer *L, const moe_tier *tier, const int32_t *ids,
                      const int32_t *keff, int32_t T, void *stream) {
    int rc;
    if ((rc = check_dims(L)) || (rc = check_T(T)) || (rc = check_tier(tier))) return rc;
    if (T == 0) return MOE_OK;
    if (!ids || !keff) return MOE_EINVAL;
    if (!tier_fits(*L, *tier, T)) return MOE_EUNSUPPORTED;
    if ((rc = check_experts(L, true, false))) return rc;
    if ((rc = check_device())) return rc;
    const TierArgs a = tier_args(*L, *tier);
    TierResolveIn in;
    memset(&in, 0, sizeof(in));
    in.ids = ids;
    in.keff = keff;
    in.T = T;
    in.k = L->top_k;
    in.prefetch = 1;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = launch_tier_resolve(a, in, st);
    if (e == hipSuccess) e = launch_tier_copy(a, tier_jobs(*L, a, T), st);
    return launched(e);
}

int moe_tier_repin(const moe_layer *L, const moe_tier *tier, int32_t max_swaps, void *stream) {
    int rc;
    if ((rc = check_dims(L)) || (rc = check_tier(tier))) return rc;
    if (max_swaps < 1 || max_swaps > 4) return MOE_EINVAL;
    if ((rc = check_experts(L, true, false))) return rc;
    if ((rc = check_device())) return rc;
    const TierArgs a = tier_args(*L, *tier);
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = launch_tier_repin(a, max_swaps, st);
    if (e == hipSuccess) e = launch_tier_copy(a, max_swaps, st);
    return launched(e);
}

size_t moe_dense_workspace_bytes(const moe_dense *D, int32_t max_tokens) {
    if (check_dense(D) != MOE_OK || max_tokens < 0 || max_tokens > MOE_MAX_TOKENS) return 0;
    return make_dense_plan(*D, max_tokens).total;
}

int moe_dense_forward(const moe_dense *D, const float *x, int32_t T, void *out, int32_t out_dtype,
                      void *ws, size_t ws_bytes, void *stream) {
    int rc;
    if ((rc = check_dense(D)) || (rc = check_T(T))) return rc;
    if (out_dtype != MOE_F32 && out_dtype != MOE_BF16) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if ((rc = check_q4(D->gate)) || (rc = check_q4(D->up)) || (rc = check_q4(D->down))) return rc;
    if (!x || !out) return MOE_EINVAL;
    if (!aligned16(x) || ((uintptr_t)out & 7u)) return MOE_EALIGN;
    if (out_dtype == MOE_F32 && !aligned16(out)) return MOE_EALIGN;
    const size_t need = moe_dense_workspace_bytes(D, T);
    if (!ws || ws_bytes < need) return MOE_EWORKSPACE;
    if (!aligned16(ws)) return MOE_EALIGN;
    if ((rc = check_device())) return rc;
    hipStream_t st = (hipStream_t)stream;
    const DensePlan p = make_dense_plan(*D, T);
    const moe_layer L = dense_as_layer(*D);
    FfnArgs a;
    memset(&a, 0, sizeof(a));
    a.gu_out = kGuSwiglu;
    a.x = x;
    a.sh_gate = D->gate;
    a.sh_up = D->up;
    a.sh_down = D->down;
    a.h_shared = at<float>(ws, p.h);
    // fp32 output: the down projection writes out directly
    a.y_shared = out_dtype == MOE_F32 ? static_cast<float *>(out) : at<float>(ws, p.y);
    a.T = T;
    a.H = D->hidden;
    a.F = L.ffn;
    a.Fs = D->ffn;
    a.max_units = 0;
    a.with_routed = 0;
    a.with_shared = 1;
    hipError_t e;
    if (T <= kGemvMaxTokens) {
        e = launch_ffn_gemv(a, st);
    } else {
        MfmaArgs m;
        memset(&m, 0, sizeof(m));
        m.gu_out = kGuSwiglu;
        m.x = x;
        m.x_frag = at<uint8_t>(ws, p.x_frag);
        m.x_step = at<float>(ws, p.x_step);
        m.sh_gate = D->gate;
        m.sh_up = D->up;
        m.sh_down = D->down;
        m.h_shared = a.h_shared;
        m.hs_frag = at<uint8_t>(ws, p.hs_frag);
        m.hs_step = at<float>(ws, p.hs_step);
        m.y_shared = a.y_shared;
        m.T = T;
        m.H = D->hidden;
        m.F = L.ffn;
        m.Fs = D->ffn;
        m.E = 1;
        m.max_units = 0;
        m.max_rows = 0;
        m.item_rows = mfma_item_rows(T, 1);
        m.max_items = 0;
        m.with_routed = 0;
        m.with_shared = 1;
        e = launch_ffn_mfma(m, st);
    }
    if (e == hipSuccess && out_dtype == MOE_BF16) {
        CombineArgs c;
        memset(&c, 0, sizeof(c));
        c.y_shared = a.y_shared;
        c.out = out;
        c.T = T;
        c.H = D->hidden;
        c.k = 0;
        c.out_bf16 = 1;
        e = launch_combine(c, st);
    }
    return launched(e);
}

int moe_residual_rmsnorm(const float *h, const float *delta, int32_t T, int32_t H, float eps,
                         float *h_out, float *x_out, void *stream) {
    if (T < 0 || H <= 0 || H % 64 || !isfinite(eps) || eps < 0.0f) return MOE_EINVAL;
    if (H > MOE_MAX_DIM) return MOE_EUNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!h || !h_out || !x_out) return MOE_EINVAL;
    if (x_out == h || (delta && x_out == delta)) return MOE_EINVAL;
    if (!aligned16(h) || !aligned16(h_out) || !aligned16(x_out) || (delta && !aligned16(delta)))
        return MOE_EALIGN;
    int rc;
    if ((rc = check_device())) return rc;
    GlueArgs a;
    a.h = h;
    a.delta = delta;
    a.h_out = h_out;
    a.x_out = x_out;
    a.T = T;
    a.H = H;
    a.eps = eps;
    return launched(launch_residual_rmsnorm(a, (hipStream_t)stream));
}

const char *moe_strerror(int code) {
    switch (code) {
        case MOE_OK: return "ok";
        case MOE_EINVAL: return "invalid argument (NULL pointer, size or hyper-parameter)";
        case MOE_EUNSUPPORTED: return "shape outside the compiled limits";
        case MOE_EWORKSPACE: return "workspace missing or smaller than moe_workspace_bytes()";
        case MOE_EALIGN: return "pointer not 16-byte aligned";
        case MOE_EDEVICE: return "no gfx950 device current, or a kernel launch failed";
        default: return "unknown error code";
    }
}

}  // extern "C"

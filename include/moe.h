/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse MoE layer forward.
 *
 * The layer is the colibrì moe() forward as described in
 *   [R] "MoE 路由与专家流式加载" (colibri-analysis 07, blog.chen3feng.top), §1.1-§1.4,
 * with weights in the int4-gs64 container of
 *   [Q] "colibrì 深度拆解：1300行纯C代码驱动7440亿参数大模型" (chenxutan.com), §5.2 (packing), and
 *   [C] "colibri 开发演进实录：从 CHANGELOG 看多引擎 MoE 推理框架的工程迭代脉络", §2.1 (gs64).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *   never allocates, frees or keeps a pointer past the call.  Scratch memory is
 *   the caller's workspace `ws` of at least moe_workspace_bytes(L, T) bytes,
 *   16-byte aligned; its contents on entry are ignored and on exit undefined.
 * - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *   enqueues work on that stream and returns: no synchronisation, no
 *   device-to-host copy.  Results are ready when the stream reaches them.
 * - Every call returns MOE_OK (0) or a negative MOE_E* code.  Arguments are
 *   validated on the host before anything is enqueued; on failure nothing is
 *   launched and no output is touched.  T == 0 is a successful no-op.
 * - Results are bitwise deterministic for identical inputs (no floating-point
 *   atomics on the data path).  Calls may come from several host threads; calls
 *   that share a workspace must be ordered by the caller (same stream).
 * - Layouts are row-major; a weight matrix W[N][K] is used as y = W x with K
 *   contiguous.
 *
 * int4-gs64 matrix W[N][K] ([Q] §5.2, [C] §2.1):
 *   q : uint8 [N][K/2]  -- element 2j in the low nibble of byte j, 2j+1 in the high
 *                          nibble, each a two's-complement int4 in [-8, 7];
 *   s : fp32  [N][K/64] -- one scale per 64 consecutive elements of a row;
 *   W[n][k] = q(n,k) * s[n][k/64].
 * Routed expert tensors are stacked by expert id: gate/up q [E][F][H/2], s [E][F][H/64];
 * down q [E][H][F/2], s [E][H][F/64].
 *
 * Other expert formats (moe_layer.expert_fmt, one format for the routed and the shared
 * experts), a matrix W[N][K] with K a multiple of 64:
 * MOE_FMT_MXFP4 -- fp4 experts with UE8M0 block scales ([C] §五; the MXFP4 experts of
 *   [C] §六), read as the OCP Microscaling FP4 element: E2M1 codes (bit 3 sign, bits 2-1
 *   exponent with bias 1, bit 0 mantissa: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6)
 *   packed two per byte like int4 (element 2j in the low nibble of byte j),
 *   q : uint8 [N][K/2];  s : uint8 [N][K/32], one UE8M0 exponent per 32 consecutive
 *   elements;  W[n][k] = e2m1(q(n,k)) * 2^(s[n][k/32] - 127), an exponent byte of 255
 *   being NaN.
 * MOE_FMT_INT3_G64 -- int3-g64 ([C] §8.3, fmt=5: 3-bit weights, one scale per 64): codes
 *   c in [-4, 3], W[n][k] = c * s[n][k/64], s : fp32 [N][K/64];  q : uint8 [N][3K/8], per
 *   row two bit planes: bytes [0, K/4) hold the codes' low two bits, bytes [K/4, 3K/8)
 *   their sign bits (c = low - 4 sign).  Element i = 16d + 8a + 2b + o (d < 4, a < 2,
 *   b < 4, o < 2) of 64-group G has its low bits at bits 2(2a+o) and 2(2a+o)+1 of byte
 *   16G + 4d + b; written i = 32h + 8m + 2b + o (h < 2, m < 4), its sign bit is bit
 *   2m+o of byte K/4 + 8G + 4h + b.  (The pages fix no bit layout.  This one lets a
 *   32-bit word of either plane give four codes of the same parity by one shift and
 *   mask, in the element order the int4 path uses.)
 * Stacked routed tensors hold E such matrices back to back (q: E*F or E*H rows of the
 * format's row bytes; s likewise).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,       /* NULL pointer, bad size or hyper-parameter */
    MOE_EUNSUPPORTED = -2, /* shape outside the compiled limits below */
    MOE_EWORKSPACE = -3,   /* workspace missing or smaller than moe_workspace_bytes */
    MOE_EALIGN = -4,       /* a pointer that must be 16-byte aligned is not */
    MOE_EDEVICE = -5       /* no gfx950 device current, or a launch failed */
};

enum { MOE_F32 = 0, MOE_BF16 = 1 };        /* output element type of moe_layer_forward */

/* Compiled limits (MOE_EUNSUPPORTED beyond them). */
#define MOE_MAX_EXPERTS 256
#define MOE_MAX_TOPK 16
#define MOE_MAX_TOKENS 4096
#define MOE_MAX_DIM 16384                  /* hidden, ffn, shared_ffn */

enum { MOE_FMT_INT4_G64 = 0, MOE_FMT_MXFP4 = 1, MOE_FMT_INT3_G64 = 2 };  /* moe_layer.expert_fmt */

/* One quantised matrix: codes and scales in the layer's expert format (int4-gs64:
 * q [N][K/2], s fp32 [N][K/64]; the other formats as described above). */
typedef struct {
    const uint8_t *q;
    const void *s;
} moe_q4;

typedef struct {
    int32_t hidden;         /* H, multiple of 64 */
    int32_t n_experts;      /* E, 1..MOE_MAX_EXPERTS */
    int32_t ffn;            /* F, routed expert width, multiple of 64 */
    int32_t shared_ffn;     /* Fs, shared expert width, multiple of 64; 0 = no shared expert */
    int32_t top_k;          /* k, 1..min(E, MOE_MAX_TOPK) */
    float top_p;            /* adaptive top-p: 0 = off, else (0, 1]; 1 keeps all k */
    int32_t norm_topk;      /* 1: kept gates renormalised to sum 1 before scaling */
    float routed_scale;     /* routed_scaling_factor, finite */
    const float *router_w;    /* [E][H] fp32 */
    const float *router_bias; /* [E] fp32 selection bias; NULL = all zero */
    moe_q4 gate, up, down;    /* routed experts, stacked by expert id */
    moe_q4 sh_gate, sh_up, sh_down; /* shared expert [Fs][H] / [H][Fs]; ignored if Fs == 0 */
    /* Group-limited routing.  The pages' engine runs one group ([R] §1.2: n_group == 1,
     * asserted); with n_group > 1 (DeepSeek-V3's noaux_tc) the experts form n_group equal
     * groups of consecutive ids, each scored by the sum of its two largest choice scores,
     * and only the topk_group best groups (equal scores: lower group id) take part in the
     * top-k.  n_group 0 or 1: no groups.  Otherwise E % n_group == 0, at least two experts
     * per group, n_group <= 64, 1 <= topk_group <= n_group and topk_group * E / n_group >= k
     * (MOE_EINVAL otherwise). */
    int32_t n_group;
    int32_t topk_group;
    /* Activations entering the expert products: 0 or 16 (default), 16-bit fixed point
     * per block as described at moe_expert_ffn; 8, the pages' opt-in quantised-activation
     * path ([C] §2.2: the integer path quantises activations and is opt-in because it
     * changes results): per block (the same blocks: 32 values for T <= 4, 256 above) the
     * codes rint(x * 2^n) in [-127, 127] with n the largest integer (at most 149) for
     * which max|x| * 2^n <= 127, for x and for the SwiGLU output; the matrix-core path
     * then runs one int8 product per group instead of two.  Other values: MOE_EINVAL.
     * With expert_fmt MOE_FMT_MXFP4 only 0 or 16 (MOE_EUNSUPPORTED for 8). */
    int32_t act_bits;
    /* Expert weight format, MOE_FMT_* (0: int4-gs64); other values MOE_EINVAL.  How each
     * format enters the products is described at moe_expert_ffn. */
    int32_t expert_fmt;
} moe_layer;

/* Optional routing outputs of moe_layer_forward.  Any member may be NULL. */
typedef struct {
    int32_t *ids;      /* [T][k] */
    float *w;          /* [T][k] */
    int32_t *keff;     /* [T] */
    int32_t *n_uniq;   /* [1] */
    int32_t *uniq;     /* [E] */
    int32_t *off;      /* [E+1] */
    int32_t *row_tok;  /* [T*k] */
    int32_t *pick_row; /* [T*k] */
} moe_route_out;

/* Workspace bytes any call below needs for up to max_tokens tokens of layer L
 * (0 for an invalid L; the calls then return MOE_EINVAL).  Pure host function. */
size_t moe_workspace_bytes(const moe_layer *L, int32_t max_tokens);

/* Steps 1-2 ([R] §1.1, §1.2): router logits and noaux_tc selection.
 *   x [T][H] fp32.  For each token: logit_e = Wr[e] . x (exact fp32 products summed
 *   in fp64); sig_e = sigmoid(logit_e) and choice_e = sig_e + bias_e in fp64; k
 *   rounds of argmax over choice, excluding experts already taken (equal scores
 *   go to the lower expert id); if 0 < top_p < 1, the k gates sorted by sig
 *   descending (equal gates keep selection order) are cut after the shortest
 *   prefix whose sum reaches top_p * (sum of all k); the kept gates (sig, never
 *   choice) are renormalised to sum 1 if norm_topk, then multiplied by
 *   routed_scale, and rounded to fp32.
 * Outputs: ids [T][k] int32, kept experts in selection order, -1 past keff;
 *          w [T][k] fp32, 0 past keff;  keff [T] int32, number kept (1..k). */
int moe_route(const moe_layer *L, const float *x, int32_t T, int32_t *ids, float *w,
              int32_t *keff, void *ws, size_t ws_bytes, void *stream);

/* Step 3 ([R] §1.3, batch-union): deduplicates the kept experts of the whole batch
 * so each is read once, and builds the token permutation.
 *   ids [T][k], keff [T] as produced by moe_route (ids outside [0, E) and slots
 *   at or past keff are ignored).  The kept ids of one token must be distinct, as
 *   moe_route produces them: a token that lists an expert twice gets one row for
 *   both picks (count, off and row_tok then differ from counting the pick twice,
 *   and both picks' pick_row name that row); nothing is read or written out of
 *   bounds either way.
 * Outputs: n_uniq [1]; uniq [E] the distinct experts ascending, -1 after n_uniq;
 *          off [E+1] exclusive prefix sum of per-expert row counts;
 *          row_tok [T*k] token of each row, rows ordered by (expert, token)
 *          ascending, -1 past off[E]; pick_row [T*k] row of pick (t, j), -1 if
 *          not kept.  All exact integers. */
int moe_union(const moe_layer *L, const int32_t *ids, const int32_t *keff, int32_t T,
              int32_t *n_uniq, int32_t *uniq, int32_t *off, int32_t *row_tok,
              int32_t *pick_row, void *ws, size_t ws_bytes, void *stream);

/* Step 4 ([R] §1.3, expert compute): for every row r < off[E] of the union, the
 * SwiGLU FFN of expert e(r) on token row_tok[r]:
 *   y_rows[r] = Wd_e (silu(Wg_e x) * (Wu_e x)),   fp32 accumulation, unweighted.
 * The int4 codes enter the products exactly; the activations (x, and the SwiGLU
 * output before the down projection) as 16-bit fixed point with a power-of-two step
 * per block of consecutive values (32 for T <= 4, 256 for larger T): one rounding of
 * less than max|x| / 32639 per value, none for values with at most 15 significant
 * bits relative to the block's largest; the dot products are exact int32 sums.
 * int3-g64 experts enter the same way, and so do MXFP4 experts for T <= 4 (their doubled
 * E2M1 values are integers in [-12, 12]; the 32-element activation blocks match the
 * exponent blocks).  Above T = 4 MXFP4 experts enter as their exact bf16 values (E2M1
 * times the block's power of two) and each activation as two bf16 terms
 * (x = hi + lo + r with |r| <= 2^-16 |x|), for bf16 matrix-core products accumulated
 * in fp32.
 * Inputs n_uniq/uniq/off/row_tok as produced by moe_union (device).
 * Output: y_rows [T*k][H] fp32; rows past off[E] are left untouched. */
int moe_expert_ffn(const moe_layer *L, const float *x, int32_t T, const int32_t *n_uniq,
                   const int32_t *uniq, const int32_t *off, const int32_t *row_tok,
                   float *y_rows, void *ws, size_t ws_bytes, void *stream);

/* Steps 1-5 ([R] §1, §1.4): the whole layer,
 *   out[t] = sum_{j < keff_t} w[t][j] * FFN_{ids[t][j]}(x_t) + FFN_shared(x_t),
 * the shared expert with weight 1 for every token.  out [T][H] is fp32
 * (out_dtype MOE_F32) or bf16 round-to-nearest-even of the fp32 result
 * (MOE_BF16).  dbg may be NULL; its non-NULL members receive the routing and
 * union outputs described above. */
int moe_layer_forward(const moe_layer *L, const float *x, int32_t T, void *out,
                      int32_t out_dtype, const moe_route_out *dbg, void *ws, size_t ws_bytes,
                      void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): moe_layer_forward with its scratch
 * in a file-scope device array of MOE_STATIC_SCRATCH_BYTES instead of a caller
 * workspace.  Same arguments (minus ws and ws_bytes), validation, outputs and errors;
 * a layer and batch whose workspace (moe_workspace_bytes(L, T)) exceeds the array give
 * MOE_EWORKSPACE and launch nothing (64 MiB: the GLM-shaped layer up to 128 tokens).
 * The call allocates nothing: the array is part of the library's device code, held on
 * every GPU the library runs on until the process ends; its address is looked up once
 * per device on the first call there (with that device current).  Every call on one
 * GPU shares that GPU's array, and its contents on entry are ignored (as a workspace's
 * are), so nothing in it needs clearing; calls that overlap in time on one GPU (other
 * streams or host threads without ordering) race on it and must be serialised by the
 * caller.  Devices numbered 64 and above give MOE_EDEVICE. */
#define MOE_STATIC_SCRATCH_BYTES (64u << 20)
int moe_layer_forward_static(const moe_layer *L, const float *x, int32_t T, void *out,
                             int32_t out_dtype, const moe_route_out *dbg, void *stream);

/* First-dense layers ([R] §1.5): the model's first layers are a plain MLP (dense_mlp),
 * not MoE.  For every token t:
 *   out[t] = Wd (silu(Wg x_t) * (Wu x_t)),
 * the same int4-gs64 SwiGLU and arithmetic as an expert in moe_expert_ffn (16-bit
 * fixed-point activation blocks, exact int32 dot products, fp32 accumulation).  x [T][H]
 * fp32; out [T][H] fp32 (MOE_F32) or bf16 round-to-nearest-even of the fp32 result
 * (MOE_BF16).  Conventions, validation and errors as moe_layer_forward; the workspace
 * comes from moe_dense_workspace_bytes (0 for an invalid D). */
typedef struct {
    int32_t hidden;       /* H, multiple of 64, up to MOE_MAX_DIM */
    int32_t ffn;          /* F, multiple of 64, up to MOE_MAX_DIM */
    moe_q4 gate, up, down; /* [F][H], [F][H], [H][F] */
} moe_dense;

size_t moe_dense_workspace_bytes(const moe_dense *D, int32_t max_tokens);
int moe_dense_forward(const moe_dense *D, const float *x, int32_t T, void *out, int32_t out_dtype,
                      void *ws, size_t ws_bytes, void *stream);

/* ---- expert residency tier ---------------------------------------------
 * HBM as a cache over an expert bank in pinned host memory ([R] §1.3 cache resolution,
 * §3 multi-level expert cache, §4 tier repin, §5 router-lookahead prefetch; [C] §2.1 VRAM
 * expert tier).  One tier serves one layer (the pages keep one LRU per layer).
 *
 * The layer's ROUTED expert tensors (gate/up/down q and s in the moe_layer) are the
 * backing store: stacked by expert id as usual, in pinned host memory (hipHostMalloc,
 * e.g. torch's pin_memory; not hipHostRegister), given as the device-side addresses of
 * that memory (hipHostGetDevicePointer), 16-byte aligned.  The router and
 * the shared expert stay in device memory.  The tier's n_slots HBM slots each hold one
 * expert (moe_tier_slot_bytes: gate q, gate s, up q, up s, down q, down s, each
 * 256-byte aligned); the first n_pinned slots form the pinned hot store.
 *
 * Per forward, after the batch union, one workgroup resolves every union expert in
 * ascending id order: a resident expert (pinned or cached) is a hit and its slot is
 * stamped with the step number; a missing one takes a victim slot and is copied there
 * from host memory.  Victims are the slots that are neither pinned nor holding an
 * expert of this union, least recently used first (empty slots first, then the
 * smallest stamp, ties to the lower slot index), handed to the misses in ascending
 * expert id order ([R] §1.3: LRU, evict the least used).  Each union expert's heat and
 * usage grow by its row count ([R] §1.2: eheat/eusage).  The copies run on the call's
 * stream before the expert FFNs, which read every union expert from its slot.  Nothing
 * is synchronised with or copied to the host.
 *
 * State (moe_tier_state_bytes, device, 256-byte aligned; all int32 unless stated, in
 * this order, each array starting at a multiple of 4 bytes):
 *   hdr[16]: [0] step count, [1] copies made by the last call, [2] hits, [3] misses,
 *            [4] swaps by repin, [5] experts prefetched, [6] n_slots, [7] n_experts
 *            (2-5 cumulative since moe_tier_init), rest 0;
 *   slot_expert[S] (-1 = empty), slot_pinned[S] (0/1), slot_used[S] (stamp, -1 empty),
 *   expert_slot[E] (-1 = not resident), heat[E] (uint32, halved by each repin pass),
 *   usage[E] (uint32, never decayed), copy_list[2*min(E,S)] (expert, slot) of the last
 *   call's copies; then, 16-byte aligned, moe_q4 table[3*E] (gate, up, down of every
 *   resident expert; the FFNs' view).
 * Calls on one tier must be ordered (one stream, or events between streams). */
typedef struct {
    int32_t n_slots;   /* S >= 1 */
    int32_t n_pinned;  /* pinned slots 0 .. n_pinned-1 (fixed by moe_tier_init) */
    void *slots;       /* device, n_slots * moe_tier_slot_bytes(L) bytes, 256-byte aligned */
    void *state;       /* device, moe_tier_state_bytes(L, n_slots) bytes, 256-byte aligned */
} moe_tier;

size_t moe_tier_slot_bytes(const moe_layer *L);
size_t moe_tier_state_bytes(const moe_layer *L, int32_t n_slots);

/* Resets the tier: every slot empty, heat and usage 0, counters 0; then loads the
 * experts pins[0 .. n_pin-1] (host array, distinct ids in [0, E), n_pin == tier->n_pinned
 * <= min(n_slots, 256)) into slots 0 .. n_pin-1 as the pinned hot store ([R] §3.1: the
 * caller picks them, e.g. the hottest experts of a usage histogram). */
int moe_tier_init(const moe_layer *L, const moe_tier *tier, const int32_t *pins, int32_t n_pin,
                  void *stream);

/* moe_layer_forward with the routed experts read through the tier (above).  Needs
 * n_slots - n_pinned >= min(E, T*k) (MOE_EUNSUPPORTED otherwise).  Same outputs,
 * bit for bit, as moe_layer_forward on the same layer held in device memory. */
int moe_tier_layer_forward(const moe_layer *L, const moe_tier *tier, const float *x, int32_t T,
                           void *out, int32_t out_dtype, const moe_route_out *dbg, void *ws,
                           size_t ws_bytes, void *stream);

/* Router-lookahead prefetch ([R] §5): makes the distinct experts of the predicted picks
 * ids [T][k] (device, slots at or past keff[t] and ids outside [0, E) ignored) resident,
 * as the resolution above does, without counting heat, usage, hits or misses and
 * without advancing the step: fetched and already-resident experts are stamped with
 * the current step.  Meant for the next layer's tier on a copy stream while this layer
 * computes (the predicted ids from moe_route of that layer's router on this layer's
 * input).  Needs n_slots - n_pinned >= min(E, T*k). */
int moe_tier_prefetch(const moe_layer *L, const moe_tier *tier, const int32_t *ids,
                      const int32_t *keff, int32_t T, void *stream);

/* Heat-driven repin ([R] §4): up to max_swaps (1..4) times, the coldest pinned expert
 * fc (lowest heat, ties to the lower expert id) is exchanged with the hottest unpinned
 * expert fh (highest heat, ties to the lower id) if heat[fh] > heat[fc] + heat[fc]/4 + 4
 * (integer division), else the pass stops.  An fh already cached takes over the pinned
 * flag (fc's slot becomes an ordinary cache slot); otherwise fh is copied into fc's slot
 * and fc leaves HBM.  Then every heat is halved (shift right by one). */
int moe_tier_repin(const moe_layer *L, const moe_tier *tier, int32_t max_swaps, void *stream);

/* Glue between stacked MoE layers -- not a step of the layer itself.  For each of
 * the T rows of H fp32 values: h_out = h + delta (delta NULL: h_out = h), then
 * x_out = h_out / sqrt(mean(h_out^2) + eps) (RMSNorm with unit gain), fp32 with
 * a fixed summation order.  h_out may alias h; x_out must not alias h or delta.
 * Same conventions as above (device pointers, 16-byte aligned, enqueue only,
 * validation before launch, T == 0 a no-op); H a positive multiple of 64 up to
 * MOE_MAX_DIM, eps finite and >= 0. */
int moe_residual_rmsnorm(const float *h, const float *delta, int32_t T, int32_t H, float eps,
                         float *h_out, float *x_out, void *stream);

/* Static description of a return code. */
const char *moe_strerror(int code);

/* ---- measurement -------------------------------------------------------
 * Kernel timing for benchmarks.  Between moe_prof_begin() and moe_prof_end(),
 * every kernel the calls above launch is bracketed by two HIP events recorded
 * on the call's own stream.  moe_prof_end() waits for those events, returns
 * per-kernel totals (summed over launches, in milliseconds) and stops the
 * timing.  The recording belongs to the calling host thread: calls made on other
 * threads are neither timed nor affected.  Measurement only: it never changes what a
 * call computes.
 * moe_prof_end writes at most max_entries entries and the number of distinct
 * kernels to *n_entries.  Both return MOE_OK, or MOE_EDEVICE if an event call
 * failed, MOE_EINVAL for bad arguments. */
typedef struct {
    char name[32];     /* kernel family, e.g. "ffn_gateup" */
    int32_t launches;
    double ms;         /* summed event-to-event time */
} moe_prof_stat;

int moe_prof_begin(void);

/* Streaming-read probe (measurement only, not a step of the layer): one kernel that
 * reads the `bytes` of device buffer `buf` once (16-byte aligned, bytes a multiple of
 * 16) with `blocks` workgroups of 256 threads, and stores the XOR of all its words to
 * sink[0] only if that XOR equals `key` (so nothing is normally written).  Its time
 * gives the part's practical HBM read ceiling.  MOE_EINVAL for bad arguments,
 * MOE_EDEVICE without a gfx950 device or on a launch failure. */
int moe_probe_read(const void *buf, size_t bytes, uint32_t key, uint32_t *sink, int32_t blocks,
                   void *stream);
int moe_prof_end(moe_prof_stat *out, int32_t max_entries, int32_t *n_entries);

/* ---- test entry point --------------------------------------------------
 * Not part of the layer's computation: for tests that check the expert products bit
 * for bit.  The same as moe_expert_ffn (same arguments, validation, errors and
 * outputs) except for what the gate/up step hands to the down projection, chosen per
 * call by gate_up_output: MOE_GU_SWIGLU silu(Wg x) * (Wu x) as in step 4 ([R] §1.3),
 * MOE_GU_GATE the gate pre-activation Wg x, MOE_GU_UP the up pre-activation Wu x.  With
 * integer activations and power-of-two group scales every product and partial sum is
 * exact, so Wd (Wg x) matches an exact reference bitwise where SiLU's exp would not.
 * Another gate_up_output value gives MOE_EINVAL.  Nothing is kept between calls: no
 * other call's result depends on this one. */
#define MOE_GU_SWIGLU 0
#define MOE_GU_GATE 1
#define MOE_GU_UP 2
int moe_expert_ffn_probe(const moe_layer *L, const float *x, int32_t T, const int32_t *n_uniq,
                         const int32_t *uniq, const int32_t *off, const int32_t *row_tok,
                         int32_t gate_up_output, float *y_rows, void *ws, size_t ws_bytes,
                         void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */

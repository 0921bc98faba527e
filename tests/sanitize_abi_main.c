/* Drives the host side of the C ABI (include/moe.h) for a library built with
 * AddressSanitizer and UndefinedBehaviorSanitizer on its host code
 * (tests/test_sanitizers.py): workspace plans, every validation error, the test entry
 * point, the static-scratch forward's size limit and error strings.  No call reaches a kernel launch: each fails validation first,
 * except one well-formed call made only when argv[1] is "nogpu", where it must report
 * MOE_EDEVICE.  Pointers are fake, aligned addresses that validation never
 * dereferences.  Exits 0 when every call returns what it should. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../include/moe.h"

static int fails = 0;
#define EXPECT(c) do { if (!(c)) { fprintf(stderr, "FAILED: %s (line %d)\n", #c, __LINE__); fails++; } } while (0)
#define FAKE(a) ((void *)(uintptr_t)(a))

static moe_layer layer(void) {
    moe_layer L;
    memset(&L, 0, sizeof L);
    L.hidden = 256; L.n_experts = 16; L.ffn = 128; L.shared_ffn = 128; L.top_k = 4;
    L.top_p = 0.0f; L.norm_topk = 1; L.routed_scale = 1.0f;
    L.router_w = FAKE(0x10000); L.router_bias = FAKE(0x10000);
    moe_q4 q = {FAKE(0x10000), FAKE(0x10000)};
    L.gate = L.up = L.down = L.sh_gate = L.sh_up = L.sh_down = q;
    return L;
}

static int forward(const moe_layer *L, int32_t T, size_t ws_bytes, const void *x, void *out) {
    return moe_layer_forward(L, x, T, out, MOE_F32, NULL, FAKE(0x40000), ws_bytes, NULL);
}

int main(int argc, char **argv) {
    moe_layer L = layer();
    const int32_t sizes[] = {0, 1, 2, 8, 63, 64, 65, 300, MOE_MAX_TOKENS};
    size_t prev = 0;
    for (int i = 0; i < 9; i++) {
        const size_t b = moe_workspace_bytes(&L, sizes[i]);
        EXPECT(b > 0 && b >= prev);
        prev = b;
    }
    EXPECT(moe_workspace_bytes(&L, -1) == 0 && moe_workspace_bytes(&L, MOE_MAX_TOKENS + 1) == 0);
    EXPECT(moe_workspace_bytes(NULL, 4) == 0);
    const size_t ws = moe_workspace_bytes(&L, 8);
    const void *x = FAKE(0x20000);
    void *out = FAKE(0x30000);

    moe_layer B = L; B.hidden = 100;
    EXPECT(forward(&B, 4, ws, x, out) == MOE_EINVAL);
    B = L; B.top_k = 0;
    EXPECT(forward(&B, 4, ws, x, out) == MOE_EINVAL);
    B = L; B.n_experts = MOE_MAX_EXPERTS + 1;
    EXPECT(forward(&B, 4, ws, x, out) != MOE_OK);
    B = L; B.top_p = 1.5f;
    EXPECT(forward(&B, 4, ws, x, out) == MOE_EINVAL);
    B = L; B.n_group = 3;                      /* 16 experts do not split into 3 groups */
    EXPECT(forward(&B, 4, ws, x, out) == MOE_EINVAL);
    B = L; B.n_group = 4; B.topk_group = 0;
    EXPECT(forward(&B, 4, ws, x, out) == MOE_EINVAL);
    B = L; B.n_group = 8; B.topk_group = 1;    /* 2 experts kept < top-4 */
    EXPECT(forward(&B, 4, ws, x, out) == MOE_EINVAL);
    B = L; B.n_group = 16; B.topk_group = 8;   /* groups of one expert */
    EXPECT(forward(&B, 4, ws, x, out) == MOE_EINVAL);
    B = L; B.n_group = -1;
    EXPECT(forward(&B, 4, ws, x, out) == MOE_EINVAL);
    B = L; B.router_w = NULL;
    EXPECT(forward(&B, 4, ws, x, out) == MOE_EINVAL);
    EXPECT(forward(&L, 4, ws, NULL, out) == MOE_EINVAL);
    EXPECT(forward(&L, 4, ws, FAKE(0x20004), out) == MOE_EALIGN);
    EXPECT(forward(&L, 4, 16, x, out) == MOE_EWORKSPACE);
    EXPECT(forward(&L, MOE_MAX_TOKENS + 1, ws, x, out) != MOE_OK);
    EXPECT(forward(&L, 0, ws, x, out) == MOE_OK);  /* T == 0: nothing to do */
    EXPECT(moe_layer_forward(&L, x, 4, out, 7, NULL, FAKE(0x40000), ws, NULL) == MOE_EINVAL);

    int32_t *i32 = FAKE(0x50000);
    EXPECT(moe_route(NULL, x, 4, i32, FAKE(0x60000), i32, FAKE(0x40000), ws, NULL) == MOE_EINVAL);
    EXPECT(moe_route(&L, x, 4, NULL, FAKE(0x60000), i32, FAKE(0x40000), ws, NULL) == MOE_EINVAL);
    EXPECT(moe_union(&L, NULL, i32, 4, i32, i32, i32, i32, i32, FAKE(0x40000), ws, NULL) == MOE_EINVAL);
    EXPECT(moe_expert_ffn(&L, x, 4, i32, i32, i32, NULL, FAKE(0x70000), FAKE(0x40000), ws, NULL) == MOE_EINVAL);
    EXPECT(moe_residual_rmsnorm(FAKE(0x20000), NULL, 4, 100, 1e-6f, FAKE(0x30000), NULL, NULL) == MOE_EINVAL);

    EXPECT(moe_expert_ffn_probe(&L, x, 4, i32, i32, i32, i32, 3, FAKE(0x70000), FAKE(0x40000), ws, NULL) == MOE_EINVAL);
    EXPECT(moe_expert_ffn_probe(&L, x, 4, i32, i32, i32, NULL, MOE_GU_GATE, FAKE(0x70000), FAKE(0x40000), ws, NULL) == MOE_EINVAL);
    /* the static-scratch forward: validation as moe_layer_forward, then the size limit */
    EXPECT(moe_layer_forward_static(&L, NULL, 4, out, MOE_F32, NULL, NULL) == MOE_EINVAL);
    EXPECT(moe_layer_forward_static(&L, x, 4, out, 7, NULL, NULL) == MOE_EINVAL);
    EXPECT(moe_layer_forward_static(&L, FAKE(0x20004), 4, out, MOE_F32, NULL, NULL) == MOE_EALIGN);
    EXPECT(moe_layer_forward_static(NULL, x, 4, out, MOE_F32, NULL, NULL) == MOE_EINVAL);
    EXPECT(moe_layer_forward_static(&L, x, 0, out, MOE_F32, NULL, NULL) == MOE_OK);
    EXPECT(moe_layer_forward_static(&L, x, MOE_MAX_TOKENS + 1, out, MOE_F32, NULL, NULL) == MOE_EUNSUPPORTED);
    B = L; B.hidden = 1024; B.ffn = 512; B.shared_ffn = 512; B.n_experts = 32; B.top_k = 8;
    EXPECT(moe_workspace_bytes(&B, MOE_MAX_TOKENS) > (size_t)MOE_STATIC_SCRATCH_BYTES);
    EXPECT(moe_layer_forward_static(&B, x, MOE_MAX_TOKENS, out, MOE_F32, NULL, NULL) == MOE_EWORKSPACE);
    for (int c = -5; c <= 0; c++) EXPECT(strcmp(moe_strerror(c), "unknown error code") != 0);
    EXPECT(strcmp(moe_strerror(99), "unknown error code") == 0);

    if (argc > 1 && strcmp(argv[1], "nogpu") == 0) {
        EXPECT(forward(&L, 4, ws, x, out) == MOE_EDEVICE);
        EXPECT(moe_layer_forward_static(&L, x, 4, out, MOE_F32, NULL, NULL) == MOE_EDEVICE);
    }
    if (fails) return 1;
    printf("abi sanitizer run ok\n");
    return 0;
}

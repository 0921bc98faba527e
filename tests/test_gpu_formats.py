"""The other expert formats on the GPU, through the C ABI: MXFP4 experts (E2M1 codes with
UE8M0 exponents per 32, "colibri 开发演进实录" §五/§六) and int3-g64 experts (same page,
§8.3), against the oracle's decoders of the same bytes.

Every case checks, as the int4-gs64 parity tests do: routing and union exact, expert rows
and the layer output within the bar, bf16 output the RNE of the fp32 output.  Shapes cover
both expert-FFN paths (the GEMV for at most 4 tokens, with the one-token fused selection;
the matrix-core path above, with 16- and 32-row items), ragged reductions (a partial
4-group chunk, a single 64-group), the largest dimensions, and exactness special cases.
"""
import numpy as np
import pytest
import torch

import oracle as R
import routed_int4_expert_amd as M
from routed_int4_expert_amd import synth as S
from test_gpu_parity import DEV, assert_close, check_routing, check_union, full_parity, say

pytestmark = pytest.mark.gpu

FMTS = [S.FMT_MXFP4, S.FMT_INT3]
FMT_IDS = ["mxfp4", "int3"]

BASE = [
    S.SHAPES["tiny"],
    S.custom("ragged", hidden=320, n_experts=24, ffn=192, shared_ffn=64, top_k=5, tokens=11,
             top_p=0.8, routed_scale=2.5, bias_amp=0.3),
    S.custom("noshared", hidden=128, n_experts=8, ffn=64, shared_ffn=0, top_k=2, tokens=5,
             norm_topk=0),
    S.custom("manytok", hidden=128, n_experts=40, ffn=64, shared_ffn=128, top_k=6, tokens=300,
             bias_amp=0.2),
    S.custom("maxk", hidden=64, n_experts=256, ffn=64, shared_ffn=64, top_k=16, tokens=70,
             top_p=0.5, router_std=0.125, bias_amp=0.05),
    S.custom("onetok", hidden=512, n_experts=32, ffn=256, shared_ffn=256, top_k=4, tokens=1,
             routed_scale=2.5),
    S.custom("onetok_noshared", hidden=256, n_experts=16, ffn=128, shared_ffn=0, top_k=4, tokens=1,
             top_p=0.9),
    S.custom("twotok", hidden=2048, n_experts=64, ffn=512, shared_ffn=512, top_k=8, tokens=2,
             router_std=1 / 45.25),
    S.custom("raggedfew", hidden=320, n_experts=24, ffn=192, shared_ffn=64, top_k=5, tokens=3,
             top_p=0.8, routed_scale=2.5, bias_amp=0.3),
    S.custom("fourtok_k64", hidden=64, n_experts=16, ffn=64, shared_ffn=64, top_k=4, tokens=4),
    S.custom("midtok", hidden=320, n_experts=48, ffn=128, shared_ffn=64, top_k=6, tokens=40,
             top_p=0.85, routed_scale=1.5, bias_amp=0.2),
    S.custom("maxdim", hidden=16384, n_experts=8, ffn=128, shared_ffn=64, top_k=2, tokens=5),
    S.custom("maxdim_gemv", hidden=16384, n_experts=8, ffn=128, shared_ffn=64, top_k=2, tokens=3),
    S.custom("maxdim_one", hidden=16384, n_experts=8, ffn=128, shared_ffn=64, top_k=2, tokens=1),
    S.custom("maxffn_gemv", hidden=128, n_experts=8, ffn=16384, shared_ffn=16384, top_k=2,
             tokens=4),
    S.custom("rows256", hidden=512, n_experts=16, ffn=256, shared_ffn=256, top_k=8, tokens=512,
             bias_amp=0.05),
]


def with_fmt(sh, fmt):
    return S.custom(f"{sh.name}_{S.FMT_NAMES[fmt]}", **{k: getattr(sh, k) for k in (
        "hidden", "n_experts", "ffn", "shared_ffn", "top_k", "top_p", "norm_topk", "routed_scale",
        "tokens", "router_std", "bias_kind", "bias_amp")}, expert_fmt=fmt)


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("base", BASE, ids=[s.name for s in BASE])
def test_format_full_parity(base, fmt):
    sh = with_fmt(base, fmt)
    say(f"{sh.name}: H={sh.hidden} E={sh.n_experts} F={sh.ffn} Fs={sh.shared_ffn} k={sh.top_k} "
        f"T={sh.tokens}")
    d = S.make_layer(sh, seed=0)
    x = S.make_batch(sh, d, seed=0)
    full_parity(sh, d, x)


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("T", [1, 3, 24, 40], ids=["one", "gemv", "mfma16", "mfma32"])
def test_format_exact_expert_products(T, fmt):
    """Exactness special case: activations in {-1, 0, 1} and every block scale 2^-6.

    Every weight is 2^-7 times an integer of at most 4 bits, so the gate pre-activations
    P are 2^-13 times integers of at most 12 bits and the down projection of P is exact in
    fp32 and, with P split into bf16 terms, on the matrix cores.  With the gate/up step
    writing P (moe_expert_ffn_probe), the expert rows Wd P must equal the exact value bit
    for bit on every path."""
    sh = S.custom(f"exact{T}_{S.FMT_NAMES[fmt]}", hidden=256, n_experts=8, ffn=128, shared_ffn=64,
                  top_k=2, tokens=T, expert_fmt=fmt)
    d = S.make_layer(sh, seed=0)
    for key in ("gate_s", "up_s", "down_s", "sh_gate_s", "sh_up_s", "sh_down_s"):
        d[key] = np.full_like(d[key], 127 - 6 if fmt == S.FMT_MXFP4 else 2.0 ** -6)
    x = np.rint(S.uniform_f32(0, f"exact{T}/x", (T, sh.hidden), -1.49, 1.49)).astype(np.float32)
    layer = M.Layer.from_host(d, DEV)
    xd = torch.from_numpy(x).to(DEV)
    ids, w, keff, rids, rw, rkeff = check_routing(d, layer, x, xd, sh)
    un, ru = check_union(layer, ids, keff, rids, rkeff, sh.n_experts, sh.top_k)
    y = M.moe_expert_ffn_probe(layer, xd, un, M.MOE_GU_GATE)
    torch.cuda.synchronize()
    rows = int(ru["off"][-1])
    x64 = x.astype(np.float64)
    H, F = sh.hidden, sh.ffn
    ref = np.empty((rows, H), np.float64)
    for e in range(sh.n_experts):
        r0, r1 = int(ru["off"][e]), int(ru["off"][e + 1])
        if r1 == r0:
            continue
        pre = x64[ru["row_tok"][r0:r1]] @ R.dequantize(fmt, d["gate_q"][e], d["gate_s"][e], H).T
        ref[r0:r1] = pre @ R.dequantize(fmt, d["down_q"][e], d["down_s"][e], F).T
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref), "reference not exact in fp32"
    np.testing.assert_array_equal(y.cpu().numpy()[:rows], ref.astype(np.float32))
    say(f"exact {S.FMT_NAMES[fmt]} T={T}: {rows} rows bit-identical")


@pytest.mark.parametrize("T", [1, 9], ids=["gemv", "mfma"])
def test_mxfp4_block_exponents_and_nan(T):
    """MXFP4 exponent bytes spread over 2^-12 .. 2^+12 independently per 32-element block
    (the two blocks of a 64-group differ): parity as usual.  Then one block of the shared
    expert's gate with exponent byte 255 (NaN): every token reads it, so the whole output
    is NaN, as in the oracle."""
    sh = S.custom(f"f4exp{T}", hidden=256, n_experts=8, ffn=128, shared_ffn=64, top_k=2, tokens=T,
                  expert_fmt=S.FMT_MXFP4)
    d = S.make_layer(sh, seed=0)
    for key in ("gate_s", "up_s", "down_s", "sh_gate_s", "sh_up_s", "sh_down_s"):
        e = S.uniform_f64(0, f"f4exp/{key}", d[key].shape, d[key].mean() - 12, d[key].mean() + 12)
        d[key] = np.rint(e).astype(np.uint8)
    x = S.make_batch(sh, d, seed=0)
    full_parity(sh, d, x)
    bad = dict(d)
    bad["sh_gate_s"] = d["sh_gate_s"].copy()
    bad["sh_gate_s"][0, 0] = 255
    layer = M.Layer.from_host(bad, DEV)
    out = M.moe_layer_forward(layer, torch.from_numpy(x).to(DEV))
    torch.cuda.synchronize()
    ref = R.layer_forward(R.Layer(bad), x)
    assert np.isnan(ref).all()
    assert np.isnan(out.cpu().numpy()).all()


# ------------------------------------------------------------------ GLM-sized layers
@pytest.fixture(scope="module", params=FMTS, ids=FMT_IDS)
def glm_fmt_bank(request):
    fmt = request.param
    sh = S.custom("glm_fmt", **{k: getattr(S.SHAPES["glm_decode"], k) for k in (
        "hidden", "n_experts", "ffn", "shared_ffn", "top_k", "top_p", "norm_topk", "routed_scale",
        "router_std", "bias_amp")}, bank="glm", expert_fmt=fmt)
    say(f"generating the GLM-shaped {S.FMT_NAMES[fmt]} expert bank (257 experts)")
    return fmt, S.Bank(sh, seed=0)


def _glm_fmt_layer(base, fmt, bank):
    import dataclasses
    sh = dataclasses.replace(S.SHAPES[base], expert_fmt=fmt)
    return sh, S.make_layer(sh, seed=0, bank=bank)


@pytest.mark.timeout(600)
def test_glm_decode_and_verify_formats(glm_fmt_bank):
    """The GLM-shaped layer (H 6144, 256 experts of F 2048, top-8) in each format, as the
    bench runs it: one-token decode on three token pools (the GEMV with the fused
    selection) and a 16-token batch (matrix cores), every output against the oracle."""
    fmt, bank = glm_fmt_bank
    sh, d = _glm_fmt_layer("glm_decode", fmt, bank)
    layer = M.Layer.from_host(d, DEV)
    Lr = R.Layer(d)
    for pool in range(3):
        x = S.make_batch(sh, d, seed=0, pool=pool)
        xd = torch.from_numpy(x).to(DEV)
        check_routing(d, layer, x, xd, sh)
        out = M.moe_layer_forward(layer, xd)
        torch.cuda.synchronize()
        rel, mx = assert_close(out.cpu().numpy(), R.layer_forward(Lr, x), f"glm {S.FMT_NAMES[fmt]} decode")
        say(f"GLM {S.FMT_NAMES[fmt]} decode pool {pool}: rel-L2 {rel:.2e} max-abs {mx:.2e}")
    x = S.tokens(sh, 16, seed=0, pool=7)
    xd = torch.from_numpy(x).to(DEV)
    ids, w, keff, rids, rw, rkeff = check_routing(d, layer, x, xd, sh)
    check_union(layer, ids, keff, rids, rkeff, sh.n_experts, sh.top_k)
    out = M.moe_layer_forward(layer, xd)
    torch.cuda.synchronize()
    rel, mx = assert_close(out.cpu().numpy(), R.layer_forward(Lr, x), f"glm {S.FMT_NAMES[fmt]} 16 tokens")
    say(f"GLM {S.FMT_NAMES[fmt]} 16 tokens: rel-L2 {rel:.2e} max-abs {mx:.2e}")


@pytest.mark.timeout(900)
def test_glm_prefill_formats(glm_fmt_bank):
    """The 512-token GLM prefill batch in each format: routing and union exact for every
    token; the rows of the expert with the most rows (moe_expert_ffn) and the layer output
    of 48 tokens spread over the batch within the bar."""
    fmt, bank = glm_fmt_bank
    sh, d = _glm_fmt_layer("glm_prefill", fmt, bank)
    x = S.make_batch(sh, d, seed=0)
    layer = M.Layer.from_host(d, DEV)
    xd = torch.from_numpy(x).to(DEV)
    ids, w, keff, rids, rw, rkeff = check_routing(d, layer, x, xd, sh)
    un, ru = check_union(layer, ids, keff, rids, rkeff, sh.n_experts, sh.top_k)
    counts = np.diff(ru["off"])
    Lr = R.Layer(d)
    y = M.moe_expert_ffn(layer, xd, un)
    out = M.moe_layer_forward(layer, xd)
    torch.cuda.synchronize()
    hot = int(np.argmax(counts))
    r0, r1 = int(ru["off"][hot]), int(ru["off"][hot + 1])
    off_e = np.clip(ru["off"], r0, r1).astype(np.int32)
    ref_rows = R.expert_ffn(Lr, x, off_e, ru["row_tok"])[r0:r1]
    rel, mx = assert_close(y.cpu().numpy()[r0:r1], ref_rows, f"glm {S.FMT_NAMES[fmt]} prefill expert {hot}")
    say(f"GLM {S.FMT_NAMES[fmt]} prefill expert {hot} ({r1 - r0} rows): rel-L2 {rel:.2e}")
    toks = np.linspace(0, sh.tokens - 1, 48).astype(np.int32)
    ref = R.layer_forward(Lr, x, toks=toks)
    got = out.cpu().numpy()[toks]
    rel, mx = assert_close(got, ref, f"glm {S.FMT_NAMES[fmt]} prefill sampled tokens")
    for i in range(len(toks)):
        assert_close(got[i], ref[i], f"glm {S.FMT_NAMES[fmt]} prefill token {toks[i]}")
    say(f"GLM {S.FMT_NAMES[fmt]} prefill, 48 tokens: rel-L2 {rel:.2e} max-abs {mx:.2e}")

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

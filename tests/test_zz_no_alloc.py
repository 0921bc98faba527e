"""moe_layer_forward_static (scratch in the library's file-scope device array, nothing
allocated) against moe_layer_forward (caller workspace), through the C ABI.

Both run the same kernels on the same inputs, so the outputs and the routing/union
outputs must be identical bit for bit.  Each case makes two calls in a row, the second
with a smaller batch, so the second call runs on the array the first one left behind.
"""
import ctypes

import numpy as np
import pytest
import torch

import routed_int4_expert_amd as M
from routed_int4_expert_amd import synth as S

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(f"[static] {msg}", flush=True)


def _dbg(T, k, E):
    i32 = dict(dtype=torch.int32, device=DEV)
    return dict(ids=torch.full((T, k), -7, **i32), w=torch.full((T, k), -7.0, device=DEV),
                keff=torch.full((T,), -7, **i32), n_uniq=torch.full((1,), -7, **i32),
                uniq=torch.full((E,), -7, **i32), off=torch.full((E + 1,), -7, **i32),
                row_tok=torch.full((max(T * k, 1),), -7, **i32), pick_row=torch.full((T, k), -7, **i32))


def _same(a, b, what):
    assert a.dtype == b.dtype and a.shape == b.shape, what
    assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.uint8) if b.dtype == torch.bfloat16 else b), what


# (shape, first batch, second batch): the matrix-core path then the GEMV path; one-token
# decode (selection inside the gate/up launch) after a 16-token batch; top-p with a
# shared expert
CASES = [
    (S.custom("st_mfma", hidden=512, n_experts=64, ffn=256, shared_ffn=256, top_k=8, tokens=64,
              top_p=0.8, routed_scale=2.5, bias_amp=0.3), 64, 3),
    (S.custom("st_decode", hidden=1024, n_experts=128, ffn=512, shared_ffn=512, top_k=8,
              tokens=16, routed_scale=2.5), 16, 1),
    (S.custom("st_small", hidden=256, n_experts=16, ffn=128, shared_ffn=0, top_k=4, tokens=40,
              top_p=0.9), 40, 9),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0].name for c in CASES])
@pytest.mark.parametrize("dtype", [M.MOE_F32, M.MOE_BF16], ids=["f32", "bf16"])
def test_static_forward_matches_workspace_forward(case, dtype):
    sh, t1, t2 = case
    d = S.make_layer(sh, seed=0)
    layer = M.Layer.from_host(d, DEV)
    k, E = sh.top_k, sh.n_experts
    for T, pool in ((t1, 0), (t2, 1)):
        say(f"{sh.name} T={T} dtype={dtype}")
        x = torch.from_numpy(S.tokens(sh, T, seed=0, pool=pool)).to(DEV)
        dbg_a, dbg_b = _dbg(T, k, E), _dbg(T, k, E)
        ref = M.moe_layer_forward(layer, x, out_dtype=dtype, dbg=dbg_a)
        got = M.moe_layer_forward_static(layer, x, out_dtype=dtype, dbg=dbg_b)
        torch.cuda.synchronize()
        _same(got, ref, f"{sh.name} T={T} output")
        for name in dbg_a:
            _same(dbg_b[name], dbg_a[name], f"{sh.name} T={T} {name}")
        assert torch.isfinite(ref.float()).all()


def test_static_forward_rejects_oversized_batch():
    """A batch whose workspace exceeds the array is refused before anything is launched,
    and the output is left untouched."""
    sh = S.custom("st_big", hidden=512, n_experts=64, ffn=256, shared_ffn=256, top_k=8,
                  tokens=2048)
    d = S.make_layer(sh, seed=0)
    layer = M.Layer.from_host(d, DEV)
    T = 2048
    assert layer.workspace_bytes(T) > M.MOE_STATIC_SCRATCH_BYTES
    x = torch.zeros((T, sh.hidden), dtype=torch.float32, device=DEV)
    out = torch.full((T, sh.hidden), 3.0, device=DEV)
    rc = M.lib().moe_layer_forward_static(layer.ref(), M._ptr(x), T, M._ptr(out), M.MOE_F32, None,
                                          M._stream(None))
    assert rc == M.MOE_EWORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
    # the largest batch that fits still runs
    T2 = max(t for t in (1024, 768, 512) if layer.workspace_bytes(t) <= M.MOE_STATIC_SCRATCH_BYTES)
    x2 = torch.from_numpy(S.tokens(sh, T2, seed=0)).to(DEV)
    ref = M.moe_layer_forward(layer, x2)
    got = M.moe_layer_forward_static(layer, x2)
    torch.cuda.synchronize()
    _same(got, ref, f"st_big T={T2}")
    say(f"oversized T={T} refused; T={T2} matches")

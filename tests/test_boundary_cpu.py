"""The C ABI without a GPU: exported symbols, workspace plan and every validation
error code, forced from the host.  No call here reaches a kernel launch: each
one fails validation first (the one valid call is made only when no GPU is
present, where it must report MOE_EDEVICE)."""
import ctypes
import os
import re

import pytest

import routed_int4_expert_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    return set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z_]+)\s*\(", src, re.M))


def test_exports_match_header():
    names = _declared()
    assert names == set(M.EXPORTS)
    lib = M.lib()
    for n in names:
        assert hasattr(lib, n), n


def _layer(**kw):
    c = M.LayerC()
    c.hidden, c.n_experts, c.ffn, c.shared_ffn, c.top_k = 256, 16, 128, 128, 4
    c.top_p, c.norm_topk, c.routed_scale = 0.0, 1, 1.0
    fake = 0x10000
    c.router_w = fake
    c.router_bias = fake
    for n in ("gate", "up", "down", "sh_gate", "sh_up", "sh_down"):
        setattr(c, n, M.Q4(fake, fake))
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def ws_bytes(c, T):
    return M.lib().moe_workspace_bytes(ctypes.byref(c), T)


def test_workspace_plan_monotone_and_invalid():
    c = _layer()
    sizes = [ws_bytes(c, T) for T in (0, 1, 2, 8, 63, 64, 65, 300, 4096)]
    assert all(s > 0 for s in sizes)
    assert sizes == sorted(sizes)
    assert ws_bytes(_layer(hidden=100), 4) == 0
    assert ws_bytes(c, -1) == 0 and ws_bytes(c, M.MOE_MAX_TOKENS + 1) == 0
    big = _layer(hidden=6144, n_experts=256, ffn=2048, shared_ffn=2048, top_k=8)
    # y rows + h rows dominate: T*k*(H+F)*4 bytes
    assert ws_bytes(big, 512) >= 512 * 8 * (6144 + 2048) * 4


def call_forward(c, T=4, x=0x20000, out=0x30000, dtype=0, ws=0x40000, wsb=None):
    if wsb is None:
        wsb = ws_bytes(c, max(T, 0)) if ws_bytes(c, max(T, 0)) else 1 << 30
    return M.lib().moe_layer_forward(ctypes.byref(c), x, T, out, dtype, None, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(hidden=0), M.MOE_EINVAL),
    (dict(hidden=100), M.MOE_EINVAL),
    (dict(ffn=96), M.MOE_EINVAL),
    (dict(shared_ffn=32), M.MOE_EINVAL),
    (dict(top_k=0), M.MOE_EINVAL),
    (dict(top_k=17, n_experts=32), M.MOE_EUNSUPPORTED),
    (dict(top_k=20), M.MOE_EINVAL),             # k > E
    (dict(n_experts=300, top_k=4), M.MOE_EUNSUPPORTED),
    (dict(top_p=1.5), M.MOE_EINVAL),
    (dict(top_p=float("nan")), M.MOE_EINVAL),
    (dict(routed_scale=float("inf")), M.MOE_EINVAL),
    (dict(hidden=32768), M.MOE_EUNSUPPORTED),
    (dict(router_w=None), M.MOE_EINVAL),
    (dict(router_w=0x10004), M.MOE_EALIGN),
    (dict(gate=M.Q4(None, 0x10000)), M.MOE_EINVAL),
    (dict(down=M.Q4(0x10008, 0x10000)), M.MOE_EALIGN),
    (dict(sh_up=M.Q4(0x10000, None)), M.MOE_EINVAL),
    (dict(n_group=3), M.MOE_EINVAL),                 # 16 experts in 3 groups
    (dict(n_group=4, topk_group=0), M.MOE_EINVAL),
    (dict(n_group=4, topk_group=5), M.MOE_EINVAL),
    (dict(n_group=8, topk_group=1), M.MOE_EINVAL),   # 2 experts kept < top-4
    (dict(n_group=16, topk_group=8), M.MOE_EINVAL),  # single-expert groups
    (dict(n_group=-1), M.MOE_EINVAL),
    (dict(act_bits=4), M.MOE_EINVAL),
    (dict(act_bits=-8), M.MOE_EINVAL),
    (dict(expert_fmt=3), M.MOE_EINVAL),
    (dict(expert_fmt=-1), M.MOE_EINVAL),
    (dict(expert_fmt=M.MOE_FMT_MXFP4, act_bits=8), M.MOE_EUNSUPPORTED),
])
def test_forward_validation_codes(kw, code):
    assert call_forward(_layer(**kw)) == code


def test_shared_tensors_ignored_without_shared_expert():
    c = _layer(shared_ffn=0, sh_gate=M.Q4(None, None), sh_up=M.Q4(None, None),
               sh_down=M.Q4(None, None))
    assert call_forward(c, x=None) == M.MOE_EINVAL  # fails on x, not on the shared tensors


def test_forward_argument_codes():
    c = _layer()
    assert M.lib().moe_layer_forward(None, 0x20000, 4, 0x30000, 0, None, 0x40000, 1 << 30, None) == M.MOE_EINVAL
    assert call_forward(c, T=-1) == M.MOE_EINVAL
    assert call_forward(c, T=M.MOE_MAX_TOKENS + 1) == M.MOE_EUNSUPPORTED
    assert call_forward(c, dtype=7) == M.MOE_EINVAL
    assert call_forward(c, x=None) == M.MOE_EINVAL
    assert call_forward(c, out=None) == M.MOE_EINVAL
    assert call_forward(c, x=0x20004) == M.MOE_EALIGN
    assert call_forward(c, ws=None) == M.MOE_EWORKSPACE
    assert call_forward(c, wsb=ws_bytes(c, 4) - 1) == M.MOE_EWORKSPACE
    assert call_forward(c, ws=0x40008) == M.MOE_EALIGN
    # T == 0 succeeds without touching anything, even with NULL buffers
    assert call_forward(c, T=0, x=None, out=None, ws=None, wsb=0) == M.MOE_OK


def test_other_entry_points_validate():
    c = _layer()
    L = M.lib()
    r = ctypes.byref(c)
    wsb = ws_bytes(c, 4)
    assert L.moe_route(r, None, 4, 1 << 16, 1 << 16, 1 << 16, 1 << 18, wsb, None) == M.MOE_EINVAL
    assert L.moe_route(r, 0x20004, 4, 1 << 16, 1 << 16, 1 << 16, 1 << 18, wsb, None) == M.MOE_EALIGN
    assert L.moe_route(r, 0x20000, 4, 1 << 16, 1 << 16, 1 << 16, 1 << 18, 16, None) == M.MOE_EWORKSPACE
    assert L.moe_union(r, None, 1, 4, 1, 1, 1, 1, 1, 1 << 18, wsb, None) == M.MOE_EINVAL
    assert L.moe_union(r, 1, 1, -3, 1, 1, 1, 1, 1, 1 << 18, wsb, None) == M.MOE_EINVAL
    assert L.moe_expert_ffn(r, 0x20000, 4, 1, 1, 1, 1, None, 1 << 18, wsb, None) == M.MOE_EINVAL
    assert L.moe_expert_ffn(r, 0x20000, 4, 1, 1, 1, 1, 0x30004, 1 << 18, wsb, None) == M.MOE_EALIGN
    assert L.moe_route(r, None, 0, None, None, None, None, 0, None) == M.MOE_OK


def test_residual_rmsnorm_validation():
    L = M.lib()
    f = L.moe_residual_rmsnorm
    a, b, c, d = 0x10000, 0x20000, 0x30000, 0x40000
    assert f(a, b, 4, 100, 1e-6, c, d, None) == M.MOE_EINVAL          # H not a multiple of 64
    assert f(a, b, -1, 128, 1e-6, c, d, None) == M.MOE_EINVAL
    assert f(a, b, 4, 128, -1.0, c, d, None) == M.MOE_EINVAL          # negative eps
    assert f(a, b, 4, 128, float("nan"), c, d, None) == M.MOE_EINVAL
    assert f(a, b, 4, 32768, 1e-6, c, d, None) == M.MOE_EUNSUPPORTED
    assert f(None, b, 4, 128, 1e-6, c, d, None) == M.MOE_EINVAL
    assert f(a, b, 4, 128, 1e-6, c, a, None) == M.MOE_EINVAL          # x_out aliases h
    assert f(a, b, 4, 128, 1e-6, c, b, None) == M.MOE_EINVAL          # x_out aliases delta
    assert f(a + 4, b, 4, 128, 1e-6, c, d, None) == M.MOE_EALIGN
    assert f(None, None, 0, 128, 1e-6, None, None, None) == M.MOE_OK  # T == 0


def test_strerror():
    for code in (0, -1, -2, -3, -4, -5):
        s = M.strerror(code)
        assert isinstance(s, str) and s and s != "unknown error code"
    assert M.strerror(99) == "unknown error code"


def test_valid_call_without_gpu_reports_device_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; fake pointers must not reach a launch")
    assert call_forward(_layer()) == M.MOE_EDEVICE


def test_expert_ffn_probe_validates():
    """The probe entry point rejects a gate/up output mode other than its three, before
    anything else, and otherwise validates like moe_expert_ffn (no device needed)."""
    lib = M.lib()
    c = _layer()
    i32 = ctypes.c_void_p(0x50000)
    wsb = ws_bytes(c, 4)
    args = lambda mode, x=0x20000: (ctypes.byref(c), ctypes.c_void_p(x), 4, i32, i32, i32, i32, mode,
                                    ctypes.c_void_p(0x70000), ctypes.c_void_p(0x40000), wsb, None)
    for mode in (3, -1, 99):
        assert lib.moe_expert_ffn_probe(*args(mode)) == M.MOE_EINVAL
    for mode in (M.MOE_GU_SWIGLU, M.MOE_GU_GATE, M.MOE_GU_UP):
        assert lib.moe_expert_ffn_probe(*args(mode, x=0x20004)) == M.MOE_EALIGN
        assert lib.moe_expert_ffn_probe(*args(mode, x=0)) == M.MOE_EINVAL


def test_missing_library_fails_loudly():
    """Without the built library every call raises: there is no other path."""
    import subprocess
    import sys
    code = ("import routed_int4_expert_amd as M\n"
            "M.LIB_PATH = '/nonexistent/libmoe_gfx950.so'\n"
            "try:\n"
            "    M.strerror(0)\n"
            "except RuntimeError as e:\n"
            "    print('raised', 'missing' in str(e))\n")
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert res.returncode == 0, res.stderr
    assert res.stdout.strip() == "raised True"


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 exits non-zero with a message, before
    touching a device."""
    import subprocess
    import sys
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert res.returncode != 0
    assert "one GPU" in (res.stdout + res.stderr)


def _dense(**kw):
    c = M.DenseC()
    c.hidden, c.ffn = 256, 192
    for n in ("gate", "up", "down"):
        setattr(c, n, M.Q4(0x10000, 0x10000))
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_dense_validation_codes():
    """moe_dense_forward validates like moe_layer_forward (no device needed)."""
    lib = M.lib()
    ok = _dense()
    nb = lambda c, T: lib.moe_dense_workspace_bytes(ctypes.byref(c), T)
    assert nb(ok, 0) > 0 and nb(ok, 4) <= nb(ok, 5) <= nb(ok, 300)
    assert nb(_dense(hidden=100), 4) == 0 and nb(ok, -1) == 0 and nb(ok, M.MOE_MAX_TOKENS + 1) == 0

    def fwd(c, T=4, x=0x20000, out=0x30000, dtype=0, ws=0x40000, wsb=None):
        wsb = (nb(c, T) or (1 << 30)) if wsb is None else wsb
        return lib.moe_dense_forward(ctypes.byref(c), x, T, out, dtype, ws, wsb, None)

    assert fwd(_dense(hidden=100)) == M.MOE_EINVAL
    assert fwd(_dense(ffn=32)) == M.MOE_EINVAL
    assert fwd(_dense(ffn=32768)) == M.MOE_EUNSUPPORTED
    assert fwd(_dense(gate=M.Q4(None, 0x10000))) == M.MOE_EINVAL
    assert fwd(_dense(down=M.Q4(0x10008, 0x10000))) == M.MOE_EALIGN
    assert fwd(ok, x=None) == M.MOE_EINVAL
    assert fwd(ok, x=0x20004) == M.MOE_EALIGN
    assert fwd(ok, dtype=5) == M.MOE_EINVAL
    assert fwd(ok, T=-1) == M.MOE_EINVAL
    assert fwd(ok, T=M.MOE_MAX_TOKENS + 1) == M.MOE_EUNSUPPORTED
    assert fwd(ok, wsb=16) == M.MOE_EWORKSPACE
    assert fwd(ok, T=0) == M.MOE_OK
    assert lib.moe_dense_forward(None, 0x20000, 4, 0x30000, 0, 0x40000, 1 << 30, None) == M.MOE_EINVAL


def test_format_workspace_and_tier_sizes():
    """Per-format byte counts the host computes: the MXFP4 matrix-core path needs larger
    activation fragments; a tier slot holds one expert in the layer's format."""
    base = _layer(hidden=2048, ffn=512, shared_ffn=512, n_experts=64, top_k=8)
    sizes = {}
    for fmt in (M.MOE_FMT_INT4_G64, M.MOE_FMT_MXFP4, M.MOE_FMT_INT3_G64):
        c = _layer(hidden=2048, ffn=512, shared_ffn=512, n_experts=64, top_k=8, expert_fmt=fmt)
        sizes[fmt] = (ws_bytes(c, 64), ws_bytes(c, 4), M.lib().moe_tier_slot_bytes(ctypes.byref(c)))
    assert sizes[M.MOE_FMT_INT4_G64][1] == sizes[M.MOE_FMT_MXFP4][1] == sizes[M.MOE_FMT_INT3_G64][1]
    assert sizes[M.MOE_FMT_MXFP4][0] > sizes[M.MOE_FMT_INT4_G64][0] == sizes[M.MOE_FMT_INT3_G64][0]
    H, F = 2048, 512
    def slot(code, scale):  # six tensors, each rounded up to 256 bytes
        r = lambda b: (b + 255) // 256 * 256
        return 3 * (r(code) + r(scale))
    assert sizes[M.MOE_FMT_INT4_G64][2] == slot(F * H // 2, F * H // 64 * 4)
    assert sizes[M.MOE_FMT_MXFP4][2] == slot(F * H // 2, F * H // 32)
    assert sizes[M.MOE_FMT_INT3_G64][2] == slot(F * 3 * H // 8, F * H // 64 * 4)
    assert ws_bytes(base, 64) == sizes[M.MOE_FMT_INT4_G64][0]

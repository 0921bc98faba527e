"""The expert residency tier on the GPU, through the C ABI.

The layer's routed experts live in pinned host memory and a tier of HBM slots caches
them ("MoE 路由与专家流式加载" §1.3, §3-§5).  Checked after every call of a sequence of
batches, repins and prefetches:
  - the layer output equals moe_layer_forward on the same layer held in device memory,
    bit for bit (the expert FFNs read the slots the tier copied);
  - the device's slot tables, heat, usage, counters and copy list equal the policy
    oracle (oracle/tier_ref.py) fed with the oracle's own routing of each batch.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle as R
import routed_int4_expert_amd as M
from oracle.tier_ref import TierRef
from routed_int4_expert_amd import synth as S

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ROUTED = ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")


def say(msg):
    print(f"[tier] {msg}", flush=True)


_HIP = None


def device_address(t):
    """The device-side address of a pinned host tensor (hipHostGetDevicePointer)."""
    global _HIP
    if _HIP is None:
        _HIP = ctypes.CDLL("libamdhip64.so")
        _HIP.hipHostGetDevicePointer.restype = ctypes.c_int
        _HIP.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p,
                                                 ctypes.c_uint]
    p = ctypes.c_void_p()
    rc = _HIP.hipHostGetDevicePointer(ctypes.byref(p), ctypes.c_void_p(t.data_ptr()), 0)
    assert rc == 0 and p.value, f"hipHostGetDevicePointer failed ({rc})"
    return p.value


def pinned_layer(d):
    """The layer with its routed experts in pinned host memory (the tier's backing store,
    passed as device-side addresses), the rest on the device."""
    ts = {}
    for k in M.TENSORS:
        v = d.get(k)
        if v is None:
            continue
        t = torch.from_numpy(np.ascontiguousarray(v))
        ts[k] = t.pin_memory() if k in ROUTED else t.to(DEV)
    layer = M.Layer(d, ts)
    for name in ("gate", "up", "down"):
        assert ts[name + "_q"].is_pinned() and ts[name + "_s"].is_pinned()
        setattr(layer.c, name, M.Q4(device_address(ts[name + "_q"]), device_address(ts[name + "_s"])))
    return layer


def check_state(tier, ref, what):
    st, r = tier.read_state(), ref.state()
    for key in ("step", "hits", "misses", "swaps", "prefetched"):
        assert st[key] == r[key], (what, key, st[key], r[key])
    for key in ("slot_expert", "slot_pinned", "slot_used", "expert_slot", "heat", "usage"):
        np.testing.assert_array_equal(st[key], np.asarray(r[key]), err_msg=f"{what}: {key}")
    assert st["copies"] == r["copies"], (what, st["copies"], r["copies"])


def route_counts(d, x):
    ids, _, keff = R.route(R.Layer(d), x)
    off = R.union(d["n_experts"], ids, keff)["off"]
    counts = {e: int(off[e + 1] - off[e]) for e in range(d["n_experts"]) if off[e + 1] > off[e]}
    return counts, ids, keff


def run_sequence(sh, d, n_slots, pins, Ts, dtype=M.MOE_F32):
    E = sh.n_experts
    dev_layer = M.Layer.from_host(d, DEV)
    tier = M.Tier(pinned_layer(d), n_slots, len(pins))
    tier.init(pins)
    ref = TierRef(E, n_slots, pins)
    check_state(tier, ref, "init")
    for i, T in enumerate(Ts):
        x = S.tokens(sh, T, seed=0, pool=i)
        xd = torch.from_numpy(x).to(DEV)
        a = M.moe_layer_forward(dev_layer, xd, out_dtype=dtype)
        b = tier.forward(xd, out_dtype=dtype)
        torch.cuda.synchronize()
        assert torch.equal(a, b), f"step {i} T={T}: tier output differs from the resident layer"
        counts, _, _ = route_counts(d, x)
        ref.forward(counts)
        check_state(tier, ref, f"step {i} T={T}")
        if i % 4 == 3:
            tier.repin(4)
            ref.repin(4)
            check_state(tier, ref, f"repin after step {i}")
        if i % 3 == 2 and i + 1 < len(Ts):
            xn = S.tokens(sh, Ts[i + 1], seed=0, pool=i + 1)
            _, ids, keff = route_counts(d, xn)
            tier.prefetch(torch.from_numpy(ids).to(DEV), torch.from_numpy(keff).to(DEV))
            ref.prefetch([int(ids[t, j]) for t in range(ids.shape[0]) for j in range(keff[t])])
            check_state(tier, ref, f"prefetch after step {i}")
    st = tier.read_state()
    say(f"{sh.name}: {len(Ts)} batches, hits {st['hits']}, misses {st['misses']}, "
        f"swaps {st['swaps']}, prefetched {st['prefetched']}")
    return st


def test_tier_evictions_gemv_path():
    """64 experts, 24 slots (4 pinned), 1-5 tokens per batch with spread-out routing (logits
    ~N(0,1), small bias): misses evict LRU slots and prefetches copy experts in."""
    sh = S.custom("tier_ev", hidden=256, n_experts=64, ffn=128, shared_ffn=64, top_k=4, tokens=5,
                  bias_amp=0.02, router_std=1 / 16.0, top_p=0.9)
    d = S.make_layer(sh, seed=0)
    st = run_sequence(sh, d, 24, [3, 17, 40, 63], [1, 2, 3, 5, 1, 4, 2, 5, 3, 1, 5, 2, 4, 4, 1])
    assert st["misses"] > 20 and st["prefetched"] > 0


def test_tier_matrix_core_path():
    """32 experts, 40 slots (4 pinned), 9-40 tokens per batch (select+union kernel, union
    kernel, matrix-core expert FFNs), bf16 output."""
    sh = S.custom("tier_mfma", hidden=320, n_experts=32, ffn=192, shared_ffn=64, top_k=4, tokens=40,
                  bias_amp=0.2)
    d = S.make_layer(sh, seed=0)
    run_sequence(sh, d, 40, [0, 9, 20, 31], [9, 40, 16, 24, 40, 12], dtype=M.MOE_BF16)


@pytest.mark.timeout(600)
def test_tier_glm_decode():
    """The GLM-shaped layer (257 experts of 21.2 MB in pinned host memory), 24 HBM slots of
    which 8 pinned, one-token decode plus one 8-token batch."""
    sh = S.SHAPES["glm_decode"]
    say("GLM-shaped bank in pinned host memory")
    d = S.make_layer(sh, seed=0)
    run_sequence(sh, d, 24, [5, 50, 100, 150, 200, 250, 7, 77], [1] * 7 + [2] + [1] * 4,
                 dtype=M.MOE_BF16)


@pytest.mark.parametrize("fmt", [S.FMT_MXFP4, S.FMT_INT3], ids=["mxfp4", "int3"])
def test_tier_other_formats(fmt):
    """The tier over MXFP4 and int3-g64 experts: slots sized for the format, copies of
    the format's bytes; GEMV (1-4 tokens) and matrix-core (9-40 tokens) batches."""
    sh = S.custom(f"tier_{S.FMT_NAMES[fmt]}", hidden=320, n_experts=32, ffn=192, shared_ffn=64,
                  top_k=4, tokens=40, bias_amp=0.05, router_std=1 / 16.0, expert_fmt=fmt)
    d = S.make_layer(sh, seed=0)
    st = run_sequence(sh, d, 40, [0, 9, 20, 31], [1, 3, 9, 40, 2, 16, 4, 24, 1])
    assert st["misses"] > 0


def test_tier_rejects_a_too_small_cache():
    sh = S.custom("tier_small", hidden=256, n_experts=64, ffn=128, shared_ffn=64, top_k=4, tokens=8)
    d = S.make_layer(sh, seed=0)
    tier = M.Tier(pinned_layer(d), 10, 2)
    tier.init([1, 2])
    x = torch.from_numpy(S.tokens(sh, 3, seed=0)).to(DEV)  # 12 picks > 8 free slots
    with pytest.raises(M.MoeError) as ei:
        tier.forward(x)
    assert ei.value.code == M.MOE_EUNSUPPORTED
    assert tier.read_state()["step"] == 0

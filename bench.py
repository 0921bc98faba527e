#!/usr/bin/env python3
"""Throughput of the sparse MoE layer forward on one MI355X.

A step is one whole layer forward (router, selection, union, int4-gs64 expert
FFNs, combine + shared expert) on one batch of synthetic tokens that are
already resident in HBM.  The headline workload (``value``) is the
GLM-5.2-shaped decode layer: H=6144, 256 routed experts (F=2048) + 1 shared
expert (Fs=2048), top-8, norm_topk, routed scale 2.5, one token per step, bf16
output.  Each step uses another token of a 64-token pool and another of several
resident copies of the layer (distinct HBM, experts permuted per copy), so
neither the routed experts nor the shared expert and router can be served from
the 256 MB last-level cache.

By default every workload is measured in the same run and reported under
``workloads`` in the one JSON line (small-expert decode, 512-token prefill,
the 16-layer stack and the compute-bound grouped-GEMM microbenchmark), each with
its step time (eager, per-step median/p10/p90, graph replay, cache-hot where it
applies), the roofline of its dominant kernel and MFMA utilisation.
``--workload NAME`` measures one workload only.  Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + achieved HBM GB/s (decode) / MFMA util (prefill), 1 GPU"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_FLOPS = 2.5e15   # dense bf16 MFMA (the peak the utilisation target names)
I8_PEAK_OPS = 5.0e15       # dense int8 MFMA (the arithmetic the matrix-core path runs)
F64_PEAK_FLOPS = 78.6e12   # dense fp64 MFMA (the router's matrix-core path for T > 8)

WORKLOADS = {
    "glm_decode": "MoE layer H=6144, 256 routed experts F=2048 + 1 shared Fs=2048, int4-gs64, "
                  "top-8 noaux_tc, norm_topk, routed_scale 2.5, 1 token/step, bf16 out",
    "small_decode": "MoE layer H=2048, 256 routed experts F=512 + 1 shared Fs=512, int4-gs64, top-8, "
                    "norm_topk, 64 tokens/step, fp32 out",
    "glm_prefill": "the GLM-shaped layer, 512 tokens/step whose router logits are a popularity-skewed "
                   "Gumbel sample (union ~200 experts), fp32 out",
    "glm_stack16": "16 GLM-shaped layers resident (distinct HBM), 32 tokens/step, top-p 0.7, "
                   "Zipf(1.1) bias, RMSNorm + residual between layers, fp32",
    "glm_rows256": "grouped-GEMM microbenchmark: 16 GLM-shaped experts + shared, 512 tokens top-8 "
                   "(~256 rows per expert), fp32 out",
    "glm_prefill_act8": "glm_prefill with the opt-in 8-bit activations (int8 codes per 256-value "
                        "block, one int8 product per group)",
    "glm_verify16": "the GLM-shaped decode layer on 16 tokens per step (a multi-token verification "
                    "or small prefill chunk: 1-2 rows per union expert), fp32 out",
    "glm_decode_int3": "glm_decode with int3-g64 experts (3-bit codes in two bit planes, fp32 scale "
                       "per 64)",
    "glm_decode_mxfp4": "glm_decode with MXFP4 experts (E2M1 codes, UE8M0 exponent per 32)",
    "glm_prefill_int3": "glm_prefill with int3-g64 experts",
    "glm_prefill_mxfp4": "glm_prefill with MXFP4 experts (bf16 matrix cores, two-term activations)",
}
DEFAULT_ORDER = ("glm_decode", "small_decode", "glm_verify16", "glm_prefill", "glm_prefill_act8",
                 "glm_stack16", "glm_rows256", "glm_decode_int3", "glm_decode_mxfp4",
                 "glm_prefill_int3", "glm_prefill_mxfp4")
# resident layer copies cycled per step (enough distinct HBM to defeat the last-level cache)
COPIES = {"glm_decode": 8, "small_decode": 8, "glm_prefill": 2, "glm_stack16": 16, "glm_rows256": 2,
          "glm_prefill_act8": 2, "glm_verify16": 8, "glm_decode_int3": 8, "glm_decode_mxfp4": 8,
          "glm_prefill_int3": 2, "glm_prefill_mxfp4": 2}
# workload-name suffixes: the opt-in 8-bit activations, or another expert format
SUFFIX_FMT = {"_int3": 2, "_mxfp4": 1}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def mat_bytes(fmt, n, k):
    """Codes + scales of an [n][k] matrix: int4-gs64 (4 bits + fp32 per 64), MXFP4 (4 bits +
    one byte per 32), int3-g64 (3 bits + fp32 per 64)."""
    if fmt == 1:
        return n * k // 2 + n * (k // 32)
    if fmt == 2:
        return n * 3 * k // 8 + n * (k // 64) * 4
    return n * k // 2 + n * (k // 64) * 4


def host_cpu():
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model


_BANKS = {}


def bank_for(sh):
    """The host expert bank of a shape (cached: the GLM-shaped workloads share one)."""
    from routed_int4_expert_amd import synth as S
    key = (sh.bank or sh.name, sh.n_experts, sh.hidden, sh.ffn, sh.shared_ffn, sh.expert_fmt)
    if key not in _BANKS:
        t0 = time.time()
        _BANKS[key] = S.Bank(sh, seed=0)
        log(f"expert bank {key[0]} x{sh.n_experts} generated on the host in {time.time() - t0:.1f} s")
    return _BANKS[key]


def build_layers(sh, n_layers, dev, shared_router=False, act_bits=0):
    """n_layers resident copies of the layer: distinct HBM, experts permuted per copy.
    With shared_router every copy uses copy 0's router (the prefill tokens are built
    for that router)."""
    import torch
    import routed_int4_expert_amd as M
    from routed_int4_expert_amd import synth as S

    bank = bank_for(sh)
    base = {k: torch.from_numpy(getattr(bank, k)).to(dev) for k in S.Bank.ROUTED + S.Bank.SHARED}
    layers, routers = [], []
    for l in range(n_layers):
        rw, rb = S.router(sh, 0, 0 if shared_router else l)
        perm = torch.from_numpy(S.layer_perm(sh, 0, l)).to(dev)
        ts = {k: base[k].index_select(0, perm) for k in S.Bank.ROUTED}
        ts.update({k: base[k].clone() for k in S.Bank.SHARED})
        ts["router_w"] = torch.from_numpy(rw).to(dev)
        ts["router_bias"] = torch.from_numpy(rb).to(dev)
        layers.append(M.Layer({**S.layer_params(sh), "act_bits": act_bits}, ts))
        routers.append((rw, rb))
    del base
    torch.cuda.synchronize()
    gb = n_layers * (sh.n_experts + 1) * S.expert_bytes(sh) / 1e9
    log(f"{sh.name}: {n_layers} resident layer copies ready ({gb:.1f} GB of experts)")
    return bank, layers, routers


def cpu_baseline(sh, bank, routers, xs_host, seconds):
    """The CPU oracle (plain C, fp64) on single-token forwards of the same layer copies:
    with the host's OpenMP threads over FFN rows, then on one thread."""
    import oracle as R
    from routed_int4_expert_amd import synth as S

    # layer copy 0 (its experts are the bank's own arrays: no host copy)
    d = S.make_layer(sh, seed=0, layer=0, bank=bank)
    d["router_w"], d["router_bias"] = routers[0]
    Ls = [R.Layer(d)]

    def run(budget):
        n, t0 = 0, time.time()
        while n == 0 or time.time() - t0 < budget:
            i = n % xs_host.shape[0]
            R.layer_forward(Ls[n % len(Ls)], xs_host[i:i + 1])
            n += 1
        return n, time.time() - t0

    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    n, dt = run(seconds)
    rec = dict(value=n / dt, unit="tokens/s", cores=cores, kind="oracle",
               sample=f"{n} single-token forwards of the GLM-shaped decode layer (copy 0), {dt:.1f} s, "
                      f"fp64 C oracle with OpenMP over FFN rows ({cores} threads)",
               cpu_model=host_cpu(), host_cpus_visible=os.cpu_count())
    try:  # one thread: the oracle's OpenMP runtime is the process's libgomp
        gomp = ctypes.CDLL("libgomp.so.1")
        gomp.omp_set_num_threads(1)
        n1, dt1 = run(seconds / 2)
        gomp.omp_set_num_threads(cores)
        rec["single_thread"] = dict(value=n1 / dt1, unit="tokens/s", cores=1,
                                    sample=f"{n1} single-token forwards, {dt1:.1f} s, one thread")
    except OSError:
        pass
    return rec


def counted_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    runs (profiles/hbm_counters.json, calibrated against a copy of known size), or None
    when there is none for this workload or the kernel's source changed since."""
    try:
        with open(os.path.join(ROOT, "profiles", "hbm_counters.json")) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    for e in data.get("entries", []):
        if e.get("workload") != workload or e.get("kernel") != kernel:
            continue
        # every source file of the kernel and its launch unchanged since the counters
        for src, sha in zip(e.get("sources", []), e.get("sources_sha256", [])):
            try:
                with open(os.path.join(ROOT, src), "rb") as f:
                    if hashlib.sha256(f.read()).hexdigest() != sha:
                        return None
            except OSError:
                return None
        if not e.get("sources"):
            return None
        return float(e["hbm_bytes_per_launch"])
    return None


def read_probe(gib=4.0, reps=10):
    """The practical HBM read ceiling: moe_probe_read over a `gib` GiB buffer, timed with
    HIP events on the launch stream; the best of a few grid sizes."""
    import torch
    import routed_int4_expert_amd as M
    nbytes = int(gib * (1 << 30))
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda:0")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    st = torch.cuda.current_stream()
    sp = ctypes.c_void_p(st.cuda_stream)
    best = None
    for blocks in (2048, 4096, 8192):
        def go():
            rc = M.lib().moe_probe_read(ctypes.c_void_p(buf.data_ptr()), nbytes, 0x9E3779B9,
                                        ctypes.c_void_p(sink.data_ptr()), blocks, sp)
            if rc != M.MOE_OK:
                raise M.MoeError(rc, "moe_probe_read")
        go()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            go()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        gbps = nbytes / (ms * 1e-3) / 1e9
        if best is None or gbps > best["read_gbps"]:
            best = dict(read_gbps=gbps, bytes=nbytes, blocks=blocks, ms=ms)
    del buf
    torch.cuda.empty_cache()
    best["frac_of_peak"] = best["read_gbps"] / HBM_PEAK_GBPS
    return best


def pct(a, q):
    return float(np.percentile(np.asarray(a, dtype=np.float64), q))


def run_workload(wl, args, dev):
    """Measure one workload; returns its record (the fields of the JSON line)."""
    import torch
    import routed_int4_expert_amd as M
    from routed_int4_expert_amd import synth as S

    import dataclasses
    act_bits = 8 if wl.endswith("_act8") else 0
    fmt = next((f for suf, f in SUFFIX_FMT.items() if wl.endswith(suf)), 0)
    base_wl = wl
    for suf in ("_act8",) + tuple(SUFFIX_FMT):
        if base_wl.endswith(suf):
            base_wl = base_wl[:-len(suf)]
    if base_wl == "glm_verify16":
        sh = dataclasses.replace(S.SHAPES["glm_decode"], tokens=16)
    else:
        sh = S.SHAPES[base_wl]
    sh = dataclasses.replace(sh, expert_fmt=fmt)
    T, H, F, Fs, E = sh.tokens, sh.hidden, sh.ffn, sh.shared_ffn, sh.n_experts
    stack = wl == "glm_stack16"
    nlay = COPIES[wl] if args.layers is None else (sh.layers if stack else args.layers)
    bank, layers, routers = build_layers(sh, nlay, dev, shared_router=(base_wl == "glm_prefill"),
                                         act_bits=act_bits)
    if base_wl == "glm_prefill":
        npool = 2
        xs_host = np.concatenate([S.gumbel_skew_batch(sh, T, routers[0][0], routers[0][1], 0, p)[0]
                                  for p in range(npool)])
    else:
        npool = max(1, 64 // T)
        xs_host = S.tokens(sh, npool * T, seed=0, pool=0)
    xpool = torch.from_numpy(xs_host).to(dev)
    out_bf16 = base_wl == "glm_decode"
    out = torch.empty((T, H), dtype=torch.bfloat16 if out_bf16 else torch.float32, device=dev)
    ws = layers[0].workspace(T, dev)
    per_step = nlay if stack else 1
    n_pct = max(args.steps, 30)
    nrec = (args.warmup + args.steps + args.steps + n_pct + 2) * per_step
    nu = torch.zeros((nrec,), dtype=torch.int32, device=dev)
    offb = torch.zeros((nrec, E + 1), dtype=torch.int32, device=dev)
    hbuf = torch.empty((T, H), dtype=torch.float32, device=dev)
    xbuf = torch.empty((T, H), dtype=torch.float32, device=dev)

    fwd = M.lib().moe_layer_forward
    glue = M.lib().moe_residual_rmsnorm
    xptr = [ctypes.c_void_p(xpool.data_ptr() + (i * T * H * 4)) for i in range(npool)]
    dbgs = [M.RouteOutC(n_uniq=nu.data_ptr() + 4 * r, off=offb.data_ptr() + 4 * (E + 1) * r)
            for r in range(nrec)]
    refs = [lay.ref() for lay in layers]
    outp, wsp, wsn = ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws.numel()
    hp, xp = ctypes.c_void_p(hbuf.data_ptr()), ctypes.c_void_p(xbuf.data_ptr())
    odt = M.MOE_BF16 if out_bf16 else M.MOE_F32

    def check(rc, what):
        if rc != M.MOE_OK:
            raise M.MoeError(rc, what)

    def step(i, rec, stream, copy=None, tok=None):
        """Step i: layer copy i mod copies, token batch i mod pool (unless pinned)."""
        c = i % len(refs) if copy is None else copy
        b = i % npool if tok is None else tok
        if not stack:
            check(fwd(refs[c], xptr[b], T, outp, odt, ctypes.byref(dbgs[rec]), wsp, wsn, stream),
                  "moe_layer_forward")
            return
        # the stack: h = tokens; per layer x = RMSNorm(h); out = MoE(x); h += out (next glue)
        check(glue(xptr[b], None, T, H, ctypes.c_float(1e-6), hp, xp, stream), "glue")
        for l in range(nlay):
            if l > 0:
                check(glue(hp, outp, T, H, ctypes.c_float(1e-6), hp, xp, stream), "glue")
            check(fwd(refs[l], xp, T, outp, odt, ctypes.byref(dbgs[rec * nlay + l]), wsp, wsn,
                      stream), "moe_layer_forward")

    cur = torch.cuda.current_stream()
    stream = ctypes.c_void_p(cur.cuda_stream)
    rec = 0
    for i in range(args.warmup):
        step(i, rec, stream)
        rec += 1
    torch.cuda.synchronize()
    log(f"{wl}: warmup {args.warmup} steps done")

    # timed region: K steps bracketed by synchronisation and HIP events on the launch stream
    s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s_ev.record()
    rec0 = rec
    for i in range(args.steps):
        step(args.warmup + i, rec, stream)
        rec += 1
    e_ev.record()
    torch.cuda.synchronize()
    ms_step = s_ev.elapsed_time(e_ev) / args.steps
    stat_sl = slice(rec0 * per_step, rec * per_step)
    log(f"{wl}: timed {args.steps} steps: {ms_step * 1e3:.1f} us/step")

    # per-step HIP events (distribution)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_pct)]
    for i in range(n_pct):
        evs[i][0].record()
        step(args.warmup + i, rec, stream)
        evs[i][1].record()
        rec += 1
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in evs]

    # per-kernel HIP events on the launch stream (the same steps again)
    M.moe_prof_begin()
    for i in range(args.steps):
        step(args.warmup + i, rec, stream)
        rec += 1
    kern = M.moe_prof_end()
    torch.cuda.synchronize()

    # graph replay: G consecutive steps captured once, replayed
    G = 8 if T * per_step <= 64 and not stack else 1
    graph_ms = None
    try:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            step(0, rec, ctypes.c_void_p(side.cuda_stream))
        cur.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            cs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for i in range(G):
                step(i, rec, cs)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        reps = max(1, args.steps // G)
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(reps):
            g.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / (reps * G)
        del g
    except Exception as exc:  # graph timing is reported when it works, never required
        log(f"{wl}: graph replay not timed ({exc})")

    # cache-hot: one layer copy and one batch every step (the weights stay in the caches
    # as far as they fit)
    hot_ms = None
    if not stack:
        for i in range(3):
            step(0, rec, stream, copy=0, tok=0)
        h0, h1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        h0.record()
        for i in range(args.steps):
            step(0, rec, stream, copy=0, tok=0)
        h1.record()
        torch.cuda.synchronize()
        hot_ms = h0.elapsed_time(h1) / args.steps

    n_uniq = nu[stat_sl].cpu().numpy().astype(np.float64)
    rows = offb[stat_sl, E].cpu().numpy().astype(np.float64)
    exp_b, sh_b = S.expert_bytes(sh), S.expert_bytes(sh, Fs)
    # algorithmic bytes and flops per step: union experts + shared expert + router + x + out
    step_bytes = per_step * (n_uniq.mean() * exp_b + sh_b + E * H * 4 + E * 4 + T * H * 4
                             + T * H * (2 if out_bf16 else 4))
    step_flops = per_step * (2.0 * 3 * H * F * rows.mean() + 2.0 * 3 * H * Fs * T + 2.0 * T * E * H)
    ffn_flops = per_step * (2.0 * 3 * H * (F * rows.mean() + Fs * T))
    gemv = T <= 4
    kernels = {}
    # gate/up: every unit's codes + scales, x read, h written; down: codes + scales, h read, y written
    units = {
        "gateup": dict(name="ffn_gateup" if gemv else "ffn_gateup_mfma",
                       bytes=(n_uniq.mean() * 2 * mat_bytes(fmt, F, H) + 2 * mat_bytes(fmt, Fs, H) + T * H * 4
                              + (rows.mean() * F + T * Fs) * 4),
                       flops=2.0 * 2 * H * (F * rows.mean() + Fs * T)),
        "down": dict(name="ffn_down" if gemv else "ffn_down_mfma",
                     bytes=(n_uniq.mean() * mat_bytes(fmt, H, F) + mat_bytes(fmt, H, Fs)
                            + (rows.mean() * F + T * Fs) * 4 + (rows.mean() + T) * H * 4),
                     flops=2.0 * H * (F * rows.mean() + Fs * T)),
    }
    for role, u in units.items():
        launches, ms = kern.get(u["name"], (0, float("nan")))
        avg = ms / max(launches, 1)
        ach = u["bytes"] / (avg * 1e-3) / 1e9
        kernels[role] = {
            "kernel": u["name"], "bound": "hbm", "achieved": float(ach), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": float(ach / HBM_PEAK_GBPS),
            "traffic": counted_traffic(wl, u["name"]),
            "bytes_per_launch": float(u["bytes"]), "avg_launch_us": float(avg * 1e3),
            "useful_tflops": float(u["flops"] / (avg * 1e-3) / 1e12),
            "mfma_util_vs_bf16_dense": float(u["flops"] / (avg * 1e-3) / BF16_PEAK_FLOPS),
            "mfma_util_vs_i8_dense": float(u["flops"] / (avg * 1e-3) / I8_PEAK_OPS),
        }
    gu = kernels["gateup"]
    rec_out = {
        "metric": METRIC,
        "value": T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the expert FFNs' arithmetic: int4 codes times 16-bit fixed-point activations
        # (carried as two int8 limbs; one int8 code with the opt-in 8-bit path) with exact
        # int32 group sums (v_dot4 in the decode GEMV for T <= 4, int8 matrix cores for
        # T > 4), then fp32 accumulation
        # (int3 codes likewise, and doubled E2M1 values on the GEMV; MXFP4 above 4 tokens:
        # exact bf16 weights times two bf16 terms per activation on the bf16 matrix cores,
        # fp32 accumulation)
        "dtype": ("i4xi8-i32-f32acc" if act_bits else
                  {0: "i4xfx16-i32-f32acc", 2: "i3xfx16-i32-f32acc"}.get(fmt) or
                  ("e2m1xfx16-i32-f32acc" if T <= 4 else "e2m1xbf16x2-f32acc")),
        "data": "synthetic",
        "config": {
            "workload": f"{wl}: {WORKLOADS[wl]}",
            "tokens_per_step": T,
            "layers_per_step": per_step,
            "layer_copies_cycled": nlay,
            "mean_union_experts": float(n_uniq.mean()),
            "mean_routed_rows": float(rows.mean()),
            "algorithmic_bytes_per_step": float(step_bytes),
            "algorithmic_flops_per_step": float(step_flops),
        },
        "timing": {
            "eager_ms_per_step": ms_step,
            "median_ms": pct(per, 50), "p10_ms": pct(per, 10), "p90_ms": pct(per, 90),
            "per_step_samples": n_pct,
            "graph_replay_ms_per_step": graph_ms,
            "graph_steps_per_replay": G,
            "cache_hot_ms_per_step": hot_ms,
        },
        "step_roofline": {
            "hbm_gbps": float(step_bytes / (ms_step * 1e-3) / 1e9),
            "frac_of_hbm_peak": float(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS),
            "useful_tflops": float(step_flops / (ms_step * 1e-3) / 1e12),
            "ffn_mfma_util_vs_bf16_dense": float(ffn_flops / (ms_step * 1e-3) / BF16_PEAK_FLOPS),
        },
        "roofline": {
            "kernel": f"{gu['kernel']} (gate+up of every union expert and the shared expert, "
                      "SiLU*up epilogue)",
            "bound": "hbm", "achieved": gu["achieved"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": gu["frac"], "traffic": gu["traffic"],
            "bytes_per_launch": gu["bytes_per_launch"], "avg_launch_us": gu["avg_launch_us"],
            "mfma_util_vs_bf16_dense": gu["mfma_util_vs_bf16_dense"],
            "mfma_util_vs_i8_dense": gu["mfma_util_vs_i8_dense"],
        },
        "kernel_rooflines": kernels,
        "kernels_us_per_step": {kname: v[1] * 1e3 / args.steps for kname, v in kern.items()},
        "other_kernels": other_kernels(kern, T, H, E, sh.top_k, rows.mean(), out_bf16),
    }
    # the bars the layer is held to: a step at 0.70 of the HBM peak on its algorithmic bytes;
    # where rows per expert make the FFN compute-bound, half the dense bf16 peak in useful flops
    frac_step = rec_out["step_roofline"]["frac_of_hbm_peak"]
    rec_out["target"] = {"hbm_frac_of_step_needed": 0.70, "hbm_frac_of_step": frac_step,
                         "ms_per_step_at_target": float(step_bytes / (0.70 * HBM_PEAK_GBPS * 1e9) * 1e3),
                         "met": bool(frac_step >= 0.70)}
    if wl == "glm_rows256":
        util = kernels["gateup"]["mfma_util_vs_bf16_dense"]
        rec_out["target"].update(bf16_util_needed=0.5, gateup_bf16_util=util, met=bool(util >= 0.5))
    if wl == "glm_prefill" and not args.no_subsets:
        sub = compute_subsets(layers[0], xpool[:T], args.steps)
        rec_out["compute_bound_subsets"] = sub
        best = max(v["ffn_util_vs_bf16_dense"] for v in sub.values() if isinstance(v, dict))
        rec_out["target"].update(bf16_util_needed_on_compute_bound_subsets=0.5,
                                 best_subset_bf16_util=best)
    extra = dict(bank=bank, routers=routers, xs_host=xs_host, sh=sh)
    del layers, ws, xpool, out, hbuf, xbuf, nu, offb
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec_out, extra


def other_kernels(kern, T, H, E, k, rows, out_bf16):
    """The router and the combine against their own bounds: the router's fp32 weight rows
    and tokens (HBM; for more than 8 tokens also the fp64 matrix cores, T*E*H products),
    the combine's routed rows, shared rows and output (HBM)."""
    res = {}
    launches, ms = kern.get("router_logits", (0, float("nan")))
    if launches:
        us = ms * 1e3 / launches
        b = E * H * 4 + T * H * 4
        r = {"avg_launch_us": us, "bytes_per_launch": float(b),
             "hbm_frac": b / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS}
        if T > 8:
            r["fp64_util"] = 2.0 * T * E * H / (us * 1e-6) / F64_PEAK_FLOPS
        res["router_logits"] = r
    launches, ms = kern.get("combine", (0, float("nan")))
    if launches:
        us = ms * 1e3 / launches
        b = rows * H * 4 + T * H * 4 + T * H * (2 if out_bf16 else 4) + T * k * 8
        res["combine"] = {"avg_launch_us": us, "bytes_per_launch": float(b),
                          "hbm_frac": b / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS}
    return res


def compute_subsets(layer, x, reps, min_rows=88):
    """Matrix-core utilisation where the prefill's expert FFNs are compute-bound.

    With about 16 rows per union expert most of the prefill layer streams weights, so
    its FFN time is bound by HBM.  Three subsets have enough rows per weight byte to be
    bound by the matrix cores instead, and each is timed alone with per-kernel HIP events:
    the routed experts that the batch gives at least ``min_rows`` rows (their rows only,
    through moe_expert_ffn), the shared expert on all of the batch's tokens
    (moe_dense_forward with the shared weights), and a grouped GEMM of the batch's eight
    most-used experts with every token routed to each of them (R_e = T rows each).
    Useful flops are 2*H*F per row for each of gate, up and down; the int8 matrix cores
    run two limb products per useful product, so their issue rate is twice the useful one."""
    import torch
    import routed_int4_expert_amd as M

    T, H, E, k = x.shape[0], layer.hidden, layer.n_experts, layer.top_k
    F = layer.c.ffn
    dev = x.device
    ws = layer.workspace(T, dev)
    ids, _w, keff = M.moe_route(layer, x, ws=ws)
    un = M.moe_union(layer, ids, keff, ws=ws)
    torch.cuda.synchronize()
    off = un["off"].cpu().numpy().astype(np.int64)
    row_tok = un["row_tok"].cpu().numpy()
    cnt = np.diff(off)

    def union_of(experts, rows_of):
        experts = sorted(experts)
        c = np.zeros(E, dtype=np.int64)
        rt = []
        for e in experts:
            r = rows_of(e)
            c[e] = len(r)
            rt.append(r)
        o = np.concatenate([[0], np.cumsum(c)]).astype(np.int32)
        rt = np.concatenate(rt).astype(np.int32) if rt else np.zeros(0, np.int32)
        u = np.full(E, -1, np.int32)
        u[:len(experts)] = experts
        nrows = int(o[-1])
        rtp = np.full(max(T * k, nrows, 1), -1, np.int32)
        rtp[:nrows] = rt
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        return dict(n_uniq=t(np.array([len(experts)], np.int32)), uniq=t(u), off=t(o), row_tok=t(rtp)), nrows

    def timed(fn, rows, ffn):
        fn()
        torch.cuda.synchronize()
        M.moe_prof_begin()
        for _ in range(reps):
            fn()
        kern = M.moe_prof_end()
        torch.cuda.synchronize()
        res = {"rows": int(rows)}
        tot_flops, tot_ms = 0.0, 0.0
        for role, name in (("gateup", "ffn_gateup_mfma"), ("down", "ffn_down_mfma")):
            launches, ms = kern.get(name, (0, float("nan")))
            us = ms * 1e3 / max(launches, 1)
            flops = 2.0 * H * ffn * rows * (2 if role == "gateup" else 1)
            tot_flops += flops
            tot_ms += ms / max(launches, 1)
            res[role] = {"kernel": name, "avg_launch_us": float(us),
                         "useful_tflops": float(flops / (us * 1e-6) / 1e12),
                         "util_vs_bf16_dense": float(flops / (us * 1e-6) / BF16_PEAK_FLOPS),
                         "i8_issue_util": float(2 * flops / (us * 1e-6) / I8_PEAK_OPS)}
        res["ffn_useful_tflops"] = float(tot_flops / (tot_ms * 1e-3) / 1e12)
        res["ffn_util_vs_bf16_dense"] = float(tot_flops / (tot_ms * 1e-3) / BF16_PEAK_FLOPS)
        return res

    out = {"min_rows": min_rows}
    hot = [int(e) for e in np.nonzero(cnt >= min_rows)[0]]
    if hot:
        sub, nrows = union_of(hot, lambda e: row_tok[off[e]:off[e + 1]])
        y = torch.zeros((max(T * k, nrows), H), dtype=torch.float32, device=dev)
        r = timed(lambda: M.moe_expert_ffn(layer, x, sub, y_rows=y, ws=ws), nrows, F)
        r["experts"] = len(hot)
        r["rows_per_expert"] = [int(cnt[e]) for e in hot]
        out["experts_ge_min_rows"] = r
    top8 = [int(e) for e in np.argsort(-cnt, kind="stable")[:8]]
    sub, nrows = union_of(top8, lambda e: np.arange(T))
    y = torch.zeros((nrows, H), dtype=torch.float32, device=dev)
    r = timed(lambda: M.moe_expert_ffn(layer, x, sub, y_rows=y, ws=ws), nrows, F)
    r["experts"] = len(top8)
    r["rows_per_expert"] = T
    out["grouped_gemm_all_tokens"] = r
    dense = M.Dense({kk: layer.t["sh_" + kk] for kk in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")})
    dws = dense.workspace(T, dev)
    yd = torch.empty((T, H), dtype=torch.float32, device=dev)
    r = timed(lambda: M.moe_dense_forward(dense, x, out=yd, ws=dws), T, dense.ffn)
    r["shared_ffn"] = dense.ffn
    out["shared_expert"] = r
    del ws, dws, y, yd
    return out


def _device_address(t):
    """Device-side address of a pinned host tensor (hipHostGetDevicePointer)."""
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipHostGetDevicePointer.restype = ctypes.c_int
    hip.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_uint]
    p = ctypes.c_void_p()
    if hip.hipHostGetDevicePointer(ctypes.byref(p), ctypes.c_void_p(t.data_ptr()), 0) != 0 or not p.value:
        raise RuntimeError("hipHostGetDevicePointer failed")
    return p.value


TIER_WORKLOADS = {"glm_tier": 0, "glm_tier_mxfp4": 1, "glm_tier_int3": 2}


def run_tier(args, dev, fmt=0, n_layers=4, n_slots=200, n_pin=64):
    """Decode through n_layers GLM-shaped layers whose routed experts (5.4 GB each) live in
    pinned host memory, each layer with a residency tier of n_slots HBM slots (n_pin pinned,
    chosen from a usage warm-up).  200 of 256 slots per layer is the share of a 370 GB
    expert bank that 288 GB of HBM holds.  One token per step, Zipf-skewed routing with
    top-p 0.7.  Timed without and with router-lookahead prefetch (layer l+1's router on
    layer l's input, on a copy stream that runs beside layer l's forward), and with every
    expert resident in HBM for comparison."""
    import dataclasses
    import torch
    import routed_int4_expert_amd as M
    from routed_int4_expert_amd import synth as S

    sh = dataclasses.replace(S.SHAPES["glm_stack16"], name="glm_tier", tokens=1, layers=n_layers,
                             expert_fmt=fmt)
    wl = next(k for k, v in TIER_WORKLOADS.items() if v == fmt)
    T, H, E = 1, sh.hidden, sh.n_experts
    bank = bank_for(sh)
    t0 = time.time()
    layers, res_layers, tiers = [], [], []
    for l in range(n_layers):
        rw, rb = S.router(sh, 0, l)
        perm = S.layer_perm(sh, 0, l)
        host = bank.permuted(perm)
        ts = {k: torch.from_numpy(host[k]).pin_memory() for k in S.Bank.ROUTED}
        del host
        ts.update({k: torch.from_numpy(getattr(bank, k)).to(dev) for k in S.Bank.SHARED})
        ts["router_w"], ts["router_bias"] = torch.from_numpy(rw).to(dev), torch.from_numpy(rb).to(dev)
        lay = M.Layer(S.layer_params(sh), ts)
        for name in ("gate", "up", "down"):
            setattr(lay.c, name, M.Q4(_device_address(ts[name + "_q"]), _device_address(ts[name + "_s"])))
        layers.append(lay)
        rts = {k: v.to(dev) if k in S.Bank.ROUTED else v for k, v in ts.items()}
        res_layers.append(M.Layer(S.layer_params(sh), rts))
    log(f"{wl}: {n_layers} layers in pinned host memory "
        f"({n_layers * (E + 1) * S.expert_bytes(sh) / 1e9:.1f} GB) and resident copies ready in "
        f"{time.time() - t0:.1f} s")
    # a fresh token every step (no token repeats within a timed run): the experts a step
    # needs are not the ones a recent step already brought in
    npool = 1024
    xs = torch.from_numpy(S.tokens(sh, npool, seed=0)).to(dev)
    hbuf = torch.empty((T, H), dtype=torch.float32, device=dev)
    xbuf = [torch.empty((T, H), dtype=torch.float32, device=dev) for _ in range(n_layers)]
    out = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws = layers[0].workspace(T, dev)
    ws2 = layers[0].workspace(T, dev)
    pid = torch.empty((T, sh.top_k), dtype=torch.int32, device=dev)
    pw = torch.empty((T, sh.top_k), dtype=torch.float32, device=dev)
    pk = torch.empty((T,), dtype=torch.int32, device=dev)
    comp = torch.cuda.current_stream()
    copy = torch.cuda.Stream()

    def step(i, fwd_of, prefetch=False):
        x = xs[i % npool:i % npool + 1]
        M.moe_residual_rmsnorm(x, None, h_out=hbuf, x_out=xbuf[0])
        done = None  # the copy stream's event after layer l's own prefetch
        for l in range(n_layers):
            if l > 0:
                M.moe_residual_rmsnorm(hbuf, out, h_out=hbuf, x_out=xbuf[l])
            if prefetch and done is not None:
                comp.wait_event(done)  # layer l's prefetch, not the one enqueued below
            if prefetch and l + 1 < n_layers:
                ev = torch.cuda.Event()
                ev.record(comp)
                copy.wait_event(ev)
                with torch.cuda.stream(copy):
                    M.moe_route(layers[l + 1], xbuf[l], pid, pw, pk, ws=ws2, stream=copy)
                    tiers[l + 1].prefetch(pid, pk, stream=copy)
                done = torch.cuda.Event()
                done.record(copy)
            fwd_of(l, xbuf[l])
        if prefetch:
            comp.wait_stream(copy)

    def tier_fwd(l, x):
        tiers[l].forward(x, out=out, ws=ws)

    def res_fwd(l, x):
        M.moe_layer_forward(res_layers[l], x, out=out, ws=ws)

    # usage warm-up with unpinned tiers, then autopin the hottest experts of each layer
    warm = [M.Tier(layers[l], n_slots, 0) for l in range(n_layers)]
    for w in warm:
        w.init([])
    tiers[:] = warm
    for i in range(32):
        step(i, tier_fwd)
    pins = []
    for w in warm:
        u = w.read_state()["usage"].astype(np.int64)
        pins.append([int(e) for e in np.argsort(-u, kind="stable")[:n_pin]])
    del warm
    tiers[:] = [M.Tier(layers[l], n_slots, n_pin) for l in range(n_layers)]
    res = {}
    K = max(args.steps, 32)
    for mode in ("no_prefetch", "prefetch"):
        for l in range(n_layers):
            tiers[l].init(pins[l])
        torch.cuda.synchronize()
        # untimed steps that fill the cache past the pinned store (steady state)
        for i in range(max(args.warmup, 96)):
            step(200 + i, tier_fwd, prefetch=(mode == "prefetch"))
        torch.cuda.synchronize()
        st0 = [t.read_state() for t in tiers]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(K):
            step(400 + i, tier_fwd, prefetch=(mode == "prefetch"))
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / K
        st1 = [t.read_state() for t in tiers]
        hits = sum(b["hits"] - a["hits"] for a, b in zip(st0, st1))
        miss = sum(b["misses"] - a["misses"] for a, b in zip(st0, st1))
        pref = sum(b["prefetched"] - a["prefetched"] for a, b in zip(st0, st1))
        copied = (miss + pref) * S.expert_bytes(sh)  # misses found resident by a prefetch are not copied twice
        res[mode] = dict(ms_per_step=ms, tokens_per_s=T / (ms * 1e-3), hit_rate=hits / max(hits + miss, 1),
                         misses_per_step=miss / K, prefetched_per_step=pref / K,
                         host_copy_gbps=copied / (K * ms * 1e-3) / 1e9)
        log(f"{wl} {mode}: {ms * 1e3:.0f} us/step, hit rate {res[mode]['hit_rate']:.2f}, "
            f"{res[mode]['misses_per_step']:.1f} misses/step")
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(K):
        step(400 + i, res_fwd)
    e1.record()
    torch.cuda.synchronize()
    ms_res = e0.elapsed_time(e1) / K
    rec = {
        # the faster of the two modes (with synthetic routers the lookahead predicts the next
        # layer's picks poorly, and every wrong prediction costs a copy)
        "value": max(r["tokens_per_s"] for r in res.values()), "unit": "tokens/s",
        "ms_per_step": min(r["ms_per_step"] for r in res.values()),
        "config": {"workload": f"{wl}: {n_layers} GLM-shaped layers, {S.FMT_NAMES[fmt]} routed experts in "
                               f"pinned host memory ({n_layers * (E + 1) * S.expert_bytes(sh) / 1e9:.1f} GB), "
                               f"{n_slots} HBM slots per layer "
                               f"({n_pin} pinned from a usage warm-up), 1 token/step, top-p 0.7, "
                               "Zipf(1.1) bias",
                   "tokens_per_step": T, "layers_per_step": n_layers, "slots_per_layer": n_slots,
                   "pinned_per_layer": n_pin, "working_set_gb": n_layers * (E + 1) * S.expert_bytes(sh) / 1e9,
                   "cache_gb": n_layers * n_slots * S.expert_bytes(sh) / 1e9},
        "tier": res,
        "all_resident_ms_per_step": ms_res,
    }
    del layers, res_layers, tiers
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="all", choices=["all"] + sorted(TIER_WORKLOADS) + sorted(WORKLOADS))
    ap.add_argument("--layers", type=int, default=None,
                    help="resident layer copies cycled per step (default: per workload)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the streaming-read ceiling probe")
    ap.add_argument("--no-tier", action="store_true", help="skip the residency-tier workload")
    ap.add_argument("--no-subsets", action="store_true",
                    help="skip the prefill's compute-bound subsets (their launches would enter a profile of "
                         "the prefill's own kernels)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only copy a BYTES-long device buffer 13 times (calibrates the HBM "
                         "byte counters against a transfer of known size) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the layer forward "
              "is built and timed on a single MI355X.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_probe:
        n = args.copy_probe // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 10
        print(json.dumps({"copy_probe_bytes_read_per_copy": n * 4, "copies": 13,
                          "copy_ms": ms, "copy_read_plus_write_gbps": 2 * n * 4 / (ms * 1e-3) / 1e9}),
              flush=True)
        return

    dev = "cuda:0"
    torch.cuda.set_device(0)
    order = DEFAULT_ORDER if args.workload == "all" else (() if args.workload in TIER_WORKLOADS else (args.workload,))
    head, head_extra, subs = None, None, {}
    for wl in order:
        rec, extra = run_workload(wl, args, dev)
        if head is None:
            head, head_extra = rec, extra
        else:
            subs[wl] = {k: rec[k] for k in ("value", "unit", "ms_per_step", "dtype", "config", "timing",
                                            "step_roofline", "roofline", "kernel_rooflines",
                                            "kernels_us_per_step", "other_kernels", "target",
                                            "compute_bound_subsets")
                        if k in rec}
            log(f"{wl}: {rec['value']:.0f} tokens/s, {rec['ms_per_step'] * 1e3:.1f} us/step, "
                f"gate/up {rec['roofline']['frac']:.2f} of HBM peak")
    tiers = list(TIER_WORKLOADS) if args.workload == "all" else [w for w in TIER_WORKLOADS if w == args.workload]
    if not args.no_tier:
        for tw in tiers:
            log(f"{tw}: residency tier over pinned host memory")
            subs[tw] = run_tier(args, dev, fmt=TIER_WORKLOADS[tw])
    if head is None:  # a tier workload alone
        print(json.dumps(subs[tiers[0]]), flush=True)
        return
    if subs:
        head["workloads"] = subs
    if not args.no_probe:
        log("streaming-read ceiling probe")
        head["hbm_read_ceiling"] = read_probe()
        head["roofline"]["frac_of_read_ceiling"] = head["roofline"]["achieved"] / head["hbm_read_ceiling"]["read_gbps"]
    if not args.no_cpu_baseline and order[0] == "glm_decode":
        log(f"CPU baseline: oracle for ~{args.cpu_seconds:.0f} s (+ one thread)")
        head["cpu_baseline"] = cpu_baseline(head_extra["sh"], head_extra["bank"], head_extra["routers"],
                                            head_extra["xs_host"], args.cpu_seconds)
    print(json.dumps(head), flush=True)


if __name__ == "__main__":
    main()

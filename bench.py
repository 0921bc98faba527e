#!/usr/bin/env python3
"""Throughput of the sparse MoE layer forward on one MI355X.

A step is one whole layer forward (router, selection, union, int4-gs64 expert
FFNs, combine + shared expert) on one batch of synthetic tokens that are
already resident in HBM.  The default workload is the GLM-5.2-shaped decode
layer: H=6144, 256 routed experts (F=2048) + 1 shared expert (Fs=2048), top-8,
norm_topk, routed scale 2.5, one token per step, bf16 output.  Each step uses
another token of a 64-token pool and another of ``--layers`` resident copies
of the layer (distinct HBM, experts permuted per copy), so neither the routed
experts nor the shared expert and router can be served from the 256 MB
last-level cache.

Prints one JSON line; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + achieved HBM GB/s (decode) / MFMA util (prefill), 1 GPU"
HBM_PEAK_GBPS = 8000.0
I8_PEAK_OPS = 5.0e15       # dense int8 MFMA (the matrix-core path's arithmetic)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def q4_bytes(n, k):
    """int4 codes + fp32 gs64 scales of an [n][k] matrix."""
    return n * k // 2 + n * (k // 64) * 4


def build_layers(sh, n_layers, dev, shared_router=False):
    """n_layers resident copies of the layer: distinct HBM, experts permuted per copy.
    With shared_router every copy uses copy 0's router (the prefill tokens are built
    for that router)."""
    import torch
    import routed_int4_expert_amd as M
    from routed_int4_expert_amd import synth as S

    t0 = time.time()
    bank = S.Bank(sh, seed=0)
    log(f"expert bank generated on the host in {time.time() - t0:.1f} s")
    base = {k: torch.from_numpy(getattr(bank, k)).to(dev) for k in S.Bank.ROUTED + S.Bank.SHARED}
    layers, routers = [], []
    for l in range(n_layers):
        rw, rb = S.router(sh, 0, 0 if shared_router else l)
        perm = torch.from_numpy(S.layer_perm(sh, 0, l)).to(dev)
        ts = {k: base[k].index_select(0, perm) for k in S.Bank.ROUTED}
        ts.update({k: base[k].clone() for k in S.Bank.SHARED})
        ts["router_w"] = torch.from_numpy(rw).to(dev)
        ts["router_bias"] = torch.from_numpy(rb).to(dev)
        layers.append(M.Layer(S.layer_params(sh), ts))
        routers.append((rw, rb))
    del base
    torch.cuda.synchronize()
    gb = n_layers * (sh.n_experts + 1) * S.expert_bytes(sh) / 1e9
    log(f"{n_layers} resident layer copies ready ({gb:.1f} GB of experts)")
    return bank, layers, routers


def cpu_baseline(sh, bank, routers, xs_host, seconds, per_token_layers=1):
    """The CPU oracle (plain C, fp64) on the same workload, one token at a time."""
    import oracle as R
    from routed_int4_expert_amd import synth as S

    Ls = []
    for l in range(per_token_layers):
        d = S.make_layer(sh, seed=0, layer=l, bank=bank)
        d["router_w"], d["router_bias"] = routers[l]
        Ls.append(R.Layer(d))
    # tokens of the pool in turn until the time budget is spent (timing excludes set-up)
    n, t0 = 0, time.time()
    while n == 0 or time.time() - t0 < seconds:
        i = n % xs_host.shape[0]
        for L in Ls:
            R.layer_forward(L, xs_host[i:i + 1])
        n += 1
    dt = time.time() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    what = "single-token forwards" if per_token_layers == 1 else \
        f"tokens each through {per_token_layers} layers (no glue)"
    return dict(value=n / dt, unit="tokens/s", cores=cores, kind="oracle",
                sample=f"{n} {what} of the same layer copies, {dt:.1f} s, fp64 C oracle "
                       "with OpenMP over FFN rows")


WORKLOADS = {
    "glm_decode": "MoE layer H=6144, 256 routed experts F=2048 + 1 shared Fs=2048, int4-gs64, "
                  "top-8 noaux_tc, norm_topk, routed_scale 2.5, 1 token/step, bf16 out",
    "glm_prefill": "the same layer, 512 tokens/step whose router logits are a popularity-skewed "
                   "Gumbel sample (union ~200 experts), fp32 out",
    "small_decode": "MoE layer H=2048, 256 routed experts F=512 + 1 shared Fs=512, int4-gs64, top-8, "
                    "norm_topk, 64 tokens/step, fp32 out",
    "glm_stack16": "16 GLM-shaped layers resident (distinct HBM), 32 tokens/step, top-p 0.7, "
                   "Zipf(1.1) bias, RMSNorm + residual between layers, fp32",
}


def counted_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    runs (profiles/hbm_counters.json, calibrated against a copy of known size), or None
    when there is none for this workload or the kernel's source changed since."""
    root = os.path.dirname(os.path.abspath(__file__))
    try:
        with open(os.path.join(root, "profiles", "hbm_counters.json")) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    for e in data.get("entries", []):
        if e.get("workload") != workload or e.get("kernel") != kernel:
            continue
        try:
            with open(os.path.join(root, e["source"]), "rb") as f:
                if hashlib.sha256(f.read()).hexdigest() != e["source_sha256"]:
                    return None
        except OSError:
            return None
        return float(e["hbm_bytes_per_launch"])
    return None


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="glm_decode", choices=sorted(WORKLOADS))
    ap.add_argument("--layers", type=int, default=8, help="resident layer copies cycled per step")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only copy a BYTES-long device buffer 13 times (calibrates the HBM "
                         "byte counters against a transfer of known size) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the layer forward "
              "is built and timed on a single MI355X.", file=sys.stderr)
        sys.exit(2)

    import torch
    import routed_int4_expert_amd as M
    from routed_int4_expert_amd import synth as S

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
    wl = args.workload
    sh = S.SHAPES[wl]
    T, H, F, Fs, E, k = sh.tokens, sh.hidden, sh.ffn, sh.shared_ffn, sh.n_experts, sh.top_k
    stack = wl == "glm_stack16"
    nlay = sh.layers if stack else args.layers
    bank, layers, routers = build_layers(sh, nlay, dev, shared_router=(wl == "glm_prefill"))
    # token pool: decode shapes draw independent tokens; prefill batches are built for the router
    if wl == "glm_prefill":
        npool = 2
        xs_host = np.concatenate([S.gumbel_skew_batch(sh, T, routers[0][0], routers[0][1], 0, p)[0]
                                  for p in range(npool)])
    else:
        npool = max(1, 64 // T)
        xs_host = S.tokens(sh, npool * T, seed=0, pool=0)
    xpool = torch.from_numpy(xs_host).to(dev)
    out_bf16 = wl == "glm_decode"
    out = torch.empty((T, H), dtype=torch.bfloat16 if out_bf16 else torch.float32, device=dev)
    ws = layers[0].workspace(T, dev)
    per_step = nlay if stack else 1
    nsteps = args.warmup + args.steps
    ncall = (nsteps + args.steps) * per_step
    nu = torch.zeros((ncall,), dtype=torch.int32, device=dev)
    offb = torch.zeros((ncall, E + 1), dtype=torch.int32, device=dev)
    hbuf = torch.empty((T, H), dtype=torch.float32, device=dev)
    xbuf = torch.empty((T, H), dtype=torch.float32, device=dev)

    # per-call C arguments prepared up front, so the host issues launches as fast as it can
    fwd = M.lib().moe_layer_forward
    glue = M.lib().moe_residual_rmsnorm
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    xptr = [ctypes.c_void_p(xpool.data_ptr() + (i * T * H * 4)) for i in range(npool)]
    dbgs = [M.RouteOutC(n_uniq=nu.data_ptr() + 4 * r, off=offb.data_ptr() + 4 * (E + 1) * r)
            for r in range(ncall)]
    refs = [lay.ref() for lay in layers]
    outp, wsp, wsn = ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws.numel()
    hp, xp = ctypes.c_void_p(hbuf.data_ptr()), ctypes.c_void_p(xbuf.data_ptr())
    odt = M.MOE_BF16 if out_bf16 else M.MOE_F32

    def check(rc, what):
        if rc != M.MOE_OK:
            raise M.MoeError(rc, what)

    def step(i, rec):
        if not stack:
            check(fwd(refs[i % len(refs)], xptr[i % npool], T, outp, odt, ctypes.byref(dbgs[rec]),
                      wsp, wsn, stream), "moe_layer_forward")
            return
        # the stack: h = tokens; per layer x = RMSNorm(h); out = MoE(x); h += out (next glue)
        check(glue(xptr[i % npool], None, T, H, ctypes.c_float(1e-6), hp, xp, stream), "glue")
        for l in range(nlay):
            if l > 0:
                check(glue(hp, outp, T, H, ctypes.c_float(1e-6), hp, xp, stream), "glue")
            check(fwd(refs[l], xp, T, outp, odt, ctypes.byref(dbgs[rec * nlay + l]), wsp, wsn,
                      stream), "moe_layer_forward")

    for i in range(args.warmup):
        step(i, i)
    torch.cuda.synchronize()
    log(f"{wl}: warmup {args.warmup} steps done")

    # timed region: K steps bracketed by synchronisation and HIP events on the launch stream
    s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s_ev.record()
    for i in range(args.steps):
        step(args.warmup + i, args.warmup + i)
    e_ev.record()
    torch.cuda.synchronize()
    ms_step = s_ev.elapsed_time(e_ev) / args.steps
    log(f"timed {args.steps} steps: {ms_step * 1e3:.1f} us/step")

    # the same steps again with per-kernel HIP events on the launch stream
    M.moe_prof_begin()
    for i in range(args.steps):
        step(args.warmup + i, nsteps + i)
    kern = M.moe_prof_end()
    torch.cuda.synchronize()

    sl = slice(args.warmup * per_step, nsteps * per_step)
    n_uniq = nu[sl].cpu().numpy().astype(np.float64)
    rows = offb[sl, E].cpu().numpy().astype(np.float64)
    exp_b, sh_b = S.expert_bytes(sh), S.expert_bytes(sh, Fs)
    # algorithmic bytes and flops per step: union experts + shared expert + router + x + out
    step_bytes = per_step * (n_uniq.mean() * exp_b + sh_b + E * H * 4 + E * 4 + T * H * 4
                             + T * H * (2 if out_bf16 else 4))
    step_flops = per_step * (2.0 * 3 * H * F * rows.mean() + 2.0 * 3 * H * Fs * T + 2.0 * T * E * H)
    # the dominant kernel: gate/up of every unit (codes + scales), x read, h written
    gu_bytes = (n_uniq.mean() * 2 * q4_bytes(F, H) + 2 * q4_bytes(Fs, H) + T * H * 4
                + (rows.mean() * F + T * Fs) * 4)
    gu_flops = 2.0 * 2 * H * (F * rows.mean() + Fs * T)
    gu_name = "ffn_gateup" if T <= 4 else "ffn_gateup_mfma"
    gu_launches, gu_ms = kern.get(gu_name, (0, float("nan")))
    gu_avg_ms = gu_ms / max(gu_launches, 1)
    achieved = gu_bytes / (gu_avg_ms * 1e-3) / 1e9
    result = {
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
        # (carried as two int8 limbs) with exact int32 group sums (v_dot4 in the decode
        # GEMV for T <= 4, int8 matrix cores for T > 4), then fp32 accumulation
        "dtype": "i4xfx16-i32-f32acc",
        "data": "synthetic",
        "config": {
            "workload": f"{wl}: {WORKLOADS[wl]}",
            "tokens_per_step": T,
            "layer_copies_cycled": nlay,
            "mean_union_experts": float(n_uniq.mean()),
            "mean_routed_rows": float(rows.mean()),
            "algorithmic_bytes_per_step": float(step_bytes),
            "step_hbm_gbps": float(step_bytes / (ms_step * 1e-3) / 1e9),
            "step_tflops": float(step_flops / (ms_step * 1e-3) / 1e12),
        },
        "roofline": {
            "kernel": (f"{gu_name} (gate+up of every union expert and the shared expert, "
                       "SiLU*up epilogue)"),
            "bound": "hbm",
            "achieved": float(achieved),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": float(achieved / HBM_PEAK_GBPS),
            "traffic": counted_traffic(wl, gu_name),
            "bytes_per_launch": float(gu_bytes),
            "avg_launch_us": float(gu_avg_ms * 1e3),
            "mfma_util_vs_i8_dense": float(gu_flops / (gu_avg_ms * 1e-3) / I8_PEAK_OPS),
        },
        "kernels_us_per_step": {kname: v[1] * 1e3 / args.steps for kname, v in kern.items()},
    }
    if not args.no_cpu_baseline:
        log(f"CPU baseline: oracle for ~{args.cpu_seconds:.0f} s")
        result["cpu_baseline"] = cpu_baseline(sh, bank, routers, xs_host, args.cpu_seconds,
                                              per_token_layers=nlay if stack else 1)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

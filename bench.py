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
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + achieved HBM GB/s (decode) / MFMA util (prefill), 1 GPU"
HBM_PEAK_GBPS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def q4_bytes(n, k):
    """int4 codes + fp32 gs64 scales of an [n][k] matrix."""
    return n * k // 2 + n * (k // 64) * 4


def build_layers(sh, n_layers, dev):
    import torch
    import routed_int4_expert_amd as M
    from routed_int4_expert_amd import synth as S

    t0 = time.time()
    bank = S.Bank(sh, seed=0)
    log(f"expert bank generated on the host in {time.time() - t0:.1f} s")
    base = {k: torch.from_numpy(getattr(bank, k)).to(dev) for k in S.Bank.ROUTED + S.Bank.SHARED}
    layers = []
    for l in range(n_layers):
        rw, rb = S.router(sh, 0, l)
        perm = torch.from_numpy(S.layer_perm(sh, 0, l)).to(dev)
        ts = {k: base[k].index_select(0, perm) for k in S.Bank.ROUTED}
        ts.update({k: base[k].clone() for k in S.Bank.SHARED})
        ts["router_w"] = torch.from_numpy(rw).to(dev)
        ts["router_bias"] = torch.from_numpy(rb).to(dev)
        layers.append(M.Layer(S.layer_params(sh), ts))
    del base
    torch.cuda.synchronize()
    log(f"{n_layers} resident layer copies ready ({n_layers * 257 * S.expert_bytes(sh) / 1e9:.1f} GB of experts)")
    return bank, layers


def cpu_baseline(sh, bank, xpool, seconds):
    """The CPU oracle (plain C, fp64) on the same layer, one token at a time."""
    import oracle as R
    from routed_int4_expert_amd import synth as S

    d = S.make_layer(sh, seed=0, bank=bank)
    L = R.Layer(d)
    n, t0 = 0, time.time()
    while n == 0 or (time.time() - t0 < seconds and n < xpool.shape[0]):
        R.layer_forward(L, xpool[n:n + 1])
        n += 1
    dt = time.time() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return dict(value=n / dt, unit="tokens/s", cores=cores, kind="oracle",
                sample=f"{n} single-token forwards of layer copy 0 (the first {n} pool tokens), "
                       f"{dt:.1f} s, fp64 C oracle with OpenMP over FFN rows")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=8, help="resident layer copies cycled per step")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only copy a BYTES-long device buffer 3 times (calibrates the HBM "
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
    sh = S.SHAPES["glm_decode"]
    T, H, F, Fs, E, k = sh.tokens, sh.hidden, sh.ffn, sh.shared_ffn, sh.n_experts, sh.top_k
    bank, layers = build_layers(sh, args.layers, dev)
    xpool_h = S.tokens(sh, 64, seed=0, pool=0)
    xpool = torch.from_numpy(xpool_h).to(dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ws = layers[0].workspace(T, dev)
    nsteps = args.warmup + args.steps
    nu = torch.zeros((nsteps + args.steps,), dtype=torch.int32, device=dev)

    # per-step C arguments prepared up front, so the host issues launches as fast as it can
    fwd = M.lib().moe_layer_forward
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    xptr = [ctypes.c_void_p(xpool.data_ptr() + (i * T * H * 4)) for i in range(64 // T)]
    dbgs = [M.RouteOutC(n_uniq=nu.data_ptr() + 4 * r) for r in range(nu.numel())]
    refs = [lay.ref() for lay in layers]
    outp, wsp, wsn = ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws.numel()

    def step(i, rec):
        rc = fwd(refs[i % len(refs)], xptr[i % len(xptr)], T, outp, M.MOE_BF16,
                 ctypes.byref(dbgs[rec]), wsp, wsn, stream)
        if rc != M.MOE_OK:
            raise M.MoeError(rc, "moe_layer_forward")

    for i in range(args.warmup):
        step(i, i)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    # timed region: K steps bracketed by synchronisation and HIP events on the launch stream
    s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s_ev.record()
    for i in range(args.steps):
        step(args.warmup + i, args.warmup + i)
    e_ev.record()
    torch.cuda.synchronize()
    ms_total = s_ev.elapsed_time(e_ev)
    ms_step = ms_total / args.steps
    log(f"timed {args.steps} steps: {ms_step * 1e3:.1f} us/step")

    # the same steps again with per-kernel HIP events on the launch stream
    M.moe_prof_begin()
    for i in range(args.steps):
        step(args.warmup + i, nsteps + i)
    kern = M.moe_prof_end()
    torch.cuda.synchronize()

    n_uniq = nu[args.warmup:nsteps].cpu().numpy().astype(np.int64)
    units = n_uniq + 1  # + the shared expert
    exp_b = S.expert_bytes(sh)
    # algorithmic bytes of a step: union experts + shared expert + router + x + out
    step_bytes = (n_uniq.mean() * exp_b + S.expert_bytes(sh, Fs) + E * H * 4 + E * 4
                  + T * H * 4 + T * H * 2)
    # the dominant kernel: gate/up of every unit (codes + scales), x read, h written
    gu_bytes = units.mean() * 2 * q4_bytes(F, H) + T * H * 4 + (n_uniq.mean() * T + T) * F * 4
    gu_launches, gu_ms = kern.get("ffn_gateup", (0, float("nan")))
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
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "glm_decode: MoE layer H=6144, 256 routed experts F=2048 + 1 shared Fs=2048, "
                        "int4-gs64, top-8 noaux_tc, norm_topk, routed_scale 2.5, 1 token/step, bf16 out",
            "tokens_per_step": T,
            "layer_copies_cycled": args.layers,
            "mean_union_experts": float(n_uniq.mean()),
            "algorithmic_bytes_per_step": float(step_bytes),
            "step_hbm_gbps": float(step_bytes / (ms_step * 1e-3) / 1e9),
        },
        "roofline": {
            "kernel": "ffn_gateup (q4_gemv_kernel, gate+up GEMV with SiLU*up epilogue)",
            "bound": "hbm",
            "achieved": float(achieved),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": float(achieved / HBM_PEAK_GBPS),
            "traffic": None,
            "bytes_per_launch": float(gu_bytes),
            "avg_launch_us": float(gu_avg_ms * 1e3),
        },
        "kernels_us_per_step": {kname: v[1] * 1e3 / max(v[0], 1) for kname, v in kern.items()},
    }
    if not args.no_cpu_baseline:
        log(f"CPU baseline: oracle for ~{args.cpu_seconds:.0f} s")
        result["cpu_baseline"] = cpu_baseline(sh, bank, xpool_h, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

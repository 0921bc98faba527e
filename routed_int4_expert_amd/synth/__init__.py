"""Seeded synthetic inputs for the sparse MoE layer.

Holds no step of the MoE forward: it draws router weights, biases, tokens and
fp32 expert weights from a counter-based SplitMix64 (``gen.c``), and converts
the expert weights into the int4-gs64 container the layer consumes.  Both the
HIP library's tests/benchmark and the CPU oracle take their inputs from here.

Workloads (shapes from the colibrì GLM-5.2 description: top-8 of 256 routed
experts with one shared expert, ~19 MB of int4 payload per 6144x2048 expert):

* ``tiny``            H=256, E=16, F=Fs=128, top-4, norm on, scale 1, 8 tokens.
* ``glm_decode``      H=6144, E=256, F=Fs=2048, top-8, norm on, scale 2.5, 1 token.
* ``glm_prefill``     the same layer, 512 tokens whose router logits are a
                      popularity-skewed Gumbel sample (union ~200 experts).
* ``small_decode``    H=2048, E=256, F=Fs=512, top-8, norm on, scale 1, 64 tokens,
                      logits ~N(0,1), bias ~U(-0.5, 0.5).
* ``glm_stack16``     16 GLM-shaped layers, 32 tokens, top-p 0.7, Zipf(1.1)
                      expert popularity in the router bias, RMSNorm + residual glue.
* ``glm_rows256``     16 GLM-shaped experts, 512 tokens top-8 (~256 rows per expert):
                      the grouped GEMM's compute-bound regime (a microbenchmark).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB_PATH = os.path.join(_HERE, "_gen.so")
_lib = None


def build() -> str:
    """Compile gen.c into _gen.so (gcc, OpenMP)."""
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-O3", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    u64, i64, d, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    lib.synth_key.restype = u64
    lib.synth_key.argtypes = [u64, u64]
    lib.synth_u64.argtypes = [u64, i64, vp]
    lib.synth_uniform_f64.argtypes = [u64, i64, d, d, vp]
    lib.synth_normal_f64.argtypes = [u64, i64, d, d, vp]
    lib.synth_normal_f32.argtypes = [u64, i64, d, d, vp]
    lib.synth_quantize_gs64.argtypes = [vp, i64, i64, vp, vp]
    lib.synth_q4_normal.argtypes = [u64, i64, i64, d, vp, vp]
    lib.synth_q3_normal.argtypes = [u64, i64, i64, d, vp, vp]
    lib.synth_f4_normal.argtypes = [u64, i64, i64, d, vp, vp]
    for f in ("synth_u64", "synth_uniform_f64", "synth_normal_f64", "synth_normal_f32",
              "synth_quantize_gs64", "synth_q4_normal", "synth_q3_normal", "synth_f4_normal"):
        getattr(lib, f).restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def stream_id(name: str) -> int:
    """64-bit FNV-1a of a stream name."""
    h = 0xCBF29CE484222325
    for b in name.encode():
        h ^= b
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def key(seed: int, name: str) -> int:
    return int(_load().synth_key(seed & 0xFFFFFFFFFFFFFFFF, stream_id(name)))


def normal_f32(seed: int, name: str, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    out = np.empty(shape, np.float32)
    _load().synth_normal_f32(key(seed, name), out.size, mean, std, _ptr(out))
    return out


def normal_f64(seed: int, name: str, shape, std: float = 1.0) -> np.ndarray:
    out = np.empty(shape, np.float64)
    _load().synth_normal_f64(key(seed, name), out.size, 0.0, std, _ptr(out))
    return out


def uniform_f64(seed: int, name: str, shape, lo: float, hi: float) -> np.ndarray:
    out = np.empty(shape, np.float64)
    _load().synth_uniform_f64(key(seed, name), out.size, lo, hi, _ptr(out))
    return out


def uniform_f32(seed: int, name: str, shape, lo: float, hi: float) -> np.ndarray:
    return uniform_f64(seed, name, shape, lo, hi).astype(np.float32)


def permutation(seed: int, name: str, n: int) -> np.ndarray:
    """Seeded Fisher-Yates permutation of 0..n-1."""
    u = uniform_f64(seed, name, (n,), 0.0, 1.0)
    p = np.arange(n, dtype=np.int64)
    for i in range(n - 1, 0, -1):
        j = min(int(u[i] * (i + 1)), i)
        p[i], p[j] = p[j], p[i]
    return p


def quantize_gs64(w: np.ndarray):
    """Symmetric absmax int4-gs64 container of an fp32 matrix W[N][K] -> (q [N][K/2] u8, s [N][K/64] f32)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    assert K % 64 == 0
    q = np.empty((N, K // 2), np.uint8)
    s = np.empty((N, K // 64), np.float32)
    _load().synth_quantize_gs64(_ptr(w), N, K, _ptr(q), _ptr(s))
    return q, s


def q4_normal(seed: int, name: str, N: int, K: int, std: float, q_out=None, s_out=None):
    """int4-gs64 container of W[N][K] ~ N(0, std^2) (fp32 draws, then quantised)."""
    q = np.empty((N, K // 2), np.uint8) if q_out is None else q_out
    s = np.empty((N, K // 64), np.float32) if s_out is None else s_out
    assert q.shape == (N, K // 2) and s.shape == (N, K // 64)
    _load().synth_q4_normal(key(seed, name), N, K, std, _ptr(q), _ptr(s))
    return q, s


# expert weight formats (the library's MOE_FMT_* values)
FMT_INT4, FMT_MXFP4, FMT_INT3 = 0, 1, 2
FMT_NAMES = {FMT_INT4: "int4-gs64", FMT_MXFP4: "mxfp4", FMT_INT3: "int3-g64"}


def code_bytes(fmt: int, K: int) -> int:
    """Bytes of one row's codes: 4 bits per element, or 3 for int3-g64."""
    return 3 * K // 8 if fmt == FMT_INT3 else K // 2


def scale_shape(fmt: int, K: int):
    """(elements per row, dtype) of one row's scales."""
    return (K // 32, np.uint8) if fmt == FMT_MXFP4 else (K // 64, np.float32)


def q_normal(fmt: int, seed: int, name: str, N: int, K: int, std: float, q_out=None, s_out=None):
    """W[N][K] ~ N(0, std^2) (the same fp32 draws for every format) in expert format fmt."""
    if fmt == FMT_INT4:
        return q4_normal(seed, name, N, K, std, q_out, s_out)
    ns, sdt = scale_shape(fmt, K)
    q = np.empty((N, code_bytes(fmt, K)), np.uint8) if q_out is None else q_out
    s = np.empty((N, ns), sdt) if s_out is None else s_out
    assert q.shape == (N, code_bytes(fmt, K)) and s.shape == (N, ns) and s.dtype == sdt
    f = _load().synth_q3_normal if fmt == FMT_INT3 else _load().synth_f4_normal
    f(key(seed, name), N, K, std, _ptr(q), _ptr(s))
    return q, s


@dataclass(frozen=True)
class Shape:
    """Layer hyper-parameters and how its synthetic inputs are drawn."""
    name: str
    hidden: int
    n_experts: int
    ffn: int
    shared_ffn: int
    top_k: int
    top_p: float
    norm_topk: int
    routed_scale: float
    tokens: int
    router_std: float
    bias_kind: str = "uniform"       # "uniform" (+-bias_amp) | "zipf" | "zero"
    bias_amp: float = 0.1
    weight_std: float = 0.02
    bank: str = ""                   # expert-bank stream name ("" = own)
    layers: int = 1
    logits: str = "router"           # "router" | "gumbel_skew" (constructed)
    extra: dict = field(default_factory=dict)
    expert_fmt: int = FMT_INT4       # expert weight format (FMT_*)


SHAPES = {
    "tiny": Shape("tiny", 256, 16, 128, 128, 4, 0.0, 1, 1.0, 8, router_std=0.02,
                  bias_amp=0.1),
    "glm_decode": Shape("glm_decode", 6144, 256, 2048, 2048, 8, 0.0, 1, 2.5, 1,
                        router_std=1.0 / math.sqrt(6144), bias_amp=0.1, bank="glm"),
    "glm_prefill": Shape("glm_prefill", 6144, 256, 2048, 2048, 8, 0.0, 1, 2.5, 512,
                         router_std=1.0 / math.sqrt(6144), bias_amp=0.1, bank="glm",
                         logits="gumbel_skew", extra={"alpha": 6.4}),
    "small_decode": Shape("small_decode", 2048, 256, 512, 512, 8, 0.0, 1, 1.0, 64,
                          router_std=1.0 / math.sqrt(2048), bias_amp=0.5),
    "glm_stack16": Shape("glm_stack16", 6144, 256, 2048, 2048, 8, 0.7, 1, 2.5, 32,
                         router_std=1.0 / math.sqrt(6144), bias_kind="zipf", bank="glm",
                         layers=16, extra={"zipf_s": 1.1, "zipf_amp": 0.5}),
    # grouped-GEMM microbenchmark in the compute-bound regime: GLM-shaped experts, 16 of
    # them, 512 tokens top-8, so each expert has about 256 rows and the shared expert 512
    "glm_rows256": Shape("glm_rows256", 6144, 16, 2048, 2048, 8, 0.0, 1, 2.5, 512,
                         router_std=1.0 / math.sqrt(6144), bias_amp=0.05, bank="glm"),
}


def custom(name: str, **kw) -> Shape:
    """A test shape derived from keyword arguments (defaults: tiny)."""
    return replace(SHAPES["tiny"], name=name, **kw)


def expert_bytes(sh: Shape, ffn: int | None = None) -> int:
    """Codes + scales of one expert's three matrices in the shape's expert format."""
    F = sh.ffn if ffn is None else ffn
    fmt = sh.expert_fmt
    total = 0
    for N, K in ((F, sh.hidden), (F, sh.hidden), (sh.hidden, F)):
        ns, sdt = scale_shape(fmt, K)
        total += N * (code_bytes(fmt, K) + ns * np.dtype(sdt).itemsize)
    return total


class Bank:
    """Stacked expert weights (the shape's expert format) plus the shared expert (host numpy)."""

    def __init__(self, sh: Shape, seed: int = 0):
        H, E, F, Fs = sh.hidden, sh.n_experts, sh.ffn, sh.shared_ffn
        fmt = sh.expert_fmt
        tag = f"bank:{sh.bank or sh.name}"
        nsh, sdt = scale_shape(fmt, H)
        nsf, _ = scale_shape(fmt, F)
        self.gate_q = np.empty((E, F, code_bytes(fmt, H)), np.uint8)
        self.gate_s = np.empty((E, F, nsh), sdt)
        self.up_q = np.empty((E, F, code_bytes(fmt, H)), np.uint8)
        self.up_s = np.empty((E, F, nsh), sdt)
        self.down_q = np.empty((E, H, code_bytes(fmt, F)), np.uint8)
        self.down_s = np.empty((E, H, nsf), sdt)
        for e in range(E):
            q_normal(fmt, seed, f"{tag}/gate/{e}", F, H, sh.weight_std, self.gate_q[e], self.gate_s[e])
            q_normal(fmt, seed, f"{tag}/up/{e}", F, H, sh.weight_std, self.up_q[e], self.up_s[e])
            q_normal(fmt, seed, f"{tag}/down/{e}", H, F, sh.weight_std, self.down_q[e], self.down_s[e])
        if Fs > 0:
            self.sh_gate_q, self.sh_gate_s = q_normal(fmt, seed, f"{tag}/shared/gate", Fs, H, sh.weight_std)
            self.sh_up_q, self.sh_up_s = q_normal(fmt, seed, f"{tag}/shared/up", Fs, H, sh.weight_std)
            self.sh_down_q, self.sh_down_s = q_normal(fmt, seed, f"{tag}/shared/down", H, Fs, sh.weight_std)
        else:
            z8, z32 = np.zeros((0,), np.uint8), np.zeros((0,), sdt)
            self.sh_gate_q = self.sh_up_q = self.sh_down_q = z8
            self.sh_gate_s = self.sh_up_s = self.sh_down_s = z32

    ROUTED = ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")
    SHARED = ("sh_gate_q", "sh_gate_s", "sh_up_q", "sh_up_s", "sh_down_q", "sh_down_s")

    def permuted(self, perm: np.ndarray) -> dict:
        """Routed tensors with expert e taken from base expert perm[e] (a copy)."""
        return {k: np.ascontiguousarray(getattr(self, k)[perm]) for k in self.ROUTED}

    def arrays(self) -> dict:
        return {k: getattr(self, k) for k in self.ROUTED + self.SHARED}


def layer_perm(sh: Shape, seed: int, layer: int) -> np.ndarray:
    """Stacked layer l's expert e is a copy of base expert (a*e + b) mod E, a odd."""
    E = sh.n_experts
    if layer == 0:
        return np.arange(E, dtype=np.int64)
    u = uniform_f64(seed, f"{sh.name}/L{layer}/perm", (2,), 0.0, 1.0)
    a = 2 * int(u[0] * (E // 2 if E > 1 else 1)) + 1
    b = int(u[1] * E)
    return (a * np.arange(E, dtype=np.int64) + b) % E


def router(sh: Shape, seed: int = 0, layer: int = 0):
    """(router_w [E][H] f32, router_bias [E] f32) of one layer."""
    E, H = sh.n_experts, sh.hidden
    if sh.logits == "gumbel_skew":
        w = _orthonormal_rows(seed, f"{sh.name}/L{layer}/router_orth", E, H).astype(np.float32)
    else:
        w = normal_f32(seed, f"{sh.name}/L{layer}/router_w", (E, H), std=sh.router_std)
    if sh.bias_kind == "uniform":
        b = uniform_f32(seed, f"{sh.name}/L{layer}/router_bias", (E,), -sh.bias_amp, sh.bias_amp)
    elif sh.bias_kind == "zipf":
        # expert popularity ~ rank^-s: bias = amp * r(e)^-s, r a seeded permutation of 1..E
        r = permutation(seed, f"{sh.name}/L{layer}/zipf_rank", E) + 1
        b = (sh.extra["zipf_amp"] * r.astype(np.float64) ** (-sh.extra["zipf_s"])).astype(np.float32)
    else:
        b = np.zeros((E,), np.float32)
    return w, b


def tokens(sh: Shape, T: int, seed: int = 0, pool: int = 0) -> np.ndarray:
    """x [T][H] ~ N(0,1) fp32; ``pool`` selects an independent batch."""
    return normal_f32(seed, f"{sh.name}/x/{pool}", (T, sh.hidden))


def _orthonormal_rows(seed: int, name: str, E: int, H: int) -> np.ndarray:
    g = normal_f64(seed, name, (H, E))
    q, r = np.linalg.qr(g)
    q = q * np.sign(np.diag(r))[None, :]
    return np.ascontiguousarray(q.T)  # [E][H], orthonormal rows


def gumbel_skew_batch(sh: Shape, T: int, router_w: np.ndarray, bias: np.ndarray,
                      seed: int = 0, pool: int = 0):
    """Tokens whose logits under a router with orthonormal rows are mu_e + Gumbel noise.

    mu_e = -alpha * pi(e) / E for a seeded permutation pi: the larger the spread alpha,
    the more the picks concentrate on the popular experts.  alpha is a fixed input
    parameter (6.4 for the GLM-shaped prefill batch of 512 tokens, chosen once so that
    its batch union is about 200 of the 256 experts; a CPU test checks the realised
    union).  Tokens are x_t = L_t Wr + (I - Wr^T Wr) z_t, so x Wr^T reproduces L up to
    fp32 rounding and x is N(0, 1) outside the router's row space.  ``bias`` is not used
    (kept for the call signature).  Returns (x f32 [T][H], alpha).
    """
    E, H = sh.n_experts, sh.hidden
    alpha = float(sh.extra["alpha"])
    wr = router_w.astype(np.float64)
    pi = permutation(seed, f"{sh.name}/popularity", E).astype(np.float64)
    u = uniform_f64(seed, f"{sh.name}/gumbel/{pool}", (T, E), 0.0, 1.0)
    G = -np.log(-np.log(u))
    L = -alpha * pi[None, :] / E + G
    z = normal_f64(seed, f"{sh.name}/z/{pool}", (T, H))
    x = L @ wr + z - (z @ wr.T) @ wr
    return np.ascontiguousarray(x.astype(np.float32)), alpha


def layer_params(sh: Shape) -> dict:
    return dict(hidden=sh.hidden, n_experts=sh.n_experts, ffn=sh.ffn, shared_ffn=sh.shared_ffn,
                top_k=sh.top_k, top_p=sh.top_p, norm_topk=sh.norm_topk,
                routed_scale=sh.routed_scale, expert_fmt=sh.expert_fmt)


def make_layer(sh: Shape, seed: int = 0, layer: int = 0, bank: Bank | None = None) -> dict:
    """One layer's full host input set (params + numpy arrays)."""
    bank = bank if bank is not None else Bank(sh, seed)
    rw, rb = router(sh, seed, layer)
    d = layer_params(sh)
    d.update(router_w=rw, router_bias=rb)
    if layer == 0:
        d.update({k: getattr(bank, k) for k in Bank.ROUTED})
    else:
        d.update(bank.permuted(layer_perm(sh, seed, layer)))
    d.update({k: getattr(bank, k) for k in Bank.SHARED})
    return d


def make_batch(sh: Shape, layer: dict, seed: int = 0, pool: int = 0, T: int | None = None):
    """Tokens x [T][H] for one step of ``layer``."""
    T = sh.tokens if T is None else T
    if sh.logits == "gumbel_skew":
        x, _alpha = gumbel_skew_batch(sh, T, layer["router_w"], layer["router_bias"], seed, pool)
        return x
    return tokens(sh, T, seed, pool)

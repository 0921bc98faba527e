"""ctypes binding of the CPU oracle (moe_ref.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  Every array is a host
numpy array; results are fp64 where the oracle computes in fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_ref.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_ref.so")
_lib = None


def build() -> str:
    """Compile the oracle with gcc (plain C11, -O2, OpenMP over independent rows)."""
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-fopenmp", "-fPIC", "-shared",
                           _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class RefLayer(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("ffn", ctypes.c_int32),
        ("shared_ffn", ctypes.c_int32), ("top_k", ctypes.c_int32), ("top_p", ctypes.c_float),
        ("norm_topk", ctypes.c_int32), ("routed_scale", ctypes.c_float),
        ("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
        ("gate_q", ctypes.c_void_p), ("gate_s", ctypes.c_void_p),
        ("up_q", ctypes.c_void_p), ("up_s", ctypes.c_void_p),
        ("down_q", ctypes.c_void_p), ("down_s", ctypes.c_void_p),
        ("sh_gate_q", ctypes.c_void_p), ("sh_gate_s", ctypes.c_void_p),
        ("sh_up_q", ctypes.c_void_p), ("sh_up_s", ctypes.c_void_p),
        ("sh_down_q", ctypes.c_void_p), ("sh_down_s", ctypes.c_void_p),
        ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32),
        ("act_bits", ctypes.c_int32), ("act_block", ctypes.c_int32),
        ("fmt", ctypes.c_int32),
    ]


# expert weight formats (moe_ref.h)
FMT_INT4, FMT_MXFP4, FMT_INT3 = 0, 1, 2


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L = ctypes.POINTER(RefLayer)
    sig = {
        "moe_ref_pack_int4": (ctypes.c_uint8, [i32, i32]),
        "moe_ref_unpack_int4": (None, [ctypes.c_uint8, vp, vp]),
        "moe_ref_quantize_gs64": (ctypes.c_int, [vp, i64, i64, vp, vp]),
        "moe_ref_dequantize_gs64": (ctypes.c_int, [vp, vp, i64, i64, vp]),
        "moe_ref_logits": (ctypes.c_int, [L, vp, i32, vp]),
        "moe_ref_select": (ctypes.c_int, [L, vp, i32, vp, vp, vp]),
        "moe_ref_route": (ctypes.c_int, [L, vp, i32, vp, vp, vp]),
        "moe_ref_union": (ctypes.c_int, [i32, i32, vp, vp, i32, vp, vp, vp, vp, vp]),
        "moe_ref_swiglu": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, i32, i32, vp, vp]),
        "moe_ref_expert_ffn": (ctypes.c_int, [L, vp, i32, vp, vp, vp]),
        "moe_ref_layer_forward": (ctypes.c_int, [L, vp, i32, vp, i32, vp]),
        "moe_ref_rmsnorm": (ctypes.c_int, [vp, i32, i32, ctypes.c_double, vp]),
        "moe_ref_dense_mlp": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, i32, i32, vp, i32, vp]),
        "moe_ref_quant_act8": (None, [vp, i32, i32, vp]),
        "moe_ref_e2m1": (ctypes.c_double, [ctypes.c_uint8]),
        "moe_ref_ue8m0": (ctypes.c_double, [ctypes.c_uint8]),
        "moe_ref_int3_code": (i32, [vp, i64, i64]),
        "moe_ref_code_bytes": (i64, [i32, i64]),
        "moe_ref_scale_bytes": (i64, [i32, i64]),
        "moe_ref_dequantize": (ctypes.c_int, [i32, vp, vp, i64, i64, vp]),
        "moe_ref_swiglu_fmt": (ctypes.c_int, [i32, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "need C-contiguous numpy"
    return a.ctypes.data


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


class Layer:
    """Host-side layer description for the oracle: numpy arrays + hyper-parameters."""

    FIELDS = ("router_w", "router_bias", "gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s",
              "sh_gate_q", "sh_gate_s", "sh_up_q", "sh_up_s", "sh_down_q", "sh_down_s")

    def __init__(self, d: dict):
        self.d = {}
        for k in self.FIELDS:
            v = d.get(k)
            self.d[k] = None if v is None else np.ascontiguousarray(v)
        self.hidden, self.n_experts, self.ffn = int(d["hidden"]), int(d["n_experts"]), int(d["ffn"])
        self.shared_ffn, self.top_k = int(d["shared_ffn"]), int(d["top_k"])
        self.top_p, self.norm_topk = float(d["top_p"]), int(d["norm_topk"])
        self.routed_scale = float(d["routed_scale"])
        self.n_group, self.topk_group = int(d.get("n_group", 0)), int(d.get("topk_group", 0))
        self.act_bits, self.act_block = int(d.get("act_bits", 0)), int(d.get("act_block", 0))
        self.fmt = int(d.get("expert_fmt", FMT_INT4))
        s = RefLayer()
        s.hidden, s.n_experts, s.ffn = self.hidden, self.n_experts, self.ffn
        s.shared_ffn, s.top_k, s.top_p = self.shared_ffn, self.top_k, self.top_p
        s.norm_topk, s.routed_scale = self.norm_topk, self.routed_scale
        s.n_group, s.topk_group = self.n_group, self.topk_group
        s.act_bits, s.act_block = self.act_bits, self.act_block
        s.fmt = self.fmt
        for k in self.FIELDS:
            setattr(s, k, _p(self.d[k]) if self.d[k] is not None and self.d[k].size else None)
        self.struct = s

    def ref(self):
        return ctypes.byref(self.struct)


def pack_int4(lo: int, hi: int) -> int:
    return int(_load().moe_ref_pack_int4(lo, hi))


def unpack_int4(b: int):
    lo, hi = ctypes.c_int32(), ctypes.c_int32()
    _load().moe_ref_unpack_int4(b, ctypes.byref(lo), ctypes.byref(hi))
    return lo.value, hi.value


def quantize_gs64(w: np.ndarray):
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    q = np.empty((N, K // 2), np.uint8)
    s = np.empty((N, K // 64), np.float32)
    _check(_load().moe_ref_quantize_gs64(_p(w), N, K, _p(q), _p(s)), "quantize")
    return q, s


def dequantize_gs64(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.float32)
    N, K = q.shape[0], q.shape[1] * 2
    w = np.empty((N, K), np.float64)
    _check(_load().moe_ref_dequantize_gs64(_p(q), _p(s), N, K, _p(w)), "dequantize")
    return w


def e2m1(code: int) -> float:
    return float(_load().moe_ref_e2m1(code))


def ue8m0(e: int) -> float:
    return float(_load().moe_ref_ue8m0(e))


def int3_code(row_q: np.ndarray, K: int, k: int) -> int:
    row_q = np.ascontiguousarray(row_q, dtype=np.uint8)
    assert row_q.size == 3 * K // 8
    return int(_load().moe_ref_int3_code(_p(row_q), K, k))


def code_bytes(fmt: int, K: int) -> int:
    return int(_load().moe_ref_code_bytes(fmt, K))


def scale_bytes(fmt: int, K: int) -> int:
    return int(_load().moe_ref_scale_bytes(fmt, K))


def dequantize(fmt: int, q: np.ndarray, s: np.ndarray, K: int) -> np.ndarray:
    """W[N][K] (fp64) of a matrix in any expert format (q [N][code bytes], s [N][...])."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s)
    N = q.shape[0]
    assert q.shape[1] == code_bytes(fmt, K) and s.nbytes == N * scale_bytes(fmt, K)
    w = np.empty((N, K), np.float64)
    _check(_load().moe_ref_dequantize(fmt, _p(q), _p(s), N, K, _p(w)), "dequantize")
    return w


def swiglu_fmt(fmt: int, gq, gs, uq, us, dq, ds, H: int, F: int, x: np.ndarray) -> np.ndarray:
    arrs = [np.ascontiguousarray(a) for a in (gq, gs, uq, us, dq, ds)]
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty((H,), np.float64)
    _check(_load().moe_ref_swiglu_fmt(fmt, *[_p(a) for a in arrs], H, F, _p(x), _p(y)), "swiglu_fmt")
    return y


def logits(L: Layer, x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    T = x.shape[0]
    out = np.empty((T, L.n_experts), np.float64)
    _check(_load().moe_ref_logits(L.ref(), _p(x), T, _p(out)), "logits")
    return out


def select(L: Layer, lg: np.ndarray):
    lg = np.ascontiguousarray(lg, dtype=np.float64)
    T = lg.shape[0]
    ids = np.empty((T, L.top_k), np.int32)
    w = np.empty((T, L.top_k), np.float32)
    keff = np.empty((T,), np.int32)
    _check(_load().moe_ref_select(L.ref(), _p(lg), T, _p(ids), _p(w), _p(keff)), "select")
    return ids, w, keff


def route(L: Layer, x: np.ndarray):
    x = np.ascontiguousarray(x, dtype=np.float32)
    T = x.shape[0]
    ids = np.empty((T, L.top_k), np.int32)
    w = np.empty((T, L.top_k), np.float32)
    keff = np.empty((T,), np.int32)
    _check(_load().moe_ref_route(L.ref(), _p(x), T, _p(ids), _p(w), _p(keff)), "route")
    return ids, w, keff


def union(E: int, ids: np.ndarray, keff: np.ndarray):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    keff = np.ascontiguousarray(keff, dtype=np.int32)
    T, k = ids.shape
    n_uniq = np.zeros((1,), np.int32)
    uniq = np.empty((E,), np.int32)
    off = np.empty((E + 1,), np.int32)
    row_tok = np.empty((max(T * k, 1),), np.int32)
    pick_row = np.empty((max(T * k, 1),), np.int32)
    _check(_load().moe_ref_union(E, k, _p(ids), _p(keff), T, _p(n_uniq), _p(uniq), _p(off),
                                 _p(row_tok), _p(pick_row)), "union")
    return dict(n_uniq=int(n_uniq[0]), uniq=uniq, off=off, row_tok=row_tok[:T * k],
                pick_row=pick_row[:T * k].reshape(T, k))


def swiglu(gq, gs, uq, us, dq, ds, x: np.ndarray) -> np.ndarray:
    arrs = [np.ascontiguousarray(a) for a in (gq, gs, uq, us, dq, ds)]
    x = np.ascontiguousarray(x, dtype=np.float32)
    F, H = arrs[0].shape[0], arrs[0].shape[1] * 2
    y = np.empty((H,), np.float64)
    _check(_load().moe_ref_swiglu(*[_p(a) for a in arrs], H, F, _p(x), _p(y)), "swiglu")
    return y


def expert_ffn(L: Layer, x: np.ndarray, off: np.ndarray, row_tok: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    off = np.ascontiguousarray(off, dtype=np.int32)
    row_tok = np.ascontiguousarray(row_tok, dtype=np.int32)
    rows = int(off[-1])
    y = np.zeros((max(rows, 1), L.hidden), np.float64)
    _check(_load().moe_ref_expert_ffn(L.ref(), _p(x), x.shape[0], _p(off), _p(row_tok), _p(y)),
           "expert_ffn")
    return y[:rows]


def layer_forward(L: Layer, x: np.ndarray, toks=None) -> np.ndarray:
    """fp64 layer output for all tokens, or for the listed tokens (in list order)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    T = x.shape[0]
    if toks is None:
        out = np.empty((T, L.hidden), np.float64)
        _check(_load().moe_ref_layer_forward(L.ref(), _p(x), T, None, 0, _p(out)), "layer_forward")
    else:
        tk = np.ascontiguousarray(np.asarray(toks, dtype=np.int32))
        out = np.empty((tk.size, L.hidden), np.float64)
        _check(_load().moe_ref_layer_forward(L.ref(), _p(x), T, _p(tk), tk.size, _p(out)),
               "layer_forward")
    return out


def dense_mlp(gq, gs, uq, us, dq, ds, x: np.ndarray) -> np.ndarray:
    """The first-dense-layer SwiGLU MLP on every token, fp64 [T][H]."""
    arrs = [np.ascontiguousarray(a) for a in (gq, gs, uq, us, dq, ds)]
    x = np.ascontiguousarray(x, dtype=np.float32)
    F, H = arrs[0].shape[0], arrs[0].shape[1] * 2
    T = x.shape[0]
    out = np.empty((T, H), np.float64)
    _check(_load().moe_ref_dense_mlp(*[_p(a) for a in arrs], H, F, _p(x), T, _p(out)), "dense_mlp")
    return out


def quant_act8(v: np.ndarray, block: int) -> np.ndarray:
    """The opt-in 8-bit activation rule on one row (fp64 in, fp64 values c * 2^-n out)."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty_like(v)
    _load().moe_ref_quant_act8(_p(v), v.size, int(block), _p(out))
    return out


def rmsnorm(h: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.float32)
    T, H = h.shape
    y = np.empty_like(h)
    _check(_load().moe_ref_rmsnorm(_p(h), T, H, eps, _p(y)), "rmsnorm")
    return y


def to_f32(out: np.ndarray) -> np.ndarray:
    """fp32 output mode: round-to-nearest-even of the fp64 result."""
    return out.astype(np.float32)


def to_bf16_bits(out: np.ndarray) -> np.ndarray:
    """bf16 output mode (uint16 bit patterns): RNE to fp32, then RNE to bf16."""
    f = out.astype(np.float32).view(np.uint32).astype(np.uint64)
    rounded = (f + 0x7FFF + ((f >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)

"""Python binding of the gfx950 MoE layer library (libmoe_gfx950.so).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels; PyTorch provides device memory and the current stream.  The entry
points mirror the C ABI in include/moe.h: ``moe_route``, ``moe_union``,
``moe_expert_ffn``, ``moe_layer_forward``, ``moe_workspace_bytes`` and
``moe_strerror``.  If the library has not been built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_gfx950.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EALIGN, MOE_EDEVICE = 0, -1, -2, -3, -4, -5
MOE_F32, MOE_BF16 = 0, 1
MOE_FMT_INT4_G64, MOE_FMT_MXFP4, MOE_FMT_INT3_G64 = 0, 1, 2
MOE_MAX_EXPERTS, MOE_MAX_TOPK, MOE_MAX_TOKENS, MOE_MAX_DIM = 256, 16, 4096, 16384

EXPORTS = ("moe_workspace_bytes", "moe_route", "moe_union", "moe_expert_ffn",
           "moe_layer_forward", "moe_residual_rmsnorm", "moe_strerror", "moe_prof_begin",
           "moe_prof_end", "moe_expert_ffn_probe", "moe_layer_forward_static", "moe_probe_read",
           "moe_dense_workspace_bytes", "moe_dense_forward", "moe_tier_slot_bytes",
           "moe_tier_state_bytes", "moe_tier_init", "moe_tier_layer_forward", "moe_tier_prefetch",
           "moe_tier_repin")
MOE_STATIC_SCRATCH_BYTES = 64 << 20
MOE_GU_SWIGLU, MOE_GU_GATE, MOE_GU_UP = 0, 1, 2


class MoeError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {strerror(code)} (code {code})")
        self.code = code


class Q4(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("s", ctypes.c_void_p)]


class LayerC(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("ffn", ctypes.c_int32),
        ("shared_ffn", ctypes.c_int32), ("top_k", ctypes.c_int32), ("top_p", ctypes.c_float),
        ("norm_topk", ctypes.c_int32), ("routed_scale", ctypes.c_float),
        ("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
        ("gate", Q4), ("up", Q4), ("down", Q4),
        ("sh_gate", Q4), ("sh_up", Q4), ("sh_down", Q4),
        ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32), ("act_bits", ctypes.c_int32),
        ("expert_fmt", ctypes.c_int32),
    ]


class DenseC(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("gate", Q4), ("up", Q4), ("down", Q4)]


class TierC(ctypes.Structure):
    _fields_ = [("n_slots", ctypes.c_int32), ("n_pinned", ctypes.c_int32),
                ("slots", ctypes.c_void_p), ("state", ctypes.c_void_p)]


class ProfStatC(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int32), ("ms", ctypes.c_double)]


class RouteOutC(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("ids", "w", "keff", "n_uniq", "uniq", "off", "row_tok", "pick_row")]


_lib = None


def lib():
    """The loaded library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    P = ctypes.POINTER(LayerC)
    L.moe_workspace_bytes.restype = sz
    L.moe_workspace_bytes.argtypes = [P, i32]
    L.moe_route.restype = ctypes.c_int
    L.moe_route.argtypes = [P, vp, i32, vp, vp, vp, vp, sz, vp]
    L.moe_union.restype = ctypes.c_int
    L.moe_union.argtypes = [P, vp, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_expert_ffn.restype = ctypes.c_int
    L.moe_expert_ffn.argtypes = [P, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_layer_forward.restype = ctypes.c_int
    L.moe_layer_forward.argtypes = [P, vp, i32, vp, i32, ctypes.POINTER(RouteOutC), vp, sz, vp]
    L.moe_residual_rmsnorm.restype = ctypes.c_int
    L.moe_residual_rmsnorm.argtypes = [vp, vp, i32, i32, ctypes.c_float, vp, vp, vp]
    L.moe_prof_begin.restype = ctypes.c_int
    L.moe_prof_begin.argtypes = []
    L.moe_prof_end.restype = ctypes.c_int
    L.moe_prof_end.argtypes = [ctypes.POINTER(ProfStatC), i32, ctypes.POINTER(i32)]
    L.moe_strerror.restype = ctypes.c_char_p
    L.moe_strerror.argtypes = [ctypes.c_int]
    L.moe_dense_workspace_bytes.restype = sz
    L.moe_dense_workspace_bytes.argtypes = [ctypes.POINTER(DenseC), i32]
    L.moe_dense_forward.restype = ctypes.c_int
    L.moe_dense_forward.argtypes = [ctypes.POINTER(DenseC), vp, i32, vp, i32, vp, sz, vp]
    T_ = ctypes.POINTER(TierC)
    L.moe_tier_slot_bytes.restype = sz
    L.moe_tier_slot_bytes.argtypes = [P]
    L.moe_tier_state_bytes.restype = sz
    L.moe_tier_state_bytes.argtypes = [P, i32]
    L.moe_tier_init.restype = ctypes.c_int
    L.moe_tier_init.argtypes = [P, T_, vp, i32, vp]
    L.moe_tier_layer_forward.restype = ctypes.c_int
    L.moe_tier_layer_forward.argtypes = [P, T_, vp, i32, vp, i32, ctypes.POINTER(RouteOutC), vp, sz, vp]
    L.moe_tier_prefetch.restype = ctypes.c_int
    L.moe_tier_prefetch.argtypes = [P, T_, vp, vp, i32, vp]
    L.moe_tier_repin.restype = ctypes.c_int
    L.moe_tier_repin.argtypes = [P, T_, i32, vp]
    L.moe_probe_read.restype = ctypes.c_int
    L.moe_probe_read.argtypes = [vp, sz, ctypes.c_uint32, vp, i32, vp]
    L.moe_layer_forward_static.restype = ctypes.c_int
    L.moe_layer_forward_static.argtypes = [P, vp, i32, vp, i32, ctypes.POINTER(RouteOutC), vp]
    L.moe_expert_ffn_probe.restype = ctypes.c_int
    L.moe_expert_ffn_probe.argtypes = [P, vp, i32, vp, vp, vp, vp, i32, vp, vp, sz, vp]
    _lib = L
    return L


def strerror(code: int) -> str:
    return lib().moe_strerror(code).decode()


def _check(code: int, what: str):
    if code != MOE_OK:
        raise MoeError(code, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


TENSORS = ("router_w", "router_bias", "gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s",
           "sh_gate_q", "sh_gate_s", "sh_up_q", "sh_up_s", "sh_down_q", "sh_down_s")
PARAMS = ("hidden", "n_experts", "ffn", "shared_ffn", "top_k", "top_p", "norm_topk",
          "routed_scale")


class Layer:
    """A layer's hyper-parameters and device tensors, plus its C description."""

    def __init__(self, params: dict, tensors: dict):
        self.params = {k: params[k] for k in PARAMS}
        self.params.update(n_group=int(params.get("n_group", 0)), topk_group=int(params.get("topk_group", 0)),
                           act_bits=int(params.get("act_bits", 0)),
                           expert_fmt=int(params.get("expert_fmt", MOE_FMT_INT4_G64)))
        self.t = dict(tensors)
        c = LayerC()
        c.hidden, c.n_experts = int(params["hidden"]), int(params["n_experts"])
        c.ffn, c.shared_ffn, c.top_k = int(params["ffn"]), int(params["shared_ffn"]), int(params["top_k"])
        c.top_p, c.norm_topk = float(params["top_p"]), int(params["norm_topk"])
        c.routed_scale = float(params["routed_scale"])
        c.n_group, c.topk_group = self.params["n_group"], self.params["topk_group"]
        c.act_bits = self.params["act_bits"]
        c.expert_fmt = self.params["expert_fmt"]
        g = self.t.get
        c.router_w = _ptr(g("router_w"))
        c.router_bias = _ptr(g("router_bias"))
        for name in ("gate", "up", "down", "sh_gate", "sh_up", "sh_down"):
            q, s = g(name + "_q"), g(name + "_s")
            setattr(c, name, Q4(_ptr(q) if q is not None and q.numel() else None,
                                _ptr(s) if s is not None and s.numel() else None))
        self.c = c
        self.hidden, self.n_experts, self.top_k = c.hidden, c.n_experts, c.top_k

    @classmethod
    def from_host(cls, d: dict, device="cuda"):
        """Copies a host layer (numpy arrays, as made by the input generator) to the device."""
        import torch
        ts = {}
        for k in TENSORS:
            v = d.get(k)
            if v is None:
                continue
            ts[k] = torch.from_numpy(np.ascontiguousarray(v)).to(device)
        return cls(d, ts)

    def ref(self):
        return ctypes.byref(self.c)

    def workspace_bytes(self, T: int) -> int:
        n = lib().moe_workspace_bytes(self.ref(), int(T))
        if n == 0:
            raise MoeError(MOE_EINVAL, "moe_workspace_bytes")
        return int(n)

    def workspace(self, T: int, device="cuda"):
        import torch
        return torch.empty(self.workspace_bytes(T), dtype=torch.uint8, device=device)


def moe_route(layer: Layer, x, ids=None, w=None, keff=None, ws=None, stream=None):
    import torch
    T, k = x.shape[0], layer.top_k
    dev = x.device
    ids = torch.empty((T, k), dtype=torch.int32, device=dev) if ids is None else ids
    w = torch.empty((T, k), dtype=torch.float32, device=dev) if w is None else w
    keff = torch.empty((T,), dtype=torch.int32, device=dev) if keff is None else keff
    ws = layer.workspace(T, dev) if ws is None else ws
    _check(lib().moe_route(layer.ref(), _ptr(x), T, _ptr(ids), _ptr(w), _ptr(keff), _ptr(ws),
                           ws.numel(), _stream(stream)), "moe_route")
    return ids, w, keff


def moe_union(layer: Layer, ids, keff, ws=None, stream=None, out=None):
    import torch
    T, k, E = ids.shape[0], layer.top_k, layer.n_experts
    dev = ids.device
    if out is None:
        out = dict(n_uniq=torch.empty((1,), dtype=torch.int32, device=dev),
                   uniq=torch.empty((E,), dtype=torch.int32, device=dev),
                   off=torch.empty((E + 1,), dtype=torch.int32, device=dev),
                   row_tok=torch.empty((max(T * k, 1),), dtype=torch.int32, device=dev),
                   pick_row=torch.empty((max(T, 1), k), dtype=torch.int32, device=dev))
    ws = layer.workspace(T, dev) if ws is None else ws
    _check(lib().moe_union(layer.ref(), _ptr(ids), _ptr(keff), T, _ptr(out["n_uniq"]),
                           _ptr(out["uniq"]), _ptr(out["off"]), _ptr(out["row_tok"]),
                           _ptr(out["pick_row"]), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_union")
    return out


def moe_expert_ffn(layer: Layer, x, un: dict, y_rows=None, ws=None, stream=None):
    import torch
    T, k, H = x.shape[0], layer.top_k, layer.hidden
    y_rows = torch.zeros((max(T * k, 1), H), dtype=torch.float32, device=x.device) if y_rows is None else y_rows
    ws = layer.workspace(T, x.device) if ws is None else ws
    _check(lib().moe_expert_ffn(layer.ref(), _ptr(x), T, _ptr(un["n_uniq"]), _ptr(un["uniq"]),
                                _ptr(un["off"]), _ptr(un["row_tok"]), _ptr(y_rows), _ptr(ws),
                                ws.numel(), _stream(stream)), "moe_expert_ffn")
    return y_rows


def moe_layer_forward(layer: Layer, x, out=None, out_dtype: int = MOE_F32, dbg: dict | None = None,
                      ws=None, stream=None):
    """out [T][H] (fp32, or bf16 for MOE_BF16).  ``dbg`` maps moe_route_out member names to
    device tensors that receive the routing/union outputs."""
    import torch
    T, H = x.shape[0], layer.hidden
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16 if out_dtype == MOE_BF16 else torch.float32,
                          device=x.device)
    ws = layer.workspace(T, x.device) if ws is None else ws
    rc = None
    if dbg:
        rc = RouteOutC(**{k: (v.data_ptr() if v is not None else None) for k, v in dbg.items()})
    _check(lib().moe_layer_forward(layer.ref(), _ptr(x), T, _ptr(out), out_dtype,
                                   ctypes.byref(rc) if rc is not None else None, _ptr(ws),
                                   ws.numel(), _stream(stream)), "moe_layer_forward")
    return out


def moe_layer_forward_static(layer: Layer, x, out=None, out_dtype: int = MOE_F32,
                             dbg: dict | None = None, stream=None):
    """moe_layer_forward without a workspace: the library's own device scratch array
    (MOE_STATIC_SCRATCH_BYTES per GPU) serves as scratch; nothing is allocated."""
    import torch
    T, H = x.shape[0], layer.hidden
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16 if out_dtype == MOE_BF16 else torch.float32,
                          device=x.device)
    rc = None
    if dbg:
        rc = RouteOutC(**{k: (v.data_ptr() if v is not None else None) for k, v in dbg.items()})
    _check(lib().moe_layer_forward_static(layer.ref(), _ptr(x), T, _ptr(out), out_dtype,
                                          ctypes.byref(rc) if rc is not None else None,
                                          _stream(stream)), "moe_layer_forward_static")
    return out


class Dense:
    """A first-dense layer's device tensors (int4-gs64 gate/up [F][H], down [H][F]) and its C
    description."""

    def __init__(self, tensors: dict):
        self.t = dict(tensors)
        c = DenseC()
        F, h2 = self.t["gate_q"].shape
        c.hidden, c.ffn = int(h2) * 2, int(F)
        for name in ("gate", "up", "down"):
            setattr(c, name, Q4(_ptr(self.t[name + "_q"]), _ptr(self.t[name + "_s"])))
        self.c = c
        self.hidden, self.ffn = c.hidden, c.ffn

    @classmethod
    def from_host(cls, d: dict, device="cuda"):
        import torch
        return cls({k: torch.from_numpy(np.ascontiguousarray(d[k])).to(device)
                    for k in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")})

    def ref(self):
        return ctypes.byref(self.c)

    def workspace(self, T: int, device="cuda"):
        import torch
        n = lib().moe_dense_workspace_bytes(self.ref(), int(T))
        if n == 0:
            raise MoeError(MOE_EINVAL, "moe_dense_workspace_bytes")
        return torch.empty(int(n), dtype=torch.uint8, device=device)


def moe_dense_forward(dense: Dense, x, out=None, out_dtype: int = MOE_F32, ws=None, stream=None):
    """First-dense-layer SwiGLU MLP on every token: out [T][H] fp32 or bf16."""
    import torch
    T, H = x.shape[0], dense.hidden
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16 if out_dtype == MOE_BF16 else torch.float32,
                          device=x.device)
    ws = dense.workspace(T, x.device) if ws is None else ws
    _check(lib().moe_dense_forward(dense.ref(), _ptr(x), T, _ptr(out), out_dtype, _ptr(ws), ws.numel(),
                                   _stream(stream)), "moe_dense_forward")
    return out


class Tier:
    """A residency tier for one layer: n_slots HBM slots (the first n_pinned pinned) over
    the layer's routed experts, which live in pinned host memory (see moe.h)."""

    def __init__(self, layer: Layer, n_slots: int, n_pinned: int = 0, device="cuda"):
        import torch
        L = lib()
        self.layer = layer
        self.slot_bytes = int(L.moe_tier_slot_bytes(layer.ref()))
        nb = int(L.moe_tier_state_bytes(layer.ref(), int(n_slots)))
        if self.slot_bytes == 0 or nb == 0:
            raise MoeError(MOE_EINVAL, "moe_tier_*_bytes")
        self.slots = torch.empty(int(n_slots) * self.slot_bytes + 256, dtype=torch.uint8, device=device)
        self.state = torch.empty(nb + 256, dtype=torch.uint8, device=device)
        sp, tp = _align256(self.slots.data_ptr()), _align256(self.state.data_ptr())
        self.c = TierC(int(n_slots), int(n_pinned), sp, tp)
        self._state_off = tp - self.state.data_ptr()
        self.n_slots, self.n_pinned, self.state_bytes = int(n_slots), int(n_pinned), nb

    def ref(self):
        return ctypes.byref(self.c)

    def init(self, pins=(), stream=None):
        arr = (ctypes.c_int32 * max(len(pins), 1))(*[int(p) for p in pins])
        _check(lib().moe_tier_init(self.layer.ref(), self.ref(), arr, len(pins), _stream(stream)),
               "moe_tier_init")

    def forward(self, x, out=None, out_dtype: int = MOE_F32, dbg: dict | None = None, ws=None,
                stream=None):
        import torch
        T, H = x.shape[0], self.layer.hidden
        if out is None:
            out = torch.empty((T, H), dtype=torch.bfloat16 if out_dtype == MOE_BF16 else torch.float32,
                              device=x.device)
        ws = self.layer.workspace(T, x.device) if ws is None else ws
        rc = None
        if dbg:
            rc = RouteOutC(**{k: (v.data_ptr() if v is not None else None) for k, v in dbg.items()})
        _check(lib().moe_tier_layer_forward(self.layer.ref(), self.ref(), _ptr(x), T, _ptr(out), out_dtype,
                                            ctypes.byref(rc) if rc is not None else None, _ptr(ws),
                                            ws.numel(), _stream(stream)), "moe_tier_layer_forward")
        return out

    def prefetch(self, ids, keff, stream=None):
        _check(lib().moe_tier_prefetch(self.layer.ref(), self.ref(), _ptr(ids), _ptr(keff),
                                       ids.shape[0], _stream(stream)), "moe_tier_prefetch")

    def repin(self, max_swaps: int = 4, stream=None):
        _check(lib().moe_tier_repin(self.layer.ref(), self.ref(), int(max_swaps), _stream(stream)),
               "moe_tier_repin")

    def read_state(self) -> dict:
        """The state arrays (waits for the device), in the layout moe.h documents."""
        import torch
        torch.cuda.synchronize()
        b = self.state[self._state_off:self._state_off + self.state_bytes].cpu().numpy()
        S, E = self.n_slots, self.layer.n_experts
        w = b.view(np.int32)
        o = 0

        def take(n):
            nonlocal o
            a = w[o:o + n].copy()
            o += n
            return a
        hdr = take(16)
        st = dict(step=int(hdr[0]), copies_last=int(hdr[1]), hits=int(hdr[2]), misses=int(hdr[3]),
                  swaps=int(hdr[4]), prefetched=int(hdr[5]))
        st["slot_expert"], st["slot_pinned"], st["slot_used"] = take(S), take(S), take(S)
        st["expert_slot"] = take(E)
        st["heat"], st["usage"] = take(E).view(np.uint32), take(E).view(np.uint32)
        mc = max(min(E, S), 4)
        cp = take(2 * mc).reshape(mc, 2)
        st["copies"] = [tuple(int(v) for v in cp[i]) for i in range(st["copies_last"])]
        return st


def _align256(p: int) -> int:
    return (p + 255) // 256 * 256


def moe_residual_rmsnorm(h, delta=None, eps: float = 1e-6, h_out=None, x_out=None, stream=None):
    """h_out = h + delta; x_out = RMSNorm(h_out) (unit gain).  Returns (h_out, x_out)."""
    import torch
    T, H = h.shape
    h_out = torch.empty_like(h) if h_out is None else h_out
    x_out = torch.empty_like(h) if x_out is None else x_out
    _check(lib().moe_residual_rmsnorm(_ptr(h), _ptr(delta), T, H, eps, _ptr(h_out), _ptr(x_out),
                                      _stream(stream)), "moe_residual_rmsnorm")
    return h_out, x_out


def moe_prof_begin():
    _check(lib().moe_prof_begin(), "moe_prof_begin")


def moe_prof_end() -> dict:
    """{kernel name: (launches, total ms)} since moe_prof_begin (waits for the events)."""
    buf = (ProfStatC * 64)()
    n = ctypes.c_int32(0)
    _check(lib().moe_prof_end(buf, 64, ctypes.byref(n)), "moe_prof_end")
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].ms)) for i in range(min(n.value, 64))}


def moe_expert_ffn_probe(layer: Layer, x, un: dict, gate_up_output: int, y_rows=None, ws=None,
                         stream=None):
    """Test entry point: moe_expert_ffn with the gate/up step handing the down projection
    SiLU(g) * u (MOE_GU_SWIGLU), the gate pre-activation (MOE_GU_GATE) or the up
    pre-activation (MOE_GU_UP), chosen for this call only."""
    import torch
    T, k, H = x.shape[0], layer.top_k, layer.hidden
    y_rows = torch.zeros((max(T * k, 1), H), dtype=torch.float32, device=x.device) if y_rows is None else y_rows
    ws = layer.workspace(T, x.device) if ws is None else ws
    _check(lib().moe_expert_ffn_probe(layer.ref(), _ptr(x), T, _ptr(un["n_uniq"]), _ptr(un["uniq"]),
                                      _ptr(un["off"]), _ptr(un["row_tok"]), int(gate_up_output),
                                      _ptr(y_rows), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_expert_ffn_probe")
    return y_rows

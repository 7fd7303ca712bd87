"""Python binding of the plain C++ fp64 oracle (oracle/cpp/*.cpp).

TEST INFRASTRUCTURE ONLY: part of the plain CPU oracle.  Only tests/,
__graft_entry__.smoke() and the CPU-baseline leg of bench.py may load it;
the product path never does, and nothing here touches the GPU library.

This is argument marshalling only: every step (decoders, router, top-k,
SwiGLU experts, combine, stack, LM head) runs in the C++ sources, which are
the definitions written out as loops (see the header of oracle/cpp/moe.cpp).
The numpy functions in oracle/moe.py, oracle/lmhead.py and oracle/formats.py
compute the same definitions independently; both are pinned by the tests
(tests/test_oracle_*.py).

build() compiles oracle/liboracle_cpp.so with g++ (-O2, OpenMP, no
floating-point contraction or fast-math, so every product and sum is the
plain IEEE fp64 operation).  Layers are taken as oracle.moe.Layer objects or
the dicts of synth.make_layer; stored formats as in oracle/formats.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = [os.path.join(_HERE, "cpp", n) for n in ("moe.cpp", "lmhead.cpp")]
_HDR = os.path.join(_HERE, "cpp", "formats.h")
_LIB = os.path.join(_HERE, "liboracle_cpp.so")
_lib = None


def build() -> str:
    """Compile the C++ oracle (always from source)."""
    tmp = _LIB + ".tmp"
    cmd = ["g++", "-std=c++17", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-o", tmp] + _SRC
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or any(os.path.getmtime(s) > os.path.getmtime(_LIB) for s in _SRC + [_HDR]):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, f64 = ctypes.c_longlong, ctypes.c_double
        sig = {
            "orc_abi_version": (ctypes.c_int, []),
            "orc_set_threads": (None, [ctypes.c_int]),
            "orc_get_threads": (ctypes.c_int, []),
            "orc_hw_threads": (ctypes.c_int, []),
            "orc_decode": (None, [ctypes.c_int, P, i64, P]),
            "orc_to_bf16": (None, [P, i64, P]),
            "orc_to_f16": (None, [P, i64, P]),
            "orc_unpack_codes": (None, [P, i64, ctypes.c_int, P]),
            "orc_pack_codes": (None, [P, i64, ctypes.c_int, P]),
            "orc_dequant": (None, [P, P, ctypes.c_float, ctypes.c_int, i64, ctypes.c_int, P]),
            "orc_quantize_int4": (None, [P, i64, ctypes.c_int, P, P]),
            "orc_router": (None, [P, P, P]),
            "orc_route": (None, [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P]),
            "orc_moe_forward": (None, [P, P, ctypes.c_int, ctypes.c_int, P, P, P, P, P]),
            "orc_moe_forward_on_set": (None, [P, P, P, ctypes.c_int, ctypes.c_int, P, P]),
            "orc_moe_forward_masked": (None, [P, P, ctypes.c_int, ctypes.c_int, P, P]),
            "orc_rmsnorm_bf16": (None, [P, ctypes.c_int, f64, P]),
            "orc_stack_forward": (None, [P, ctypes.c_int, P, ctypes.c_int, f64, ctypes.c_int, P, P, P, P]),
            "orc_group_by_expert": (None, [P, ctypes.c_int, ctypes.c_int, P, P, P, P]),
            "orc_lmhead": (None, [P, P, ctypes.c_int, ctypes.c_int, P, ctypes.c_int, P, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def get_threads() -> int:
    return lib().orc_get_threads()


def hw_threads() -> int:
    """std::thread::hardware_concurrency() of this host."""
    return lib().orc_hw_threads()


# ------------------------------------------------------------------ formats


def _decode(kind: int, a, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=dtype)
    out = np.empty(a.shape, np.float64)
    lib().orc_decode(kind, _p(a), a.size, _p(out))
    return out


def bf16_to_f64(bits):
    return _decode(0, bits, np.uint16)


def f16_to_f64(bits):
    return _decode(1, bits, np.uint16)


def e2m1_to_f64(codes):
    return _decode(2, codes, np.uint8)


def e8m0_to_f64(b):
    return _decode(3, b, np.uint8)


def e4m3_to_f64(b):
    return _decode(4, b, np.uint8)


def f64_to_bf16_bits(x):
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    lib().orc_to_bf16(_p(x), x.size, _p(out))
    return out


def f64_to_f16_bits(x):
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    lib().orc_to_f16(_p(x), x.size, _p(out))
    return out


def unpack_codes(q, K: int) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    rows = q.size // (K // 2)
    u = np.empty(q.shape[:-1] + (K,), np.uint8)
    lib().orc_unpack_codes(_p(q), rows, K, _p(u))
    return u


def pack_codes(u) -> np.ndarray:
    u = np.ascontiguousarray(u, dtype=np.uint8)
    K = u.shape[-1]
    q = np.empty(u.shape[:-1] + (K // 2,), np.uint8)
    lib().orc_pack_codes(_p(u), u.size // K, K, _p(q))
    return q


def dequant(q, s, K: int, fmt: int = 0, ts: float = 1.0) -> np.ndarray:
    """Stored matrix [..][K/2] (fmt 0 int4, 1 MXFP4, 2 NVFP4 with matrix scale ts) -> fp64."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint16 if fmt == 0 else np.uint8)
    w = np.empty(q.shape[:-1] + (K,), np.float64)
    lib().orc_dequant(_p(q), _p(s), float(ts), fmt, q.size // (K // 2), K, _p(w))
    return w


def quantize(w):
    """fp32 [..][K] -> (codes u [..][K], binary16 scale bits [..][K/32])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    K = w.shape[-1]
    u = np.empty(w.shape, np.uint8)
    s = np.empty(w.shape[:-1] + (K // 32,), np.uint16)
    lib().orc_quantize_int4(_p(w), w.size // K, K, _p(u), _p(s))
    return u.astype(np.int64), s


# ------------------------------------------------------------------ layers


class _Mat(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("s", ctypes.c_void_p), ("ts", ctypes.c_void_p)]


class _Layer(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("f", ctypes.c_int32), ("E", ctypes.c_int32), ("fmt", ctypes.c_int32),
                ("has_shared", ctypes.c_int32), ("pad", ctypes.c_int32),
                ("router_w", ctypes.c_void_p), ("router_b", ctypes.c_void_p),
                ("gate", _Mat), ("up", _Mat), ("down", _Mat),
                ("sh_gate", _Mat), ("sh_up", _Mat), ("sh_down", _Mat)]


def _get(layer, name):
    if isinstance(layer, dict):
        return layer.get(name)
    if name.startswith("shared_") and name[7:] in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s"):
        sh = getattr(layer, "shared", None)
        if sh is None:
            return None
        return sh[("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s").index(name[7:])]
    if name.endswith("_ts"):
        ts = getattr(layer, "tscales", None)
        return None if ts is None else ts.get(name)
    return getattr(layer, name)


class CLayer:
    """A layer's arrays held contiguous for the C++ oracle, with its struct."""

    def __init__(self, layer):
        self.keep = []
        rw = self._arr(_get(layer, "router_w"), np.float32)
        E, d = rw.shape
        f = _get(layer, "gate_q").shape[-2]
        gs = np.asarray(_get(layer, "gate_s"))
        nv = _get(layer, "gate_ts") is not None
        fmt = 2 if nv else (1 if gs.dtype == np.uint8 else 0)
        sdt = np.uint16 if fmt == 0 else np.uint8
        st = _Layer(d=d, f=f, E=E, fmt=fmt)
        st.router_w = self._ptr(rw)
        rb = _get(layer, "router_b")
        st.router_b = None if rb is None else self._ptr(self._arr(rb, np.float32))

        def mat(prefix):
            q = _get(layer, prefix + "_q")
            if q is None:
                return None
            m = _Mat(self._ptr(self._arr(q, np.uint8)), self._ptr(self._arr(_get(layer, prefix + "_s"), sdt)), None)
            ts = _get(layer, prefix + "_ts")
            if nv:
                m.ts = self._ptr(self._arr(np.atleast_1d(np.asarray(ts, np.float32)), np.float32))
            return m

        st.gate, st.up, st.down = mat("gate"), mat("up"), mat("down")
        sh = mat("shared_gate")
        if sh is not None:
            st.has_shared = 1
            st.sh_gate, st.sh_up, st.sh_down = sh, mat("shared_up"), mat("shared_down")
        self.st, self.E, self.d, self.f = st, E, d, f

    def _arr(self, a, dt):
        a = np.ascontiguousarray(a, dtype=dt)
        self.keep.append(a)
        return a

    @staticmethod
    def _ptr(a):
        return a.ctypes.data_as(ctypes.c_void_p).value

    @property
    def ref(self):
        return ctypes.byref(self.st)


def as_clayer(layer) -> CLayer:
    return layer if isinstance(layer, CLayer) else CLayer(layer)


def router_logits(layer, x_bits) -> np.ndarray:
    L = as_clayer(layer)
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    out = np.empty(L.E, np.float64)
    lib().orc_router(L.ref, _p(x), _p(out))
    return out


def route(l, k: int, norm_topk: bool = True):
    l = np.ascontiguousarray(l, dtype=np.float64)
    S = np.empty(k, np.int32)
    w = np.empty(k, np.float64)
    lib().orc_route(_p(l), l.size, k, int(norm_topk), _p(S), _p(w))
    return S.astype(np.int64), w


def moe_forward(layer, x_bits, k: int, norm_topk: bool = True) -> dict:
    """One bf16 token through one layer (only the chosen experts run)."""
    L = as_clayer(layer)
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    y = np.empty(L.d, np.float64)
    idx = np.empty(k, np.int32)
    w = np.empty(k, np.float64)
    lg = np.empty(L.E, np.float64)
    rd = ctypes.c_longlong(0)
    lib().orc_moe_forward(L.ref, _p(x), k, int(norm_topk), _p(y), _p(idx), _p(w), _p(lg), ctypes.byref(rd))
    return dict(y=y, y32=y.astype(np.float32), idx=idx.astype(np.int64), w=w, logits=lg, weights_read=rd.value)


def moe_forward_tokens(layer, X_bits, k: int, norm_topk: bool = True) -> dict:
    """T tokens, each routed on its own (row t of X is token t)."""
    L = as_clayer(layer)
    rs = [moe_forward(L, X_bits[t], k, norm_topk) for t in range(X_bits.shape[0])]
    return {n: np.stack([r[n] for r in rs]) for n in ("y", "y32", "idx", "w", "logits")}


def moe_forward_on_set(layer, x_bits, S, norm_topk: bool = True) -> dict:
    L = as_clayer(layer)
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    S = np.ascontiguousarray(S, dtype=np.int32)
    y = np.empty(L.d, np.float64)
    w = np.empty(S.size, np.float64)
    lib().orc_moe_forward_on_set(L.ref, _p(x), _p(S), S.size, int(norm_topk), _p(y), _p(w))
    return dict(y=y, y32=y.astype(np.float32), idx=S.astype(np.int64), w=w)


def moe_forward_masked(layer, x_bits, k: int, norm_topk: bool = True):
    """Brute force (all experts, then the 0/1 mask): (y, weights read)."""
    L = as_clayer(layer)
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    y = np.empty(L.d, np.float64)
    rd = ctypes.c_longlong(0)
    lib().orc_moe_forward_masked(L.ref, _p(x), k, int(norm_topk), _p(y), ctypes.byref(rd))
    return y, rd.value


def rmsnorm_bf16(r, eps: float) -> np.ndarray:
    r = np.ascontiguousarray(r, dtype=np.float32)
    x = np.empty(r.shape, np.uint16)
    lib().orc_rmsnorm_bf16(_p(r), r.size, float(eps), _p(x))
    return x


def stack_forward(layers, x0_bits, k: int, eps: float = 1e-6, norm_topk: bool = True) -> dict:
    """Pre-norm residual stack; r, xs, ys and idx as in oracle.moe.stack_forward."""
    Ls = [as_clayer(l) for l in layers]
    n, d = len(Ls), Ls[0].d
    arr = (ctypes.c_void_p * n)(*[ctypes.addressof(L.st) for L in Ls])
    x0 = np.ascontiguousarray(x0_bits, dtype=np.uint16)
    r = np.empty(d, np.float32)
    xs = np.empty((n, d), np.uint16)
    ys = np.empty((n, d), np.float32)
    idx = np.empty((n, k), np.int32)
    lib().orc_stack_forward(arr, n, _p(x0), k, float(eps), int(norm_topk), _p(r), _p(xs), _p(ys), _p(idx))
    return dict(r=r, xs=list(xs), ys=list(ys), idx=[i.astype(np.int64) for i in idx])


def group_by_expert(idx, E: int):
    flat = np.ascontiguousarray(np.asarray(idx).reshape(-1), dtype=np.int32)
    off = np.empty(E + 1, np.int32)
    order = np.empty(flat.size, np.int32)
    active = np.empty(E, np.int32)
    na = ctypes.c_int32(0)
    lib().orc_group_by_expert(_p(flat), flat.size, E, _p(off), _p(order), _p(active), ctypes.byref(na))
    return off.astype(np.int64), order.astype(np.int64), active[:na.value].astype(np.int64)


def lmhead_argmax(w_q, w_s, x_bits, want_logits: bool = True):
    """(token [B], max logit [B], logits [B][V] or None) of the int4 LM head."""
    wq = np.ascontiguousarray(w_q, dtype=np.uint8)
    ws = np.ascontiguousarray(w_s, dtype=np.uint16)
    X = np.ascontiguousarray(np.atleast_2d(x_bits), dtype=np.uint16)
    V, d = wq.shape[0], 2 * wq.shape[1]
    B = X.shape[0]
    tok = np.empty(B, np.int32)
    zmax = np.empty(B, np.float64)
    z = np.empty((B, V), np.float64) if want_logits else None
    lib().orc_lmhead(_p(wq), _p(ws), V, d, _p(X), B, _p(tok), _p(zmax), _p(z))
    return tok.astype(np.int64), zmax, z

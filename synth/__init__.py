"""Seeded synthetic inputs for the MoE decode path (shared by tests and bench).

This module holds the input recipe only: shapes of the five workloads, the
counter-based random streams, normal draws, bf16 activations, the offline int4
(and MXFP4) quantize-and-pack steps that produce stored weights, and the Zipf popularity
bias of the batched workload.  It contains none of the decode step's
arithmetic, and it imports neither the oracle nor the GPU library.

Workloads (the pages give no hidden or expert widths; these shapes reproduce
the pages' totals: 256 routed experts per MoE layer and a 4-bit output layer,
"Flint 40B: Best Mid Sized LLM", transcript 02:35-04:07):

  tiny     d=256  f=128 E=16  k=2 T=1   router N(0,0.05), experts N(0,0.02)
  layer    d=2048 f=512 E=256 k=8 T=1   router N(0,0.02), experts N(0,0.02)
  batch    layer shapes, T=64, router bias ln p_e with Zipf(1.1) popularity
  stack    49 independent layers of the `layer` shape, T=1
  lmhead   V=131072 d=2048, B in {1, 8}, weights N(0,0.02)

Activations are bf16 N(0,1).  Margin resampling (drawing x again, with the
next attempt counter, until the top-k logit margin holds) needs the router and
so is done by the callers that own an oracle; this module only hands out the
draw for a given attempt.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_SRC_NORMAL = os.path.join(_HERE, "normal.c")
_OBJ_NORMAL = os.path.join(_HERE, "normal.o")
_LIB = os.path.join(_HERE, "libsynth.so")

# normal.c alone is built with -ffast-math (vector math); the link step is not,
# so the library does not switch the process to flush-to-zero.
GCC_NORMAL = ["gcc", "-O3", "-ffast-math", "-fopenmp-simd", "-fPIC", "-c", "-o", _OBJ_NORMAL, _SRC_NORMAL]
GCC_LIB = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", _LIB, _SRC, _OBJ_NORMAL, "-lm", "-lmvec"]


def build() -> str:
    """Compile libsynth.so in place (always recompiles)."""
    subprocess.check_call(GCC_NORMAL)
    subprocess.check_call(GCC_LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        u64, i64, p, d = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
        L.synth_key.restype = u64
        L.synth_key.argtypes = [u64, u64]
        L.synth_u64.restype = u64
        L.synth_u64.argtypes = [u64, u64]
        L.synth_normal_f32.argtypes = [p, i64, u64, d, d]
        L.synth_bf16.argtypes = [p, i64, u64, d, d]
        L.synth_int4.argtypes = [p, p, i64, i64, u64, d, p]
        L.synth_int4_experts.argtypes = [p, p, i64, i64, i64, u64, d]
        L.synth_quantize_pack.argtypes = [p, i64, i64, p, p]
        L.synth_mxfp4_experts.argtypes = [p, p, i64, i64, i64, u64, d]
        L.synth_quantize_pack_mxfp4.argtypes = [p, i64, i64, p, p]
        L.synth_nvfp4_experts.argtypes = [p, p, p, i64, i64, i64, u64, d]
        L.synth_quantize_nvfp4.restype = ctypes.c_float
        L.synth_quantize_nvfp4.argtypes = [p, i64, i64, p, p]
        L.synth_pack_codes.argtypes = [p, i64, i64, p]
        L.synth_permutation.argtypes = [p, ctypes.c_int32, u64]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# ---------------------------------------------------------------- keys

_TAGS = {"router": 1, "gate": 2, "up": 3, "down": 4, "bias": 5, "x": 6, "lmhead": 7}


def key(*path: int | str) -> int:
    """Derive a stream key from a path of integer or named tags."""
    k = 0x5EED
    for t in path:
        if isinstance(t, str):
            t = _TAGS.get(t, None) if t in _TAGS else int.from_bytes(t.encode()[:8].ljust(8, b"\0"), "little")
        k = lib().synth_key(k, int(t) & 0xFFFFFFFFFFFFFFFF)
    return k


# ---------------------------------------------------------------- draws


def normal_f32(n: int, k: int, mu: float = 0.0, sigma: float = 1.0) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().synth_normal_f32(_ptr(out), n, k, mu, sigma)
    return out


def bf16(n: int, k: int, mu: float = 0.0, sigma: float = 1.0) -> np.ndarray:
    """n bf16 values (as uint16 bit patterns), N(mu, sigma) rounded RNE."""
    out = np.empty(n, np.uint16)
    lib().synth_bf16(_ptr(out), n, k, mu, sigma)
    return out


def int4_matrix(rows: int, K: int, k: int, sigma: float, with_fp32: bool = False):
    """Quantized N(0, sigma) matrix: (packed uint8 [rows][K/2], scales uint16 [rows][K/32][, fp32 draws])."""
    assert K % 128 == 0
    q = np.empty((rows, K // 2), np.uint8)
    s = np.empty((rows, K // 32), np.uint16)
    w = np.empty((rows, K), np.float32) if with_fp32 else None
    lib().synth_int4(_ptr(q), _ptr(s), rows, K, k, sigma, _ptr(w) if with_fp32 else None)
    return (q, s, w) if with_fp32 else (q, s)


def int4_experts(E: int, rows: int, K: int, k: int, sigma: float):
    q = np.empty((E, rows, K // 2), np.uint8)
    s = np.empty((E, rows, K // 32), np.uint16)
    lib().synth_int4_experts(_ptr(q), _ptr(s), E, rows, K, k, sigma)
    return q, s


def mxfp4_experts(E: int, rows: int, K: int, k: int, sigma: float):
    """MXFP4 counterpart of int4_experts (same draws): codes uint8 [E][rows][K/2], E8M0 bytes [E][rows][K/32]."""
    q = np.empty((E, rows, K // 2), np.uint8)
    s = np.empty((E, rows, K // 32), np.uint8)
    lib().synth_mxfp4_experts(_ptr(q), _ptr(s), E, rows, K, k, sigma)
    return q, s


def nvfp4_experts(E: int, rows: int, K: int, k: int, sigma: float):
    """NVFP4 counterpart of int4_experts (same draws): codes uint8 [E][rows][K/2],
    E4M3 bytes [E][rows][K/16], fp32 tensor scales [E]."""
    q = np.empty((E, rows, K // 2), np.uint8)
    s = np.empty((E, rows, K // 16), np.uint8)
    t = np.empty(E, np.float32)
    lib().synth_nvfp4_experts(_ptr(q), _ptr(s), _ptr(t), E, rows, K, k, sigma)
    return q, s, t


def quantize_nvfp4(w: np.ndarray):
    """Quantize a caller-given fp32 matrix [rows][K] into stored NVFP4 (codes, scale bytes, tensor scale)."""
    w = np.ascontiguousarray(w, np.float32)
    rows, K = w.shape
    assert K % 128 == 0
    q = np.empty((rows, K // 2), np.uint8)
    s = np.empty((rows, K // 16), np.uint8)
    t = lib().synth_quantize_nvfp4(_ptr(w), rows, K, _ptr(q), _ptr(s))
    return q, s, np.float32(t)


def quantize_pack_mxfp4(w: np.ndarray):
    """Quantize caller-given fp32 weights [rows][K] into stored MXFP4."""
    w = np.ascontiguousarray(w, np.float32)
    rows, K = w.shape
    assert K % 128 == 0
    q = np.empty((rows, K // 2), np.uint8)
    s = np.empty((rows, K // 32), np.uint8)
    lib().synth_quantize_pack_mxfp4(_ptr(w), rows, K, _ptr(q), _ptr(s))
    return q, s


def quantize_pack(w: np.ndarray):
    """Quantize caller-given fp32 weights [rows][K] into the stored format."""
    w = np.ascontiguousarray(w, np.float32)
    rows, K = w.shape
    assert K % 128 == 0
    q = np.empty((rows, K // 2), np.uint8)
    s = np.empty((rows, K // 32), np.uint16)
    lib().synth_quantize_pack(_ptr(w), rows, K, _ptr(q), _ptr(s))
    return q, s


def pack_codes(u: np.ndarray) -> np.ndarray:
    """Pack codes u[rows][K] in 0..15 into the stored nibble layout."""
    u = np.ascontiguousarray(u, np.uint8)
    rows, K = u.shape
    assert K % 128 == 0 and u.max(initial=0) <= 15
    q = np.empty((rows, K // 2), np.uint8)
    lib().synth_pack_codes(_ptr(u), rows, K, _ptr(q))
    return q


def permutation(n: int, k: int) -> np.ndarray:
    out = np.empty(n, np.int32)
    lib().synth_permutation(_ptr(out), n, k)
    return out


# ---------------------------------------------------------------- workloads


@dataclass(frozen=True)
class MoEConfig:
    name: str
    d: int
    f: int
    E: int
    k: int
    T: int = 1
    router_sigma: float = 0.02
    expert_sigma: float = 0.02
    zipf_s: float = 0.0      # >0: router bias b_e = ln p_e, p_e ~ rank^-s
    layers: int = 1
    margin: float = 1e-2
    shared: int = 0          # always-on experts (0 or 1), same shape, weight 1
    fmt: str = "int4"        # expert weights: "int4" (fp16 scales), "mxfp4" (E2M1, E8M0 scales) or "nvfp4"


@dataclass(frozen=True)
class LMHeadConfig:
    name: str
    V: int
    d: int
    B: int
    sigma: float = 0.02
    margin: float = 1e-2


TINY = MoEConfig("tiny", d=256, f=128, E=16, k=2, router_sigma=0.05)
LAYER = MoEConfig("layer", d=2048, f=512, E=256, k=8)
BATCH = replace(LAYER, name="batch", T=64, zipf_s=1.1)
STACK = replace(LAYER, name="stack", layers=49)
# the pages' own routing: top-6 of the 256 routed experts plus one shared expert
FLINT = replace(LAYER, name="flint", k=6, shared=1)
FLINT_BATCH = replace(FLINT, name="flint_batch", T=64, zipf_s=1.1)
TINY_SHARED = replace(TINY, shared=1)
# the same draws quantized to MXFP4 (the pages' released model is FP4)
TINY_FP4 = replace(TINY, name="tiny_fp4", fmt="mxfp4")
LAYER_FP4 = replace(LAYER, name="layer_fp4", fmt="mxfp4")
FLINT_FP4 = replace(FLINT, name="flint_fp4", fmt="mxfp4")
BATCH_FP4 = replace(BATCH, name="batch_fp4", fmt="mxfp4")
TINY_NV = replace(TINY, name="tiny_nv", fmt="nvfp4")
LAYER_NV = replace(LAYER, name="layer_nv", fmt="nvfp4")
FLINT_NV = replace(FLINT, name="flint_nv", fmt="nvfp4")
BATCH_NV = replace(BATCH, name="batch_nv", fmt="nvfp4")
LMHEAD1 = LMHeadConfig("lmhead", V=131072, d=2048, B=1)
LMHEAD8 = replace(LMHEAD1, B=8)


def zipf_bias(cfg: MoEConfig, seed: int) -> np.ndarray:
    """Router bias b_e = ln p_e, p_e = rank_e^-s / H, rank_e = 1 + perm(e)."""
    perm = permutation(cfg.E, key(seed, cfg.name, "bias"))
    ranks = 1.0 + perm.astype(np.float64)
    H = np.sum(np.arange(1, cfg.E + 1, dtype=np.float64) ** -cfg.zipf_s)
    return (np.log(ranks ** -cfg.zipf_s / H)).astype(np.float32)


def make_layer(cfg: MoEConfig, seed: int, layer: int = 0) -> dict:
    """All weights of one MoE layer, in the stored format (host numpy arrays)."""
    d, f, E = cfg.d, cfg.f, cfg.E
    # The batch and stack workloads reuse the `layer` streams: the batch runs
    # the same layer, and layer 0 of the stack is that layer.
    base = (seed, "tiny" if cfg.d == TINY.d and cfg.E == TINY.E else "layer", layer)
    rw = normal_f32(E * d, key(*base, "router"), 0.0, cfg.router_sigma).reshape(E, d)
    rb = zipf_bias(cfg, seed) if cfg.zipf_s > 0 else None
    out = dict(router_w=rw, router_b=rb)
    for name, rows, K in (("gate", f, d), ("up", f, d), ("down", d, f)):
        if cfg.fmt == "nvfp4":
            out[name + "_q"], out[name + "_s"], out[name + "_ts"] = nvfp4_experts(E, rows, K, key(*base, name),
                                                                                  cfg.expert_sigma)
        else:
            experts = mxfp4_experts if cfg.fmt == "mxfp4" else int4_experts
            out[name + "_q"], out[name + "_s"] = experts(E, rows, K, key(*base, name), cfg.expert_sigma)
    if cfg.shared:
        out.update(make_shared(cfg, seed, layer))
    return out


def make_shared(cfg: MoEConfig, seed: int, layer: int = 0) -> dict:
    """The shared expert of a layer (streams of its own, the routed experts'
    distribution): shared_{gate,up,down}_{q,s}."""
    d, f = cfg.d, cfg.f
    base = (seed, "tiny" if cfg.d == TINY.d and cfg.E == TINY.E else "layer", layer)
    out = {}
    for name, rows, K in (("gate", f, d), ("up", f, d), ("down", d, f)):
        if cfg.fmt == "nvfp4":
            q, sc, ts = nvfp4_experts(1, rows, K, key(*base, "shared_" + name), cfg.expert_sigma)
            out["shared_" + name + "_ts"] = ts
        else:
            experts = mxfp4_experts if cfg.fmt == "mxfp4" else int4_experts
            q, sc = experts(1, rows, K, key(*base, "shared_" + name), cfg.expert_sigma)
        out["shared_" + name + "_q"], out["shared_" + name + "_s"] = q[0], sc[0]
    return out


def draw_x(cfg: MoEConfig, seed: int, layer: int, token: int, attempt: int) -> np.ndarray:
    """bf16 activation row for (layer, token) at the given resampling attempt."""
    return bf16(cfg.d, key(seed, cfg.name, "x", layer, token, attempt))


def make_lmhead(cfg: LMHeadConfig, seed: int, copy: int = 0):
    return int4_matrix(cfg.V, cfg.d, key(seed, "lmhead", cfg.V, cfg.d, copy), cfg.sigma)


def draw_hidden(cfg: LMHeadConfig, seed: int, row: int, attempt: int) -> np.ndarray:
    return bf16(cfg.d, key(seed, "hidden", cfg.d, row, attempt))

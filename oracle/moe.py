"""Plain fp64 oracle of one sparse MoE layer decode step (and of a stack).

TEST INFRASTRUCTURE ONLY: part of the plain CPU oracle.  Nothing in the
product path may import this package.

What the pages fix ("Flint 40B: Best Mid Sized LLM", transcript 02:35): each
MoE layer holds 256 routed experts and a small router picks a few of them per
token; only the picked experts run ("O que diferencia um MoE de 40 bilhões com
2,5 bilhões ativos", noticiai.com.br page).  What they leave open is read as
follows (each reading is also listed in the design notes):

* router: logits l = W_r x + b in fp64 from fp32 weights and a bf16 x;
* softmax over all E experts, then the k largest probabilities (ties: lower
  expert index first), then the weights renormalized over the chosen set
  (norm_topk=True) or kept as the softmax values (norm_topk=False);
* expert: SwiGLU, h = silu(W_g x) * (W_u x) with silu(z) = z / (1 + e^-z),
  then o = W_d h, all on dequantized 4-bit weights in fp64 (int4 with fp16
  scales; MXFP4 -- E2M1 codes with E8M0 scales -- when the scale arrays
  hold bytes; NVFP4 -- E2M1 codes, E4M3 scales per 16, an fp32 scale per
  matrix -- when the layer carries tensor scales; formats.py);
* combine: y = sum over chosen experts of w_j o_j, added in ascending expert
  index, rounded once to fp32 for comparison;
* shared expert (the pages' layer adds one always-on expert to the routed
  ones, "Flint 40B: Best Mid Sized LLM", transcript 02:35): when a layer has
  one, its output o_s, same SwiGLU form and shape, is added with weight 1
  after the routed sum (it takes no part in the softmax or the
  renormalization).

Functions take host numpy arrays in the stored formats (see formats.py) and
never share code with the GPU path.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from itertools import combinations

import numpy as np

from .formats import bf16_to_f64, dequant, dequant_mxfp4, dequant_nvfp4, f64_to_bf16_bits, f64_to_f32


def dequant_4bit(q: np.ndarray, s: np.ndarray, K: int, t=None) -> np.ndarray:
    """A stored 4-bit matrix in any of the formats: a tensor scale t means
    NVFP4 (E4M3 per 16), else byte scales MXFP4 (E8M0 per 32), else int4
    (binary16 per 32)."""
    s = np.asarray(s)
    if t is not None:
        return dequant_nvfp4(q, s, t, K)
    return dequant_mxfp4(q, s, K) if s.dtype == np.uint8 else dequant(q, s, K)


@dataclass
class Layer:
    """One MoE layer in the stored formats, with a count of weights read."""

    router_w: np.ndarray            # fp32 [E][d]
    router_b: np.ndarray | None     # fp32 [E] or None
    gate_q: np.ndarray              # uint8 [E][f][d/2]
    gate_s: np.ndarray              # uint16 [E][f][d/32] (int4), or uint8 (MXFP4)
    up_q: np.ndarray
    up_s: np.ndarray
    down_q: np.ndarray              # uint8 [E][d][f/2]
    down_s: np.ndarray              # uint16 [E][d][f/32]
    shared: tuple | None = None     # (gate_q, gate_s, up_q, up_s, down_q, down_s) of the shared expert, or None
    weights_read: int = field(default=0)
    tscales: dict | None = None     # NVFP4: fp32 tensor scales gate_ts/up_ts/down_ts [E] (+ shared_*_ts scalars)

    @classmethod
    def from_dict(cls, t: dict) -> "Layer":
        sh = None
        if t.get("shared_gate_q") is not None:
            sh = tuple(t["shared_" + n] for n in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s"))
        ts = None
        if t.get("gate_ts") is not None:
            ts = {n: t[n] for n in ("gate_ts", "up_ts", "down_ts", "shared_gate_ts", "shared_up_ts",
                                    "shared_down_ts") if t.get(n) is not None}
        return cls(t["router_w"], t.get("router_b"), t["gate_q"], t["gate_s"], t["up_q"], t["up_s"],
                   t["down_q"], t["down_s"], sh, tscales=ts)

    def _t(self, name: str, e=None):
        """Tensor scale of a matrix (NVFP4), or None."""
        if self.tscales is None:
            return None
        v = np.asarray(self.tscales[name])
        return v if e is None else v[e]

    @property
    def E(self) -> int:
        return self.router_w.shape[0]

    @property
    def d(self) -> int:
        return self.router_w.shape[1]

    @property
    def f(self) -> int:
        return self.gate_q.shape[1]

    def expert(self, e: int):
        """Dequantized (W_g [f][d], W_u [f][d], W_d [d][f]) of expert e, counted as read."""
        d, f = self.d, self.f
        Wg = dequant_4bit(self.gate_q[e], self.gate_s[e], d, self._t("gate_ts", e))
        Wu = dequant_4bit(self.up_q[e], self.up_s[e], d, self._t("up_ts", e))
        Wd = dequant_4bit(self.down_q[e], self.down_s[e], f, self._t("down_ts", e))
        self.weights_read += Wg.size + Wu.size + Wd.size
        return Wg, Wu, Wd

    def shared_expert(self):
        """Dequantized (W_g, W_u, W_d) of the shared expert, counted as read."""
        gq, gs, uq, us, dq, ds = self.shared
        Wg = dequant_4bit(gq, gs, self.d, self._t("shared_gate_ts"))
        Wu = dequant_4bit(uq, us, self.d, self._t("shared_up_ts"))
        Wd = dequant_4bit(dq, ds, self.f, self._t("shared_down_ts"))
        self.weights_read += Wg.size + Wu.size + Wd.size
        return Wg, Wu, Wd


# ------------------------------------------------------------------ steps


def router_logits(layer: Layer, x: np.ndarray) -> np.ndarray:
    """l_e = sum_k W_r[e,k] x_k + b_e (fp64)."""
    layer.weights_read += layer.router_w.size
    l = layer.router_w.astype(np.float64) @ x
    if layer.router_b is not None:
        l = l + layer.router_b.astype(np.float64)
    return l


def softmax(l: np.ndarray) -> np.ndarray:
    z = np.exp(l - l.max())
    return z / z.sum()


def select_topk(p: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest p, largest first, lower index first on ties."""
    order = sorted(range(len(p)), key=lambda e: (-p[e], e))
    return np.array(order[:k], dtype=np.int64)


def route(l: np.ndarray, k: int, norm_topk: bool = True):
    """(chosen experts S, their weights w) from router logits.  The softmax
    is strictly increasing in the logit, so its k largest probabilities are
    those of the k largest logits (ties alike): S is selected on l, which
    stays exact where the fp64 probabilities of far smaller logits underflow
    to 0 and would tie."""
    p = softmax(l)
    S = select_topk(l, k)
    w = p[S] / p[S].sum() if norm_topk else p[S]
    return S, w


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def expert_forward(Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray, x: np.ndarray) -> np.ndarray:
    """SwiGLU expert: o = W_d (silu(W_g x) * (W_u x))."""
    g = Wg @ x
    u = Wu @ x
    return Wd @ (silu(g) * u)


def combine(S: np.ndarray, w: np.ndarray, outs: dict) -> np.ndarray:
    """y = sum_j w_j o_j over the chosen experts in ascending expert index."""
    y = np.zeros_like(next(iter(outs.values())))
    for j in np.argsort(S, kind="stable"):
        y = y + w[j] * outs[int(S[j])]
    return y


def add_shared(layer: Layer, y: np.ndarray, x: np.ndarray) -> np.ndarray:
    """y + o_s, the shared expert's output with weight 1 (y unchanged without one)."""
    if layer.shared is None:
        return y
    return y + expert_forward(*layer.shared_expert(), x)


def topk_margin(l: np.ndarray, k: int) -> float:
    """Gap between the k-th and (k+1)-th largest logit (inf when k == E)."""
    s = np.sort(l)[::-1]
    return float(s[k - 1] - s[k]) if k < len(s) else float("inf")


# ------------------------------------------------------------------ layer


def moe_forward(layer: Layer, x_bits: np.ndarray, k: int, norm_topk: bool = True) -> dict:
    """One token through one MoE layer: only the chosen experts are evaluated."""
    x = bf16_to_f64(x_bits)
    l = router_logits(layer, x)
    S, w = route(l, k, norm_topk)
    outs = {int(e): expert_forward(*layer.expert(int(e)), x) for e in S}
    y = add_shared(layer, combine(S, w, outs), x)
    return dict(y=y, y32=f64_to_f32(y), idx=S, w=w, logits=l)


def moe_forward_on_set(layer: Layer, x_bits: np.ndarray, S, norm_topk: bool = True) -> dict:
    """One token with the chosen set S given instead of selected: the weights
    are the softmax over all E experts restricted to S (renormalized over S
    when norm_topk), the rest as in moe_forward.  Used where another
    selection of equal-to-rounding logits is also correct."""
    x = bf16_to_f64(x_bits)
    l = router_logits(layer, x)
    p = softmax(l)
    S = np.asarray(S, dtype=np.int64)
    w = p[S] / p[S].sum() if norm_topk else p[S]
    outs = {int(e): expert_forward(*layer.expert(int(e)), x) for e in S}
    y = add_shared(layer, combine(S, w, outs), x)
    return dict(y=y, y32=f64_to_f32(y), idx=S, w=w, logits=l)


def moe_forward_tokens(layer: Layer, X_bits: np.ndarray, k: int, norm_topk: bool = True) -> dict:
    """T tokens, each routed on its own (row t of X is token t)."""
    rs = [moe_forward(layer, X_bits[t], k, norm_topk) for t in range(X_bits.shape[0])]
    return dict(y=np.stack([r["y"] for r in rs]), y32=np.stack([r["y32"] for r in rs]),
                idx=np.stack([r["idx"] for r in rs]), w=np.stack([r["w"] for r in rs]),
                logits=np.stack([r["logits"] for r in rs]))


def moe_forward_masked(layer: Layer, x_bits: np.ndarray, k: int, norm_topk: bool = True) -> np.ndarray:
    """Brute force: evaluate every expert, then keep the chosen ones by a
    0/1 mask, y = sum_{e=0}^{E-1} (m_e w_e) o_e in ascending e."""
    x = bf16_to_f64(x_bits)
    l = router_logits(layer, x)
    S, w = route(l, k, norm_topk)
    mw = np.zeros(layer.E)
    mw[S] = w
    y = np.zeros(layer.d)
    for e in range(layer.E):
        o = expert_forward(*layer.expert(e), x)
        y = y + mw[e] * o
    if layer.shared is not None:  # mask 1 for the always-on expert
        y = y + 1.0 * expert_forward(*layer.shared_expert(), x)
    return y


def moe_forward_dense_einsum(layer: Layer, x_bits: np.ndarray, k: int, norm_topk: bool = True) -> np.ndarray:
    """Independent formulation: dequantize all experts as one tensor and
    contract with einsum; chosen experts by a weight vector over all E."""
    x = bf16_to_f64(x_bits)
    l = layer.router_w.astype(np.float64) @ x + (0 if layer.router_b is None else layer.router_b.astype(np.float64))
    p = np.exp(l - l.max())
    p /= p.sum()
    # k-subset with the largest total logit, ties by the lexicographically smallest set
    chosen = np.lexsort((np.arange(layer.E), -l))[:k]
    wv = np.zeros(layer.E)
    wv[chosen] = p[chosen] / p[chosen].sum() if norm_topk else p[chosen]
    Wg = dequant_4bit(layer.gate_q, layer.gate_s, layer.d, layer._t("gate_ts"))
    Wu = dequant_4bit(layer.up_q, layer.up_s, layer.d, layer._t("up_ts"))
    Wd = dequant_4bit(layer.down_q, layer.down_s, layer.f, layer._t("down_ts"))
    G = np.einsum("efd,d->ef", Wg, x)
    U = np.einsum("efd,d->ef", Wu, x)
    H = G / (1.0 + np.exp(-G)) * U
    O = np.einsum("edf,ef->ed", Wd, H)
    y = np.einsum("e,ed->d", wv, O)
    if layer.shared is not None:
        gq, gs, uq, us, dq, ds = layer.shared
        Ws = [dequant_4bit(gq, gs, layer.d, layer._t("shared_gate_ts")), dequant_4bit(uq, us, layer.d, layer._t("shared_up_ts")),
              dequant_4bit(dq, ds, layer.f, layer._t("shared_down_ts"))]
        gs_, us_ = np.einsum("fd,d->f", Ws[0], x), np.einsum("fd,d->f", Ws[1], x)
        y = y + np.einsum("df,f->d", Ws[2], gs_ / (1.0 + np.exp(-gs_)) * us_)
    return y


def group_by_expert(idx: np.ndarray, E: int):
    """The T*k assignments a = t*k + j (token t's j-th chosen expert idx[t][j])
    grouped by expert: offsets [E+1] (expert e owns positions offsets[e] ..
    offsets[e+1]-1), the assignments in that order (ascending a within an
    expert), and the experts that own any (ascending)."""
    flat = np.asarray(idx).reshape(-1)
    lists = [[a for a in range(flat.size) if flat[a] == e] for e in range(E)]
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + len(lists[e])
    order = np.array([a for e in range(E) for a in lists[e]], dtype=np.int64)
    active = np.array([e for e in range(E) if lists[e]], dtype=np.int64)
    return offsets, order, active


def best_subset_bruteforce(l: np.ndarray, k: int):
    """All C(E, k) subsets: the one with the largest sum of logits."""
    best, best_sum = None, -np.inf
    for c in combinations(range(len(l)), k):
        s = float(np.sum(l[list(c)]))
        if s > best_sum:
            best, best_sum = c, s
    return np.array(best)


def active_weights(E: int, d: int, f: int, k: int, shared: int = 0) -> int:
    """Weights a sparse token reads: the router (E*d) and k routed plus the
    shared experts (3*d*f each)."""
    return E * d + (k + shared) * 3 * d * f


# ------------------------------------------------------------------ stack


def rmsnorm_bf16(r: np.ndarray, eps: float) -> np.ndarray:
    """x = bf16_RNE(r / sqrt(mean(r^2) + eps)), unit weight; returns bf16 bits."""
    r = np.asarray(r, dtype=np.float64)
    return f64_to_bf16_bits(r / np.sqrt(np.mean(r * r) + eps))


def stack_forward(layers, x0_bits: np.ndarray, k: int, eps: float = 1e-6, norm_topk: bool = True) -> dict:
    """Pre-norm residual stack: r_0 = x_0; for each layer x_l = RMSNorm(r_l)
    in bf16, y_l = layer(x_l), r_{l+1} = fp32(r_l + y_l) with y_l in fp32."""
    r = bf16_to_f64(x0_bits).astype(np.float32)
    xs, ys, idxs = [], [], []
    for layer in layers:
        x = rmsnorm_bf16(r, eps)
        out = moe_forward(layer, x, k, norm_topk)
        xs.append(x)
        ys.append(out["y32"])
        idxs.append(out["idx"])
        r = (r.astype(np.float64) + out["y32"].astype(np.float64)).astype(np.float32)
    return dict(r=r, xs=xs, ys=ys, idx=idxs)

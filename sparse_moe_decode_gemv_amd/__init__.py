"""Python binding of the sparse MoE decode library (libmoe_decode.so, gfx950).

Argument marshalling only: every step of the decode path runs in the HIP
kernels behind the C ABI declared in include/moe_decode.h.  PyTorch provides
device memory (tensors) and the current HIP stream; no torch compute op is
used on the decode path.  The functions below carry the C names.

If the library has not been built this module still imports (so that host
code and error paths can be tested without a GPU), but every call raises
RuntimeError; nothing falls back to a CPU implementation.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_decode.so")

MOE_OK = 0
MOE_ERR_NULL = -1
MOE_ERR_SHAPE = -2
MOE_ERR_ALIGN = -3
MOE_ERR_WORKSPACE = -4
MOE_ERR_HIP = -5
MOE_ERR_UNSUPPORTED = -6
MOE_MAX_TOPK = 16
MOE_MAX_TOKENS = 4096
MOE_LMHEAD_MAX_B = 16
WEIGHTS_INT4 = 0    # int4 codes, binary16 scales per 32
WEIGHTS_MXFP4 = 1   # FP4 E2M1 codes, E8M0 scale bytes per 32
WEIGHTS_NVFP4 = 2   # FP4 E2M1 codes, E4M3 scale bytes per 16, fp32 scale per matrix

EXPORTED = (
    "moe_decode_workspace_bytes", "moe_decode_init", "moe_decode_forward", "moe_decode_stack_forward",
    "moe_decode_destroy", "moe_decode_expert_groups", "lmhead_int4_argmax_workspace_bytes", "lmhead_int4_argmax", "moe_status_str",
    "moe_decode_abi_version", "moe_decode_error_flags", "moe_decode_set_wait_limit", "lmhead_int4_argmax_noalloc",
    "moe_decode_stack_forward_ex", "moe_decode_read_probe", "moe_int4_repack", "moe_decode_phase_trace",
    "moe_decode_init_on_stream",
)
MOE_STACK_PERSISTENT = 1
DEFAULT_WAIT_POLLS = 1 << 21


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_str(status)} (status {status})")
        self.status = status


class LayerDesc(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("f", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("norm_topk", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("weight_format", ctypes.c_int32)]


WEIGHT_NAMES = ("router_w", "router_b", "gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s",
                "shared_gate_q", "shared_gate_s", "shared_up_q", "shared_up_s", "shared_down_q", "shared_down_s",
                "gate_tscale", "up_tscale", "down_tscale",
                "shared_gate_tscale", "shared_up_tscale", "shared_down_tscale")


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_NAMES]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built ({LIB_PATH}); run `python -m sparse_moe_decode_gemv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        p, sz, i32, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_float
        L.moe_decode_workspace_bytes.restype = sz
        L.moe_decode_workspace_bytes.argtypes = [ctypes.POINTER(LayerDesc)]
        L.moe_decode_init.restype = i32
        L.moe_decode_init.argtypes = [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights), p, sz,
                                      ctypes.POINTER(p)]
        L.moe_decode_init_on_stream.restype = i32
        L.moe_decode_init_on_stream.argtypes = [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights), p, sz, p,
                                                ctypes.POINTER(p)]
        L.moe_decode_forward.restype = i32
        L.moe_decode_forward.argtypes = [p, p, i32, p, p, p, p]
        L.moe_decode_stack_forward.restype = i32
        L.moe_decode_stack_forward.argtypes = [ctypes.POINTER(p), i32, p, i32, f32, p, p, p, p]
        L.moe_decode_stack_forward_ex.restype = i32
        L.moe_decode_stack_forward_ex.argtypes = [ctypes.POINTER(p), i32, p, i32, f32, p, p, p, i32, p]
        L.moe_int4_repack.restype = i32
        L.moe_int4_repack.argtypes = [p, p, ctypes.c_int64, i32, p]
        L.moe_decode_read_probe.restype = i32
        L.moe_decode_read_probe.argtypes = [p, sz, p, p]
        L.moe_decode_phase_trace.restype = i32
        L.moe_decode_phase_trace.argtypes = [p, ctypes.c_int64]
        L.moe_decode_expert_groups.restype = i32
        L.moe_decode_expert_groups.argtypes = [p, i32, p, p, p, p, p]
        L.moe_decode_destroy.restype = None
        L.moe_decode_destroy.argtypes = [p]
        L.lmhead_int4_argmax_workspace_bytes.restype = sz
        L.lmhead_int4_argmax_workspace_bytes.argtypes = [i32, i32, i32]
        L.lmhead_int4_argmax.restype = i32
        L.lmhead_int4_argmax.argtypes = [p, p, i32, i32, p, i32, p, p, p, sz, p]
        L.lmhead_int4_argmax_noalloc.restype = i32
        L.lmhead_int4_argmax_noalloc.argtypes = [p, p, i32, i32, p, i32, p, p, p]
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_status_str.argtypes = [i32]
        L.moe_decode_abi_version.restype = i32
        L.moe_decode_abi_version.argtypes = []
        L.moe_decode_error_flags.restype = i32
        L.moe_decode_error_flags.argtypes = [p, p, i32, p]
        L.moe_decode_set_wait_limit.restype = i32
        L.moe_decode_set_wait_limit.argtypes = [p, ctypes.c_uint32, i32]
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().moe_status_str(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoEError(status, where)


def _ptr(t) -> int | None:
    """Device address of a tensor (None passes NULL); requires contiguity."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


# ------------------------------------------------------------ C-named calls


def moe_decode_workspace_bytes(desc: LayerDesc) -> int:
    return lib().moe_decode_workspace_bytes(ctypes.byref(desc))


def moe_decode_init(desc: LayerDesc, weights: LayerWeights, workspace, workspace_bytes: int | None = None) -> int:
    """Returns the opaque handle (an integer address)."""
    h = ctypes.c_void_p()
    nbytes = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    _check(lib().moe_decode_init(ctypes.byref(desc), ctypes.byref(weights), _ptr(workspace), nbytes,
                                 ctypes.byref(h)), "moe_decode_init")
    return h.value


def moe_decode_init_on_stream(desc: LayerDesc, weights: LayerWeights, workspace, workspace_bytes: int | None = None,
                              stream=None) -> int:
    """moe_decode_init with its device work on `stream` (default: the current
    torch stream), synchronizing that stream only.  Returns the handle."""
    h = ctypes.c_void_p()
    nbytes = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    _check(lib().moe_decode_init_on_stream(ctypes.byref(desc), ctypes.byref(weights), _ptr(workspace), nbytes,
                                           _stream(stream), ctypes.byref(h)), "moe_decode_init_on_stream")
    return h.value


def moe_decode_forward(handle: int, x, T: int, y, topk_idx=None, topk_w=None, stream=None) -> None:
    _check(lib().moe_decode_forward(handle, _ptr(x), T, _ptr(y), _ptr(topk_idx), _ptr(topk_w), _stream(stream)),
           "moe_decode_forward")


def moe_decode_stack_forward(handles, residual, T: int, eps: float, x_trace=None, y_trace=None, idx_trace=None,
                             stream=None) -> None:
    arr = (ctypes.c_void_p * len(handles))(*handles)
    _check(lib().moe_decode_stack_forward(arr, len(handles), _ptr(residual), T, eps, _ptr(x_trace), _ptr(y_trace),
                                          _ptr(idx_trace), _stream(stream)), "moe_decode_stack_forward")


def moe_decode_stack_forward_ex(handles, residual, T: int, eps: float, x_trace=None, y_trace=None, idx_trace=None,
                                flags: int = 0, stream=None) -> None:
    arr = (ctypes.c_void_p * len(handles))(*handles)
    _check(lib().moe_decode_stack_forward_ex(arr, len(handles), _ptr(residual), T, eps, _ptr(x_trace), _ptr(y_trace),
                                             _ptr(idx_trace), int(flags), _stream(stream)),
           "moe_decode_stack_forward_ex")


def moe_int4_repack(src, dst, rows: int, K: int, stream=None) -> None:
    _check(lib().moe_int4_repack(_ptr(src), _ptr(dst), int(rows), int(K), _stream(stream)), "moe_int4_repack")


def moe_decode_read_probe(buf, nbytes: int, sink, stream=None) -> None:
    _check(lib().moe_decode_read_probe(_ptr(buf), int(nbytes), _ptr(sink), _stream(stream)), "moe_decode_read_probe")


def moe_decode_phase_trace(host_out) -> None:
    """host_out: a C-contiguous numpy uint64 array (filled in place)."""
    _check(lib().moe_decode_phase_trace(host_out.ctypes.data, int(host_out.size)), "moe_decode_phase_trace")


def moe_decode_expert_groups(handle: int, T: int, offsets=None, assignments=None, active=None, n_active=None,
                             stream=None) -> None:
    _check(lib().moe_decode_expert_groups(handle, T, _ptr(offsets), _ptr(assignments), _ptr(active),
                                          _ptr(n_active), _stream(stream)), "moe_decode_expert_groups")


def moe_decode_error_flags(handle: int, flags=None, clear: int = 1, stream=None) -> None:
    _check(lib().moe_decode_error_flags(handle, _ptr(flags), int(clear), _stream(stream)), "moe_decode_error_flags")


def moe_decode_set_wait_limit(handle: int, polls: int, unreachable: int = 0) -> None:
    _check(lib().moe_decode_set_wait_limit(handle, int(polls), int(unreachable)), "moe_decode_set_wait_limit")


def moe_decode_destroy(handle: int) -> None:
    lib().moe_decode_destroy(handle)


def lmhead_int4_argmax_workspace_bytes(V: int, d: int, B: int) -> int:
    return lib().lmhead_int4_argmax_workspace_bytes(V, d, B)


def lmhead_int4_argmax(w_q, w_s, V: int, d: int, x, B: int, token, max_logit, workspace,
                       workspace_bytes: int | None = None, stream=None) -> None:
    nbytes = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    _check(lib().lmhead_int4_argmax(_ptr(w_q), _ptr(w_s), V, d, _ptr(x), B, _ptr(token), _ptr(max_logit),
                                    _ptr(workspace), nbytes, _stream(stream)), "lmhead_int4_argmax")


def lmhead_int4_argmax_noalloc(w_q, w_s, V: int, d: int, x, B: int, token, max_logit, stream=None) -> None:
    _check(lib().lmhead_int4_argmax_noalloc(_ptr(w_q), _ptr(w_s), V, d, _ptr(x), B, _ptr(token), _ptr(max_logit),
                                            _stream(stream)), "lmhead_int4_argmax_noalloc")


# ------------------------------------------------------------ conveniences


@dataclass
class MoELayer:
    """One layer bound to device tensors (kept alive here) and its handle."""

    d: int
    f: int
    E: int
    k: int
    norm_topk: int
    max_tokens: int
    tensors: dict
    workspace: object
    handle: int

    @classmethod
    def create(cls, tensors: dict, d: int, f: int, E: int, k: int, norm_topk: int = 1, max_tokens: int = 1,
               init_stream=None):
        """tensors: device tensors router_w, router_b (or None), gate_q, gate_s, up_q, up_s, down_q, down_s,
        and shared_gate_q ... shared_down_s when the layer has a shared expert.  init_stream: a torch
        stream to initialize on (moe_decode_init_on_stream); None uses moe_decode_init."""
        import torch
        n_shared = 1 if tensors.get("shared_gate_q") is not None else 0
        # matrix scales: NVFP4; byte scales: MXFP4 (E8M0); 16-bit scales: int4 (binary16)
        if tensors.get("gate_ts") is not None:
            fmt = WEIGHTS_NVFP4
            tensors = dict(tensors, gate_tscale=tensors["gate_ts"], up_tscale=tensors["up_ts"],
                           down_tscale=tensors["down_ts"], shared_gate_tscale=tensors.get("shared_gate_ts"),
                           shared_up_tscale=tensors.get("shared_up_ts"),
                           shared_down_tscale=tensors.get("shared_down_ts"))
        else:
            fmt = WEIGHTS_MXFP4 if tensors["gate_s"].dtype == torch.uint8 else WEIGHTS_INT4
        desc = LayerDesc(d, f, E, k, norm_topk, max_tokens, n_shared, fmt)
        nbytes = moe_decode_workspace_bytes(desc)
        if nbytes == 0:
            raise MoEError(MOE_ERR_SHAPE, "moe_decode_workspace_bytes")
        ws = torch.empty(nbytes, dtype=torch.uint8, device=tensors["router_w"].device)
        w = LayerWeights(*[_ptr(tensors.get(n)) for n in WEIGHT_NAMES])
        if init_stream is None:
            h = moe_decode_init(desc, w, ws)
        else:
            init_stream.wait_stream(torch.cuda.current_stream())  # the workspace tensor was made on the current stream
            h = moe_decode_init_on_stream(desc, w, ws, stream=init_stream)
        return cls(d, f, E, k, norm_topk, max_tokens, tensors, ws, h)

    def forward(self, x, y=None, topk_idx=None, topk_w=None, stream=None):
        import torch
        T = x.shape[0] if x.dim() == 2 else 1
        dev = x.device
        if y is None:
            y = torch.empty((T, self.d), dtype=torch.float32, device=dev)
        moe_decode_forward(self.handle, x, T, y, topk_idx, topk_w, stream)
        return y

    def error_flags(self, clear: bool = True, stream=None) -> int:
        """The single-launch kernel's error flags (0 when every wait
        completed); synchronizes the stream."""
        import torch
        out = torch.full((1,), -1, dtype=torch.int32, device=self.workspace.device)
        moe_decode_error_flags(self.handle, out, 1 if clear else 0, stream)
        torch.cuda.current_stream().synchronize() if stream is None else torch.cuda.synchronize()
        return int(out.item())

    def close(self) -> None:
        if self.handle:
            moe_decode_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def lmhead_argmax(w_q, w_s, x, token=None, max_logit=None, workspace=None, stream=None):
    """Convenience wrapper: x [B][d] bf16 bits on the device -> (token, max_logit)."""
    import torch
    B, d = x.shape
    V = w_q.shape[0]
    dev = x.device
    if token is None:
        token = torch.empty(B, dtype=torch.int32, device=dev)
    if max_logit is None:
        max_logit = torch.empty(B, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.zeros(lmhead_int4_argmax_workspace_bytes(V, d, B), dtype=torch.uint8, device=dev)
    lmhead_int4_argmax(w_q, w_s, V, d, x, B, token, max_logit, workspace, stream=stream)
    return token, max_logit


def upload(arrays: dict, device="cuda") -> dict:
    """Host numpy arrays in the stored formats -> device tensors (bit copies:
    uint16 bit patterns travel as int16)."""
    import numpy as np
    import torch
    out = {}
    for k, v in arrays.items():
        if v is None:
            out[k] = None
            continue
        a = np.ascontiguousarray(v)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        out[k] = torch.from_numpy(a).to(device)
    return out

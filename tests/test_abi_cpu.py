"""The C ABI on the host: the library loads, exports every function that
include/moe_decode.h declares, sizes workspaces, and rejects bad arguments
with the documented status before anything reaches the GPU.  Only fake,
never-dereferenced device addresses are used here."""
import ctypes
import os
import re

import pytest

import sparse_moe_decode_gemv_amd as M

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe_decode.h")
FAKE = 0x10000  # aligned, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    names = re.findall(r"^[A-Za-z_][\w \t\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_header_declares_the_three_entry_points():
    names = declared_functions()
    for n in ("moe_decode_init", "moe_decode_forward", "lmhead_int4_argmax"):
        assert n in names
    assert sorted(names) == sorted(M.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = M.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    assert L.moe_decode_abi_version() == 5


def test_status_strings():
    assert M.status_str(0) == "ok"
    for s in range(-6, 0):
        assert M.status_str(s) != "unknown status"
    assert M.status_str(-99) == "unknown status"


def desc(**kw):
    base = dict(d=2048, f=512, n_experts=256, top_k=8, norm_topk=1, max_tokens=1)
    base.update(kw)
    return M.LayerDesc(**base)


def test_workspace_bytes_layout():
    n1 = M.moe_decode_workspace_bytes(desc())
    n64 = M.moe_decode_workspace_bytes(desc(max_tokens=64))
    assert n1 > 0 and n64 > n1
    # the per-assignment expert outputs alone are T*k*d floats
    assert n64 >= 64 * 8 * 2048 * 4
    assert n1 % 256 == 0


@pytest.mark.parametrize("kw", [dict(top_k=0), dict(top_k=17), dict(top_k=300, n_experts=256), dict(max_tokens=0),
                                dict(max_tokens=4097), dict(d=2040), dict(f=500), dict(norm_topk=2),
                                dict(n_experts=2000), dict(d=0), dict(n_shared=2), dict(n_shared=-1),
                                dict(weight_format=3), dict(weight_format=-1)])
def test_bad_shapes_have_no_workspace(kw):
    assert M.moe_decode_workspace_bytes(desc(**kw)) == 0


def init_status(d, w, ws_ptr=FAKE, ws_bytes=1 << 30):
    h = ctypes.c_void_p()
    return M.lib().moe_decode_init(ctypes.byref(d), ctypes.byref(w), ws_ptr, ws_bytes, ctypes.byref(h)), h


def weights(**kw):
    base = {n: FAKE for n in ("router_w", "gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")}
    base["router_b"] = None
    base.update(kw)
    return M.LayerWeights(**base)


def test_init_validation_codes():
    assert init_status(desc(), weights(gate_q=None))[0] == M.MOE_ERR_NULL
    assert init_status(desc(), weights(up_s=FAKE + 2))[0] == M.MOE_ERR_ALIGN
    assert init_status(desc(), weights(router_b=FAKE + 1))[0] == M.MOE_ERR_ALIGN
    assert init_status(desc(top_k=0), weights())[0] == M.MOE_ERR_SHAPE
    assert init_status(desc(d=1536), weights())[0] == M.MOE_ERR_UNSUPPORTED
    assert init_status(desc(f=96), weights())[0] == M.MOE_ERR_UNSUPPORTED
    need = M.moe_decode_workspace_bytes(desc())
    st, h = init_status(desc(), weights(), FAKE, need - 1)
    assert st == M.MOE_ERR_WORKSPACE and h.value is None
    assert init_status(desc(), weights(), None, need)[0] == M.MOE_ERR_WORKSPACE
    assert init_status(desc(), weights(), FAKE + 16, need)[0] == M.MOE_ERR_ALIGN
    assert M.lib().moe_decode_init(None, ctypes.byref(weights()), FAKE, need, None) == M.MOE_ERR_NULL


def test_init_on_stream_validation_codes():
    """The stream form validates like moe_decode_init, before any GPU work."""
    L = M.lib()

    def st(d, w, ws_ptr=FAKE, ws_bytes=1 << 30):
        h = ctypes.c_void_p()
        return L.moe_decode_init_on_stream(ctypes.byref(d), ctypes.byref(w), ws_ptr, ws_bytes, None, ctypes.byref(h)), h

    assert st(desc(), weights(gate_q=None))[0] == M.MOE_ERR_NULL
    assert st(desc(), weights(up_s=FAKE + 2))[0] == M.MOE_ERR_ALIGN
    assert st(desc(top_k=0), weights())[0] == M.MOE_ERR_SHAPE
    assert st(desc(d=1536), weights())[0] == M.MOE_ERR_UNSUPPORTED
    need = M.moe_decode_workspace_bytes(desc())
    s, h = st(desc(), weights(), FAKE, need - 1)
    assert s == M.MOE_ERR_WORKSPACE and h.value is None
    assert st(desc(), weights(), FAKE + 16, need)[0] == M.MOE_ERR_ALIGN
    assert L.moe_decode_init_on_stream(ctypes.byref(desc()), ctypes.byref(weights()), FAKE, need, None,
                                       None) == M.MOE_ERR_NULL


def test_shared_expert_validation_and_workspace():
    """n_shared = 1 needs all six shared matrices, 16-byte aligned; the
    batched workspace grows by the shared expert's assignments and copy."""
    sh = {n: FAKE for n in ("shared_gate_q", "shared_gate_s", "shared_up_q", "shared_up_s", "shared_down_q",
                            "shared_down_s")}
    need = M.moe_decode_workspace_bytes(desc(n_shared=1, top_k=6))
    assert need > 0
    assert init_status(desc(n_shared=1, top_k=6), weights())[0] == M.MOE_ERR_NULL
    assert init_status(desc(n_shared=1, top_k=6), weights(**dict(sh, shared_down_s=None)))[0] == M.MOE_ERR_NULL
    assert init_status(desc(n_shared=1, top_k=6), weights(**dict(sh, shared_up_q=FAKE + 8)))[0] == M.MOE_ERR_ALIGN
    n64 = M.moe_decode_workspace_bytes(desc(max_tokens=64, top_k=6))
    s64 = M.moe_decode_workspace_bytes(desc(max_tokens=64, top_k=6, n_shared=1))
    # 64 more assignments (fp32 outputs and fp16 h) and one more expert in the tile-major copies
    assert s64 - n64 >= 64 * 2048 * 4 + 64 * 512 * 2 + 3 * 2048 * 512 // 2


def test_forward_and_stack_reject_null_handles():
    L = M.lib()
    assert L.moe_decode_forward(None, FAKE, 1, FAKE, None, None, None) == M.MOE_ERR_NULL
    arr = (ctypes.c_void_p * 2)(None, None)
    assert L.moe_decode_stack_forward(arr, 2, FAKE, 1, 1e-6, None, None, None, None) == M.MOE_ERR_NULL
    assert L.moe_decode_stack_forward(arr, 0, FAKE, 1, 1e-6, None, None, None, None) == M.MOE_ERR_SHAPE
    assert L.moe_decode_stack_forward(None, 1, FAKE, 1, 1e-6, None, None, None, None) == M.MOE_ERR_NULL
    assert L.moe_decode_expert_groups(None, 1, FAKE, FAKE, FAKE, FAKE, None) == M.MOE_ERR_NULL
    assert L.moe_decode_error_flags(None, FAKE, 1, None) == M.MOE_ERR_NULL
    assert L.moe_int4_repack(None, FAKE, 1, 128, None) == M.MOE_ERR_NULL
    assert L.moe_int4_repack(FAKE, FAKE + (1 << 20), 1, 96, None) == M.MOE_ERR_SHAPE
    assert L.moe_int4_repack(FAKE, FAKE + (1 << 20), 0, 128, None) == M.MOE_ERR_SHAPE
    assert L.moe_int4_repack(FAKE, FAKE + 32, 1, 128, None) == M.MOE_ERR_SHAPE  # overlapping
    assert L.moe_int4_repack(FAKE + 8, FAKE + (1 << 20), 1, 128, None) == M.MOE_ERR_ALIGN
    assert L.moe_decode_read_probe(FAKE, 100, FAKE, None) == M.MOE_ERR_SHAPE
    assert L.moe_decode_read_probe(None, 128, FAKE, None) == M.MOE_ERR_NULL
    assert L.moe_decode_set_wait_limit(None, 1, 0) == M.MOE_ERR_NULL
    M.moe_decode_destroy(None)  # ignored


def test_phase_trace_only_in_the_diagnostic_build():
    """The product library records no phase timestamps: the call says so
    (and checks its arguments first); no GPU work is involved."""
    L = M.lib()
    out = (ctypes.c_uint64 * 16)()
    assert L.moe_decode_phase_trace(None, 16) == M.MOE_ERR_NULL
    assert L.moe_decode_phase_trace(out, 0) == M.MOE_ERR_SHAPE
    assert L.moe_decode_phase_trace(out, 16) == M.MOE_ERR_UNSUPPORTED


def test_lmhead_validation_codes():
    L = M.lib()
    ws = M.lmhead_int4_argmax_workspace_bytes(131072, 2048, 8)
    assert ws > 0
    assert M.lmhead_int4_argmax_workspace_bytes(131072, 2048, 17) == 0
    assert M.lmhead_int4_argmax_workspace_bytes(0, 2048, 1) == 0
    assert M.lmhead_int4_argmax_workspace_bytes(16, 2000, 1) == 0
    call = lambda **kw: L.lmhead_int4_argmax(*[kw.get(n, v) for n, v in [
        ("wq", FAKE), ("ws", FAKE), ("V", 131072), ("d", 2048), ("x", FAKE), ("B", 8), ("tok", FAKE),
        ("ml", FAKE), ("work", FAKE), ("wb", ws), ("s", None)]])
    assert call(wq=None) == M.MOE_ERR_NULL
    assert call(tok=None) == M.MOE_ERR_NULL
    assert call(B=0) == M.MOE_ERR_SHAPE
    assert call(B=17) == M.MOE_ERR_SHAPE
    assert call(V=0) == M.MOE_ERR_SHAPE
    assert call(d=2000) == M.MOE_ERR_SHAPE
    assert call(d=1536) == M.MOE_ERR_UNSUPPORTED
    assert call(x=FAKE + 8) == M.MOE_ERR_ALIGN
    assert call(ml=FAKE + 2) == M.MOE_ERR_ALIGN
    assert call(wb=ws - 1) == M.MOE_ERR_WORKSPACE
    assert call(work=None) == M.MOE_ERR_WORKSPACE


def test_python_errors_are_raised():
    with pytest.raises(M.MoEError) as ei:
        M.lmhead_int4_argmax(None, FAKE, 16, 256, FAKE, 1, FAKE, None, FAKE, 1 << 20, stream=0)
    assert ei.value.status == M.MOE_ERR_NULL


def test_mxfp4_layer_workspace():
    """MXFP4 layers are accepted at any max_tokens; a 1-token layer on the
    single-launch shapes carries no tile-major copy (same workspace as int4),
    a batched one the same copy size as int4 (byte scales fit the binary16
    scales' room)."""
    fp4 = dict(weight_format=M.WEIGHTS_MXFP4)
    assert M.moe_decode_workspace_bytes(desc(**fp4)) == M.moe_decode_workspace_bytes(desc())
    assert M.moe_decode_workspace_bytes(desc(max_tokens=64, **fp4)) == M.moe_decode_workspace_bytes(desc(max_tokens=64))


def test_nvfp4_needs_matrix_scales():
    """NVFP4 layers need the fp32 matrix scales (NULL -> MOE_ERR_NULL,
    misaligned -> MOE_ERR_ALIGN, checked before any device work)."""
    nv = desc(weight_format=M.WEIGHTS_NVFP4)
    assert init_status(nv, weights())[0] == M.MOE_ERR_NULL
    ts = dict(gate_tscale=FAKE, up_tscale=FAKE, down_tscale=FAKE)
    assert init_status(nv, weights(**dict(ts, up_tscale=FAKE + 2)))[0] == M.MOE_ERR_ALIGN

"""The LM head's allocation-free entry point (lmhead_int4_argmax_noalloc),
called through the C ABI, against the workspace entry point on the same
inputs: two calls in a row, the second with a smaller input, each bit for
bit equal to the workspace call (same kernels, same reduction order)."""
import ctypes

import numpy as np
import pytest

import synth
import sparse_moe_decode_gemv_amd as M
from gpu_common import device
from oracle import lmhead as OH
from oracle.inputs import pick_hidden

pytestmark = pytest.mark.gpu


def _case(V, d, B, seed, margin):
    """Head and rows; with margin, rows resampled until the oracle's top-1 -
    top-2 logit gap is at least 1e-2 (so the argmax is unique)."""
    q, s = synth.int4_matrix(V, d, synth.key(seed, "noalloc-lm", V, d), 0.02)
    draw = lambda b, a: synth.bf16(d, synth.key(seed, "noalloc-x", b, a))
    if margin:
        xs = np.stack([pick_hidden(q, s, 1e-2, lambda a, b=b: draw(b, a))[0] for b in range(B)])
    else:
        xs = np.stack([draw(b, 0) for b in range(B)])
    return q, s, xs


def _run_both(q, s, xs):
    import torch
    dev = device()
    V, d, B = q.shape[0], q.shape[1] * 2, xs.shape[0]
    wq = torch.from_numpy(q).to(dev)
    ws = torch.from_numpy(s.view(np.int16)).to(dev)
    x = torch.from_numpy(xs.view(np.int16)).to(dev)
    tok_w = torch.full((B,), -1, dtype=torch.int32, device=dev)
    ml_w = torch.full((B,), float("nan"), dtype=torch.float32, device=dev)
    work = torch.zeros(M.lmhead_int4_argmax_workspace_bytes(V, d, B), dtype=torch.uint8, device=dev)
    M.lmhead_int4_argmax(wq, ws, V, d, x, B, tok_w, ml_w, work)
    tok_n = torch.full((B,), -1, dtype=torch.int32, device=dev)
    ml_n = torch.full((B,), float("nan"), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    st = M.lib().lmhead_int4_argmax_noalloc(wq.data_ptr(), ws.data_ptr(), V, d, x.data_ptr(), B, tok_n.data_ptr(),
                                           ml_n.data_ptr(), stream)
    assert st == M.MOE_OK, M.status_str(st)
    torch.cuda.synchronize()
    return tok_w.cpu().numpy(), ml_w.cpu().numpy(), tok_n.cpu().numpy(), ml_n.cpu().numpy()


def test_noalloc_lmhead_matches_the_workspace_call_twice():
    """The full-size head (V = 131072, d = 2048) at B = 8, then smaller
    inputs: V = 4096, d = 512, B = 3 and V = 8192, d = 2048, B = 1 (these two
    also against the fp64 oracle)."""
    for V, d, B, seed, oracle in ((131072, 2048, 8, 1, False), (4096, 512, 3, 2, True), (8192, 2048, 1, 3, True)):
        q, s, xs = _case(V, d, B, seed, oracle)
        tw, mw, tn, mn = _run_both(q, s, xs)
        assert np.array_equal(tw, tn), f"V={V} B={B}: tokens {tn} vs {tw}"
        assert np.array_equal(mw.view(np.uint32), mn.view(np.uint32)), f"V={V} B={B}: max logits differ"
        if oracle:
            otok, oml, _ = OH.lmhead_argmax(q, s, xs)
            assert np.array_equal(tn, otok), f"V={V} B={B}: tokens {tn} vs oracle {otok}"


def test_noalloc_lmhead_rejects_bad_arguments():
    L = M.lib()
    FAKE = 0x10000
    assert L.lmhead_int4_argmax_noalloc(FAKE, FAKE, 16, 256, FAKE, 17, FAKE, None, None) == M.MOE_ERR_SHAPE
    assert L.lmhead_int4_argmax_noalloc(None, FAKE, 16, 256, FAKE, 1, FAKE, None, None) == M.MOE_ERR_NULL
    assert L.lmhead_int4_argmax_noalloc(FAKE, FAKE, 16, 1536, FAKE, 1, FAKE, None, None) == M.MOE_ERR_UNSUPPORTED

"""Value ranges at the edges, on the GPU against the fp64 oracle.

* Activations of any magnitude: tokens scaled by 2^s (s = +-20, +-40) through
  the single-launch step and the batched kernels.  Both hand binary16
  operands on as x 2^a and h 2^(2a), with 2^a putting the token's largest
  |x| in [1, 2), and scale the output back, so the result is exact however
  large or small x is.  The chosen experts are those of the unscaled token
  (the logits scale by 2^s, margin included).
* MXFP4 scale bytes: 104 and 140 (the batched kernels' exact range) pass
  on the batched path; 103 and 141 are rejected at init for a layer that
  may run it, and accepted and exact on the single-launch step; 255 (NaN)
  is rejected for every layer.
* NVFP4 E4M3 scales: every finite byte (0x00..0x7E and the negative
  0x80..0xFE), at every position of a piece, through the down and the gate
  projection of the single-launch step, each row checked against the
  oracle to 2e-3 of the row's own sum of magnitudes.
* moe_int4_repack: canonical nibble order to the stored order, bit for
  bit against the oracle's packer."""
import numpy as np
import pytest

import synth
import sparse_moe_decode_gemv_amd as M
from gpu_common import Y_TOL, as_i16, compare_layer, device, tokens
from oracle import formats as F
from oracle import moe as OM
from oracle.inputs import pick_token

pytestmark = pytest.mark.gpu


def _scale_bits(X, s):
    """bf16 bit patterns times 2^s (exponent field shifted; zeros stay)."""
    X = X.astype(np.int32)
    mag = X & 0x7FFF
    out = np.where(mag == 0, X, (X & 0x8000) | (mag + (s << 7)))
    assert np.all((mag == 0) | (((mag >> 7) + s > 0) & ((mag >> 7) + s < 255)))
    return out.astype(np.uint16)


@pytest.mark.parametrize("s", [-40, -20, 20, 40])
@pytest.mark.parametrize("cfg", [synth.LAYER, synth.TINY], ids=["flagship", "tiny"])
def test_activation_magnitudes_both_paths(cfg, s):
    import torch
    dev = device()
    lay = synth.make_layer(cfg, 7)
    OL = OM.Layer.from_dict(lay)
    T = 4
    X = _scale_bits(tokens(cfg, OL, 7, T), s)
    with np.errstate(over="ignore", invalid="ignore"):
        out = OM.moe_forward_tokens(OL, X, cfg.k)
    up = M.upload(lay, dev)
    xd = torch.from_numpy(as_i16(X)).to(dev)
    for mt in (1, T):  # single-launch steps, then one batched call
        L = M.MoELayer.create(up, cfg.d, cfg.f, cfg.E, cfg.k, 1, mt)
        y = torch.full((T, cfg.d), float("nan"), device=dev)
        idx = torch.full((T, cfg.k), -1, dtype=torch.int32, device=dev)
        w = torch.full((T, cfg.k), float("nan"), device=dev)
        if mt == 1:
            for t in range(T):
                L.forward(xd[t:t + 1], y[t:t + 1], idx[t:t + 1], w[t:t + 1])
        else:
            L.forward(xd, y, idx, w)
        torch.cuda.synchronize()
        assert np.all(np.isfinite(y.cpu().numpy())), f"2^{s}, max_tokens {mt}: non-finite output"
        compare_layer(out, idx.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy(), f"2^{s} max_tokens {mt}")
        L.close()


def _mx_layer_with(byte):
    """The tiny MXFP4 layer with scale byte `byte` on the first block of every
    third row of every expert's W_d (in W_d a large scale only scales output
    rows; in W_g or W_u it would push h past the binary16 range)."""
    lay = dict(synth.make_layer(synth.TINY_FP4, 8))
    a = lay["down_s"].copy()
    a[:, ::3, 0] = byte
    lay["down_s"] = a
    return lay


@pytest.mark.parametrize("byte", [104, 140])
def test_mxfp4_scale_bytes_at_the_batched_limits(byte):
    import torch
    dev = device()
    cfg = synth.TINY_FP4
    lay = _mx_layer_with(byte)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 8, 8)
    L = M.MoELayer.create(M.upload(lay, dev), cfg.d, cfg.f, cfg.E, cfg.k, 1, 8)
    y = torch.empty((8, cfg.d), device=dev)
    idx = torch.empty((8, cfg.k), dtype=torch.int32, device=dev)
    w = torch.empty((8, cfg.k), device=dev)
    L.forward(torch.from_numpy(as_i16(X)).to(dev), y, idx, w)
    torch.cuda.synchronize()
    compare_layer(OM.moe_forward_tokens(OL, X, cfg.k), idx.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy(),
                  f"byte {byte}")
    L.close()


@pytest.mark.parametrize("byte", [103, 141, 0, 255])
def test_mxfp4_scale_bytes_outside_the_batched_range(byte):
    """Rejected at init for a layer that may run the batched kernels; on the
    single-launch step every byte but 255 is accepted and exact."""
    import torch
    dev = device()
    cfg = synth.TINY_FP4
    lay = _mx_layer_with(byte)
    up = M.upload(lay, dev)
    with pytest.raises(M.MoEError) as ei:
        M.MoELayer.create(up, cfg.d, cfg.f, cfg.E, cfg.k, 1, 8)
    assert ei.value.status == M.MOE_ERR_UNSUPPORTED
    if byte == 255:
        with pytest.raises(M.MoEError) as ei:
            M.MoELayer.create(up, cfg.d, cfg.f, cfg.E, cfg.k, 1, 1)
        assert ei.value.status == M.MOE_ERR_UNSUPPORTED
        return
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 8, 3)
    L = M.MoELayer.create(up, cfg.d, cfg.f, cfg.E, cfg.k, 1, 1)
    y = torch.empty((3, cfg.d), device=dev)
    idx = torch.empty((3, cfg.k), dtype=torch.int32, device=dev)
    w = torch.empty((3, cfg.k), device=dev)
    xd = torch.from_numpy(as_i16(X)).to(dev)
    for t in range(3):
        L.forward(xd[t:t + 1], y[t:t + 1], idx[t:t + 1], w[t:t + 1])
    torch.cuda.synchronize()
    compare_layer(OM.moe_forward_tokens(OL, X, cfg.k), idx.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy(),
                  f"byte {byte}")
    L.close()


# ---------------------------------------------------------------- NVFP4 E4M3 scale sweep

E_NV, K_NV, D_NV, F_NV = 16, 8, 2048, 512


def _sweep_byte(i):
    """i-th byte of a sweep over every finite E4M3 byte: 0x00..0x7E, 0x80..0xFE."""
    c = i % 254
    return c if c < 127 else c + 1


def _one_block_rows(rows, K, block_of_row, byte_of_row, seed):
    """NVFP4 codes and scale bytes of a [rows][K] matrix whose row r holds
    E2M1 1.0 (code 2) in the 16 elements of block block_of_row(r) and 0
    elsewhere, with scale byte byte_of_row(r) on that block (other blocks:
    arbitrary finite bytes)."""
    u = np.zeros((rows, K), np.uint8)
    sb = ((np.arange(rows)[:, None] * 7 + np.arange(K // 16)[None, :] * 13 + seed) % 127).astype(np.uint8)
    for r in range(rows):
        b = block_of_row(r)
        u[r, 16 * b:16 * b + 16] = 2
        sb[r, b] = byte_of_row(r)
    return F.pack_codes(u), sb


def _nv_layer(gate, down, seed):
    """NVFP4 layer of E_NV identical experts: gate/down (codes, bytes) given
    or drawn, up drawn; matrix scales 1 for the given ones."""
    q1, s1, t1 = synth.nvfp4_experts(1, F_NV, D_NV, synth.key(seed, "nvsweep", "gate"), 0.02)
    qu, su, tu = synth.nvfp4_experts(1, F_NV, D_NV, synth.key(seed, "nvsweep", "up"), 0.02)
    qd, sd, td = synth.nvfp4_experts(1, D_NV, F_NV, synth.key(seed, "nvsweep", "down"), 0.02)
    if gate is not None:
        q1, s1, t1 = gate[0][None], gate[1][None], np.ones(1, np.float32)
    if down is not None:
        qd, sd, td = down[0][None], down[1][None], np.ones(1, np.float32)
    rep = lambda a: np.ascontiguousarray(np.broadcast_to(a, (E_NV,) + a.shape[1:]))
    return dict(router_w=synth.normal_f32(E_NV * D_NV, synth.key(seed, "nvsweep", "router"), 0.0, 0.02).reshape(E_NV, D_NV),
                router_b=None, gate_q=rep(q1), gate_s=rep(s1), gate_ts=rep(t1), up_q=rep(qu), up_s=rep(su),
                up_ts=rep(tu), down_q=rep(qd), down_s=rep(sd), down_ts=rep(td))


def _run_nv(lay, seed):
    import torch
    dev = device()
    OL = OM.Layer.from_dict(lay)
    x, _ = pick_token(OL, K_NV, 1e-2, lambda a: synth.bf16(D_NV, synth.key(seed, "nvsweep", "x", a)))
    L = M.MoELayer.create(M.upload(lay, dev), D_NV, F_NV, E_NV, K_NV, 1, 1)
    y = torch.full((1, D_NV), float("nan"), device=dev)
    L.forward(torch.from_numpy(as_i16(x[None])).to(dev), y)
    torch.cuda.synchronize()
    L.close()
    with np.errstate(over="ignore"):
        out = OM.moe_forward(OL, x, K_NV)
    # the experts are identical: h of any one, and the weights sum to 1
    Wg, Wu, Wd = OL.expert(0)
    xs = F.bf16_to_f64(x)
    with np.errstate(over="ignore"):
        h = OM.silu(Wg @ xs) * (Wu @ xs)
    return y.cpu().numpy()[0].astype(np.float64), out["y"], h, Wd


def test_nvfp4_every_e4m3_byte_in_the_down_projection():
    """Row r of W_d: E2M1 1.0 on the 16 elements of block r % 32, scale byte
    sweep(r): y_r = e4m3(byte) * (sum of those 16 h)."""
    code = _one_block_rows(D_NV, F_NV, lambda r: r % 32, lambda r: _sweep_byte(37 * r), 1)
    y, yo, h, Wd = _run_nv(_nv_layer(None, code, 11), 11)
    seen = {_sweep_byte(37 * r) for r in range(D_NV)}
    assert len(seen) == 254
    bound = np.abs(Wd) @ np.abs(h)  # per row: the sum of the magnitudes of its terms
    assert np.abs(y - yo).max() <= Y_TOL * np.abs(yo).max()
    bad = np.nonzero(np.abs(y - yo) > Y_TOL * bound + 1e-30)[0]
    assert bad.size == 0, f"rows {bad[:8]} (bytes {[hex(_sweep_byte(37 * r)) for r in bad[:8]]})"


def test_nvfp4_every_e4m3_byte_in_the_gate_projection():
    """Row i of W_g: E2M1 1.0 on block i % 128, scale byte sweep(i); W_d
    picks h_(r % 512) into output row r: y_r = h_(r % 512), each checked to
    2e-3 of its own magnitude (plus the binary16 quantum of h)."""
    gate = _one_block_rows(F_NV, D_NV, lambda i: i % 128, lambda i: _sweep_byte(37 * i + 5), 2)
    u = np.zeros((D_NV, F_NV), np.uint8)
    u[np.arange(D_NV), np.arange(D_NV) % F_NV] = 2
    sd = np.full((D_NV, F_NV // 16), 0x38, np.uint8)  # E4M3 1.0
    y, yo, h, Wd = _run_nv(_nv_layer(gate, (F.pack_codes(u), sd), 12), 12)
    assert {_sweep_byte(37 * i + 5) for i in range(F_NV)} == {_sweep_byte(c) for c in range(254)}
    hr = np.abs(h[np.arange(D_NV) % F_NV])
    bad = np.nonzero(np.abs(y - yo) > Y_TOL * hr + 2.0 ** -20)[0]
    assert bad.size == 0, f"rows {bad[:8]} (gate bytes {[hex(_sweep_byte(37 * (r % F_NV) + 5)) for r in bad[:8]]})"


# ---------------------------------------------------------------- repack


@pytest.mark.parametrize("rows,K", [(3, 128), (64, 512), (1000, 2048), (7, 8192)])
def test_int4_repack_matches_the_stored_layout(rows, K):
    import torch
    dev = device()
    u = np.random.default_rng(rows + K).integers(0, 16, size=(rows, K), dtype=np.uint8)
    canon = (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)  # element k in byte k/2, low nibble for even k
    src = torch.from_numpy(canon).to(dev)
    dst = torch.full((rows, K // 2), 0xAA, dtype=torch.uint8, device=dev)
    M.moe_int4_repack(src, dst, rows, K)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy(), F.pack_codes(u))


# ---------------------------------------------------------------- init on a stream

def test_init_on_stream_matches_init():
    """A flagship layer that may run the batched kernels, initialized on a
    side stream (moe_decode_init_on_stream: workspace clear, tile-major
    copies and argument copy on that stream, only it synchronized): 1-token
    steps and a T = 64 call bit-identical to the layer initialized by
    moe_decode_init, and the 1-token steps within the bar of the oracle."""
    import torch
    dev = device()
    cfg = synth.BATCH
    lay = synth.make_layer(cfg, 3)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 3, cfg.T)
    up = M.upload(lay, dev)
    side = torch.cuda.Stream()
    La = M.MoELayer.create(up, cfg.d, cfg.f, cfg.E, cfg.k, 1, cfg.T)
    Lb = M.MoELayer.create(up, cfg.d, cfg.f, cfg.E, cfg.k, 1, cfg.T, init_stream=side)
    torch.cuda.current_stream().wait_stream(side)
    xd = torch.from_numpy(as_i16(X)).to(dev)
    outs = []
    for L in (La, Lb):
        y1 = torch.empty((2, cfg.d), device=dev)
        i1 = torch.empty((2, cfg.k), dtype=torch.int32, device=dev)
        w1 = torch.empty((2, cfg.k), device=dev)
        for t in range(2):
            L.forward(xd[t:t + 1], y1[t:t + 1], i1[t:t + 1], w1[t:t + 1])
        yb = torch.empty((cfg.T, cfg.d), device=dev)
        ib = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev)
        L.forward(xd, yb, ib)
        torch.cuda.synchronize()
        outs.append([a.cpu().numpy() for a in (y1, i1, w1, yb, ib)])
        assert L.error_flags() == 0
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    compare_layer(OM.moe_forward_tokens(OL, X[:2], cfg.k), outs[1][1], outs[1][2], outs[1][0], "init on a stream")
    La.close()
    Lb.close()


def test_init_on_stream_rejects_like_init():
    """An MXFP4 scale byte outside the batched path's range: the stream form
    of init returns the same status."""
    import torch
    dev = device()
    cfg = synth.TINY_FP4
    up = M.upload(_mx_layer_with(141), dev)
    with pytest.raises(M.MoEError) as ei:
        M.MoELayer.create(up, cfg.d, cfg.f, cfg.E, cfg.k, 1, 8, init_stream=torch.cuda.Stream())
    assert ei.value.status == M.MOE_ERR_UNSUPPORTED

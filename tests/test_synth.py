"""The seeded generator: determinism, element addressability, distribution,
and that its packer and quantizer agree bit for bit with the oracle's
independently written ones."""
import numpy as np

import synth
from oracle import formats as F


def test_same_seed_same_bytes_and_distinct_streams():
    a = synth.make_layer(synth.TINY, 3)
    b = synth.make_layer(synth.TINY, 3)
    c = synth.make_layer(synth.TINY, 4)
    for k in a:
        if a[k] is not None:
            assert np.array_equal(a[k], b[k])
    assert not np.array_equal(a["gate_q"], c["gate_q"])
    assert not np.array_equal(a["gate_q"], a["up_q"])


def test_thread_count_does_not_change_output():
    import os
    import subprocess
    import sys
    code = ("import synth,hashlib;L=synth.make_layer(synth.TINY,5);"
            "print(hashlib.sha256(b''.join(v.tobytes() for v in L.values() if v is not None)).hexdigest())")
    outs = []
    for n in ("1", "3"):
        env = dict(os.environ, OMP_NUM_THREADS=n)
        outs.append(subprocess.check_output([sys.executable, "-c", code], env=env,
                                            cwd=os.path.dirname(os.path.dirname(__file__))).strip())
    assert outs[0] == outs[1]


def test_normal_moments():
    x = synth.normal_f32(1 << 20, synth.key(1, "moments"))
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1) < 5e-3
    assert abs(np.mean(x ** 4) - 3) < 0.05


def test_bf16_draws_are_rounded_normals():
    b = synth.bf16(1 << 16, synth.key(2, "bf"))
    f = synth.normal_f32(1 << 16, synth.key(2, "bf"))
    np.testing.assert_array_equal(b, F.f64_to_bf16_bits(f.astype(np.float64)))


def test_quantizer_and_packer_agree_with_oracle():
    q, s, w = synth.int4_matrix(512, 384, synth.key(6, "q"), 0.02, with_fp32=True)
    u, s2 = F.quantize(w)
    np.testing.assert_array_equal(s, s2)
    np.testing.assert_array_equal(q, F.pack_codes(u))
    u3 = np.random.default_rng(0).integers(0, 16, size=(8, 256))
    np.testing.assert_array_equal(synth.pack_codes(u3), F.pack_codes(u3))


def test_zipf_bias_is_a_log_probability_vector():
    b = synth.zipf_bias(synth.BATCH, 1).astype(np.float64)
    p = np.exp(b)
    assert abs(p.sum() - 1) < 1e-5
    ranks = np.argsort(-p)
    assert np.allclose(p[ranks[0]] / p[ranks[1]], 2 ** 1.1, rtol=1e-5)


def test_mxfp4_quantizer_agrees_with_oracle():
    """The generator's MXFP4 quantizer (C) and the oracle's (numpy), written
    independently from the MX conversion rule, agree bit for bit: on
    N(0, 0.02) draws, on wide-range values, on exact ties and on zero blocks;
    and an MXFP4 layer draws the same normals as the int4 one."""
    rng = np.random.default_rng(5)
    w = np.concatenate([
        synth.normal_f32(64 * 256, synth.key(7, "fp4"), 0.0, 0.02).reshape(64, 256),
        (rng.normal(0, 1, (64, 256)) * 2.0 ** rng.integers(-30, 30, (64, 1))),
        # exact ties between neighbouring E2M1 values at scale 1 (block max 4)
        np.tile(np.array([4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0] * 4), (8, 8)),
        np.zeros((8, 256)),
    ]).astype(np.float32)
    q, s = synth.quantize_pack_mxfp4(w)
    u, s2 = F.quantize_mxfp4(w)
    np.testing.assert_array_equal(s, s2)
    np.testing.assert_array_equal(q, F.pack_codes(u))
    a = synth.make_layer(synth.TINY, 3)
    b = synth.make_layer(synth.TINY_FP4, 3)
    assert b["gate_s"].dtype == np.uint8 and b["gate_q"].shape == a["gate_q"].shape
    np.testing.assert_array_equal(a["router_w"], b["router_w"])
    # same draws: the MXFP4 weights are within half a step of the int4 ones' source values
    Wi = F.dequant(a["gate_q"][0], a["gate_s"][0], 256)
    Wf = F.dequant_mxfp4(b["gate_q"][0], b["gate_s"][0], 256)
    assert np.corrcoef(Wi.ravel(), Wf.ravel())[0, 1] > 0.95


def test_nvfp4_quantizer_agrees_with_oracle():
    """The generator's NVFP4 quantizer (C: direct E4M3 rounding through
    frexp) and the oracle's (numpy: nearest of all E4M3 values) agree bit for
    bit, tensor scale included, on N(0, 0.02) draws, on blocks of very
    different magnitudes and on a zero matrix."""
    rng = np.random.default_rng(15)
    mats = [
        synth.normal_f32(64 * 256, synth.key(8, "nv"), 0.0, 0.02).reshape(64, 256),
        (rng.normal(0, 1, (32, 256)) * 2.0 ** rng.integers(-12, 4, (32, 16)).repeat(16, axis=1)).astype(np.float32),
        np.zeros((4, 128), np.float32),
    ]
    for w in mats:
        q, s, t = synth.quantize_nvfp4(w)
        u, s2, t2 = F.quantize_nvfp4(w)
        assert t == t2
        np.testing.assert_array_equal(s, s2)
        np.testing.assert_array_equal(q, F.pack_codes(u))
    lay = synth.make_layer(synth.TINY_NV, 3)
    assert lay["gate_ts"].shape == (synth.TINY.E,) and lay["gate_s"].shape[-1] == synth.TINY.d // 16
    q, s, t = synth.quantize_nvfp4(np.asarray(synth.normal_f32(128 * 256, synth.key(9, "nv"), 0.0, 0.02)).reshape(128, 256))
    assert t > 0

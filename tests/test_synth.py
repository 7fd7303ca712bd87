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

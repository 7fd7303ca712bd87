"""The seeded input generator's C code (synth/synth.c, synth/normal.c) built
with AddressSanitizer and UndefinedBehaviorSanitizer into a small driver
program: every generator entry point runs on small shapes (ragged sizes
included) with no sanitizer report.  Its outputs match the normal build's
through the Python wrappers: every code, scale, bf16 draw and permutation
bit for bit, and the fp32 normal draws (and the NVFP4 matrix scales, taken
from their maxima) within a few units in the last place (the instrumented build does not vectorize the Box-Muller transform's
log and sine the same way, so those round differently)."""
import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

import synth

HERE = os.path.dirname(os.path.abspath(synth.__file__))

DRIVER = r"""
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
uint64_t synth_key(uint64_t, uint64_t);
void synth_normal_f32(float*, int64_t, uint64_t, double, double);
void synth_bf16(uint16_t*, int64_t, uint64_t, double, double);
void synth_int4(uint8_t*, uint16_t*, int64_t, int64_t, uint64_t, double, float*);
void synth_int4_experts(uint8_t*, uint16_t*, int64_t, int64_t, int64_t, uint64_t, double);
void synth_mxfp4_experts(uint8_t*, uint8_t*, int64_t, int64_t, int64_t, uint64_t, double);
void synth_nvfp4_experts(uint8_t*, uint8_t*, float*, int64_t, int64_t, int64_t, uint64_t, double);
void synth_permutation(int32_t*, int32_t, uint64_t);
static void dump(const char* name, const void* p, size_t n) {
  FILE* f = fopen(name, "wb");
  if (!f || fwrite(p, 1, n, f) != n) exit(3);
  fclose(f);
}
int main(void) {
  const uint64_t k = synth_key(0x5EED, 7);
  float* nf = malloc(1003 * sizeof(float));
  synth_normal_f32(nf, 1003, k, 0.5, 2.0);
  dump("normal.bin", nf, 1003 * sizeof(float));
  uint16_t* bf = malloc(517 * 2);
  synth_bf16(bf, 517, k + 1, 0.0, 1.0);
  dump("bf16.bin", bf, 517 * 2);
  const int64_t R = 19, K = 256, E = 3;
  uint8_t* q = malloc(E * R * K / 2);
  uint16_t* s = malloc(E * R * (K / 32) * 2);
  float* w = malloc(R * K * sizeof(float));
  synth_int4(q, s, R, K, k + 2, 0.02, w);
  dump("int4_q.bin", q, R * K / 2);
  dump("int4_s.bin", s, R * (K / 32) * 2);
  dump("int4_w.bin", w, R * K * sizeof(float));
  synth_int4_experts(q, s, E, R, K, k + 3, 0.02);
  dump("int4e_q.bin", q, E * R * K / 2);
  dump("int4e_s.bin", s, E * R * (K / 32) * 2);
  uint8_t* ms = malloc(E * R * (K / 32));
  synth_mxfp4_experts(q, ms, E, R, K, k + 4, 0.02);
  dump("mx_q.bin", q, E * R * K / 2);
  dump("mx_s.bin", ms, E * R * (K / 32));
  uint8_t* ns = malloc(E * R * (K / 16));
  float* nt = malloc(E * sizeof(float));
  synth_nvfp4_experts(q, ns, nt, E, R, K, k + 5, 0.02);
  dump("nv_q.bin", q, E * R * K / 2);
  dump("nv_s.bin", ns, E * R * (K / 16));
  dump("nv_t.bin", nt, E * sizeof(float));
  int32_t* pm = malloc(37 * 4);
  synth_permutation(pm, 37, k + 6);
  dump("perm.bin", pm, 37 * 4);
  free(nf); free(bf); free(q); free(s); free(w); free(ms); free(ns); free(nt); free(pm);
  return 0;
}
"""


def _load(tmp, name, dtype):
    return np.fromfile(os.path.join(tmp, name), dtype=dtype)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_generator_under_address_and_undefined_sanitizers(tmp_path):
    tmp = str(tmp_path)
    with open(os.path.join(tmp, "driver.c"), "w") as fh:
        fh.write(DRIVER)
    exe = os.path.join(tmp, "driver")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
    # each source with the optimization flags of the library build (normal.c's
    # vector math under -ffast-math decides the draws' last bits)
    norm_o, synth_o = os.path.join(tmp, "normal.o"), os.path.join(tmp, "synth.o")
    subprocess.check_call(["gcc", *san, "-O3", "-ffast-math", "-fopenmp-simd", "-c", "-o", norm_o,
                           os.path.join(HERE, "normal.c")])
    subprocess.check_call(["gcc", *san, "-O2", "-fopenmp", "-c", "-o", synth_o, os.path.join(HERE, "synth.c")])
    subprocess.check_call(["gcc", *san, "-O2", "-fopenmp", "-o", exe, os.path.join(tmp, "driver.c"), synth_o, norm_o,
                           "-lm", "-lmvec"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="2")
    r = subprocess.run([exe], cwd=tmp, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-3000:]
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-3000:]

    L = synth.lib()
    k = L.synth_key(0x5EED, 7)

    def call(fn, *args):
        getattr(L, fn)(*[a.ctypes.data if isinstance(a, np.ndarray) else a for a in args])

    nf = np.empty(1003, np.float32)
    call("synth_normal_f32", nf, 1003, k, 0.5, 2.0)
    bf = np.empty(517, np.uint16)
    call("synth_bf16", bf, 517, k + 1, 0.0, 1.0)
    R, K, E = 19, 256, 3
    q = np.empty(E * R * K // 2, np.uint8)
    s = np.empty(E * R * (K // 32), np.uint16)
    w = np.empty(R * K, np.float32)
    call("synth_int4", q, s, R, K, k + 2, 0.02, w)
    assert np.array_equal(q[:R * K // 2], _load(tmp, "int4_q.bin", np.uint8))
    assert np.array_equal(s[:R * (K // 32)], _load(tmp, "int4_s.bin", np.uint16))
    np.testing.assert_allclose(w, _load(tmp, "int4_w.bin", np.float32), rtol=2e-6, atol=0)
    call("synth_int4_experts", q, s, E, R, K, k + 3, 0.02)
    assert np.array_equal(q, _load(tmp, "int4e_q.bin", np.uint8))
    assert np.array_equal(s, _load(tmp, "int4e_s.bin", np.uint16))
    ms = np.empty(E * R * (K // 32), np.uint8)
    call("synth_mxfp4_experts", q, ms, E, R, K, k + 4, 0.02)
    assert np.array_equal(q, _load(tmp, "mx_q.bin", np.uint8))
    assert np.array_equal(ms, _load(tmp, "mx_s.bin", np.uint8))
    ns = np.empty(E * R * (K // 16), np.uint8)
    nt = np.empty(E, np.float32)
    call("synth_nvfp4_experts", q, ns, nt, E, R, K, k + 5, 0.02)
    assert np.array_equal(q, _load(tmp, "nv_q.bin", np.uint8))
    assert np.array_equal(ns, _load(tmp, "nv_s.bin", np.uint8))
    np.testing.assert_allclose(nt, _load(tmp, "nv_t.bin", np.float32), rtol=2e-6, atol=0)  # from max |w|
    pm = np.empty(37, np.int32)
    call("synth_permutation", pm, 37, k + 6)
    assert np.array_equal(pm, _load(tmp, "perm.bin", np.int32))
    np.testing.assert_allclose(nf, _load(tmp, "normal.bin", np.float32), rtol=2e-6, atol=1e-6)  # sigma 2: values near 0
    assert np.array_equal(bf, _load(tmp, "bf16.bin", np.uint16))

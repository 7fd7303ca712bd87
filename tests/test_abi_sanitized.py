"""The library's host code (argument checks, workspace layout, status
strings -- everything tests/test_abi_cpu.py exercises) built with
AddressSanitizer and UndefinedBehaviorSanitizer on the host side only
(device code unchanged), and tests/test_abi_cpu.py run against that build in
a child process with the sanitizer runtime preloaded: the tests pass and
the sanitizers report nothing.  Takes about a minute and a half (the
build)."""
import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from sparse_moe_decode_gemv_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.slow
@pytest.mark.skipif(not os.path.exists(B.HIPCC) or _asan_runtime() is None, reason="hipcc or its ASan runtime missing")
def test_host_code_under_address_and_undefined_sanitizers(tmp_path):
    tmp = str(tmp_path)
    # each -fsanitize behind -Xarch_host: the host pass only
    san = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
           "-Xarch_host", "-g"]

    def compile_one(src):
        obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
        subprocess.check_call([B.HIPCC, *B.FLAGS, *san, "-c", os.path.join(B.CSRC, src), "-o", obj],
                              stderr=subprocess.DEVNULL)
        return obj

    with ThreadPoolExecutor(max_workers=len(B.SOURCES)) as ex:
        objs = list(ex.map(compile_one, B.SOURCES))
    lib = os.path.join(tmp, "libmoe_decode_sanitized.so")
    subprocess.check_call([B.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *san[:2], "-o", lib, *objs])

    runner = (
        "import sys\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "import sparse_moe_decode_gemv_amd as M\n"
        f"M.LIB_PATH = {lib!r}\n"
        "import pytest\n"
        f"sys.exit(pytest.main([{os.path.join(ROOT, 'tests', 'test_abi_cpu.py')!r}, '-q', '-p', 'no:cacheprovider']))\n"
    )
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", runner], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in r.stdout, out[-2000:]

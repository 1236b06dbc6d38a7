"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
libkda.so is rebuilt with the sanitizers on its host side only (-Xarch_host;
device code is compiled as usual), and tests/test_abi_host.py runs against it in
a child process with the sanitizer runtime preloaded.  Every argument check of
the C ABI thus runs instrumented, without a GPU (no call here reaches HIP)."""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]


def _runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_abi_host_under_sanitizers(tmp_path):
    sys.path.insert(0, ROOT)
    from gated_delta_rule_99_amd import build as kb

    rt = _runtime()
    if not os.path.exists(kb.HIPCC) or rt is None:
        pytest.skip("hipcc or the clang sanitizer runtime is not available")
    flags = [f for f in kb.COMMON if f != "-O3"] + ["-O1", "-g"]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.run([kb.HIPCC, *flags, *kb.DEVICE_FLAGS, *SAN, "-c", src, "-o", obj],
                       check=True, capture_output=True, text=True)
        return obj

    with ThreadPoolExecutor(8) as ex:
        objs = list(ex.map(compile_one, kb.sources()))
    lib = str(tmp_path / "libkda_san.so")
    subprocess.run([kb.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", lib,
                    *SAN[:4], "-shared-libsan"], check=True, capture_output=True, text=True)

    log = str(tmp_path / "san")
    env = dict(os.environ, LD_PRELOAD=rt,
               ASAN_OPTIONS=f"detect_leaks=0:verify_asan_link_order=0:log_path={log}",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={log}")
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from gated_delta_rule_99_amd import kda\n"
            "kda.load(%r)\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', %r]))\n"
            % (ROOT, lib, os.path.join(HERE, "test_abi_host.py")))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=600)
    reports = "".join(open(p).read() for p in glob.glob(log + "*"))
    assert r.returncode == 0 and not reports, r.stdout[-2000:] + r.stderr[-2000:] + reports
    assert " passed" in r.stdout

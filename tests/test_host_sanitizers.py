"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every source is compiled for the host only, with the sanitizers (each -fsanitize= behind
-Xarch_host) and an empty device binary in place of the kernels, linked with tests/host_check.cpp
and run on the CPU: parameter layouts, the workspace carve of every shipped configuration,
schedules and the argument checks that reject calls before any launch.  No kernel is launched and
no GPU is used.  Objects are cached under gpt_lm_step_amd/_build/san and rebuilt when their
source or a header changes.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gpt_lm_step_amd", "csrc")
OUT = os.path.join(ROOT, "gpt_lm_step_amd", "_build", "san")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
EMPTY = os.path.join(OUT, "empty_device_binary")
FLAGS = ["--offload-arch=gfx950", "--cuda-host-only", "-O1", "-g", "-std=c++17", "-fPIC",
         "-Xclang", "-fcuda-include-gpubinary", "-Xclang", EMPTY,
         "-I", os.path.join(ROOT, "include"), "-x", "hip"]


def _newest_header():
    hs = glob.glob(os.path.join(CSRC, "*.h")) + glob.glob(os.path.join(ROOT, "include", "*.h"))
    return max(os.path.getmtime(h) for h in hs)


def _compile(src, extra=()):
    obj = os.path.join(OUT, os.path.basename(src) + ".o")
    if (os.path.exists(obj) and os.path.getmtime(obj) > os.path.getmtime(src)
            and os.path.getmtime(obj) > _newest_header()):
        return obj
    cmd = [HIPCC, *FLAGS, *SAN, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return obj


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.timeout(600)
def test_host_code_under_address_and_undefined_behaviour_sanitizers():
    import concurrent.futures as cf
    os.makedirs(OUT, exist_ok=True)
    open(EMPTY, "wb").close()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(min(len(srcs), 8)) as ex:
        objs = list(ex.map(_compile, srcs))
    objs.append(_compile(os.path.join(ROOT, "tests", "host_check.cpp")))
    exe = os.path.join(OUT, "host_check")
    # the link is a host step: the host compiler with the sanitizer runtimes and the HIP runtime
    r = subprocess.run([CLANG, "-fsanitize=address,undefined", *objs, "-o", exe,
                        "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "host checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr

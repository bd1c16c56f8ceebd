"""The host side of libcsa (argument validation, workspace sizing, dispatch) under
AddressSanitizer and UndefinedBehaviorSanitizer: the library is rebuilt with both on its host
compilation only (device code as usual), and the C-ABI tests run against it in a separate
process that preloads the sanitizer runtime.  Any report fails the test.  No GPU is used."""
import glob
import os
import subprocess
import sys

import pytest

from coreset_softmax_attention_amd import build_lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_DIR = os.path.join(build_lib.BUILD, "san")
SAN_LIB = os.path.join(SAN_DIR, "libcsa_san.so")


def asan_runtime():
    base = os.path.join(os.path.dirname(build_lib.hipcc()), "..", "llvm", "lib", "clang")
    hits = sorted(glob.glob(os.path.join(base, "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


def build_sanitized():
    os.makedirs(SAN_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(build_lib.CSRC, "*.hip")))
    deps = sources + glob.glob(os.path.join(build_lib.CSRC, "*.hpp")) + [os.path.join(ROOT, "include", "csa.h")]
    if os.path.exists(SAN_LIB) and os.path.getmtime(SAN_LIB) > max(os.path.getmtime(f) for f in deps):
        return SAN_LIB
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    flags = [f"--offload-arch={build_lib.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", f"-I{os.path.join(ROOT, 'include')}"]
    procs, objs = [], []
    for src in sources:
        obj = os.path.join(SAN_DIR, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        procs.append(subprocess.Popen([build_lib.hipcc(), *flags, *san, "-c", src, "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    for p in procs:
        out, err = p.communicate()
        assert p.returncode == 0, err[-2000:]
    link = [build_lib.hipcc(), f"--offload-arch={build_lib.ARCH}", "-shared", "-fPIC", *san[:4], "-shared-libasan",
            "-o", SAN_LIB, *objs]
    subprocess.run(link, check=True, capture_output=True)
    return SAN_LIB


def test_c_abi_validation_is_clean_under_address_and_undefined_behavior_sanitizers():
    rt = asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime next to hipcc")
    lib = build_sanitized()
    env = dict(os.environ, LD_PRELOAD=rt, CSA_LIBRARY=lib, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], env=env, capture_output=True, text=True,
                       timeout=600, cwd=ROOT)
    text = r.stdout + r.stderr
    assert "AddressSanitizer" not in text and "runtime error:" not in text, text[-4000:]
    assert r.returncode == 0, text[-4000:]
    assert " passed" in r.stdout

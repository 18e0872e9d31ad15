"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds, each exercised by its own CPU tests in a child process that preloads the sanitizer
runtime, with every report fatal:
  - the oracle (oracle.c, gcc -fsanitize=address,undefined), run through the oracle pins;
  - the HIP library with the sanitizers on its host pass only (hipcc -Xarch_host), run through
    the ABI tests: argument validation of every entry point and the exported symbols.
Device code is never sanitized (no GPU sanitizer runs here).  The builds are cached under
tests/.sanitize_build, keyed by the sources they come from."""
import glob
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "tests", ".sanitize_build")
CSRC = os.path.join(ROOT, "expert_grouped_gemm_softmax_amd", "csrc")
ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
       "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _digest(paths, flags):
    h = hashlib.sha256(" ".join(flags).encode())
    for p in sorted(paths):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _cached(name, srcs, flags, build):
    os.makedirs(BUILD, exist_ok=True)
    out = os.path.join(BUILD, f"{name}_{_digest(srcs, flags)}.so")
    if not os.path.exists(out):
        for old in glob.glob(os.path.join(BUILD, f"{name}_*.so")):
            os.remove(old)
        tmp = out + ".tmp%d" % os.getpid()
        build(tmp)
        os.replace(tmp, out)
    return out


def _run_child(preload, script, timeout):
    env = dict(os.environ, LD_PRELOAD=preload, **ENV)
    res = subprocess.run([sys.executable, "-c", script], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=timeout)
    report = [ln for ln in (res.stdout + res.stderr).splitlines()
              if "Sanitizer" in ln or "runtime error" in ln]
    assert res.returncode == 0 and not report, (res.returncode, "\n".join(report[:20]), res.stdout[-3000:],
                                                res.stderr[-3000:])
    return res.stdout


def test_oracle_under_address_and_undefined_sanitizers():
    src = os.path.join(ROOT, "oracle", "oracle.c")
    flags = ["-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
    lib = _cached("oracle_asan", [src], flags,
                  lambda out: subprocess.run(["gcc", *flags, src, "-o", out, "-lm"], check=True))
    runtime = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    script = ("import sys, oracle; oracle._LIB_PATH = %r\n"
              "import pytest; sys.exit(pytest.main(['tests/test_oracle_pins.py', '-q', '-x', '-p', 'no:cacheprovider']))"
              % lib)
    out = _run_child(runtime, script, 900)
    assert " passed" in out


def test_library_host_code_under_address_and_undefined_sanitizers():
    runtimes = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not runtimes or not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("no hipcc / clang sanitizer runtime")
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "common.h"),
                                                            os.path.join(ROOT, "include", "moe.h")]
    flags = ["--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-g"]

    def build(out):
        subprocess.run(["/opt/rocm/bin/hipcc", *flags, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                        *[s for s in srcs if s.endswith(".hip")], "-o", out], check=True, capture_output=True)
    lib = _cached("moe_host_asan", srcs, flags, build)
    script = ("import sys; sys.path.insert(0, '.')\n"
              "from expert_grouped_gemm_softmax_amd import _abi; _abi.load(%r)\n"
              "import pytest; sys.exit(pytest.main(['tests/test_abi.py', '-q', '-x', '-p', 'no:cacheprovider', "
              "'-k', 'not code_object']))" % lib)
    out = _run_child(runtimes[0], script, 600)
    assert " passed" in out

"""Sanitizer builds on the host.

Two programs are built with AddressSanitizer and UndefinedBehaviorSanitizer and
run to completion with no report:

* the CPU oracle (gcc), driven by ``tests/sanitize_oracle.c`` through every
  exported function on small seeded inputs, edge shapes and argument errors;
* the C ABI's host code (hipcc; the sanitizers apply to the host side only),
  driven by ``tests/sanitize_api.cpp`` through every entry point with
  arguments the library rejects before any HIP call, and through the size
  queries and the id validator.

Neither run touches a GPU: the oracle is host code, and no call of the C ABI
driver passes validation, so nothing is launched.
"""

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "speculative_decoding_argmax_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")

# Sanitizer flags for gcc, and the same for hipcc restricted to the host side.
GCC_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer"]
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
# Device code is compiled (the kernels' registration needs it) but never run.
DEVICE = ["--offload-arch=gfx950", "-Xarch_device", "-O0", "-Xclang", "-target-feature",
          "-Xclang", "-packed-fp32-ops"]


def _run(cmd, **kw):
    return subprocess.run(cmd, capture_output=True, text=True, **kw)


def _sanitizers_available(compiler, tmp_path, flags, lang="c"):
    src = tmp_path / ("probe." + lang)
    src.write_text("int main(void) { return 0; }\n")
    r = _run([compiler, *flags, str(src), "-o", str(tmp_path / "probe")])
    return r.returncode == 0


def test_oracle_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if not gcc or not _sanitizers_available(gcc, tmp_path, GCC_SAN):
        pytest.skip("gcc with AddressSanitizer / UBSan not available")
    exe = tmp_path / "san_oracle"
    r = _run([gcc, "-std=c11", "-O1", "-g", *GCC_SAN, "-ffp-contract=off", "-Wall",
              "-Wno-unknown-pragmas", os.path.join(ROOT, "tests", "sanitize_oracle.c"),
              os.path.join(ROOT, "oracle", "mtp_oracle.c"), "-lm", "-o", str(exe)])
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = _run([str(exe)], env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "sanitized oracle run ok" in r.stdout


def test_c_abi_host_code_under_asan_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    srcs = [os.path.join(CSRC, n) for n in sorted(os.listdir(CSRC))
            if n.endswith(".hip") or n.endswith(".cpp")]
    srcs.append(os.path.join(ROOT, "tests", "sanitize_api.cpp"))

    def compile_one(src):
        obj = tmp_path / (os.path.basename(src) + ".o")
        r = _run([hipcc, "-x", "hip", "-O1", "-g", "-std=c++17", *DEVICE, *HOST_SAN,
                  "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", str(obj)])
        return src, obj, r

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(compile_one, srcs))
    for src, _, r in results:
        assert r.returncode == 0, f"{src}:\n{r.stderr}"
    exe = tmp_path / "san_api"
    r = _run([hipcc, "--offload-arch=gfx950", *HOST_SAN, *[str(o) for _, o, _ in results],
              "-o", str(exe)])
    assert r.returncode == 0, r.stderr
    # the HIP runtime keeps its own allocations until exit: leak checks off
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = _run([str(exe)], env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "sanitized C ABI run ok" in r.stdout


def test_sanitizer_build_reports_a_planted_overflow(tmp_path):
    """The gcc flags above do catch errors: a one-element heap overflow in a
    throwaway program built the same way fails with a report."""
    gcc = shutil.which("gcc")
    if not gcc or not _sanitizers_available(gcc, tmp_path, GCC_SAN):
        pytest.skip("gcc with AddressSanitizer / UBSan not available")
    src = tmp_path / "overflow.c"
    src.write_text("#include <stdlib.h>\n"
                   "int main(int argc, char **argv) {\n"
                   "  (void)argv; int *p = malloc(4 * sizeof(int));\n"
                   "  int v = p[argc + 3]; free(p); return v == 12345;\n}\n")
    exe = tmp_path / "overflow"
    r = _run([gcc, "-O0", "-g", *GCC_SAN, str(src), "-o", str(exe)])
    assert r.returncode == 0, r.stderr
    r = _run([str(exe)], timeout=60)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr

"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

- The C routing oracle (oracle/route_oracle.c), built with gcc and the two sanitizers,
  driven by tests/native/oracle_sanitize_main.c over exp, the pairwise sum, softmax up
  to 256 experts and full routings (drops, ties, capacity 0, 256 experts, empty input,
  rejected arguments), checking the maps' invariants on the way.
- The host side of the library (descriptor checks, workspace sizing, argument
  validation of every entry point in csrc/*.hip): the same sources as libmoe.so, with
  the sanitizers on the host half only (the device code is built as usual), linked into
  tests/native/abi_sanitize_main.c, which calls the host helpers over a grid of valid and
  invalid descriptors and every device entry point with arguments the validation
  rejects before any HIP call, so nothing is launched.
Any sanitizer report aborts the program (-fno-sanitize-recover=all) and fails the test.
"""
import concurrent.futures
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "token_dispatch_expert_router_amd", "csrc")
SOURCES = ["api.hip", "route.hip", "rows.hip", "gemm_mfma.hip", "gemm_valu.hip"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    pytest.skip("hipcc is not available")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout[-4000:] + r.stderr[-4000:]
    return r


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not available")
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g", "-O1",
          "-ffp-contract=off", "-fno-fast-math", os.path.join(ROOT, "oracle", "route_oracle.c"),
          os.path.join(NATIVE, "oracle_sanitize_main.c"), "-o", exe, "-lm"])
    r = _run([exe], env=ENV, timeout=300)
    assert r.stdout.strip().endswith("ok"), r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr


def test_abi_host_side_under_sanitizers(tmp_path):
    hipcc = _hipcc()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    inc = ["-I", os.path.join(ROOT, "include")]

    def obj(src):
        out = str(tmp_path / (os.path.basename(src) + ".o"))
        flags = ["-ffp-contract=off"] if src.endswith("route.hip") else []
        _run([hipcc, "--offload-arch=gfx950", "-O3", "-g", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *flags, *san, *inc,
              "-c", src, "-o", out])
        return out

    with concurrent.futures.ThreadPoolExecutor(max_workers=5) as ex:
        objs = list(ex.map(obj, [os.path.join(CSRC, s) for s in SOURCES]))
    main_o = str(tmp_path / "abi_main.o")
    _run([hipcc, "-x", "c", "-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
          "-fsanitize=undefined", *inc, "-c", os.path.join(NATIVE, "abi_sanitize_main.c"),
          "-o", main_o])
    exe = str(tmp_path / "abi_san")
    _run([hipcc, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
          "-fsanitize=undefined", "-o", exe, main_o, *objs])
    r = _run([exe], env=ENV, timeout=300)
    assert r.stdout.strip().startswith("ok"), r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr

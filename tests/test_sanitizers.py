"""The CPU code under AddressSanitizer and UndefinedBehaviorSanitizer.

* The oracle (gcc, -fsanitize=address,undefined, no recovery) runs every pin
  of tests/oracle_pins.py in a child process that preloads gcc's ASan runtime.
* The library's host code (argument checks, the launch planner, the launch
  set-up) is rebuilt with clang's host-side sanitizers and the CPU ABI and
  work-list tests run against it in a child process that preloads clang's
  runtime.
Each half first shows that its set-up reports a planted heap overrun, so a
clean run means something.  Any report fails the test (no recovery, non-zero
exit).
"""
import os
import subprocess
import sys
import textwrap

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g", "-fno-omit-frame-pointer"]


def _gcc_asan():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's ASan runtime is not installed")
    return path


def _run(code, preload, timeout=600):
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    return subprocess.run([sys.executable, "-c", textwrap.dedent(code)], capture_output=True,
                          text=True, env=env, timeout=timeout, cwd=ROOT)


PINS = """
    import sys
    sys.path[:0] = [{root!r}, {tests!r}]
    import oracle
    from oracle_pins import ALL_PINS
    orc = oracle.Oracle({lib!r})
    for name in {names!r}:
        ALL_PINS[name](orc)
        print(name, "ok", flush=True)
"""


def _oracle_variant(tmp, name, source):
    src = os.path.join(tmp, name + ".c")
    with open(src, "w") as f:
        f.write(source)
    import shutil
    shutil.copy(oracle.HDR, os.path.join(tmp, "pa_oracle.h"))
    return oracle.build(src, os.path.join(tmp, f"lib{name}.so"), extra_flags=SAN)


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    rt = _gcc_asan()
    src = open(oracle.SRC).read()
    # canary: the logit buffer one element short, so the row that reads all
    # max_context_len keys writes one past its end
    bad = src.replace("malloc(sizeof(double) * (size_t)(a->max_context_len > 0 ? a->max_context_len : 1))",
                      "malloc(sizeof(double) * (size_t)(a->max_context_len > 1 ? a->max_context_len - 1 : 1))")
    assert bad != src
    lib = _oracle_variant(str(tmp_path), "canary", bad)
    r = _run(PINS.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib, names=["hand"]), rt)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, r.stderr[-2000:]

    from oracle_pins import ALL_PINS
    lib = _oracle_variant(str(tmp_path), "checked", src)
    r = _run(PINS.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib,
                         names=sorted(ALL_PINS)), rt)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    assert r.stdout.count(" ok") == len(ALL_PINS)


HOST_TESTS = """
    import sys
    sys.path[:0] = [{root!r}, {tests!r}]
    import speculative_decoding_verify_paged_amd as pav
    pav.LIB_PATH = {lib!r}
    import pytest
    sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "-p", "no:xdist",
                          {abi!r}, {wl!r}]))
"""


def test_host_library_under_asan_and_ubsan(tmp_path):
    from speculative_decoding_verify_paged_amd import build as b
    if not os.path.exists(os.path.join(b.BUILD, "pa_combine.hip.o")):
        pytest.skip("no regular build objects in _build/ (run the package build first)")
    rt = b.asan_runtime()
    # canary: a host function compiled with the same flags that reads one past
    # a heap array
    canary = tmp_path / "canary.hip"
    canary.write_text(textwrap.dedent("""
        #include <hip/hip_runtime.h>
        #include <cstdlib>
        extern "C" int canary(int n) {
          int* p = static_cast<int*>(std::malloc(sizeof(int) * n));
          for (int i = 0; i < n; ++i) p[i] = i;
          int s = p[n];
          std::free(p);
          return s;
        }
    """))
    so = str(tmp_path / "libcanary.so")
    r = subprocess.run([b.hipcc(), "--offload-arch=" + b.ARCH, "-O1", "-g", "-fPIC", "-shared",
                        *b.HOST_SANITIZE, str(canary), "-o", so], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = _run(f"import ctypes; print(ctypes.CDLL({so!r}).canary(5))", rt)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, r.stderr[-2000:]

    lib = b.build_host_checked(str(tmp_path / "checked"))
    r = _run(HOST_TESTS.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib,
                               abi=os.path.join(ROOT, "tests", "test_abi.py"),
                               wl=os.path.join(ROOT, "tests", "test_worklist_model.py")), rt)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-3000:]
    assert " passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]

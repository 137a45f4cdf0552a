"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

s2r_oracle.cpp is compiled with -fsanitize=address,undefined into a temporary library and the
whole pin suite runs against it in a child process (the sanitizer runtime has to be loaded
before the Python interpreter's own libraries, so it is preloaded into that process only).
Any out-of-bounds access, use after free, signed overflow, misaligned or null access or
other undefined behaviour stops the child with a report, and the test fails.
"""
import os
import subprocess
import sys

import pytest

import oracle

_CHILD = """
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, pins
with oracle.using({lib!r}):
    for pin in pins.ALL_PINS:
        pin()
print("ALL PINS PASSED UNDER SANITIZERS")
"""


def _runtime(name):
    path = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.timeout(900)
def test_pins_under_asan_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("no AddressSanitizer runtime for g++")
    lib = str(tmp_path / "liboracle_sanitized.so")
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-ffp-contract=off", "-fPIC", "-shared",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-o", lib, oracle.source_path()], check=True)
    tests = os.path.dirname(os.path.abspath(__file__))
    env = dict(os.environ)
    # the runtime goes first; whatever the environment already preloads stays after it
    env["LD_PRELOAD"] = asan + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    code = _CHILD.format(root=os.path.dirname(tests), tests=tests, lib=lib)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       timeout=900)
    report = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, report
    assert "ALL PINS PASSED UNDER SANITIZERS" in r.stdout, report
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, report


@pytest.mark.timeout(900)
def test_sanitizer_is_live(tmp_path):
    """A copy of the oracle with a planted out-of-bounds write (a block bit computed from the
    element index, past the end of a block-granular bitmap) must be reported."""
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("no AddressSanitizer runtime for g++")
    src = open(oracle.source_path()).read()
    old = "const uint64_t b = block_of(p, i);\n    bitmap[b / 64]"
    assert src.count(old) == 1
    bad = tmp_path / "planted.cpp"
    bad.write_text(src.replace(old, "const uint64_t b = i;\n    bitmap[b / 64]"))
    lib = str(tmp_path / "libplanted.so")
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-ffp-contract=off", "-fPIC", "-shared",
                    "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-o", lib,
                    str(bad)], check=True)
    tests = os.path.dirname(os.path.abspath(__file__))
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    code = _CHILD.format(root=os.path.dirname(tests), tests=tests, lib=lib)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       timeout=900)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, (r.stdout + r.stderr)[-2000:]

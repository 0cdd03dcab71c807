"""Host sanitizer pass (CPU only): the oracle, the allocator (recipe.cpp) and
the packed-file writer and parser (packfile.cpp) built with AddressSanitizer
and UndefinedBehaviorSanitizer and driven by tests/host/sanitize_driver.cpp
over random weights with special values, random and hostile allocation
inputs, and thousands of damaged files (flipped header and table bytes,
offsets and sizes near 2^64, truncation).  A parser with the old bounds check
that adds offset and size (which wraps) planted back must be caught."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixed_precision_weight_dq_amd", "csrc")
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]


def build(tmp, packfile_src: str) -> str:
    if not (shutil.which("gcc") and shutil.which("g++")):
        pytest.skip("gcc/g++ not found")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    for cc, src, extra in (("gcc", os.path.join(ROOT, "oracle", "dq_oracle.c"), ["-fopenmp", "-ffp-contract=off"]),
                           ("g++", os.path.join(CSRC, "recipe.cpp"), ["-std=c++17"] + inc),
                           ("g++", packfile_src, ["-std=c++17"] + inc)):
        obj = os.path.join(tmp, os.path.basename(src) + ".o")
        subprocess.run([cc, *SAN, *extra, "-c", src, "-o", obj], check=True, capture_output=True)
        objs.append(obj)
    exe = os.path.join(tmp, "driver")
    subprocess.run(["g++", *SAN, "-std=c++17", os.path.join(ROOT, "tests", "host", "sanitize_driver.cpp"),
                    *objs, "-fopenmp", "-o", exe], check=True, capture_output=True)
    return exe


def run(exe: str, tmp: str) -> subprocess.CompletedProcess:
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="1")
    return subprocess.run([exe, tmp], capture_output=True, text=True, timeout=600, env=env)


def test_host_code_is_sanitizer_clean(tmp_path):
    exe = build(str(tmp_path), os.path.join(CSRC, "packfile.cpp"))
    r = run(exe, str(tmp_path))
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "sanitize driver: 0 failures" in out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out


def test_wrapping_bounds_check_is_caught(tmp_path):
    src = open(os.path.join(CSRC, "packfile.cpp")).read()
    for good, bad in (("doff <= size &&\n             db <= size - doff;", "doff + db <= size;"),
                      ("soff <= size && sb <= size - soff;", "soff + sb <= size;")):
        assert src.count(good) == 1
        src = src.replace(good, bad)
    planted = tmp_path / "packfile.cpp"
    planted.write_text(src)
    shutil.copy(os.path.join(CSRC, "layout.hpp"), tmp_path / "layout.hpp")
    exe = build(str(tmp_path), str(planted))
    r = run(exe, str(tmp_path))
    assert r.returncode != 0

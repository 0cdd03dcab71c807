"""The quantize kernels' rounded quotient (quant_rule.hpp: a multiply by
fl32(1/s), with the IEEE divide only near a rounding tie) against the IEEE
divide, brute-forced on the CPU around every tie and level of every width,
including scales whose reciprocal is subnormal or overflows.  The harness
compiles the product header itself for the host, so it checks the code the
kernels inline.  A copy with a planted thinner margin must fail.

Source: "量化" tutorial (aiknowledge.cn), Step 1 (q = round(w / scale), numpy's
round half to even, fp32 arithmetic)."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HARNESS = os.path.join(ROOT, "tests", "host", "quant_rule_check.hip")
HEADER = os.path.join(ROOT, "mixed_precision_weight_dq_amd", "csrc", "quant_rule.hpp")


def hipcc():
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    pytest.skip("hipcc not found")


def build_and_run(src: str, exe: str) -> subprocess.CompletedProcess:
    subprocess.run([hipcc(), "--offload-arch=gfx950", "-O2", "-std=c++17", "-ffp-contract=off",
                    src, "-o", exe], check=True, capture_output=True, text=True)
    return subprocess.run([exe], capture_output=True, text=True, timeout=300)


def test_rounded_quotient_matches_ieee_divide(tmp_path):
    r = build_and_run(HARNESS, str(tmp_path / "qrc"))
    assert r.returncode == 0, r.stdout + r.stderr
    assert " bad 0 " in r.stdout


def test_thin_margin_is_caught(tmp_path):
    """The harness has teeth: with the safety margin cut from 2^-21 * limit to
    2^-27 * limit, some element near a tie rounds the wrong way."""
    src = open(HEADER).read()
    anchor = "return 0.5f - ldexpf(limit, -21);"
    assert src.count(anchor) == 1
    hdr_dir = tmp_path / "mixed_precision_weight_dq_amd" / "csrc"
    hdr_dir.mkdir(parents=True)
    (hdr_dir / "quant_rule.hpp").write_text(src.replace(anchor, "return 0.5f - ldexpf(limit, -27);"))
    (tmp_path / "tests" / "host").mkdir(parents=True)
    shutil.copy(HARNESS, tmp_path / "tests" / "host" / "quant_rule_check.hip")
    r = build_and_run(str(tmp_path / "tests" / "host" / "quant_rule_check.hip"), str(tmp_path / "qrc"))
    assert r.returncode != 0 and "MISMATCH" in r.stdout

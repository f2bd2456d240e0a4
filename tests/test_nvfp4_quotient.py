"""The NVFP4 insert kernel replaces the fp32 division y = r / S by a product
with an fp64 reciprocal (see the comment at the quotient in rope_insert.hip).
nvfp4_quotient_check.c restates that arithmetic on the host and compares the
E2M1 code it leads to with the code of the correctly rounded quotient, for
every E4M3 scale significand, every float r of [2^-4, 2^4) (sampled here with
stride 16; stride 1, 4.5e9 cases, is the full run), specials, and subnormal
quotients around the zero/nonzero boundary.  A planted fp32-only product
(r * fp32(1/S)) fails it."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nvfp4_quotient_check.c")


def build(tmp_path, src=SRC):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    exe = str(tmp_path / "nvq")
    subprocess.run([cc, "-O2", "-std=c11", "-ffp-contract=off", "-o", exe, src, "-lm"], check=True)
    return exe


def test_quotient_method_matches_correct_division(tmp_path):
    exe = build(tmp_path)
    r = subprocess.run([exe, "16"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches 0" in r.stdout


def test_check_detects_an_fp32_only_product(tmp_path):
    """The check has teeth: with the product taken in fp32 it reports
    mismatches."""
    text = open(SRC).read()
    planted = text.replace("const float q = (float)((double)r * inv_s);", "const float q = r * (float)inv_s;")
    assert planted != text
    src = tmp_path / "planted.c"
    src.write_text(planted)
    exe = build(tmp_path, str(src))
    r = subprocess.run([exe, "64"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 1 and "mismatches 0" not in r.stdout

"""The NVFP4 insert kernel replaces the fp32 division y = r / S by fp32
products and fmas (q0 = r * y0, e = fma(-q0, S, r), q = fma(e, y0, q0)), with
an fp64 reciprocal product when q is not a normal float (see the comment at
the quotient in rope_insert.hip).  nvfp4_quotient_check.c restates that
arithmetic on the host and compares the E2M1 code it leads to with the code of
the correctly rounded quotient, for every E4M3 scale significand, every
reciprocal within 2 ulps of 1/S, every float r of [2^-4, 2^4) (sampled here
with stride 16; stride 1 is the full run), specials, and quotients around the
zero/nonzero and subnormal/normal boundaries; it also requires every kept
quotient of magnitude 2^-100 or more to equal r / S bit for bit.  Planted
mistakes (no correction step, no fallback for non-normal quotients) fail it."""

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
    assert "mismatches 0 " in r.stdout and "quotients_off_by_bits 0" in r.stdout


@pytest.mark.parametrize("old,new", [
    ("float q = fmaf(e, y0, q0);", "float q = q0;"),                                  # no correction step
    ("if (!fast) q = (float)((double)r * inv_s_of(S, y0));", "(void)fast;"),          # no fallback
])
def test_check_detects_planted_mistakes(tmp_path, old, new):
    """The check has teeth: each planted mistake makes it report mismatches."""
    text = open(SRC).read()
    planted = text.replace(old, new)
    assert planted != text
    src = tmp_path / "planted.c"
    src.write_text(planted)
    exe = build(tmp_path, str(src))
    r = subprocess.run([exe, "64"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 1, r.stdout

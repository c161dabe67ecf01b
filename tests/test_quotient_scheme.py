"""The quantizers' fp32 quotient scheme (correctly rounded reciprocal and two
FMA residual steps, Markstein's theorem) gives the same INT4 and INT8 codes as
an IEEE divide: a C restatement of the scheme, compiled for the host CPU and
run over every fp16 scale and over random block maxima, with quotients next
to every rounding boundary. Needs clang (for _Float16 on the host)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _clang():
    for c in ("/opt/rocm/llvm/bin/clang", shutil.which("clang")):
        if c and os.path.exists(c):
            return c
    return None


def test_quotient_scheme_matches_divide(tmp_path):
    cc = _clang()
    if cc is None:
        pytest.skip("clang not found")
    exe = tmp_path / "quotient_scheme"
    subprocess.run([cc, "-O2", "-ffp-contract=off", os.path.join(HERE, "quotient_scheme.c"), "-o", str(exe), "-lm"],
                   check=True)
    r = subprocess.run([str(exe), "100000"], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "int4: " in r.stdout and "int8: " in r.stdout

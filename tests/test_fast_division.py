"""The four-over-six kernel replaces some true fp32 divisions by a
three-operation sequence (reciprocal multiply, exact FMA remainder, FMA
correction).  This CPU test proves, by exhausting every float32 numerator (and
every bf16 numerator for the block-scale division by 6), that the sequence is
correctly rounded wherever the kernel uses it: |n| >= 2**-117 and finite.
Elsewhere the kernel takes the true division.  The C check runs with IEEE
float32 and hardware FMA on the host (gcc -mfma, no contraction)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path_factory.mktemp("fastdiv") / "fastdiv_check")
    subprocess.run(["gcc", "-O2", "-mfma", "-fopenmp", "-ffp-contract=off", "-o", exe,
                    os.path.join(HERE, "c", "fastdiv_check.c"), "-lm"], check=True)
    return exe


@pytest.mark.parametrize("D,mode", [(6.0, "bf16"), (6.0, "f32"), (1536.0, "f32"), (2688.0, "f32")])
def test_fast_division_is_correctly_rounded(checker, D, mode):
    args = [checker, repr(D)] + (["bf16"] if mode == "bf16" else [])
    res = subprocess.run(args, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "bad_in_range=0" in res.stdout

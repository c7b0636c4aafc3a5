"""The page encoder's division (a reciprocal and one fused correction) decides
every stored code exactly as correctly rounded division does, over every
input the encoder can meet: an exhaustive check over all fp16 and bf16 source
values, in C (tests/division/check_recip_div.c and check_scale_div.c), no GPU."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "division", "check_recip_div.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_reciprocal_division_is_exact_on_reachable_inputs(tmp_path):
    exe = str(tmp_path / "check_recip_div")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-o", exe, SRC, "-lm"], check=True)
    env = dict(os.environ, OMP_NUM_THREADS=str(min(os.cpu_count() or 1, 16)))
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=900)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.split() == ["fp8_fp16", "0", "fp8_bf16", "0", "int_fp16", "0", "int_bf16", "0"]


SCALE_SRC = os.path.join(HERE, "division", "check_scale_div.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_group_scale_division_and_reciprocal_are_exact(tmp_path):
    """The INT group scale m / qmax (a multiply by the constant RN(1 / qmax)
    and one fused correction) and the reciprocal of the stored fp16 scale (the
    hardware estimate and one Newton step) equal the correctly rounded results
    for every fp16 and bf16 absmax and every fp16 scale."""
    exe = str(tmp_path / "check_scale_div")
    subprocess.run(["gcc", "-O2", "-o", exe, SCALE_SRC, "-lm"], check=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.split() == ["scale_div", "0", "recip_fp16", "0"]


AFFINE2_SRC = os.path.join(HERE, "division", "check_affine2_div.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_int2_code_division_is_exact(tmp_path):
    """The INT2 code's quotient RN((x - z) / s), taken as a multiply by
    RN(1 / s) and one fused correction, equals the correctly rounded quotient
    for every fp16 step s, over every fp32 dividend within 4,096 units in the
    last place of the rounding boundaries 0.5, 1.5, 2.5 and 3.5 steps, and
    over 512 dividends spread across [0, 3.6 s] per step."""
    exe = str(tmp_path / "check_affine2_div")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-o", exe, AFFINE2_SRC, "-lm"], check=True)
    env = dict(os.environ, OMP_NUM_THREADS=str(min(os.cpu_count() or 1, 16)))
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.split() == ["affine2_div", "0", "affine2_code", "0"]

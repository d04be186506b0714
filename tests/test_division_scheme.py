"""CPU check of the shared-divisor division the HIP kernels use.

The kernels divide many elements by one scale with a reciprocal and two
fused multiply-add corrections instead of a full IEEE division per element.
tests/pins/division_check.c sweeps every bf16 input, inputs next to every
E2M1 rounding midpoint and random binary32 inputs against thousands of
divisors and requires the result to equal the correctly rounded quotient
wherever a code can depend on it; the signed form (negated residuals, which
keeps the sign of x on zero quotients) must equal the magnitude form with the
sign copied back, bit for bit, everywhere it is checked.
"""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_reciprocal_two_corrections_is_correctly_rounded(tmp_path):
    exe = str(tmp_path / "divchk")
    subprocess.run(["gcc", "-O2", "-mfma", "-fopenmp", "-ffp-contract=off", "-o", exe,
                    os.path.join(ROOT, "tests", "pins", "division_check.c"), "-lm"], check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True,
                         env=dict(os.environ, OMP_NUM_THREADS="8")).stdout.split()
    checked, exact_bad, code_bad, signed_bad = map(int, out)
    assert checked > 10**8
    assert exact_bad == 0 and code_bad == 0 and signed_bad == 0

"""The binary64 exponential of the speculative-verification kernels is
Cody and Waite's reduction with a two-double ln 2 plus a degree-13 Taylor
polynomial (Horner) and ldexp.  This checks that method, written out in C
from the mathematics (coefficients computed as 1/n!), against the C
library's exp: within 1 ulp on 10^6 arguments in [-746, 0] and on the edge
arguments (subnormal results, the underflow threshold, -inf), NaN passes
through.  The GPU kernels' own outputs are checked against the oracle by
tests/test_gpu_verify.py."""
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))


def test_exp_method_within_one_ulp():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "exp_method")
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe,
                        os.path.join(HERE, "exp_method", "exp_method.c"), "-lm"], check=True)
        out = subprocess.run([exe, "1000000"], check=True, capture_output=True,
                             text=True).stdout.split()
    worst, nan_ok = float(out[0]), int(out[1])
    assert worst <= 1.0, worst
    assert nan_ok == 1

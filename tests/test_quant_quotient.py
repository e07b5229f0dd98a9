"""Host check of the FP8 quantiser's division (CPU only).

The quantiser divides each element by its block scale through one reciprocal per thread and
a corrected product (Markstein's correction step) instead of a full IEEE division.  This test
builds a small C program (`tests/native/quotient_check.c`, C99 `fmaf` and IEEE float
division on the host) and checks, over millions of random and midpoint-adjacent cases, that
the E4M3 encoding of the corrected quotient always equals that of the IEEE quotient, which
is what the oracle encodes.
"""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler on this host")
    exe = str(tmp_path_factory.mktemp("quot") / "quotient_check")
    # no contraction: every product and sum rounds exactly as written
    subprocess.run([cc, "-O2", "-std=c99", "-ffp-contract=off", os.path.join(HERE, "native", "quotient_check.c"),
                    "-o", exe, "-lm"], check=True)
    return exe


def test_corrected_quotient_encodes_like_ieee_division(checker):
    out = subprocess.run([checker, "20000000"], check=True, capture_output=True, text=True).stdout.split()
    stats = dict(zip(out[0::2], map(int, out[1::2])))
    assert stats["cases"] > 10_000_000
    assert stats["code_mismatches"] == 0, stats
    # the quotients themselves differ only where the residual underflows (|x| < 2^-102), a
    # handful of cases in this sample
    assert stats["quotient_mismatches"] < stats["cases"] // 100_000, stats

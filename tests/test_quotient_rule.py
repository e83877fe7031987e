"""Host check of the quotient rule inside the FP8 quantizer kernels.

The quantizers of "Helion in vLLM: A Unified Route to Tunable Linear
Kernels" ("What the integration changes", FP8 dynamic quantization and
Block-FP8) divide every value of a group by the group scale s = amax / 448.
The GPU kernels replace the division by the reciprocal of s and one
fma-based correction (Markstein's scheme) when s lies in [2^-64, 2^64].
tests/quot_check.c runs that scheme with IEEE fp32 on the host and compares
it with the correctly rounded division: bitwise equal, or both below 2^-10
(the same signed e4m3 zero).  The full check over every (x, amax) bf16 pair
takes a minute; here every 7th amax is taken (all x for each), which covers
every binade of s.
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
        pytest.skip("no C compiler")
    exe = str(tmp_path_factory.mktemp("quot") / "quot_check")
    subprocess.run([cc, "-O2", "-ffp-contract=off", os.path.join(HERE, "quot_check.c"),
                    "-o", exe, "-lm"], check=True)
    return exe


def test_reciprocal_quotient_matches_division(checker):
    r = subprocess.run([checker, "7"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout
    pairs, exact, bad = (int(v) for v in r.stdout.split()[1::2])
    assert bad == 0 and pairs > 40_000_000
    assert exact > 0.99 * pairs

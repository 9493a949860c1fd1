"""The division-free quotient of the coding kernels (one correction step with the exact residual,
given the correctly rounded reciprocal of the block scale) equals the IEEE fp32 quotient for every
fp16 value inside its block maximum and every fp16 block maximum, for the 8-bit (L = 127) and 4-bit
(L = 7) code ranges: the exhaustive host check of tests/quotient_identity.c."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    exe = str(tmp_path_factory.mktemp("quot") / "quotient_identity")
    subprocess.run([cc, "-O2", "-ffp-contract=off", "-o", exe, os.path.join(HERE, "quotient_identity.c"), "-lm"],
                   check=True)
    return exe


@pytest.mark.parametrize("limit", [127, 7])
def test_quotient_identity_exhaustive(checker, limit):
    r = subprocess.run([checker, str(limit)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "differ=0 codes_out_of_range=0" in r.stdout
    assert "pairs=1007713278" in r.stdout  # every (maximum, value) pair of positive finite fp16 maxima

"""The quantiser computes the scale (mx - mn) / L and the reciprocal 1 / s of the stored fp16 scale with
shorter sequences than an IEEE division (a product and one remainder correction; the hardware reciprocal and
one Newton step). The codes and parameters are bit-exact only if those sequences return the IEEE quotient
for every input: this test checks both identities on the host (tests/quant_arith_check.c). The dividends are
visited with a stride of 61 bit patterns by default; KVQ_EXHAUSTIVE=1 visits all 2^31 (about a minute per
thread)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_fast_division_and_reciprocal_are_exact(tmp_path):
    exe = str(tmp_path / "quant_arith_check")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-o", exe,
                    os.path.join(HERE, "quant_arith_check.c"), "-lm"], check=True)
    stride = "1" if os.environ.get("KVQ_EXHAUSTIVE") == "1" else "61"
    res = subprocess.run([exe, stride], capture_output=True, text=True)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.count(" 0 mismatches") == 4

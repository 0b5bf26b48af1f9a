"""The quantizer's reciprocal-based element quotient equals IEEE division x / D bit for bit
(signed zeros included) wherever the GPU uses it (CPU only; tests/quotient_sweep.c restates the
kernel's arithmetic with C's fmaf and sweeps D = B*T over every E4M3 scale and x next to every
E2M1/E2M3 rounding midpoint). The recipe's element code is Round(x / (B * T)) (onedev.kr
MicroQonv digest, section "How it differs"), read as one fp32 division."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_reciprocal_quotient_equals_division(tmp_path):
    exe = str(tmp_path / "quotient_sweep")
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off",
                           os.path.join(HERE, "quotient_sweep.c"), "-o", exe, "-lm"])
    r = subprocess.run([exe, "400"], capture_output=True, text=True, timeout=300)
    vals = dict(zip(r.stdout.split()[0::2], (int(v) for v in r.stdout.split()[1::2])))
    assert vals["pairs"] > 2 * 10 ** 7
    assert vals["mismatches"] == 0, r.stderr
    # the sweep sees errors: without the correction step, or without the sign of x
    assert vals["q0_mismatches"] > 0 and vals["nosign_mismatches"] > 0
    assert r.returncode == 0

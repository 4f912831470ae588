"""CPU: the fused decode kernel forms its int8 codes without a division: a
fast code fma(x, r, 128) with r = fl32(1/s), and for chunks near a tie the
corrected quotient fma(x - q0 s, r, q0), q0 = fl32(x r).  This is exact only
where it has been shown to be; the C program checks every fp16 value against
every per-token scale fl32(a / 127) of an fp16 a >= |x|."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_fma_quotient_is_the_correctly_rounded_quotient(tmp_path):
    exe = str(tmp_path / "fma_quotient_check")
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                           os.path.join(HERE, "c", "fma_quotient_check.c"), "-o", exe, "-lm"])
    out = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "unflagged-misses 0 " in out.stdout and out.stdout.rstrip().endswith("mismatches 0")
    assert out.stdout.startswith("pairs 1007713278 ")

"""CPU pin of the division the quantize kernels use: reciprocal of the
block scale once, then per element a product and one FMA correction (the
sequence restated in tests/c/div_by_scale_sweep.c, which documents the
claim).  Over 1.25e8 random (x, s) pairs with scales derived from random
amax values or given anywhere in the range the kernels use the shortcut,
plus 8e7 quotients within +-8 ulps of every midpoint between adjacent FP8
values of both formats, the shortcut must give the IEEE quotient bit for bit
whenever that is at least 2^-20, and a value that rounds to the FP8 code 0
otherwise -- so the codes equal those of the division the pages' quant()
performs ("Mixed precision and FP8 training", section "FP8 training").  The
uncorrected product must fail the same sweep, so the check has teeth."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "c", "div_by_scale_sweep.c")


def _build(tmp_path):
    exe = str(tmp_path / "div_by_scale_sweep")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-Wall",
                    "-Wextra", "-Werror", "-o", exe, SRC, "-lm"], check=True)
    return exe


def _run(exe, *args):
    r = subprocess.run([exe, *args], capture_output=True, text=True, timeout=300)
    counts = dict(line.split()[:2] for line in r.stdout.splitlines()
                  if line.startswith(("pairs", "mismatches")))
    return r.returncode, int(counts["pairs"]), int(counts["mismatches"]), r.stdout


def test_reciprocal_fma_division_gives_the_ieee_quotient(tmp_path):
    exe = _build(tmp_path)
    rc, pairs, bad, out = _run(exe, "50000000")
    assert rc == 0 and bad == 0, out
    assert pairs >= 2e8, out
    for line in out.splitlines()[:8]:
        assert line.endswith(" 0 mismatches"), out


def test_uncorrected_product_fails_the_sweep(tmp_path):
    exe = _build(tmp_path)
    rc, pairs, bad, out = _run(exe, "200000", "--uncorrected")
    assert rc == 0 and bad > 0.01 * pairs, out

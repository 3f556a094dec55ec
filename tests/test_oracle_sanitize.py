"""The CPU oracle (oracle/nvfp4_oracle.c) built with AddressSanitizer and
UndefinedBehaviorSanitizer (gcc, host code only; no GPU code is involved) and
run through every C entry point on inputs that reach its edge cases: empty
products, an empty expert, bad arguments and offsets, subnormal and signed
zero weights, a non-finite weight.  Any out-of-bounds access, leak or
undefined operation aborts the run."""
import os
import subprocess
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_under_address_and_ub_sanitizers():
    tmp = tempfile.mkdtemp(prefix="oracle_san_")
    exe = os.path.join(tmp, "driver")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "tests", "oracle_sanitize", "driver.c"),
           os.path.join(ROOT, "oracle", "nvfp4_oracle.c"), "-o", exe, "-lm"]
    subprocess.run(cmd, check=True)
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "oracle driver ok" in res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr

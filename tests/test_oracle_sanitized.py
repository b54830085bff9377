"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

oracle/sanitize_main.c drives every entry point of oracle/nf4_oracle.c on small
inputs (edge shapes, refusal paths); built with gcc -fsanitize=address,undefined
and run as a child process, any out-of-bounds access, leak or undefined
arithmetic in the oracle ends it with a report and a non-zero status.  Host code
only: nothing here touches a GPU."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_clean_under_address_and_undefined_sanitizers():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "oracle_sanitized")
        cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=all", "-ffp-contract=off", "-fno-fast-math", "-Wno-unknown-pragmas",
               "-o", exe, os.path.join(ORACLE, "nf4_oracle.c"), os.path.join(ORACLE, "sanitize_main.c"), "-lm"]
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
        assert res.returncode == 0, res.stdout + res.stderr
        assert "oracle sanitizer run: ok" in res.stdout
        assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr

"""The oracle under the host's address and undefined-behaviour sanitizers (CPU only): oracle/asan_driver.c calls
every routine of oracle/mxq_oracle.c on small seeded inputs in buffers of exactly their documented sizes (ragged
shapes, empty tensors, empty expert groups, several threads); any out-of-bounds access, use after free, leak or
undefined operation fails the run. Values are checked by the pinned oracle tests, not here."""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

ORACLE = os.path.join(ROOT, "oracle")


def test_oracle_is_clean_under_address_and_ub_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no host gcc")
    exe = str(tmp_path / "oracle_asan")
    cmd = [gcc, "-O1", "-g", "-std=c11", "-D_GNU_SOURCE", "-ffp-contract=off", "-fexcess-precision=standard",
           "-pthread", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-o", exe, os.path.join(ORACLE, "mxq_oracle.c"), os.path.join(ORACLE, "asan_driver.c"), "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0 and "asan driver: ok" in run.stdout, run.stderr[-4000:]

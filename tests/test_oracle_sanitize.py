"""The oracle under AddressSanitizer, LeakSanitizer and UndefinedBehaviorSanitizer (CPU).

oracle_sanitize_main.c runs every oracle function on 80 small seeded random layers; it
is compiled with gcc and the sanitizers into a standalone program (the oracle's C source
included directly) and must exit cleanly. Planted memory errors in copies of the oracle
must be caught, so the check is known to bite."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "oracle_sanitize_main.c")
ORACLE_C = os.path.join(os.path.dirname(HERE), "oracle", "moe_oracle.c")
FLAGS = ["-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer"]
ENV = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")


def _build_and_run(tmp_path, oracle_source):
    driver = os.path.join(tmp_path, "driver.c")
    with open(DRIVER) as f:
        src = f.read()
    src = src.replace('#include "../oracle/moe_oracle.c"', f'#include "{oracle_source}"')
    with open(driver, "w") as f:
        f.write(src)
    exe = os.path.join(tmp_path, "driver")
    subprocess.run(["gcc", *FLAGS, driver, "-o", exe, "-lm"], check=True, capture_output=True, text=True)
    return subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=600)


def test_oracle_clean_under_sanitizers(tmp_path):
    r = _build_and_run(tmp_path, ORACLE_C)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stderr[-3000:]


@pytest.mark.parametrize("name,old,new", [
    # combine writes one element past each output row
    ("combine_row_overrun", "for (int64_t d = 0; d < D; ++d) y[t * D + d] = 0.0;",
     "for (int64_t d = 0; d <= D; ++d) y[t * D + d] = 0.0;"),
    # the expert FFN's hidden vector allocated one element short
    ("hidden_short_alloc", "double* h = (double*)malloc(sizeof(double) * (size_t)F);",
     "double* h = (double*)malloc(sizeof(double) * (size_t)(F - 1));"),
])
def test_planted_memory_error_is_caught(tmp_path, name, old, new):
    with open(ORACLE_C) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site of {name} not found exactly once"
    mutant = os.path.join(tmp_path, "moe_oracle_mut.c")
    with open(mutant, "w") as f:
        f.write(src.replace(old, new))
    r = _build_and_run(tmp_path, mutant)
    assert r.returncode != 0 and "Sanitizer" in r.stderr, f"{name} not caught"

"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/oracle_sanitize_main.c drives every oracle function over seeded shapes
(every pad mode, bad ids, empty batches, the balanced layout) with buffers of
exactly the documented sizes; built with -fsanitize=address,undefined (the C
driver with gcc, the C++ oracle with g++), an out-of-bounds access, a leak or
undefined arithmetic stops it.  A second run
plants an off-by-one in a copy of the oracle to show the harness catches one.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
MAIN_SRC = os.path.join(HERE, "oracle_sanitize_main.c")
ORACLE = os.path.join(ROOT, "oracle", "moe_oracle.cpp")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="gcc / g++ not found")

FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")


def _build_and_run(oracle_src, exe):
    main_o, oracle_o = str(exe) + "_main.o", str(exe) + "_oracle.o"
    for cmd in (["gcc", "-std=c11", *FLAGS, "-c", MAIN_SRC, "-o", main_o],
                ["g++", "-std=c++17", *FLAGS, "-c", oracle_src, "-o", oracle_o],
                ["g++", *FLAGS, main_o, oracle_o, "-lm", "-o", str(exe)]):
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
    return subprocess.run([str(exe)], capture_output=True, text=True, env=ENV, timeout=300)


def test_oracle_clean_under_sanitizers(tmp_path):
    r = _build_and_run(ORACLE, tmp_path / "oracle_sanitize")
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all cases passed" in r.stdout


def test_sanitizer_catches_planted_overrun(tmp_path):
    src = open(ORACLE).read()
    good = "for (int64_t b = 0; b < row_bytes; ++b) recv[r * row_bytes + b] = 0;"
    assert src.count(good) == 1
    planted = tmp_path / "moe_oracle_planted.cpp"
    planted.write_text(src.replace(good, "for (int64_t b = 0; b <= row_bytes; ++b) recv[r * row_bytes + b] = 0;"))
    r = _build_and_run(str(planted), tmp_path / "oracle_planted")
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr

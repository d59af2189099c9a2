"""The public header is plain C: a C11 program (tests/c/abi_check.c) compiles against
include/kvtc.h with every warning an error, links libkvtc.so and gets the sizes,
plan and validation errors the header documents (no GPU: no call reaches a launch)."""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

LIB_DIR = os.path.join(ROOT, "decode_attention_04_amd")


@pytest.fixture(scope="module")
def run_check(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    if not os.path.exists(os.path.join(LIB_DIR, "libkvtc.so")):
        pytest.skip("libkvtc.so is not built")
    exe = str(tmp_path_factory.mktemp("c") / "abi_check")
    cmd = [gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_check.c"), "-L", LIB_DIR, "-lkvtc", f"-Wl,-rpath,{LIB_DIR}",
           "-o", exe]
    p = subprocess.run(cmd, capture_output=True, text=True)
    assert p.returncode == 0, p.stderr
    p = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert p.returncode == 0, p.stderr
    return dict(line.split(" ", 1) for line in p.stdout.strip().splitlines())


def test_record_words_from_c(run_check):
    assert run_check["record_words"].split() == ["9", "4", "0"]  # (64,4), (16,6), unsupported rank 48


def test_cache_bytes_from_c(run_check):
    # 3 sequences x 1000 records x (9 + 9 words): K heads (64,4) and (32,8), V heads (128,2) and (64,4)
    assert run_check["cache_bytes"].split() == ["0", "216000", "0", "216000"]


def test_plan_from_c(run_check):
    # both heads' formats are in the 256-bit budget class; 1000 tokens take one split per unit
    assert run_check["plan"].split() == ["0", "2", "1", "6"]


def test_validation_errors_from_c(run_check):
    assert run_check["attend_null"].split() == ["1", "1"]  # KV_ERR_INVALID with a message
    assert run_check["head_dim_64"].split() == ["2"]       # KV_ERR_UNSUPPORTED

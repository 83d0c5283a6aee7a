"""The oracle (oracle/dwref.c) built with gcc's AddressSanitizer and
UndefinedBehaviorSanitizer and driven over random small shapes by
tests/oracle_sanitize_driver.c: no access outside the buffers a shape needs,
no undefined behaviour, and the selected-output entry points agree with the
full passes.  Host only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_sanitize"
    cmd = ["gcc", "-O1", "-g", "-std=c99", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "dwref.c"),
           os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"), "-lm", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr + r.stdout).lower():
        pytest.skip("the sanitizer runtimes are not installed: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr
    # verify_asan_link_order=0: the run may start with other libraries
    # already preloaded into every process
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe), "400"], capture_output=True, text=True, env=env,
                         timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "oracle sanitizer driver" in run.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_sanitizers_catch_a_planted_overflow(tmp_path):
    """The same build stops on a copy of the oracle with one write moved one
    element past its buffer (the filter gradient's accumulation), so the run
    above would have caught such a mistake."""
    src = open(os.path.join(ROOT, "oracle", "dwref.c")).read()
    old = "dw[o + c] += prod;"
    assert src.count(old) == 1
    bad = tmp_path / "dwref_bad.c"
    bad.write_text(src.replace(old, "dw[o + c + 1] += prod;"))
    exe = tmp_path / "oracle_bad"
    r = subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=all", str(bad),
                        os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"), "-lm", "-o",
                        str(exe)], capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr + r.stdout).lower():
        pytest.skip("the sanitizer runtimes are not installed")
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="verify_asan_link_order=0")
    run = subprocess.run([str(exe), "100"], capture_output=True, text=True, env=env,
                         timeout=120)
    assert run.returncode != 0 and "AddressSanitizer" in run.stderr

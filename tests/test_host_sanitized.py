"""CPU builds with AddressSanitizer and UndefinedBehaviorSanitizer.

* The library's host placement logic (decode_attention_tkv_amd/csrc/plan.cpp,
  which holds no HIP code) with its unit test tests/cpp/test_plan.cpp:
  random reassignments simulated move by move, and the first placement and
  tier counts of a grid of cases compared with the oracle's tiering
  ("Not All Thoughts Need HBM", gist.science summary, Method §1 and §4).
* The oracle's C attention (oracle/attend.c) with a driver on random small
  inputs (weights sum to 1 over the live rows).
Both are built with g++/gcc for the host only.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import tiering

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                                reason="needs the host compilers")


@pytest.fixture(scope="module")
def plan_bin(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("plan") / "test_plan")
    subprocess.check_call(["g++", "-std=c++17", *SAN, "-o", out,
                           os.path.join(ROOT, "tests", "cpp", "test_plan.cpp"),
                           os.path.join(ROOT, "decode_attention_tkv_amd", "csrc", "plan.cpp")])
    return out


def test_plan_simulated_reassignments(plan_bin):
    r = subprocess.run([plan_bin], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "plan checks: 0 failures" in r.stdout


def test_plan_tier_rules_match_oracle(plan_bin):
    r = subprocess.run([plan_bin, "cases"], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stderr
    firsts = cuts = 0
    for line in r.stdout.splitlines():
        head, _, tail = line.partition(":")
        f = head.split()
        if f[0] == "first":
            n, prompt, sinks, recent, h, no_t1 = int(f[1]), int(f[2]), int(f[3]), int(f[4]), float(f[5]), int(f[6])
            got = np.array([int(x) for x in tail.split()], np.uint8)
            ref = tiering.initial_placement(n, prompt, sinks, recent, h, bool(no_t1))
            assert np.array_equal(got, ref), line
            firsts += 1
        elif f[0] == "cut":
            n, np_, nev = int(f[1]), int(f[2]), int(f[3])
            h, e, t2, no_t1 = float(f[4]), float(f[5]), float(f[6]), int(f[7])
            got = tuple(int(x) for x in tail.split())
            assert got == tiering.tier_counts(n, np_, n - np_ - nev, nev, h, e, t2, bool(no_t1)), line
            cuts += 1
    assert firsts > 100 and cuts > 500


def test_oracle_attend_sanitized(tmp_path):
    out = str(tmp_path / "attend")
    subprocess.check_call(["gcc", "-std=c11", *SAN, "-o", out, os.path.join(ROOT, "tests", "cpp", "attend_driver.c"),
                           os.path.join(ROOT, "oracle", "attend.c"), "-lm"])
    r = subprocess.run([out], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "attend checks: 0 failures" in r.stdout

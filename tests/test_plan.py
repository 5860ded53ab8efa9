"""The host launch planner (csrc/plan.h), built with g++ into a small program and checked
without a GPU: every split plan covers the key range with no empty split, respects the unit
and the length cap, offers about the target number of workgroups without splits shorter than
eight rounds, and leaves short verify contexts unsplit."""

import itertools
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_sparse_speculative_amd", "csrc")

KVSS_F32, KVSS_BF16 = 0, 1
TARGET, UNIT_MFMA, UNIT_SIMPLE, UNSPLIT_BELOW = 1024, 128, 32, 16384


def _cdiv(a, b):
    return -(-a // b)


@pytest.fixture(scope="module")
def planner(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = tmp_path_factory.mktemp("plan") / "plan_check"
    cmd = ["g++", "-std=c++17", "-O1", "-Wall", "-Werror", "-I" + os.path.join(ROOT, "include"),
           "-I" + CSRC, os.path.join(ROOT, "tests", "c", "plan_check.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr

    def run(queries):
        text = "".join(" ".join(str(x) for x in q) + "\n" for q in queries)
        out = subprocess.run([str(exe)], input=text, capture_output=True, text=True, timeout=60)
        assert out.returncode == 0, out.stderr
        return [tuple(int(x) for x in line.split()) for line in out.stdout.splitlines()]
    return run


def test_split_plans_cover_the_range(planner):
    grid = list(itertools.product([1, 7, 64, 512, 1024, 5000],              # pairs
                                  [1, 100, 127, 128, 1025, 8192, 32005, 100005, 10**7],
                                  [UNIT_SIMPLE, UNIT_MFMA],
                                  [1 << 30, 4096 * 16],                    # length cap
                                  [TARGET, 512, 3072],
                                  [0, UNSPLIT_BELOW]))
    plans = planner([("split",) + q for q in grid])
    assert len(plans) == len(grid)
    for (pairs, total, unit, max_len, target, unsplit), (ns, ln) in zip(grid, plans):
        where = (pairs, total, unit, max_len, target, unsplit, ns, ln)
        assert ns >= 1 and ln >= unit and ln % unit == 0, where
        assert ln <= max_len, where
        assert ns * ln >= total and (ns - 1) * ln < total, where          # no empty split
        forced = _cdiv(total, max_len)                                       # splits the cap needs
        if ns > forced:
            # splitting beyond the cap only while the launch is short of its target and every
            # split still does at least eight rounds of `unit` keys
            assert ns <= _cdiv(target, pairs), where
            assert ns <= _cdiv(total, 8 * unit), where
            assert total >= unsplit, where
        if total < unsplit and forced <= 1:
            assert ns == 1, where


def test_empty_ranges_and_batches_plan_one_split(planner):
    plans = planner([("split", 0, 1000, UNIT_MFMA, 1 << 30, TARGET, 0),
                     ("split", 64, 0, UNIT_MFMA, 1 << 30, TARGET, 0),
                     ("split", 64, -5, UNIT_MFMA, 1 << 30, TARGET, 0)])
    assert plans == [(1, UNIT_MFMA)] * 3


def test_verify_plans_of_the_measured_shapes(planner):
    # (dtype, batch, Hkv, max_kv_len) -> expected (nsplit, split_len)
    cases = {
        (KVSS_BF16, 64, 8, 32005): (2, 16128),     # Llama-3.1-8B layer, 32k context, gamma 4
        (KVSS_BF16, 16, 8, 100005): (8, 12544),    # 100k context, batch 16
        (KVSS_BF16, 32, 8, 8196): (1, 8320),       # 8k context: below 16k keys, unsplit
        (KVSS_BF16, 1, 8, 20005): (20, 1024),      # one sequence: split until 8 rounds a split
    }
    plans = planner([("verify",) + k for k in cases])
    for (key, want), got in zip(cases.items(), plans):
        assert got == want, (key, got)
    # fp32 caches use the 32-key unit and no unsplit threshold
    (ns, ln), = planner([("verify", KVSS_F32, 2, 2, 515)])
    assert ln % UNIT_SIMPLE == 0 and ns * ln >= 515 and ns > 1

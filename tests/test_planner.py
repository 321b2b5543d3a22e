"""The host planner (csrc/planner.cpp) under AddressSanitizer and
UndefinedBehaviorSanitizer, CPU only.

tests/planner/check_plans.cpp replays the plans of the five workloads' shapes
and of ragged and edge shapes against a model of their launches (coverage
exactly once, dependency order, error-buffer halves, races between the two
streams).  The planted-mistake cases recompile the planner with one plausible
slip each and require the checker to reject it.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "post_weight_quantization_gptq_amd", "csrc")
CHECKER = os.path.join(ROOT, "tests", "planner", "check_plans.cpp")
GXX = shutil.which("g++")
FLAGS = ["-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-Wall", "-Wextra", "-Werror"]

pytestmark = pytest.mark.skipif(GXX is None, reason="g++ not found")


def _compile(src, obj):
    b = subprocess.run([GXX] + FLAGS + ["-I", CSRC, "-c", src, "-o", obj], capture_output=True, text=True)
    assert b.returncode == 0, b.stdout + b.stderr


@pytest.fixture(scope="module")
def checker_obj(tmp_path_factory):
    obj = str(tmp_path_factory.mktemp("planner") / "check_plans.o")
    _compile(CHECKER, obj)
    return obj


def _build_and_run(tmp_path, checker_obj, planner_src):
    obj, exe = str(tmp_path / "planner.o"), str(tmp_path / "check_plans")
    _compile(planner_src, obj)
    b = subprocess.run([GXX] + FLAGS + [obj, checker_obj, "-o", exe], capture_output=True, text=True)
    assert b.returncode == 0, b.stdout + b.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    return subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)


def test_plans_pass_the_checker_under_sanitizers(tmp_path, checker_obj):
    r = _build_and_run(tmp_path, checker_obj, os.path.join(CSRC, "planner.cpp"))
    assert r.returncode == 0, r.stdout + r.stderr
    assert "planner checks passed" in r.stdout


# (name, text in planner.cpp, replacement, phrases ("a|b") one of which the checker must print)
MISTAKES = [
    ("factor-missing-join",
     "      if (side_busy) add_sync(PL_JOIN);  // the previous bulk update touches the columns updated now\n",
     "", "pending side launch"),
    ("factor-half-pair-update",
     "inner.push_back(Seg{p, 0, ncol * nrow - ncol * (ncol - 1) / 2, GK_CHOL_TRAIL, k0, pw, c0, P1});",
     "inner.push_back(Seg{p, 0, ncol * nrow - ncol * (ncol - 1) / 2, GK_CHOL_TRAIL, k0, 64, c0, P1});",
     "applied 0 times"),
    ("factor-y-rows-short",
     "crit.push_back(Seg{p, 0, cdiv(S - P1, 64) * cdiv(P1, 64), GK_ZUPD, P0, P1 - P0, P1, S});",
     "crit.push_back(Seg{p, 0, cdiv(S - P1 - 64, 64) * cdiv(P1, 64), GK_ZUPD, P0, P1 - P0, P1, S - 64});",
     "Y("),
    ("quantize-wrong-error-half",
     "const int par = ((k / sb) & 1) * jobs[p].out * sbw;",
     "const int par = (k & 1) * jobs[p].out * sbw;",
     "reads half"),
    ("quantize-missing-join",
     "      if (side_busy) add_sync(PL_JOIN);  // the previous far update covers the columns updated now\n",
     "", "pending side launch"),
    ("quantize-bulk-on-main-before-crit",
     "        add_launch(QK_TRAIL, 128, bulk, true);",
     "        add_launch(QK_TRAIL, 128, bulk, true);\n        add_launch(QK_TRAIL, 128, bulk, true);",
     "after [0,"),
    ("factor-diag-launch-dropped",
     "      add_launch(FK_DIAG2, dg);\n", "", "reads the diagonal chain"),
    ("hessian-slice-gap",
     "const int k0 = (int)(32 * (c32 * sl / S)), k1 = (int)(32 * (c32 * (sl + 1) / S));",
     "const int k0 = (int)(32 * (c32 * sl / S)), k1 = (int)(32 * (c32 * (sl + 1) / S)) - (sl + 1 < S ? 32 : 0);",
     "task range|gap"),
    ("hessian-diagonal-blocks-dropped",
     "            if (ti == tj && a > b && !full) continue;",
     "            if (ti == tj && a >= b && !full) continue;",
     "reduced 0 times"),
]


@pytest.mark.parametrize("name,old,new,phrase", MISTAKES, ids=[m[0] for m in MISTAKES])
def test_checker_rejects_a_planted_mistake(tmp_path, checker_obj, name, old, new, phrase):
    src = open(os.path.join(CSRC, "planner.cpp")).read()
    assert src.count(old) == 1, "the planted text must appear once: %r" % old
    mutant = str(tmp_path / "planner_mutant.cpp")
    with open(mutant, "w") as f:
        f.write(src.replace(old, new))
    r = _build_and_run(tmp_path, checker_obj, mutant)
    assert r.returncode != 0, "the checker accepted the mistake %s" % name
    assert any(ph in r.stderr for ph in phrase.split("|")), r.stderr[-2000:]

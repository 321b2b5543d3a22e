"""The pair order of the Rayleigh-Ritz step's one-sided Jacobi sweeps
(csrc/jacobi_order.h, read by k_ritz), checked on the host for every even
width up to 128 by tests/jacobi/check_order.cpp under AddressSanitizer and
UndefinedBehaviorSanitizer.  Planted mistakes in the order must be rejected.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "post_weight_quantization_gptq_amd", "csrc")
CHECKER = os.path.join(ROOT, "tests", "jacobi", "check_order.cpp")
GXX = shutil.which("g++")
FLAGS = ["-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-Wall", "-Wextra", "-Werror"]

pytestmark = pytest.mark.skipif(GXX is None, reason="g++ not found")


def _run(tmp_path, header_dir):
    exe = str(tmp_path / "check_order")
    b = subprocess.run([GXX] + FLAGS + ["-I", header_dir, CHECKER, "-o", exe], capture_output=True, text=True)
    assert b.returncode == 0, b.stdout + b.stderr
    return subprocess.run([exe], capture_output=True, text=True, timeout=120)


def test_order_passes_the_checker(tmp_path):
    r = _run(tmp_path, CSRC)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "jacobi order checks passed" in r.stdout


# (name, text in jacobi_order.h, replacement, phrase the checker must print)
MISTAKES = [
    ("cross-shift-by-two", "b = G * g + q + (v + ri) % q;", "b = G * g + q + (v + 2 * ri) % q;",
     "not held in round 0|met 0 times|met 2 times"),
    ("circle-pairs-wrong-places", "b = base + 1 + (q - j - 1 + ri) % q;", "b = base + 1 + (q - j + ri) % q;",
     "met"),
    ("levels-stop-early", "    if (q & 1) return q > 1 ? R + q : R;", "    if (q & 1) return R;",
     "rounds|met 0 times"),
]


@pytest.mark.parametrize("name,old,new,phrase", MISTAKES, ids=[m[0] for m in MISTAKES])
def test_checker_rejects_a_planted_mistake(tmp_path, name, old, new, phrase):
    src = open(os.path.join(CSRC, "jacobi_order.h")).read()
    assert src.count(old) == 1, "the planted text must appear once: %r" % old
    d = tmp_path / "hdr"
    d.mkdir()
    (d / "jacobi_order.h").write_text(src.replace(old, new))
    r = _run(tmp_path, str(d))
    assert r.returncode != 0, "the checker accepted the mistake %s" % name
    assert any(ph in r.stderr for ph in phrase.split("|")), r.stderr[-2000:]

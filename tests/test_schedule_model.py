"""CPU model of the GEMMs' tile order and the one-launch GEMM1 -> GEMM2 tile list.

tests/sched_model.cpp is compiled for the host against the kernels' own
scheduling header (mixture_experts_layer_topk_amd/csrc/sched.h) and checks, on
the DeepSeek-V3-like, skewed and 256-expert tile counts and 3000 random cases,
that every tile is listed exactly once, that every GEMM2 tile of an m-tile comes
after all GEMM1 tiles of that m-tile ("MegaMoE" study notes, "Scheduler" and
"Wave"), and that a resident grid whose GEMM2 tiles wait on ready counters
always finishes.  Planted mistakes in a copy of the header must make it fail.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_layer_topk_amd", "csrc")
MODEL = os.path.join(ROOT, "tests", "sched_model.cpp")


def _run(include_dir, tmp_path, name="model"):
    exe = os.path.join(str(tmp_path), name)
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", include_dir, MODEL, "-o", exe], check=True)
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    return r.returncode, r.stdout


def test_schedule_model_passes(tmp_path):
    rc, out = _run(CSRC, tmp_path)
    print(out)
    assert rc == 0, out
    assert re.search(r"^\d+ cases, 0 failures$", out.strip().splitlines()[-1])


# (original, planted) pairs: GEMM2 of a wave listed one wave early; the last
# GEMM2 segment taken one segment early; n-tiles numbered across a short group;
# the XCD slot mapping no longer a bijection
MUTATIONS = [
    ("w = s / 2 - 1;", "w = s / 2;"),
    ("if (s == 2 * nw - 1) {", "if (s == 2 * nw - 2) {"),
    ("*ntile = in_grp / gm;", "*ntile = in_grp / kGM;"),
    ("(b % kXCDs) * (grid / kXCDs) + b / kXCDs", "(b % kXCDs) * (grid / kXCDs)"),
]


@pytest.mark.parametrize("orig,planted", MUTATIONS)
def test_schedule_model_catches_planted_mistake(tmp_path, orig, planted):
    src = open(os.path.join(CSRC, "sched.h")).read()
    assert orig in src
    d = tmp_path / "inc"
    d.mkdir()
    (d / "sched.h").write_text(src.replace(orig, planted))
    rc, out = _run(str(d), tmp_path, "mutant")
    assert rc != 0, f"planted mistake {planted!r} went unnoticed:\n{out}"

"""The accumulation accuracy of the matrix instructions, measured: the parity
bounds on h (tests/gpu_common.py make_hq_bound, tests/test_gpu_blockfp8.py) take
each instruction's error as at most a fixed fraction of sum_k |a_k b_k| over its
128 products.  tests/probes/mfma_precision (built with the library) multiplies 1000
random E4M3 / E2M1 tiles and reports the largest error against exact sums."""
import os
import re
import subprocess
import sys

import pytest

from tests import gpu_common as G

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes", "mfma_precision")


def test_matrix_instruction_accuracy_is_within_the_bounds_used():
    assert os.path.exists(PROBE), "build the library first (it builds the probe too)"
    print("matrix instruction accuracy probe", flush=True)
    r = subprocess.run([PROBE], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout
    got = {m.group(1): float(m.group(2)) for m in re.finditer(r"^(\w+) max_err_over_sum_abs (\S+)", r.stdout, re.M)}
    assert set(got) == {"fp8xfp4", "fp8xfp8", "bf16"}
    # the FP8 x FP4 scaled instruction of the main path does not sum in FP32 ...
    assert got["fp8xfp4"] <= G.MFMA_FP8_FP4_REL
    # ... neither does FP8 x FP8 (reported; the block-FP8 path does not use it) ...
    print(f"fp8 x fp8: {got['fp8xfp8']:.3e} of sum|ab|", flush=True)
    # ... while BF16 (the block-FP8 path, values widened exactly) is FP32-accurate
    assert got["bf16"] <= G.MFMA_BF16_REL

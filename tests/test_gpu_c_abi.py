"""The C ABI on its own: tests/c_abi/c_abi_example.c (plain C99, linked
against libmoe_route.so and the oracle's library, no Python or torch) runs
route + dispatch in one call and combine with identity experts on a seeded
batch; the group-limited router, the separate dispatch with E4M3 rows and
the packed dispatch on a second batch; and the plain router, the one-call
packed and no-alloc dispatches and the fused residual + RMSNorm epilogue
(bf16 and E4M3 output) on a third.  Every entry point of the library runs.
It checks ids, weights, counts, slots, offsets, sources, codes, scales,
rows, the updated residual and the normalised rows against the oracle.  It
runs as a child process of the test."""
import os
import subprocess

import pytest

from gpu_common import require_gpu, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_abi", "c_abi_example")


def test_plain_c_program_matches_the_oracle():
    require_gpu()
    if not os.path.exists(EXE):
        raise RuntimeError(f"{EXE} is missing: run __graft_entry__.build() first")
    say("[c-abi] running the plain-C program")
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and "c-abi ok" in res.stdout, res.stdout + res.stderr

"""The benchmark's algorithmic byte model (every GB/s and roofline figure is
derived from it), pinned to totals worked out by hand for the five
workloads: route 4E + 8k, count/scan/slot 12k, pack 2H + 4k + k*row (row =
2H bf16, H + H/32 fp8), combine 2kH + 8k + 2H bytes per token (+ 4E per
call for the counts).  The hand figures are in decimal units, rounded to
the digits given."""
import pytest

import bench
import workloads as W

# workload -> (total, combine) in bytes
TABLE = {
    "tiny": (0.203e6, None),
    "mixtral_prefill": (201.7e6, 100.7e6),
    "dsr1_decode": (26.1e6, 16.5e6),
    "dsr1_prefill": (4.249e9, 2.115e9),
    "glm_prefill": (5.713e9, 3.626e9),
}


@pytest.mark.parametrize("name", W.ORDER)
def test_totals_match_the_table(name):
    b = bench.algorithmic_bytes(W.WORKLOADS[name])
    total, combine = TABLE[name]
    assert b["total"] == pytest.approx(total, rel=2e-3)
    if combine is not None:
        assert b["combine"] == pytest.approx(combine, rel=2e-3)
    assert b["total"] == b["route"] + b["count_scan_slot"] + b["pack"] + b["combine"]


def test_epilogue_terms():
    w = W.WORKLOADS["mixtral_prefill"]
    T, H = w.T, w.H
    plain = bench.algorithmic_bytes(w)["combine"]
    # residual read + residual written + gamma
    assert bench.algorithmic_bytes(w, "rmsnorm")["combine"] - plain == 4 * T * H + 2 * H
    # the normalised rows as E4M3 codes + one fp32 scale per 128 instead of bf16
    assert bench.algorithmic_bytes(w, "rmsnorm-fp8")["combine"] - plain == 4 * T * H + 2 * H - T * H + T * H // 32

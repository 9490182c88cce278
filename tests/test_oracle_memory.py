"""Pins for the oracle's model-state memory formula against the figures the
pages print (tests/golden/memory_figures.json): the 1.5B and 1T examples and
the stage reduction ratios on the ZeRO paper card ("Bottleneck", "Method",
"Evidence") and the ZeRO-2 article (model state memory)."""
import json
import os

import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "memory_figures.json")


def _entries():
    with open(GOLDEN) as f:
        return json.load(f)["entries"]


def test_page_byte_figures(oracle):
    for e in _entries():
        if "bytes" not in e or "stage" not in e:
            continue
        got = oracle.state_bytes(e["psi"], e["nd"], e["k"], e["stage"])
        if e["relation"] == ">=":
            assert got >= e["bytes"], e["what"]
            assert got == e["bytes"], "16 B/param makes the page's lower bound exact"
        else:
            assert abs(got - e["bytes"]) <= e["tolerance_rel"] * e["bytes"], (e["what"], got)
        if "budget_bytes" in e:
            assert got < e["budget_bytes"]


def test_fp16_weights_stay_replicated_under_stage2(oracle):
    # Stage 2 partitions optimizer state and gradients but keeps the fp16
    # parameters on every rank: with one parameter per rank the per-rank
    # bytes are the fp16 weights (2 B/param, "about 3 GB" for 1.5B) plus the
    # owned parameter's 2 + K bytes.
    e = next(x for x in _entries() if x.get("bytes_per_param") == 2)
    psi = e["psi"]
    got = oracle.state_bytes(psi, psi, 12, 2) - (2 + 12)
    assert got == 2 * psi
    assert abs(got - e["bytes"]) <= e["tolerance_rel"] * e["bytes"]


@pytest.mark.parametrize("stage,limit", [(1, 4.0), (2, 8.0)])
def test_stage_reduction_limits(oracle, stage, limit):
    psi = 10 ** 12
    base = oracle.state_bytes(psi, 1, 12, 0)
    ratios = [base / oracle.state_bytes(psi, nd, 12, stage) for nd in (16, 1024, 10 ** 6)]
    assert ratios[0] < ratios[1] < ratios[2] < limit       # grows toward the limit
    assert abs(ratios[-1] - limit) < 1e-4 * limit


def test_stage3_proportional_to_nd(oracle):
    psi = 2 ** 40
    base = oracle.state_bytes(psi, 1, 12, 0)
    for nd in (2, 64, 1024, 4096):
        assert base == nd * oracle.state_bytes(psi, nd, 12, 3)


def test_stage_ordering_and_nd1_identity(oracle):
    psi = 1_557_611_200
    vals = [oracle.state_bytes(psi, 1, 12, s) for s in range(4)]
    assert len(set(vals)) == 1                              # Nd = 1: nothing to partition
    vals = [oracle.state_bytes(psi, 16, 12, s) for s in range(4)]
    assert vals[0] > vals[1] > vals[2] > vals[3]


def test_ceil_partition(oracle):
    # A rank owns ceil(psi/Nd) parameters: 7 params over 2 ranks -> 4 each.
    assert oracle.state_bytes(7, 2, 12, 3) == 16 * 4
    assert oracle.state_bytes(7, 2, 12, 1) == 4 * 7 + 12 * 4


def test_rejects_bad_arguments(oracle):
    with pytest.raises(ValueError):
        oracle.state_bytes(10, 0, 12, 3)
    with pytest.raises(ValueError):
        oracle.state_bytes(10, 1, 12, 4)
    with pytest.raises(ValueError):
        oracle.state_bytes(2 ** 63, 1, 12, 0)              # 16 * 2^63 overflows 64 bits

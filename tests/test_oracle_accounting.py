"""Pins for the 16-bytes-per-parameter accounting against figures the pages print.

Every expected value lives in tests/golden/accounting_pages.jsonl with the page and passage it
comes from; GB there means 10^9 bytes, as the pages use it.
"""

import json
import os
from fractions import Fraction

import pytest

from oracle import accounting as acc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "accounting_pages.jsonl")
SCHEMES = {"mixed": acc.MIXED, "fp32": acc.FP32}
UNIT = {"B": 1, "GB": 10 ** 9, "GPUs": 1}


def _rows():
    with open(GOLDEN) as f:
        return [json.loads(line) for line in f if line.strip()]


def _evaluate(q, a):
    s = SCHEMES[a["scheme"]]
    P = int(a["P"]) if "P" in a else None
    if q == "bytes_per_param":
        return acc.bytes_per_param(s)
    if q == "model_state":
        return acc.model_state_bytes(P, s)
    if q == "gpus_needed":
        return Fraction(acc.model_state_bytes(P, s), a["gpu_GB"] * 10 ** 9)
    if q == "component":
        return P * s[a["part"]]
    if q == "component_per_rank":
        return Fraction(P * s[a["part"]], a["N"])
    if q == "full_shard_per_rank":
        return acc.full_shard_per_rank(P, a["N"], s)
    if q == "unit_buffer":
        return Fraction(P * s["param"], a["M"])
    if q == "full_shard_peak":
        return acc.full_shard_peak(P, a["N"], a["M"], s)
    if q == "shard_grad_op_saving_per_param":
        return acc.shard_grad_op_saving(1, a["N"], s)
    if q == "full_shard_saving_per_param":
        return acc.full_shard_saving(1, a["N"], s)
    if q == "adam_state":
        return acc.adam_state_bytes(P, s)
    if q == "adam_state_per_rank":
        return Fraction(acc.adam_state_bytes(P, s), a["N"])
    raise KeyError(q)


@pytest.mark.parametrize("row", _rows(), ids=lambda r: r["quantity"] + ":" + r["source"][-40:])
def test_page_figure(row):
    got = Fraction(_evaluate(row["quantity"], row["args"])) / UNIT[row["unit"]]
    want = Fraction(str(row["expected"]))
    tol = Fraction(str(row["rel_tol"])) * abs(want)
    assert abs(got - want) <= tol, (row["source"], float(got))


def test_golden_has_citations():
    for r in _rows():
        assert " -- " in r["source"]


def test_shard_bytes_split():
    # 2 + 2 + 4 + 8 bytes per element of a shard; Adam state alone (master + m + v) is 12
    assert acc.shard_state_bytes(1) == 16
    assert acc.adam_state_bytes(1, acc.MIXED) == 12

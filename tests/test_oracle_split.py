"""Pins of the oracle's adaptive split (O1) to what the pages fix: the worked
example c = 64 -> 10.3x / 6.2x, the floor 0.2 and ceiling 0.8 of r, and the
closed form c^r * c^(1-r) = c.  Source: "RocketKV-adapted -- Two-Stage
Compression", section "The one setting worth tuning"."""
import json
import math
import os

import pytest

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "split_worked_example.json")))


def test_worked_example_c64():
    ex = GOLD["worked_example"]
    r, c1, c2, _ = oracle.split_ratio(ex["c"], 32768, 32)
    assert round(c1, 1) == ex["stage1_ratio_1dp"]
    assert round(c2, 1) == ex["stage2_ratio_1dp"]
    assert r == pytest.approx(0.2 + 0.06 * 6, abs=1e-15)


@pytest.mark.parametrize("c", [1.0, 1.5, 2.0, 3.7, 16.0, 64.0, 100.0, 428.0, 1024.0, 5e6])
def test_product_of_stages_is_target(c):
    _, c1, c2, _ = oracle.split_ratio(c, 1000, 0)
    assert c1 * c2 == pytest.approx(c, rel=1e-12)
    assert c1 >= 1.0 and c2 >= 1.0


def test_floor_and_ceiling():
    r, c1, c2, keep = oracle.split_ratio(1.0, 1234, 7)
    assert r == GOLD["r_floor"] and c1 == 1.0 and c2 == 1.0 and keep == 1234
    # below c = 1 the formula would go under the floor; c = 1 is the smallest
    # valid ratio and r grows with c from there
    rs = [oracle.split_ratio(c, 10, 0)[0] for c in (1, 2, 4, 64, 400, 1024, 4096, 1e9)]
    assert rs == sorted(rs)
    assert rs[-1] == GOLD["r_ceiling"] and rs[-2] == GOLD["r_ceiling"]
    r, c1, c2, _ = oracle.split_ratio(1024.0, 10, 0)
    assert r == pytest.approx(0.8) and c1 == pytest.approx(256.0) and c2 == pytest.approx(4.0)


def test_ranges_of_the_table():
    lo, hi = GOLD["small_ratio_range"]
    for c in (lo, hi):
        assert oracle.split_ratio(c, 10, 0)[0] <= 0.2 + 0.06 * 2 + 1e-12   # near the floor
    lo, hi = GOLD["large_ratio_range"]
    assert 0.5 < oracle.split_ratio(lo, 10, 0)[0] < oracle.split_ratio(hi, 10, 0)[0] < 0.8


def test_keep_counts_of_the_workloads():
    # 32K prompt at budget 512: c = 64 -> keep floor(32768 / 64^0.56)
    assert oracle.split_ratio(64.0, 32768, 32)[3] == math.floor(32768 / 64 ** 0.56) == 3191
    # 109,568 tokens at budget 256: c = 428, stage 1 keeps about 1,360 rows
    assert oracle.split_ratio(109568 / 256, 109568, 32)[3] == 1359
    # keep never drops below the window nor exceeds the prompt
    assert oracle.split_ratio(1e9, 100, 32)[3] == 32
    assert oracle.split_ratio(1.0, 100, 32)[3] == 100
    assert oracle.split_ratio(2.0, 10, 32)[3] == 10


@pytest.mark.parametrize("bad", [0.5, 0.0, -3.0, float("nan"), float("inf")])
def test_invalid_ratio(bad):
    with pytest.raises(oracle.OracleError):
        oracle.split_ratio(bad, 100, 0)

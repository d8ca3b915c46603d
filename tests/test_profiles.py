"""The committed counter figures agree with the summaries they come from.

`profiles/traffic.json` gives, per workload, the HBM bytes one call of the
roofline entry point moves; `bench.py` reports them as `roofline.traffic`.
Each figure must be the calibrated sum of the FETCH_SIZE / WRITE_SIZE rows of
its own summary: the named kernel's row, or, for an entry point that launches
several kernels, every row of that entry point exactly once."""

import json
import os

import pytest

from conftest import ROOT

TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")
ALL_KERNELS = ": all kernels of the call"


def records():
    return sorted(json.load(open(TRAFFIC)).items())


def counter_rows(summary):
    """(label, raw fetch KiB, raw write KiB) of a summary's traffic table."""
    text = open(os.path.join(ROOT, summary)).read()
    table = text.split("## HBM-side traffic", 1)[1]
    rows = []
    for line in table.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 5 and cells[1].replace(".", "").isdigit():
            rows.append((cells[0], float(cells[1]), float(cells[2])))
    return rows


@pytest.mark.parametrize("workload,rec", records(), ids=[w for w, _ in records()])
def test_traffic_is_the_sum_of_its_kernels(workload, rec):
    rows = counter_rows(rec["summary"])
    if rec["kernel"].endswith(ALL_KERNELS):
        prefix = rec["kernel"][: -len(ALL_KERNELS)] + ":"
        picked = [r for r in rows if r[0].startswith(prefix)]
        assert len(picked) >= 2
    else:
        picked = [r for r in rows if r[0] == rec["kernel"]]
        assert len(picked) == 1
    cal = rec["calibration"]
    fetch = sum(r[1] for r in picked) * cal["fetch_factor"] * 1024
    write = sum(r[2] for r in picked) * cal["write_factor"] * 1024
    # the summaries print whole KiB, so allow one KiB of rounding per row
    slack = 1024 * 2 * len(picked)
    assert abs(rec["fetch_bytes"] - fetch) <= slack
    assert abs(rec["write_bytes"] - write) <= slack
    assert abs(rec["bytes_per_launch"] - rec["fetch_bytes"] - rec["write_bytes"]) <= 1

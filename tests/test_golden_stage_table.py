"""The stage shapes the workloads use, and the top-k clamp, against the stage
table printed on the pages (tests/golden/stage_table.json cites it)."""
import json
import os

import oracle
from vision_transformer_sparse_region_amd.workloads import WORKLOADS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "stage_table.json")


def _table():
    with open(GOLDEN) as f:
        return json.load(f)


def test_stage_workloads_follow_the_table():
    tab = _table()
    for name, row in zip(("stage1", "stage2", "stage3"), tab["stages"][:3]):
        wl = WORKLOADS[name]
        assert (wl.height, wl.width) == (row["map"], row["map"])
        assert wl.topk == row["top_k"]
        assert wl.num_heads == row["heads"]
        assert wl.head_dim == row["head_dim"]
        assert wl.n_win == tab["n_win"]


def test_last_stage_routes_every_region():
    tab = _table()
    row = tab["stages"][3]
    n = tab["n_win"]
    cfg = oracle.OracleConfig(1, row["map"], row["map"], row["heads"] * row["head_dim"],
                              row["heads"], n, row["top_k"])
    assert oracle.topk_effective(cfg) == n * n == row["top_k"]
    # the settings list writes the same stage as -1 ("all")
    cfg_all = oracle.OracleConfig(1, row["map"], row["map"], 32, 1, n, tab["settings_topks"][3])
    assert oracle.topk_effective(cfg_all) == n * n

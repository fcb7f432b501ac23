"""bench.py end to end on the GPU, on the small shards: one JSON line with
the fields of its contract, whole steps counted, the roofline entry present,
the fixed placement or the measured one reported, a secondary shard
(device-resident and host step control, and the inf/NaN protocol of the
fragmented-bucket workload); and the smoke() entry point."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FIELDS = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
          "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "roofline")


def _bench(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--no-cpu-baseline", *args],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    line = r.stdout.strip().splitlines()[-1]
    return json.loads(line)


@pytest.mark.parametrize("control", [[], ["--host-control"]])
def test_toy_json_line(control):
    b = _bench("--workload", "toy", "--steps", "4", "--warmup", "1", *control)
    for f in FIELDS:
        assert f in b, f
    assert b["n_gpus"] == 1 and b["steps"] == 4 and b["applied_steps"] == 4
    assert b["value"] > 0 and b["ms_per_step"] > 0
    assert "model" not in b["config"] and "workload" in b["config"]
    r = b["roofline"]
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and 0 < r["frac"] < 1
    # the dominant kernel of the step: the longer of the two phases
    dom = max(("adamw", "reduce_check"), key=lambda k: b["phases"][k]["ms"])
    assert r["kernel"].startswith({"adamw": "adamw_kernel", "reduce_check": "reduce_kernel"}[dom])
    assert r["achieved"] == pytest.approx(b["phases"][dom]["bytes_per_elem"]
                                          * b["config"]["owned_elems"]
                                          / (b["phases"][dom]["ms"] * 1e-3) / 1e9, rel=1e-3)
    # the fixed default order, no placement search
    assert "buffer order ranks_first" in b["config"]["placement"]
    assert b["config"]["placement_search"] is False and b["config"]["placement_setup_ms"] is None
    assert b["final_norm"] is not None and b["final_norm"] > 0


def test_placement_search_and_secondary_shard():
    """--placement auto times the orders at setup and reports the finalists;
    --secondary times a second shard in the same run and reports it as its
    own object with the same measured fields."""
    b = _bench("--workload", "toy", "--steps", "3", "--warmup", "1", "--placement", "auto",
               "--secondary", "bert", "--secondary-steps", "3")
    assert b["config"]["placement_search"] is True and b["config"]["placement_setup_ms"]
    s = b["secondary"]
    assert s["workload"].startswith("bert") and s["steps"] == 3 and s["applied_steps"] == 3
    assert s["value"] > 0 and 0 < s["step_frac_of_peak"] < 1
    assert s["roofline"]["bound"] == "hbm" and s["config"]["owned_elems"] == 13_685_280
    assert "secondary_tuned" not in b           # the primary already searched
    # fixed placement: the secondary is also run with its placement measured
    c = _bench("--workload", "toy", "--steps", "3", "--warmup", "1", "--secondary", "bert",
               "--secondary-steps", "3")
    assert c["secondary"]["config"]["placement_search"] is False
    t = c["secondary_tuned"]
    assert t["config"]["placement_search"] is True and t["config"]["placement_candidates"] > 1
    assert t["applied_steps"] == 3 and t["config"]["arena_slack_gib"] > 0


def test_buckets_overflow_protocol():
    """An inf/NaN every 4th step: those steps are skipped and halve the
    scale (16 steps: 4 skipped, 2^16 / 2^4)."""
    b = _bench("--workload", "buckets", "--steps", "16", "--warmup", "1")
    assert b["applied_steps"] == 12 and b["skipped_steps"] == 4
    assert b["final_loss_scale"] == 2.0 ** 12
    assert b["final_norm"] is None              # the last step overflowed
    # 16 ranks: the reduce (34 B per element) outweighs AdamW (28 B)
    r = b["roofline"]
    assert r["kernel"].startswith("reduce_kernel") and 0 < r["frac"] < 1
    assert b["phases"]["reduce_check"]["ms"] > b["phases"]["adamw"]["ms"]


def test_smoke_entry_point():
    """The round-end entry point: one small owner step on cuda:0, checked
    against the oracle inside smoke() itself (it raises on a mismatch)."""
    import __graft_entry__
    __graft_entry__.smoke()


def test_in_place_reduce_option():
    """--in-place-reduce: the sum goes into rank 0's buffer, reported in the
    config; the line is otherwise complete."""
    b = _bench("--workload", "toy", "--steps", "3", "--warmup", "1", "--in-place-reduce")
    assert b["config"]["in_place_reduce"] is True
    assert b["applied_steps"] == 3 and b["value"] > 0
    assert b["roofline"]["traffic"] is None or b["roofline"]["traffic"] > 0
    d = _bench("--workload", "toy", "--steps", "3", "--warmup", "1")
    assert d["config"]["in_place_reduce"] is False

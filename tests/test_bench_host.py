"""Host-side logic of bench.py that needs no GPU: the source hash that
decides whether the stored HBM counters still describe the kernels, the row
lists of the floor probes, and the guard that keeps counters of refused
launches out of the profiles."""
import os
import shutil

import bench


def _copy_sources(tmp_path):
    root = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "combine_ll_moe_amd", "csrc")
    dst = tmp_path / "csrc"
    dst.mkdir()
    for name in bench.PATH_SOURCES:
        shutil.copy(os.path.join(root, name), dst / name)
    return root, dst


def test_source_hash_ignores_comments_and_spacing(tmp_path):
    root, dst = _copy_sources(tmp_path)
    assert bench.kernel_source_hash(str(dst)) == bench.kernel_source_hash(root)
    f = dst / "combine.hip"
    text = f.read_text()
    f.write_text("// a new comment line\n/* and a\n   block */\n" + text.replace("\n", "\n\n", 3))
    assert bench.kernel_source_hash(str(dst)) == bench.kernel_source_hash(root)


def test_source_hash_sees_code_changes(tmp_path):
    root, dst = _copy_sources(tmp_path)
    f = dst / "kernels.h"
    text = f.read_text()
    assert "constexpr int kTargetBlocks = 512;" in text
    f.write_text(text.replace("constexpr int kTargetBlocks = 512;", "constexpr int kTargetBlocks = 513;"))
    assert bench.kernel_source_hash(str(dst)) != bench.kernel_source_hash(root)



def test_more_than_one_gpu_is_refused():
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "measures one GPU" in r.stderr


def test_floor_probe_rows_match_the_oracle_routing():
    """The floor probes write and read exactly the rows the dispatch and the
    combine use: the bench's stable-sort slots against the oracle's walk."""
    import numpy as np
    import oracle
    import workloads as W
    for name in ("tiny", "decode", "wide_zipf", "worst_fill"):
        w = W.WORKLOADS[name]
        idx = W.routing(w)
        slot, _ = oracle.route(idx, w.num_experts, w.capacity)
        rows = bench.slot_rows(idx, w.num_experts, w.capacity)
        assert np.array_equal(rows, idx.astype(np.int64) * w.capacity + slot), name


def test_refused_counter_runs_are_not_summarized(tmp_path):
    import json
    import pytest
    good = {"metric": "m", "two_phase_combine": {"refusals": False},
            "expert_side": {"refusals": False}}
    bad = dict(good, expert_side={"refusals": True})
    assert bench._refusals(good) == []
    assert bench._refusals(bad) == ["expert_side"]
    log = tmp_path / "f.log"
    log.write_text("[bench] noise\n" + json.dumps(bad) + "\n")
    assert bench._bench_line(str(log)) == bad

    class A:
        fetch_log, write_log = str(log), None
    with pytest.raises(SystemExit, match="refusals"):
        bench.summarize_profiles(A())

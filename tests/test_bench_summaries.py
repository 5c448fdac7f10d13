"""The bench's rocprofv3 summary writers on small synthetic profiler outputs
(host logic only).  They turn a kernel trace and two counter passes into the
figures the profiles report: a split launch's merge kernel belongs to the
attention launch dispatched before it, launches of one kernel with another
grid are the one-share launches, and the counters are scaled by what they read
for a plain copy of known size."""

import csv
import json
import os
import re
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

ATTN = "void sp::(anonymous namespace)::attn_bf16_kernel<128, false, true, false>(sp::(anonymous namespace)::AttnArgs)"
MERGE = "void sp::(anonymous namespace)::attn_combine_kernel<128, false, false>(sp::(anonymous namespace)::AttnArgs)"
MOVE = "sp::(anonymous namespace)::relayout_kernel(sp::(anonymous namespace)::RelayoutArgs)"
G_ALL, G_SHARE, M_ALL, M_SHARE = 4325376, 589824, 393216, 540672


@pytest.fixture
def profile_dir(tmp_path, monkeypatch):
    out = tmp_path / "profiles"
    out.mkdir()
    monkeypatch.setattr(bench, "PROFILE_DIR", str(out))
    return out


def test_kernel_trace_summary_labels_each_merge_by_its_launch(tmp_path, profile_dir):
    # dispatch order of a bench run: a move, then all-ranks launches each with
    # its merge, then one-share launches each with its merge (durations in us)
    seq = [(MOVE, 1000, 500)]
    seq += [x for i in range(3) for x in ((ATTN, G_ALL, 28000 + 10 * i), (MERGE, M_ALL, 8 + i))]
    seq += [x for i in range(2) for x in ((ATTN, G_SHARE, 3500 + 20 * i), (MERGE, M_SHARE, 11 + 2 * i))]
    trace = tmp_path / "trace.csv"
    with open(trace, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z", "Start_Timestamp", "End_Timestamp"])
        t = 10_000
        # rows out of order on purpose: the writer orders dispatches by start time
        rows = []
        for name, grid, us in seq:
            rows.append([name, grid, 1, 1, t, t + us * 1000])
            t += us * 1000 + 5000
        w.writerows(reversed(rows))
    line = {"metric": "attention_tflops", "config": {"workload": "long_hires"}, "kernel_source_hash": "abc",
            "roofline": {"avg_launch_ms": 27.96, "achieved": 1258.3, "frac": 0.5033, "split": True},
            "roofline_share": {"avg_launch_ms": 3.4766, "achieved": 1265.1, "frac": 0.506, "split": True},
            "kernels": {}}
    bj = tmp_path / "bench.json"
    bj.write_text("noise\n" + json.dumps(line) + "\n")
    bench.write_kernel_trace_summary(str(trace), str(bj), "title", "cmd", "trace.md")
    text = (profile_dir / "trace.md").read_text()
    rows = {}
    for l in text.splitlines():
        m = re.match(r"\| `(.+?)` \| (\d+) \| (.*?) \| (\d+) \| ([\d.]+) \|", l)
        if m:
            rows[int(m.group(2))] = (m.group(3), int(m.group(4)), float(m.group(5)))
    assert rows[G_ALL] == ("all ranks (R = 8)", 3, 28010.0)
    assert rows[G_SHARE] == ("one share (R = 1)", 2, 3510.0)
    assert rows[M_ALL] == ("merge of the all-ranks launch", 3, 9.0)
    assert rows[M_SHARE] == ("merge of the split share", 2, 12.0)
    assert rows[1000][0] == ""
    assert "attention, all ranks (split + merge): 27960.0 us" in text
    assert "one share (R = 1, split + merge): 3476.6 us" in text


def _counter_dir(tmp_path, name, counter, dispatches):
    d = tmp_path / name / "host"
    d.mkdir(parents=True)
    with open(d / "p_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        for i, (kname, grid, kib) in enumerate(dispatches):
            # a counter can come back as several rows (one per XCD, say): the writer sums them
            w.writerow([i + 1, kname, grid, counter, kib / 2])
            w.writerow([i + 1, kname, grid, counter, kib / 2])
    return str(tmp_path / name)


def test_traffic_summary_scales_counters_and_counts_merges_with_their_launch(tmp_path, profile_dir):
    copy_kib = bench.COPY_PROBE_BYTES / 1024
    # FETCH_SIZE reads half of the true bytes (scale 2), WRITE_SIZE all of them
    # (scale 1); true KiB per launch: all ranks 1000 read + 100 written, its
    # merge 10 + 5; share 300 + 40, its merge 20 + 6; the first launch of each
    # kind (cold) is left out of the averages
    def seq(rd):
        k = (lambda r, w: r / 2) if rd else (lambda r, w: w)
        return [("copyBuffer", 1, k(copy_kib, copy_kib)), (MOVE, 9, k(70, 70)),
                (ATTN, G_ALL, k(5000, 900)), (MERGE, M_ALL, k(10, 5)),
                (ATTN, G_ALL, k(1000, 100)), (MERGE, M_ALL, k(10, 5)),
                (ATTN, G_ALL, k(1000, 100)), (MERGE, M_ALL, k(10, 5)),
                (ATTN, G_SHARE, k(900, 90)), (MERGE, M_SHARE, k(20, 6)),
                (ATTN, G_SHARE, k(300, 40)), (MERGE, M_SHARE, k(20, 6))]
    fd = _counter_dir(tmp_path, "fetch", "FETCH_SIZE", seq(True))
    wd = _counter_dir(tmp_path, "write", "WRITE_SIZE", seq(False))
    bench.write_traffic_summary("long_hires", fd, wd, ["cmd"])
    text = (profile_dir / "attention_traffic_long_hires.md").read_text()
    rec = json.loads(re.search(r"^traffic_json:\s*(\{.*\})\s*$", text, flags=re.M).group(1))
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["fetch_bytes"] == pytest.approx(1010 * 1024, abs=2)
    assert rec["write_bytes"] == pytest.approx(105 * 1024, abs=2)
    assert rec["share_bytes_per_launch"] == pytest.approx((320 + 46) * 1024, abs=2)

"""The measurement records that bench.py reads or that back its headline line
are taken on the kernel source in the tree.

bench.py reports a launch's HBM traffic only from a
profiles/sparse_attn_<config>_traffic.json whose kernel hash matches the
attention sources (attn.hip and mcs_common.h, code lines only), so a kernel
change without a new counter run would silently turn the traffic field into
null; the committed headline line must carry the same hash.
"""
import glob
import json
import os

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def current_hash():
    return bench.source_hash("attn.hip", "mcs_common.h")


def test_traffic_records_match_the_kernel_source():
    files = sorted(glob.glob(os.path.join(ROOT, "profiles", "sparse_attn_*_traffic.json")))
    assert files, "no traffic records"
    h = current_hash()
    for f in files:
        t = json.load(open(f))
        assert t["kernel_src_hash"] == h, f"{os.path.basename(f)} was taken on kernel {t['kernel_src_hash']}, tree has {h}"
        assert t["bytes_per_launch"] > 0
        # the calibration: a 1 GiB copy reads back as FETCH 0.5 GiB and WRITE 1 GiB (in KiB)
        assert abs(t["fetch_scale"] * t["copy_1GiB_fetch_kib"] - 1048576.0) < 1.0
        assert abs(t["write_scale"] * t["copy_1GiB_write_kib"] - 1048576.0) < 1.0
        cfg = os.path.basename(f)[len("sparse_attn_"):-len("_traffic.json")]
        assert bench.load_traffic(cfg, h) == t["bytes_per_launch"]


def test_headline_line_matches_the_kernel_source():
    line = json.loads(open(os.path.join(ROOT, "profiles", "bench_hunyuan720p_25_line.json")).read())
    assert line["roofline"]["kernel_src_hash"] == current_hash()
    assert line["roofline"]["traffic"] is not None
    assert line["config"]["workload"].startswith("hunyuan720p_25")
    assert abs(line["roofline"]["frac"] - line["roofline"]["achieved"] / line["roofline"]["peak"]) < 1e-3


def test_source_hash_ignores_comments_and_blank_lines(tmp_path, monkeypatch):
    d = tmp_path / "sparse_attention_diffusion_attn_amd" / "csrc"
    d.mkdir(parents=True)
    (d / "a.hip").write_text("int x = 1;  // one\n\n  int   y = 2;\n")
    (d / "b.hip").write_text("// header\nint x = 1;\nint y = 2;   // two\n")
    (d / "c.hip").write_text("int x = 1;\nint y = 3;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.source_hash("a.hip") == bench.source_hash("b.hip")
    assert bench.source_hash("a.hip") != bench.source_hash("c.hip")

"""The benchmark's regression guard (bench.py --guard): CPU only, on synthetic lines."""

import json

import bench


def line(us, gemm_us, sweep_ms):
    return {"roofline": {"avg_launch_us": us}, "gemm": {"mean_us": gemm_us},
            "extra": {"sweep_64_layers_fused": {"ms_per_sweep": sweep_ms}}}


def test_guard_flags_only_slowdowns_beyond_ten_percent(tmp_path):
    ref = tmp_path / "ref.json"
    ref.write_text("log line that is not json\n" + json.dumps(line(12.0, 350.0, 3.3)) + "\n")
    ok, rep = bench.guard(line(12.9, 300.0, 3.4), str(ref))  # 7.5 % slower, faster, 3 % slower
    assert ok and not any(v["regression"] for v in rep.values())
    ok, rep = bench.guard(line(13.5, 350.0, 3.3), str(ref))  # 12.5 % slower headline
    assert not ok and rep["roofline.avg_launch_us"]["regression"]
    assert not rep["gemm.mean_us"]["regression"]
    ok, rep = bench.guard({"roofline": {"avg_launch_us": 12.0}}, str(ref))  # missing entries are skipped
    assert ok and list(rep) == ["roofline.avg_launch_us"]

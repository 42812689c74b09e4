"""The HBM-traffic figure in the bench line is reported only for the run the
counters were taken on (host logic of bench.py, no GPU)."""
import json

import bench


def _write(tmp_path, **over):
    rec = {"kernel": "decode_splitkv", "workload": "v2_b64_ragged", "bytes_per_launch": 4.2e8,
           "kernel_source_sha256": bench.kernel_source_sha256()}
    rec.update(over)
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(rec))
    return str(p)


def test_current_record_is_used(tmp_path):
    assert bench.recorded_traffic("v2_b64_ragged", 0, _write(tmp_path)) == 4.2e8


def test_stale_sources_give_none(tmp_path):
    assert bench.recorded_traffic("v2_b64_ragged", 0, _write(tmp_path, kernel_source_sha256="0" * 64)) is None


def test_other_workload_or_workgroups_give_none(tmp_path):
    p = _write(tmp_path)
    assert bench.recorded_traffic("v2_b32_ragged", 0, p) is None
    assert bench.recorded_traffic("v2_b64_ragged", 128, p) is None


def test_missing_or_broken_record_gives_none(tmp_path):
    assert bench.recorded_traffic("v2_b64_ragged", 0, str(tmp_path / "absent.json")) is None
    bad = tmp_path / "bad.json"
    bad.write_text("{not json")
    assert bench.recorded_traffic("v2_b64_ragged", 0, str(bad)) is None


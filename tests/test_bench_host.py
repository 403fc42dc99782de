"""Host-side checks of bench.py's reading of the committed profile summaries (no GPU)."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_traffic_lines_parse_and_name_existing_sources():
    """Every machine-readable 'traffic' line of profiles/prefill_128k_video_traffic.md parses, names
    sources that exist, and gives positive byte counts; read_traffic() returns no more kernels
    than there are such lines (entries whose sources changed are left out, never misread)."""
    path = os.path.join(ROOT, "profiles", "prefill_128k_video_traffic.md")
    lines = [ln for ln in open(path) if ln.startswith("traffic ") and "fetch_bytes=" in ln]
    assert lines, "no traffic lines"
    for ln in lines:
        f = dict(kv.split("=", 1) for kv in ln.split()[2:])
        names, digests = f["source"].split(","), f["sha256"].split(",")
        assert len(names) == len(digests)
        for n in names:
            assert os.path.exists(os.path.join(ROOT, "sparse_attention_long_04_amd", "csrc", n)), n
        assert int(f["fetch_bytes"]) > 0 and int(f["write_bytes"]) > 0
    got = bench.read_traffic()
    assert set(got) <= {ln.split()[1] for ln in lines}
    assert all(v > 0 for v in got.values())

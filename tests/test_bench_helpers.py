"""Host logic of bench.py that its JSON line depends on: the counter summaries
behind roofline.traffic are read back, and dropped once the kernels they were
taken on change."""
import os
import shutil

import bench


def test_committed_traffic_summaries_match_sources():
    # both summaries in profiles/ were taken on the kernels as committed
    assert bench.measured_traffic() is not None
    assert bench.measured_traffic(bench.PREFILL_TRAFFIC_FILE, bench.PREFILL_SOURCES) is not None


def test_traffic_is_dropped_when_sources_change(tmp_path):
    root = tmp_path / "repo"
    for rel in bench.DECODE_SOURCES:
        dst = root / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(bench.ROOT, rel), dst)
    summary = tmp_path / "traffic.txt"
    digest_of = lambda: bench.sources_digest([str(root / r) for r in bench.DECODE_SOURCES])
    summary.write_text(f"# comment: 1\nbytes_per_call: 1234\nsources_sha256_16: {digest_of()}\n")
    srcs = [str(root / r) for r in bench.DECODE_SOURCES]
    assert bench.measured_traffic(str(summary), srcs) == 1234
    with open(srcs[0], "a") as f:            # any edit of a kernel source
        f.write("\n// edited\n")
    assert bench.measured_traffic(str(summary), srcs) is None
    assert bench.measured_traffic(str(tmp_path / "missing.txt"), srcs) is None

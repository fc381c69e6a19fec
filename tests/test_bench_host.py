"""bench.py on the host: the one-GPU guard, and the committed rocprofv3 records it reads are
those of the current kernel sources (bench.py reports HBM traffic only from counters taken on
the source it runs)."""
import os
import re
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_traffic_records_match_the_kernel_sources():
    assert bench.traffic_for("long_gqa") is not None
    assert bench.traffic_for("long_gqa", backward=True) is not None


def test_kernel_trace_summaries_name_the_current_sources():
    for md, src in (("attn_fwd_long_gqa_kernel_trace.md", bench.KERNEL_SRC),
                    ("attn_bwd_long_gqa_kernel_trace.md", bench.KERNEL_SRC_BWD)):
        text = open(os.path.join(ROOT, "profiles", md)).read()
        m = re.search(r"sha256\s+([0-9a-f]{64})", text)
        assert m, md
        assert m.group(1) == bench.kernel_sha(src), md

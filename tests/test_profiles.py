"""The committed rocprofv3 summaries name the kernels bench.py picks out of them.

bench.py finds the timed kernels in a kernel trace and in the counter runs by regular
expressions over their demangled names (template arguments included), so a change to a kernel's
template parameters must come with a change to those patterns, or the summaries silently lose
those kernels.  This checks every pattern against the names in the committed trace summary.
"""
import glob
import json
import os
import re

import bench

PROFILES = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles")


def _stats_kernel_names():
    names = []
    for path in glob.glob(os.path.join(PROFILES, "kernel_stats_*.txt")):
        with open(path) as fh:
            names += [ln.split(" | ")[0] for ln in fh if " | " in ln]
    return names


def test_every_kernel_pattern_names_a_profiled_kernel():
    names = _stats_kernel_names()
    assert names, "no kernel-trace summary under profiles/"
    for pattern in bench.KERNEL_PATTERNS:
        hits = [n for n in names if re.search(pattern, n)]
        assert len(hits) == 1, f"{pattern!r} matches {len(hits)} profiled kernels"


def test_traffic_summaries_are_complete():
    paths = glob.glob(os.path.join(PROFILES, "traffic_*.json"))
    assert paths
    for path in paths:
        with open(path) as fh:
            d = json.load(fh)
        for key in ("source_hash", "hbm_bytes_per_launch", "algorithmic_bytes_per_launch",
                    "traffic_over_algorithmic"):
            assert key in d, f"{os.path.basename(path)} lacks {key}"
        assert d["hbm_bytes_per_launch"] >= d["algorithmic_bytes_per_launch"] * 0.99, path

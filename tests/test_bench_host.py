"""Host-side pieces of bench.py that need no GPU."""

import os
import re

import bench

CSRC = os.path.join(bench.ROOT, "decode_attention_kv_attn_amd", "csrc")
KERNELS = {"gqa": ["gqa_valu.hip", "gqa_mfma.hip"], "mla": ["mla_mfma.hip"]}


def local_includes(name, seen=None):
    """Every header of csrc that `name` includes, directly or through others."""
    seen = set() if seen is None else seen
    text = open(os.path.join(CSRC, name)).read()
    for inc in re.findall(r'^\s*#include\s+"([^"]+)"', text, flags=re.M):
        if inc not in seen and os.path.exists(os.path.join(CSRC, inc)):
            seen.add(inc)
            local_includes(inc, seen)
    return seen


def test_traffic_hash_covers_kernel_sources():
    """A recorded traffic figure is dropped when any source of its kernel
    changes, so the hash must cover every device source the kernel compiles
    from."""
    for kind, roots in KERNELS.items():
        needed = set(roots)
        for r in roots:
            needed |= local_includes(r)
        missing = needed - set(bench.KERNEL_SOURCES[kind])
        assert not missing, (kind, sorted(missing))


def test_traffic_records_are_consistent():
    """Each committed traffic record is the counters scaled by its own copy
    calibration, and names the commands and workload it came from.  (Whether
    it still matches the sources is bench.py's business: it reports null
    traffic once the hash differs.)"""
    import json
    prof = os.path.join(bench.ROOT, "profiles")
    recs = [f for f in sorted(os.listdir(prof))
            if f.startswith("traffic_") and f.endswith(".json")]
    assert recs
    for f in recs:
        t = json.load(open(os.path.join(prof, f)))
        w = f[len("traffic_"):-len(".json")]
        assert t["workload"] == w
        c = t["copy_calibration"]
        assert abs(c["fetch_scale"] - c["bytes"] / (c["fetch_kib_raw"] * 1024)) < 1e-3
        assert abs(c["write_scale"] - c["bytes"] / (c["write_kib_raw"] * 1024)) < 1e-3
        rd = t["fetch_kib_per_dispatch_raw"] * 1024 * c["fetch_scale"]
        wr = t["write_kib_per_dispatch_raw"] * 1024 * c["write_scale"]
        assert abs(t["read_bytes_per_launch"] - rd) <= 1e-4 * rd + 1024
        assert abs(t["write_bytes_per_launch"] - wr) <= 1e-4 * wr + 1024
        assert abs(t["bytes_per_launch"] - t["read_bytes_per_launch"]
                   - t["write_bytes_per_launch"]) <= 1  # each rounded down on its own
        # HBM traffic of a decode launch is at least its algorithmic bytes
        assert t["read_bytes_per_launch"] >= t["algorithmic_bytes_per_launch"]
        assert all(f"--workload {w} " in cmd for cmd in t["commands"][:2])

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


def test_traffic_records_match_sources():
    """Committed traffic records carry the hash of the sources they were
    taken on; bench.py reports them only while it matches."""
    prof = os.path.join(bench.ROOT, "profiles")
    for f in sorted(os.listdir(prof)):
        if f.startswith("traffic_") and f.endswith(".json"):
            w = f[len("traffic_"):-len(".json")]
            kind = "mla" if w.startswith("mla") else "gqa"
            assert bench.traffic_from_profile(w, kind) is not None, w

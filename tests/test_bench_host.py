"""Host-side pieces of bench.py that need no GPU."""

import os
import re

import bench

CSRC = os.path.join(bench.ROOT, "decode_attention_kv_attn_amd", "csrc")
KERNELS = {"gqa": ["gqa_valu.hip", "gqa_mfma.hip", "combine.hip"],
           "mla": ["mla_mfma.hip", "mla_pair.hip", "combine.hip"]}


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
    """Each committed traffic record is the counters of each kernel of a step
    (decode, and the merge of a split plan) scaled by its own copy
    calibration, summed per step, and names the commands and workload it came
    from.  (Whether it still matches the sources is bench.py's business: it
    reports null traffic once the hash differs.)"""
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
        assert any(k.startswith(("gqa_decode_", "mla_")) for k in t["kernels"])
        rd_sum = wr_sum = 0
        for k in t["kernels"].values():
            rd = k["fetch_kib_per_dispatch_raw"] * 1024 * c["fetch_scale"]
            wr = k["write_kib_per_dispatch_raw"] * 1024 * c["write_scale"]
            assert abs(k["read_bytes"] - rd) <= 1e-4 * rd + 1024
            assert abs(k["write_bytes"] - wr) <= 1e-4 * wr + 1024
            rd_sum += k["read_bytes"]
            wr_sum += k["write_bytes"]
        assert t["read_bytes_per_step"] == rd_sum
        assert t["write_bytes_per_step"] == wr_sum
        assert t["bytes_per_step"] == rd_sum + wr_sum
        # HBM traffic of a decode step is at least its algorithmic bytes
        assert t["read_bytes_per_step"] >= t["algorithmic_bytes_per_step"]
        assert all(f"--workload {w} " in cmd for cmd in t["commands"][:2])


def test_algorithmic_bytes_of_the_workloads():
    """The byte count the bench divides by: the attention-head note's
    512 MiB per layer for MHA at B=1, T=32768 (section 1), 64 times that at
    B=64; a window of 4096 over a 32768-row linear cache counts only the
    window; the MLA latent (section 5.4) counts (512 + 64) * 2 bytes a row."""
    import synth
    alg = lambda name: bench.algorithmic_bytes(synth.workload(name))
    assert alg("mha_t32k_b1") == 512 * 2**20
    assert alg("mha_t32k_b64") == 64 * 512 * 2**20
    assert alg("mqa_t32k_b1") == 16 * 2**20
    assert alg("llama3_8b_gqa_t4096") == 512 * 2**20
    assert alg("swa_linear_w4096_t32k") == alg("swa_ring_w4096_t32k") == 256 * 2**20
    assert alg("mla_b64_t8192") == 64 * 8192 * 576 * 2


def test_sample_stride_bounds_the_host_copy():
    assert bench.sample_stride(2048, 16 << 20) == 16      # 128 units of 16 MiB
    assert bench.sample_stride(256, 4 << 20) == 1         # 1 GiB: all of it
    assert bench.sample_stride(1, 64 << 30) == 1


def test_headline_traffic_record_is_current():
    """The default workload's bench line reports HBM traffic only from a
    record taken on the current kernel sources; any edit to a source the
    hash covers must be followed by new counter passes (or, where the
    compiled code is unchanged, a re-keyed record)."""
    assert bench.traffic_from_profile(bench.DEFAULT_WORKLOAD, "gqa") is not None

"""Decode-attention benchmark: KV-read GB/s (% of HBM peak) and us/step.

One step = one library call = one layer's decode attention for every
sequence of the batch.  Inputs are seeded synthetic tensors drawn on the GPU
(``synth``), already resident in HBM when timing starts; several copies of
the cache are rotated so the working set exceeds the 256 MB Infinity Cache.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

prints ONE JSON line.  The default workload is the largest single-GPU
configuration: MHA at B=64, 32 heads, d=128, T=32768, bf16 -- 32 GiB of K/V
per layer (the attention-head note's 512 MiB-per-layer MHA example, section
1, for 64 sequences).

``value`` = algorithmic KV bytes per step / measured step time, where the
algorithmic bytes are 2 * s * d * H_kv * (visible positions summed over the
batch) -- only what the method must read (xuesongtap "attention-head" note,
section 1, Bytes_KV), never masked or padded capacity.  The K timed steps run
as TIMED_SEGMENTS back-to-back segments, each between its own pair of HIP
events on the launch stream; the step time reported is the median segment's.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, datasheet
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
METRIC = "decode-attention KV-read GB/s (% of HBM peak) and µs/step per layer"
DEFAULT_WORKLOAD = "mha_t32k_b64"
TIMED_SEGMENTS = 5  # the K timed steps are cut into this many event-timed runs
SETTLE_S = 0.3  # seconds of untimed calls before the warmup (clock ramp-up)
CPU_SAMPLE_BYTES = 2 << 30  # host copy of the CPU baseline's sample, at most
KERNEL_SOURCES = {"gqa": ["gqa_valu.hip", "gqa_mfma.hip", "combine.hip", "balance.h",
                          "visible.h", "device_common.h", "internal.h"],
                  "mla": ["mla_mfma.hip", "mla_pair.hip", "mla_common.h", "combine.hip",
                          "balance.h", "visible.h", "device_common.h", "internal.h"]}
MERGE_KERNEL = "lse_combine"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--rotate-bytes", type=float, default=1.0,
                    help="GiB of rotating cache copies (defeats the MALL)")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--record-traffic", metavar="PMC_DIR",
                    help="write profiles/traffic_<workload>.json from rocprofv3 "
                         "--pmc FETCH_SIZE / WRITE_SIZE runs of this workload "
                         "(PMC_DIR/{FETCH_SIZE,WRITE_SIZE}/run_counter_collection.csv) "
                         "and of the --probe copy (--copy-dir)")
    ap.add_argument("--copy-dir", metavar="PMC_DIR",
                    help="the --pmc runs of `bench.py --probe` (the 1 GiB plain copy)")
    ap.add_argument("--probe", action="store_true",
                    help="only run the HBM read probe and a 1 GiB plain copy")
    return ap.parse_args()


def visible_counts(w, seq_lens):
    """Visible positions per sequence, from the lengths, window and ring."""
    import numpy as np
    T_cap, window, ring = w["T_cap"], w.get("window", 0), bool(w.get("ring"))
    lens = (np.full(w["B"], T_cap) if seq_lens is None
            else seq_lens.cpu().numpy().astype(np.int64))
    lens = np.maximum(lens, 0)
    if not ring:
        lens = np.minimum(lens, T_cap)
    lo = np.zeros_like(lens)
    if window > 0:
        lo = np.maximum(lo, lens - window)
    if ring:
        lo = np.maximum(lo, lens - T_cap)
    return lens - lo


def kernel_source_hash(kind="gqa"):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "decode_attention_kv_attn_amd", "csrc")
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload, kind="gqa"):
    """HBM bytes per step (decode kernel plus its merge, if any) from
    committed rocprofv3 --pmc results, if they were taken on the current
    kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_hash") != kernel_source_hash(kind):
        print(f"bench: traffic_{workload}.json was taken on other kernel sources; "
              "traffic is null until it is recorded again", file=sys.stderr, flush=True)
        return None
    return rec.get("bytes_per_step")


# ---------------------------------------------------------------- CPU baseline
def host_workers():
    """Host threads for the CPU baseline: the cores this process may use, at
    most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def timed_passes(tasks, seconds, workers):
    """Run every task (a callable returning the KV bytes it covered) on a
    pool of `workers` host threads, each numpy call on one BLAS thread, pass
    after pass until `seconds` have passed.  Returns (bytes, tasks, s)."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits
    done = n = 0
    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=workers) as ex:
        t0 = time.perf_counter()
        while True:
            for nb in ex.map(lambda f: f(), tasks):
                done += nb
                n += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
    return done, n, dt


def sample_stride(n_units, unit_bytes):
    """Every how many units the sample takes one, so its host copy stays
    within CPU_SAMPLE_BYTES."""
    keep = max(1, min(n_units, CPU_SAMPLE_BYTES // max(1, unit_bytes)))
    return max(1, math.ceil(n_units / keep))


def cpu_baseline(w, inp, seconds):
    """The float64 oracle as it stands, on the host's cores: a sample of the
    workload's (sequence, KV head) units spread over the batch, each copied
    to host memory on its own (never the whole cache), then timed over
    passes with one unit per task on a pool of host threads (one BLAS thread
    per task: the per-unit products are small) until `seconds` have passed."""
    import oracle
    s = 2 if w.get("dtype", "bf16") == "bf16" else 4
    B, H_q, H_kv, d = w["B"], w["H_q"], w["H_kv"], w["d"]
    n = H_q // H_kv
    sl = None if inp["seq_lens"] is None else inp["seq_lens"].cpu()
    rh = None if inp["ring_head"] is None else inp["ring_head"].cpu()
    vis = visible_counts(w, sl)
    q = inp["q"].cpu()
    units = [(b, g) for b in range(B) for g in range(H_kv)]
    stride = sample_stride(len(units), 2 * s * d * w["T_cap"])
    tasks = []
    for b, g in units[::stride]:
        qs = q[b:b + 1, g * n:(g + 1) * n].clone()
        ks = inp["k"][b:b + 1, g:g + 1].cpu()
        vs = inp["v"][b:b + 1, g:g + 1].cpu()
        sls = None if sl is None else sl[b:b + 1].clone()
        rhs = None if rh is None else rh[b:b + 1].clone()
        nb = 2 * s * d * int(vis[b])
        tasks.append(lambda qs=qs, ks=ks, vs=vs, sls=sls, rhs=rhs, nb=nb: (
            oracle.gqa_decode_ref(qs, ks, vs, sls, rhs, inp["window"], inp["scale"]),
            nb)[1])
    workers = host_workers()
    done, n_tasks, dt = timed_passes(tasks, seconds, workers)
    return {"value": done / dt / 1e9, "unit": "GB/s", "cores": workers,
            "kind": "oracle",
            "sample": f"{len(tasks)} of the {len(units)} (sequence, KV-head) units of "
                      f"{w['name']} (every {stride}th, copied to the host one by one), "
                      f"{n_tasks} unit calls in {dt:.1f} s on {workers} host threads "
                      "with one BLAS thread each, float64 numpy"}


def cpu_baseline_mla(w, inp, seconds):
    """The float64 MLA oracle on the host's cores over a sample of whole
    sequences (copied to host memory one by one), one sequence per task."""
    import oracle
    B, T = w["B"], w["T_cap"]
    row_bytes = (w["d_c"] + w["d_rope"]) * 2
    sl = None if inp["seq_lens"] is None else inp["seq_lens"].cpu()
    q = inp["q"].cpu()
    stride = sample_stride(B, T * row_bytes)
    tasks = []
    for b in range(0, B, stride):
        qs = q[b:b + 1].clone()
        lat = inp["latent"][b:b + 1].cpu()
        sls = None if sl is None else sl[b:b + 1].clone()
        nb = row_bytes * (T if sl is None else int(sl[b].clamp(0, T)))
        tasks.append(lambda qs=qs, lat=lat, sls=sls, nb=nb: (
            oracle.mla_decode_ref(qs, lat, w["d_c"], w["scale"], sls), nb)[1])
    workers = host_workers()
    done, n_tasks, dt = timed_passes(tasks, seconds, workers)
    return {"value": done / dt / 1e9, "unit": "GB/s", "cores": workers,
            "kind": "oracle",
            "sample": f"{len(tasks)} of the {B} sequences of {w['name']} (copied to "
                      f"the host one by one), {n_tasks} sequence calls in {dt:.1f} s "
                      f"on {workers} host threads with one BLAS thread each, "
                      "float64 numpy"}


# ---------------------------------------------------------------- GPU probes
def probe_read_gbs(dev, nbytes=4 << 30, reps=10):
    """Best streaming-read rate of this GPU (attn_probe_read over a buffer far
    larger than the caches), in GB/s."""
    import torch

    import decode_attention_kv_attn_amd as L
    x = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    x.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    best = 0.0
    stream = torch.cuda.current_stream(dev)
    for blocks in (256 * 8, 256 * 32):
        for _ in range(2):
            L.attn_probe_read(x, sink, blocks)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            L.attn_probe_read(x, sink, blocks)
        e1.record(stream)
        torch.cuda.synchronize()
        best = max(best, nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del x
    return best


def run_probe(dev):
    """Read probe plus a plain 1 GiB copy (the known-size kernel that scales
    the FETCH_SIZE / WRITE_SIZE counters)."""
    import torch

    import decode_attention_kv_attn_amd as L
    read = probe_read_gbs(dev)
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        L.attn_probe_copy(dst, src)
    torch.cuda.synchronize()
    print(json.dumps({"probe_read_GBps": round(read, 1), "copy_bytes": n,
                      "copy_launches": 3}), flush=True)


# ---------------------------------------------------------------- traffic
def _counter_kib_per_dispatch(csv_path, kernel_substr):
    """Mean over dispatches of a kernel (name containing kernel_substr) of the
    counter in a rocprofv3 counter_collection.csv, summed per dispatch;
    (0, 0) when no dispatch matches."""
    import csv
    per = {}
    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            if kernel_substr in row["Kernel_Name"]:
                per[row["Dispatch_Id"]] = per.get(row["Dispatch_Id"], 0.0) + float(row["Counter_Value"])
    if not per:
        return 0.0, 0
    return sum(per.values()) / len(per), len(per)


def algorithmic_bytes(w):
    """Bytes the method must read per step: K and V of every visible position
    (attention-head section 1, Bytes_KV), or the latent rows (section 5.4,
    Bytes_MLA)."""
    lens = workload_seq_lens(w)
    if w["kind"] == "mla":
        Tsum = w["B"] * w["T_cap"] if lens is None else int(lens.clamp(0, w["T_cap"]).sum())
        return Tsum * (w["d_c"] + w["d_rope"]) * 2
    s = 2 if w.get("dtype", "bf16") == "bf16" else 4
    return int(2 * s * w["d"] * w["H_kv"] * int(visible_counts(w, lens).sum()))


def record_traffic(args):
    """HBM bytes per step of the workload -- its decode kernel and, for a
    split plan, its merge kernel -- from FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for the 1 GiB plain
    copy of --probe, into profiles/traffic_<workload>.json with a hash of the
    kernel sources."""
    import synth
    w = synth.workload(args.workload)
    kind = "mla" if w["kind"] == "mla" else "gqa"
    decode = "mla_" if kind == "mla" else "gqa_decode_"  # mla_pair_decode, mla_decode_mfma
    d = args.record_traffic
    if not args.copy_dir:
        sys.exit("--record-traffic needs --copy-dir: the --pmc runs of the plain copy")
    csv_of = lambda root, c: os.path.join(root, c, "run_counter_collection.csv")
    cf, _ = _counter_kib_per_dispatch(csv_of(args.copy_dir, "FETCH_SIZE"), "plain_copy")
    cw, _ = _counter_kib_per_dispatch(csv_of(args.copy_dir, "WRITE_SIZE"), "plain_copy")
    if cf <= 0 or cw <= 0:
        sys.exit("no plain_copy dispatch in the --copy-dir runs")
    copy_bytes = 1 << 30
    fs, ws = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    kernels = {}
    for name in (decode, MERGE_KERNEL):
        fk, nf = _counter_kib_per_dispatch(csv_of(d, "FETCH_SIZE"), name)
        wk, nw = _counter_kib_per_dispatch(csv_of(d, "WRITE_SIZE"), name)
        if nf == 0 and nw == 0:
            continue
        if nf == 0 or nw == 0:
            sys.exit(f"{name}: dispatches in only one of the two counter runs")
        kernels[name + "*"] = {
            "dispatches": [nf, nw],
            "fetch_kib_per_dispatch_raw": round(fk, 1),
            "write_kib_per_dispatch_raw": round(wk, 1),
            "read_bytes": int(fk * 1024 * fs),
            "write_bytes": int(wk * 1024 * ws),
        }
    if decode + "*" not in kernels:
        sys.exit(f"no dispatch of {decode} in {d}")
    rd = sum(k["read_bytes"] for k in kernels.values())
    wr = sum(k["write_bytes"] for k in kernels.values())
    cmd = (f"python bench.py --workload {w['name']} --steps 3 --warmup 1 "
           "--no-cpu-baseline")
    rec = {
        "workload": w["name"],
        "kernel_source_hash": kernel_source_hash(kind),
        "commands": [
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/FETCH_SIZE -o run -- {cmd}",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/WRITE_SIZE -o run -- {cmd}",
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {args.copy_dir}/FETCH_SIZE -o run -- python bench.py --probe",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {args.copy_dir}/WRITE_SIZE -o run -- python bench.py --probe",
        ],
        "copy_calibration": {"bytes": copy_bytes, "fetch_kib_raw": round(cf, 1),
                             "write_kib_raw": round(cw, 1), "fetch_scale": round(fs, 4),
                             "write_scale": round(ws, 4)},
        "kernels": kernels,
        "read_bytes_per_step": rd,
        "write_bytes_per_step": wr,
        "bytes_per_step": rd + wr,
        "algorithmic_bytes_per_step": algorithmic_bytes(w),
    }
    rec["read_over_algorithmic"] = round(rd / rec["algorithmic_bytes_per_step"], 4)
    path = os.path.join(ROOT, "profiles", f"traffic_{w['name']}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def workload_seq_lens(w):
    """The workload's seq_lens on the CPU (None when every sequence is full),
    drawn exactly as the input generator draws them."""
    import torch

    import synth
    base = 1234 + 100 * w["index"]
    if w.get("ragged"):
        lo, hi = w["ragged"]
        return synth.draw_ints(w["B"], lo, hi, base + 3)
    if w.get("logical_len"):
        return torch.full((w["B"],), w["logical_len"], dtype=torch.int32)
    return None


# ---------------------------------------------------------------- timing
def run_timed(step, args, dev):
    """Settle, warm up, then time exactly args.steps calls of step(i).

    The settle phase runs the same step for at least SETTLE_S seconds before
    the warmup, so the memory and core clocks have left their idle states
    when the timed region starts.  The args.steps timed calls run as
    TIMED_SEGMENTS back-to-back segments, each bracketed by a pair of HIP
    events on the launch stream and nothing else (an event pair around every
    call costs the GPU about 3.5 us per event, measured, which would inflate
    short steps).  Each step launches the decode kernel once (plus its merge
    when the plan splits), so a segment's mean step time is the average
    launch period of that kernel pair.  Returns (median segment's ms per
    step, every segment's ms per step, settle steps)."""
    import torch

    settle = 0
    t_end = time.perf_counter() + SETTLE_S
    while time.perf_counter() < t_end:
        for _ in range(10):
            step(settle)
            settle += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    nseg = max(1, min(TIMED_SEGMENTS, args.steps))
    cuts = [args.steps * j // nseg for j in range(nseg + 1)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nseg + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for j in range(nseg):
        for i in range(cuts[j], cuts[j + 1]):
            step(i)
        ev[j + 1].record(stream)
    torch.cuda.synchronize()
    seg = [ev[j].elapsed_time(ev[j + 1]) / (cuts[j + 1] - cuts[j]) for j in range(nseg)]
    med = sorted(seg)[(nseg - 1) // 2] if nseg % 2 else \
        0.5 * (sorted(seg)[nseg // 2 - 1] + sorted(seg)[nseg // 2])
    return med, seg, settle


def common_fields(args, value, ms, seg, B):
    return {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "us_per_step": round(ms * 1e3, 2),
        "us_per_step_segments": [round(x * 1e3, 2) for x in seg],
        "tokens_per_s": round(B / (ms * 1e-3), 1),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
    }


def main():
    args = parse()
    if args.record_traffic:
        return record_traffic(args)
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the path runs on a single GPU).", file=sys.stderr)
        sys.exit(2)
    import torch

    import decode_attention_kv_attn_amd as L
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.probe:
        return run_probe(dev)
    w = synth.workload(args.workload)
    if w["kind"] == "mla":
        return bench_mla(args, w, dev)
    print(f"bench: workload {w['name']}: drawing inputs", file=sys.stderr, flush=True)
    inp = synth.gqa_inputs(w, dev)
    s = 2 if w.get("dtype", "bf16") == "bf16" else 4
    kv_bytes_cap = inp["k"].numel() * s * 2
    R = max(1, math.ceil(args.rotate_bytes * 2**30 / kv_bytes_cap))
    ks = [inp["k"]] + [inp["k"].clone() for _ in range(R - 1)]
    vs = [inp["v"]] + [inp["v"].clone() for _ in range(R - 1)]
    B, H_q, H_kv, d, T = w["B"], w["H_q"], w["H_kv"], w["d"], w["T_cap"]
    vis = visible_counts(w, inp["seq_lens"])
    alg_bytes = int(2 * s * d * H_kv * int(vis.sum()))
    out = torch.empty(B, H_q, d, dtype=torch.float32, device=dev)
    lse = torch.empty(B, H_q, dtype=torch.float32, device=dev)
    dt_code = L.ATTN_BF16 if s == 2 else L.ATTN_F32
    ring = inp["ring_head"] is not None
    plan = L.attn_decode_gqa_plan(B, H_q, H_kv, T, d, dt_code, inp["window"], ring,
                                  0, args.num_splits)
    ws = torch.empty(max(plan["workspace_bytes"], 1), dtype=torch.uint8, device=dev)
    balanced = bool(plan["balanced_groups"] and inp["seq_lens"] is not None
                    and args.num_splits == 0)
    merged = plan["splits"] > 1 or balanced

    def step(i):
        L.attn_decode_gqa(inp["q"], ks[i % R], vs[i % R], inp["seq_lens"],
                          inp["ring_head"], inp["window"], inp["scale"],
                          args.num_splits, out=out, lse=lse, workspace=ws)

    kernel = "gqa_decode_" + plan["kernel"]
    print(f"bench: {R} cache copies, {plan['splits']} split(s), {kernel}; "
          f"warmup {args.warmup}", file=sys.stderr, flush=True)
    ms, seg, settle = run_timed(step, args, dev)
    value = alg_bytes / (ms * 1e-3) / 1e9
    print(f"bench: {ms * 1e3:.1f} us/step (segments "
          f"{', '.join(f'{x * 1e3:.1f}' for x in seg)}), {value:.0f} GB/s "
          f"(settled over {settle} steps)", file=sys.stderr, flush=True)

    res = common_fields(args, value, ms, seg, B)
    res.update({
        "dtype": "bf16" if s == 2 else "f32",
        "data": "synthetic",
        "config": {"workload": w["name"], "B": B, "H_q": H_q, "H_kv": H_kv,
                   "d": d, "T": T, "window": inp["window"], "ring": ring,
                   "splits": plan["splits"], "balanced_list": balanced,
                   "cache_copies": R, "settle_steps": settle,
                   "kv_bytes_per_step": alg_bytes},
        "roofline": {
            "bound": "hbm",
            "achieved": round(value, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(value / HBM_PEAK_GBS, 4),
            "traffic": traffic_from_profile(w["name"]),
            "kernel": kernel + (f" + {MERGE_KERNEL}_rows" if merged else ""),
            "launches_per_step": 2 if merged else 1,
            "step_us": round(ms * 1e3, 2),
        },
    })
    del ks[1:], vs[1:]
    probe = probe_read_gbs(dev)
    res["read_probe"] = {"GBps": round(probe, 1),
                         "value_pct": round(100 * value / probe, 1)}
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def mla_kernel_name(w, inp, args):
    """The decode kernel a call runs: the 512 + 64 latent's fixed splits go to
    the role-split kernel, ragged batches (the balanced list) and the 256 + 64
    latent to the shared-latent kernel."""
    shared = os.environ.get("ATTN_DECODE_MLA_KERNEL", "")[:1] == "s"
    fixed = inp["seq_lens"] is None or args.num_splits > 0 or w["B"] > 256
    return "mla_pair_decode" if w["d_c"] == 512 and fixed and not shared else "mla_decode_mfma"


def bench_mla(args, w, dev):
    """The absorbed-MLA workload: latent bytes (d_c + d_rope) * s per visible
    position (attention-head section 5.4, Bytes_MLA), both rooflines."""
    import torch

    import decode_attention_kv_attn_amd as L
    import synth

    print(f"bench: workload {w['name']}: drawing inputs", file=sys.stderr, flush=True)
    inp = synth.mla_inputs(w, dev)
    B, H, T = w["B"], w["H"], w["T_cap"]
    dk = w["d_c"] + w["d_rope"]
    lat_bytes = inp["latent"].numel() * 2
    R = max(1, math.ceil(args.rotate_bytes * 2**30 / lat_bytes))
    lats = [inp["latent"]] + [inp["latent"].clone() for _ in range(R - 1)]
    Tsum = B * T if inp["seq_lens"] is None else int(inp["seq_lens"].clamp(0, T).sum())
    alg_bytes = Tsum * dk * 2
    flops = 2 * H * (dk + w["d_c"]) * Tsum
    S = L.attn_decode_mla_splits(B, H, T, w["d_c"], w["d_rope"], args.num_splits)
    wsb = L.attn_decode_mla_workspace_bytes(B, H, T, w["d_c"], w["d_rope"], args.num_splits)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    out = torch.empty(B, H, w["d_c"], dtype=torch.float32, device=dev)
    lse = torch.empty(B, H, dtype=torch.float32, device=dev)

    def step(i):
        L.attn_decode_mla(inp["q"], lats[i % R], inp["d_c"], inp["scale"],
                          inp["seq_lens"], args.num_splits, out=out, lse=lse,
                          workspace=ws)

    ms, seg, settle = run_timed(step, args, dev)
    value = alg_bytes / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    res = common_fields(args, value, ms, seg, B)
    res.update({
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w["name"], "B": B, "H": H, "T": T, "d_c": w["d_c"],
                   "d_rope": w["d_rope"], "splits": S, "cache_copies": R,
                   "settle_steps": settle,
                   "latent_bytes_per_step": alg_bytes, "flops_per_step": flops},
        "roofline": {"bound": "hbm", "achieved": round(value, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile(w["name"], "mla"),
                     "kernel": mla_kernel_name(w, inp, args) +
                               ("" if S == 1 else f" + {MERGE_KERNEL}_rows"),
                     "launches_per_step": 1 if S == 1 else 2,
                     "step_us": round(ms * 1e3, 2)},
        "mfma_roofline": {"achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                          "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                          "note": "algorithmic flops 2*H*(d_c+d_rope+d_c) per position"},
    })
    print(f"bench: {ms * 1e3:.1f} us/step, {value:.0f} GB/s, {tflops:.0f} TFLOP/s",
          file=sys.stderr, flush=True)
    del lats[1:]
    probe = probe_read_gbs(dev)
    res["read_probe"] = {"GBps": round(probe, 1),
                         "value_pct": round(100 * value / probe, 1)}
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline_mla(w, inp, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

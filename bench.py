"""Decode-attention benchmark: KV-read GB/s (% of HBM peak) and us/step.

One step = one library call = one layer's decode attention for every
sequence of the batch.  Inputs are seeded synthetic tensors drawn on the GPU
(``synth``), already resident in HBM when timing starts; several copies of
the cache are rotated so the working set exceeds the 256 MB Infinity Cache.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

prints ONE JSON line.  The default workload is the Llama-3-8B-shaped GQA
layer (B=32, 32 query heads over 8 KV heads, d=128, T=4096, bf16).

``value`` = algorithmic KV bytes per step / measured step time, where the
algorithmic bytes are 2 * s * d * H_kv * (visible positions summed over the
batch) -- only what the method must read (xuesongtap "attention-head" note,
section 1, Bytes_KV), never masked or padded capacity.
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
DEFAULT_WORKLOAD = "llama3_8b_gqa_t4096"
SETTLE_S = 0.3  # seconds of untimed calls before the warmup (clock ramp-up)
KERNEL_SOURCES = {"gqa": ["gqa_valu.hip", "gqa_mfma.hip", "balance.h", "visible.h",
                          "device_common.h", "internal.h"],
                  "mla": ["mla_mfma.hip", "balance.h", "visible.h", "device_common.h",
                          "internal.h"]}


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
    """HBM bytes per launch from committed rocprofv3 --pmc results, if they
    were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_hash") != kernel_source_hash(kind):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, inp, seconds):
    """Time the float64 oracle on the host over a bounded sample of the same
    workload: whole (b, KV-head) units, repeated until `seconds` have passed."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    q = inp["q"].cpu()
    k = inp["k"].cpu()
    v = inp["v"].cpu()
    sl = None if inp["seq_lens"] is None else inp["seq_lens"].cpu()
    rh = None if inp["ring_head"] is None else inp["ring_head"].cpu()
    vis = visible_counts(w, sl)
    s = 2 if w.get("dtype", "bf16") == "bf16" else 4
    unit_bytes = 2 * s * w["d"]
    B, H_kv = w["B"], w["H_kv"]
    units = [(b, g) for b in range(B) for g in range(H_kv)]
    done_bytes = 0
    n_units = 0
    t0 = time.perf_counter()
    i = 0
    while True:
        b, g = units[i % len(units)]
        oracle.gqa_decode_ref(q, k, v, sl, rh, inp["window"], inp["scale"],
                              batches=[b], kv_heads=[g])
        done_bytes += unit_bytes * int(vis[b])
        n_units += 1
        i += 1
        if time.perf_counter() - t0 >= seconds and n_units >= 1:
            break
    dt = time.perf_counter() - t0
    return {"value": done_bytes / dt / 1e9, "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n_units} (sequence, KV-head) units of {w['name']} "
                      f"({len(units)} per step) in {dt:.1f} s, float64 numpy"}


def probe_read_gbs(dev, nbytes=4 << 30, reps=10):
    """Best streaming-read rate of this GPU (attn_probe_read over a buffer far
    larger than the caches), in GB/s."""
    import torch

    import decode_attention_kv_attn_amd as L
    x = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    x.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    best = 0.0
    for blocks in (256 * 8, 256 * 32):
        for _ in range(2):
            L.attn_probe_read(x, sink, blocks)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            L.attn_probe_read(x, sink, blocks)
        e1.record()
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


def _counter_kib_per_dispatch(csv_path, kernel_substr):
    """Mean over dispatches of a kernel (name containing kernel_substr) of the
    counter in a rocprofv3 counter_collection.csv, summed per dispatch."""
    import csv
    per = {}
    name = None
    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            if kernel_substr in row["Kernel_Name"]:
                per[row["Dispatch_Id"]] = per.get(row["Dispatch_Id"], 0.0) + float(row["Counter_Value"])
                name = row["Counter_Name"]
    if not per:
        raise SystemExit(f"no dispatch of {kernel_substr} in {csv_path}")
    return sum(per.values()) / len(per), name, len(per)


def record_traffic(args):
    """HBM bytes per launch of the workload's decode kernel from FETCH_SIZE
    and WRITE_SIZE (KiB per dispatch), each scaled by what the same counter
    reads for the 1 GiB plain copy of --probe, into
    profiles/traffic_<workload>.json with a hash of the kernel sources."""
    import synth
    w = synth.workload(args.workload)
    kind = "mla" if w["kind"] == "mla" else "gqa"
    kern = "mla_decode_mfma" if kind == "mla" else "gqa_decode_"
    d = args.record_traffic
    if not args.copy_dir:
        sys.exit("--record-traffic needs --copy-dir: the --pmc runs of the plain copy")
    fk, _, nf = _counter_kib_per_dispatch(os.path.join(d, "FETCH_SIZE", "run_counter_collection.csv"), kern)
    wk, _, nw = _counter_kib_per_dispatch(os.path.join(d, "WRITE_SIZE", "run_counter_collection.csv"), kern)
    cf, _, _ = _counter_kib_per_dispatch(os.path.join(args.copy_dir, "FETCH_SIZE", "run_counter_collection.csv"), "plain_copy")
    cw, _, _ = _counter_kib_per_dispatch(os.path.join(args.copy_dir, "WRITE_SIZE", "run_counter_collection.csv"), "plain_copy")
    copy_bytes = 1 << 30
    fs, ws = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    if kind == "mla":
        lens = workload_seq_lens(w)
        Tsum = w["B"] * w["T_cap"] if lens is None else int(lens.clamp(0, w["T_cap"]).sum())
        alg = Tsum * (w["d_c"] + w["d_rope"]) * 2
    else:
        s = 2 if w.get("dtype", "bf16") == "bf16" else 4
        alg = int(2 * s * w["d"] * w["H_kv"] * int(visible_counts(w, workload_seq_lens(w)).sum()))
    rec = {
        "workload": w["name"], "kernel": kern + "*",
        "kernel_source_hash": kernel_source_hash(kind),
        "commands": [
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/FETCH_SIZE -o run -- "
            f"python bench.py --workload {w['name']} --steps 3 --warmup 1 --no-cpu-baseline",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/WRITE_SIZE -o run -- "
            f"python bench.py --workload {w['name']} --steps 3 --warmup 1 --no-cpu-baseline",
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {args.copy_dir}/FETCH_SIZE -o run -- python bench.py --probe",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {args.copy_dir}/WRITE_SIZE -o run -- python bench.py --probe",
        ],
        "dispatches": [nf, nw],
        "fetch_kib_per_dispatch_raw": round(fk, 1),
        "write_kib_per_dispatch_raw": round(wk, 1),
        "copy_calibration": {"bytes": copy_bytes, "fetch_kib_raw": round(cf, 1),
                             "write_kib_raw": round(cw, 1), "fetch_scale": round(fs, 4),
                             "write_scale": round(ws, 4)},
        "read_bytes_per_launch": int(fk * 1024 * fs),
        "write_bytes_per_launch": int(wk * 1024 * ws),
        "bytes_per_launch": int(fk * 1024 * fs + wk * 1024 * ws),
        "algorithmic_bytes_per_launch": alg,
    }
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


def run_timed(step, args, dev):
    """Settle, warm up, then time exactly args.steps calls of step(i).

    The settle phase runs the same step for at least SETTLE_S seconds before
    the warmup, so the memory and core clocks have left their idle states
    when the timed region starts.  The timed region is bracketed by one HIP
    event pair on the launch stream and nothing else: an event pair around
    every call costs the GPU about 3.5 us per event (measured), which would
    inflate short steps by up to 15 %.  Each step launches the decode kernel
    once (plus its merge when the plan splits), so the region's mean step
    time is also the average launch period of that kernel pair.  Returns
    (ms per step, settle steps)."""
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
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / args.steps, settle


def main():
    args = parse()
    if args.record_traffic:
        return record_traffic(args)
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the path runs on a single GPU).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
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
    S = L.attn_decode_gqa_splits(B, H_q, H_kv, T, d, dt_code, inp["window"],
                                 ring, args.num_splits)
    wsb = L.attn_decode_gqa_workspace_bytes(B, H_q, H_kv, T, d, dt_code,
                                            inp["window"], ring, args.num_splits)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)

    def step(i):
        L.attn_decode_gqa(inp["q"], ks[i % R], vs[i % R], inp["seq_lens"],
                          inp["ring_head"], inp["window"], inp["scale"],
                          args.num_splits, out=out, lse=lse, workspace=ws)

    plan = L.attn_decode_gqa_plan(B, H_q, H_kv, T, d, dt_code, inp["window"], ring,
                                  0, args.num_splits)
    kernel = "gqa_decode_" + plan["kernel"]
    print(f"bench: {R} cache copies, {S} split(s), {kernel}; warmup {args.warmup}",
          file=sys.stderr, flush=True)
    ms_per_step, settle = run_timed(step, args, dev)
    call_ms = ms_per_step
    value = alg_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = alg_bytes / (call_ms * 1e-3) / 1e9
    print(f"bench: {ms_per_step * 1e3:.1f} us/step, call {call_ms * 1e3:.1f} us, "
          f"{value:.0f} GB/s (settled over {settle} steps)", file=sys.stderr, flush=True)

    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "tokens_per_s": round(B / (ms_per_step * 1e-3), 1),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if s == 2 else "f32",
        "data": "synthetic",
        "config": {"workload": w["name"], "B": B, "H_q": H_q, "H_kv": H_kv,
                   "d": d, "T": T, "window": inp["window"], "ring": ring,
                   "splits": S,
                   "balanced_list": bool(plan["balanced_groups"] and inp["seq_lens"] is not None
                                         and args.num_splits == 0),
                   "cache_copies": R, "settle_steps": settle,
                   "kv_bytes_per_step": alg_bytes},
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_from_profile(w["name"]),
            "kernel": kernel + ("" if S == 1 else " + lse_combine"),
            "kernel_us": round(call_ms * 1e3, 2),
        },
    }
    del ks[1:], vs[1:]
    probe = probe_read_gbs(dev)
    res["read_probe"] = {"GBps": round(probe, 1),
                         "value_pct": round(100 * value / probe, 1),
                         "achieved_pct": round(100 * achieved / probe, 1)}
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
        # the same oracle on one BLAS thread, over a shorter sample
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                one = cpu_baseline(w, inp, args.cpu_seconds / 2)
            res["cpu_baseline_1thread"] = {k: one[k] for k in ("value", "unit", "cores", "sample")}
        except ImportError:  # pragma: no cover
            pass
    print(json.dumps(res), flush=True)


def bench_mla(args, w, dev):
    """The absorbed-MLA workload: latent bytes (d_c + d_rope) * s per visible
    position (attention-head section 5.4, Bytes_MLA), both rooflines."""
    import numpy as np
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

    ms, settle = run_timed(step, args, dev)
    call_ms = ms
    value = alg_bytes / (ms * 1e-3) / 1e9
    tflops = flops / (call_ms * 1e-3) / 1e12
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "us_per_step": round(ms * 1e3, 2), "tokens_per_s": round(B / (ms * 1e-3), 1),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w["name"], "B": B, "H": H, "T": T, "d_c": w["d_c"],
                   "d_rope": w["d_rope"], "splits": S, "cache_copies": R,
                   "settle_steps": settle,
                   "latent_bytes_per_step": alg_bytes, "flops_per_step": flops},
        "roofline": {"bound": "hbm", "achieved": round(alg_bytes / (call_ms * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(alg_bytes / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile(w["name"], "mla"),
                     "kernel": "mla_decode_mfma" + ("" if S == 1 else " + lse_combine"),
                     "kernel_us": round(call_ms * 1e3, 2)},
        "mfma_roofline": {"achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                          "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                          "note": "algorithmic flops 2*H*(d_c+d_rope+d_c) per position; "
                                  "the kernel issues %.2fx that (bf16 hi+lo weights)"
                                  % ((3 * w["d_c"] + w["d_rope"]) / (2 * w["d_c"] + w["d_rope"]))},
    }
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


def cpu_baseline_mla(w, inp, seconds):
    """The float64 MLA oracle on the host over whole sequences of the
    workload, repeated until `seconds` have passed."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    q = inp["q"].cpu()
    lat = inp["latent"].cpu()
    sl = None if inp["seq_lens"] is None else inp["seq_lens"].cpu()
    B, T = w["B"], w["T_cap"]
    row_bytes = (w["d_c"] + w["d_rope"]) * 2
    done, n, i = 0, 0, 0
    t0 = time.perf_counter()
    while True:
        b = i % B
        oracle.mla_decode_ref(q, lat, w["d_c"], w["scale"], sl, batches=[b])
        done += row_bytes * (T if sl is None else int(sl[b].clamp(0, T)))
        n += 1
        i += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": done / dt / 1e9, "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n} sequences of {w['name']} ({B} per step) in {dt:.1f} s, "
                      "float64 numpy"}


if __name__ == "__main__":
    main()

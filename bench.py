#!/usr/bin/env python3
"""Throughput of the fused-softmax MX attention forward on one MI355X.

One step = one call of ``fsa_attention_fwd`` on the 16K-token Video-DiT-shaped
workload (B=1, H=40, S=16384, D=128, non-causal, MXFP8 E4M3): MX quantisation
of Q, K, V plus the fused attention kernel, inputs resident in HBM.  The same
inputs are also timed with E2M3 and E2M1 operands and through the BF16
flash-attention baseline, and under causal masking; the outlier workload
(MXFP4, S=32768, planted +8 sigma scores) and the long hybrid FP6/FP4
schedule (S=75600) are timed as well ("workloads" in the JSON line), and the
P~ variants of fsa_options.p_variant on the Video-DiT tensors ("variants";
an E4M3 P~ over FP6/FP4 operands is rated against the MXFP8 peak, since half
its products run at FP8 width).  FLOPs are 4*B*H*S^2*D (halved for causal).

Prints ONE JSON line.  Options:
  --gpus N        only 1 is supported (the path is a single-GPU kernel)
  --steps K       timed steps (default 20)
  --warmup W      untimed steps first (default 10: the first launches after
                  idle run up to 30 % slower while the clock settles)
  --no-cpu        skip the CPU-oracle baseline
  --no-extra      skip the other workloads (outliers, hybrid, causal)
  --only FMT      time only one element format (e4m3, e2m3, e2m1)
  --workload NAME time another workload of workloads.py instead (its own
                  formats, per head for the hybrid schedule) and print one
                  JSON line for it; no BF16 or CPU legs
  --copy-bytes N  also run one plain device copy of N bytes (counter calibration)
  --write-traffic FETCH_DB WRITE_DB
                  no timing: read two rocprofv3 --pmc result databases (one
                  with FETCH_SIZE, one with WRITE_SIZE) of a run with
                  --copy-bytes, scale the fused kernel's per-dispatch counters
                  by the copy kernel's bytes-per-count, and write
                  profiles/fsa_fwd_traffic.json (tagged with the kernel-source
                  hash, so a later kernel change invalidates it)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"e4m3": 5000.0, "e2m3": 10100.0, "e2m1": 10100.0, "bf16": 2500.0}
METRIC = "attention fwd TFLOP/s and % of MX MFMA peak (MXFP8/6/4, S=16K, D=128)"
KERNEL_SOURCES = ("softmax_mx_quantize_amd/csrc/fsa_common.h",
                  "softmax_mx_quantize_amd/csrc/fsa_attn.h",
                  "softmax_mx_quantize_amd/csrc/fsa_fwd.hip",
                  "softmax_mx_quantize_amd/csrc/fsa_internal.h",
                  "softmax_mx_quantize_amd/csrc/fsa_device.h",
                  "softmax_mx_quantize_amd/csrc/lds_dma.h")


def kernel_hash() -> str:
    """Hash of the kernel sources' code: comments and whitespace are left
    out, so that editing a comment does not invalidate stored counters."""
    import re
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def stored_traffic(fmt: str):
    """HBM traffic per launch measured with rocprofv3 counters, if the kernel
    source is unchanged since the measurement."""
    p = os.path.join(ROOT, "profiles", "fsa_fwd_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("kernel_hash") != kernel_hash():
        return None
    return d.get("bytes_per_launch", {}).get(fmt)


# fsa_fwd_kernel<FSET, PM, PX, D, CAUSAL, REBASE>: FSET is the set of formats
# the launch holds (bit 0 E4M3, bit 1 E2M3, bit 2 E2M1), PM the P~ variant,
# PX 1 for E4M3 P~ over FP6/FP4 operands.
FMT_OF_FSET = {1: "e4m3", 2: "e2m3", 4: "e2m1"}


def traffic_key(kernel_name: str) -> str:
    """Key of profiles/fsa_fwd_traffic.json for one fused-kernel instance:
    the format for the default P~ map of a one-format launch, else a tag
    naming the format set and the variant."""
    args = [a.strip() for a in kernel_name.split("fsa_fwd_kernel<")[1].split(">")[0].split(",")]
    fset, pm, px = int(args[0]), int(args[1]), int(args[2])
    if pm == 0 and px == 0 and fset in FMT_OF_FSET:
        return FMT_OF_FSET[fset]
    return "fset%d_pm%d_px%d" % (fset, pm, px)


def _pmc_per_kernel(db_path: str, counter: str):
    """Average per-dispatch value of `counter` (summed over its instances)
    for each kernel name in a rocprofv3 results database."""
    import sqlite3
    import collections
    db = sqlite3.connect(db_path)
    rows = db.execute("select dispatch_id, kernel_name, counter_name, value "
                      "from counters_collection").fetchall()
    per_dispatch = collections.defaultdict(float)
    names = {}
    for did, kn, cn, val in rows:
        if cn == counter:
            per_dispatch[did] += val
            names[did] = kn
    by_kernel = collections.defaultdict(list)
    for did, v in per_dispatch.items():
        by_kernel[names[did]].append(v)
    return {k: sum(v) / len(v) for k, v in by_kernel.items()}


def write_traffic(fetch_db: str, write_db: str, copy_bytes: int) -> dict:
    fetch = _pmc_per_kernel(fetch_db, "FETCH_SIZE")
    write = _pmc_per_kernel(write_db, "WRITE_SIZE")
    copy = [k for k in fetch if "neg_kernel" in k]
    if len(copy) != 1:
        raise RuntimeError("expected one copy (neg) kernel in the counter run, found %r" % copy)
    # FETCH_SIZE / WRITE_SIZE are in KiB; the copy reads and writes copy_bytes
    f_scale = copy_bytes / (fetch[copy[0]] * 1024.0)
    w_scale = copy_bytes / (write[copy[0]] * 1024.0)
    out = {"kernel_hash": kernel_hash(), "copy_bytes": copy_bytes,
           "fetch_bytes_per_count_byte": f_scale, "write_bytes_per_count_byte": w_scale,
           "bytes_per_launch": {}, "fetch_bytes": {}, "write_bytes": {}}
    # a call launches the kernel twice (the sweep, then the re-based pass
    # that exits at once unless a row is beyond its reach): both count
    for k in fetch:
        if "fsa_fwd_kernel<" not in k:
            continue
        fmt = traffic_key(k)
        fb = fetch[k] * 1024.0 * f_scale
        wb = write.get(k, 0.0) * 1024.0 * w_scale
        out["fetch_bytes"][fmt] = out["fetch_bytes"].get(fmt, 0.0) + fb
        out["write_bytes"][fmt] = out["write_bytes"].get(fmt, 0.0) + wb
        out["bytes_per_launch"][fmt] = out["bytes_per_launch"].get(fmt, 0.0) + fb + wb
    with open(os.path.join(ROOT, "profiles", "fsa_fwd_traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
    return out


def time_fsa(fsa, torch, q, k, v, fmt, steps, warmup, causal=False, **kw):
    """Whole-step time (ms) and fused-kernel time (ms).  The whole steps run
    back to back with nothing between them; the kernel time comes from a
    second run of the same steps with HIP events on the stream the library
    launches on (recorded by the library between the quantisation and the
    attention kernels, and after the call), because each timing event
    leaves the GPU idle for a few microseconds."""
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fsa.attention_fwd(q, k, v, fmt, causal, out=out, **kw)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fsa.attention_fwd(q, k, v, fmt, causal, out=out, **kw)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    mids = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for m in mids:          # create the underlying HIP events before the library records them
        m.record(stream)
    torch.cuda.synchronize()
    for i in range(steps):
        fsa.attention_fwd(q, k, v, fmt, causal, out=out, event_after_quantize=mids[i], **kw)
        ends[i].record(stream)
    torch.cuda.synchronize()
    kern_ms = sum(m.elapsed_time(e) for m, e in zip(mids, ends)) / steps
    return wall_ms, kern_ms, out


def time_bf16(fsa, torch, q, k, v, steps, warmup):
    out = torch.empty_like(q)
    for _ in range(warmup):
        fsa.attention_bf16_ref(q, k, v, False, out=out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fsa.attention_bf16_ref(q, k, v, False, out=out)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def cpu_baseline(w, budget_s: float = 15.0):
    """The oracle as it stands, on a bounded sample: all keys for a growing
    number of query rows of head 0, until about `budget_s` seconds of work."""
    import numpy as np
    import workloads as W
    import oracle as O
    q, k, v = (W.bf16_bits_to_f64(x) for x in W.generate_head(w, 0, 0))
    rows_done, t_used, n = 0, 0.0, 8
    rng = np.random.default_rng(0)
    while t_used < budget_s:
        rows = np.sort(rng.choice(w.S, n, replace=False))
        t0 = time.perf_counter()
        O.fused_attention(q, k, v, w.head_fmts[0], w.causal, rows=rows)
        t_used += time.perf_counter() - t0
        rows_done += n
        n = min(2 * n, 256)
    flops = 4.0 * rows_done * w.S * w.D
    try:
        cores = len(os.sched_getaffinity(0))
    except Exception:
        cores = os.cpu_count()
    return {
        "value": flops / t_used / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": "%d query rows of head 0 against all %d keys (float64 numpy oracle incl. "
                  "MX quantisation of that head's K and V per call), %.1f s" % (rows_done, w.S, t_used),
    }


EXTRA_WORKLOADS = ("outliers_e2m1", "hybrid_long", "video_dit_e4m3_causal")


def bench_workload(name: str, steps: int, warmup: int, tensors=None) -> dict:
    """Whole-call and kernel TFLOP/s of one workload in its own formats
    (per head for the hybrid schedule), inputs resident in HBM."""
    import numpy as np
    import torch
    import softmax_mx_quantize_amd as fsa
    import workloads as W
    w = W.WORKLOADS[name]
    if tensors is None:
        print("[bench] generating %s inputs" % w.name, file=sys.stderr, flush=True)
        qb, kb, vb = W.generate(w, workers=16)
        dev = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        q, k, v = dev(qb), dev(kb), dev(vb)
        del qb, kb, vb
    else:
        q, k, v = tensors
    print("[bench] timing %s" % w.name, file=sys.stderr, flush=True)
    hf = list(w.head_fmts)
    kw = {} if len(set(hf)) == 1 else {"head_fmt": hf}
    wall_ms, kern_ms, _ = time_fsa(fsa, torch, q, k, v, hf[0], steps, warmup, w.causal, **kw)
    # the hybrid heads run at the FP6/FP4 peak (both 10.1 PFLOP/s)
    peak = max(PEAK_TFLOPS[f] for f in hf)
    return {"workload": w.name, "B": w.B, "H": w.H, "S": w.S, "D": w.D, "causal": w.causal,
            "head_fmts": sorted(set(hf)), "steps": steps, "warmup": warmup,
            "ms_per_step": wall_ms, "tflops": w.flops / (wall_ms * 1e-3) / 1e12,
            "kernel_ms": kern_ms, "kernel_tflops": w.flops / (kern_ms * 1e-3) / 1e12,
            "kernel_frac_of_peak": w.flops / (kern_ms * 1e-3) / 1e12 / peak, "peak_tflops": peak}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--only", default=None)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DB", "WRITE_DB"))
    args = ap.parse_args()
    if args.write_traffic:
        if not args.copy_bytes:
            print("bench.py: --write-traffic needs the --copy-bytes of the counter run", file=sys.stderr)
            return 2
        print(json.dumps(write_traffic(*args.write_traffic, args.copy_bytes)))
        return 0
    if args.gpus != 1:
        print("bench.py: only --gpus 1 is supported; the fused attention path runs on one GPU "
              "(heads shard across GPUs with no communication, see the design notes)",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import softmax_mx_quantize_amd as fsa
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    if args.workload:
        print(json.dumps(bench_workload(args.workload, args.steps, args.warmup)), flush=True)
        return 0
    w = W.WORKLOADS["video_dit_e4m3"]
    print("[bench] generating %s inputs" % w.name, file=sys.stderr, flush=True)
    qb, kb, vb = W.generate(w)
    dev = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = dev(qb), dev(kb), dev(vb)
    flops = w.flops

    fmts = [args.only] if args.only else ["e4m3", "e2m3", "e2m1"]
    per = {}
    for fmt in fmts:
        print("[bench] timing fused %s" % fmt, file=sys.stderr, flush=True)
        wall_ms, kern_ms, _ = time_fsa(fsa, torch, q, k, v, fmt, args.steps, args.warmup)
        per[fmt] = {
            "ms_per_step": wall_ms,
            "tflops": flops / (wall_ms * 1e-3) / 1e12,
            "kernel_ms": kern_ms,
            "kernel_tflops": flops / (kern_ms * 1e-3) / 1e12,
            "kernel_frac_of_peak": flops / (kern_ms * 1e-3) / 1e12 / PEAK_TFLOPS[fmt],
            "peak_tflops": PEAK_TFLOPS[fmt],
        }
    bf16 = None
    if not args.only:
        print("[bench] timing bf16 baseline", file=sys.stderr, flush=True)
        bms = time_bf16(fsa, torch, q, k, v, args.steps, args.warmup)
        bf16 = {"ms_per_step": bms, "tflops": flops / (bms * 1e-3) / 1e12,
                "frac_of_peak": flops / (bms * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"]}
        for fmt in fmts:
            per[fmt]["speedup_vs_bf16"] = bms / per[fmt]["ms_per_step"]

    # the P~ variants on the same inputs (kernel time: quantisation excluded)
    variants = {}
    if not args.only and not args.no_extra:
        for vname, fmt in (("row", "e4m3"), ("e4m3", "e2m3"), ("e4m3", "e2m1"), ("e3m2", "e2m3"),
                           ("affine", "e2m1"),
                           ("exact_exp", "e4m3"), ("exact_exp", "e2m3"), ("exact_exp", "e2m1")):
            print("[bench] timing variant %s over %s" % (vname, fmt), file=sys.stderr, flush=True)
            wall_ms, kern_ms, _ = time_fsa(fsa, torch, q, k, v, fmt, args.steps, args.warmup,
                                           p_variant=vname)
            # peak of the narrower of the two product formats the variant runs
            peak = PEAK_TFLOPS["e4m3" if (fmt == "e4m3" or vname == "e4m3") else fmt]
            variants["%s-%s" % (vname, fmt)] = {
                "ms_per_step": wall_ms, "tflops": flops / (wall_ms * 1e-3) / 1e12,
                "kernel_ms": kern_ms, "kernel_tflops": flops / (kern_ms * 1e-3) / 1e12,
                "kernel_frac_of_peak": flops / (kern_ms * 1e-3) / 1e12 / peak, "peak_tflops": peak}

    # the other workloads of the method: planted outliers (fallbacks),
    # the long hybrid FP6/FP4 schedule, and causal masking
    extra = {}
    if not args.only and not args.no_extra:
        extra["video_dit_e4m3_causal"] = bench_workload("video_dit_e4m3_causal", args.steps,
                                                        args.warmup, tensors=(q, k, v))
        for name in ("outliers_e2m1", "hybrid_long"):
            extra[name] = bench_workload(name, args.steps, args.warmup)
            torch.cuda.empty_cache()

    if args.copy_bytes:
        # a plain streaming kernel of known traffic: reads and writes copy_bytes
        n = args.copy_bytes // 4
        a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.neg(a, out=b)
        torch.cuda.synchronize()

    head = fmts[0]
    res = per[head]
    traffic = stored_traffic(head)
    line = {
        "metric": METRIC,
        "value": res["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"e4m3": "mxfp8_e4m3", "e2m3": "mxfp6_e2m3", "e2m1": "mxfp4_e2m1"}[head],
        "data": "synthetic (seeded N(0,1) bf16, per-head gain U[0.5,2] on q and k)",
        "config": {"workload": w.name if head == "e4m3" else "video_dit_" + head,
                   "B": w.B, "H": w.H, "S": w.S, "D": w.D, "causal": w.causal,
                   "fmt": head, "seed": w.seed},
        "roofline": {
            "bound": "mfma",
            "achieved": res["kernel_tflops"],
            "peak": PEAK_TFLOPS[head],
            "unit": "TFLOP/s",
            "frac": res["kernel_frac_of_peak"],
            "traffic": traffic,
        },
        "formats": per,
        "bf16_baseline": bf16,
        "workloads": extra,
        "variants": variants,
    }
    if not args.no_cpu:
        print("[bench] cpu oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

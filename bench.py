#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  * attn_fwd on the MHA causal prefill workload (B=4, Hq=Hkv=32, N=8192,
    d=128, bf16), and
  * attn_decode_paged on the paged decode workload (16 sequences of
    8000..32000 cached tokens, Hq=32, Hkv=8, d=128, 16-token blocks in a
    40000-block pool).

Prints ONE JSON line.  `value` is the prefill throughput in TFLOP/s
(causal-adjusted: 4*d FLOPs per visible query/key pair), timed with HIP events
around each launch on the stream the kernels run on; the decode throughput in
GB/s of algorithmic HBM bytes is reported beside it.  `roofline` is for the
prefill kernel (bound: bf16 MFMA), `decode.roofline` for the decode kernels
(bound: HBM).  `cpu_baseline` times the fp64 oracle on a bounded sample (16
(batch, head) pairs of the prefill workload) on the host cores and scales it
to TFLOP/s.

`traffic` is the measured HBM bytes per launch, read from profiles/traffic.json
when that file was written for the kernel sources as they are now (a hash of
the sources is stored with it).  `--traffic-from DIR` writes that file from
four rocprofv3 --pmc runs under DIR (fetch/, write/ of this bench, and
copy_fetch/, copy_write/ of `--mode copy`): each counter is scaled by what it
reads for the plain 1 GiB device copy.

The backward pass (attn_bwd, the gradients of the same prefill workload for a
seeded dO) is timed after the steps, on its own, and reported under
`backward` (TFLOP/s counting 2.5x the forward's flops, against the bf16 MFMA
peak); it is not part of the step.  --skip-backward leaves it out.

The packed-sequence forward (attn_fwd_varlen on 65536 tokens of sequences
averaging about 600 tokens, at most 2048, 32 heads of 128, causal per
sequence) is timed the same way and reported under `varlen`, with the
fraction of a padded batch's work that would be useful (each sequence padded
to 2048), and its backward (attn_bwd_varlen, 2.5x the forward's flops).
--skip-varlen leaves both out.

The merge of two partial results (attn_merge) at the prefill shape is reported
under `merge` in GB/s of algorithmic bytes (two O and LSE read, one written).

The fp32 single-head case (attn_fwd_f32, 1 x 256 x 1 x 64, non-causal) is
timed in microseconds under `f32_single_head` (launch-latency bound).

Chunked prefill over the paged cache (attn_prefill_paged: the decode batch's
16 sequences of 8000..32000 cached tokens, each taking 512 new tokens) is
reported under `prefill_paged` the same way; --skip-prefill-paged leaves it out.

With the CPU baseline on, the backward, packed and chunked-prefill objects
carry their own `cpu_baseline`: the fp64 oracle timed on a bounded sample of
that workload (one head, sixteen sequences, one sequence), scaled by the
sample's flops.

The other dense configurations are timed alone after the step and reported
as objects of their own, each with TFLOP/s (causal- or window-adjusted
flops), its roofline fraction and a `cpu_baseline` (the oracle on 2 (batch,
head) pairs, scaled): `gqa_causal_16k` (B=2, Hq=32, Hkv=8, N=16384),
`mqa_causal_16k` (Hkv=1) and `swa_causal_32k_w4096` (B=1, Hq=32, Hkv=8,
N=32768, W=4096).  --skip-dense-extra leaves them out.

Other workloads can be timed with --workload NAME (one of the dense configs);
the default line is the one described above.
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

METRIC = "attn fwd TFLOP/s + % bf16 MFMA peak; paged decode HBM GB/s + % peak"
PREFILL = "mha_causal_8k"
DECODE = "paged_decode_16x32k"
PACKED = "packed_causal_64k_mean600"
PREFILL_PAGED = "paged_prefill_16x32k_chunk512"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "exact_softmax_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(key, files):
    """HBM bytes per launch from committed PMC counters, if they match the source."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(key)
    if not ent or ent.get("source_hash") != kernel_source_hash(files):
        return None
    return ent.get("bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # after an idle spell the GPU's clock ramps up over the first 10-15 launches
    # (about 20-40 ms of work); 25 untimed steps put every timed region past it
    ap.add_argument("--warmup", type=int, default=25)
    ap.add_argument("--workload", default=None,
                    help="time only this dense workload's forward (extra lines)")
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--skip-backward", action="store_true")
    ap.add_argument("--skip-varlen", action="store_true")
    ap.add_argument("--skip-prefill-paged", action="store_true")
    ap.add_argument("--skip-dense-extra", action="store_true",
                    help="leave out the GQA/MQA 16K and sliding-window 32K objects")
    ap.add_argument("--mode", choices=["bench", "copy", "stream", "ceiling"], default="bench",
                    help="copy: a plain device copy of known size (counter calibration); "
                         "stream: a contiguous read of the decode workload's byte count "
                         "(the memory system's rate for a plain streaming read); "
                         "ceiling: the read_ceiling program (contiguous, random-block and "
                         "per-KV-head-slice reads of the decode workload's bytes)")
    ap.add_argument("--traffic-from", default=None, metavar="DIR",
                    help="write profiles/traffic.json from rocprofv3 --pmc runs under DIR "
                         "(no GPU needed)")
    return ap.parse_args()


FWD_FILES = ["fwd_bf16.hip", "device_common.h", "launch.h"]
DECODE_FILES = ["decode_paged.hip", "device_common.h", "launch.h"]
COPY_BYTES = 1 << 30


def _pmc_means(path, counter):
    """Mean counter value per dispatch, by kernel name, from a rocprofv3 counter CSV dir."""
    import csv
    import glob
    sums, counts = {}, {}
    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"bench: no counter_collection.csv under {path}")
    for fn in files:
        with open(fn) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                name = row["Kernel_Name"]
                sums[name] = sums.get(name, 0.0) + float(row["Counter_Value"])
                counts[name] = counts.get(name, 0) + 1
    return {n: sums[n] / counts[n] for n in sums}


def _pick(means, key):
    hits = [v for n, v in means.items() if key in n]
    if len(hits) != 1:
        raise SystemExit(f"bench: expected one kernel matching {key!r}, found {len(hits)}")
    return hits[0]


def write_traffic(src_dir):
    """HBM bytes per launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch) runs.

    Each counter is scaled so that it reads the true byte count for a plain
    1 GiB device-to-device copy (the runtime's copy kernel) measured the same way.
    """
    fetch = _pmc_means(os.path.join(src_dir, "fetch"), "FETCH_SIZE")
    write = _pmc_means(os.path.join(src_dir, "write"), "WRITE_SIZE")
    cfetch = _pick(_pmc_means(os.path.join(src_dir, "copy_fetch"), "FETCH_SIZE"), "copyBuffer")
    cwrite = _pick(_pmc_means(os.path.join(src_dir, "copy_write"), "WRITE_SIZE"), "copyBuffer")
    f_fetch = COPY_BYTES / (cfetch * 1024.0)
    f_write = COPY_BYTES / (cwrite * 1024.0)
    out = {"calibration": {"copy_bytes": COPY_BYTES, "fetch_kib": cfetch, "write_kib": cwrite,
                           "fetch_factor": round(f_fetch, 4), "write_factor": round(f_write, 4)}}
    # the dense forward: fwd_bf16_kernel<head dim, scale > 0, dense mode>
    groups = {f"fwd:{PREFILL}": (["fwd_bf16_kernel<128, true, 0>"], FWD_FILES),
              f"decode:{DECODE}": (["decode_split_kernel", "decode_combine_kernel"],
                                   DECODE_FILES)}
    for key, (kernels, files) in groups.items():
        rd = sum(_pick(fetch, kn) for kn in kernels) * 1024.0 * f_fetch
        wr = sum(_pick(write, kn) for kn in kernels) * 1024.0 * f_write
        out[key] = {"kernels": kernels, "fetch_bytes": round(rd), "write_bytes": round(wr),
                    "bytes_per_launch": round(rd + wr), "source_hash": kernel_source_hash(files)}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def cpu_baseline(q, k, v, cfg, n_heads=16):
    """Time the fp64 oracle on `n_heads` (batch, head) pairs (all rows); scale to TFLOP/s."""
    import numpy as np
    import oracle
    from exact_softmax_attention_amd import metrics
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()
                        if i.get("user_api") == "blas"), default=1)
    except Exception:  # pragma: no cover
        threads = 1
    total = cfg.B * cfg.Hq
    step = max(1, total // n_heads)
    heads = [divmod(i, cfg.Hq) for i in range(0, total, step)][:n_heads]
    t0 = time.perf_counter()
    oracle.attention(q, k, v, cfg.scale, cfg.causal, cfg.window, heads=heads)
    dt = time.perf_counter() - t0
    flops = 4.0 * cfg.d * metrics.visible_pairs(cfg.Nq, cfg.Nk, cfg.causal, cfg.window) * len(heads)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{len(heads)} of {cfg.B * cfg.Hq} (batch, head) pairs of {cfg.name}, all "
                      f"{cfg.Nq} rows, fp64 NumPy materialising S and P; {dt:.2f} s, scaled by "
                      "causal-adjusted FLOPs",
            "seconds": round(dt, 3), "host_cpus": len(os.sched_getaffinity(0))}


def cpu_sample(fn, flops, sample):
    """Time one call of an oracle function on a bounded sample; its flops -> TFLOP/s."""
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()
                        if i.get("user_api") == "blas"), default=1)
    except Exception:  # pragma: no cover
        threads = 1
    t0 = time.perf_counter()
    fn()
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "sample": sample, "seconds": round(dt, 3)}


EXTRA_DENSE = ("gqa_causal_16k", "mqa_causal_16k", "swa_causal_32k_w4096")


def dense_object(name, args, torch, dev):
    """One more dense forward workload, timed alone: TFLOP/s, roofline, CPU baseline."""
    import workloads
    from exact_softmax_attention_amd import attn_fwd, metrics
    cfg = workloads.DENSE_CONFIGS[name]
    print(f"bench: {name}", file=sys.stderr, flush=True)
    q, k, v = workloads.make_dense_config(cfg)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty_like(qd)
    lse = torch.empty((cfg.B, cfg.Hq, cfg.Nq), dtype=torch.float32, device=dev)

    def fwd():
        attn_fwd(qd, kd, vd, causal=cfg.causal, window=cfg.window, scale=cfg.scale, out=out,
                 lse=lse)

    per, _ = time_loop([fwd], args.steps, args.warmup, torch)
    flops = metrics.fwd_flops(cfg.B, cfg.Hq, cfg.Nq, cfg.Nk, cfg.d, cfg.causal, cfg.window)
    tf = flops / (per[0] * 1e-3) / 1e12
    obj = {"value": round(tf, 2), "unit": "TFLOP/s", "ms": round(per[0], 4),
           "config": {"B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "N": cfg.Nq, "d": cfg.d,
                      "causal": cfg.causal, "window": cfg.window, "seed": cfg.seed},
           "flop_per_launch": flops,
           "roofline": {"bound": "mfma", "achieved": round(tf, 2),
                        "peak": metrics.PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tf / metrics.PEAK_BF16_TFLOPS, 4),
                        "traffic": measured_traffic(f"fwd:{name}", FWD_FILES),
                        "kernel": "fwd_bf16_kernel<128>",
                        "algorithmic_bytes": metrics.fwd_bytes(cfg.B, cfg.Hq, cfg.Hkv, cfg.Nq,
                                                               cfg.Nk, cfg.d)}}
    del qd, kd, vd, out, lse
    torch.cuda.empty_cache()
    if not args.skip_cpu_baseline:
        obj["cpu_baseline"] = cpu_baseline(q, k, v, cfg, n_heads=2)
    return obj


def time_loop(fns, steps, warmup, torch):
    """Run each fn once per step; per-fn average ms from HIP events, total wall ms."""
    for _ in range(warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        ev[s][0].record()
        for i, f in enumerate(fns):
            f()
            ev[s][i + 1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    per = [sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)) / steps
           for i in range(len(fns))]
    return per, wall


def main():
    args = parse()
    if args.traffic_from:
        write_traffic(args.traffic_from)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU layout is described, not built", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    from exact_softmax_attention_amd import (attn_bwd, attn_bwd_workspace_size,
                                             attn_decode_paged, attn_fwd, metrics)

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")

    if args.mode == "ceiling":
        # a program of its own (built with the library), run as a child process
        import subprocess
        from exact_softmax_attention_amd.build import CEILING_BIN
        if not os.path.exists(CEILING_BIN):
            print(f"bench.py: {CEILING_BIN} is missing: run the build first", file=sys.stderr)
            sys.exit(1)
        out = subprocess.run([CEILING_BIN], capture_output=True, text=True)
        if out.returncode != 0:
            print(out.stderr, file=sys.stderr)
            sys.exit(out.returncode)
        res = json.loads(out.stdout.strip().splitlines()[-1])
        res = {"mode": "ceiling", **res,
               "of_peak": {k: round(v / metrics.PEAK_HBM_GBS, 4) for k, v in res.items()
                           if k.endswith("GBps")}}
        print(json.dumps(res))
        return

    if args.mode == "copy":
        n = COPY_BYTES
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "copy", "bytes_read": n, "bytes_written": n,
                          "launches": max(1, args.steps)}))
        return

    if args.mode == "stream":
        # the decode workload's algorithmic bytes moved by plain torch kernels:
        # reductions reading them once, and a device copy of half of them (the
        # same bytes, half read and half written); the fastest is what the
        # memory system gives a plain contiguous stream
        import workloads as _w
        pc = _w.PAGED_CONFIGS[DECODE]
        nbytes = metrics.decode_bytes(_w.paged_seq_lens(pc), pc.Hq, pc.Hkv, pc.d, pc.block_size)
        x = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        acc = torch.empty((), dtype=torch.float32, device=dev)
        half = torch.empty(x.numel() // 2, dtype=torch.float32, device=dev)
        kinds = {"sum": lambda: torch.sum(x, dim=0, out=acc),
                 "amax": lambda: torch.amax(x, dim=0, out=acc),
                 "copy": lambda: half.copy_(x[: half.numel()])}
        res = {"mode": "stream", "bytes": int(x.numel() * 4)}
        for kind, fn in kinds.items():
            per, _ = time_loop([fn], max(5, args.steps), max(2, args.warmup), torch)
            moved = x.numel() * 4 if kind != "copy" else half.numel() * 8
            res[kind] = {"ms": round(per[0], 4),
                         "GB/s": round(moved / (per[0] * 1e-3) / 1e9, 1)}
        best = max(v["GB/s"] for k, v in res.items() if isinstance(v, dict))
        res["best_GB/s"] = best
        res["of_peak"] = round(best / metrics.PEAK_HBM_GBS, 4)
        print(json.dumps(res))
        return

    name = args.workload or PREFILL
    cfg = workloads.DENSE_CONFIGS[name]
    print(f"bench: generating {name}", file=sys.stderr, flush=True)
    q, k, v = workloads.make_dense_config(cfg)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    if cfg.dtype != "bf16":
        raise SystemExit("bench: the prefill line is the bf16 kernel")
    out = torch.empty_like(qd)
    lse = torch.empty((cfg.B, cfg.Hq, cfg.Nq), dtype=torch.float32, device=dev)

    def fwd():
        attn_fwd(qd, kd, vd, causal=cfg.causal, window=cfg.window, scale=cfg.scale, out=out,
                 lse=lse)

    fns = [fwd]
    dec = None
    if args.workload is None:
        pc = workloads.PAGED_CONFIGS[DECODE]
        print(f"bench: generating {DECODE}", file=sys.stderr, flush=True)
        inp = workloads.make_paged_config(pc)
        dd = {kk: t.to(dev) for kk, t in inp.items()}
        dout = torch.empty_like(dd["q"])
        dlse = torch.empty(dd["q"].shape[:2], dtype=torch.float32, device=dev)
        from exact_softmax_attention_amd import attn_decode_paged_workspace_size
        ws = torch.empty(attn_decode_paged_workspace_size(pc.B, pc.Hq, pc.d, pc.block_size,
                                                          pc.max_blocks_per_seq),
                         dtype=torch.uint8, device=dev)

        def decode():
            attn_decode_paged(dd["q"], dd["kcache"], dd["vcache"], dd["block_table"],
                              dd["seq_lens"], scale=pc.scale, out=dout, lse=dlse, workspace=ws)

        fns.append(decode)
        dec = (pc, inp["seq_lens"].numpy())

    print("bench: timing", file=sys.stderr, flush=True)
    per, wall = time_loop(fns, args.steps, args.warmup, torch)

    flops = metrics.fwd_flops(cfg.B, cfg.Hq, cfg.Nq, cfg.Nk, cfg.d, cfg.causal, cfg.window)
    fwd_ms = per[0]
    tflops = flops / (fwd_ms * 1e-3) / 1e12
    res = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sum(per), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name if dec is None else f"{name}+{DECODE}",
                   "prefill": {"name": name, "B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv,
                               "N": cfg.Nq, "d": cfg.d, "causal": cfg.causal,
                               "window": cfg.window, "seed": cfg.seed}},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                     "peak": metrics.PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / metrics.PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(f"fwd:{name}", FWD_FILES),
                     "kernel": "fwd_bf16_kernel<128>", "ms": round(fwd_ms, 4),
                     "flop_per_launch": flops,
                     "algorithmic_bytes": metrics.fwd_bytes(cfg.B, cfg.Hq, cfg.Hkv, cfg.Nq,
                                                            cfg.Nk, cfg.d)},
        "wall_ms_per_step": round(wall, 4),
    }
    if dec is not None:
        pc, lens = dec
        nbytes = metrics.decode_bytes(lens, pc.Hq, pc.Hkv, pc.d, pc.block_size)
        gbs = nbytes / (per[1] * 1e-3) / 1e9
        res["config"]["decode"] = {"name": pc.name, "B": pc.B, "Hq": pc.Hq, "Hkv": pc.Hkv,
                                   "d": pc.d, "block_size": pc.block_size,
                                   "num_blocks": pc.num_blocks, "seq_lens_sum": int(lens.sum()),
                                   "seed": pc.seed}
        res["decode"] = {"value": round(gbs, 1), "unit": "GB/s", "ms": round(per[1], 4),
                         "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                      "peak": metrics.PEAK_HBM_GBS, "unit": "GB/s",
                                      "frac": round(gbs / metrics.PEAK_HBM_GBS, 4),
                                      "traffic": measured_traffic(f"decode:{pc.name}",
                                                                  DECODE_FILES),
                                      "kernels": "decode_split_kernel<128> + "
                                                 "decode_combine_kernel<128>",
                                      "algorithmic_bytes": nbytes}}
    if not args.skip_backward:
        print("bench: backward", file=sys.stderr, flush=True)
        do = workloads.make_dout(cfg.B, cfg.Nq, cfg.Hq, cfg.d, cfg.seed).to(dev)
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        bws = torch.empty(max(1, attn_bwd_workspace_size(cfg.B, cfg.Hq, cfg.Nq)),
                          dtype=torch.uint8, device=dev)
        fwd()

        def bwd():
            attn_bwd(qd, kd, vd, out, do, lse, causal=cfg.causal, window=cfg.window,
                     scale=cfg.scale, dq=dq, dk=dk, dv=dv, workspace=bws)

        bper, _ = time_loop([bwd], max(2, args.steps // 2), max(1, args.warmup // 2), torch)
        bflops = metrics.bwd_flops(cfg.B, cfg.Hq, cfg.Nq, cfg.Nk, cfg.d, cfg.causal, cfg.window)
        btf = bflops / (bper[0] * 1e-3) / 1e12
        res["backward"] = {"value": round(btf, 2), "unit": "TFLOP/s", "ms": round(bper[0], 4),
                           "workload": name, "flop_per_call": bflops,
                           "kernels": "bwd_prep_kernel + bwd_dkdv_kernel + bwd_dq_kernel",
                           "cpu_baseline": None if args.skip_cpu_baseline else cpu_sample(
                               lambda: __import__("oracle").attention_backward(
                                   q, k, v, do.cpu(), cfg.scale, cfg.causal, cfg.window,
                                   heads=[(0, 0)]),
                               bflops / (cfg.B * cfg.Hq),
                               f"1 of {cfg.B * cfg.Hq} (batch, head) pairs of {name}, fp64 "
                               "gradients of the materialised definition"),
                           "roofline": {"bound": "mfma", "achieved": round(btf, 2),
                                        "peak": metrics.PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                        "frac": round(btf / metrics.PEAK_BF16_TFLOPS, 4)},
                           # what the kernels execute: dK/dV recomputes S and dP, and dQ
                           # recomputes them again (seven products, 3.5x the forward)
                           "executed": {"flop_per_call": metrics.bwd_executed_flops(
                               cfg.B, cfg.Hq, cfg.Nq, cfg.Nk, cfg.d, cfg.causal, cfg.window),
                               "TFLOP/s": round(btf * 3.5 / 2.5, 2),
                               "frac": round(btf * 3.5 / 2.5 / metrics.PEAK_BF16_TFLOPS, 4)}}
    if not args.skip_varlen and args.workload is None:
        print(f"bench: varlen {PACKED}", file=sys.stderr, flush=True)
        from exact_softmax_attention_amd import attn_fwd_varlen
        vc = workloads.PACKED_CONFIGS[PACKED]
        pq, pk, pv, cu_q, cu_k = [t.to(dev) for t in workloads.make_packed_config(vc)]
        pout = torch.empty_like(pq)
        plse = torch.empty((vc.Hq, vc.total), dtype=torch.float32, device=dev)

        def varlen():
            attn_fwd_varlen(pq, pk, pv, cu_q, cu_k, causal=vc.causal, window=vc.window,
                            scale=vc.scale, out=pout, lse=plse)

        vper, _ = time_loop([varlen], max(2, args.steps), max(1, args.warmup), torch)
        # its backward (attn_bwd_varlen) on a seeded dO
        from exact_softmax_attention_amd import attn_bwd_varlen, attn_bwd_workspace_size
        pdo = workloads.make_dout(1, vc.total, vc.Hq, vc.d, vc.seed)[0].to(dev)
        pdq, pdk, pdv = torch.empty_like(pq), torch.empty_like(pk), torch.empty_like(pv)
        pws = torch.empty(max(1, attn_bwd_workspace_size(1, vc.Hq, vc.total)), dtype=torch.uint8,
                          device=dev)
        varlen()

        def varlen_bwd():
            attn_bwd_varlen(pq, pk, pv, pout, pdo, plse, cu_q, cu_k, causal=vc.causal,
                            window=vc.window, scale=vc.scale, dq=pdq, dk=pdk, dv=pdv,
                            workspace=pws)

        vbper, _ = time_loop([varlen_bwd], max(2, args.steps // 2), max(1, args.warmup // 2), torch)
        lens = (cu_q[1:] - cu_q[:-1]).cpu().numpy()
        vflops = metrics.varlen_fwd_flops(lens, lens, vc.Hq, vc.d, vc.causal, vc.window)
        padded = metrics.fwd_flops(len(lens), vc.Hq, vc.max_len, vc.max_len, vc.d, vc.causal,
                                   vc.window)
        vtf = vflops / (vper[0] * 1e-3) / 1e12
        hq_, hk_, hv_ = pq.cpu(), pk.cpu(), pv.cpu()
        hcu = cu_q.cpu().numpy()
        res["varlen"] = {"value": round(vtf, 2), "unit": "TFLOP/s", "ms": round(vper[0], 4),
                         "workload": vc.name, "num_seqs": int(len(lens)),
                         "mean_len": round(float(lens.mean()), 1), "max_len": int(lens.max()),
                         "flop_per_call": vflops,
                         "useful_fraction_if_padded": round(vflops / padded, 4),
                         "kernel": "fwd_bf16_kernel<128, varlen>",
                         "cpu_baseline": None if args.skip_cpu_baseline else cpu_sample(
                             lambda: __import__("oracle").attention_varlen(
                                 hq_, hk_, hv_, hcu, hcu, vc.scale, vc.causal, vc.window,
                                 seqs=list(range(16))),
                             metrics.varlen_fwd_flops(lens[:16], lens[:16], vc.Hq, vc.d, vc.causal,
                                                      vc.window),
                             f"the first 16 of {len(lens)} sequences, all {vc.Hq} heads, fp64"),
                         "backward": {"value": round(2.5 * vflops / (vbper[0] * 1e-3) / 1e12, 2),
                                      "unit": "TFLOP/s", "ms": round(vbper[0], 4),
                                      "flop_per_call": 2.5 * vflops},
                         "roofline": {"bound": "mfma", "achieved": round(vtf, 2),
                                      "peak": metrics.PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                      "frac": round(vtf / metrics.PEAK_BF16_TFLOPS, 4)}}
    if not args.skip_prefill_paged and args.workload is None:
        print(f"bench: prefill over the paged cache {PREFILL_PAGED}", file=sys.stderr, flush=True)
        from exact_softmax_attention_amd import attn_prefill_paged
        ppc = workloads.PREFILL_PAGED_CONFIGS[PREFILL_PAGED]
        hpin = workloads.make_prefill_paged_config(ppc)
        pin = {kk: t.to(dev) for kk, t in hpin.items()}
        ppout = torch.empty_like(pin["q"])
        pplse = torch.empty((ppc.Hq, pin["q"].shape[0]), dtype=torch.float32, device=dev)
        from exact_softmax_attention_amd import attn_prefill_paged_workspace_size
        ppws = torch.empty(max(1, attn_prefill_paged_workspace_size(
            ppc.B, pin["q"].shape[0], ppc.Hq, ppc.d, ppc.block_size, ppc.max_blocks_per_seq)),
            dtype=torch.uint8, device=dev)

        def prefill_paged():
            attn_prefill_paged(pin["q"], pin["kcache"], pin["vcache"], pin["block_table"],
                               pin["seq_lens"], pin["cu_seqlens_q"], scale=ppc.scale,
                               window=ppc.window, out=ppout, lse=pplse, workspace=ppws)

        pper, _ = time_loop([prefill_paged], max(2, args.steps), max(1, args.warmup), torch)
        plens = pin["seq_lens"].cpu().numpy()
        pch = (pin["cu_seqlens_q"][1:] - pin["cu_seqlens_q"][:-1]).cpu().numpy()
        pflops = metrics.prefill_paged_flops(plens, pch, ppc.Hq, ppc.d, ppc.window)
        ptf = pflops / (pper[0] * 1e-3) / 1e12
        smin = int(plens.argmin())
        res["prefill_paged"] = {"value": round(ptf, 2), "unit": "TFLOP/s", "ms": round(pper[0], 4),
                                "workload": ppc.name, "new_tokens": int(pch.sum()),
                                "cached_tokens": int(plens.sum()), "flop_per_call": pflops,
                                "kernels": "fwd_bf16_kernel<128, paged> + prefill_merge_kernel<128>",
                                "cpu_baseline": None if args.skip_cpu_baseline else cpu_sample(
                                    lambda: __import__("oracle").prefill_paged(
                                        hpin["q"], hpin["kcache"], hpin["vcache"],
                                        hpin["block_table"], hpin["seq_lens"],
                                        hpin["cu_seqlens_q"], ppc.scale, ppc.window,
                                        seqs=[smin]),
                                    metrics.prefill_paged_flops(plens[smin:smin + 1],
                                                                pch[smin:smin + 1], ppc.Hq,
                                                                ppc.d, ppc.window),
                                    f"the shortest of {len(plens)} sequences ({int(plens[smin])} "
                                    f"cached tokens, {int(pch[smin])} new), all {ppc.Hq} heads, "
                                    "fp64"),
                                "workspace_bytes": int(ppws.numel()),
                                "roofline": {"bound": "mfma", "achieved": round(ptf, 2),
                                             "peak": metrics.PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                             "frac": round(ptf / metrics.PEAK_BF16_TFLOPS, 4)}}
    if args.workload is None:
        # the merge of two partial results at the prefill shape (one device's
        # combine step when the keys are split into shards)
        from exact_softmax_attention_amd import attn_merge
        ob_, lb_ = out.clone(), lse.clone()
        mo, ml = torch.empty_like(out), torch.empty_like(lse)

        def merge():
            attn_merge(out, lse, ob_, lb_, out=mo, lse=ml)

        mper, _ = time_loop([merge], max(5, args.steps), max(2, args.warmup), torch)
        mbytes = 3 * out.numel() * 2 + 3 * lse.numel() * 4
        mgbs = mbytes / (mper[0] * 1e-3) / 1e9
        res["merge"] = {"value": round(mgbs, 1), "unit": "GB/s", "ms": round(mper[0], 4),
                        "workload": f"two partial results of {name}",
                        "algorithmic_bytes": mbytes, "kernel": "merge_kernel<128>",
                        "roofline": {"bound": "hbm", "achieved": round(mgbs, 1),
                                     "peak": metrics.PEAK_HBM_GBS, "unit": "GB/s",
                                     "frac": round(mgbs / metrics.PEAK_HBM_GBS, 4)}}
        # the fp32 single-head case (1 x 256 x 1 x 64): launch-latency bound,
        # reported in microseconds only
        from exact_softmax_attention_amd import attn_fwd_f32
        fc = workloads.DENSE_CONFIGS["f32_single_head_256"]
        fq, fk, fv = [t.to(dev) for t in workloads.make_dense_config(fc)]
        fout, flse = torch.empty_like(fq), torch.empty((1, 1, fc.Nq), device=dev)

        def f32_fwd():
            attn_fwd_f32(fq, fk, fv, causal=fc.causal, window=fc.window, scale=fc.scale,
                         out=fout, lse=flse)

        fper, _ = time_loop([f32_fwd], max(20, args.steps), max(3, args.warmup), torch)
        res["f32_single_head"] = {"us": round(fper[0] * 1e3, 2), "workload": fc.name,
                                  "kernel": "fwd_f32_kernel<64>",
                                  "note": "launch-latency bound; no roofline fraction"}
    if args.workload is None and not args.skip_dense_extra:
        # the other dense configurations: GQA and MQA causal 16K, sliding window 32K
        for nm in EXTRA_DENSE:
            res[nm] = dense_object(nm, args, torch, dev)
    if not args.skip_cpu_baseline:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(q, k, v, cfg)
    print(json.dumps(res))


if __name__ == "__main__":
    main()

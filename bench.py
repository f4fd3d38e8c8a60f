#!/usr/bin/env python3
"""Throughput of the paged-attention forward pass on one MI355X.

One step is one full forward pass (plan + attention + merge) over one batch of
the named synthetic workload.  The default is the largest decode workload,
the long-context skewed decode: batch 256, 64 query / 8 KV heads, head size
128, block size 128, fp16, context lengths log-uniform in [256, 32768] with
four sequences at 32768.  Inputs are resident in HBM before timing starts;
the timed steps rotate over several copies of the KV cache so no step finds
the previous step's KV bytes in the caches.

Prints one JSON line: tokens/s (query tokens per second), the step time's
p10 / p50 / p90, the attention kernel's achieved HBM bandwidth on the KV
bytes the method must read (each visible (sequence, KV head, token) row of K
and V once) against the 8 TB/s peak and against a measured streaming-read
ceiling of this device, the oracle's own throughput on the host cores, and
(unless --no-table) the same figures for the five named configurations:
tiny decode as latency, GQA decode, skewed long decode, splitfuse with the
causal mask (matrix-core roofline) and MLA decode.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged-attn decode tokens/s + achieved HBM GB/s (KV bytes read) vs peak, 1 GPU"
HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0   # dense fp16 / bf16 matrix-core peak
RIDGE = MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)   # FLOP per byte where the bounds meet
CPU_SHARE = 16          # host threads the CPU baseline uses at most (the host cores per GPU)


def kernel_sources_digest():
    """Digest of the kernel sources with comments and blank lines removed, so
    that counters stay attached to the code they were taken on."""
    import re

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_attention_18_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            text = open(os.path.join(csrc, f)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            text = re.sub(r"//[^\n]*", "", text)
            h.update("\n".join(l.rstrip() for l in text.splitlines() if l.strip()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_sources") != kernel_sources_digest():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def attention_flops(p):
    """2 * (Dk + Dv) FLOP per visible (row, KV token) pair: the QK dot and the
    PV update, counted for every query head (masked pairs are not counted)."""
    import numpy as np

    w = p.workload
    kv = p.context_lens_np.astype(np.int64)
    ql = np.ones(p.batch, np.int64) if p.q_seq_lens_np is None else p.q_seq_lens_np.astype(np.int64)
    if w.mask in ("causal", "band"):
        prefix = np.maximum(kv - ql, 0)
        right = w.window_right if w.mask == "band" else 0
        left = w.window_left if w.mask == "band" else None
        pairs = 0
        for b in range(p.batch):
            pos = prefix[b] + np.arange(ql[b])          # row i sits at position prefix + i
            hi = np.minimum(pos + 1 + right, kv[b])
            lo = np.zeros_like(pos) if left is None else np.maximum(pos - left, 0)
            pairs += int(np.maximum(hi - lo, 0).sum())
    elif w.mask == "sparse":
        # list entries that select a visible token, for each query head of the KV head
        return p.sparse_entries() * (w.head_num // w.kv_head_num) * 2 * (w.head_size_k + w.head_size_v)
    else:
        pairs = int((ql * kv).sum())
    return pairs * w.head_num * 2 * (w.head_size_k + w.head_size_v)


def cpu_baseline(p, target_s, threads):
    """The oracle on a bounded sample of the same workload (whole sequences,
    all heads), timed on the host cores."""
    import numpy as np
    import torch

    from oracle import pa_ref

    w = p.workload
    kv = p.context_lens_np.astype(np.int64)
    ql = np.ones(p.batch, np.int64) if p.q_seq_lens_np is None else p.q_seq_lens_np.astype(np.int64)
    cu = np.concatenate([[0], np.cumsum(ql)])
    # oracle work per sequence ~ rows x visible tokens x (Dk + Dv)
    seen = np.minimum(kv, w.window_left + 1 + w.window_right) if w.mask == "band" else kv
    if w.mask == "sparse":
        seen = np.minimum(kv, w.topk)
    cost = ql * seen * w.head_num * (w.head_size_k + w.head_size_v)
    order = np.random.default_rng(0).permutation(p.batch)

    def sub_problem(seqs):
        bs = w.block_size
        blocks, tables = [], []
        for b in seqs:
            n = int((kv[b] + bs - 1) // bs)
            tables.append(list(range(len(blocks), len(blocks) + n)))
            blocks.extend(p.block_tables_np[b, :n].tolist())
        mb = max(1, max(len(t) for t in tables))
        bt = np.zeros((len(seqs), mb), np.int32)
        for i, t in enumerate(tables):
            bt[i, :len(t)] = t
        idx = torch.tensor(blocks, dtype=torch.long, device=p.key_cache.device)
        qidx = torch.cat([torch.arange(int(cu[b]), int(cu[b + 1])) for b in seqs]).to(p.query.device)
        return pa_ref.Inputs(p.query[qidx], p.key_cache[idx],
                             None if p.value_cache is None else p.value_cache[idx], bt, kv[seqs],
                             None if p.q_seq_lens_np is None else ql[seqs], w.head_num, w.kv_head_num,
                             w.dtype, w.mask, w.scale, w.head_size_v, (w.window_left, w.window_right),
                             p.mask_tensor, None if p.topk_idx is None else p.topk_idx[qidx])

    # calibrate the oracle's rate on the cheapest sequence
    b0 = int(np.argmin(cost))
    inp0 = sub_problem([b0])
    t = time.perf_counter()
    pa_ref.forward(inp0, threads=1)
    rate = cost[b0] / max(1e-6, time.perf_counter() - t)           # work units / s / thread
    budget = target_s * rate * threads
    seqs, acc = [], 0.0
    for b in order:
        if acc + cost[b] > budget and seqs:
            continue
        seqs.append(int(b))
        acc += cost[b]
    seqs.sort()
    inp = sub_problem(seqs)
    # repeat a sample that finishes early (the whole workload can take well
    # under a second), so the rate is not one short, noisy interval
    reps = 0
    t = time.perf_counter()
    while True:
        pa_ref.forward(inp, threads=threads)
        reps += 1
        dt = time.perf_counter() - t
        if dt >= min(3.0, target_s):
            break
    tokens = int(ql[seqs].sum())
    return {"value": tokens * reps / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(seqs)} of {p.batch} sequences ({tokens} query tokens, all {w.head_num} heads, "
                      f"{int(kv[seqs].sum())} KV tokens), fp64, {reps} run(s) in {dt:.1f} s wall"}


TABLE = ("tiny_decode", "gqa_decode", "skewed_long_decode", "splitfuse_causal", "mla_decode")


def pct(xs):
    import numpy as np

    a = np.asarray(xs, dtype=np.float64)
    return {"p10": float(np.percentile(a, 10)), "p50": float(np.percentile(a, 50)),
            "p90": float(np.percentile(a, 90)), "mean": float(a.mean())}


def read_peak(dev, nbytes=2 << 30, reps=10):
    """The device's streaming-read rate: a plain kernel reading one large
    buffer in contiguous per-workgroup shares (the library's read probe),
    timed with events on the stream it runs on.  Best and median of reps."""
    import torch

    from paged_kv_attention_18_amd import binding

    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(7)
    wgs = 2048
    sink = torch.empty(wgs, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    for _ in range(3):
        binding.pa_read_probe(buf.data_ptr(), nbytes, sink.data_ptr(), wgs, sp)
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        binding.pa_read_probe(buf.data_ptr(), nbytes, sink.data_ptr(), wgs, sp)
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    del buf, sink
    torch.cuda.empty_cache()
    times.sort()
    return {"gbps_best": nbytes / (times[0] * 1e-3) / 1e9, "gbps_median": nbytes / (times[len(times) // 2] * 1e-3) / 1e9,
            "bytes": nbytes, "reps": reps,
            "method": f"pa_read_probe: {wgs} workgroups x 256 threads, contiguous shares, 8 x 16-byte loads in flight per thread"}


def measure(w, dev, steps, warmup, flags=0, partitions=0, graph=False, copies=0, peak=None, warmup_ms=150.0):
    """Times `steps` forward passes of workload w (after `warmup` untimed
    ones): the whole pass without per-kernel events (throughput), each pass
    on its own (percentiles), and each kernel with the library's HIP events
    (roofline).  warmup None: at least 5 passes and at least warmup_ms of GPU
    time (the matrix-core kernels run 15-25 % slower in their first ~50 ms of
    sustained work, while the clocks settle)."""
    import numpy as np
    import torch

    from paged_kv_attention_18_amd import binding, synth

    p = synth.generate(w, device=dev)
    vc_numel = 0 if p.value_cache is None else p.value_cache.numel()
    cache_bytes = (p.key_cache.numel() + vc_numel) * p.key_cache.element_size()
    copies = copies or max(3, math.ceil((1.5 * (1 << 30)) / cache_bytes))
    kcs = [p.key_cache] + [p.key_cache.clone() for _ in range(copies - 1)]
    # shared K/V: no value cache (V is read from the K rows)
    vcs = [None] * copies if p.value_cache is None else [p.value_cache] + [p.value_cache.clone() for _ in range(copies - 1)]
    att = binding.for_problem(p, flags=flags, num_partitions=partitions)
    desc = att.describe()
    out = torch.empty(p.num_q_tokens, w.head_num, w.head_size_v, dtype=p.query.dtype, device=dev)
    ql_max = max(1, p.max_q_seq_len)

    def step(k):
        att.forward(p.query, kcs[k % copies], vcs[k % copies], p.block_tables, p.context_lens,
                    p.q_seq_lens, max_q_seq_len=ql_max, out=out, topk_indices=p.topk_idx)

    if warmup is None:
        # two passes for the one-time costs, then one timed to size the rest
        step(0)
        step(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        step(2)
        e1.record()
        torch.cuda.synchronize()
        warmup = min(20000, max(5, 3 + math.ceil(warmup_ms / max(e0.elapsed_time(e1), 1e-3))))
        for k in range(3, warmup):
            step(k)
    else:
        for k in range(warmup):
            step(k)
    torch.cuda.synchronize()
    if att.device_error() != 0:
        raise RuntimeError("device error flag set during warm-up")

    stream = torch.cuda.current_stream()
    run = step
    if graph:
        # one captured forward pass per KV copy, replayed in the same rotation
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for k in range(copies):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    step(k)
                graphs.append(g)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        run = lambda k: graphs[k % copies].replay()
        for k in range(warmup):
            run(k)
        torch.cuda.synchronize()

    # (1) whole-pass throughput: events only around the K steps
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for k in range(steps):
        run(k)
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    # (2) the same steps with an event between consecutive passes (percentiles)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for k in range(steps):
        run(k)
        evs[k + 1].record(stream)
    torch.cuda.synchronize()
    step_ms = [evs[k].elapsed_time(evs[k + 1]) for k in range(steps)]
    # (3) eager passes with HIP events around each kernel, recorded by the
    #     library on the stream its kernels run on
    binding.pa_set_timing(att.handle, 1)
    for k in range(steps):
        step(k)
    torch.cuda.synchronize()
    kms, passes, planned, per_pass = binding.pa_read_timing(att.handle, per_pass_cap=steps)
    binding.pa_set_timing(att.handle, 0)
    assert passes == steps
    if att.device_error() != 0:
        raise RuntimeError("device error flag set during the timed steps")

    ms_per_step = total_ms / steps
    kv_bytes = synth.kv_bytes(p)
    attn = [r[1] for r in per_pass]
    attn_ms = kms[1] / passes
    kernel = {"valu": "decode_kernel", "mfma": "tile_kernel", "stream": "stream_kernel"}[desc["path"]]
    traffic = measured_traffic(w.name, kernel)
    flops = attention_flops(p)
    hbm_gbps = kv_bytes / (attn_ms * 1e-3) / 1e9
    if flops / kv_bytes > RIDGE:
        # compute-bound (long splitfuse chunks): matrix-core roofline
        achieved = flops / (attn_ms * 1e-3) / 1e12
        roofline = {"kernel": kernel, "bound": "mfma", "achieved": achieved, "peak": MFMA_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": achieved / MFMA_PEAK_TFLOPS, "traffic": traffic,
                    "flops_per_launch": flops, "hbm_gbps_on_kv_bytes": hbm_gbps}
    else:
        roofline = {"kernel": kernel, "bound": "hbm", "achieved": hbm_gbps, "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": hbm_gbps / HBM_PEAK_GBPS, "traffic": traffic,
                    "kv_bytes_per_launch": kv_bytes}
        if peak:
            roofline["measured_read_peak"] = peak
            roofline["frac_of_measured_read_peak"] = hbm_gbps / peak
    res = {
        "p": p, "desc": desc, "copies": copies, "warmup": warmup, "ms_per_step": ms_per_step, "step_ms": pct(step_ms),
        "attention_ms": pct(attn), "kv_bytes": kv_bytes, "flops": flops, "roofline": roofline,
        "kernels_ms": {"plan": kms[0] / planned if planned else None, "attention": attn_ms,
                       "merge": kms[2] / passes},
    }
    del kcs, vcs, out, att
    return res


def table_row(w, r):
    p = r["p"]
    row = {"workload": w.name, "batch": p.batch, "query_tokens": p.num_q_tokens, "kv_tokens": p.kv_tokens(),
           "kv_bytes": r["kv_bytes"], "path": r["desc"]["path"], "step_ms": r["step_ms"],
           "attention_ms": r["attention_ms"], "kernels_ms": r["kernels_ms"]}
    if w.name == "tiny_decode":
        # parity-sized: reported as latency
        row["latency_us"] = {k: v * 1e3 for k, v in r["step_ms"].items()}
        return row
    row["tokens_per_s"] = p.num_q_tokens / (r["ms_per_step"] * 1e-3)
    rf = r["roofline"]
    row["roofline"] = {k: rf[k] for k in ("bound", "achieved", "unit", "frac") if k in rf}
    if "frac_of_measured_read_peak" in rf:
        row["roofline"]["frac_of_measured_read_peak"] = rf["frac_of_measured_read_peak"]
    if rf["bound"] == "mfma":
        row["roofline"]["hbm_gbps_on_kv_bytes"] = rf["hbm_gbps_on_kv_bytes"]
    return row


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed passes before the timed ones (default: at least 5 and at least --warmup-ms)")
    ap.add_argument("--warmup-ms", type=float, default=150.0,
                    help="GPU time of the default warm-up, in ms (the compute-bound kernels speed up over the "
                         "first ~50 ms of sustained work)")
    ap.add_argument("--workload", default="skewed_long_decode",
                    help="tiny_decode | gqa_decode | skewed_long_decode | splitfuse_causal | mla_decode | ...")
    ap.add_argument("--copies", type=int, default=0, help="KV cache copies to rotate over (0 = auto)")
    ap.add_argument("--flags", type=int, default=0, help="pa_config.flags (PA_FLAG_* bits; 0 = automatic)")
    ap.add_argument("--partitions", type=int, default=0, help="pa_config.num_partitions (0 = automatic)")
    ap.add_argument("--graph", action="store_true",
                    help="replay the forward pass from HIP graphs (one per KV copy) for the throughput figure")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle sample size, in seconds")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-table", action="store_true", help="time the named workload only")
    ap.add_argument("--table-steps", type=int, default=20, help="timed steps per workload of the table")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not supported "
              "(the attention has no cross-GPU path here)", file=sys.stderr)
        sys.exit(2)

    import torch

    from paged_kv_attention_18_amd import synth

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)
        return

    peak = read_peak(dev)
    print(f"# measured streaming read: {peak['gbps_best']:.0f} GB/s best, {peak['gbps_median']:.0f} median",
          file=sys.stderr, flush=True)
    w = synth.WORKLOADS[int(args.workload)] if args.workload.isdigit() else synth.by_name(args.workload)
    r = measure(w, dev, args.steps, args.warmup, args.flags, args.partitions, args.graph, args.copies,
                peak["gbps_best"], args.warmup_ms)
    print(f"# {w.name}: {r['ms_per_step'] * 1e3:.1f} us per step", file=sys.stderr, flush=True)
    p = r["p"]
    tokens = p.num_q_tokens
    result = {
        "metric": METRIC,
        "value": tokens / (r["ms_per_step"] * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": r["warmup"],
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": p.batch, "head_num": w.head_num, "kv_head_num": w.kv_head_num,
            "head_size_k": w.head_size_k, "head_size_v": w.head_size_v, "block_size": w.block_size,
            "mask": w.mask, "shared_kv": w.shared_kv, "query_tokens": tokens, "kv_tokens": p.kv_tokens(),
            "kv_bytes": r["kv_bytes"], "seed": w.seed, "kv_cache_copies": r["copies"], "path": r["desc"]["path"],
            "partitions": r["desc"]["partitions"], "flags": args.flags, "parallelism": "none (1 GPU)",
        },
        "step_ms": r["step_ms"],
        "pass_hbm_gbps": r["kv_bytes"] / (r["ms_per_step"] * 1e-3) / 1e9,
        "launch": "hip graph replay" if args.graph else "eager",
        "kernels_ms": r["kernels_ms"],
        "attention_ms": r["attention_ms"],
        "read_peak": peak,
        "roofline": r["roofline"],
        "cpu_baseline": None,
        "configs": None,
    }
    headline = r
    if not args.no_table:
        rows = []
        for name in TABLE:
            wt = synth.by_name(name)
            rt = headline if name == w.name else measure(wt, dev, args.table_steps, None, peak=peak["gbps_best"],
                                                             warmup_ms=args.warmup_ms)
            rows.append(table_row(wt, rt))
            print(f"# table {name}: {rt['step_ms']['p50'] * 1e3:.1f} us p50", file=sys.stderr, flush=True)
            if rt is not headline:
                del rt
                torch.cuda.empty_cache()
        result["configs"] = rows
    if not args.no_cpu_baseline:
        threads = min(CPU_SHARE, len(os.sched_getaffinity(0)))
        result["cpu_baseline"] = cpu_baseline(p, args.cpu_seconds, threads)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

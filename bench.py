"""Benchmark of the relative-bias attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input, one
call sequence per workload the path is quoted on:
  * local_prefill: rba_prefill on the Inkling-Small local-layer prefill (one
    8,192-token sequence, 32 query / 8 KV heads, head size 128, window 512,
    rel extent 512, paged in permuted 128-token blocks);
  * global_prefill: the global-layer chunked prefill, a 32,768-token
    sequence as 4 rba_prefill calls of 8,192 rows each over all cached keys
    before them (no window, rel extent 1024);
  * decode: rba_decode on the global-layer paged decode (16 sequences with
    seeded lengths uniform in [8K, 128K], one query token each, 32/8 heads,
    rel extent 1024; every sequence on its own blocks, so no block is read
    twice) as its two stages, split-KV then log-sum-exp combine;
  * verify_b1, verify_b8: rba_decode on the diff-headdim verify (100,000-token
    context, 4 query tokens per sequence, 64/8 heads, value head 64, rel
    extent 1024) at batch 1 and batch 8, again as split + combine.
Inputs are resident in HBM before timing. Each call is timed with HIP events
on the stream it is launched on, and the whole step with host clocks around
synchronisations.

value = whole-step fraction of the MI355X roofline, in percent:
  100 * sum_calls max(F/peak_mfma, B/peak_hbm) / sum_calls measured time
with F, B the algorithmic flops / bytes (visible (query, key) pairs only; K/V,
q, rel, out and tables read or written once). Per-leg TFLOP/s, GB/s and roof
fractions are reported beside it, plus the roofline of the dominant kernel
(and of the decode split kernel) and the float64 CPU oracle timed on a
bounded sample of the same workloads.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
for _p in (ROOT, os.path.join(ROOT, "tests")):
    if _p not in sys.path:
        sys.path.insert(0, _p)

METRIC = "rel-bias attn prefill TFLOP/s + decode HBM GB/s, % of MI355X roofline"
PEAK_MFMA_BF16 = 2516.6e12   # dense bf16 MFMA, FLOP/s (256 CU x 2.4 GHz x 4096)
PEAK_HBM = 8.0e12            # HBM3E, B/s
DQK = 128
# (leg, workload) of one step
LEGS = [
    ("local_prefill", "local_prefill_8k"),
    ("global_prefill", "global_chunked_prefill_32k"),
    ("decode", "paged_decode_16x8k_128k_disjoint"),
    ("verify_b1", "verify_decode_b1_100k"),
    ("verify_b8", "verify_decode_b8_100k"),
]

PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILES = {
    "decode": os.path.join(PROFILES, "decode16_split_kernel_paged_decode_16_disjoint_traffic.txt"),
    "global_prefill": os.path.join(PROFILES, "prefill_tail_kernel_global_chunked_prefill_32k_traffic.txt"),
}
CSRC = os.path.join(ROOT, "relative_position_bias_amd", "csrc")
KERNEL_SRCS = [os.path.join(CSRC, "rba_kernels.hip"), os.path.join(CSRC, "rba_internal.h")]
HOST_SRCS = [os.path.join(CSRC, "rba_host.cpp")]


def code_digest(paths):
    """SHA-256 of source files with comments, blank lines and trailing blanks
    removed: it changes when the code changes, not when a comment does."""
    import hashlib
    import re

    h = hashlib.sha256()
    for path in paths:
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        lines = [ln.rstrip() for ln in text.splitlines() if ln.strip()]
        h.update(("\n".join(lines) + "\n").encode())
    return h.hexdigest()


def measured_traffic(leg):
    """HBM bytes per launch of a leg's dominant kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or None when there is none or
    the kernel code or the host code (which sets the launch, e.g. the split
    count) has changed since those counters were taken."""
    path = TRAFFIC_FILES.get(leg)
    if path is None or not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.lstrip().startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_code_sha256") != code_digest(KERNEL_SRCS) or \
            kv.get("host_code_sha256") != code_digest(HOST_SRCS):
        return None
    return int(float(kv["traffic_bytes_per_launch"]))


def visible_counts(q_lens, seq_lens, W, R):
    """Per call: visible (row, key) pairs, visible keys with a bias entry
    (distance < R), and the distinct keys any query sees (for K/V bytes)."""
    pairs = biased = keys = 0
    for ql, L in zip(q_lens, seq_lens):
        first = L - ql
        for i in range(first, L):
            n = min(i + 1, W) if W else i + 1
            pairs += n
            biased += min(n, R)
        lo = max(0, first - W + 1) if W else 0
        keys += L - lo
    return pairs, biased, keys


def algorithmic(b, kind):
    """(flops, bytes) of one call on Batch b, plus the bytes of the split
    stage alone for decode (what the split kernel reads)."""
    seq_lens = b.seq_lens.tolist()
    pairs, biased, keys = visible_counts(b.q_lens, seq_lens, b.W, b.R)
    flops = pairs * b.Hq * (2 * DQK + 2 * b.dv)
    rows = b.rows
    q_bytes = rows * b.Hq * DQK * 2
    kv_bytes = keys * b.Hkv * (DQK + b.dv) * (1 if getattr(b, "kv_fp8", False) else 2)  # e4m3: 1 byte
    if getattr(b, "r", None) is not None:  # bias made in the kernel: r and the projection are read,
        d_r = b.r.shape[2]                 # and each used bias entry costs a d_r-long dot product
        rel_bytes = rows * b.Hq * d_r * 2 + b.proj.numel() * 2
        flops += biased * b.Hq * 2 * d_r
    else:
        rel_bytes = biased * b.Hq * 4
    out_bytes = rows * b.Hq * b.dv * 4
    blocks = sum((L + 127) // 128 for L in seq_lens)
    table_bytes = blocks * 4
    read = q_bytes + kv_bytes + rel_bytes + table_bytes
    return flops, read + out_bytes, read


def roof_time(flops, nbytes):
    return max(flops / PEAK_MFMA_BF16, nbytes / PEAK_HBM)


def _sequence(b, m):
    """Sequence m of a decode Batch as a Batch of its own (CPU)."""
    import workloads as W
    sub = W.Batch(**{**b.__dict__})
    sub.q = b.q[m * b.n_q:(m + 1) * b.n_q]
    sub.rel = b.rel[m * b.n_q:(m + 1) * b.n_q]
    sub.seq_lens = b.seq_lens[m:m + 1]
    sub.block_tables = b.block_tables[m:m + 1]
    sub.q_lens = b.q_lens[m:m + 1]
    return sub


def _sampled_prefill_work(b, rows):
    """Algorithmic (flops, bytes) of the given contiguous rows of a
    one-sequence prefill Batch."""
    L = int(b.seq_lens[0])
    ctx = L - b.q_lens[0]
    pairs = biased = 0
    for r in rows:
        i = ctx + r
        n = min(i + 1, b.W) if b.W else i + 1
        pairs += n
        biased += min(n, b.R)
    lo = max(0, ctx + rows[0] - b.W + 1) if b.W else 0
    keys = ctx + rows[-1] + 1 - lo
    flops = pairs * b.Hq * (2 * DQK + 2 * b.dv)
    nbytes = (len(rows) * b.Hq * DQK * 2 + keys * b.Hkv * (DQK + b.dv) * 2 + biased * b.Hq * 4
              + len(rows) * b.Hq * b.dv * 4)
    return flops, nbytes


def cpu_baseline(inputs, budget_s):
    """The float64 oracle (its loop form, as it stands) on a bounded sample of
    every leg of the step: local prefill rows 0-255 and 4096-4351, the last 2
    rows of the last global-prefill chunk (its most expensive rows), the
    batch-1 verify call whole, then decode sequences one at a time until about
    `budget_s` seconds of CPU work in total. Reported as the fraction of the
    MI355X roofline the oracle reaches on that sample."""
    from harness import oracle_batch

    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    t_cpu = t_roof = flops = 0.0
    parts = []

    def timed(batch, rows=None):
        t0 = time.perf_counter()
        oracle_batch(batch, rows=rows, form="loop")
        return time.perf_counter() - t0

    pre = inputs["local_prefill"][0][0]
    for seg in (range(0, 256), range(4096, 4352)):
        t_cpu += timed(pre, list(seg))
        f, nb = _sampled_prefill_work(pre, list(seg))
        t_roof += roof_time(f, nb)
        flops += f
    parts.append("local prefill rows 0-255 and 4096-4351 (all heads)")
    ch = inputs["global_prefill"][-1][0]
    rows = [ch.rows - 2, ch.rows - 1]
    t_cpu += timed(ch, rows)
    f, nb = _sampled_prefill_work(ch, rows)
    t_roof += roof_time(f, nb)
    flops += f
    parts.append(f"global prefill chunk {len(inputs['global_prefill']) - 1} rows {rows[0]}-{rows[1]}")
    vb1 = inputs["verify_b1"][0][0]
    t_cpu += timed(vb1)
    f, nb, _ = algorithmic(vb1, "decode")
    t_roof += roof_time(f, nb)
    flops += f
    parts.append("verify B=1 whole call")
    dec = inputs["decode"][0][0]
    m = 0
    while m < len(dec.q_lens) and (m == 0 or t_cpu < budget_s):
        one = _sequence(dec, m)
        t_cpu += timed(one)
        f, nb, _ = algorithmic(one, "decode")
        t_roof += roof_time(f, nb)
        flops += f
        m += 1
    parts.append(f"decode sequences 0-{m - 1} of {len(dec.q_lens)}")
    return {
        "value": round(100.0 * t_roof / t_cpu, 6),
        "unit": "% of MI355X roofline",
        "cores": threads,
        "kind": "oracle",
        "sample": "; ".join(parts) + "; float64 C oracle (loop form), OpenMP",
        "seconds": round(t_cpu, 3),
        "gflops": round(flops / t_cpu / 1e9, 3),
    }


def copy_probe(mib, dev):
    """One plain device-to-device copy of `mib` MiB (torch copy_), used to
    calibrate rocprofv3's FETCH_SIZE / WRITE_SIZE counters in the same run."""
    import torch

    src = torch.empty(mib << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def workload_report(name, steps, warmup, dev, flush=True, copy_mib=0):
    """Per-call times of one named workload (each call timed with events on
    its stream), with algorithmic TFLOP/s, GB/s and roofline fractions."""
    import torch

    import workloads as W
    from harness import run_decode, run_prefill

    if copy_mib > 0:
        copy_probe(copy_mib, dev)

    full = W.build(name)
    gpu = full.to(dev)
    if W.WORKLOADS[name]["kind"] == "chunked":
        calls = list(zip(W.chunks(name, full), W.chunks(name, gpu)))
    else:
        calls = [(full, gpu)]
    stream = torch.cuda.current_stream()
    # Between timed calls a 1 GiB scratch read (outside the timed region)
    # evicts the L2 and the 256 MB Infinity Cache, so no call is served from a
    # previous call's cached inputs. A read leaves clean lines behind; a write
    # would leave dirty ones whose write-back lands inside the next timed call.
    scratch = torch.ones(1 << 28, dtype=torch.float32, device=dev) if flush else None
    res = []
    for b_cpu, b in calls:
        fn = (lambda b=b: run_prefill(b)) if b.kind == "prefill" else (lambda b=b: run_decode(b))
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = []
        for k in range(steps):
            if scratch is not None:
                scratch.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            ev.append((e0, e1))
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b2) for a, b2 in ev)
        f, nbytes, _ = algorithmic(b_cpu, b.kind)
        t = ms[len(ms) // 2] / 1e3
        res.append({"ms_median": round(ms[len(ms) // 2], 4), "ms_min": round(ms[0], 4),
                    "tflops": round(f / t / 1e12, 2), "gbps": round(nbytes / t / 1e9, 1),
                    "frac_mfma": round(f / t / PEAK_MFMA_BF16, 4), "frac_hbm": round(nbytes / t / PEAK_HBM, 4),
                    "roof_ms": round(roof_time(f, nbytes) * 1e3, 4), "flops": f, "bytes": nbytes})
    tot = sum(r["ms_median"] for r in res)
    roof = sum(r["roof_ms"] for r in res)
    print(json.dumps({"workload": name, "cache_flush": flush, "calls": res, "total_ms": round(tot, 4),
                      "roofline_frac": round(roof / tot, 4),
                      "tflops_total": round(sum(r["flops"] for r in res) / tot / 1e9, 2)}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--workload", default=None,
                    help="time one named workload on its own (a report line, not the step line)")
    ap.add_argument("--no-flush", action="store_true",
                    help="with --workload: skip the 1 GiB cache-evicting read between timed calls")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads as W
    from relative_position_bias_amd import rba

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload:
        workload_report(args.workload, args.steps, args.warmup, dev, flush=not args.no_flush,
                        copy_mib=args.copy_probe_mib)
        return
    stream = torch.cuda.current_stream()
    n_cus = torch.cuda.get_device_properties(dev).multi_processor_count

    # inputs of every leg, on the CPU (for the algorithmic counts and the
    # oracle sample) and on the GPU; a leg is a list of (cpu, gpu) calls
    t_gen = time.perf_counter()
    inputs = {}
    for leg, name in LEGS:
        full = W.build(name)
        gpu = full.to(dev)
        if W.WORKLOADS[name]["kind"] == "chunked":
            inputs[leg] = list(zip(W.chunks(name, full), W.chunks(name, gpu)))
        else:
            inputs[leg] = [(full, gpu)]
        print(f"[bench] {leg}: {name} ready ({time.perf_counter() - t_gen:.1f}s)", file=sys.stderr, flush=True)

    # the calls of one step, in order: (leg, call name, fn, flops, bytes)
    calls = []
    splits_of = {}
    for leg, _ in LEGS:
        for c, (b_cpu, b) in enumerate(inputs[leg]):
            f, nbytes, read = algorithmic(b_cpu, b.kind)
            if b.kind == "prefill":
                out = torch.empty((b.rows, b.Hq, b.dv), dtype=torch.float32, device=dev)

                def prefill_call(b=b, out=out):
                    rba.prefill(b.q, b.k_cache, b.v_cache, b.rel, b.cu_q, b.seq_lens, b.block_tables,
                                window=b.W, scale=b.scale, max_q_len=b.max_q_len, max_seq_len=b.max_seq_len,
                                out=out, stream=stream)
                calls.append((leg, f"prefill{c}", prefill_call, f, nbytes))
                continue
            batch = len(b.q_lens)
            splits = rba.plan_splits(b.Hq, b.Hkv, b.dv, b.R, b.W, b.scale, batch, b.n_q, b.max_seq_len, n_cus)
            splits_of[leg] = splits
            ws = torch.empty(rba.workspace_size(b.Hq, b.Hkv, b.dv, b.R, b.W, b.scale, batch, b.n_q,
                                                b.max_seq_len, splits), dtype=torch.uint8, device=dev)
            out = torch.empty((b.rows, b.Hq, b.dv), dtype=torch.float32, device=dev)

            def split_call(b=b, ws=ws, splits=splits):
                rba.decode_split(b.q, b.k_cache, b.v_cache, b.rel, b.seq_lens, b.block_tables, n_q=b.n_q,
                                 window=b.W, scale=b.scale, max_seq_len=b.max_seq_len, num_splits=splits,
                                 workspace=ws, stream=stream)

            def combine_call(b=b, ws=ws, splits=splits, out=out, batch=batch):
                rba.decode_combine(Hq=b.Hq, Hkv=b.Hkv, dv=b.dv, rel_extent=b.R, window=b.W, scale=b.scale,
                                   batch=batch, n_q=b.n_q, num_splits=splits, workspace=ws, out=out,
                                   stream=stream)
            # the split kernel reads the inputs; the combine writes out (the
            # workspace traffic is not algorithmic)
            calls.append((leg, "split", split_call, f, read))
            calls.append((leg, "combine", combine_call, 0, nbytes - read))

    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib, dev)

    for _ in range(args.warmup):
        for _, _, fn, _, _ in calls:
            fn()
    torch.cuda.synchronize()

    events = [[] for _ in calls]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for k, (_, _, fn, _, _) in enumerate(calls):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            events[k].append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [sum(a.elapsed_time(b) for a, b in ev) / len(ev) for ev in events]
    ms_per_step = 1e3 * wall / args.steps

    # per leg: time, rates, roof fractions; roofline-weighted step value
    legs = {}
    roof_sum = t_sum = 0.0
    for leg, name in LEGS:
        ks = [k for k, c in enumerate(calls) if c[0] == leg]
        t = sum(ms[k] for k in ks) / 1e3
        f = sum(calls[k][3] for k in ks)
        nb = sum(calls[k][4] for k in ks)
        # roof per call: each prefill chunk is its own call; a decode is one call (split + combine)
        if calls[ks[0]][1].startswith("prefill"):
            roof = sum(roof_time(calls[k][3], calls[k][4]) for k in ks)
        else:
            roof = roof_time(f, nb)
        roof_sum += roof
        t_sum += t
        legs[leg] = {"workload": name, "ms": round(t * 1e3, 4), "tflops": round(f / t / 1e12, 2),
                     "gbps": round(nb / t / 1e9, 1), "frac_mfma": round(f / t / PEAK_MFMA_BF16, 4),
                     "frac_hbm": round(nb / t / PEAK_HBM, 4), "frac_roof": round(roof / t, 4),
                     "flops": f, "bytes": nb}
        if len(ks) > 1 and calls[ks[0]][1].startswith("prefill"):
            legs[leg]["chunk_ms"] = [round(ms[k], 4) for k in ks]
        if leg in splits_of:
            legs[leg].update(split_ms=round(ms[ks[0]], 4), combine_ms=round(ms[ks[1]], 4), splits=splits_of[leg])
    value = 100.0 * roof_sum / t_sum

    def prefill_roofline(leg):
        ks = [k for k, c in enumerate(calls) if c[0] == leg]
        b = inputs[leg][0][1]
        t = sum(ms[k] for k in ks) / 1e3
        f = sum(calls[k][3] for k in ks)
        nb = sum(calls[k][4] for k in ks)
        kname = f"prefill_ring_kernel<{b.dv}>" if b.W > 0 else f"prefill_tail_kernel<{b.dv}>"
        if f / PEAK_MFMA_BF16 >= nb / PEAK_HBM:
            achieved = f / t / 1e12
            blk = {"kernel": kname, "bound": "mfma", "achieved": round(achieved, 1),
                   "peak": PEAK_MFMA_BF16 / 1e12, "unit": "TFLOP/s", "frac": round(achieved / (PEAK_MFMA_BF16 / 1e12), 4)}
        else:
            achieved = nb / t / 1e9
            blk = {"kernel": kname, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM / 1e9,
                   "unit": "GB/s", "frac": round(achieved / (PEAK_HBM / 1e9), 4)}
        blk.update(traffic=measured_traffic(leg), launches=len(ks),
                   algorithmic_flops_per_launch=f // len(ks), algorithmic_bytes_per_launch=nb // len(ks),
                   avg_launch_ms=round(t * 1e3 / len(ks), 4))
        return blk

    def decode_roofline(leg):
        ks = [k for k, c in enumerate(calls) if c[0] == leg]
        b = inputs[leg][0][1]
        t = ms[ks[0]] / 1e3
        nb = calls[ks[0]][4]
        achieved = nb / t / 1e9
        cols = b.Hq // b.Hkv * b.n_q
        kname = (f"decode16_split_kernel<{b.dv}, false>" if cols <= 16 else f"decode_split_kernel<{b.dv}, false>")
        return {"kernel": kname, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM / 1e9,
                "unit": "GB/s", "frac": round(achieved / (PEAK_HBM / 1e9), 4), "traffic": measured_traffic(leg),
                "algorithmic_bytes_per_launch": nb, "avg_launch_ms": round(ms[ks[0]], 4)}

    # dominant kernel: the leg with the largest share of the step
    dom = max(legs, key=lambda leg: legs[leg]["ms"])
    roofline = prefill_roofline(dom) if "prefill" in dom else decode_roofline(dom)

    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "% of MI355X roofline",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": " + ".join(name for _, name in LEGS),
            "local_prefill": {"seq_len": 8192, "Hq": 32, "Hkv": 8, "head_dim": DQK, "dv": 128, "window": 512,
                              "rel_extent": 512, "block_size": 128},
            "global_prefill": {"seq_len": 32768, "chunks": 4, "chunk": 8192, "Hq": 32, "Hkv": 8, "head_dim": DQK,
                               "dv": 128, "window": 0, "rel_extent": 1024, "block_size": 128},
            "decode": {"batch": 16, "n_q": 1, "seq_lens_sum": int(sum(inputs["decode"][0][0].seq_lens.tolist())),
                       "Hq": 32, "Hkv": 8, "dv": 128, "rel_extent": 1024, "block_size": 128},
            "verify": {"batch": [1, 8], "n_q": 4, "seq_len": 100000, "Hq": 64, "Hkv": 8, "dv": 64,
                       "rel_extent": 1024, "block_size": 128},
        },
        **legs,
        "roofline": roofline,
        "roofline_decode": decode_roofline("decode"),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the float64 oracle on a sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(inputs, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

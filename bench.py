"""Benchmark of the relative-bias attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  * rba_prefill on the Inkling-Small local-layer prefill (one 8,192-token
    sequence, 32 query / 8 KV heads, head size 128, window 512, rel extent
    512, paged in permuted 128-token blocks), then
  * rba_decode on the global-layer paged decode (16 sequences with seeded
    lengths uniform in [8K, 128K], one query token each, 32/8 heads, rel
    extent 1024, block size 128; every sequence on its own blocks, so no block
    is read twice) as its two stages, split-KV then log-sum-exp combine.
Inputs are resident in HBM before timing. Each call is timed with HIP events
on the stream it is launched on, and the whole step with host clocks around
synchronisations.

value = whole-step fraction of the MI355X roofline, in percent:
  100 * sum_calls max(F/peak_mfma, B/peak_hbm) / sum_calls measured time
with F, B the algorithmic flops / bytes (visible (query, key) pairs only; K/V,
q, rel, out and tables read or written once). Per-call TFLOP/s and GB/s are
reported beside it, plus the roofline of the dominant kernel and the float64
CPU oracle timed on a bounded sample of the same workload.
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
PREFILL = "local_prefill_8k"
DECODE = "paged_decode_16x8k_128k_disjoint"
DQK = 128


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode16_split_kernel_paged_decode_16_disjoint_traffic.txt")
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


def measured_traffic():
    """HBM bytes per launch of the decode split kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or None when the kernel code
    or the host code (which sets the launch, e.g. the split count) has changed
    since those counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
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


def _first_sequences(b, m):
    import workloads as W
    sub = W.Batch(**{**b.__dict__})
    sub.q = b.q[:m * b.n_q]
    sub.rel = b.rel[:m * b.n_q]
    sub.seq_lens = b.seq_lens[:m]
    sub.block_tables = b.block_tables[:m]
    sub.q_lens = b.q_lens[:m]
    return sub


def cpu_baseline(pre_cpu, dec_cpu, budget_s):
    """The float64 oracle (as it stands) on a bounded sample of the step:
    prefill query rows 0..1023 (all heads), then decode sequences one at a
    time until about `budget_s` seconds of CPU work in total."""
    from harness import oracle_batch

    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    rows = list(range(0, 1024))
    t0 = time.perf_counter()
    oracle_batch(pre_cpu, rows=rows)
    t_pre = time.perf_counter() - t0
    t_dec, m = 0.0, 0
    while m < len(dec_cpu.q_lens) and (m == 0 or t_pre + t_dec < budget_s):
        one = _first_sequences(dec_cpu, m + 1)
        one.q, one.rel = one.q[m * one.n_q:], one.rel[m * one.n_q:]
        one.seq_lens, one.block_tables, one.q_lens = one.seq_lens[m:], one.block_tables[m:], one.q_lens[m:]
        t0 = time.perf_counter()
        oracle_batch(one)
        t_dec += time.perf_counter() - t0
        m += 1
    f_pre, b_pre = _sampled_prefill_work(pre_cpu, rows)
    f_dec, b_dec, _ = algorithmic(_first_sequences(dec_cpu, m), "decode")
    t_roof = roof_time(f_pre, b_pre) + roof_time(f_dec, b_dec)
    t_cpu = t_pre + t_dec
    return {
        "value": round(100.0 * t_roof / t_cpu, 6),
        "unit": "% of MI355X roofline",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"prefill rows 0-{len(rows) - 1} of {pre_cpu.rows} (all {pre_cpu.Hq} heads) + "
                   f"decode sequences 0-{m - 1} of {len(dec_cpu.q_lens)}; float64 C oracle, OpenMP"),
        "seconds": round(t_cpu, 3),
        "gflops": round((f_pre + f_dec) / t_cpu / 1e9, 3),
    }


def _sampled_prefill_work(b, rows):
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


def workload_report(name, steps, warmup, dev, flush=True):
    """Per-call times of one named workload (each call timed with events on
    its stream), with algorithmic TFLOP/s, GB/s and roofline fractions."""
    import torch

    import workloads as W
    from harness import run_decode, run_prefill

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
        workload_report(args.workload, args.steps, args.warmup, dev, flush=not args.no_flush)
        return
    t_gen = time.perf_counter()
    pre_cpu = W.build(PREFILL)
    dec_cpu = W.build(DECODE)
    pre = pre_cpu.to(dev)
    dec = dec_cpu.to(dev)
    print(f"[bench] inputs ready in {time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)

    splits = rba.plan_splits(dec.Hq, dec.Hkv, dec.dv, dec.R, dec.W, dec.scale, len(dec.q_lens), dec.n_q,
                             dec.max_seq_len, torch.cuda.get_device_properties(dev).multi_processor_count)
    ws = torch.empty(rba.workspace_size(dec.Hq, dec.Hkv, dec.dv, dec.R, dec.W, dec.scale, len(dec.q_lens),
                                        dec.n_q, dec.max_seq_len, splits), dtype=torch.uint8, device=dev)
    pre_out = torch.empty((pre.rows, pre.Hq, pre.dv), dtype=torch.float32, device=dev)
    dec_out = torch.empty((dec.rows, dec.Hq, dec.dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def prefill_call():
        rba.prefill(pre.q, pre.k_cache, pre.v_cache, pre.rel, pre.cu_q, pre.seq_lens, pre.block_tables,
                    window=pre.W, scale=pre.scale, max_q_len=pre.max_q_len, max_seq_len=pre.max_seq_len,
                    out=pre_out, stream=stream)

    def split_call():
        rba.decode_split(dec.q, dec.k_cache, dec.v_cache, dec.rel, dec.seq_lens, dec.block_tables,
                         n_q=dec.n_q, window=dec.W, scale=dec.scale, max_seq_len=dec.max_seq_len,
                         num_splits=splits, workspace=ws, stream=stream)

    def combine_call():
        rba.decode_combine(Hq=dec.Hq, Hkv=dec.Hkv, dv=dec.dv, rel_extent=dec.R, window=dec.W,
                           scale=dec.scale, batch=len(dec.q_lens), n_q=dec.n_q, num_splits=splits,
                           workspace=ws, out=dec_out, stream=stream)

    calls = [("prefill", prefill_call), ("decode_split", split_call), ("decode_combine", combine_call)]
    if args.copy_probe_mib > 0:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        for _, fn in calls:
            fn()
    torch.cuda.synchronize()

    events = {name: [] for name, _ in calls}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for name, fn in calls:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            events[name].append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {name: sum(a.elapsed_time(b) for a, b in ev) / len(ev) for name, ev in events.items()}
    ms_per_step = 1e3 * wall / args.steps

    f_pre, b_pre, _ = algorithmic(pre_cpu, "prefill")
    f_dec, b_dec, b_split = algorithmic(dec_cpu, "decode")
    t_pre = ms["prefill"] / 1e3
    t_split = ms["decode_split"] / 1e3
    t_dec = (ms["decode_split"] + ms["decode_combine"]) / 1e3
    roof_pre, roof_dec = roof_time(f_pre, b_pre), roof_time(f_dec, b_dec)
    value = 100.0 * (roof_pre + roof_dec) / (t_pre + t_dec)

    # dominant kernel: the one with the larger share of the step
    if t_split >= t_pre:
        achieved = b_split / t_split / 1e9
        # G * n_q <= 16 runs the 16-column split kernel
        kname = "decode16_split_kernel<128, false>" if dec.Hq // dec.Hkv * dec.n_q <= 16 else "decode_split_kernel<128, false>"
        roofline = {"kernel": kname, "bound": "hbm", "achieved": round(achieved, 1),
                    "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": round(achieved / (PEAK_HBM / 1e9), 4),
                    "traffic": measured_traffic(), "algorithmic_bytes_per_launch": b_split,
                    "avg_launch_ms": round(ms["decode_split"], 4)}
    else:
        achieved = b_pre / t_pre / 1e9
        pname = "prefill_kernel<128, true>" if pre.W > 0 else "prefill_kernel<128, false>"
        roofline = {"kernel": pname, "bound": "hbm", "achieved": round(achieved, 1),
                    "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": round(achieved / (PEAK_HBM / 1e9), 4),
                    "traffic": None, "algorithmic_bytes_per_launch": b_pre,
                    "avg_launch_ms": round(ms["prefill"], 4)}

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
            "workload": f"{PREFILL} + {DECODE}",
            "prefill": {"seq_len": pre.max_seq_len, "Hq": pre.Hq, "Hkv": pre.Hkv, "head_dim": DQK,
                        "dv": pre.dv, "window": pre.W, "rel_extent": pre.R, "block_size": 128},
            "decode": {"batch": len(dec.q_lens), "n_q": dec.n_q, "seq_lens_sum": int(sum(dec_cpu.seq_lens.tolist())),
                       "Hq": dec.Hq, "Hkv": dec.Hkv, "dv": dec.dv, "rel_extent": dec.R, "splits": splits,
                       "block_size": 128},
        },
        "prefill": {"ms": round(ms["prefill"], 4), "tflops": round(f_pre / t_pre / 1e12, 2),
                    "gbps": round(b_pre / t_pre / 1e9, 1), "frac_mfma": round(f_pre / t_pre / PEAK_MFMA_BF16, 4),
                    "frac_hbm": round(b_pre / t_pre / PEAK_HBM, 4), "flops": f_pre, "bytes": b_pre},
        "decode": {"ms": round(t_dec * 1e3, 4), "split_ms": round(ms["decode_split"], 4),
                   "combine_ms": round(ms["decode_combine"], 4), "gbps": round(b_dec / t_dec / 1e9, 1),
                   "frac_hbm": round(b_dec / t_dec / PEAK_HBM, 4), "flops": f_dec, "bytes": b_dec},
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the float64 oracle on a sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(pre_cpu, dec_cpu, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

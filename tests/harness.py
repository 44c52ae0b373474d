"""Test/bench glue: run the library on a workloads.Batch and run the oracle on
the same inputs. Test infrastructure (it imports the oracle)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads
from relative_position_bias_amd import rba

TOL_MAX = 1.5e-2   # max |gpu - oracle| over every compared element
TOL_MEAN = 2e-3    # mean |gpu - oracle|


def oracle_batch(batch: workloads.Batch, rows=None, form="dense"):
    """Float64 oracle on a CPU Batch, one sequence at a time (paging undone by
    a plain gather of that sequence's blocks). rows: optional global rows,
    computed with the dense row form of the oracle (form="dense"; each
    sampled row at position i sees keys 0..i of its sequence) or one row at a
    time by the loop form (form="loop"); without rows every row is computed by
    the loop form."""
    total = batch.rows
    out = np.full((total, batch.Hq, batch.dv), np.nan)
    lse = np.full((total, batch.Hq), np.nan)
    want = None if rows is None else set(int(r) for r in rows)
    kw = dict(rel_extent=batch.R, window=batch.W, scale=batch.scale)

    def rel_rows(a, b_):
        if batch.rel is not None:
            return batch.rel[a:b_].double().numpy()
        return oracle.rel_from_proj(batch.r[a:b_].double().numpy(), batch.proj.double().numpy())
    start = 0
    for b, ql in enumerate(batch.q_lens):
        L = int(batch.seq_lens[b])
        local = None
        if want is not None:
            local = [r - start for r in range(start, start + ql) if r in want]
            if not local:
                start += ql
                continue
        nb = (L + workloads.BLOCK - 1) // workloads.BLOCK
        blocks = batch.block_tables[b, :nb].long()
        if batch.kv_fp8:  # e4m3 bytes times the per-tensor scale
            kb = oracle.e4m3_to_float(batch.k_cache[blocks].numpy()) * batch.k_scale
            vb = oracle.e4m3_to_float(batch.v_cache[blocks].numpy()) * batch.v_scale
        else:
            kb = batch.k_cache[blocks].double().numpy()
            vb = batch.v_cache[blocks].double().numpy()
        k = oracle.unpage(kb, [list(range(nb))], [L])
        v = oracle.unpage(vb, [list(range(nb))], [L])
        def gated(a, b_):
            return dict(sink=batch.sink[a:b_].double().numpy() if batch.sink is not None else None,
                        gate=batch.gate[a:b_].double().numpy() if batch.gate is not None else None,
                        logit_scale=batch.lscale[a:b_].double().numpy() if batch.lscale is not None else None)
        if local is None:
            o, l = oracle.attend(batch.q[start:start + ql].double().numpy(), k, v,
                                 rel_rows(start, start + ql), [ql], [L], **kw,
                                 **gated(start, start + ql))
            out[start:start + ql] = o
            lse[start:start + ql] = l
        elif form == "loop":
            for r in local:
                i = L - ql + r
                t = start + r
                o, l = oracle.attend(batch.q[t:t + 1].double().numpy(), k[:i + 1], v[:i + 1],
                                     rel_rows(t, t + 1), [1], [i + 1], **kw, **gated(t, t + 1))
                out[t] = o[0]
                lse[t] = l[0]
        else:
            # sampled rows: the dense row form of the oracle (pinned to the
            # loop form on the CPU), one matmul per group of rows and head
            ts = np.asarray([start + r for r in local], dtype=np.int64)
            g = gated(0, batch.rows)
            sub = {n: (a[ts] if a is not None else None) for n, a in g.items()}
            if batch.rel is not None:
                rel_s = batch.rel[torch.from_numpy(ts)].double().numpy()
            else:
                rel_s = oracle.rel_from_proj(batch.r[torch.from_numpy(ts)].double().numpy(),
                                             batch.proj.double().numpy())
            o, l = oracle.attend_rows_dense(batch.q[torch.from_numpy(ts)].double().numpy(), k, v, rel_s,
                                            L - ql + np.asarray(local), **kw, **sub)
            out[ts] = o
            lse[ts] = l
        start += ql
    return out, lse


def run_prefill(b: workloads.Batch, want_lse=False, **kw):
    if b.kv_fp8:
        kw.setdefault("kv_scales", (b.k_scale, b.v_scale))
    if b.sink is not None:
        kw.setdefault("sink", b.sink)
    if b.gate is not None:
        kw.setdefault("gate", b.gate)
    if b.lscale is not None:
        kw.setdefault("logit_scale", b.lscale)
    if b.r is not None:
        return rba.prefill_relproj(b.q, b.k_cache, b.v_cache, b.r, b.proj, b.cu_q, b.seq_lens, b.block_tables,
                                   window=b.W, scale=b.scale, max_q_len=b.max_q_len,
                                   max_seq_len=b.max_seq_len, want_lse=want_lse, **kw)
    return rba.prefill(b.q, b.k_cache, b.v_cache, b.rel, b.cu_q, b.seq_lens, b.block_tables,
                       window=b.W, scale=b.scale, max_q_len=b.max_q_len, max_seq_len=b.max_seq_len,
                       want_lse=want_lse, **kw)


def run_decode(b: workloads.Batch, num_splits=0, want_lse=False, **kw):
    if b.kv_fp8:
        kw.setdefault("kv_scales", (b.k_scale, b.v_scale))
    if b.sink is not None:
        kw.setdefault("sink", b.sink)
    if b.gate is not None:
        kw.setdefault("gate", b.gate)
    if b.lscale is not None:
        kw.setdefault("logit_scale", b.lscale)
    if b.r is not None:
        return rba.decode_relproj(b.q, b.k_cache, b.v_cache, b.r, b.proj, b.seq_lens, b.block_tables, n_q=b.n_q,
                                  window=b.W, scale=b.scale, max_seq_len=b.max_seq_len, num_splits=num_splits,
                                  want_lse=want_lse, **kw)
    return rba.decode(b.q, b.k_cache, b.v_cache, b.rel, b.seq_lens, b.block_tables, n_q=b.n_q,
                      window=b.W, scale=b.scale, max_seq_len=b.max_seq_len, num_splits=num_splits,
                      want_lse=want_lse, **kw)


def run(b: workloads.Batch, **kw):
    return run_prefill(b, **kw) if b.kind == "prefill" else run_decode(b, **kw)


def errors(gpu_out: torch.Tensor, ref: np.ndarray, rows=None):
    g = gpu_out.detach().float().cpu().numpy().astype(np.float64)
    if rows is not None:
        g, ref = g[rows], ref[rows]
    if not np.isfinite(g).all():
        return float("inf"), float("inf")
    d = np.abs(g - ref)
    return float(d.max()), float(d.mean())


def assert_close(gpu_out, ref, rows=None, what=""):
    mx, mean = errors(gpu_out, ref, rows)
    assert mx <= TOL_MAX and mean <= TOL_MEAN, f"{what}: max {mx:.3e} mean {mean:.3e}"
    return mx, mean


def sample_rows(batch: workloads.Batch, per_edge=16, extra=16, seed=0):
    """Rows the oracle computes one by one on large inputs: the first and last
    rows of each sequence, rows whose distance to the first key crosses R or W,
    and a seeded random sample."""
    rng = np.random.default_rng(seed)
    rows, start = set(), 0
    for b, ql in enumerate(batch.q_lens):
        L = int(batch.seq_lens[b])
        ctx = L - ql
        rows.update(range(start, start + min(per_edge, ql)))
        rows.update(range(start + max(0, ql - per_edge), start + ql))
        for edge in (batch.R, batch.W):
            if edge and ctx < edge < L:
                r0 = start + (edge - ctx)
                rows.update(r for r in range(r0 - 4, r0 + 4) if start <= r < start + ql)
        rows.update((start + rng.integers(0, ql, size=min(extra, ql))).tolist())
        start += ql
    return sorted(rows)


def tile_sample_rows(batch: workloads.Batch, edge=256, tile=64, per_tile=2, seed=0):
    """Rows of a long prefill call to check against the oracle: per sequence
    the first and last `edge` rows (whole query tiles at both ends), `per_tile`
    seeded rows from every `tile`-row query tile, and the rows whose position
    lies within 4 of the extent R or the window W (where the bias or the
    visible range ends)."""
    rng = np.random.default_rng(seed)
    rows, start = set(), 0
    for b, ql in enumerate(batch.q_lens):
        L = int(batch.seq_lens[b])
        ctx = L - ql
        rows.update(range(start, start + min(edge, ql)))
        rows.update(range(start + max(0, ql - edge), start + ql))
        for t0 in range(0, ql, tile):
            n = min(tile, ql - t0)
            rows.update((start + t0 + rng.choice(n, size=min(per_tile, n), replace=False)).tolist())
        for e in (batch.R, batch.W):
            if e and ctx < e + 4 and e - 4 < L:
                rows.update(start + p - ctx for p in range(e - 4, e + 4) if ctx <= p < L)
        start += ql
    return sorted(rows)


def bf16_p_bound(batch: workloads.Batch, rows=None, slack=1e-5):
    """Per-element bound on |o1 - o2| for two GPU results of the same call
    that differ only in the reference against which P is rounded to bf16
    (another split count, another block order). Each result is
    sum_j p~_j v_j / sum_j p_j with |p~_j - p_j| <= 2^-8 p_j (round to nearest
    even with 8 significant bits: the unit roundoff is 2^-8), so it lies
    within 2^-8 * E_p|v| of the exact value, E_p|v| being the softmax-weighted
    mean of |v|: the oracle run on |V|. Two results differ by at most
    2^-7 * E_p|v|, plus fp32 rounding (`slack`). bf16 caches only."""
    babs = workloads.Batch(**{**batch.__dict__, "v_cache": batch.v_cache.abs()})
    ev, _ = oracle_batch(babs, rows)
    return 2.0 ** -7 * ev + slack

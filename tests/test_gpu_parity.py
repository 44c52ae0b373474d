"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Bar: max |gpu - oracle| <= 1.5e-2 and mean <= 2e-3 on bf16 inputs (fp32
output), every output finite. Small cases are compared element by element on
every row; the full-size workloads either fully (when the oracle finishes in
seconds) or on sampled rows that always include each sequence's first and
last rows and the rows around the distance R / W edges.
"""
import os
import sys

import numpy as np
import pytest
import torch

import workloads as W
from harness import (assert_close, bf16_p_bound, errors, oracle_batch, run, run_decode, run_prefill,
                     sample_rows, tile_sample_rows)
from relative_position_bias_amd import rba

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_vs_oracle(b_cpu, rows=None, what="", **kw):
    b = b_cpu.to(DEV)
    out, lse = run(b, want_lse=True, **kw)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_batch(b_cpu, rows=rows)
    mx, mean = assert_close(out, ref, rows, what)
    lmx, _ = errors(lse, ref_lse, rows)
    assert lmx <= 1e-3, f"{what}: lse max err {lmx:.3e}"
    return out, mx, mean


# ---------------------------------------------------------------------------
# small prefill cases: several tiles, ragged tails, every row compared
# ---------------------------------------------------------------------------
PREFILL_GRID = [
    # q_lens, ctx_lens, Hq, Hkv, dv, R, W
    ([256], [0], 4, 1, 128, 128, 64),          # the tiny workload's shape
    ([200, 77], [0, 300], 8, 2, 128, 64, 0),
    ([130], [1000], 8, 2, 64, 128, 100),
    ([1], [0], 4, 4, 128, 4, 0),               # one token, G = 1
    ([300], [33], 16, 2, 128, 256, 0),         # G = 8
    ([97, 5, 64], [31, 400, 0], 12, 2, 128, 40, 37),  # G = 6, odd window
    ([64], [4096], 4, 1, 64, 1024, 0),         # chunk over a long context
    ([333], [0], 2, 2, 128, 8, 1),             # window of 1: only the key itself
    ([0, 50, 0, 70], [10, 20, 5, 0], 8, 2, 128, 64, 0),  # sequences with no new tokens
    ([64, 128], [64, 0], 8, 2, 64, 128, 0),    # tile-aligned, no ragged tail
]


@pytest.mark.parametrize("case", PREFILL_GRID, ids=lambda c: f"q{c[0]}ctx{c[1]}H{c[2]}/{c[3]}dv{c[4]}R{c[5]}W{c[6]}")
def test_prefill_small(case):
    q_lens, ctx, Hq, Hkv, dv, R, Wn = case
    say(f"prefill small {case}")
    b = W.make_prefill(11, q_lens, ctx, Hq, Hkv, dv, R, Wn)
    gpu_vs_oracle(b, what=str(case))


# Without a window the prefill walks a tile's blocks whole up to the first
# block in which some row of the tile has bias, and the rest in half blocks
# through the bias ring. The switch depends on the tile's first position i_lo:
# the first subtile with bias starts at the multiple of 32 above i_lo - 31 - R.
# With R = 256 and one 64-row tile per sequence (G = 4), the contexts below
# put it at the first block (100, 286, 287), at each 32-key offset inside a
# block (383, 415, 447, 479) and after one, two or three whole blocks (383,
# 511, 543, 639: odd and even counts, which use the two whole-block buffers
# in the other order), and late in a long context (1200, 3001). R = 1 leaves
# bias on the diagonal subtiles only; R = 2000 puts it on every block.
TAIL_SWITCH = [
    # q_lens, ctx_lens, dv, R
    ([64] * 12, [100, 286, 287, 383, 415, 447, 479, 511, 543, 639, 1200, 3001], 128, 256),
    ([200, 130], [0, 1000], 128, 256),
    ([64, 150], [700, 2000], 64, 1),
    ([100, 64], [300, 1500], 64, 2000),
]


@pytest.mark.parametrize("kv_fp8", [False, True], ids=["bf16", "e4m3"])
@pytest.mark.parametrize("case", TAIL_SWITCH, ids=lambda c: f"dv{c[2]}R{c[3]}_{len(c[0])}seq")
def test_prefill_whole_blocks_then_ring(case, kv_fp8):
    q_lens, ctx, dv, R = case
    say(f"prefill whole blocks then ring {case} e4m3={kv_fp8}")
    b = W.make_prefill(12, q_lens, ctx, 8, 2, dv, R, 0, kv_fp8=kv_fp8)
    gpu_vs_oracle(b, what=f"{case} e4m3={kv_fp8}")


def test_tiny_prefill_workload():
    say("tiny_prefill_256")
    gpu_vs_oracle(W.build("tiny_prefill_256"), what="tiny")


def test_local_prefill_8k_full():
    say("local_prefill_8k (all rows)")
    _, mx, mean = gpu_vs_oracle(W.build("local_prefill_8k"), what="local 8k")
    say(f"  max {mx:.3e} mean {mean:.3e}")


def test_global_chunked_prefill_sampled():
    name = "global_chunked_prefill_32k"
    full = W.build(name)
    full_gpu = full.to(DEV)
    for c, (ch_cpu, ch) in enumerate(zip(W.chunks(name, full), W.chunks(name, full_gpu))):
        say(f"chunk {c}")
        out, _ = run_prefill(ch)
        torch.cuda.synchronize()
        # every row of the first and last 256 of the chunk (its first and
        # last four 64-row query tiles), two seeded rows of every 64-row
        # tile, and the rows within 4 of position R
        rows = tile_sample_rows(ch_cpu, seed=c)
        ref, _ = oracle_batch(ch_cpu, rows=rows)
        mx, mean = assert_close(out, ref, rows, f"chunk {c}")
        say(f"  rows {len(rows)} max {mx:.3e} mean {mean:.3e}")
        assert torch.isfinite(out).all()


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
DECODE_GRID = [
    # batch, n_q, lens, Hq, Hkv, dv, R, W, pool
    (3, 1, [129, 1000, 5000], 32, 8, 128, 1024, 0, None),
    (2, 4, [700, 4096], 64, 8, 64, 1024, 0, None),
    (4, 3, [3, 250, 520, 1300], 16, 4, 128, 256, 300, None),
    (2, 8, [900, 2000], 48, 8, 128, 512, 0, None),      # G = 6, 48 columns: 2 column groups
    (5, 2, [128, 256, 384, 4000, 77], 8, 8, 64, 64, 128, 64),   # G = 1, aliased pool
    (2, 4, [300, 1100], 16, 4, 128, 256, 0, None),      # G * n_q = 16: the 16-column kernel's limit
    (2, 5, [300, 1100], 16, 4, 64, 256, 0, None),       # G * n_q = 20: the 32-column kernel, one group
    (2, 4, [4, 1000], 16, 4, 128, 256, 0, None),        # a sequence holding only its n_q new tokens
    (2, 4, [700, 4096], 64, 8, 64, 1024, 300, None),    # 32 columns, dv 64, window
    (2, 3, [700, 3000], 64, 2, 64, 1024, 0, None),      # G = 32, 96 columns: three column groups
    (3, 2, [130, 900, 2600], 64, 2, 128, 256, 384, None),  # 64 columns: two column groups, dv 128, window
    (1, 16, [2000], 128, 8, 64, 1024, 0, None),         # G * n_q = 256, the largest accepted: 8 groups
]


@pytest.mark.parametrize("case", DECODE_GRID, ids=lambda c: f"B{c[0]}nq{c[1]}H{c[3]}/{c[4]}dv{c[5]}W{c[7]}")
@pytest.mark.parametrize("splits", [1, 3, 0])
def test_decode_small(case, splits):
    batch, n_q, lens, Hq, Hkv, dv, R, Wn, pool = case
    say(f"decode small {case} splits={splits}")
    b = W.make_decode(21, batch, n_q, Hq, Hkv, dv, R, Wn, seq_lens=lens, pool_blocks=pool)
    gpu_vs_oracle(b, what=f"{case} s{splits}", num_splits=splits)


def test_paged_decode_16_workload():
    say("paged_decode_16x8k_128k (aliased 2560-block pool)")
    _, mx, mean = gpu_vs_oracle(W.build("paged_decode_16x8k_128k"), what="decode16")
    say(f"  max {mx:.3e} mean {mean:.3e}")


def test_paged_decode_16_disjoint_workload():
    say("paged_decode_16x8k_128k_disjoint")
    _, mx, mean = gpu_vs_oracle(W.build("paged_decode_16x8k_128k_disjoint"), what="decode16 disjoint")
    say(f"  max {mx:.3e} mean {mean:.3e}")


@pytest.mark.parametrize("splits", [1, 2, 5, 17, 40])
@pytest.mark.parametrize("fp8", [False, True])
def test_decode_dv64_one_and_two_workgroups_per_cu(splits, fp8):
    """The 32-column dv-64 decode over e4m3 K/V runs 8-wave workgroups (even
    and odd blocks on two wave groups) when its grid fits one workgroup per
    CU, else 4-wave ones, as over bf16 K/V: 2 x 8 x splits workgroups cross
    256 between 5 and 17 splits. Odd block counts per split leave the
    odd-block waves one block short, and the 700-token sequence leaves some
    splits empty."""
    say(f"decode dv64 splits={splits} fp8={fp8}")
    b = W.make_decode(41, 2, 4, 64, 8, 64, 1024, 0, seq_lens=[700, 4096], kv_fp8=fp8)
    gpu_vs_oracle(b, what=f"dv64 s{splits} fp8{int(fp8)}", num_splits=splits)


@pytest.mark.parametrize("name", ["verify_decode_b1_100k", "verify_decode_b8_100k"])
def test_verify_decode_workloads(name):
    say(name)
    _, mx, mean = gpu_vs_oracle(W.build(name), what=name)
    say(f"  max {mx:.3e} mean {mean:.3e}")


# ---------------------------------------------------------------------------
# decode over e4m3 (FP8) K/V caches
# ---------------------------------------------------------------------------
FP8_GRID = [
    # (batch, n_q, seq_lens, Hq, Hkv, dv, R, W)
    (3, 1, [129, 1000, 5000], 32, 8, 128, 1024, 0),   # G * n_q = 4: the 16-column kernel
    (2, 4, [300, 1100], 16, 4, 64, 256, 0),            # 16-column kernel, dv 64
    (2, 4, [700, 4096], 64, 8, 64, 1024, 0),           # G * n_q = 32: 32-column kernel with prefetch
    (2, 8, [900, 2000], 48, 8, 128, 512, 0),           # 48 columns, dv 128: two groups, no prefetch
    (4, 3, [3, 250, 520, 1300], 16, 4, 128, 256, 300), # window; a sequence shorter than a block
    (2, 4, [700, 2000], 64, 4, 64, 1024, 0),           # 64 columns, dv 64: two column groups
]


@pytest.mark.parametrize("case", FP8_GRID, ids=lambda c: f"B{c[0]}nq{c[1]}H{c[3]}/{c[4]}dv{c[5]}W{c[7]}")
@pytest.mark.parametrize("splits", [1, 0])
def test_decode_fp8_small(case, splits):
    batch, n_q, lens, Hq, Hkv, dv, R, Wn = case
    say(f"decode fp8 {case} splits={splits}")
    b = W.make_decode(31, batch, n_q, Hq, Hkv, dv, R, Wn, seq_lens=lens, kv_fp8=True)
    gpu_vs_oracle(b, what=f"fp8 {case} s{splits}", num_splits=splits)


def test_decode_fp8_equals_bf16_on_dequantized_cache():
    """Same attention as the bf16 path over caches holding the dequantized
    values (exact in bf16 for the workloads' scales). Only the place where the
    scales are applied differs: K's is folded into the score scale, V's into
    the split outputs, so the two agree to fp32 rounding."""
    say("fp8 vs bf16 on the dequantized cache")
    b8 = W.make_decode(33, 3, 2, 32, 8, 128, 1024, 0, seq_lens=[500, 3000, 9000], kv_fp8=True)
    k = (b8.k_cache.view(torch.float8_e4m3fn).float() * b8.k_scale).to(torch.bfloat16)
    v = (b8.v_cache.view(torch.float8_e4m3fn).float() * b8.v_scale).to(torch.bfloat16)
    bb = W.Batch(**{**b8.__dict__, "k_cache": k, "v_cache": v, "kv_fp8": False, "k_scale": 1.0,
                    "v_scale": 1.0})
    o8, l8 = run_decode(b8.to(DEV), want_lse=True)
    ob, lb = run_decode(bb.to(DEV), want_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o8).all()
    assert float((o8 - ob).abs().max()) <= 4e-3 and float((o8 - ob).abs().mean()) <= 1e-4
    assert float((l8 - lb).abs().max()) <= 1e-4


@pytest.mark.parametrize("name", ["paged_decode_16x8k_128k_disjoint_fp8", "verify_decode_b1_100k_fp8",
                                  "verify_decode_b8_100k_fp8"])
def test_fp8_decode_workloads(name):
    say(name)
    _, mx, mean = gpu_vs_oracle(W.build(name), what=name)
    say(f"  max {mx:.3e} mean {mean:.3e}")


# ---------------------------------------------------------------------------
# gated attention output (sink logit + sigmoid gate, Inkling 2 Small)
# ---------------------------------------------------------------------------
GATED_PREFILL = [
    # (q_lens, ctx_lens, Hq, Hkv, dv, R, W)
    ([200, 77], [0, 300], 48, 8, 128, 1024, 0),    # 6:1 GQA, no window
    ([130, 64], [1000, 0], 48, 8, 128, 1024, 96),  # window
    ([97], [31], 8, 2, 64, 128, 0),                # dv 64
]


@pytest.mark.parametrize("case", GATED_PREFILL, ids=lambda c: f"q{c[0]}H{c[2]}/{c[3]}dv{c[4]}W{c[6]}")
def test_prefill_gated_small(case):
    q_lens, ctx, Hq, Hkv, dv, R, Wn = case
    say(f"prefill gated {case}")
    gpu_vs_oracle(W.make_prefill(41, q_lens, ctx, Hq, Hkv, dv, R, Wn, gated=True), what=f"gated {case}")


GATED_DECODE = [
    # (batch, n_q, seq_lens, Hq, Hkv, dv, R, W, kv_fp8)
    (2, 8, [900, 3000], 48, 8, 128, 1024, 0, False),   # 48 columns: two 32-column groups
    (2, 8, [900, 3000], 48, 8, 128, 1024, 0, True),
    (3, 1, [129, 1000, 5000], 32, 8, 128, 1024, 300, False),  # 16-column kernel, window
    (2, 4, [700, 2000], 64, 8, 64, 1024, 0, True),
]


@pytest.mark.parametrize("case", GATED_DECODE, ids=lambda c: f"B{c[0]}nq{c[1]}H{c[3]}/{c[4]}W{c[7]}fp8{int(c[8])}")
@pytest.mark.parametrize("splits", [1, 0])
def test_decode_gated_small(case, splits):
    batch, n_q, lens, Hq, Hkv, dv, R, Wn, fp8 = case
    say(f"decode gated {case} splits={splits}")
    b = W.make_decode(43, batch, n_q, Hq, Hkv, dv, R, Wn, seq_lens=lens, kv_fp8=fp8, gated=True)
    gpu_vs_oracle(b, what=f"gated {case} s{splits}", num_splits=splits)


def test_gated_without_sink_or_gate_is_the_plain_path():
    """sink = -inf and gate = +inf everywhere reproduce the ungated calls bitwise."""
    say("gated, neutral inputs")
    b = W.make_prefill(45, [150, 40], [60, 0], 16, 4, 128, 256, 0).to(DEV)
    neg = torch.full((b.rows, b.Hq), -float("inf"), device=DEV)
    pos = torch.full((b.rows, b.Hq), float("inf"), device=DEV)
    o1, l1 = run_prefill(b, want_lse=True)
    o2, l2 = run_prefill(b, want_lse=True, sink=neg, gate=pos)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    d = W.make_decode(45, 2, 2, 16, 4, 128, 256, 0, seq_lens=[300, 2000]).to(DEV)
    neg = torch.full((d.rows, d.Hq), -float("inf"), device=DEV)
    pos = torch.full((d.rows, d.Hq), float("inf"), device=DEV)
    o1, l1 = run_decode(d, num_splits=3, want_lse=True)
    o2, l2 = run_decode(d, num_splits=3, want_lse=True, sink=neg, gate=pos)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_inkling2_gated_local_prefill_sampled():
    name = "inkling2_local_prefill_8k_gated"
    say(name)
    b = W.build(name)
    rows = sample_rows(b)
    _, mx, mean = gpu_vs_oracle(b, rows=rows, what=name)
    say(f"  {len(rows)} rows: max {mx:.3e} mean {mean:.3e}")


def test_inkling2_gated_verify_decode():
    name = "inkling2_verify_b1_100k_gated"
    say(name)
    _, mx, mean = gpu_vs_oracle(W.build(name), what=name)
    say(f"  max {mx:.3e} mean {mean:.3e}")


# ---------------------------------------------------------------------------
# invariants on the GPU
# ---------------------------------------------------------------------------
def test_split_count_invariance():
    """Different split counts agree: lse (built from fp32 sums) to fp32
    rounding; out element by element within the bf16 rounding of P, which is
    taken relative to each split's own reference max: |o1 - o2| <=
    2^-7 * E_p|v| + 1e-5, E_p|v| being the softmax-weighted mean of |v| (the
    oracle on |V|), under the 1.5e-2 parity bar on these inputs."""
    say("split invariance")
    b_cpu = W.make_decode(5, 2, 2, 32, 8, 128, 1024, 0, seq_lens=[3000, 7000])
    b = b_cpu.to(DEV)
    outs = []
    for s in (1, 2, 0, 55, 300):  # 300: more splits than blocks (empty splits) and than one combine pass
        o, l = run_decode(b, num_splits=s, want_lse=True)
        outs.append((o.clone(), l.clone()))
    bound = torch.from_numpy(bf16_p_bound(b_cpu)).float()
    assert float(bound.max()) < 1.5e-2
    for o, l in outs[1:]:
        d = (o - outs[0][0]).abs().cpu()
        assert bool((d <= bound).all()), f"max excess {float((d - bound).max()):.3e}"
        assert float(d.mean()) <= 2e-4
        assert torch.allclose(l, outs[0][1], rtol=0, atol=2e-5)


def test_block_permutation_is_bitwise_invariant():
    say("block permutation")
    b = W.make_prefill(3, [300, 90], [100, 700], 8, 2, 128, 128, 0, extra_blocks=5)
    o1, _ = run_prefill(b.to(DEV))
    perm = torch.randperm(b.k_cache.shape[0], generator=torch.Generator().manual_seed(9))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(perm.numel())
    b2 = W.Batch(**{**b.__dict__})
    b2.k_cache = b.k_cache[perm].contiguous()
    b2.v_cache = b.v_cache[perm].contiguous()
    t = b.block_tables.clone().long()
    b2.block_tables = torch.where(t >= 0, inv[t.clamp(min=0)], t).to(torch.int32)
    o2, _ = run_prefill(b2.to(DEV))
    assert torch.equal(o1, o2)


def test_window_blocks_outside_are_never_read():
    """Blocks wholly outside every query's window: table entry -1 or NaN
    poison leave the output bitwise unchanged (the local-window equivalence)."""
    say("window skipping")
    Wn = 200
    b = W.make_prefill(4, [150], [1500], 8, 2, 128, 128, Wn)
    o1, _ = run_prefill(b.to(DEV))
    first_needed = (1500 - Wn + 1) // 128
    b2 = W.Batch(**{**b.__dict__})
    b2.block_tables = b.block_tables.clone()
    b2.k_cache = b.k_cache.clone()
    b2.v_cache = b.v_cache.clone()
    for n in range(first_needed):
        blk = int(b.block_tables[0, n])
        b2.k_cache.view(torch.int16)[blk] = W.BF16_NAN
        b2.v_cache.view(torch.int16)[blk] = W.BF16_NAN
    o2, _ = run_prefill(b2.to(DEV))
    b2.block_tables[0, :first_needed] = -1
    o3, _ = run_prefill(b2.to(DEV))
    assert torch.equal(o1, o2) and torch.equal(o1, o3)


def test_chunked_prefill_is_bitwise_equal_to_one_shot():
    say("chunking")
    full = W.make_prefill(6, [512], [0], 8, 2, 128, 256, 0).to(DEV)
    o_full, _ = run_prefill(full)
    parts = [run_prefill(W.chunk_of(full, c, 128))[0] for c in range(4)]
    assert torch.equal(torch.cat(parts), o_full)


def test_windowed_chunked_prefill_within_the_bf16_p_bound():
    """With a window, a tile starts at the first 64-key stage that any of its
    rows can see. A chunk's tiles start at other rows than the one-shot
    call's, so a row's keys may be visited from another first stage and P
    rounded against other running references: the two agree element by
    element within the bf16-P bound (2^-7 E_p|v|), not bitwise."""
    say("chunking, windowed")
    full_cpu = W.make_prefill(6, [640], [0], 8, 2, 128, 256, 300)
    full = full_cpu.to(DEV)
    o_full, l_full = run_prefill(full, want_lse=True)
    parts = [run_prefill(W.chunk_of(full, c, 160), want_lse=True) for c in range(4)]
    o_ch = torch.cat([p[0] for p in parts])
    l_ch = torch.cat([p[1] for p in parts])
    bound = torch.from_numpy(bf16_p_bound(full_cpu)).float()
    d = (o_ch - o_full).abs().cpu()
    assert bool((d <= bound).all()), f"max excess {float((d - bound).max()):.3e}"
    assert torch.allclose(l_ch, l_full, rtol=0, atol=2e-5)


def test_decode_rows_match_prefill_rows():
    say("decode vs prefill rows")
    full = W.make_prefill(8, [600], [0], 16, 4, 128, 256, 0)
    o_pre, _ = run_prefill(full.to(DEV))
    n_q = 3
    dec = W.Batch(kind="decode", Hq=16, Hkv=4, dv=128, R=256, W=0, scale=full.scale,
                  q=full.q[-n_q:].contiguous(), k_cache=full.k_cache, v_cache=full.v_cache,
                  rel=full.rel[-n_q:].contiguous(), seq_lens=full.seq_lens, block_tables=full.block_tables,
                  n_q=n_q, q_lens=[n_q], max_q_len=n_q, max_seq_len=600)
    o_dec, _ = run_decode(dec.to(DEV))
    assert torch.allclose(o_dec, o_pre[-n_q:], rtol=0, atol=2e-3)


def test_shear_probe_selects_exact_value_rows():
    """q = k = 0 and a +40 bias at one visible distance per (row, head): the
    output must be exactly that key's value row (every row's shear offset,
    the GQA map and the paging checked at once)."""
    say("shear probe")
    b = W.make_prefill(12, [100, 37], [50, 222], 8, 2, 128, 96, 0)
    b.q.zero_()
    b.k_cache.zero_()
    rel = torch.zeros_like(b.rel)
    rng = np.random.default_rng(1)
    expect = torch.empty((b.rows, 8, 128))
    kv_tab = b.block_tables
    t = 0
    for s, (ql, L) in enumerate(zip(b.q_lens, b.seq_lens.tolist())):
        for r in range(ql):
            i = L - ql + r
            for h in range(8):
                d0 = int(rng.integers(0, min(i + 1, 96)))
                rel[t, h, d0] = 40.0
                j = i - d0
                blk = int(kv_tab[s, j // 128])
                expect[t, h] = b.v_cache[blk, h // 4, j % 128].float()
            t += 1
    b.rel = rel
    out, _ = run_prefill(b.to(DEV))
    assert torch.allclose(out.cpu(), expect, rtol=0, atol=1e-6)


def test_repeatable_bitwise():
    """50 runs of the same decode and prefill are bitwise identical (no
    atomics, no order that depends on timing)."""
    say("repeatability")
    b = W.make_decode(2, 4, 2, 32, 8, 128, 1024, 0, seq_lens=[9000, 300, 1500, 4100]).to(DEV)
    ref, _ = run_decode(b)
    for _ in range(50):
        o, _ = run_decode(b)
        assert torch.equal(o, ref)
    p = W.make_prefill(2, [500], [700], 8, 2, 128, 512, 300).to(DEV)
    pref, _ = run_prefill(p)
    for _ in range(50):
        assert torch.equal(run_prefill(p)[0], pref)


def test_repeatable_bitwise_e4m3():
    """The same over e4m3 K/V caches: 50 runs of a decode (16- and 32-column
    kernels) and of a prefill are bitwise identical."""
    say("repeatability, e4m3")
    for n_q in (1, 4):
        b = W.make_decode(3, 3, n_q, 32, 8, 128, 1024, 0, seq_lens=[7000, 260, 2100], kv_fp8=True).to(DEV)
        ref, _ = run_decode(b)
        for _ in range(50):
            o, _ = run_decode(b)
            assert torch.equal(o, ref), f"decode n_q={n_q}"
    p = W.make_prefill(3, [300, 77], [900, 0], 8, 2, 128, 512, 0, kv_fp8=True).to(DEV)
    pref, _ = run_prefill(p)
    for _ in range(50):
        assert torch.equal(run_prefill(p)[0], pref)


def test_graph_capture_replay():
    say("graph capture")
    b = W.make_decode(13, 2, 4, 64, 8, 64, 1024, 0, seq_lens=[2000, 5000]).to(DEV)
    ws = torch.empty(rba.workspace_size(64, 8, 64, 1024, 0, b.scale, 2, 4, 5000), dtype=torch.uint8,
                     device=DEV)
    out = torch.empty((8, 64, 64), device=DEV)
    eager, _ = run_decode(b, workspace=ws)
    eager = eager.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run_decode(b, workspace=ws, out=out)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_decode(b, workspace=ws, out=out)
    for _ in range(3):
        out.fill_(7.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
        run_prefill(W.make_prefill(1, [64], [0], 4, 1, 128, 128, 0).to(DEV))   # eager work between


def test_graph_capture_replay_e4m3():
    """A decode and a prefill over e4m3 caches captured in one graph: every
    replay, with eager work between them, reproduces the eager outputs."""
    say("graph capture, e4m3")
    b = W.make_decode(14, 2, 1, 32, 8, 128, 1024, 0, seq_lens=[3000, 9000], kv_fp8=True).to(DEV)
    p = W.make_prefill(14, [200, 64], [500, 1000], 8, 2, 128, 256, 0, kv_fp8=True).to(DEV)
    ws = torch.empty(rba.workspace_size(32, 8, 128, 1024, 0, b.scale, 2, 1, b.max_seq_len), dtype=torch.uint8,
                     device=DEV)
    out_d = torch.empty((2, 32, 128), device=DEV)
    out_p = torch.empty((p.rows, p.Hq, p.dv), device=DEV)
    eager_d = run_decode(b, workspace=ws)[0].clone()
    eager_p = run_prefill(p)[0].clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run_decode(b, workspace=ws, out=out_d)
        run_prefill(p, out=out_p)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_decode(b, workspace=ws, out=out_d)
        run_prefill(p, out=out_p)
    for _ in range(3):
        out_d.fill_(7.0)
        out_p.fill_(7.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_d, eager_d) and torch.equal(out_p, eager_p)
        run_decode(W.make_decode(1, 1, 1, 32, 8, 128, 1024, 0, seq_lens=[500], kv_fp8=True).to(DEV))


@pytest.mark.parametrize("shape", [(1, 8, 2, 128), (4, 64, 8, 64)], ids=["4col_dv128", "32col_dv64"])
def test_invalid_block_id_gives_nan_not_a_fault(shape):
    n_q, Hq, Hkv, dv = shape
    say(f"invalid block id {shape}")
    b = W.make_decode(3, 2, n_q, Hq, Hkv, dv, 64, 0, seq_lens=[500, 600])
    b.block_tables[1, 2] = 10_000          # out of range for this pool
    out, _ = run_decode(b.to(DEV))
    out = out.cpu().view(2, n_q, Hq, dv)   # [sequence, token, head, dv]
    assert torch.isnan(out[1]).all()
    assert torch.isfinite(out[0]).all()

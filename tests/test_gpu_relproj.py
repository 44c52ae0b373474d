"""GPU parity of the prefill that makes its bias in the kernel from the R
branch (rba_prefill_relproj) against the float64 oracle, which forms
rel = r @ rel_logits_proj^T in float64 and then attends.

Same bar as the other parity tests (max 1.5e-2, mean 2e-3, finite). The band
the kernel keeps per wave covers the 63 distances of one 32-key subtile and
is carried from subtile to subtile, so the grid includes runs where the bias
starts mid-sweep (long context, small R), windows narrower and wider than R,
the smallest R, and several GQA ratios (4, 6, 8 query heads per KV head).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from harness import assert_close, bf16_p_bound, errors, oracle_batch, run_prefill, sample_rows, tile_sample_rows
from relative_position_bias_amd import rba

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_vs_oracle(b_cpu, rows=None, what=""):
    b = b_cpu.to(DEV)
    out, lse = run_prefill(b, want_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_batch(b_cpu, rows=rows)
    mx, mean = assert_close(out, ref, rows, what)
    lmx, _ = errors(lse, ref_lse, rows)
    assert lmx <= 1e-3, f"{what}: lse max err {lmx:.3e}"
    return out, mx, mean


RELPROJ_GRID = [
    # q_lens, ctx_lens, Hq, Hkv, dv, R, W, proj_heads
    ([300], [0], 8, 2, 128, 128, 0, 1),              # no window: bias near the diagonal only
    ([257], [200], 8, 2, 64, 96, 160, 8),            # window wider than R, per-head projection
    ([100, 333], [1000, 37], 4, 1, 128, 512, 512, 1),  # local-layer shape, two sequences
    ([200], [70], 12, 2, 128, 200, 0, 12),           # G = 6
    ([130], [4000], 16, 2, 128, 1024, 0, 1),         # G = 8, bias starts mid-sweep
    ([77], [0], 8, 2, 128, 1024, 0, 1),              # R beyond every distance
    ([90], [50], 4, 1, 64, 4, 0, 1),                 # smallest R (a multiple of 4): distances 0..3
    ([150], [20], 8, 2, 128, 300, 33, 1),            # window narrower than R
    ([0, 65, 0], [10, 0, 5], 8, 2, 128, 64, 0, 1),   # sequences with no new tokens
    ([64, 128], [64, 0], 8, 2, 64, 128, 64, 8),      # tile-aligned
]


def _id(c):
    return f"q{c[0]}ctx{c[1]}H{c[2]}/{c[3]}dv{c[4]}R{c[5]}W{c[6]}P{c[7]}"


@pytest.mark.parametrize("case", RELPROJ_GRID, ids=_id)
def test_relproj_small(case):
    q_lens, ctx, Hq, Hkv, dv, R, Wn, Hp = case
    say(f"relproj small {case}")
    b = W.make_prefill(23, q_lens, ctx, Hq, Hkv, dv, R, Wn, d_r=64, proj_heads=Hp)
    gpu_vs_oracle(b, what=str(case))


@pytest.mark.parametrize("d_r", [32, 128])
@pytest.mark.parametrize("case", [RELPROJ_GRID[i] for i in (0, 1, 2, 3, 7)], ids=_id)
def test_relproj_other_r_widths(case, d_r):
    """r of width 32 or 128 (the pages do not give the width of the R branch)."""
    q_lens, ctx, Hq, Hkv, dv, R, Wn, Hp = case
    say(f"relproj d_r={d_r} {case}")
    b = W.make_prefill(24, q_lens, ctx, Hq, Hkv, dv, R, Wn, d_r=d_r, proj_heads=Hp)
    gpu_vs_oracle(b, what=f"d_r={d_r} {case}")


@pytest.mark.parametrize("case", RELPROJ_GRID[:5], ids=_id)
def test_relproj_equals_materialised_bias(case):
    """The same call through rba_prefill with rel formed by the oracle
    (float64, rounded to fp32): the two calls visit the keys in the same
    order (both run the ring body, with or without whole blocks before the
    first block with bias, and differ only in where its bands come from), so
    they differ only by the fp32 rounding of the bias. Element by element
    they must agree within the bf16-P bound (a rounding of some P that the
    bias difference flips costs at most 2^-7 of that weight: |o1 - o2| <=
    2^-7 E_p|v| + 1e-5, E_p|v| the softmax-weighted mean of |v| from the
    oracle on |V|),
    and in the max within 2e-4. lse is built from fp32 sums either way."""
    q_lens, ctx, Hq, Hkv, dv, R, Wn, Hp = case
    say(f"relproj vs rel {case}")
    b_cpu = W.make_prefill(29, q_lens, ctx, Hq, Hkv, dv, R, Wn, d_r=64, proj_heads=Hp)
    rel = torch.from_numpy(oracle.rel_from_proj(b_cpu.r.double().numpy(), b_cpu.proj.double().numpy())).float()
    b = b_cpu.to(DEV)
    o1, l1 = run_prefill(b, want_lse=True)
    o2, l2 = rba.prefill(b.q, b.k_cache, b.v_cache, rel.to(DEV), b.cu_q, b.seq_lens, b.block_tables,
                         window=b.W, scale=b.scale, max_q_len=b.max_q_len, max_seq_len=b.max_seq_len,
                         want_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o1).all()
    diff = (o1 - o2).abs()
    d, dm = diff.max().item(), diff.mean().item()
    dl = (l1 - l2).abs().max().item()
    say(f"  max |relproj - rel| {d:.3e}, mean {dm:.3e}, lse {dl:.3e}")
    bound = torch.from_numpy(bf16_p_bound(b_cpu)).float()
    assert bool((diff.cpu() <= bound).all()), f"max excess {float((diff.cpu() - bound).max()):.3e}"
    assert d <= 2e-4
    assert dl <= 2e-5


def test_shared_projection_equals_replicated_per_head():
    say("shared vs replicated projection")
    b_cpu = W.make_prefill(31, [180], [60], 8, 2, 128, 256, 0, d_r=64, proj_heads=1)
    b = b_cpu.to(DEV)
    o1, l1 = run_prefill(b, want_lse=True)
    b.proj = b.proj.expand(8, -1, -1).contiguous()
    o2, l2 = run_prefill(b, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_relproj_bad_width_is_rejected():
    """Widths other than 32, 64 and 128 are refused before any launch."""
    b = W.make_prefill(3, [40], [0], 4, 1, 128, 32, 0, d_r=64).to(DEV)
    with pytest.raises(rba.RbaError):
        rba.prefill_relproj(
            b.q, b.k_cache, b.v_cache, b.r[:, :, :48].contiguous(), b.proj[:, :, :48].contiguous(), b.cu_q,
            b.seq_lens, b.block_tables, window=0, scale=b.scale, max_q_len=40, max_seq_len=40)


GATED_RELPROJ = [
    ([200, 77], [0, 300], 48, 8, 128, 1024, 0),
    ([130], [1000], 48, 8, 128, 1024, 96),
]


@pytest.mark.parametrize("case", GATED_RELPROJ, ids=lambda c: f"q{c[0]}H{c[2]}/{c[3]}W{c[6]}")
def test_relproj_gated_small(case):
    q_lens, ctx, Hq, Hkv, dv, R, Wn = case
    say(f"relproj gated {case}")
    gpu_vs_oracle(W.make_prefill(43, q_lens, ctx, Hq, Hkv, dv, R, Wn, gated=True, d_r=64),
                  what=f"gated {case}")


def test_local_prefill_8k_relproj_full():
    say("local_prefill_8k_relproj (all rows)")
    _, mx, mean = gpu_vs_oracle(W.build("local_prefill_8k_relproj"), what="local 8k relproj")
    say(f"  max {mx:.3e} mean {mean:.3e}")


def test_global_chunked_prefill_relproj_sampled():
    name = "global_chunked_prefill_32k_relproj"
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

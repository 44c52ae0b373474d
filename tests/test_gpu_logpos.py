"""GPU parity of the per-row logit scale (rba_prefill_logpos, rba_decode_logpos)
against the float64 oracle, which multiplies row t's q and rel by the row's
factor (the log-position scale of global layers, "Inkling-Small on Gaudi 2",
"What was built"; the factor is the caller's, since the pages give no formula).
Same bar as the other parity tests."""
import sys

import pytest
import torch

import workloads as W
from harness import assert_close, errors, oracle_batch, run_decode, run_prefill, sample_rows, tile_sample_rows
from relative_position_bias_amd import rba

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_vs_oracle(b_cpu, rows=None, what="", **kw):
    b = b_cpu.to(DEV)
    run = run_prefill if b.kind == "prefill" else run_decode
    out, lse = run(b, want_lse=True, **kw)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_batch(b_cpu, rows=rows)
    mx, mean = assert_close(out, ref, rows, what)
    lmx, _ = errors(lse, ref_lse, rows)
    assert lmx <= 1e-3, f"{what}: lse max err {lmx:.3e}"
    return out, lse


LOGPOS_PREFILL = [
    # q_lens, ctx_lens, Hq, Hkv, dv, R, W
    ([300], [0], 8, 2, 128, 128, 0),
    ([200, 77], [100, 2000], 8, 2, 64, 256, 0),
    ([257], [300], 12, 2, 128, 512, 160),        # G = 6, window
    ([130], [40], 16, 2, 128, 64, 0),            # G = 8
    ([0, 65], [10, 0], 4, 1, 128, 128, 64),      # an empty sequence
]


@pytest.mark.parametrize("case", LOGPOS_PREFILL, ids=lambda c: f"q{c[0]}H{c[2]}/{c[3]}dv{c[4]}W{c[6]}")
def test_logpos_prefill_small(case):
    q_lens, ctx, Hq, Hkv, dv, R, Wn = case
    say(f"logpos prefill {case}")
    gpu_vs_oracle(W.make_prefill(51, q_lens, ctx, Hq, Hkv, dv, R, Wn, logpos=True), what=str(case))


LOGPOS_DECODE = [
    # batch, n_q, lens, Hq, Hkv, dv, R, W
    (3, 1, [129, 1000, 5000], 32, 8, 128, 1024, 0),    # G * n_q = 4: the 16-column kernel
    (2, 4, [700, 4096], 64, 8, 64, 1024, 0),           # 32 columns
    (2, 8, [900, 2000], 48, 8, 128, 512, 0),           # 48 columns: two groups
    (4, 3, [3, 250, 520, 1300], 16, 4, 128, 256, 300),  # window
]


@pytest.mark.parametrize("case", LOGPOS_DECODE, ids=lambda c: f"B{c[0]}nq{c[1]}H{c[3]}/{c[4]}dv{c[5]}W{c[7]}")
@pytest.mark.parametrize("splits", [1, 0])
def test_logpos_decode_small(case, splits):
    batch, n_q, lens, Hq, Hkv, dv, R, Wn = case
    say(f"logpos decode {case} splits={splits}")
    b = W.make_decode(53, batch, n_q, Hq, Hkv, dv, R, Wn, seq_lens=lens, logpos=True)
    gpu_vs_oracle(b, what=f"{case} s{splits}", num_splits=splits)


@pytest.mark.parametrize("splits", [3, 17])  # 2 x 8 x splits workgroups: one per CU, or more
def test_logpos_one_is_the_plain_path_bitwise(splits):
    say(f"logit scale 1 == plain kernels, {splits} splits")
    pre = W.make_prefill(55, [300], [500], 8, 2, 128, 256, 0).to(DEV)
    one = torch.ones(pre.rows, dtype=torch.float32, device=DEV)
    o1, l1 = run_prefill(pre, want_lse=True)
    o2, l2 = run_prefill(pre, want_lse=True, logit_scale=one)
    dec = W.make_decode(55, 2, 4, 64, 8, 64, 1024, 0, seq_lens=[900, 3000]).to(DEV)
    one = torch.ones(dec.rows, dtype=torch.float32, device=DEV)
    d1, m1 = run_decode(dec, want_lse=True, num_splits=splits)
    d2, m2 = run_decode(dec, want_lse=True, num_splits=splits, logit_scale=one)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(d1, d2) and torch.equal(m1, m2)


def test_global_chunked_prefill_logpos_sampled():
    name = "global_chunked_prefill_32k_logpos"
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


def test_paged_decode_16_logpos_workload():
    say("paged_decode_16x8k_128k_disjoint_logpos")
    gpu_vs_oracle(W.build("paged_decode_16x8k_128k_disjoint_logpos"), what="decode16 logpos")

"""Randomised GPU parity: seeded draws over the whole argument space of the
prefill and decode calls (head counts and grouping, value head size, rel
extent, window, sequence and context lengths, query tokens per sequence,
split count, score scale, the optional terms, r in place of rel, and
aliased pools), each checked against the float64 oracle at the parity bar.
The draws are fixed by their seeds, so every run checks the same cases;
each is small enough for the oracle to finish in well under a second.
"""
import random
import sys

import pytest
import torch

import workloads as W
from harness import assert_close, errors, oracle_batch, run_decode, run_prefill

pytestmark = pytest.mark.gpu
DEV = "cuda"

HEADS = [(4, 1), (8, 2), (8, 8), (12, 2), (16, 2), (32, 8), (48, 8), (6, 3), (5, 5), (64, 8)]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def prefill_case(seed):
    rnd = random.Random(1000 + seed)
    Hq, Hkv = rnd.choice(HEADS)
    dv = rnd.choice([64, 128])
    R = rnd.choice([1, 3, 16, 64, 100, 128, 257, 512, 1024])
    Wn = rnd.choice([0, 0, 1, 31, 64, 200, 512])
    batch = rnd.randint(1, 3)
    q_lens = [rnd.choice([0, 1, 7, 33, 64, 65, 130, 200]) for _ in range(batch)]
    ctx = [rnd.choice([0, 0, 5, 127, 128, 300, 1000]) for _ in range(batch)]
    if sum(q_lens) == 0:
        q_lens[0] = 17
    opts = dict(gated=rnd.random() < 0.25, logpos=rnd.random() < 0.25)
    if rnd.random() < 0.25:
        opts.update(d_r=rnd.choice([32, 64, 128]), proj_heads=rnd.choice([1, Hq]))
    if rnd.random() < 0.25:   # e4m3 caches
        opts.update(kv_fp8=True)
    if rnd.random() < 0.25:   # a score scale other than 1/sqrt(128)
        opts.update(scale=rnd.choice([0.03, 0.25]))
    return (q_lens, ctx, Hq, Hkv, dv, R, Wn), opts


def decode_case(seed):
    rnd = random.Random(2000 + seed)
    Hq, Hkv = rnd.choice(HEADS)
    G = Hq // Hkv
    dv = rnd.choice([64, 128])
    R = rnd.choice([1, 5, 64, 128, 512, 1024])
    Wn = rnd.choice([0, 0, 0, 64, 300, 512])
    n_q = rnd.choice([n for n in (1, 2, 3, 4, 8, 16) if G * n <= 256])
    batch = rnd.randint(1, 4)
    lens = [max(n_q, rnd.choice([1, 100, 128, 129, 1000, 2500, 6000])) for _ in range(batch)]
    splits = rnd.choice([0, 0, 1, 2, 7, 40])
    opts = dict(kv_fp8=rnd.random() < 0.3, gated=rnd.random() < 0.25, logpos=rnd.random() < 0.25)
    if rnd.random() < 0.25:   # bias rows made from r
        opts.update(d_r=rnd.choice([32, 64, 128]), proj_heads=rnd.choice([1, Hq]))
    if rnd.random() < 0.2:    # sequences drawing their blocks from one small shared pool (aliased blocks)
        opts.update(pool_blocks=max((L + 127) // 128 for L in lens) + rnd.randint(0, 8))
    if rnd.random() < 0.25:   # a score scale other than 1/sqrt(128)
        opts.update(scale=rnd.choice([0.03, 0.25]))
    return (batch, n_q, lens, Hq, Hkv, dv, R, Wn), splits, opts


def check(b_cpu, what, **kw):
    b = b_cpu.to(DEV)
    out, lse = (run_prefill if b.kind == "prefill" else run_decode)(b, want_lse=True, **kw)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_batch(b_cpu)
    assert_close(out, ref, what=what)
    lmx, _ = errors(lse, ref_lse)
    assert lmx <= 1e-3, f"{what}: lse max err {lmx:.3e}"


@pytest.mark.parametrize("seed", range(256))
def test_random_prefill(seed):
    case, opts = prefill_case(seed)
    say(f"random prefill {seed}: {case} {opts}")
    check(W.make_prefill(3000 + seed, *case, **opts), f"prefill seed {seed} {case} {opts}")


@pytest.mark.parametrize("seed", range(256))
def test_random_decode(seed):
    (batch, n_q, lens, Hq, Hkv, dv, R, Wn), splits, opts = decode_case(seed)
    say(f"random decode {seed}: B{batch} n_q{n_q} {lens} H{Hq}/{Hkv} dv{dv} R{R} W{Wn} splits{splits} {opts}")
    b = W.make_decode(4000 + seed, batch, n_q, Hq, Hkv, dv, R, Wn, seq_lens=lens, **opts)
    check(b, f"decode seed {seed}", num_splits=splits)

"""GPU parity of the decode whose bias rows the library makes from the R
branch (rba_decode_relproj) against the float64 oracle, which forms
rel = r @ rel_logits_proj^T in float64 and then attends.

Same bar as the other parity tests (max 1.5e-2, mean 2e-3, lse 1e-3). The
grid covers the three widths of r, a shared and a per-head projection, rel
extents that are not a multiple of the producer's 64-distance tiles (1, 5,
100, 1023), windows, the 16- and 32-column decode kernels, forced and
planned split counts, and the optional terms. A tighter check compares the
call with rba_decode fed the oracle's bias rows rounded to fp32: the two
differ only by the producer's fp32 sums.
"""
import sys

import pytest
import torch

import oracle
import workloads as W
from harness import assert_close, bf16_p_bound, errors, oracle_batch, run_decode
from relative_position_bias_amd import rba

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_vs_oracle(b_cpu, what="", **kw):
    b = b_cpu.to(DEV)
    out, lse = run_decode(b, want_lse=True, **kw)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_batch(b_cpu)
    mx, mean = assert_close(out, ref, what=what)
    lmx, _ = errors(lse, ref_lse)
    assert lmx <= 1e-3, f"{what}: lse max err {lmx:.3e}"
    return out, mx, mean


# (batch, n_q, lens, Hq, Hkv, dv, R, W, d_r, proj_heads, splits)
GRID = [
    (3, 1, [129, 1000, 5000], 32, 8, 128, 1024, 0, 64, 1, 0),
    (2, 4, [700, 4096], 64, 8, 64, 1024, 0, 64, 64, 0),
    (1, 1, [3000], 8, 2, 128, 1, 0, 32, 1, 3),
    (2, 2, [300, 2500], 16, 2, 64, 5, 0, 128, 16, 0),
    (2, 3, [900, 1800], 12, 2, 128, 100, 64, 64, 12, 2),
    (4, 1, [128, 129, 1, 6000], 32, 8, 128, 1023, 300, 128, 1, 0),
    (1, 8, [4000], 48, 8, 64, 1024, 1024, 64, 1, 0),
    (2, 16, [2000, 700], 8, 8, 128, 512, 0, 32, 8, 40),
]


@pytest.mark.parametrize("case", GRID, ids=[f"c{i}" for i in range(len(GRID))])
def test_decode_relproj_grid(case):
    batch, n_q, lens, Hq, Hkv, dv, R, Wn, d_r, ph, splits = case
    say(f"decode relproj {case}")
    b = W.make_decode(70, batch, n_q, Hq, Hkv, dv, R, Wn, seq_lens=lens, d_r=d_r, proj_heads=ph)
    gpu_vs_oracle(b, what=f"decode relproj {case}", num_splits=splits)


@pytest.mark.parametrize("terms", ["fp8", "gated", "logpos", "fp8_gated_logpos"])
@pytest.mark.parametrize("shape", [(3, 1, [2000, 129, 7000], 32, 8, 128), (2, 4, [900, 5000], 64, 8, 64)],
                         ids=["16col", "32col"])
def test_decode_relproj_options(shape, terms):
    batch, n_q, lens, Hq, Hkv, dv = shape
    say(f"decode relproj options {shape} {terms}")
    b = W.make_decode(71, batch, n_q, Hq, Hkv, dv, 1024, 0, seq_lens=lens, d_r=64, proj_heads=1,
                      kv_fp8="fp8" in terms, gated="gated" in terms, logpos="logpos" in terms)
    gpu_vs_oracle(b, what=f"decode relproj {shape} {terms}")


@pytest.mark.parametrize("case", [(3, 1, [2000, 129, 7000], 32, 8, 128, 1024, 0, 64, 1),
                                  (2, 4, [900, 5000], 64, 8, 64, 1023, 300, 128, 64)], ids=["shared", "per_head"])
def test_decode_relproj_equals_decode_on_the_oracle_bias(case):
    """rba_decode_relproj against rba_decode over the oracle's rel rounded to
    fp32. The producer's fp32 sums differ from that by a few ulps of the bias;
    where such a difference moves a probability across a bf16 rounding
    boundary, the output moves by at most that probability's rounding. So
    the outputs must agree element by element within the bf16-P bound (2^-7
    of the softmax-weighted mean |v|, plus fp32 slack), and the lse, which
    sums the fp32 probabilities, to 1e-5."""
    batch, n_q, lens, Hq, Hkv, dv, R, Wn, d_r, ph = case
    say(f"decode relproj vs decode on the oracle bias {case}")
    b = W.make_decode(72, batch, n_q, Hq, Hkv, dv, R, Wn, seq_lens=lens, d_r=d_r, proj_heads=ph)
    rel = torch.from_numpy(oracle.rel_from_proj(b.r.double().numpy(), b.proj.double().numpy())).float()
    bm = W.Batch(**{**b.__dict__, "rel": rel, "r": None, "proj": None})
    o1, l1 = run_decode(b.to(DEV), want_lse=True)
    o2, l2 = run_decode(bm.to(DEV), want_lse=True)
    torch.cuda.synchronize()
    bound = torch.from_numpy(bf16_p_bound(b)).float()
    diff = (o1 - o2).abs().cpu()
    assert bool((diff <= bound).all()), f"max excess {float((diff - bound).max()):.3e}"
    assert float(diff.mean()) <= 5e-6
    assert float((l1 - l2).abs().max()) <= 1e-5


@pytest.mark.parametrize("name", ["verify_decode_b1_100k_relproj", "paged_decode_16x8k_128k_disjoint_relproj"])
def test_decode_relproj_workloads(name):
    say(name)
    _, mx, mean = gpu_vs_oracle(W.build(name), what=name)
    say(f"  max {mx:.3e} mean {mean:.3e}")


GUARD = 4096
CANARY = 1.2345678e30


def test_decode_relproj_writes_only_out_lse_and_workspace():
    """Guard bands around out, lse and the workspace (split partials plus the
    bias rows): nothing outside them changes, for forced and planned splits."""
    batch, n_q, Hq, Hkv, dv, R = 2, 4, 64, 8, 64, 1023
    b = W.make_decode(73, batch, n_q, Hq, Hkv, dv, R, 0, seq_lens=[3000, 800], d_r=64, proj_heads=1).to(DEV)
    rows = batch * n_q
    for splits in (1, 3, 0):
        say(f"decode relproj guard bands, splits={splits}")
        need = rba.relproj_workspace_size(Hq, Hkv, dv, R, 0, b.scale, batch, n_q, b.max_seq_len, splits)
        assert need >= rba.workspace_size(Hq, Hkv, dv, R, 0, b.scale, batch, n_q, b.max_seq_len, splits) + \
            rows * Hq * R * 4
        fw = torch.full((need + 8 * GUARD,), 0xA5, dtype=torch.uint8, device=DEV)
        ws = fw[4 * GUARD:4 * GUARD + need]
        fo = torch.full((rows * Hq * dv + 2 * GUARD,), CANARY, device=DEV)
        out = fo[GUARD:GUARD + rows * Hq * dv].view(rows, Hq, dv)
        fl = torch.full((rows * Hq + 2 * GUARD,), CANARY, device=DEV)
        lse = fl[GUARD:GUARD + rows * Hq].view(rows, Hq)
        run_decode(b, num_splits=splits, workspace=ws, out=out, lse=lse)
        torch.cuda.synchronize()
        assert bool((torch.cat([fw[:4 * GUARD], fw[4 * GUARD + need:]]) == 0xA5).all()), "workspace guard"
        assert bool((torch.cat([fo[:GUARD], fo[GUARD + out.numel():]]) == CANARY).all()), "out guard"
        assert bool((torch.cat([fl[:GUARD], fl[GUARD + lse.numel():]]) == CANARY).all()), "lse guard"
        assert torch.isfinite(out).all()


def test_decode_relproj_graph_capture_replay():
    """The bias-row kernel, the split kernel and the merge captured in one
    graph: every replay, with eager work between them, reproduces the eager
    output."""
    say("decode relproj graph capture")
    b = W.make_decode(74, 2, 4, 64, 8, 64, 1024, 0, seq_lens=[2500, 6000], d_r=64, proj_heads=1).to(DEV)
    need = rba.relproj_workspace_size(64, 8, 64, 1024, 0, b.scale, 2, 4, b.max_seq_len)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    out = torch.empty((8, 64, 64), device=DEV)
    eager = run_decode(b, workspace=ws)[0].clone()
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
        ws.fill_(0xA5)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
        run_decode(W.make_decode(1, 1, 1, 32, 8, 128, 1024, 0, seq_lens=[500], d_r=32).to(DEV))

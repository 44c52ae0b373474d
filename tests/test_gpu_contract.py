"""GPU tests of the C ABI's contract beyond the parity grid: any rel extent
R >= 1, device lengths that break the caller's contract (NaN rows, nothing
read past a block-table row), and guard bands around every buffer the
library writes (nothing is written outside out, lse and the workspace).
"""
import sys

import pytest
import torch

import workloads as W
from harness import errors, oracle_batch, assert_close, run_decode, run_prefill
from relative_position_bias_amd import rba

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check(b_cpu, what, **kw):
    b = b_cpu.to(DEV)
    out, lse = (run_prefill if b.kind == "prefill" else run_decode)(b, want_lse=True, **kw)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_batch(b_cpu)
    mx, mean = assert_close(out, ref, what=what)
    lmx, _ = errors(lse, ref_lse)
    assert lmx <= 1e-3, f"{what}: lse max err {lmx:.3e}"
    return mx, mean


# ---------------------------------------------------------------------------
# rel extents that are not multiples of 4 (rows of rel then start at any
# 4-byte multiple; the decode reads the piece holding distance R - 1 element
# by element)
# ---------------------------------------------------------------------------
ODD_R = [1, 5, 127, 1023]


@pytest.mark.parametrize("R", ODD_R)
@pytest.mark.parametrize("Wn", [0, 200])
def test_prefill_any_rel_extent(R, Wn):
    say(f"prefill R={R} W={Wn}")
    check(W.make_prefill(51, [300, 77], [900, 0], 8, 2, 128, R, Wn), f"prefill R{R} W{Wn}")


@pytest.mark.parametrize("R", ODD_R)
@pytest.mark.parametrize("shape", [(3, 1, 32, 8, 128), (2, 4, 64, 8, 64), (2, 3, 64, 2, 128)],
                         ids=["16col", "32col_dv64", "96col"])
def test_decode_any_rel_extent(R, shape):
    batch, n_q, Hq, Hkv, dv = shape
    lens = [1500, 300, 2700][:batch]
    say(f"decode R={R} shape={shape}")
    check(W.make_decode(52, batch, n_q, Hq, Hkv, dv, R, 0, seq_lens=lens), f"decode R{R} {shape}")
    check(W.make_decode(53, batch, n_q, Hq, Hkv, dv, R, 0, seq_lens=lens, kv_fp8=True),
          f"decode fp8 R{R} {shape}")


@pytest.mark.parametrize("R", ODD_R)
def test_relproj_any_rel_extent(R):
    say(f"relproj R={R}")
    check(W.make_prefill(54, [200, 90], [700, 0], 8, 2, 128, R, 0, d_r=64), f"relproj R{R}")
    check(W.make_prefill(55, [150], [400], 8, 2, 64, R, 160, d_r=64, proj_heads=8), f"relproj W R{R}")


# ---------------------------------------------------------------------------
# device lengths outside the contract: NaN rows, other sequences unchanged
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "e4m3"])
@pytest.mark.parametrize("bad_len", ["past_table", "short_of_rows"])
def test_prefill_bad_device_length_gives_nan_rows(bad_len, fp8):
    say(f"prefill bad length {bad_len} fp8={fp8}")
    b = W.make_prefill(56, [100, 50], [200, 0], 8, 2, 128, 128, 0, kv_fp8=fp8).to(DEV)
    ref, _ = run_prefill(b)
    maxb = b.block_tables.shape[1]
    bad = W.Batch(**{**b.__dict__})
    bad.seq_lens = b.seq_lens.clone()
    bad.seq_lens[0] = maxb * 128 + 10 if bad_len == "past_table" else 40   # the host bounds stay as they were
    out, _ = run_prefill(bad)
    torch.cuda.synchronize()
    assert torch.isnan(out[:100]).all()
    assert torch.equal(out[100:], ref[100:])


@pytest.mark.parametrize("bad_len", ["past_table", "past_split_plan", "short_of_tokens"])
@pytest.mark.parametrize("shape", [(1, 32, 8, 128), (4, 64, 8, 64)], ids=["16col", "32col"])
def test_decode_bad_device_length_gives_nan_rows(bad_len, shape):
    n_q, Hq, Hkv, dv = shape
    say(f"decode bad length {bad_len} {shape}")
    b = W.make_decode(57, 2, n_q, Hq, Hkv, dv, 256, 0, seq_lens=[500, 600]).to(DEV)
    ref, _ = run_decode(b, num_splits=2)
    maxb = b.block_tables.shape[1]
    if bad_len == "past_table":
        L = maxb * 128 + 1
    elif bad_len == "past_split_plan":
        # the table is wide enough, but two splits planned for max_seq_len 600
        # (5 blocks, 3 per split) do not reach block 6
        b.block_tables = torch.cat([b.block_tables, b.block_tables[:, :3]], dim=1).contiguous()
        L = 7 * 128
    else:
        L = n_q - 1
    bad = W.Batch(**{**b.__dict__})
    bad.seq_lens = b.seq_lens.clone()
    bad.seq_lens[0] = L
    out, _ = run_decode(bad, num_splits=2)
    torch.cuda.synchronize()
    assert torch.isnan(out[:n_q]).all()
    assert torch.equal(out[n_q:], ref[n_q:])


# ---------------------------------------------------------------------------
# guard bands: nothing is written outside out, lse and the workspace
# ---------------------------------------------------------------------------
GUARD = 4096  # floats on each side (16 KiB)
CANARY = 1.2345678e30


def guarded(n, dtype=torch.float32):
    """An n-element view with GUARD canary elements on each side (the view
    stays 16-byte aligned)."""
    if dtype == torch.uint8:
        full = torch.full((n + 8 * GUARD,), 0xA5, dtype=torch.uint8, device=DEV)
        return full, full[4 * GUARD:4 * GUARD + n]
    full = torch.full((n + 2 * GUARD,), CANARY, dtype=dtype, device=DEV)
    return full, full[GUARD:GUARD + n]


def untouched(full, n):
    if full.dtype == torch.uint8:
        g = torch.cat([full[:4 * GUARD], full[4 * GUARD + n:]])
        return bool((g == 0xA5).all())
    g = torch.cat([full[:GUARD], full[GUARD + n:]])
    return bool((g == CANARY).all())


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "e4m3"])
@pytest.mark.parametrize("case", [([300, 77], [900, 0], 8, 2, 128, 256, 0), ([130], [100], 48, 8, 64, 128, 96)],
                         ids=["nowin", "win_dv64"])
def test_prefill_writes_only_out_and_lse(case, fp8):
    q_lens, ctx, Hq, Hkv, dv, R, Wn = case
    say(f"guard bands prefill {case} fp8={fp8}")
    b = W.make_prefill(58, q_lens, ctx, Hq, Hkv, dv, R, Wn, kv_fp8=fp8).to(DEV)
    fo, out = guarded(b.rows * Hq * dv)
    fl, lse = guarded(b.rows * Hq)
    run_prefill(b, out=out.view(b.rows, Hq, dv), lse=lse.view(b.rows, Hq))
    torch.cuda.synchronize()
    assert untouched(fo, out.numel()) and untouched(fl, lse.numel())
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("case", [(3, 1, 32, 8, 128, 0, False), (2, 4, 64, 8, 64, 0, True),
                                  (2, 8, 48, 8, 128, 300, False)], ids=["16col", "32col_fp8", "48col_win"])
def test_decode_writes_only_out_lse_and_workspace(case):
    batch, n_q, Hq, Hkv, dv, Wn, fp8 = case
    say(f"guard bands decode {case}")
    lens = [2000, 700, 5000][:batch]
    b = W.make_decode(59, batch, n_q, Hq, Hkv, dv, 1024, Wn, seq_lens=lens, kv_fp8=fp8).to(DEV)
    rows = batch * n_q
    for splits in (1, 3, 0):
        need = rba.workspace_size(Hq, Hkv, dv, 1024, Wn, b.scale, batch, n_q, b.max_seq_len, splits)
        fw, ws = guarded(need, torch.uint8)
        fo, out = guarded(rows * Hq * dv)
        fl, lse = guarded(rows * Hq)
        run_decode(b, num_splits=splits, workspace=ws, out=out.view(rows, Hq, dv), lse=lse.view(rows, Hq))
        torch.cuda.synchronize()
        assert untouched(fw, need), f"workspace guard, splits={splits}"
        assert untouched(fo, out.numel()) and untouched(fl, lse.numel()), f"out/lse guard, splits={splits}"
        assert torch.isfinite(out).all()


# ---------------------------------------------------------------------------
# calls on several streams at once: each with its own outputs and workspace,
# every result equals the same call made alone
# ---------------------------------------------------------------------------
def test_concurrent_calls_on_separate_streams():
    say("concurrent calls on four streams")
    decs = [W.make_decode(80 + i, 3, n_q, 32, 8, 128, 1024, 0, seq_lens=[4000, 900, 7000]).to(DEV)
            for i, n_q in enumerate((1, 4))]
    pres = [W.make_prefill(90 + i, [300, 64], [800, 0], 8, 2, 128, 512, w).to(DEV) for i, w in enumerate((0, 200))]
    alone = [run_decode(b)[0].clone() for b in decs] + [run_prefill(b)[0].clone() for b in pres]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(4)]
    outs = [torch.full_like(a, 7.0) for a in alone]
    wss = [torch.empty(rba.workspace_size(32, 8, 128, 1024, 0, b.scale, 3, b.n_q, b.max_seq_len), dtype=torch.uint8,
                       device=DEV) for b in decs]
    cur = torch.cuda.current_stream()
    for s in streams:
        s.wait_stream(cur)
    for rep in range(5):
        for i, b in enumerate(decs):
            run_decode(b, workspace=wss[i], out=outs[i], stream=streams[i])
        for i, b in enumerate(pres):
            run_prefill(b, out=outs[2 + i], stream=streams[2 + i])
    for s in streams:
        cur.wait_stream(s)
    torch.cuda.synchronize()
    for i, (o, a) in enumerate(zip(outs, alone)):
        assert torch.equal(o, a), f"call {i}"

"""GPU tests of the optional terms in combination (rba_prefill_ex,
rba_prefill_relproj_ex, rba_decode_ex, rba_decode_split_ex): the gated output
(sink, gate; "Inkling 2 Small on vLLM: Day-0 Support", model-architecture
section), the per-row logit scale ("Inkling-Small on Gaudi 2", "What was
built") and the e4m3 K/V cache ("vLLM TML Inkling Support", "Future
Roadmap"). The float64 oracle applies the scale to q and rel, adds the sink
to the normaliser unscaled and the gate to the normalised output, over the
dequantised caches; the bar is the parity bar of the other tests. The
dedicated entry points (rba_prefill_gated, rba_decode_fp8, ...) must give
bitwise the same result as the options call that spells the same terms.
"""
import ctypes
import sys

import pytest
import torch

import workloads as W
from harness import assert_close, errors, oracle_batch, run_decode, run_prefill
from relative_position_bias_amd import rba

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_vs_oracle(b_cpu, what="", **kw):
    b = b_cpu.to(DEV)
    run = run_prefill if b.kind == "prefill" else run_decode
    out, lse = run(b, want_lse=True, **kw)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_batch(b_cpu)
    assert_close(out, ref, what=what)
    lmx, _ = errors(lse, ref_lse)
    assert lmx <= 1e-3, f"{what}: lse max err {lmx:.3e}"
    return out, lse


PREFILL = [
    # q_lens, ctx_lens, Hq, Hkv, dv, R, W
    ([300, 77], [900, 0], 8, 2, 128, 256, 0),
    ([130], [100], 48, 8, 64, 128, 96),          # 48 / 8 heads, window
    ([257], [300], 12, 2, 128, 512, 160),        # G = 6
]


@pytest.mark.parametrize("case", PREFILL, ids=lambda c: f"H{c[2]}/{c[3]}dv{c[4]}W{c[6]}")
def test_prefill_gated_with_logit_scale(case):
    q_lens, ctx, Hq, Hkv, dv, R, Wn = case
    say(f"prefill gated + logpos {case}")
    gpu_vs_oracle(W.make_prefill(61, q_lens, ctx, Hq, Hkv, dv, R, Wn, gated=True, logpos=True), str(case))


@pytest.mark.parametrize("gated", [False, True], ids=["plain", "gated"])
@pytest.mark.parametrize("case", [([200, 90], [700, 0], 8, 2, 128, 300, 0, 1),
                                  ([150], [400], 8, 2, 64, 256, 160, 8)],
                         ids=["nowin_shared", "win_perhead"])
def test_relproj_with_logit_scale(case, gated):
    q_lens, ctx, Hq, Hkv, dv, R, Wn, ph = case
    say(f"relproj + logpos {case} gated={gated}")
    gpu_vs_oracle(W.make_prefill(62, q_lens, ctx, Hq, Hkv, dv, R, Wn, d_r=64, proj_heads=ph, gated=gated,
                                 logpos=True), f"{case} gated={gated}")


DECODE = [
    # batch, n_q, lens, Hq, Hkv, dv, R, W
    (3, 1, [129, 1000, 5000], 32, 8, 128, 1024, 0),   # 16-column kernel
    (2, 4, [700, 4096], 64, 8, 64, 1024, 0),          # 32 columns, dv 64
    (1, 4, [20000], 64, 8, 64, 1024, 0),              # one workgroup per CU: 8-wave e4m3 dv 64 kernel
    (2, 8, [900, 2000], 48, 8, 128, 512, 0),          # 48 columns: two groups
    (4, 3, [3, 250, 520, 1300], 16, 4, 128, 256, 300),  # window
]


@pytest.mark.parametrize("terms", ["fp8_logpos", "fp8_gated_logpos", "gated_logpos", "fp8_gated"])
@pytest.mark.parametrize("case", DECODE, ids=lambda c: f"B{c[0]}nq{c[1]}H{c[3]}/{c[4]}dv{c[5]}W{c[7]}")
def test_decode_option_combinations(case, terms):
    batch, n_q, lens, Hq, Hkv, dv, R, Wn = case
    say(f"decode {terms} {case}")
    b = W.make_decode(63, batch, n_q, Hq, Hkv, dv, R, Wn, seq_lens=lens, kv_fp8="fp8" in terms,
                      gated="gated" in terms, logpos="logpos" in terms)
    gpu_vs_oracle(b, f"{terms} {case}")


def test_split_and_combine_with_options_equal_the_whole_call():
    """rba_decode_split_ex (e4m3 + logit scale) then rba_decode_combine_gated
    is exactly rba_decode_ex with the same terms."""
    say("split_ex + combine_gated")
    b = W.make_decode(64, 2, 4, 64, 8, 64, 1024, 0, seq_lens=[700, 4096], kv_fp8=True, gated=True,
                      logpos=True).to(DEV)
    whole, whole_lse = run_decode(b, num_splits=3, want_lse=True)
    ws = torch.empty(rba.workspace_size(64, 8, 64, 1024, 0, b.scale, 2, 4, b.max_seq_len, 3), dtype=torch.uint8,
                     device=DEV)
    rba.decode_split(b.q, b.k_cache, b.v_cache, b.rel, b.seq_lens, b.block_tables, n_q=4, window=0,
                     scale=b.scale, max_seq_len=b.max_seq_len, num_splits=3, workspace=ws,
                     kv_scales=(b.k_scale, b.v_scale), logit_scale=b.lscale)
    out = torch.empty_like(whole)
    lse = torch.empty_like(whole_lse)
    rba.decode_combine(Hq=64, Hkv=8, dv=64, rel_extent=1024, window=0, scale=b.scale, batch=2, n_q=4,
                       num_splits=3, workspace=ws, out=out, lse=lse, sink=b.sink, gate=b.gate)
    torch.cuda.synchronize()
    assert torch.equal(out, whole) and torch.equal(lse, whole_lse)


# ---------------------------------------------------------------------------
# the dedicated entry points are the options call that spells the same terms
# ---------------------------------------------------------------------------
def _p(t):
    return t.data_ptr() if t is not None else None


def _stream():
    return torch.cuda.current_stream().cuda_stream


def test_dedicated_prefill_entry_points_equal_the_options_call():
    say("dedicated prefill entry points")
    L = rba.lib()
    b = W.make_prefill(65, [200, 77], [300, 0], 8, 2, 128, 256, 0, gated=True, logpos=True).to(DEV)
    p = rba.params(8, 2, 128, 256, 0, b.scale)
    head = (ctypes.byref(p), _p(b.q), _p(b.k_cache), _p(b.v_cache), b.k_cache.shape[0], _p(b.rel), _p(b.cu_q),
            _p(b.seq_lens), _p(b.block_tables), b.block_tables.shape[1], 2, b.max_q_len, b.max_seq_len)

    def run(fn, *extra):
        out = torch.full((b.rows, 8, 128), float("nan"), device=DEV)
        lse = torch.full((b.rows, 8), float("nan"), device=DEV)
        rba._check(fn(*head, *extra, _p(out), _p(lse), _stream()))
        torch.cuda.synchronize()
        return out, lse

    def ex(**terms):
        return run(L.rba_prefill_ex, ctypes.byref(rba.call_options(b.rows, 8, **terms)))

    pairs = [
        (run(L.rba_prefill_gated, _p(b.sink), _p(b.gate)), ex(sink=b.sink, gate=b.gate)),
        (run(L.rba_prefill_logpos, _p(b.lscale)), ex(logit_scale=b.lscale)),
        (run(L.rba_prefill), run(L.rba_prefill_ex, None)),
    ]
    for (o1, l1), (o2, l2) in pairs:
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_dedicated_decode_entry_points_equal_the_options_call():
    say("dedicated decode entry points")
    L = rba.lib()
    bf = W.make_decode(66, 2, 4, 64, 8, 64, 1024, 0, seq_lens=[700, 4096], gated=True, logpos=True).to(DEV)
    b8 = W.make_decode(66, 2, 4, 64, 8, 64, 1024, 0, seq_lens=[700, 4096], kv_fp8=True).to(DEV)
    rows = 8
    splits = 3
    need = rba.workspace_size(64, 8, 64, 1024, 0, bf.scale, 2, 4, bf.max_seq_len, splits)

    def head(b):
        p = rba.params(64, 8, 64, 1024, 0, b.scale)
        return (ctypes.byref(p), _p(b.q), _p(b.k_cache), _p(b.v_cache), b.k_cache.shape[0])

    def mid(b):
        return (_p(b.rel), _p(b.seq_lens), _p(b.block_tables), b.block_tables.shape[1], 2, 4, b.max_seq_len,
                splits)

    def run(fn, pre, post):
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        out = torch.full((rows, 64, 64), float("nan"), device=DEV)
        lse = torch.full((rows, 64), float("nan"), device=DEV)
        rba._check(fn(*pre, _p(ws), need, *post, _p(out), _p(lse), _stream()))
        torch.cuda.synchronize()
        return out, lse

    def opts(b, **terms):
        return (ctypes.byref(rba.call_options(rows, 64, **terms)),)

    ks = (b8.k_scale, b8.v_scale)
    pairs = [
        (run(L.rba_decode_gated, head(bf) + mid(bf), (_p(bf.sink), _p(bf.gate))),
         run(L.rba_decode_ex, head(bf) + mid(bf), opts(bf, sink=bf.sink, gate=bf.gate))),
        (run(L.rba_decode_logpos, head(bf) + mid(bf), (_p(bf.lscale),)),
         run(L.rba_decode_ex, head(bf) + mid(bf), opts(bf, logit_scale=bf.lscale))),
        (run(L.rba_decode_fp8, head(b8) + (ctypes.c_float(ks[0]), ctypes.c_float(ks[1])) + mid(b8), ()),
         run(L.rba_decode_ex, head(b8) + mid(b8), opts(b8, kv_scales=ks))),
        (run(L.rba_decode, head(bf) + mid(bf), ()), run(L.rba_decode_ex, head(bf) + mid(bf), (None,))),
    ]
    for i, ((o1, l1), (o2, l2)) in enumerate(pairs):
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"pair {i}"

    # split stage alone: rba_decode_split_fp8 and rba_decode_split against the _ex form
    def split(fn, pre, post):
        ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
        rba._check(fn(*pre, _p(ws), need, *post, _stream()))
        torch.cuda.synchronize()
        return ws

    a = split(L.rba_decode_split_fp8, head(b8) + (ctypes.c_float(ks[0]), ctypes.c_float(ks[1])) + mid(b8), ())
    c = split(L.rba_decode_split_ex, head(b8) + mid(b8), opts(b8, kv_scales=ks))
    assert torch.equal(a, c)
    a = split(L.rba_decode_split, head(bf) + mid(bf), ())
    c = split(L.rba_decode_split_ex, head(bf) + mid(bf), (None,))
    assert torch.equal(a, c)


# ---------------------------------------------------------------------------
# prefill over e4m3 K/V caches (chunked prefill of a layer whose cache is FP8)
# ---------------------------------------------------------------------------
FP8_PREFILL = [
    # q_lens, ctx_lens, Hq, Hkv, dv, R, W
    ([300, 77], [900, 0], 8, 2, 128, 256, 0),
    ([130], [100], 48, 8, 64, 128, 96),
    ([257], [300], 12, 2, 128, 512, 160),
    ([64, 65, 0], [1000, 3, 9], 4, 1, 128, 64, 0),
    ([200], [4000], 32, 8, 128, 1024, 0),
]


@pytest.mark.parametrize("terms", ["", "gated", "logpos", "gated_logpos"])
@pytest.mark.parametrize("case", FP8_PREFILL, ids=lambda c: f"q{c[0]}H{c[2]}/{c[3]}dv{c[4]}W{c[6]}")
def test_prefill_e4m3(case, terms):
    q_lens, ctx, Hq, Hkv, dv, R, Wn = case
    say(f"prefill e4m3 {case} {terms}")
    b = W.make_prefill(67, q_lens, ctx, Hq, Hkv, dv, R, Wn, kv_fp8=True, gated="gated" in terms,
                       logpos="logpos" in terms)
    gpu_vs_oracle(b, f"e4m3 {case} {terms}")


@pytest.mark.parametrize("Wn", [0, 96])
def test_prefill_e4m3_equals_bf16_on_dequantized_cache(Wn):
    """The e4m3 prefill computes the bf16 prefill over caches that hold the
    dequantised values (exact in bf16 for the workloads' scales). The K scale
    is a power of two, so folding it into the score scale changes no logit
    and lse is bitwise equal; the V scale is applied to the output instead of
    to V, which moves it by fp32 rounding only."""
    say(f"prefill e4m3 vs bf16 on the dequantized cache, W={Wn}")
    b8 = W.make_prefill(68, [300, 77], [900, 0], 8, 2, 128, 256, Wn, kv_fp8=True)
    k = (b8.k_cache.view(torch.float8_e4m3fn).float() * b8.k_scale).to(torch.bfloat16)
    v = (b8.v_cache.view(torch.float8_e4m3fn).float() * b8.v_scale).to(torch.bfloat16)
    bb = W.Batch(**{**b8.__dict__, "k_cache": k, "v_cache": v, "kv_fp8": False, "k_scale": 1.0, "v_scale": 1.0})
    o8, l8 = run_prefill(b8.to(DEV), want_lse=True)
    ob, lb = run_prefill(bb.to(DEV), want_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o8).all()
    assert torch.equal(l8, lb)
    assert float((o8 - ob).abs().max()) <= 1e-5


def test_prefill_e4m3_32k_chunks_sampled():
    """The 32K chunked prefill over an e4m3 cache, ~760 sampled rows of each
    chunk (every 64-row tile, the first and last 256 rows, rows near R)."""
    from harness import tile_sample_rows
    name = "global_chunked_prefill_32k_fp8"
    full = W.build(name)
    g = full.to(DEV)
    for c, (ch_gpu, ch_cpu) in enumerate(zip(W.chunks(name, g), W.chunks(name, full))):
        rows = tile_sample_rows(ch_cpu, seed=c)
        say(f"{name} chunk {c}: {len(rows)} rows")
        out, lse = run_prefill(ch_gpu, want_lse=True)
        torch.cuda.synchronize()
        ref, ref_lse = oracle_batch(ch_cpu, rows=rows)
        assert_close(out, ref, rows, f"{name} chunk {c}")
        lmx, _ = errors(lse, ref_lse, rows)
        assert lmx <= 1e-3, f"chunk {c}: lse max err {lmx:.3e}"


@pytest.mark.parametrize("terms", ["", "gated_logpos"])
@pytest.mark.parametrize("case", [([200, 90], [700, 0], 8, 2, 128, 300, 0, 1, 64),
                                  ([150], [400], 8, 2, 64, 256, 160, 8, 32),
                                  ([130], [1000], 16, 2, 128, 1024, 0, 1, 128)],
                         ids=["nowin_shared", "win_perhead_dr32", "g8_dr128"])
def test_relproj_e4m3(case, terms):
    """The in-kernel-bias prefill over e4m3 caches (each half-block stage
    staged as bytes and widened to bf16)."""
    q_lens, ctx, Hq, Hkv, dv, R, Wn, ph, d_r = case
    say(f"relproj e4m3 {case} {terms}")
    b = W.make_prefill(69, q_lens, ctx, Hq, Hkv, dv, R, Wn, d_r=d_r, proj_heads=ph, kv_fp8=True,
                       gated="gated" in terms, logpos="logpos" in terms)
    gpu_vs_oracle(b, f"relproj e4m3 {case} {terms}")

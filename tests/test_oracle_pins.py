"""Pins of the float64 oracle against things other than itself.

Each check ties the oracle to the pages or to mathematics it cannot share a
mistake with: an independent dense NumPy brute force, PyTorch's own
scaled-dot-product attention for the special cases that reduce to it
(no bias; ALiBi), closed forms, invariants, and the numbers the pages print
(tests/golden). A mutation test at the end shows that plausible slips in the
oracle (a dropped term, a reversed or shifted index, a wrong head map) are
caught by these pins.
"""
import json
import math
import os
import shutil
import subprocess
import tempfile
import ctypes

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------
def make_case(rng, q_lens, seq_lens, Hq, Hkv, dqk, dv, R, scale_qk=1.0):
    tq, tk = int(sum(q_lens)), int(sum(seq_lens))
    return dict(
        q=rng.standard_normal((tq, Hq, dqk)) * scale_qk,
        k=rng.standard_normal((tk, Hkv, dqk)) * scale_qk,
        v=rng.standard_normal((tk, Hkv, dv)),
        rel=0.5 * rng.standard_normal((tq, Hq, R)),
        q_lens=np.asarray(q_lens, dtype=np.int64),
        seq_lens=np.asarray(seq_lens, dtype=np.int64),
    )


def run_oracle(c, R, W, scale, rows=None):
    return oracle.attend(c["q"], c["k"], c["v"], c["rel"], c["q_lens"], c["seq_lens"],
                         rel_extent=R, window=W, scale=scale, rows=rows)


def brute(c, R, W, scale):
    """Dense float64 attention with explicit [Lq, L] mask and bias matrices,
    written independently of the oracle (vectorised NumPy, no online softmax)."""
    q, k, v, rel = c["q"], c["k"], c["v"], c["rel"]
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    outs, lses = [], []
    q0 = k0 = 0
    for Lq, L in zip(c["q_lens"], c["seq_lens"]):
        Lq, L = int(Lq), int(L)
        qi = np.arange(L - Lq, L)[:, None]          # absolute query positions
        kj = np.arange(L)[None, :]
        dist = qi - kj                              # [Lq, L]
        visible = dist >= 0
        if W > 0:
            visible &= dist < W
        in_extent = (dist >= 0) & (dist < R)
        o = np.zeros((Lq, Hq, v.shape[2]))
        ls = np.zeros((Lq, Hq))
        for h in range(Hq):
            g = h // G
            S = scale * (q[q0:q0 + Lq, h] @ k[k0:k0 + L, g].T)
            relh = rel[q0:q0 + Lq, h]                # [Lq, R]
            B = np.where(in_extent, np.take_along_axis(relh, np.clip(dist, 0, R - 1), axis=1), 0.0)
            X = np.where(visible, S + B, -np.inf)
            m = X.max(axis=1, keepdims=True)
            P = np.exp(X - m)
            den = P.sum(axis=1, keepdims=True)
            o[:, h] = (P / den) @ v[k0:k0 + L, g]
            ls[:, h] = (m + np.log(den))[:, 0]
        outs.append(o)
        lses.append(ls)
        q0 += Lq
        k0 += L
    return np.concatenate(outs), np.concatenate(lses)


def sdpa_f64(q, k, v, mask, scale, G):
    """torch scaled_dot_product_attention in float64 on the CPU.
    q [Lq, Hq, d], k/v [L, Hkv, d], mask [Lq, L] (bool = attend, or additive float)."""
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2)[None]
    tm = torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=tm, scale=scale, enable_gqa=(G > 1))
    return o[0].permute(1, 0, 2).numpy()


# ----------------------------------------------------------------------------
# P1: brute force on tiny inputs
# ----------------------------------------------------------------------------
BRUTE_GRID = [
    # q_lens, seq_lens, Hq, Hkv, dqk, dv, R, W
    ([5], [5], 4, 1, 8, 8, 3, 0),
    ([7, 3], [20, 3], 4, 2, 16, 8, 5, 4),
    ([1, 1, 1], [9, 1, 17], 2, 2, 8, 16, 7, 0),
    ([12], [40], 6, 2, 16, 4, 64, 6),
    ([0, 9], [4, 30], 4, 4, 8, 8, 1, 1),
    ([16], [16], 4, 1, 16, 16, 16, 16),
    ([4, 6], [48, 80], 4, 1, 16, 8, 9, 20),
    ([31], [47], 3, 1, 8, 8, 2, 33),
]


@pytest.mark.parametrize("case", BRUTE_GRID)
def test_p1_brute_force(case):
    q_lens, seq_lens, Hq, Hkv, dqk, dv, R, W = case
    rng = np.random.default_rng(1234 + len(q_lens) + R + W)
    c = make_case(rng, q_lens, seq_lens, Hq, Hkv, dqk, dv, R)
    scale = 1.0 / math.sqrt(dqk)
    o, l = run_oracle(c, R, W, scale)
    ob, lb = brute(c, R, W, scale)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, lb, rtol=0, atol=1e-12)


def test_p1_row_subset_matches_full():
    rng = np.random.default_rng(7)
    c = make_case(rng, [6, 10], [30, 12], 4, 2, 8, 8, 8, 5)
    full, lfull = run_oracle(c, 8, 5, 0.3)
    rows = [0, 3, 15, 7]
    sub, lsub = run_oracle(c, 8, 5, 0.3, rows=rows)
    np.testing.assert_array_equal(sub[rows], full[rows])
    np.testing.assert_array_equal(lsub[rows], lfull[rows])
    others = [r for r in range(16) if r not in rows]
    assert np.isnan(sub[others]).all()


# ----------------------------------------------------------------------------
# P2: rel = 0 and no window is ordinary causal softmax attention
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("Lq,L,Hq,Hkv", [(24, 24, 4, 1), (10, 37, 4, 2), (1, 50, 8, 2), (16, 40, 2, 2)])
def test_p2_rel_zero_is_causal_sdpa(Lq, L, Hq, Hkv):
    rng = np.random.default_rng(Lq * 100 + L)
    R = 5
    c = make_case(rng, [Lq], [L], Hq, Hkv, 16, 8, R)
    c["rel"][:] = 0.0
    scale = 0.25
    o, _ = run_oracle(c, R, 0, scale)
    mask = np.arange(L)[None, :] <= np.arange(L - Lq, L)[:, None]
    ref = sdpa_f64(c["q"], c["k"], c["v"], mask, scale, Hq // Hkv)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# P3: local-window prefill over only the last blocks equals the full context
# ----------------------------------------------------------------------------
def truncated_to_window(c, W, bs):
    """Keep only the blocks a window-W query chunk can see (one sequence);
    positions shift by a whole number of blocks."""
    Lq, L = int(c["q_lens"][0]), int(c["seq_lens"][0])
    first = L - Lq
    kb_lo = max(0, first - W + 1) // bs
    drop = kb_lo * bs
    t = dict(c)
    t["k"] = c["k"][drop:]
    t["v"] = c["v"][drop:]
    t["seq_lens"] = np.asarray([L - drop], dtype=np.int64)
    return t, kb_lo


def test_p3_local_window_equivalence_40_cases():
    g = json.load(open(os.path.join(GOLDEN, "local_window_blocks.json")))
    rng = np.random.default_rng(40)
    for case in range(g["random_cases"]):
        bs = int(rng.choice([4, 8, 16]))
        W = int(rng.integers(1, 6 * bs))
        L = int(rng.integers(1, 12 * bs))
        Lq = int(rng.integers(1, L + 1))
        R = int(rng.integers(1, W + 3))
        c = make_case(rng, [Lq], [L], 4, 2, 8, 8, R)
        scale = float(rng.uniform(0.1, 0.5))
        full, lf = run_oracle(c, R, W, scale)
        t, _ = truncated_to_window(c, W, bs)
        trunc, lt = run_oracle(t, R, W, scale)
        np.testing.assert_array_equal(trunc, full, err_msg=f"case {case}")
        np.testing.assert_array_equal(lt, lf, err_msg=f"case {case}")


def test_p3_pages_five_blocks_for_window_512():
    g = json.load(open(os.path.join(GOLDEN, "local_window_blocks.json")))
    W, bs = g["window"], g["block_size"]
    # a decode query at any position needs blocks floor((i-W+1)/bs) .. floor(i/bs)
    need = max((i // bs) - (max(0, i - W + 1) // bs) + 1 for i in range(W, W + 4 * bs))
    assert need == g["context_blocks_needed"]
    assert need == -(-(W - 1) // bs) + 1
    # and with that many blocks the output is unchanged (small head size)
    rng = np.random.default_rng(5)
    L, Lq = 3 * W + 77, 3
    c = make_case(rng, [Lq], [L], 2, 1, 8, 4, W)
    full, _ = run_oracle(c, W, W, 0.3)
    t, kb_lo = truncated_to_window(c, W, bs)
    assert (L + bs - 1) // bs - kb_lo <= need + 1   # the chunk's last query may start a block
    trunc, _ = run_oracle(t, W, W, 0.3)
    np.testing.assert_array_equal(trunc, full)


# ----------------------------------------------------------------------------
# P4: rel = -m_h * d is ALiBi
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("Lq,L", [(20, 20), (6, 33)])
def test_p4_alibi_special_case(Lq, L):
    rng = np.random.default_rng(Lq + 7 * L)
    Hq, Hkv, R = 4, 2, L + 5          # R beyond every distance
    c = make_case(rng, [Lq], [L], Hq, Hkv, 16, 8, R)
    slopes = 2.0 ** (-np.arange(1, Hq + 1))
    c["rel"] = np.broadcast_to(-slopes[None, :, None] * np.arange(R)[None, None, :], (Lq, Hq, R)).copy()
    scale = 0.25
    o, _ = run_oracle(c, R, 0, scale)
    qi = np.arange(L - Lq, L)[:, None]
    kj = np.arange(L)[None, :]
    for h in range(Hq):
        mask = np.where(kj <= qi, -slopes[h] * (qi - kj).astype(np.float64), -np.inf)
        g = h // (Hq // Hkv)
        ref = sdpa_f64(c["q"][:, h:h + 1], c["k"][:, g:g + 1], c["v"][:, g:g + 1], mask, scale, 1)
        np.testing.assert_allclose(o[:, h:h + 1], ref, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# P5: a one-hot bias selects exactly the key at distance d0
# ----------------------------------------------------------------------------
def test_p5_shear_index_probe():
    rng = np.random.default_rng(55)
    q_lens, seq_lens = [9, 4], [25, 60]
    Hq, Hkv, R, W = 4, 2, 30, 24
    c = make_case(rng, q_lens, seq_lens, Hq, Hkv, 8, 8, R)
    c["q"][:] = 0
    c["k"][:] = 0
    c["rel"][:] = 0
    expect = np.zeros((sum(q_lens), Hq, 8))
    t = 0
    k0 = 0
    for Lq, L in zip(q_lens, seq_lens):
        for r in range(Lq):
            i = L - Lq + r
            for h in range(Hq):
                d0 = int(rng.integers(0, min(i + 1, W, R)))
                c["rel"][t, h, d0] = 40.0
                expect[t, h] = c["v"][k0 + i - d0, h // 2]
            t += 1
        k0 += L
    o, _ = run_oracle(c, R, W, 0.3)
    np.testing.assert_allclose(o, expect, rtol=0, atol=1e-9)


# ----------------------------------------------------------------------------
# P6: window of exactly W keys including the query's own key
# ----------------------------------------------------------------------------
def test_p6_window_closed_form_and_boundary_probe():
    rng = np.random.default_rng(66)
    L, Lq, W, R = 70, 50, 16, 32
    c = make_case(rng, [Lq], [L], 2, 1, 8, 8, R)
    c["q"][:] = 0
    c["k"][:] = 0
    c["rel"][:] = 0
    o, _ = run_oracle(c, R, W, 0.5)
    for r in range(Lq):
        i = L - Lq + r
        lo = max(0, i - W + 1)
        np.testing.assert_allclose(o[r, 0], c["v"][lo:i + 1, 0].mean(axis=0), rtol=0, atol=1e-12)
    # d0 = W-1 is visible, d0 = W is not
    for d0, visible in ((W - 1, True), (W, False)):
        c2 = dict(c)
        c2["rel"] = np.zeros_like(c["rel"])
        c2["rel"][:, :, d0] = 40.0
        o2, _ = run_oracle(c2, R, W, 0.5)
        r = Lq - 1
        i = L - 1
        if visible:
            np.testing.assert_allclose(o2[r, 0], c["v"][i - d0, 0], rtol=0, atol=1e-9)
        else:
            np.testing.assert_allclose(o2[r, 0], c["v"][i - W + 1:i + 1, 0].mean(axis=0), rtol=0, atol=1e-12)


def test_golden_decode_window_counts():
    """The pages' decode-window numbers follow from the reading 'visible iff
    0 <= i-j < W': a 4-block decode context shows 385..512 keys, 5 blocks
    show exactly 512."""
    g = json.load(open(os.path.join(GOLDEN, "decode_window.json")))
    W, bs = g["window"], g["block_size"]

    def count_visible(i, n_blocks):
        # one decode query at position i whose context is the last n_blocks blocks
        first_block = max(0, i // bs - (n_blocks - 1))
        drop = first_block * bs
        L = i + 1 - drop
        kv = np.zeros((L, 1, 2))
        kv[:, 0, 1] = np.arange(L)                  # value = position
        c = dict(q=np.zeros((1, 1, 2)), k=np.zeros((L, 1, 2)), v=kv,
                 rel=np.zeros((1, 1, W)), q_lens=np.array([1]), seq_lens=np.array([L]))
        o, _ = run_oracle(c, W, W, 1.0)
        mean_pos = o[0, 0, 1]
        return int(round(2 * ((L - 1) - mean_pos) + 1))   # contiguous range ending at i

    positions = range(4 * bs, 4 * bs + bs)                # every residue i mod 128
    before = [count_visible(i, g["decode_blocks_before_fix"]) for i in positions]
    after = [count_visible(i, g["decode_blocks_after_fix"]) for i in positions]
    assert min(before) == g["visible_keys_before_fix"]["min"]
    assert max(before) == g["visible_keys_before_fix"]["max"]
    assert set(after) == {g["visible_keys_after_fix"]}


def test_golden_kv_page_bytes():
    g = json.load(open(os.path.join(GOLDEN, "kv_page_bytes.json")))
    per_rank_heads = g["num_kv_heads"] // g["tensor_parallel"]
    page = g["block_size"] * per_rank_heads * g["head_dim"] * g["bytes_per_element"] * g["tensors"]
    assert page == g["page_bytes_per_block_per_layer"]


# ----------------------------------------------------------------------------
# P7: beyond the relative extent the bias is 0 (closed form)
# ----------------------------------------------------------------------------
def test_p7_beyond_extent_closed_form():
    rng = np.random.default_rng(77)
    L, Lq, R, cst = 60, 20, 12, 1.7
    c = make_case(rng, [Lq], [L], 2, 1, 8, 8, R)
    c["q"][:] = 0
    c["k"][:] = 0
    c["rel"][:] = cst
    o, _ = run_oracle(c, R, 0, 0.5)
    v = c["v"][:, 0]
    for r in range(Lq):
        i = L - Lq + r
        n = i + 1
        near = v[i - min(R, n) + 1:i + 1].sum(axis=0)      # distances < R
        far = v[:max(0, n - R)].sum(axis=0)                 # distances >= R
        den = min(R, n) * math.exp(cst) + max(0, n - R)
        np.testing.assert_allclose(o[r, 0], (math.exp(cst) * near + far) / den, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# P8: adding a per-row constant to rel leaves the output unchanged
# ----------------------------------------------------------------------------
def test_p8_row_shift_invariance():
    rng = np.random.default_rng(88)
    c = make_case(rng, [10, 5], [30, 41], 4, 2, 8, 8, 64)
    o, l = run_oracle(c, 64, 0, 0.3)
    shift = rng.uniform(-3, 3, size=c["rel"].shape[:2])
    c2 = dict(c)
    c2["rel"] = c["rel"] + shift[:, :, None]
    o2, l2 = run_oracle(c2, 64, 0, 0.3)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l + shift, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# P9: chunked prefill and decode rows equal the one-shot prefill rows
# ----------------------------------------------------------------------------
def test_p9_chunking_and_decode_rows():
    rng = np.random.default_rng(99)
    L, R, W = 48, 10, 0
    full = make_case(rng, [L], [L], 4, 2, 8, 8, R)
    o_full, l_full = run_oracle(full, R, W, 0.3)
    for cuts in ([0, 12, 30, 48], [0, 47, 48], [0, 16, 32, 48]):
        for a, b in zip(cuts[:-1], cuts[1:]):
            ch = dict(q=full["q"][a:b], k=full["k"][:b], v=full["v"][:b], rel=full["rel"][a:b],
                      q_lens=np.array([b - a]), seq_lens=np.array([b]))
            o, l = run_oracle(ch, R, W, 0.3)
            np.testing.assert_array_equal(o, o_full[a:b])
            np.testing.assert_array_equal(l, l_full[a:b])


# ----------------------------------------------------------------------------
# P10: GQA head map h -> h // G
# ----------------------------------------------------------------------------
def test_p10_gqa_replication():
    rng = np.random.default_rng(1010)
    Hq, Hkv = 6, 2
    c = make_case(rng, [7], [19], Hq, Hkv, 8, 8, 6)
    o, _ = run_oracle(c, 6, 5, 0.3)
    rep = dict(c)
    rep["k"] = np.repeat(c["k"], Hq // Hkv, axis=1)
    rep["v"] = np.repeat(c["v"], Hq // Hkv, axis=1)
    o2, _ = run_oracle(rep, 6, 5, 0.3)
    np.testing.assert_array_equal(o2, o)


# ----------------------------------------------------------------------------
# P11: a narrower value head is a column slice
# ----------------------------------------------------------------------------
def test_p11_diff_headdim_is_column_slice():
    rng = np.random.default_rng(1111)
    c = make_case(rng, [9], [21], 4, 1, 16, 8, 7)
    o, l = run_oracle(c, 7, 0, 0.25)
    wide = dict(c)
    wide["v"] = np.concatenate([c["v"], rng.standard_normal(c["v"].shape)], axis=2)
    ow, lw = run_oracle(wide, 7, 0, 0.25)
    np.testing.assert_array_equal(ow[:, :, :8], o)
    np.testing.assert_array_equal(lw, l)


def test_degenerate_single_key_and_extent_one():
    rng = np.random.default_rng(3)
    c = make_case(rng, [4], [9], 2, 1, 8, 8, 1)
    o, l = run_oracle(c, 1, 1, 0.3)         # W = 1: only the query's own key
    np.testing.assert_allclose(o[:, 0], c["v"][5:9, 0], rtol=0, atol=0)
    qk = 0.3 * np.einsum("td,td->t", c["q"][:, 0], c["k"][5:9, 0])
    np.testing.assert_allclose(l[:, 0], qk + c["rel"][:, 0, 0], rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# Mutation check: planted slips in the oracle (on the CPU) must fail a pin
# ----------------------------------------------------------------------------
MUTANTS = {
    "dropped_bias": ("x[j - lo] = scale * s + bias;", "x[j - lo] = scale * s;"),
    "reversed_distance": ("relr[dist] : 0.0", "relr[R - 1 - dist] : 0.0"),
    "clamped_beyond_extent": ("relr[dist] : 0.0", "relr[dist] : relr[R - 1]"),
    "window_off_by_one": ("i - W + 1 > 0 ? i - W + 1 : 0", "i - W > 0 ? i - W : 0"),
    "head_map_modulo": ("const int64_t g = h / G;", "const int64_t g = h % Hkv;"),
    "dropped_scale": ("x[j - lo] = scale * s + bias;", "x[j - lo] = s + bias;"),
    "key_offset": ("(kv_start[b] + j) * Hkv + g) * dqk", "(kv_start[b] + j + (j > 0 ? -1 : 0)) * Hkv + g) * dqk"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_are_caught(name, monkeypatch):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, name
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "m.c")
        open(path, "w").write(src.replace(old, new))
        so = os.path.join(d, "libm.so")
        subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", path, "-o", so, "-lm"], check=True)
        lib = ctypes.CDLL(so)
        i64, dbl, P = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.rba_oracle_attend.argtypes = [i64, P, P, i64, i64, i64, i64, i64, i64, dbl,
                                          P, P, P, P, P, P, P, i64, P, P]
        lib.rba_oracle_attend.restype = ctypes.c_int
        monkeypatch.setattr(oracle, "_lib", lib)
        caught = False
        for case in BRUTE_GRID:
            q_lens, seq_lens, Hq, Hkv, dqk, dv, R, W = case
            rng = np.random.default_rng(1234 + len(q_lens) + R + W)
            c = make_case(rng, q_lens, seq_lens, Hq, Hkv, dqk, dv, R)
            scale = 1.0 / math.sqrt(dqk)
            o, l = run_oracle(c, R, W, scale)
            ob, lb = brute(c, R, W, scale)
            if not (np.allclose(o, ob, rtol=0, atol=1e-12) and np.allclose(l, lb, rtol=0, atol=1e-12)):
                caught = True
                break
        assert caught, f"mutant {name} passed the brute-force pin"


# ---------------------------------------------------------------------------
# e4m3 decoding of the FP8-KV decode's caches
# ---------------------------------------------------------------------------
def test_e4m3_decode_hand_values():
    """Values fixed by the OCP FP8 e4m3 definition (bias 7, 3 mantissa bits,
    subnormals below 2^-6, S.1111.111 = NaN, no infinities)."""
    table = {0x00: 0.0, 0x38: 1.0, 0x40: 2.0, 0x3C: 1.5, 0x7E: 448.0, 0xFE: -448.0, 0x08: 2.0 ** -6,
             0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x30: 0.5, 0xB8: -1.0, 0x77: 240.0}
    codes = np.array(list(table), dtype=np.uint8)
    got = oracle.e4m3_to_float(codes)
    assert np.array_equal(got, np.array(list(table.values())))
    assert np.signbit(oracle.e4m3_to_float(np.array([0x80], dtype=np.uint8)))[0]  # -0
    assert np.isnan(oracle.e4m3_to_float(np.array([0x7F, 0xFF], dtype=np.uint8))).all()


def test_e4m3_decode_matches_torch_for_every_code():
    """All 256 codes against an independent decoder (torch.float8_e4m3fn)."""
    codes = np.arange(256, dtype=np.uint8)
    a = oracle.e4m3_to_float(codes)
    b = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(a), np.isnan(b))
    ok = ~np.isnan(a)
    assert np.array_equal(a[ok], b[ok]) and np.array_equal(np.signbit(a[ok]), np.signbit(b[ok]))


def test_fp8_decode_oracle_is_bf16_oracle_on_dequantized_cache():
    """The oracle of an e4m3 batch equals the oracle of the same batch with the
    caches replaced by their dequantized values (exact in bf16 for these
    scales), i.e. the FP8 path changes only where K/V come from."""
    import workloads as W
    from harness import oracle_batch
    b8 = W.make_decode(7, 2, 2, 8, 2, 64, 128, 0, seq_lens=[130, 300], kv_fp8=True)
    k = torch.from_numpy(oracle.e4m3_to_float(b8.k_cache.numpy()) * b8.k_scale)
    v = torch.from_numpy(oracle.e4m3_to_float(b8.v_cache.numpy()) * b8.v_scale)
    assert torch.equal(k.to(torch.bfloat16).double().nan_to_num(7.0), k.nan_to_num(7.0))  # exact in bf16
    bb = W.Batch(**{**b8.__dict__, "k_cache": k.to(torch.bfloat16), "v_cache": v.to(torch.bfloat16),
                    "kv_fp8": False, "k_scale": 1.0, "v_scale": 1.0})
    o8, l8 = oracle_batch(b8)
    ob, lb = oracle_batch(bb)
    assert np.array_equal(o8, ob) and np.array_equal(l8, lb)


# ---------------------------------------------------------------------------
# gated-attention output: per-(token, head) sink logit and sigmoid gate
# ---------------------------------------------------------------------------
def _gated_case(seed=5):
    rng = np.random.default_rng(seed)
    c = make_case(rng, [7, 12], [20, 12], 4, 2, 16, 8, 6)
    tq = int(sum(c["q_lens"]))
    sink = rng.standard_normal((tq, 4)) * 2.0
    gate = rng.standard_normal((tq, 4)) * 2.0
    return c, sink, gate


def test_gated_sink_minus_inf_and_gate_plus_inf_are_the_plain_attention():
    c, _, _ = _gated_case()
    o, l = run_oracle(c, 6, 0, 0.25)
    tq = o.shape[0]
    og, lg = oracle.attend(c["q"], c["k"], c["v"], c["rel"], c["q_lens"], c["seq_lens"], rel_extent=6, window=0,
                           scale=0.25, sink=np.full((tq, 4), -np.inf), gate=np.full((tq, 4), np.inf))
    assert np.array_equal(o, og) and np.array_equal(l, lg)


def test_gated_gate_zero_halves_the_output():
    c, sink, _ = _gated_case()
    o, l = oracle.attend(c["q"], c["k"], c["v"], c["rel"], c["q_lens"], c["seq_lens"], rel_extent=6, window=0,
                         scale=0.25, sink=sink)
    og, lg = oracle.attend(c["q"], c["k"], c["v"], c["rel"], c["q_lens"], c["seq_lens"], rel_extent=6, window=0,
                           scale=0.25, sink=sink, gate=np.zeros_like(sink))
    assert np.array_equal(og, 0.5 * o) and np.array_equal(lg, l)


def test_gated_sink_closed_form_uniform_scores():
    """q = k = 0, rel = 0: every visible logit is 0, so with n visible keys
    out = sum_j v_j / (n + e^s) and lse = log(n + e^s); the gate multiplies by
    1 / (1 + e^-a)."""
    c, sink, gate = _gated_case(9)
    c = dict(c, q=np.zeros_like(c["q"]), k=np.zeros_like(c["k"]), rel=np.zeros_like(c["rel"]))
    W = 5
    o, l = oracle.attend(c["q"], c["k"], c["v"], c["rel"], c["q_lens"], c["seq_lens"], rel_extent=6, window=W,
                         scale=0.25, sink=sink, gate=gate)
    t = 0
    k0 = 0
    for Lq, L in zip(c["q_lens"], c["seq_lens"]):
        for r in range(int(Lq)):
            i = int(L) - int(Lq) + r
            lo = max(0, i - W + 1)
            for h in range(4):
                g = h // 2
                n = i - lo + 1
                vs = c["v"][k0 + lo:k0 + i + 1, g].sum(axis=0)
                den = n + math.exp(sink[t, h])
                want = vs / den / (1.0 + math.exp(-gate[t, h]))
                assert np.allclose(o[t, h], want, rtol=1e-13, atol=1e-13)
                assert abs(l[t, h] - math.log(den)) <= 1e-13
            t += 1
        k0 += int(L)


def test_gated_large_sink_takes_all_the_weight():
    c, sink, _ = _gated_case()
    big = np.full_like(sink, 800.0)
    o, l = oracle.attend(c["q"], c["k"], c["v"], c["rel"], c["q_lens"], c["seq_lens"], rel_extent=6, window=0,
                         scale=0.25, sink=big)
    assert np.abs(o).max() < 1e-300 and np.allclose(l, 800.0, rtol=0, atol=1e-12)


GATED_MUTANTS = {
    "sink_dropped_from_sum": ("double l = sink ? exp(sk - m) : 0.0;", "double l = 0.0;"),
    "gate_sign": ("exp(-gate[t * Hq + h])", "exp(gate[t * Hq + h])"),
    "sink_value_not_zero": ("const double p = x[j - lo] / l;", "const double p = x[j - lo] / (l - (sink ? exp(sk - m) : 0.0));"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(GATED_MUTANTS))
def test_gated_mutants_are_caught(name, monkeypatch):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    old, new = GATED_MUTANTS[name]
    assert src.count(old) == 1, name
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "m.c")
        open(path, "w").write(src.replace(old, new))
        so = os.path.join(d, "libm.so")
        subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", path, "-o", so, "-lm"], check=True)
        lib = ctypes.CDLL(so)
        i64, dbl, P = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.rba_oracle_attend.argtypes = [i64, P, P, i64, i64, i64, i64, i64, i64, dbl,
                                          P, P, P, P, P, P, P, i64, P, P]
        lib.rba_oracle_attend.restype = ctypes.c_int
        monkeypatch.setattr(oracle, "_lib", lib)
        with pytest.raises(AssertionError):
            test_gated_sink_closed_form_uniform_scores()


# ----------------------------------------------------------------------------
# The bias producer rel = r @ rel_logits_proj ("Inkling-Small on Gaudi 2",
# section "Attention with a relative bias"). Reading: r is [rows, Hq, d_r],
# the projection [Hp, R, d_r] in linear-weight layout, shared (Hp = 1) or one
# per query head (Hp = Hq).
# ----------------------------------------------------------------------------

def _one_hot_case(rows, Hq, d_r, R, Hp):
    """r rows are scaled one-hot vectors; the weights are 100 hp + 10 d + c.
    Then rel[t, h, d] = a(t, h) * (100 hp(h) + 10 d + c(t, h)) exactly."""
    r = np.zeros((rows, Hq, d_r))
    a = np.zeros((rows, Hq))
    sel = np.zeros((rows, Hq), dtype=np.int64)
    for t in range(rows):
        for h in range(Hq):
            sel[t, h] = (t + 2 * h + 1) % d_r
            a[t, h] = t + 1 + 0.5 * h
            r[t, h, sel[t, h]] = a[t, h]
    hp = np.arange(Hp).reshape(Hp, 1, 1)
    d = np.arange(R).reshape(1, R, 1)
    c = np.arange(d_r).reshape(1, 1, d_r)
    proj = (100.0 * hp + 10.0 * d + c) * np.ones((Hp, R, d_r))
    return r, proj, a, sel


@pytest.mark.parametrize("d_r,R", [(8, 6), (8, 8), (5, 11)])
@pytest.mark.parametrize("shared", [False, True])
def test_relproj_one_hot_selects_the_weight(d_r, R, shared):
    rows, Hq = 5, 3
    Hp = 1 if shared else Hq
    r, proj, a, sel = _one_hot_case(rows, Hq, d_r, R, Hp)
    rel = oracle.rel_from_proj(r, proj)
    assert rel.shape == (rows, Hq, R)
    for t in range(rows):
        for h in range(Hq):
            hp = 0 if shared else h
            want = a[t, h] * (100.0 * hp + 10.0 * np.arange(R) + sel[t, h])
            np.testing.assert_array_equal(rel[t, h], want)


def test_relproj_constant_r_gives_row_sums():
    # r = c * ones: rel[t, h, d] = c(t, h) * sum_k proj[hp, d, k]; with
    # proj[hp, d, k] = k + d*d_r + hp the row sum is d_r*(d_r-1)/2 + d_r*(d*d_r + hp).
    rows, Hq, d_r, R = 4, 2, 6, 7
    cst = np.array([[1.0, -2.0], [0.5, 3.0], [0.0, 1.0], [-1.5, 0.25]])
    r = cst[:, :, None] * np.ones((rows, Hq, d_r))
    k = np.arange(d_r).reshape(1, 1, d_r)
    d = np.arange(R).reshape(1, R, 1)
    hp = np.arange(Hq).reshape(Hq, 1, 1)
    proj = (k + d * d_r + hp) * np.ones((Hq, R, d_r))
    rel = oracle.rel_from_proj(r, proj)
    for h in range(Hq):
        rowsum = d_r * (d_r - 1) / 2 + d_r * (np.arange(R) * d_r + h)
        np.testing.assert_array_equal(rel[:, h, :], cst[:, h:h + 1] * rowsum)


def test_relproj_rejects_bad_head_count():
    with pytest.raises(ValueError):
        oracle.rel_from_proj(np.zeros((2, 4, 8)), np.zeros((2, 5, 8)))


def _relproj_mutant(kind):
    def f(r, proj):
        r, proj = np.asarray(r, dtype=np.float64), np.asarray(proj, dtype=np.float64)
        rows, Hq, d_r = r.shape
        Hp = proj.shape[0]
        rel = np.empty((rows, Hq, proj.shape[1]))
        for h in range(Hq):
            hp = h if Hp == Hq else 0
            if kind == "head_zero":
                hp = 0
            elif kind == "head_reversed" and Hp == Hq:
                hp = Hq - 1 - h
            w = proj[hp] if kind == "no_transpose" else proj[hp].T
            rel[:, h, :] = r[:, h, :] @ w
        return rel
    return f


@pytest.mark.parametrize("kind", ["no_transpose", "head_zero", "head_reversed"])
def test_relproj_mutants_are_caught(kind, monkeypatch):
    monkeypatch.setattr(oracle, "rel_from_proj", _relproj_mutant(kind))
    with pytest.raises(AssertionError):
        for d_r, R in [(8, 8)]:
            test_relproj_one_hot_selects_the_weight(d_r, R, shared=False)


# ----------------------------------------------------------------------------
# Log-position scale ("Inkling-Small on Gaudi 2", "What was built": a scale on
# q and on the rel logits; no formula on the pages). Reading: the caller gives
# one factor f_t per query row, which multiplies row t's q and rel.
# ----------------------------------------------------------------------------

def _logpos_ramp_case(f):
    """q = 0 and rel = -a d: row t's weights over its keys are exp(-f_t a d)."""
    L, Hq, R, dv, a = 9, 2, 16, 3, 0.7
    rng = np.random.default_rng(5)
    q = np.zeros((L, Hq, 4))
    k = rng.standard_normal((L, 1, 4))
    v = rng.standard_normal((L, 1, dv))
    d = np.arange(R)
    rel = np.broadcast_to(-a * d, (L, Hq, R)).copy()
    out, _ = oracle.attend(q, k, v, rel, [L], [L], rel_extent=R, window=0, scale=0.3, logit_scale=f)
    for t in range(L):
        w = np.exp(-f[t] * a * (t - np.arange(t + 1)))
        want = (w[:, None] * v[:t + 1, 0, :]).sum(0) / w.sum()
        for h in range(Hq):
            np.testing.assert_allclose(out[t, h], want, rtol=1e-12, atol=1e-12)


def _logpos_q_case(f):
    """rel = 0, q_t = e_0 and k_j = kappa_j e_0: weights exp(f_t scale kappa_j)."""
    L, scale, dv = 7, 0.5, 2
    q = np.zeros((L, 1, 4))
    q[:, 0, 0] = 1.0
    kappa = np.linspace(-2.0, 3.0, L)
    k = np.zeros((L, 1, 4))
    k[:, 0, 0] = kappa
    v = np.arange(L * dv, dtype=np.float64).reshape(L, 1, dv)
    rel = np.zeros((L, 1, 8))
    out, lse = oracle.attend(q, k, v, rel, [L], [L], rel_extent=8, window=0, scale=scale, logit_scale=f)
    for t in range(L):
        z = f[t] * scale * kappa[:t + 1]
        w = np.exp(z - z.max())
        np.testing.assert_allclose(out[t, 0], (w[:, None] * v[:t + 1, 0, :]).sum(0) / w.sum(), rtol=1e-12)
        np.testing.assert_allclose(lse[t, 0], z.max() + np.log(w.sum()), rtol=1e-12)


LOGPOS_F = np.array([1.0, 1.3, 0.6, 2.0, 1.05, 0.9, 1.7, 1.2, 3.0])


def test_logpos_scales_the_bias():
    _logpos_ramp_case(LOGPOS_F)


def test_logpos_scales_q_dot_k():
    _logpos_q_case(LOGPOS_F[:7])


def test_logpos_one_is_the_plain_oracle():
    b = dict(q_lens=[40], seq_lens=[90])
    rng = np.random.default_rng(9)
    q, k, v = rng.standard_normal((40, 4, 8)), rng.standard_normal((90, 2, 8)), rng.standard_normal((90, 2, 5))
    rel = rng.standard_normal((40, 4, 32))
    o1, l1 = oracle.attend(q, k, v, rel, b["q_lens"], b["seq_lens"], rel_extent=32, window=20, scale=0.4)
    o2, l2 = oracle.attend(q, k, v, rel, b["q_lens"], b["seq_lens"], rel_extent=32, window=20, scale=0.4,
                           logit_scale=np.ones(40))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("kind", ["q_only", "rel_only", "squared"])
def test_logpos_mutants_are_caught(kind, monkeypatch):
    real = oracle.attend

    def mutant(q, k, v, rel, q_lens, seq_lens, *, logit_scale=None, **kw):
        if logit_scale is None:
            return real(q, k, v, rel, q_lens, seq_lens, **kw)
        f = np.asarray(logit_scale, dtype=np.float64).reshape(-1)
        q, rel = np.asarray(q, dtype=np.float64), np.asarray(rel, dtype=np.float64)
        if kind in ("q_only", "squared"):
            q = q * (f * f if kind == "squared" else f)[:, None, None]
        if kind in ("rel_only", "squared"):
            rel = rel * (f * f if kind == "squared" else f)[:, None, None]
        return real(q, k, v, rel, q_lens, seq_lens, **kw)

    monkeypatch.setattr(oracle, "attend", mutant)
    with pytest.raises(AssertionError):
        test_logpos_scales_the_bias()
        test_logpos_scales_q_dot_k()


# ---------------------------------------------------------------------------
# un-paging: the gather that turns a block-table cache into contiguous keys
# ---------------------------------------------------------------------------
def _paged_case(seed=17, Hk=3, d=5, bs=8):
    """Two sequences (one ending inside its last block) in a pool of blocks
    placed by a seeded permutation, plus a spare block that no table uses."""
    rng = np.random.default_rng(seed)
    seq_lens = [19, 8]
    nbs = [(L + bs - 1) // bs for L in seq_lens]
    perm = rng.permutation(sum(nbs) + 1)
    tables, o = [], 0
    for nb in nbs:
        tables.append([int(x) for x in perm[o:o + nb]] + [-1])   # a trailing unused entry
        o += nb
    cache = rng.standard_normal((sum(nbs) + 1, Hk, bs, d))
    return cache, tables, seq_lens, bs


def _per_token_gather(cache, tables, seq_lens, bs):
    """Position j of sequence b is slot j % bs of the block in table entry
    j // bs ("Inkling-Small on Gaudi 2", "Attention with a relative bias":
    key positions are block ordinal x block size + slot), one token at a time."""
    rows = []
    for b, L in enumerate(seq_lens):
        for j in range(L):
            rows.append(cache[tables[b][j // bs], :, j % bs, :])
    return np.stack(rows)


def test_unpage_matches_per_token_gather():
    cache, tables, seq_lens, bs = _paged_case()
    got = oracle.unpage(cache, tables, seq_lens, block_size=bs)
    want = _per_token_gather(cache, tables, seq_lens, bs)
    assert got.shape == (sum(seq_lens), cache.shape[1], cache.shape[3])
    np.testing.assert_array_equal(got, want)


def _unpage_mutant(kind):
    def f(cache, block_tables, seq_lens, block_size=128):
        cache = np.asarray(cache)
        parts = []
        for b, L in enumerate(seq_lens):
            nb = (int(L) + block_size - 1) // block_size
            idx = np.asarray(block_tables[b][:nb], dtype=np.int64)
            if kind == "reversed_table":
                idx = idx[::-1]
            blocks = cache[idx]
            if kind == "no_transpose":   # [nb, H, bs, d] reshaped as if it were [nb, bs, H, d]
                seq = blocks.reshape(nb * block_size, cache.shape[1], cache.shape[3])
            else:
                seq = blocks.transpose(0, 2, 1, 3).reshape(nb * block_size, cache.shape[1], cache.shape[3])
            if kind == "first_slots_dropped":
                seq = seq[1:]
                parts.append(seq[:int(L) - 1])
                continue
            parts.append(seq[:int(L)])
        return np.concatenate(parts, axis=0)
    return f


@pytest.mark.parametrize("kind", ["no_transpose", "reversed_table", "first_slots_dropped"])
def test_unpage_mutants_are_caught(kind):
    cache, tables, seq_lens, bs = _paged_case()
    want = _per_token_gather(cache, tables, seq_lens, bs)
    got = _unpage_mutant(kind)(cache, tables, seq_lens, block_size=bs)
    assert got.shape != want.shape or not np.array_equal(got, want), kind


# ---------------------------------------------------------------------------
# the dense row form of the oracle (used for many sampled rows of long inputs)
# ---------------------------------------------------------------------------
DENSE_GRID = [
    # seq_len, positions, Hq, Hkv, dqk, dv, R, W
    (40, [0, 1, 5, 39, 20, 33], 4, 1, 16, 8, 9, 0),
    (70, [69, 3, 64, 12], 6, 2, 8, 16, 64, 20),
    (33, list(range(33)), 4, 4, 8, 8, 1, 1),
    (90, [10, 89, 45, 50, 51, 88], 8, 2, 16, 16, 7, 33),
]


@pytest.mark.parametrize("case", DENSE_GRID)
@pytest.mark.parametrize("extras", ["plain", "gated", "logpos"])
def test_dense_rows_match_the_loop_oracle(case, extras):
    """attend_rows_dense equals attend (the loop form, pinned by everything
    above) on the same rows, to float64 rounding."""
    L, pos, Hq, Hkv, dqk, dv, R, W = case
    rng = np.random.default_rng(L + R + W)
    k = rng.standard_normal((L, Hkv, dqk))
    v = rng.standard_normal((L, Hkv, dv))
    qa = rng.standard_normal((L, Hq, dqk))
    rela = 0.5 * rng.standard_normal((L, Hq, R))
    kw = {}
    if extras == "gated":
        kw = dict(sink=2 * rng.standard_normal((L, Hq)), gate=2 * rng.standard_normal((L, Hq)))
    if extras == "logpos":
        kw = dict(logit_scale=1.0 + 0.25 * rng.random(L))
    scale = 1.0 / math.sqrt(dqk)
    full, lfull = oracle.attend(qa, k, v, rela, [L], [L], rel_extent=R, window=W, scale=scale, **kw)
    p = np.asarray(pos)
    sub = {n: (a[p] if a is not None else None) for n, a in kw.items()}
    o, l = oracle.attend_rows_dense(qa[p], k, v, rela[p], p, rel_extent=R, window=W, scale=scale,
                                    group=4, **sub)
    np.testing.assert_allclose(o, full[p], rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, lfull[p], rtol=0, atol=1e-12)

"""Seeded synthetic inputs for relative-bias attention (no attention arithmetic).

Shared by the tests, the smoke check and the benchmark; neither the library
nor the oracle imports anything else from the other side. Every tensor is
drawn on the CPU from one torch.Generator seeded per workload, so the values
are identical on every machine:

  draw order: random sequence lengths (if any), q, k-pool, v-pool, rel, then
  the block-table permutations.
  bf16 tensors: fp32 standard normal rounded to bf16 (round to nearest even);
  rel: 0.5 * standard normal in fp32.
  Pool blocks that no table references, and slots past a sequence's length in
  its last block, are filled with bf16 NaN so that stray reads show up.
  Gated-attention inputs (Inkling 2 Small), drawn after everything else:
  sink = 2 * standard normal and gate = 2 * standard normal, fp32 [rows, Hq].
  e4m3 (OCP FP8) K/V caches, for the FP8-KV decode: the bf16 draws above
  divided by the per-tensor scale (K_SCALE_FP8, V_SCALE_FP8) and rounded to
  e4m3 by torch (round to nearest even; |x / scale| stays far below 448), kept
  as raw bytes; NaN slots stay NaN.

The workloads stand in for the pages' traffic (8K-token prompts, 32K-256K
agentic sessions, a 100K-context decode at batch 1, 16 sequences in a
2,560-block pool); only their lengths, head counts and extents matter to the
attention cost, so nothing of any dataset is used.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import torch

BLOCK = 128
HEAD_DIM = 128
_CHUNK = 1 << 24
BF16_NAN = 0x7FC0
K_SCALE_FP8 = 0.0625     # per-tensor dequantization scales of the e4m3 workloads
V_SCALE_FP8 = 0.09375

# Named workloads (sizes as the pages and the task describe them).
WORKLOADS = {
    "tiny_prefill_256": dict(kind="prefill", q_lens=[256], ctx_lens=[0], Hq=4, Hkv=1, dv=128, R=128,
                             W=64, permute=False),
    "local_prefill_8k": dict(kind="prefill", q_lens=[8192], ctx_lens=[0], Hq=32, Hkv=8, dv=128, R=512,
                             W=512, permute=True),
    "global_chunked_prefill_32k": dict(kind="chunked", total=32768, chunk=8192, Hq=32, Hkv=8, dv=128,
                                       R=1024, W=0),
    "paged_decode_16x8k_128k": dict(kind="decode", batch=16, len_range=(8192, 131072), n_q=1, Hq=32,
                                    Hkv=8, dv=128, R=1024, W=0, pool_blocks=2560),
    "paged_decode_16x8k_128k_disjoint": dict(kind="decode", batch=16, len_range=(8192, 131072), n_q=1,
                                             Hq=32, Hkv=8, dv=128, R=1024, W=0, pool_blocks=None),
    "verify_decode_b1_100k": dict(kind="decode", batch=1, seq_len=100000, n_q=4, Hq=64, Hkv=8, dv=64,
                                  R=1024, W=0, pool_blocks=None),
    "verify_decode_b8_100k": dict(kind="decode", batch=8, seq_len=100000, n_q=4, Hq=64, Hkv=8, dv=64,
                                  R=1024, W=0, pool_blocks=None),
}
# Inkling 2 Small shapes (48 query / 8 KV heads on every layer, window 1024
# on local layers, 7 draft tokens + 1 verified = 8 verify tokens) with the
# gated-attention output (sink and gate inputs).
WORKLOADS["inkling2_local_prefill_8k_gated"] = dict(kind="prefill", q_lens=[8192], ctx_lens=[0], Hq=48, Hkv=8,
                                                    dv=128, R=1024, W=1024, permute=True, gated=True)
WORKLOADS["inkling2_verify_b1_100k_gated"] = dict(kind="decode", batch=1, seq_len=100000, n_q=8, Hq=48, Hkv=8,
                                                  dv=128, R=1024, W=0, pool_blocks=None, gated=True)
# The prefills with the bias given by its producer, r (width 64 per token and
# head; the pages do not give the width) and one shared projection.
WORKLOADS["local_prefill_8k_relproj"] = dict(WORKLOADS["local_prefill_8k"], d_r=64)
WORKLOADS["global_chunked_prefill_32k_relproj"] = dict(WORKLOADS["global_chunked_prefill_32k"], d_r=64)
# Global-layer calls with a per-row log-position logit scale.
WORKLOADS["global_chunked_prefill_32k_logpos"] = dict(WORKLOADS["global_chunked_prefill_32k"], logpos=True)
WORKLOADS["global_chunked_prefill_32k_fp8"] = dict(WORKLOADS["global_chunked_prefill_32k"], kv_fp8=True)
WORKLOADS["paged_decode_16x8k_128k_disjoint_logpos"] = dict(WORKLOADS["paged_decode_16x8k_128k_disjoint"],
                                                          logpos=True)
# Decode workloads whose bias rows are made from r (width 64) and one shared
# projection instead of being given.
for _name in ("paged_decode_16x8k_128k_disjoint", "verify_decode_b1_100k"):
    WORKLOADS[_name + "_relproj"] = dict(WORKLOADS[_name], d_r=64)
# The decode workloads again over e4m3 K/V caches.
for _name in ("paged_decode_16x8k_128k_disjoint", "verify_decode_b1_100k", "verify_decode_b8_100k"):
    WORKLOADS[_name + "_fp8"] = dict(WORKLOADS[_name], kv_fp8=True)


@dataclass
class Batch:
    """One call's inputs (CPU tensors unless moved with .to())."""
    kind: str                       # "prefill" or "decode"
    Hq: int
    Hkv: int
    dv: int
    R: int
    W: int
    scale: float
    q: torch.Tensor                 # bf16 [rows, Hq, 128]
    k_cache: torch.Tensor           # bf16 [num_blocks, Hkv, 128, 128]
    v_cache: torch.Tensor           # bf16 [num_blocks, Hkv, 128, dv]
    rel: Optional[torch.Tensor]     # fp32 [rows, Hq, R] (None when r / proj give it)
    seq_lens: torch.Tensor          # int32 [B]
    block_tables: torch.Tensor      # int32 [B, max_blocks]
    cu_q: Optional[torch.Tensor] = None   # int32 [B+1] (prefill)
    n_q: int = 0                          # decode tokens per sequence
    q_lens: List[int] = field(default_factory=list)
    max_q_len: int = 0
    max_seq_len: int = 0
    sink: Optional[torch.Tensor] = None   # fp32 [rows, Hq] gated-attention sink logits
    gate: Optional[torch.Tensor] = None   # fp32 [rows, Hq] gated-attention gate logits
    kv_fp8: bool = False                  # k_cache / v_cache hold e4m3 bytes (uint8)
    k_scale: float = 1.0                  # dequantization scales of e4m3 caches
    v_scale: float = 1.0
    r: Optional[torch.Tensor] = None      # bf16 [rows, Hq, d_r] R-branch vectors (rel not given)
    proj: Optional[torch.Tensor] = None   # bf16 [1 or Hq, R, d_r] rel_logits_proj, linear-weight layout
    lscale: Optional[torch.Tensor] = None  # fp32 [rows] per-row logit scale (log-position scale)

    def to(self, device) -> "Batch":
        kw = {}
        for name, val in self.__dict__.items():
            kw[name] = val.to(device) if isinstance(val, torch.Tensor) else val
        return Batch(**kw)

    @property
    def rows(self) -> int:
        return self.q.shape[0]


def _randn_into(out: torch.Tensor, gen: torch.Generator, std: float = 1.0) -> torch.Tensor:
    flat = out.view(-1)
    for s in range(0, flat.numel(), _CHUNK):
        e = min(flat.numel(), s + _CHUNK)
        x = torch.randn(e - s, generator=gen, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        flat[s:e] = x.to(out.dtype)
    return out


def _bf16(shape, gen):
    return _randn_into(torch.empty(shape, dtype=torch.bfloat16), gen)


def _poison(k_cache, v_cache, tables: List[List[int]], seq_lens: List[int]) -> None:
    """NaN in every slot no sequence uses (unreferenced blocks, tails)."""
    nb = k_cache.shape[0]
    valid = torch.zeros(nb, dtype=torch.int64)
    for tab, L in zip(tables, seq_lens):
        nblk = (L + BLOCK - 1) // BLOCK
        for n in range(nblk):
            blk = tab[n]
            if blk < 0:
                continue
            valid[blk] = max(int(valid[blk]), min(BLOCK, L - BLOCK * n))
    kv = k_cache.view(torch.int16)
    vv = v_cache.view(torch.int16)
    for blk in torch.nonzero(valid < BLOCK).flatten().tolist():
        s = int(valid[blk])
        kv[blk, :, s:, :] = BF16_NAN
        vv[blk, :, s:, :] = BF16_NAN


def _gated(rows: int, Hq: int, gen: torch.Generator) -> dict:
    sink = _randn_into(torch.empty((rows, Hq), dtype=torch.float32), gen, 2.0)
    gate = _randn_into(torch.empty((rows, Hq), dtype=torch.float32), gen, 2.0)
    return dict(sink=sink, gate=gate)


def _logpos(rows: int, gen: torch.Generator) -> torch.Tensor:
    """Synthetic per-row logit scales, uniform in [1, 1.25] (drawn last). The
    pages give no formula for the log-position scale; a factor a little above
    1 is what such a scale does to rows past its threshold."""
    return 1.0 + 0.25 * torch.rand(rows, generator=gen, dtype=torch.float32)


def _to_e4m3(x: torch.Tensor, scale: float) -> torch.Tensor:
    """x / scale rounded to e4m3 by torch, as raw bytes (chunked)."""
    out = torch.empty(x.shape, dtype=torch.uint8)
    src, dst = x.view(-1), out.view(-1)
    for s in range(0, src.numel(), _CHUNK):
        e = min(src.numel(), s + _CHUNK)
        dst[s:e] = (src[s:e].float() / scale).to(torch.float8_e4m3fn).view(torch.uint8)
    return out


def _tables_tensor(tables: List[List[int]], max_blocks: int) -> torch.Tensor:
    t = torch.full((len(tables), max_blocks), -1, dtype=torch.int32)
    for b, tab in enumerate(tables):
        t[b, :len(tab)] = torch.tensor(tab, dtype=torch.int32)
    return t


def make_prefill(seed: int, q_lens: List[int], ctx_lens: List[int], Hq: int, Hkv: int, dv: int, R: int,
                 W: int, permute: bool = True, scale: Optional[float] = None,
                 extra_blocks: int = 0, gated: bool = False, d_r: int = 0, proj_heads: int = 1,
                 logpos: bool = False, kv_fp8: bool = False) -> Batch:
    """Sequences with ctx_lens[b] cached tokens followed by q_lens[b] new ones
    (whose K/V are already in the cache). One pool holds every sequence's
    blocks, disjoint, permuted if `permute`. With d_r > 0 the bias is given
    by its producer instead: r ~ N(0, 1) [rows, Hq, d_r] and a projection
    ~ N(0, 0.25 / d_r) [proj_heads, R, d_r], so that rel = r @ proj^T has the
    N(0, 0.5^2) entries of the materialised workloads; rel is then None.
    With kv_fp8 the caches are converted to e4m3 bytes after every draw
    (as in make_decode)."""
    gen = torch.Generator().manual_seed(seed)
    seq_lens = [c + q for c, q in zip(ctx_lens, q_lens)]
    nblk = [(L + BLOCK - 1) // BLOCK for L in seq_lens]
    num_blocks = sum(nblk) + extra_blocks
    total_q = sum(q_lens)
    q = _bf16((total_q, Hq, HEAD_DIM), gen)
    k_cache = _bf16((num_blocks, Hkv, BLOCK, HEAD_DIM), gen)
    v_cache = _bf16((num_blocks, Hkv, BLOCK, dv), gen)
    rel, relproj = None, {}
    if d_r > 0:
        relproj["r"] = _bf16((total_q, Hq, d_r), gen)
        relproj["proj"] = _randn_into(torch.empty((proj_heads, R, d_r), dtype=torch.bfloat16), gen,
                                      0.5 / d_r ** 0.5)
    else:
        rel = _randn_into(torch.empty((total_q, Hq, R), dtype=torch.float32), gen, 0.5)
    order = torch.randperm(num_blocks, generator=gen).tolist() if permute else list(range(num_blocks))
    tables, o = [], 0
    for n in nblk:
        tables.append(order[o:o + n])
        o += n
    _poison(k_cache, v_cache, tables, seq_lens)
    max_blocks = max(nblk)
    extra = _gated(total_q, Hq, gen) if gated else {}
    if logpos:
        extra["lscale"] = _logpos(total_q, gen)
    if kv_fp8:
        k_cache = _to_e4m3(k_cache, K_SCALE_FP8)
        v_cache = _to_e4m3(v_cache, V_SCALE_FP8)
        extra.update(kv_fp8=True, k_scale=K_SCALE_FP8, v_scale=V_SCALE_FP8)
    cu = [0]
    for ql in q_lens:
        cu.append(cu[-1] + ql)
    return Batch(kind="prefill", Hq=Hq, Hkv=Hkv, dv=dv, R=R, W=W,
                 scale=scale if scale is not None else HEAD_DIM ** -0.5,
                 q=q, k_cache=k_cache, v_cache=v_cache, rel=rel,
                 seq_lens=torch.tensor(seq_lens, dtype=torch.int32),
                 block_tables=_tables_tensor(tables, max_blocks),
                 cu_q=torch.tensor(cu, dtype=torch.int32), q_lens=list(q_lens),
                 max_q_len=max(q_lens), max_seq_len=max(seq_lens), **extra, **relproj)


def make_decode(seed: int, batch: int, n_q: int, Hq: int, Hkv: int, dv: int, R: int, W: int,
                seq_lens: Optional[List[int]] = None, len_range=None, seq_len: Optional[int] = None,
                pool_blocks: Optional[int] = None, scale: Optional[float] = None, kv_fp8: bool = False,
                gated: bool = False, logpos: bool = False, d_r: int = 0, proj_heads: int = 1) -> Batch:
    """`batch` sequences decoding n_q tokens each. Lengths: explicit, one fixed
    `seq_len`, or uniform integers in `len_range` (inclusive). With
    pool_blocks=None every sequence gets its own blocks (one global
    permutation of a pool of exactly the needed size); otherwise each sequence
    takes the first blocks of its own permutation of a `pool_blocks` pool, so
    blocks may be shared between sequences (read-only aliasing). With d_r > 0
    the bias comes from r and a projection drawn as in make_prefill (rel is
    then None)."""
    gen = torch.Generator().manual_seed(seed)
    if seq_lens is None:
        if seq_len is not None:
            seq_lens = [seq_len] * batch
        else:
            lo, hi = len_range
            seq_lens = torch.randint(lo, hi + 1, (batch,), generator=gen).tolist()
    assert len(seq_lens) == batch and all(L >= n_q for L in seq_lens)
    nblk = [(L + BLOCK - 1) // BLOCK for L in seq_lens]
    num_blocks = sum(nblk) if pool_blocks is None else pool_blocks
    assert max(nblk) <= num_blocks
    q = _bf16((batch * n_q, Hq, HEAD_DIM), gen)
    k_cache = _bf16((num_blocks, Hkv, BLOCK, HEAD_DIM), gen)
    v_cache = _bf16((num_blocks, Hkv, BLOCK, dv), gen)
    rel, relproj = None, {}
    if d_r > 0:
        relproj["r"] = _bf16((batch * n_q, Hq, d_r), gen)
        relproj["proj"] = _randn_into(torch.empty((proj_heads, R, d_r), dtype=torch.bfloat16), gen,
                                      0.5 / d_r ** 0.5)
    else:
        rel = _randn_into(torch.empty((batch * n_q, Hq, R), dtype=torch.float32), gen, 0.5)
    tables = []
    if pool_blocks is None:
        order = torch.randperm(num_blocks, generator=gen).tolist()
        o = 0
        for n in nblk:
            tables.append(order[o:o + n])
            o += n
    else:
        for n in nblk:
            tables.append(torch.randperm(num_blocks, generator=gen)[:n].tolist())
    _poison(k_cache, v_cache, tables, seq_lens)
    kw = _gated(batch * n_q, Hq, gen) if gated else {}
    if logpos:
        kw["lscale"] = _logpos(batch * n_q, gen)
    if kv_fp8:
        k_cache = _to_e4m3(k_cache, K_SCALE_FP8)
        v_cache = _to_e4m3(v_cache, V_SCALE_FP8)
        kw.update(kv_fp8=True, k_scale=K_SCALE_FP8, v_scale=V_SCALE_FP8)
    return Batch(kind="decode", Hq=Hq, Hkv=Hkv, dv=dv, R=R, W=W,
                 scale=scale if scale is not None else HEAD_DIM ** -0.5,
                 q=q, k_cache=k_cache, v_cache=v_cache, rel=rel,
                 seq_lens=torch.tensor(seq_lens, dtype=torch.int32),
                 block_tables=_tables_tensor(tables, max(nblk)), n_q=n_q,
                 q_lens=[n_q] * batch, max_q_len=n_q, max_seq_len=max(seq_lens), **kw, **relproj)


def chunk_of(full: Batch, c: int, chunk: int) -> Batch:
    """Chunk c of a one-sequence prefill: query rows [c*chunk, (c+1)*chunk),
    attending to the first (c+1)*chunk cached tokens."""
    a, b = c * chunk, (c + 1) * chunk
    nb = (b + BLOCK - 1) // BLOCK
    dev = full.q.device
    return Batch(kind="prefill", Hq=full.Hq, Hkv=full.Hkv, dv=full.dv, R=full.R, W=full.W,
                 scale=full.scale, q=full.q[a:b], k_cache=full.k_cache, v_cache=full.v_cache,
                 rel=full.rel[a:b] if full.rel is not None else None, seq_lens=torch.tensor([b], dtype=torch.int32, device=dev),
                 block_tables=full.block_tables[:, :nb].contiguous(),
                 cu_q=torch.tensor([0, b - a], dtype=torch.int32, device=dev), q_lens=[b - a],
                 max_q_len=b - a, max_seq_len=b,
                 sink=full.sink[a:b] if full.sink is not None else None,
                 gate=full.gate[a:b] if full.gate is not None else None,
                 r=full.r[a:b] if full.r is not None else None, proj=full.proj,
                 lscale=full.lscale[a:b] if full.lscale is not None else None,
                 kv_fp8=full.kv_fp8, k_scale=full.k_scale, v_scale=full.v_scale)


def build(name: str, seed: int = 0) -> Batch:
    """Inputs of a named workload. For the chunked prefill this is the whole
    sequence; split it with chunks() (after moving it to the GPU once)."""
    w = dict(WORKLOADS[name])
    kind = w.pop("kind")
    if kind == "prefill":
        return make_prefill(seed, **w)
    if kind == "chunked":
        total = w.pop("total")
        w.pop("chunk")
        return make_prefill(seed, [total], [0], w["Hq"], w["Hkv"], w["dv"], w["R"], w["W"],
                            d_r=w.get("d_r", 0), proj_heads=w.get("proj_heads", 1), logpos=w.get("logpos", False),
                            kv_fp8=w.get("kv_fp8", False))
    return make_decode(seed, **w)


def chunks(name: str, full: Batch) -> List[Batch]:
    """The chunk calls of a chunked-prefill workload over its full sequence."""
    w = WORKLOADS[name]
    return [chunk_of(full, c, w["chunk"]) for c in range(w["total"] // w["chunk"])]

"""ctypes binding over librba.so: argument marshalling only.

Every step of the attention runs in the library's gfx950 kernels; this module
checks torch dtypes/devices/shapes, passes raw pointers and the current HIP
stream, and raises if the library reports an error. It never computes
attention itself and has no fallback: if librba.so is missing it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librba.so")

RBA_OK = 0
RBA_ERR_NULL = -1
RBA_ERR_SHAPE = -2
RBA_ERR_UNSUPPORTED = -3
RBA_ERR_WORKSPACE = -4
RBA_ERR_HIP = -5
BLOCK_SIZE = 128

_i32 = ctypes.c_int32
_ptr = ctypes.c_void_p
_size = ctypes.c_size_t


class AttnParams(ctypes.Structure):
    """Mirror of rba_attn_params in include/rba.h."""
    _fields_ = [
        ("num_heads_q", _i32),
        ("num_heads_kv", _i32),
        ("head_dim_qk", _i32),
        ("head_dim_v", _i32),
        ("rel_extent", _i32),
        ("window", _i32),
        ("scale", ctypes.c_float),
        ("block_size", _i32),
    ]


class CallOptions(ctypes.Structure):
    """Mirror of rba_call_options in include/rba.h."""
    _fields_ = [
        ("sink", _ptr),
        ("gate", _ptr),
        ("logit_scale", _ptr),
        ("kv_e4m3", _i32),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
    ]


class RbaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"librba error {code}: {msg}")
        self.code = code


# (name, restype, argtypes) of every symbol include/rba.h declares
_SIGNATURES = {
    "rba_version": (ctypes.c_char_p, []),
    "rba_last_error": (ctypes.c_char_p, []),
    "rba_prefill": (ctypes.c_int, [ctypes.POINTER(AttnParams), _ptr, _ptr, _ptr, _i32, _ptr, _ptr, _ptr,
                                   _ptr, _i32, _i32, _i32, _i32, _ptr, _ptr, _ptr]),
    "rba_validate_prefill": (ctypes.c_int, [ctypes.POINTER(AttnParams), _ptr, _ptr, _ptr, _i32, _ptr, _ptr,
                                            _ptr, _ptr, _i32, _i32, _i32, _i32, _ptr]),
    "rba_decode": (ctypes.c_int, [ctypes.POINTER(AttnParams), _ptr, _ptr, _ptr, _i32, _ptr, _ptr, _ptr, _i32,
                                  _i32, _i32, _i32, _i32, _ptr, _size, _ptr, _ptr, _ptr]),
    "rba_validate_decode": (ctypes.c_int, [ctypes.POINTER(AttnParams), _ptr, _ptr, _ptr, _i32, _ptr, _ptr,
                                           _ptr, _i32, _i32, _i32, _i32, _i32, _ptr, _size, _ptr]),
    "rba_decode_plan_splits": (_i32, [ctypes.POINTER(AttnParams), _i32, _i32, _i32, _i32]),
    "rba_decode_workspace_size": (_size, [ctypes.POINTER(AttnParams), _i32, _i32, _i32, _i32]),
    "rba_decode_split": (ctypes.c_int, [ctypes.POINTER(AttnParams), _ptr, _ptr, _ptr, _i32, _ptr, _ptr, _ptr,
                                        _i32, _i32, _i32, _i32, _i32, _ptr, _size, _ptr]),
    "rba_decode_combine": (ctypes.c_int, [ctypes.POINTER(AttnParams), _i32, _i32, _i32, _ptr, _size, _ptr,
                                          _ptr, _ptr]),
    "rba_prefill_gated": (ctypes.c_int, [ctypes.POINTER(AttnParams), _ptr, _ptr, _ptr, _i32, _ptr, _ptr, _ptr,
                                         _ptr, _i32, _i32, _i32, _i32, _ptr, _ptr, _ptr, _ptr, _ptr]),
    "rba_decode_gated": (ctypes.c_int, [ctypes.POINTER(AttnParams), _ptr, _ptr, _ptr, _i32, _ptr, _ptr, _ptr,
                                        _i32, _i32, _i32, _i32, _i32, _ptr, _size, _ptr, _ptr, _ptr, _ptr, _ptr]),
    "rba_decode_combine_gated": (ctypes.c_int, [ctypes.POINTER(AttnParams), _i32, _i32, _i32, _ptr, _size,
                                                _ptr, _ptr, _ptr, _ptr, _ptr]),
    "rba_decode_fp8": (ctypes.c_int, [ctypes.POINTER(AttnParams), _ptr, _ptr, _ptr, _i32, ctypes.c_float,
                                      ctypes.c_float, _ptr, _ptr, _ptr, _i32, _i32, _i32, _i32, _i32, _ptr,
                                      _size, _ptr, _ptr, _ptr]),
    "rba_prefill_logpos": (ctypes.c_int, [ctypes.POINTER(AttnParams), _ptr, _ptr, _ptr, _i32, _ptr, _ptr, _ptr,
                                          _ptr, _i32, _i32, _i32, _i32, _ptr, _ptr, _ptr, _ptr]),
    "rba_decode_logpos": (ctypes.c_int, [ctypes.POINTER(AttnParams), _ptr, _ptr, _ptr, _i32, _ptr, _ptr, _ptr,
                                         _i32, _i32, _i32, _i32, _i32, _ptr, _size, _ptr, _ptr, _ptr, _ptr]),
    "rba_prefill_relproj": (ctypes.c_int, [ctypes.POINTER(AttnParams), _ptr, _ptr, _ptr, _i32, _ptr, _ptr, _i32,
                                           _i32, _ptr, _ptr, _ptr, _i32, _i32, _i32, _i32, _ptr, _ptr, _ptr,
                                           _ptr, _ptr]),
    "rba_decode_split_fp8": (ctypes.c_int, [ctypes.POINTER(AttnParams), _ptr, _ptr, _ptr, _i32, ctypes.c_float,
                                            ctypes.c_float, _ptr, _ptr, _ptr, _i32, _i32, _i32, _i32, _i32,
                                            _ptr, _size, _ptr]),
    "rba_decode_noalloc": (ctypes.c_int, [ctypes.POINTER(AttnParams), _ptr, _ptr, _ptr, _i32, _ptr, _ptr, _ptr,
                                          _i32, _i32, _i32, _i32, _i32, _ptr, _ptr, _ptr]),
    "rba_prefill_ex": (ctypes.c_int, [ctypes.POINTER(AttnParams), _ptr, _ptr, _ptr, _i32, _ptr, _ptr, _ptr,
                                      _ptr, _i32, _i32, _i32, _i32, ctypes.POINTER(CallOptions), _ptr, _ptr,
                                      _ptr]),
    "rba_prefill_relproj_ex": (ctypes.c_int, [ctypes.POINTER(AttnParams), _ptr, _ptr, _ptr, _i32, _ptr, _ptr,
                                              _i32, _i32, _ptr, _ptr, _ptr, _i32, _i32, _i32, _i32,
                                              ctypes.POINTER(CallOptions), _ptr, _ptr, _ptr]),
    "rba_decode_ex": (ctypes.c_int, [ctypes.POINTER(AttnParams), _ptr, _ptr, _ptr, _i32, _ptr, _ptr, _ptr, _i32,
                                     _i32, _i32, _i32, _i32, _ptr, _size, ctypes.POINTER(CallOptions), _ptr, _ptr,
                                     _ptr]),
    "rba_decode_split_ex": (ctypes.c_int, [ctypes.POINTER(AttnParams), _ptr, _ptr, _ptr, _i32, _ptr, _ptr, _ptr,
                                           _i32, _i32, _i32, _i32, _i32, _ptr, _size,
                                           ctypes.POINTER(CallOptions), _ptr]),
    "rba_decode_relproj_workspace_size": (_size, [ctypes.POINTER(AttnParams), _i32, _i32, _i32, _i32]),
    "rba_decode_relproj": (ctypes.c_int, [ctypes.POINTER(AttnParams), _ptr, _ptr, _ptr, _i32, _ptr, _ptr, _i32,
                                          _i32, _ptr, _ptr, _i32, _i32, _i32, _i32, _i32, _ptr, _size,
                                          ctypes.POINTER(CallOptions), _ptr, _ptr, _ptr]),
}

NOALLOC_SCRATCH_BYTES = 16 << 20   # RBA_NOALLOC_SCRATCH_BYTES in include/rba.h

_lib = None


def lib() -> ctypes.CDLL:
    """Load librba.so (built in-tree). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def version() -> str:
    return lib().rba_version().decode()


def last_error() -> str:
    return lib().rba_last_error().decode()


def _check(rc: int) -> None:
    if rc != RBA_OK:
        raise RbaError(rc, last_error())


def params(num_heads_q: int, num_heads_kv: int, head_dim_v: int, rel_extent: int, window: int,
           scale: float, head_dim_qk: int = 128, block_size: int = BLOCK_SIZE) -> AttnParams:
    return AttnParams(num_heads_q, num_heads_kv, head_dim_qk, head_dim_v, rel_extent, window, scale,
                      block_size)


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _shape(t: Optional[torch.Tensor], shape, name: str) -> None:
    """Raise unless tensor t (if given) has exactly this shape."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {list(shape)}, got {list(t.shape)}")


def _cache_shapes(q, k_cache, v_cache, block_tables, batch):
    """q [rows, Hq, 128]; caches [nb, Hkv, 128, 128] / [nb, Hkv, 128, dv];
    block_tables [>= batch, max_blocks]."""
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.dim() != 4:
        raise ValueError("q must be 3-D and k_cache / v_cache 4-D")
    if v_cache.shape[:3] != k_cache.shape[:3] or k_cache.shape[3] != q.shape[2]:
        raise ValueError("k_cache [nb, Hkv, 128, dqk] and v_cache [nb, Hkv, 128, dv] disagree with q")
    if block_tables.dim() != 2 or block_tables.shape[0] < batch:
        raise ValueError("block_tables must be [batch, max_blocks]")


def _opt(t: Optional[torch.Tensor], name: str, shape) -> Optional[int]:
    """Device pointer of an optional fp32 [rows, Hq] input (sink / gate)."""
    if t is None:
        return None
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {list(shape)}")
    return _dev(t, torch.float32, name)


def call_options(rows: int, Hq: int, sink: Optional[torch.Tensor] = None, gate: Optional[torch.Tensor] = None,
                 logit_scale: Optional[torch.Tensor] = None,
                 kv_scales: Optional[Tuple[float, float]] = None) -> Optional[CallOptions]:
    """rba_call_options for the given optional terms (None if there are
    none): sink / gate fp32 [rows, Hq], logit_scale fp32 [rows], kv_scales =
    (k_scale, v_scale) for e4m3 caches."""
    if sink is None and gate is None and logit_scale is None and kv_scales is None:
        return None
    if logit_scale is not None and tuple(logit_scale.shape) != (rows,):
        raise ValueError(f"logit_scale must be [{rows}]")
    o = CallOptions()
    o.sink = _opt(sink, "sink", (rows, Hq))
    o.gate = _opt(gate, "gate", (rows, Hq))
    o.logit_scale = _dev(logit_scale, torch.float32, "logit_scale") if logit_scale is not None else None
    o.kv_e4m3 = 1 if kv_scales is not None else 0
    o.k_scale, o.v_scale = (float(kv_scales[0]), float(kv_scales[1])) if kv_scales is not None else (1.0, 1.0)
    return o


def _prefill_batch(cu_q, seq_lens) -> int:
    """Sequence count of a prefill call: cu_q holds batch + 1 offsets and
    seq_lens one length per sequence."""
    if cu_q.dim() != 1 or cu_q.numel() < 1:
        raise ValueError("cu_q must hold batch + 1 offsets")
    batch = cu_q.numel() - 1
    if seq_lens.numel() != batch:
        raise ValueError(f"seq_lens must have {batch} entries (cu_q.numel() - 1)")
    return batch


def prefill(q, k_cache, v_cache, rel, cu_q, seq_lens, block_tables, *, window: int, scale: float,
            max_q_len: int, max_seq_len: int, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None, want_lse: bool = False,
            sink: Optional[torch.Tensor] = None, gate: Optional[torch.Tensor] = None,
            logit_scale: Optional[torch.Tensor] = None, kv_scales: Optional[Tuple[float, float]] = None,
            stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """rba_prefill. q [total_q, Hq, 128] bf16; k_cache [nb, Hkv, 128, 128] bf16;
    v_cache [nb, Hkv, 128, dv] bf16; rel [total_q, Hq, R] fp32; cu_q [B+1],
    seq_lens [B], block_tables [B, max_blocks] int32. max_q_len / max_seq_len
    are host-side bounds (no device read happens here). With sink and/or gate
    (fp32 [total_q, Hq]), logit_scale (fp32 [total_q]) and/or kv_scales =
    (k_scale, v_scale) for e4m3 caches (uint8 or torch.float8_e4m3fn), in
    any combination, rba_prefill_ex runs."""
    total_q, Hq, dqk = q.shape
    nb, Hkv, bs, _ = k_cache.shape
    dv = v_cache.shape[3]
    R = rel.shape[2]
    if rel.dim() != 3 or rel.shape[:2] != (total_q, Hq):
        raise ValueError("rel must be [total_q, Hq, R]")
    batch = _prefill_batch(cu_q, seq_lens)
    _cache_shapes(q, k_cache, v_cache, block_tables, batch)
    if out is None:
        out = torch.empty((total_q, Hq, dv), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((total_q, Hq), dtype=torch.float32, device=q.device)
    _shape(out, (total_q, Hq, dv), "out")
    _shape(lse, (total_q, Hq), "lse")
    p = params(Hq, Hkv, dv, R, window, scale, dqk, bs)
    kvt = torch.uint8 if kv_scales is not None else torch.bfloat16
    k_cache, v_cache = (_kv8(k_cache), _kv8(v_cache)) if kv_scales is not None else (k_cache, v_cache)
    args = (ctypes.byref(p), _dev(q, torch.bfloat16, "q"), _dev(k_cache, kvt, "k_cache"),
            _dev(v_cache, kvt, "v_cache"), nb, _dev(rel, torch.float32, "rel"),
            _dev(cu_q, torch.int32, "cu_q"), _dev(seq_lens, torch.int32, "seq_lens"),
            _dev(block_tables, torch.int32, "block_tables"), block_tables.shape[1], batch, int(max_q_len),
            int(max_seq_len))
    tail = (_dev(out, torch.float32, "out"), _dev(lse, torch.float32, "lse") if lse is not None else None,
            _stream(stream))
    opts = call_options(total_q, Hq, sink, gate, logit_scale, kv_scales)
    if opts is None:
        _check(lib().rba_prefill(*args, *tail))
    else:
        _check(lib().rba_prefill_ex(*args, ctypes.byref(opts), *tail))
    return out, lse


def prefill_relproj(q, k_cache, v_cache, r, proj, cu_q, seq_lens, block_tables, *, window: int, scale: float,
                    max_q_len: int, max_seq_len: int, out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, want_lse: bool = False,
                    sink: Optional[torch.Tensor] = None, gate: Optional[torch.Tensor] = None,
                    logit_scale: Optional[torch.Tensor] = None, kv_scales: Optional[Tuple[float, float]] = None,
                    stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """rba_prefill_relproj: as prefill, with the bias made in the kernel from
    r [total_q, Hq, d_r] bf16 and proj [1 or Hq, R, d_r] bf16 (d_r 32, 64 or
    128; rel_logits_proj in linear-weight layout; R = proj.shape[1]). With
    logit_scale (fp32 [total_q]) and/or kv_scales (e4m3 caches)
    rba_prefill_relproj_ex runs."""
    total_q, Hq, dqk = q.shape
    nb, Hkv, bs, _ = k_cache.shape
    dv = v_cache.shape[3]
    if r.dim() != 3 or r.shape[:2] != (total_q, Hq):
        raise ValueError("r must be [total_q, Hq, d_r]")
    d_r = r.shape[2]
    if proj.dim() != 3 or proj.shape[2] != d_r:
        raise ValueError("proj must be [proj_heads, R, d_r]")
    proj_heads, R = proj.shape[0], proj.shape[1]
    batch = _prefill_batch(cu_q, seq_lens)
    _cache_shapes(q, k_cache, v_cache, block_tables, batch)
    if out is None:
        out = torch.empty((total_q, Hq, dv), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((total_q, Hq), dtype=torch.float32, device=q.device)
    _shape(out, (total_q, Hq, dv), "out")
    _shape(lse, (total_q, Hq), "lse")
    p = params(Hq, Hkv, dv, R, window, scale, dqk, bs)
    kvt = torch.uint8 if kv_scales is not None else torch.bfloat16
    k_cache, v_cache = (_kv8(k_cache), _kv8(v_cache)) if kv_scales is not None else (k_cache, v_cache)
    args = (ctypes.byref(p), _dev(q, torch.bfloat16, "q"), _dev(k_cache, kvt, "k_cache"),
            _dev(v_cache, kvt, "v_cache"), nb, _dev(r, torch.bfloat16, "r"),
            _dev(proj, torch.bfloat16, "proj"), d_r, proj_heads,
            _dev(cu_q, torch.int32, "cu_q"), _dev(seq_lens, torch.int32, "seq_lens"),
            _dev(block_tables, torch.int32, "block_tables"), block_tables.shape[1], batch, int(max_q_len),
            int(max_seq_len))
    tail = (_dev(out, torch.float32, "out"), _dev(lse, torch.float32, "lse") if lse is not None else None,
            _stream(stream))
    if logit_scale is None and kv_scales is None:
        _check(lib().rba_prefill_relproj(*args, _opt(sink, "sink", (total_q, Hq)), _opt(gate, "gate", (total_q, Hq)),
                                         *tail))
    else:
        opts = call_options(total_q, Hq, sink, gate, logit_scale, kv_scales)
        _check(lib().rba_prefill_relproj_ex(*args, ctypes.byref(opts), *tail))
    return out, lse


def _num_cus(device) -> int:
    return torch.cuda.get_device_properties(device).multi_processor_count


def plan_splits(Hq, Hkv, dv, rel_extent, window, scale, batch, n_q, max_seq_len, num_cus=256) -> int:
    p = params(Hq, Hkv, dv, rel_extent, window, scale)
    n = lib().rba_decode_plan_splits(ctypes.byref(p), batch, n_q, max_seq_len, num_cus)
    if n < 1:
        raise RbaError(n, last_error())
    return n


def workspace_size(Hq, Hkv, dv, rel_extent, window, scale, batch, n_q, max_seq_len, num_splits=0) -> int:
    p = params(Hq, Hkv, dv, rel_extent, window, scale)
    return lib().rba_decode_workspace_size(ctypes.byref(p), batch, n_q, max_seq_len, num_splits)


def _decode_common(q, k_cache, v_cache, rel, seq_lens, block_tables, n_q, window, scale):
    rows, Hq, dqk = q.shape
    nb, Hkv, bs, _ = k_cache.shape
    dv = v_cache.shape[3]
    R = rel.shape[2]
    if rows % n_q != 0:
        raise ValueError("q rows must be batch * n_q")
    if rel.shape[:2] != (rows, Hq):
        raise ValueError("rel must be [batch * n_q, Hq, R]")
    batch = rows // n_q
    if seq_lens.numel() != batch:
        raise ValueError("seq_lens must have batch entries")
    _cache_shapes(q, k_cache, v_cache, block_tables, batch)
    return params(Hq, Hkv, dv, R, window, scale, dqk, bs), batch, rows, Hq, dv, nb


def _kv8(t: torch.Tensor) -> torch.Tensor:
    """An e4m3 cache as raw bytes (uint8 or torch.float8_e4m3fn accepted)."""
    return t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t


def decode(q, k_cache, v_cache, rel, seq_lens, block_tables, *, n_q: int, window: int, scale: float,
           max_seq_len: int, num_splits: int = 0, workspace: Optional[torch.Tensor] = None,
           out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
           want_lse: bool = False, kv_scales: Optional[Tuple[float, float]] = None,
           sink: Optional[torch.Tensor] = None, gate: Optional[torch.Tensor] = None,
           logit_scale: Optional[torch.Tensor] = None,
           stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """rba_decode (split-KV + combine). q [batch*n_q, Hq, 128] bf16; rel
    [batch*n_q, Hq, R] fp32. `workspace` (uint8, on the GPU) is allocated with
    torch if not given. Optional terms, in any combination (rba_decode_ex):
    kv_scales = (k_scale, v_scale) for e4m3 caches (uint8 or
    torch.float8_e4m3fn), sink and/or gate (fp32 [batch*n_q, Hq]) and
    logit_scale (fp32 [batch*n_q])."""
    p, batch, rows, Hq, dv, nb = _decode_common(q, k_cache, v_cache, rel, seq_lens, block_tables, n_q,
                                                window, scale)
    L = lib()
    need = L.rba_decode_workspace_size(ctypes.byref(p), batch, n_q, int(max_seq_len), int(num_splits))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((rows, Hq, dv), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((rows, Hq), dtype=torch.float32, device=q.device)
    _shape(out, (rows, Hq, dv), "out")
    _shape(lse, (rows, Hq), "lse")
    k8 = _kv8(k_cache) if kv_scales is not None else k_cache
    v8 = _kv8(v_cache) if kv_scales is not None else v_cache
    kvt = torch.uint8 if kv_scales is not None else torch.bfloat16
    args = (ctypes.byref(p), _dev(q, torch.bfloat16, "q"), _dev(k8, kvt, "k_cache"), _dev(v8, kvt, "v_cache"), nb,
            _dev(rel, torch.float32, "rel"), _dev(seq_lens, torch.int32, "seq_lens"),
            _dev(block_tables, torch.int32, "block_tables"), block_tables.shape[1], batch, n_q, int(max_seq_len),
            int(num_splits), _dev(workspace, torch.uint8, "workspace"), workspace.numel())
    tail = (_dev(out, torch.float32, "out"), _dev(lse, torch.float32, "lse") if lse is not None else None,
            _stream(stream))
    opts = call_options(rows, Hq, sink, gate, logit_scale, kv_scales)
    if opts is None:
        _check(L.rba_decode(*args, *tail))
    else:
        _check(L.rba_decode_ex(*args, ctypes.byref(opts), *tail))
    return out, lse


def relproj_workspace_size(Hq, Hkv, dv, rel_extent, window, scale, batch, n_q, max_seq_len, num_splits=0) -> int:
    p = params(Hq, Hkv, dv, rel_extent, window, scale)
    return lib().rba_decode_relproj_workspace_size(ctypes.byref(p), batch, n_q, max_seq_len, num_splits)


def decode_relproj(q, k_cache, v_cache, r, proj, seq_lens, block_tables, *, n_q: int, window: int,
                   scale: float, max_seq_len: int, num_splits: int = 0, workspace: Optional[torch.Tensor] = None,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   want_lse: bool = False, kv_scales: Optional[Tuple[float, float]] = None,
                   sink: Optional[torch.Tensor] = None, gate: Optional[torch.Tensor] = None,
                   logit_scale: Optional[torch.Tensor] = None,
                   stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """rba_decode_relproj: as decode, with the bias rows made by the library
    from r [batch*n_q, Hq, d_r] bf16 and proj [1 or Hq, R, d_r] bf16 (d_r 32,
    64 or 128; R = proj.shape[1]). `workspace` (uint8) holds the split
    partials and the bias rows; allocated with torch if not given."""
    rows, Hq, dqk = q.shape
    if r.dim() != 3 or r.shape[:2] != (rows, Hq):
        raise ValueError("r must be [batch * n_q, Hq, d_r]")
    d_r = r.shape[2]
    if proj.dim() != 3 or proj.shape[2] != d_r:
        raise ValueError("proj must be [proj_heads, R, d_r]")
    proj_heads, R = proj.shape[0], proj.shape[1]
    nb, Hkv, bs, _ = k_cache.shape
    dv = v_cache.shape[3]
    if rows % n_q != 0:
        raise ValueError("q rows must be batch * n_q")
    batch = rows // n_q
    if seq_lens.numel() != batch:
        raise ValueError("seq_lens must have batch entries")
    _cache_shapes(q, k_cache, v_cache, block_tables, batch)
    p = params(Hq, Hkv, dv, R, window, scale, dqk, bs)
    L = lib()
    need = L.rba_decode_relproj_workspace_size(ctypes.byref(p), batch, n_q, int(max_seq_len), int(num_splits))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((rows, Hq, dv), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((rows, Hq), dtype=torch.float32, device=q.device)
    _shape(out, (rows, Hq, dv), "out")
    _shape(lse, (rows, Hq), "lse")
    k8 = _kv8(k_cache) if kv_scales is not None else k_cache
    v8 = _kv8(v_cache) if kv_scales is not None else v_cache
    kvt = torch.uint8 if kv_scales is not None else torch.bfloat16
    opts = call_options(rows, Hq, sink, gate, logit_scale, kv_scales)
    _check(L.rba_decode_relproj(
        ctypes.byref(p), _dev(q, torch.bfloat16, "q"), _dev(k8, kvt, "k_cache"), _dev(v8, kvt, "v_cache"), nb,
        _dev(r, torch.bfloat16, "r"), _dev(proj, torch.bfloat16, "proj"), d_r, proj_heads,
        _dev(seq_lens, torch.int32, "seq_lens"), _dev(block_tables, torch.int32, "block_tables"),
        block_tables.shape[1], batch, n_q, int(max_seq_len), int(num_splits), _dev(workspace, torch.uint8, "workspace"),
        workspace.numel(), ctypes.byref(opts) if opts is not None else None, _dev(out, torch.float32, "out"),
        _dev(lse, torch.float32, "lse") if lse is not None else None, _stream(stream)))
    return out, lse


def decode_split(q, k_cache, v_cache, rel, seq_lens, block_tables, *, n_q: int, window: int, scale: float,
                 max_seq_len: int, num_splits: int, workspace: torch.Tensor,
                 kv_scales: Optional[Tuple[float, float]] = None, logit_scale: Optional[torch.Tensor] = None,
                 stream=None) -> None:
    """rba_decode_split: partial outputs of every split into `workspace`
    (rba_decode_split_ex with kv_scales (e4m3 caches) and/or logit_scale)."""
    p, batch, rows, Hq, dv, nb = _decode_common(q, k_cache, v_cache, rel, seq_lens, block_tables, n_q,
                                                window, scale)
    k8 = _kv8(k_cache) if kv_scales is not None else k_cache
    v8 = _kv8(v_cache) if kv_scales is not None else v_cache
    kvt = torch.uint8 if kv_scales is not None else torch.bfloat16
    args = (ctypes.byref(p), _dev(q, torch.bfloat16, "q"), _dev(k8, kvt, "k_cache"), _dev(v8, kvt, "v_cache"), nb,
            _dev(rel, torch.float32, "rel"), _dev(seq_lens, torch.int32, "seq_lens"),
            _dev(block_tables, torch.int32, "block_tables"), block_tables.shape[1], batch, n_q, int(max_seq_len),
            int(num_splits), _dev(workspace, torch.uint8, "workspace"), workspace.numel())
    opts = call_options(rows, Hq, logit_scale=logit_scale, kv_scales=kv_scales)
    if opts is None:
        _check(lib().rba_decode_split(*args, _stream(stream)))
    else:
        _check(lib().rba_decode_split_ex(*args, ctypes.byref(opts), _stream(stream)))


def decode_combine(*, Hq: int, Hkv: int, dv: int, rel_extent: int, window: int, scale: float, batch: int,
                   n_q: int, num_splits: int, workspace: torch.Tensor, out: torch.Tensor,
                   lse: Optional[torch.Tensor] = None, sink: Optional[torch.Tensor] = None,
                   gate: Optional[torch.Tensor] = None, stream=None) -> None:
    """rba_decode_combine: log-sum-exp merge of the partials in `workspace`
    (rba_decode_combine_gated with sink and/or gate)."""
    p = params(Hq, Hkv, dv, rel_extent, window, scale)
    _shape(out, (batch * n_q, Hq, dv), "out")
    _shape(lse, (batch * n_q, Hq), "lse")
    if sink is not None or gate is not None:
        rows = batch * n_q
        _check(lib().rba_decode_combine_gated(
            ctypes.byref(p), batch, n_q, int(num_splits), _dev(workspace, torch.uint8, "workspace"),
            workspace.numel(), _opt(sink, "sink", (rows, Hq)), _opt(gate, "gate", (rows, Hq)),
            _dev(out, torch.float32, "out"), _dev(lse, torch.float32, "lse") if lse is not None else None,
            _stream(stream)))
        return
    _check(lib().rba_decode_combine(
        ctypes.byref(p), batch, n_q, int(num_splits), _dev(workspace, torch.uint8, "workspace"),
        workspace.numel(), _dev(out, torch.float32, "out"),
        _dev(lse, torch.float32, "lse") if lse is not None else None, _stream(stream)))


def decode_noalloc(q, k_cache, v_cache, rel, seq_lens, block_tables, *, n_q: int, window: int, scale: float,
                   max_seq_len: int, num_splits: int = 0, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, want_lse: bool = False,
                   stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """rba_decode_noalloc: rba_decode with the split partials in the
    library's own device scratch (no workspace argument; the library
    allocates nothing). Calls that overlap on one GPU share that scratch and
    race. bf16 caches; out / lse are allocated with torch if not given."""
    p, batch, rows, Hq, dv, nb = _decode_common(q, k_cache, v_cache, rel, seq_lens, block_tables, n_q,
                                                window, scale)
    if out is None:
        out = torch.empty((rows, Hq, dv), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((rows, Hq), dtype=torch.float32, device=q.device)
    _shape(out, (rows, Hq, dv), "out")
    _shape(lse, (rows, Hq), "lse")
    _check(lib().rba_decode_noalloc(
        ctypes.byref(p), _dev(q, torch.bfloat16, "q"), _dev(k_cache, torch.bfloat16, "k_cache"),
        _dev(v_cache, torch.bfloat16, "v_cache"), nb, _dev(rel, torch.float32, "rel"),
        _dev(seq_lens, torch.int32, "seq_lens"), _dev(block_tables, torch.int32, "block_tables"),
        block_tables.shape[1], batch, n_q, int(max_seq_len), int(num_splits), _dev(out, torch.float32, "out"),
        _dev(lse, torch.float32, "lse") if lse is not None else None, _stream(stream)))
    return out, lse

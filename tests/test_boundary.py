"""CPU tests of the C-ABI boundary: the library loads, exports every symbol
the header declares, and its host-side validation / planning behave as the
header documents. No compute call is made (no GPU here); pointers passed to
the validators are fake aligned addresses that are never dereferenced."""
import ctypes
import math
import os
import re

import pytest

from relative_position_bias_amd import rba

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rba.h")
P = 0x10000          # a fake, 16-byte aligned device address


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rba_[a-z0-9_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = rba.lib()
    names = declared_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), f"{name} declared in rba.h but not exported"
    assert set(names) == set(rba._SIGNATURES), "binding and header disagree"
    assert rba.version().startswith("librba")


def prm(**kw):
    base = dict(num_heads_q=32, num_heads_kv=8, head_dim_v=128, rel_extent=512, window=512,
                scale=128 ** -0.5)
    base.update(kw)
    return rba.params(**base)


def vprefill(p, q=P, k=P, v=P, nb=64, rel=P, cu=P, sl=P, tab=P, maxb=64, batch=1, mql=8192, msl=8192,
             out=P):
    return rba.lib().rba_validate_prefill(ctypes.byref(p) if p is not None else None, q, k, v, nb, rel, cu,
                                          sl, tab, maxb, batch, mql, msl, out)


def vdecode(p, q=P, k=P, v=P, nb=2560, rel=P, sl=P, tab=P, maxb=1024, batch=16, n_q=1, msl=131072,
            splits=0, ws=P, ws_bytes=1 << 30, out=P):
    return rba.lib().rba_validate_decode(ctypes.byref(p) if p is not None else None, q, k, v, nb, rel, sl,
                                         tab, maxb, batch, n_q, msl, splits, ws, ws_bytes, out)


def test_validate_prefill_accepts_the_workloads():
    assert vprefill(prm()) == rba.RBA_OK
    assert vprefill(prm(num_heads_q=4, num_heads_kv=1, rel_extent=128, window=64), nb=2, maxb=2, mql=256,
                    msl=256) == rba.RBA_OK
    assert vprefill(prm(rel_extent=1024, window=0), nb=256, maxb=256, msl=32768) == rba.RBA_OK
    assert rba.last_error() == ""


@pytest.mark.parametrize("kw,code", [
    (dict(num_heads_q=0), rba.RBA_ERR_SHAPE),
    (dict(num_heads_q=30), rba.RBA_ERR_SHAPE),          # not a multiple of Hkv
    (dict(head_dim_v=96), rba.RBA_ERR_UNSUPPORTED),
    (dict(rel_extent=0), rba.RBA_ERR_SHAPE),
    (dict(window=-1), rba.RBA_ERR_SHAPE),
    (dict(scale=math.inf), rba.RBA_ERR_SHAPE),
    (dict(scale=math.nan), rba.RBA_ERR_SHAPE),
])
def test_validate_prefill_rejects_bad_params(kw, code):
    assert vprefill(prm(**kw)) == code
    assert rba.last_error() != ""


def test_validate_params_head_dim_and_block_size():
    p = prm()
    p.head_dim_qk = 64
    assert vprefill(p) == rba.RBA_ERR_UNSUPPORTED
    p = prm()
    p.block_size = 64
    assert vprefill(p) == rba.RBA_ERR_UNSUPPORTED
    assert vprefill(None) == rba.RBA_ERR_NULL


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), rba.RBA_ERR_NULL),
    (dict(k=None), rba.RBA_ERR_NULL),
    (dict(rel=None), rba.RBA_ERR_NULL),
    (dict(cu=None), rba.RBA_ERR_NULL),
    (dict(tab=None), rba.RBA_ERR_NULL),
    (dict(out=None), rba.RBA_ERR_NULL),
    (dict(q=P + 8), rba.RBA_ERR_UNSUPPORTED),          # misaligned
    (dict(rel=P + 2), rba.RBA_ERR_UNSUPPORTED),        # fp32 rel needs 4-byte alignment
    (dict(nb=0), rba.RBA_ERR_SHAPE),
    (dict(maxb=63), rba.RBA_ERR_SHAPE),                # < ceil(8192/128)
    (dict(batch=-1), rba.RBA_ERR_SHAPE),
    (dict(mql=-1), rba.RBA_ERR_SHAPE),
    (dict(mql=100, msl=50), rba.RBA_ERR_SHAPE),
])
def test_validate_prefill_rejects_bad_arguments(kw, code):
    assert vprefill(prm(), **kw) == code


@pytest.mark.parametrize("R", [1, 5, 127, 510, 1023])
def test_any_rel_extent_is_accepted(R):
    """R >= 1 of any size: fp32 rel rows then start at 4-byte multiples,
    which is all the kernels ask of rel."""
    assert vprefill(prm(rel_extent=R), rel=P + 4) == rba.RBA_OK
    assert vdecode(prm(rel_extent=R, window=0), rel=P + 4) == rba.RBA_OK


def test_validate_prefill_empty_call_needs_no_pointers():
    assert vprefill(prm(), q=None, k=None, v=None, rel=None, cu=None, sl=None, tab=None, out=None,
                    batch=0) == rba.RBA_OK
    assert vprefill(prm(), q=None, k=None, v=None, rel=None, cu=None, sl=None, tab=None, out=None,
                    mql=0) == rba.RBA_OK


def dprm(**kw):
    base = dict(num_heads_q=32, num_heads_kv=8, head_dim_v=128, rel_extent=1024, window=0,
                scale=128 ** -0.5)
    base.update(kw)
    return rba.params(**base)


def test_validate_decode_accepts_the_workloads():
    assert vdecode(dprm()) == rba.RBA_OK
    p5 = dprm(num_heads_q=64, head_dim_v=64)
    assert vdecode(p5, batch=8, n_q=4, msl=100000, maxb=782, nb=6256) == rba.RBA_OK


@pytest.mark.parametrize("kw,code", [
    (dict(n_q=0), rba.RBA_ERR_SHAPE),
    (dict(n_q=65), rba.RBA_ERR_UNSUPPORTED),          # G * n_q = 260 > 256
    (dict(msl=0), rba.RBA_ERR_SHAPE),
    (dict(splits=-1), rba.RBA_ERR_SHAPE),
    (dict(splits=1025), rba.RBA_ERR_SHAPE),
    (dict(ws=None), rba.RBA_ERR_WORKSPACE),
    (dict(ws_bytes=1000), rba.RBA_ERR_WORKSPACE),
    (dict(ws=P + 4), rba.RBA_ERR_UNSUPPORTED),
    (dict(out=None), rba.RBA_ERR_NULL),
    (dict(sl=None), rba.RBA_ERR_NULL),
    (dict(maxb=1023), rba.RBA_ERR_SHAPE),
    (dict(batch=-2), rba.RBA_ERR_SHAPE),
])
def test_validate_decode_rejects_bad_arguments(kw, code):
    assert vdecode(dprm(), **kw) == code
    assert rba.last_error() != ""


def test_workspace_size_formula():
    # [batch*n_q, Hq, splits, dv] + [batch*n_q, Hq, splits] fp32
    assert rba.workspace_size(32, 8, 128, 1024, 0, 0.1, 16, 1, 131072, 16) == 16 * 32 * 16 * 129 * 4
    assert rba.workspace_size(64, 8, 64, 1024, 0, 0.1, 8, 4, 100000, 7) == 32 * 64 * 7 * 65 * 4
    assert rba.workspace_size(64, 8, 64, 1024, 0, 0.1, 8, 4, 100000, 2000) == 0   # bad split count


def test_split_plan():
    # 16 sequences x 8 KV heads, up to 1024 blocks: one round of 512 units
    # would need 256 blocks per split, so 32-block splits
    assert rba.plan_splits(32, 8, 128, 1024, 0, 0.1, 16, 1, 131072, 256) == 32
    # batch 1, 100K context, dv 64 (a prefetching kernel): one workgroup per CU,
    # 32 splits of 25 blocks
    assert rba.plan_splits(64, 8, 64, 1024, 0, 0.1, 1, 4, 100000, 256) == 32
    # the same with dv 128 (no prefetch in the 32-column kernel): two per CU would
    # be 64 splits, bounded by ~16 blocks per split
    assert rba.plan_splits(64, 8, 128, 1024, 0, 0.1, 1, 4, 100000, 256) == 49
    # batch 8: exactly one round of 2 x 256 units (98 blocks per split)
    assert rba.plan_splits(64, 8, 64, 1024, 0, 0.1, 8, 4, 100000, 256) == 8
    # a window bounds the blocks any query group can see
    assert rba.plan_splits(32, 8, 128, 512, 512, 0.1, 1, 1, 131072, 256) == 1
    for batch in (1, 3, 64, 1000):
        for msl in (1, 127, 128, 129, 5000, 1 << 20):
            s = rba.plan_splits(32, 8, 128, 1024, 0, 0.1, batch, 1, msl, 256)
            nb = -(-msl // 128)
            assert 1 <= s <= min(256, max(1, -(-nb // 16)))
    with pytest.raises(rba.RbaError):
        rba.plan_splits(32, 8, 128, 1024, 0, 0.1, 1, 1, 100, 0)


def test_combine_validation():
    lib = rba.lib()
    p = dprm()
    assert lib.rba_decode_combine(ctypes.byref(p), 4, 1, 0, P, 1 << 20, P, None, None) == rba.RBA_ERR_SHAPE
    assert lib.rba_decode_combine(ctypes.byref(p), 4, 1, 2, P, 100, P, None, None) == rba.RBA_ERR_WORKSPACE
    assert lib.rba_decode_combine(ctypes.byref(p), 4, 1, 2, P, 1 << 20, None, None, None) == rba.RBA_ERR_NULL
    assert lib.rba_decode_combine(ctypes.byref(p), 0, 1, 2, None, 0, None, None, None) == rba.RBA_OK


def test_decode_split_needs_resolved_split_count():
    lib = rba.lib()
    p = dprm()
    rc = lib.rba_decode_split(ctypes.byref(p), P, P, P, 2560, P, P, P, 1024, 16, 1, 131072, 0, P, 1 << 30,
                              None)
    assert rc == rba.RBA_ERR_SHAPE


def test_errors_are_thread_local():
    import threading
    assert vprefill(prm(num_heads_q=0)) == rba.RBA_ERR_SHAPE
    seen = []
    t = threading.Thread(target=lambda: seen.append(rba.last_error()))
    t.start()
    t.join()
    assert seen == [""]
    assert rba.last_error() != ""


def test_fp8_decode_rejects_bad_scales():
    """Scale checks run before any HIP call (no device needed)."""
    lib = rba.lib()
    p = dprm()
    for ks, vs in ((0.0, 1.0), (1.0, -2.0), (float("nan"), 1.0), (1.0, float("inf"))):
        rc = lib.rba_decode_fp8(ctypes.byref(p), P, P, P, 2560, ks, vs, P, P, P, 1024, 16, 1, 131072, 0, P,
                                1 << 30, P, None, None)
        assert rc == rba.RBA_ERR_SHAPE, (ks, vs, rc)
        rc = lib.rba_decode_split_fp8(ctypes.byref(p), P, P, P, 2560, ks, vs, P, P, P, 1024, 16, 1, 131072, 8,
                                      P, 1 << 30, None)
        assert rc == rba.RBA_ERR_SHAPE, (ks, vs, rc)


def test_relproj_prefill_rejects_bad_arguments():
    """rba_prefill_relproj's own checks run before any HIP call (no device needed)."""
    lib = rba.lib()
    p = prm()

    def call(r=P, proj=P, d_r=64, heads=1, q=P, out=P, batch=1):
        return lib.rba_prefill_relproj(ctypes.byref(p), q, P, P, 64, r, proj, d_r, heads, P, P, P, 64, batch,
                                       8192, 8192, None, None, out, None, None)

    assert call(d_r=48) == rba.RBA_ERR_UNSUPPORTED
    assert "d_r" in rba.last_error()
    assert call(d_r=16) == rba.RBA_ERR_UNSUPPORTED
    assert call(d_r=256) == rba.RBA_ERR_UNSUPPORTED
    assert call(heads=3) == rba.RBA_ERR_SHAPE
    assert call(heads=0) == rba.RBA_ERR_SHAPE
    assert call(proj=None) == rba.RBA_ERR_NULL
    assert call(proj=P + 8) == rba.RBA_ERR_UNSUPPORTED   # not 16-byte aligned
    assert call(r=None) == rba.RBA_ERR_NULL
    assert "r" in rba.last_error()
    assert call(r=P + 4) == rba.RBA_ERR_UNSUPPORTED
    assert call(q=None) == rba.RBA_ERR_NULL
    assert call(batch=0) == rba.RBA_OK                    # empty call: nothing to do, no launch


def test_logpos_rejects_missing_or_misaligned_scale():
    """Checks of rba_prefill_logpos / rba_decode_logpos run before any HIP call."""
    lib = rba.lib()
    p = prm()
    rc = lib.rba_prefill_logpos(ctypes.byref(p), P, P, P, 64, P, P, P, P, 64, 1, 8192, 8192, None, P, None, None)
    assert rc == rba.RBA_ERR_NULL and "logit_scale" in rba.last_error()
    rc = lib.rba_prefill_logpos(ctypes.byref(p), P, P, P, 64, P, P, P, P, 64, 1, 8192, 8192, P + 2, P, None, None)
    assert rc == rba.RBA_ERR_UNSUPPORTED
    assert lib.rba_prefill_logpos(ctypes.byref(p), P, P, P, 64, P, P, P, P, 64, 0, 8192, 8192, None, P, None,
                                  None) == rba.RBA_OK   # empty call
    d = dprm()
    rc = lib.rba_decode_logpos(ctypes.byref(d), P, P, P, 2560, P, P, P, 1024, 16, 1, 131072, 8, P, 1 << 30, None,
                               P, None, None)
    assert rc == rba.RBA_ERR_NULL
    rc = lib.rba_decode_logpos(ctypes.byref(d), P, P, P, 2560, P, P, P, 1024, 16, 1, 131072, 8, P, 1 << 30, P + 2,
                               P, None, None)
    assert rc == rba.RBA_ERR_UNSUPPORTED


def test_options_are_checked_before_any_launch():
    """rba_*_ex: the options struct is read and checked on the host first."""
    lib = rba.lib()
    p = prm()
    d = dprm()

    def opts(**kw):
        o = rba.CallOptions()
        o.k_scale = o.v_scale = 1.0
        for k, v in kw.items():
            setattr(o, k, v)
        return ctypes.byref(o)

    def pre(o, batch=1):
        return lib.rba_prefill_ex(ctypes.byref(p), P, P, P, 64, P, P, P, P, 64, batch, 8192, 8192, o, P, None, None)

    def rel(o):
        return lib.rba_prefill_relproj_ex(ctypes.byref(p), P, P, P, 64, P, P, 64, 1, P, P, P, 64, 1, 8192, 8192, o,
                                          P, None, None)

    def dec(o, splits=0):
        return lib.rba_decode_ex(ctypes.byref(d), P, P, P, 2560, P, P, P, 1024, 16, 1, 131072, splits, P, 1 << 30,
                                 o, P, None, None)

    def split(o, splits=8):
        return lib.rba_decode_split_ex(ctypes.byref(d), P, P, P, 2560, P, P, P, 1024, 16, 1, 131072, splits, P,
                                       1 << 30, o, None)

    assert rel(opts(kv_e4m3=1, k_scale=-1.0)) == rba.RBA_ERR_SHAPE
    assert pre(opts(kv_e4m3=1, k_scale=0.0)) == rba.RBA_ERR_SHAPE
    assert pre(opts(kv_e4m3=1, v_scale=float("inf"))) == rba.RBA_ERR_SHAPE
    assert pre(opts(kv_e4m3=2)) == rba.RBA_ERR_SHAPE
    assert dec(opts(kv_e4m3=-1)) == rba.RBA_ERR_SHAPE
    for field in ("sink", "gate", "logit_scale"):
        assert pre(opts(**{field: P + 2})) == rba.RBA_ERR_UNSUPPORTED, field
        assert dec(opts(**{field: P + 2})) == rba.RBA_ERR_UNSUPPORTED, field
    for ks, vs in ((0.0, 1.0), (1.0, float("nan")), (float("inf"), 1.0)):
        assert dec(opts(kv_e4m3=1, k_scale=ks, v_scale=vs)) == rba.RBA_ERR_SHAPE
        assert split(opts(kv_e4m3=1, k_scale=ks, v_scale=vs)) == rba.RBA_ERR_SHAPE
    assert split(opts(sink=P)) == rba.RBA_ERR_UNSUPPORTED         # sink / gate act in the combine
    assert "combine" in rba.last_error()
    assert split(opts(gate=P)) == rba.RBA_ERR_UNSUPPORTED
    assert split(None, splits=0) == rba.RBA_ERR_SHAPE             # resolved split count needed
    assert pre(opts(kv_e4m3=1), batch=0) == rba.RBA_OK
    assert pre(opts(sink=P, gate=P, logit_scale=P), batch=0) == rba.RBA_OK   # empty call, no launch


def test_call_options_marshalling():
    """The binding's options struct matches the header's field order."""
    names = [f[0] for f in rba.CallOptions._fields_]
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct rba_call_options \{(.*?)\} rba_call_options;", text, re.S).group(1)
    declared = re.findall(r"\b(\w+)\s*[;,]", body)
    assert declared == names
    assert rba.call_options(4, 2) is None


def test_decode_relproj_checks_before_any_launch():
    """rba_decode_relproj: the producer's arguments, the decode's and the
    workspace (partials, then the bias rows from the next multiple of 256
    bytes) are checked on the host before the first launch."""
    lib = rba.lib()
    d = dprm()
    ws = lib.rba_decode_workspace_size(ctypes.byref(d), 16, 1, 131072, 0)
    wr = lib.rba_decode_relproj_workspace_size(ctypes.byref(d), 16, 1, 131072, 0)
    assert wr == (ws + 255) // 256 * 256 + 16 * 1 * 32 * 1024 * 4
    assert lib.rba_decode_relproj_workspace_size(ctypes.byref(d), 16, 0, 131072, 0) == 0

    def call(r=P, proj=P, d_r=64, ph=1, nbytes=wr, o=None, batch=16):
        return lib.rba_decode_relproj(ctypes.byref(d), P, P, P, 2560, r, proj, d_r, ph, P, P, 1024, batch, 1,
                                      131072, 0, P, nbytes, o, P, None, None)

    assert call(d_r=48) == rba.RBA_ERR_UNSUPPORTED
    assert call(d_r=16) == rba.RBA_ERR_UNSUPPORTED
    assert call(ph=3) == rba.RBA_ERR_SHAPE
    assert call(r=None) == rba.RBA_ERR_NULL
    assert "q/r/seq_lens" in rba.last_error()
    assert call(proj=None) == rba.RBA_ERR_NULL
    assert call(r=P + 8) == rba.RBA_ERR_UNSUPPORTED
    assert call(proj=P + 4) == rba.RBA_ERR_UNSUPPORTED
    assert call(nbytes=wr - 1) == rba.RBA_ERR_WORKSPACE
    assert call(nbytes=ws) == rba.RBA_ERR_WORKSPACE          # room for the partials only
    o = rba.CallOptions()
    o.kv_e4m3, o.k_scale, o.v_scale = 1, 0.0, 1.0
    assert call(o=ctypes.byref(o)) == rba.RBA_ERR_SHAPE
    assert call(batch=0, nbytes=0) == rba.RBA_OK            # empty call, no launch

"""rba_decode_noalloc (the decode entry point that allocates nothing: its
split partials live in the library's own device scratch) against rba_decode
with a caller's workspace: same kernels and split plan, so the outputs are
bitwise equal. Two calls in a row, the second smaller, so the second reuses
the scratch the first left behind."""
import sys

import pytest
import torch

import workloads as W
from harness import run_decode
from relative_position_bias_amd import rba

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def noalloc(b, **kw):
    return rba.decode_noalloc(b.q, b.k_cache, b.v_cache, b.rel, b.seq_lens, b.block_tables, n_q=b.n_q,
                              window=b.W, scale=b.scale, max_seq_len=b.max_seq_len, want_lse=True, **kw)


CALLS = [
    # (seed, batch, n_q, Hq, Hkv, dv, R, W, seq_lens, splits): the second call of each pair is smaller
    ((61, 4, 1, 32, 8, 128, 1024, 0, [9000, 300, 20000, 4100], 0),
     (62, 2, 1, 32, 8, 128, 1024, 0, [700, 1500], 3)),
    ((63, 2, 4, 64, 8, 64, 1024, 0, [30000, 5000], 0),
     (64, 1, 4, 64, 8, 64, 512, 300, [2000], 0)),
    # 48 columns (both column groups in one workgroup)
    ((66, 2, 8, 48, 8, 128, 1024, 0, [12000, 3000], 0),
     (67, 1, 8, 48, 8, 128, 1024, 0, [2500], 2)),
]


@pytest.mark.parametrize("pair", CALLS, ids=["16col", "32col", "48col"])
def test_noalloc_decode_equals_workspace_decode(pair):
    for seed, batch, n_q, Hq, Hkv, dv, R, Wn, lens, splits in pair:
        say(f"no-alloc decode seed={seed} lens={lens} splits={splits}")
        b = W.make_decode(seed, batch, n_q, Hq, Hkv, dv, R, Wn, seq_lens=lens).to(DEV)
        o_ref, l_ref = run_decode(b, num_splits=splits, want_lse=True)
        o, l = noalloc(b, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.isfinite(o).all()
        assert torch.equal(o, o_ref) and torch.equal(l, l_ref)


def test_noalloc_rejects_calls_beyond_its_scratch():
    say("no-alloc size limit")
    b = W.make_decode(65, 16, 1, 32, 8, 128, 1024, 0, seq_lens=[40000] * 16).to(DEV)
    need = rba.workspace_size(32, 8, 128, 1024, 0, b.scale, 16, 1, b.max_seq_len, 256)
    assert need > rba.NOALLOC_SCRATCH_BYTES
    with pytest.raises(rba.RbaError) as e:
        noalloc(b, num_splits=256)
    assert e.value.code == rba.RBA_ERR_WORKSPACE

"""lvq_decode_attn_noalloc against lvq_decode_attn (MI355X).

The allocation-free entry point runs the same kernels with the library's
static device workspace instead of the caller's.  Its output must equal the
workspace entry point's (same plan, same kernels, merge in slot order: the
same bits) and stay within the oracle's 2e-3 row bar, on two calls in a row
with the second smaller, in each merge mode and with one workgroup per
(b, h) beyond the static workspace's head limit.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
from cases import DeviceCache, make_cache, oracle_decode, rel_err_rows

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.fixture(scope="module")
def lv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sub_bit_vq_amd import loopvq
    loopvq.library()
    return loopvq


def _note(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def _noalloc(lv, dc, t, cfg=None):
    cfg = cfg or dc.cfg
    out = torch.full_like(dc.out, float("nan"))
    lv.lvq_decode_attn_noalloc(cfg, t, dc.q[t].contiguous(), dc.ctx, max(dc.c.lengths),
                               dc.k_index, dc.v_index, dc.k_cb, dc.v_cb, dc.k_win, dc.v_win, out,
                               vq_len=dc.vq)
    torch.cuda.synchronize()
    return out.double().cpu().numpy()


def _pair(lv, dc, t):
    """noalloc output, workspace output, oracle rel err of the noalloc one"""
    got = _noalloc(lv, dc, t)
    ref_ws = dc.decode(t)
    err = rel_err_rows(got, oracle_decode(oracle, dc.c, t))
    return got, ref_ws, err


CASES = {
    # name: (first cache, second (smaller) cache, forced splits)
    "window merge": (dict(batch=1, n_heads=16, head_dim=128, group=16, lengths=(16384,), seed=81),
                     dict(batch=1, n_heads=4, head_dim=128, group=16, lengths=(3000,), seed=82), 0),
    "ticket merge": (dict(batch=3, n_heads=4, head_dim=64, group=16, lengths=(4000, 900, 2500),
                          seed=83),
                     dict(batch=2, n_heads=2, head_dim=64, group=16, lengths=(2000, 700), seed=84),
                     50),
    "0.25 bit": (dict(batch=2, n_heads=8, head_dim=128, group=32, lengths=(9000, 5000), seed=85),
                 dict(batch=1, n_heads=2, head_dim=128, group=32, lengths=(1500,), seed=86), 0),
    "head pairs": (dict(batch=1, n_heads=4, q_heads=16, head_dim=128, group=16, lengths=(12000,), seed=89),
                   dict(batch=2, n_heads=2, q_heads=4, head_dim=128, group=16, lengths=(3000, 900), seed=90),
                   0),
    "one workgroup per head, 512 heads": (
        dict(batch=64, n_heads=8, head_dim=64, group=16,
             lengths=tuple(300 + 37 * i for i in range(64)), seed=87),
        dict(batch=32, n_heads=8, head_dim=64, group=16,
             lengths=tuple(200 + 29 * i for i in range(32)), seed=88), 1),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_noalloc_matches_workspace_entry(lv, name):
    first, second, splits = CASES[name]
    for which, kw in (("first", first), ("second, smaller", second)):
        _note(f"{name}: {which} call")
        c = make_cache(codeword_tokens=True, **kw)
        dc = DeviceCache(lv, c, decode_splits=splits)
        merges = lv.lvq_decode_splits(dc.cfg, max(c.lengths)) > 1
        assert merges == (name != "one workgroup per head, 512 heads")
        for t in (0, 3):
            got, ref_ws, err = _pair(lv, dc, t)
            assert np.isfinite(got).all()
            assert np.array_equal(got, ref_ws), (name, which, t)
            assert err <= TOL, (name, which, t, err)


def test_noalloc_rejects_merging_beyond_limit(lv):
    """A merging plan over more than 256 (b, h) pairs does not fit the static
    workspace: rejected before any launch, the output untouched."""
    c = make_cache(batch=20, n_heads=16, head_dim=64, group=16,
                   lengths=tuple([1200] * 20), seed=89, codeword_tokens=True)
    dc = DeviceCache(lv, c, decode_splits=2)
    assert lv.lvq_decode_splits(dc.cfg, 1200) == 2
    out = torch.full_like(dc.out, 7.0)
    with pytest.raises(lv.LoopVQError) as e:
        lv.lvq_decode_attn_noalloc(dc.cfg, 0, dc.q[0].contiguous(), dc.ctx, 1200, dc.k_index,
                                   dc.v_index, dc.k_cb, dc.v_cb, dc.k_win, dc.v_win, out)
    assert e.value.status == lv.LVQ_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    # the same cache with the library's plan (one workgroup per (b, h)) runs
    dc1 = DeviceCache(lv, c)
    assert lv.lvq_decode_splits(dc1.cfg, 1200) == 1
    got = _noalloc(lv, dc1, 1)
    assert np.array_equal(got, dc1.decode(1))
    assert rel_err_rows(got, oracle_decode(oracle, c, 1)) <= TOL

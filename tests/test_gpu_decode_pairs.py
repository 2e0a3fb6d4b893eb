"""GPU parity of the head-pair decode (grouped-query attention: one workgroup
serves two consecutive query heads of a KV head and reads each index row and
window row once for both) against the CPU oracle, against the one-head
kernel, across plans, repeats and the workspace's epoch wrap.
Bar: as in test_gpu_decode.py, max_ch |gpu - oracle| / max_ch |oracle| <= 2e-3
per (b, h) row; between the two kernels, the weight-rounding bound.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
from cases import DeviceCache, make_cache, oracle_decode, rel_err_rows, weight_rounding_bound

pytestmark = pytest.mark.gpu
TOL = 2e-3
EPOCH_WRAP = 0xFFFFFFFF


@pytest.fixture(scope="module")
def lv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sub_bit_vq_amd import loopvq
    loopvq.library()
    return loopvq


def _note(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def _check(dc, t, cfg=None):
    got = dc.decode(t, cfg=cfg)
    ref = oracle_decode(oracle, dc.c, t)
    err = rel_err_rows(got, ref)
    assert np.isfinite(got).all()
    assert err <= TOL, f"loop step {t}: rel err {err:.3e}"
    return got, ref


LENGTHS = (1, 40, 64, 320, 321, 700, 2500, 5000)


@pytest.mark.parametrize("q_heads,kv_heads", [(4, 2), (8, 2), (16, 8), (2, 1)])
def test_pairs_match_oracle(lv, q_heads, kv_heads):
    """Ragged batch (no VQ tokens, window only, several splits, a ragged
    tail), 2 and 4 query heads per KV head, every second loop step."""
    _note(f"pairs {q_heads}q/{kv_heads}kv")
    c = make_cache(batch=len(LENGTHS), n_heads=kv_heads, q_heads=q_heads, head_dim=128, group=16,
                   lengths=LENGTHS, seed=900 + q_heads + kv_heads, codeword_tokens=True)
    dc = DeviceCache(lv, c)
    assert lv.lvq_decode_heads_per_workgroup(dc.cfg, 1, max(LENGTHS)) == 2
    for t in (0, 2, 3):
        _check(dc, t)


@pytest.mark.parametrize("splits,wgroups", [(1, 0), (2, 0), (3, 1), (5, 3), (9, 4), (16, 1), (20, 2)])
def test_pair_plans(lv, splits, wgroups):
    """Forced plans (one workgroup per pair, and 1..4 window workgroups):
    every one matches the oracle."""
    _note(f"pair plan {splits} splits, {wgroups} window groups")
    lengths = (5000, 321, 2600)
    c = make_cache(batch=len(lengths), n_heads=2, q_heads=8, head_dim=128, group=16, lengths=lengths,
                   seed=930 + splits, codeword_tokens=True)
    dc = DeviceCache(lv, c, decode_splits=splits, decode_window_groups=wgroups)
    assert lv.lvq_decode_heads_per_workgroup(dc.cfg, 1, max(lengths)) == 2
    assert lv.lvq_decode_splits(dc.cfg, max(lengths)) == splits
    for t in (1, 3):
        _check(dc, t)


def test_pairs_against_one_head(lv):
    """The pair kernel and the one-head kernel on one cache: both match the
    oracle, and each other within the weight-rounding bound (they split the
    tokens differently)."""
    _note("pairs against one head per workgroup")
    lengths = (3000, 700)
    c = make_cache(batch=2, n_heads=2, q_heads=8, head_dim=128, group=16, lengths=lengths, seed=951,
                   codeword_tokens=True)
    dc = DeviceCache(lv, c)
    one = dataclasses.replace(dc.cfg, decode_heads_per_group=1)
    two = dataclasses.replace(dc.cfg, decode_heads_per_group=2)
    assert lv.lvq_decode_heads_per_workgroup(one, 1, 3000) == 1
    assert lv.lvq_decode_heads_per_workgroup(two, 1, 3000) == 2
    for t in (0, 3):
        a, ref = _check(dc, t, cfg=one)
        b, _ = _check(dc, t, cfg=two)
        bound = weight_rounding_bound(c, t, ref)
        assert (np.abs(a - b) <= bound).all(), float(np.max(np.abs(a - b) - bound))


def test_pair_not_possible_is_refused(lv):
    """decode_heads_per_group = 2 where the kernel has no pair variant (odd
    query heads per KV head, or head_dim 64) returns LVQ_ERR_UNSUPPORTED."""
    for q, kv, d in ((6, 2, 128), (4, 2, 64)):
        c = make_cache(batch=1, n_heads=kv, q_heads=q, head_dim=d, group=16, lengths=(800,), seed=960,
                       codeword_tokens=True)
        dc = DeviceCache(lv, c, decode_heads_per_group=2)
        assert lv.lvq_decode_heads_per_workgroup(dc.cfg, 1, 800) == 0
        with pytest.raises(lv.LoopVQError) as e:
            dc.decode(0)
        assert e.value.status == lv.LVQ_ERR_UNSUPPORTED


def test_pair_repeats_and_epoch_wrap(lv):
    """Repeated calls give identical bits, and with every block at the last
    epoch before the wrap two calls in a row (different loop steps) are both
    right, each head's block advancing 2^32 - 2 -> 0 -> 1."""
    _note("pairs: repeats and epoch wrap")
    c = make_cache(batch=2, n_heads=2, q_heads=4, head_dim=128, group=16, lengths=(2600, 900), seed=971,
                   codeword_tokens=True)
    dc = DeviceCache(lv, c, decode_splits=6)
    assert lv.lvq_decode_heads_per_workgroup(dc.cfg, 1, 2600) == 2
    first, _ = _check(dc, 1)
    for _ in range(3):
        assert np.array_equal(dc.decode(1), first)
    n = dc.cfg.batch * dc.cfg.n_heads
    hdr = lv.WORKSPACE_HEADER_BYTES
    per = (lv.lvq_cache_layout(dc.cfg)["workspace_bytes"] - hdr) // n
    offs = [hdr + i * per for i in range(n)]
    val = torch.from_numpy(np.array([(EPOCH_WRAP - 1) << 32], np.uint64).view(np.uint8)).to(dc.ws.device)
    for off in offs:
        dc.ws[off:off + 8] = val
    torch.cuda.synchronize()
    for t, want in ((0, 0), (1, 1)):
        _check(dc, t)
        host = dc.ws.cpu().numpy()
        assert all(int(host[o:o + 8].view(np.uint64)[0]) == want << 32 for o in offs), t


def test_pair_page_lag_vq_len(lv):
    """vq_len above the exact-window count (the recent ring holds fewer than
    256 tokens, some of its slots stale), with head pairs."""
    _note("pairs: page lag")
    lengths = (700, 1000, 3333)
    vq = [L - 320 + e for L, e in zip(lengths, (8, 5, 255))]
    c = make_cache(batch=3, n_heads=2, q_heads=4, head_dim=128, group=16, lengths=lengths, seed=981,
                   codeword_tokens=True, vq_len=vq)
    dc = DeviceCache(lv, c)
    assert lv.lvq_decode_heads_per_workgroup(dc.cfg, 1, max(lengths)) == 2
    for t in (0, 2):
        _check(dc, t)


def test_pair_small_windows(lv):
    """Window ranges that are empty or a single slot, with head pairs (the
    merger's own range may be empty)."""
    for n_sink, n_recent, splits, w in ((2, 3, 6, 4), (0, 1, 5, 3), (1, 2, 3, 2)):
        _note(f"pairs: small windows {n_sink}+{n_recent}, {splits} splits, {w} window groups")
        c = make_cache(batch=2, n_heads=1, q_heads=2, head_dim=128, group=16, lengths=(1800, 900),
                       seed=991 + w, codeword_tokens=True, n_sink=n_sink, n_recent=n_recent)
        dc = DeviceCache(lv, c, decode_splits=splits, decode_window_groups=w)
        assert lv.lvq_decode_heads_per_workgroup(dc.cfg, 1, 1800) == 2
        for t in (1, 3):
            _check(dc, t)


def test_pair_merge_timeout_is_flagged(lv):
    """A merger bounded to one poll gives up on both heads: both rows NaN,
    the status word flagged; after clearing, the default bound is right."""
    _note("pairs: merge timeout")
    c = make_cache(batch=1, n_heads=1, q_heads=2, head_dim=128, group=16, lengths=(32768,), seed=995,
                   codeword_tokens=True)
    dc = DeviceCache(lv, c, decode_splits=3)
    assert lv.lvq_decode_heads_per_workgroup(dc.cfg, 1, 32768) == 2
    got = dc.decode(2, cfg=dataclasses.replace(dc.cfg, decode_poll_limit=1))
    flags = lv.lvq_decode_status(dc.ws, clear=True)
    assert np.isnan(got).all()
    assert flags == lv.LVQ_STATUS_MERGE_TIMEOUT
    dc.ws.zero_()
    _check(dc, 2)
    assert lv.lvq_decode_status(dc.ws) == 0

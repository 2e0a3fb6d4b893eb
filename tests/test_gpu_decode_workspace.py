"""GPU checks of the decode workspace and the split merge (MI355X).

The workspace is a status word and a fixed grid of per-(layer, b, h) blocks;
each block counts its calls in a 32-bit epoch and tags split partials with
it.  These tests drive the cases the epoch and the grid exist for: an epoch
that wraps, a workspace shared by calls of different batch sizes, a merge
that gives up waiting (forced from the host with a one-poll bound), value
codebook entries outside fp16's range, and repeated calls (bit-identical:
the merge adds the split partials in slot order whichever workgroup merges).
Every output is checked against the CPU oracle (2e-3 row bar).
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
EPOCH_WRAP = 0xFFFFFFFF          # epochs run 0 .. 2^32 - 2


@pytest.fixture(scope="module")
def lv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sub_bit_vq_amd import loopvq
    loopvq.library()
    return loopvq


def _note(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def _arrival_offsets(lv, dc):
    """byte offsets of the arrival words of the call's (b, h) blocks (the
    header, then one fixed-size block per (b, h); the word opens a block)"""
    n = dc.cfg.batch * dc.cfg.n_heads
    hdr = lv.WORKSPACE_HEADER_BYTES
    per = (lv.lvq_cache_layout(dc.cfg)["workspace_bytes"] - hdr) // n
    return [hdr + i * per for i in range(n)]


def _set_epochs(lv, dc, epoch):
    val = torch.from_numpy(np.array([epoch << 32], np.uint64).view(np.uint8)).to(dc.ws.device)
    for off in _arrival_offsets(lv, dc):
        dc.ws[off:off + 8] = val
    torch.cuda.synchronize()


def _epochs(lv, dc):
    host = dc.ws.cpu().numpy()
    return [int(host[off:off + 8].view(np.uint64)[0]) for off in _arrival_offsets(lv, dc)]


@pytest.mark.parametrize("mode", ["window", "ticket"])
def test_epoch_wrap(lv, mode):
    """Blocks at the last epoch before the wrap: two calls in a row (loop
    steps 0 then 1, so the first call's partials are stale and different
    when the second looks for its own) are both correct, and the epoch
    advances 2^32 - 2 -> 0 -> 1.  'window' merges by a window workgroup,
    'ticket' (more than 256 workgroups) by the last to arrive."""
    _note(f"epoch wrap, {mode} merge")
    c = make_cache(batch=3, n_heads=2, head_dim=64, group=16, lengths=(2500, 900, 1600),
                   seed=71, codeword_tokens=True)
    splits = 6 if mode == "window" else 50          # 6 * 6 <= 256 < 50 * 6
    dc = DeviceCache(lv, c, decode_splits=splits)
    assert (lv.lvq_decode_window_groups(dc.cfg, 2500) > 0) == (mode == "window")
    _set_epochs(lv, dc, EPOCH_WRAP - 1)
    for t, want in ((0, 0), (1, 1)):
        got = dc.decode(t)
        err = rel_err_rows(got, oracle_decode(oracle, c, t))
        _note(f"  t={t} rel err {err:.2e}")
        assert err <= TOL, t
        assert all(e == want << 32 for e in _epochs(lv, dc)), (t, _epochs(lv, dc))


def test_workspace_across_batch_sizes(lv):
    """One workspace (sized for batch 64) serves batch 64, then batch 32, then
    64 again, with a merge in every call: each batch's blocks keep their
    places, so every row is right."""
    rng = np.random.default_rng(5)
    big = make_cache(batch=64, n_heads=4, head_dim=64, group=16,
                     lengths=tuple(int(x) for x in rng.integers(400, 1500, 64)), seed=72,
                     codeword_tokens=True, t_max=1500)
    small = make_cache(batch=32, n_heads=4, head_dim=64, group=16,
                       lengths=tuple(int(x) for x in rng.integers(400, 1500, 32)), seed=73,
                       codeword_tokens=True, t_max=1500)
    d64 = DeviceCache(lv, big, decode_splits=2)
    d32 = DeviceCache(lv, small, decode_splits=2)
    d32.ws = d64.ws                                  # shared
    for name, dc, t in (("64", d64, 0), ("32", d32, 1), ("64", d64, 2), ("32", d32, 3)):
        _note(f"batch {name}, loop step {t}")
        err = rel_err_rows(dc.decode(t), oracle_decode(oracle, dc.c, t))
        assert err <= TOL, (name, t, err)
    assert lv.lvq_decode_status(d64.ws) == 0


def test_merge_timeout_is_flagged(lv):
    """A merger bounded to one poll (decode_poll_limit = 1) gives up long
    before its peers' 16384-token chunks are done: its row is NaN and the
    status word says so.  After the workspace is cleared, the default bound
    gives correct rows and a clear status."""
    _note("merge timeout")
    c = make_cache(batch=1, n_heads=2, head_dim=128, group=16, lengths=(32768,), seed=74,
                   codeword_tokens=True)
    dc = DeviceCache(lv, c, decode_splits=3)         # 2 VQ chunks + 1 window workgroup
    assert lv.lvq_decode_window_groups(dc.cfg, 32768) == 1
    ref = oracle_decode(oracle, c, 2)
    got = dc.decode(2, cfg=dataclasses.replace(dc.cfg, decode_poll_limit=1))
    nan_rows = np.isnan(got).any(axis=-1)
    flags = lv.lvq_decode_status(dc.ws, clear=True)
    _note(f"  rows NaN {int(nan_rows.sum())} of {nan_rows.size}, status {flags}")
    assert nan_rows.all() and np.isnan(got).all()
    assert flags == lv.LVQ_STATUS_MERGE_TIMEOUT
    assert lv.lvq_decode_status(dc.ws) == 0
    dc.ws.zero_()
    got = dc.decode(2)
    assert rel_err_rows(got, ref) <= TOL
    assert lv.lvq_decode_status(dc.ws) == 0


@pytest.mark.parametrize("splits", [0, 40, 1])
def test_value_range_is_flagged(lv, splits):
    """A bf16 value codebook entry of 2^17 in slice 1 (beyond fp16): a decode
    of loop step 1 flags it; decodes of other steps (which read other
    slices) do not.  The VQ workgroups of a head share the check of the
    slice they stage (role s of n checks the staged units u = s mod
    min(n, 8)); the plans cover the library's (VQ splits beside window
    workgroups), 40 splits (arrival tickets) and one workgroup per (b, h)
    (it checks everything it stages)."""
    _note(f"value range flag, splits {splits}")
    c = make_cache(batch=1, n_heads=8, head_dim=128, group=16, lengths=(3000,), seed=75,
                   codeword_tokens=True)
    dc = DeviceCache(lv, c, decode_splits=splits)
    wg = lv.lvq_decode_window_groups(dc.cfg, 3000)
    assert (wg > 0) == (splits == 0)
    for t in range(4):
        dc.decode(t)
        assert lv.lvq_decode_status(dc.ws, clear=True) == 0, t
    for code, sub in ((200, 17), (0, 0), (255, 31)):
        dc.v_cb[1, 5, code, sub, 2] = 2.0 ** 17
        for t in (0, 2, 3):
            dc.decode(t)
            assert lv.lvq_decode_status(dc.ws, clear=True) == 0, (code, sub, t)
        dc.decode(1)
        assert lv.lvq_decode_status(dc.ws, clear=True) == lv.LVQ_STATUS_VALUE_RANGE, (code, sub)
        dc.v_cb[1, 5, code, sub, 2] = -2.0 ** 16
        dc.decode(1)
        assert lv.lvq_decode_status(dc.ws, clear=True) == lv.LVQ_STATUS_VALUE_RANGE, (code, sub)
        dc.v_cb[1, 5, code, sub, 2] = 65280.0          # the largest bf16 below 2^16: in range
        dc.decode(1)
        assert lv.lvq_decode_status(dc.ws, clear=True) == 0, (code, sub)
    # in range, the flag-free decode is still right
    assert rel_err_rows(dc.decode(1), oracle_decode(oracle, _with_codebooks(c, dc), 1)) <= TOL


def _with_codebooks(c, dc):
    """the cache with the device's (edited) codebooks"""
    import copy
    c2 = copy.copy(c)
    c2.k_codebook, c2.v_codebook = dc.k_cb.cpu(), dc.v_cb.cpu()
    return c2


@pytest.mark.parametrize("splits", [0, 6, 50])
def test_repeats_are_bit_identical(lv, splits):
    """Repeated calls on one workspace give identical bits, in every merge
    mode (library plan, forced window workgroups, forced arrival tickets)."""
    _note(f"repeat, splits {splits}")
    c = make_cache(batch=3, n_heads=2, head_dim=64, group=16, lengths=(3000, 900, 2000),
                   seed=76, codeword_tokens=True)
    dc = DeviceCache(lv, c, decode_splits=splits)
    first = dc.decode(1)
    assert rel_err_rows(first, oracle_decode(oracle, c, 1)) <= TOL
    for _ in range(4):
        assert np.array_equal(dc.decode(1), first)

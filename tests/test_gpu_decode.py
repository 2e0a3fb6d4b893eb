"""GPU parity of lvq_decode_attn against the CPU oracle (MI355X).

Bar: per (b, h) row, max_ch |gpu - oracle| / max_ch |oracle| <= 2e-3 (fp32
accumulation on the GPU, fp64 in the oracle).  Inputs are seeded; index
caches are drawn, or encoded by the oracle -- never by the HIP encoder.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
from cases import (DeviceCache, make_cache, merge_loop_groups, oracle_decode, oracle_encoder,
                   rel_err_rows, weight_rounding_bound)
from sub_bit_vq_amd import synth

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


def _check(dc, t, sm_scale=1.0, heads=None, tol=TOL):
    got = dc.decode(t, sm_scale)
    ref = oracle_decode(oracle, dc.c, t, sm_scale, heads=heads)
    if heads is not None:
        got, ref = got[:, heads[0]:heads[1]], ref[:, heads[0]:heads[1]]
    err = rel_err_rows(got, ref)
    assert np.isfinite(got).all()
    assert err <= tol, f"loop step {t}: rel err {err:.3e}"
    return got, err


def test_tiny_workload_every_loop_step(lv):
    """B1 H1 d64 Tc4 G16, fp32 codebooks, 512-token context (middle 192 tokens
    VQ-coded), indices from the oracle encoder, all four loop steps."""
    _note("tiny workload")
    c = make_cache(batch=1, n_heads=1, head_dim=64, group=16, lengths=(512,),
                   cb_dtype=torch.float32, seed=1000,
                   encode=oracle_encoder(oracle, 1, 64, 4, 16))
    dc = DeviceCache(lv, c)
    for t in range(4):
        _check(dc, t)


SHAPES = [  # (head_dim, group, cb dtype)
    (64, 16, torch.bfloat16),
    (128, 16, torch.bfloat16),
    (128, 32, torch.bfloat16),
    (64, 32, torch.bfloat16),
    (64, 16, torch.float32),
    (128, 8, torch.bfloat16),
    (32, 16, torch.bfloat16),
    (64, 8, torch.float32),
]


@pytest.mark.parametrize("head_dim,group,cb_dtype", SHAPES)
def test_ragged_shapes(lv, head_dim, group, cb_dtype):
    """Ragged batch covering L <= 64, <= 320 and > 320, several splits and a
    ragged tail; VQ tokens are exact codewords of drawn indices."""
    _note(f"ragged d={head_dim} G={group} {cb_dtype}")
    lengths = (1, 40, 64, 200, 320, 321, 700, 2500, 5000)
    c = make_cache(batch=len(lengths), n_heads=2, head_dim=head_dim, group=group,
                   lengths=lengths, cb_dtype=cb_dtype, seed=head_dim + group,
                   codeword_tokens=True)
    dc = DeviceCache(lv, c)
    for t in (0, 3):
        _check(dc, t)


@pytest.mark.parametrize("q_heads,kv_heads,head_dim,group,cb_dtype", [
    (8, 2, 128, 16, torch.bfloat16),
    (6, 3, 64, 32, torch.bfloat16),
    (4, 1, 64, 16, torch.float32),
])
def test_grouped_query_heads(lv, q_heads, kv_heads, head_dim, group, cb_dtype):
    """Grouped-query attention: each query head attends over the index
    stream, codebooks and windows of its KV head (h // (Hq / Hk))."""
    _note(f"GQA {q_heads}q/{kv_heads}kv d={head_dim} G={group} {cb_dtype}")
    lengths = (40, 320, 900, 5000)
    c = make_cache(batch=len(lengths), n_heads=kv_heads, q_heads=q_heads, head_dim=head_dim,
                   group=group, lengths=lengths, cb_dtype=cb_dtype, seed=400 + q_heads,
                   codeword_tokens=True)
    dc = DeviceCache(lv, c)
    for t in (0, 1, 3):
        _check(dc, t)


@pytest.mark.parametrize("groups,q_heads", [(2, 0), (3, 4)])
def test_loop_groups(lv, groups, q_heads):
    """A model with R = groups * 4 loop steps (one index row per group of 4
    steps): every loop step r reads the rows of group r // 4, codebook slice r
    and window step r; also under grouped-query attention."""
    _note(f"loop groups {groups} q_heads={q_heads}")
    lengths = (100, 800, 3000)
    parts = [make_cache(batch=3, n_heads=2, q_heads=q_heads or None, head_dim=128, group=16,
                        lengths=lengths, seed=600 + 17 * g, codeword_tokens=True)
             for g in range(groups)]
    c = merge_loop_groups(parts)
    dc = DeviceCache(lv, c)
    for r in range(4 * groups):
        _check(dc, r)


def test_loop_correlated_encoded_cache(lv):
    """Realistic (skewed) code histogram: loop-correlated K/V encoded by the
    oracle, 0.5-bit, 4 heads, 3000-token context."""
    _note("oracle-encoded cache")
    c = make_cache(batch=2, n_heads=4, head_dim=128, group=16, lengths=(3000, 1500), seed=7,
                   encode=oracle_encoder(oracle, 4, 128, 4, 16))
    dc = DeviceCache(lv, c)
    for t in range(4):
        _check(dc, t)


def test_split_count_invariance(lv):
    _note("split invariance")
    c = make_cache(batch=2, n_heads=2, head_dim=128, group=16, lengths=(9000, 4000), seed=11,
                   codeword_tokens=True)
    dc = DeviceCache(lv, c)
    ref = oracle_decode(oracle, c, 1)
    outs = []
    for splits in (1, 2, 5, 17, 64):
        cfg = dataclasses.replace(dc.cfg, decode_splits=splits)
        got = dc.decode(1, cfg=cfg)
        assert rel_err_rows(got, ref) <= TOL, splits
        outs.append(got)
    # split counts change each wave's running max and hence the fp16 rounding
    # of the token weights (2^-11 relative): the outputs may differ by the
    # bound that rounding implies (a dropped or doubled split would move the
    # output by ~1/splits)
    bound = weight_rounding_bound(c, 1, ref)
    for o in outs[1:]:
        assert (np.abs(o - outs[0]) <= bound).all()
        _note(f"  largest difference / bound: {float((np.abs(o - outs[0]) / bound).max()):.3f}")


def test_window_group_counts(lv):
    """The bf16 window slots split over 1..4 window workgroups (forced plans
    and the library's own for short and long contexts, 0.5 and 0.25 bit):
    every plan against the oracle and against the others.  320 slots split
    into 80/107/160-slot ranges, so the ranges' ends fall inside the sink
    window, the recent ring and passes of each wave."""
    for G, lengths in ((16, (2048, 700)), (32, (5000, 1500))):
        _note(f"window groups G={G}")
        c = make_cache(batch=2, n_heads=2, head_dim=128, group=G, lengths=lengths, seed=21 + G,
                       codeword_tokens=True)
        dc = DeviceCache(lv, c)
        for t in (0, 3):
            ref = oracle_decode(oracle, c, t)
            base = dc.decode(t)
            assert rel_err_rows(base, ref) <= TOL, (G, t)
            bound = weight_rounding_bound(c, t, ref)
            for splits, w in ((2, 1), (5, 2), (5, 3), (6, 4), (9, 4)):
                cfg = dataclasses.replace(dc.cfg, decode_splits=splits, decode_window_groups=w)
                got = dc.decode(t, cfg=cfg)
                assert rel_err_rows(got, ref) <= TOL, (G, t, splits, w)
                assert (np.abs(got - base) <= bound).all(), (G, t, splits, w)


def test_window_groups_small_windows(lv):
    """Window ranges that are empty or a single slot: 5 window slots (2 sink,
    3 recent) over 4 window workgroups, and 1 slot over 3; the merger's own
    range may be empty."""
    for n_sink, n_recent, splits, w in ((2, 3, 6, 4), (0, 1, 5, 3), (1, 2, 3, 2)):
        _note(f"small windows {n_sink}+{n_recent}, {splits} splits, {w} window groups")
        c = make_cache(batch=2, n_heads=2, head_dim=64, group=16, lengths=(1800, 900), seed=51 + w,
                       codeword_tokens=True, n_sink=n_sink, n_recent=n_recent)
        dc = DeviceCache(lv, c)
        cfg = dataclasses.replace(dc.cfg, decode_splits=splits, decode_window_groups=w)
        for t in (1, 3):
            assert rel_err_rows(dc.decode(t, cfg=cfg), oracle_decode(oracle, c, t)) <= TOL, (n_sink, n_recent, t)


def test_longest_first_order(lv):
    """One workgroup per (b, h) (forced single split): workgroups take the
    sequences longest first, ranked by (length, index), including ties and
    window-only sequences.  Every row against the oracle, so a wrong or
    repeated rank shows as a wrong row."""
    _note("longest-first order")
    c = make_cache(batch=7, n_heads=3, head_dim=64, group=16,
                   lengths=(700, 3000, 700, 1500, 3000, 64, 2200), seed=41, codeword_tokens=True)
    dc = DeviceCache(lv, c)
    cfg = dataclasses.replace(dc.cfg, decode_splits=1)
    for t in (0, 2):
        ref = oracle_decode(oracle, c, t)
        got = dc.decode(t, cfg=cfg)
        assert rel_err_rows(got, ref) <= TOL, t
        assert (np.abs(got - dc.decode(t)) <= weight_rounding_bound(c, t, ref)).all(), t


@pytest.mark.parametrize("batch", [256, 257])
def test_longest_first_order_limit(lv, batch):
    """256 sequences (the largest batch ranked by length) and 257 (dispatch
    order), one workgroup per (b, h): ragged short contexts, every row
    against the oracle."""
    _note(f"longest-first limit, batch {batch}")
    rng = np.random.default_rng(batch)
    lengths = tuple(int(x) for x in rng.integers(1, 1500, size=batch))
    c = make_cache(batch=batch, n_heads=1, head_dim=64, group=16, lengths=lengths, seed=61,
                   codeword_tokens=True)
    dc = DeviceCache(lv, c)
    assert lv.lvq_decode_splits(dc.cfg, max(lengths)) == 1
    ref = oracle_decode(oracle, c, 1)
    assert rel_err_rows(dc.decode(1), ref) <= TOL


def test_token_permutation_invariance(lv):
    """Permuting the VQ tokens (their K and V index rows together) changes
    only the rounding."""
    _note("token permutation")
    c = make_cache(batch=1, n_heads=2, head_dim=64, group=16, lengths=(4000,), seed=12,
                   codeword_tokens=True)
    dc = DeviceCache(lv, c)
    base = dc.decode(2)
    bound = weight_rounding_bound(c, 2, oracle_decode(oracle, c, 2))
    lo, hi = c.vq_range(0).start, c.vq_range(0).stop
    perm = torch.randperm(hi - lo, generator=torch.Generator().manual_seed(3)) + lo
    dc.k_index[0, :, lo:hi] = dc.k_index[0, :, perm.cuda()]
    dc.v_index[0, :, lo:hi] = dc.v_index[0, :, perm.cuda()]
    assert (np.abs(dc.decode(2) - base) <= bound).all()


def test_slice_isolation_nan(lv):
    """NaN in codebook slices t' != t must not reach the step-t output."""
    _note("slice isolation")
    c = make_cache(batch=1, n_heads=2, head_dim=128, group=16, lengths=(2000,), seed=13,
                   codeword_tokens=True)
    dc = DeviceCache(lv, c)
    for t in range(4):
        clean = oracle_decode(oracle, c, t)
        kcb, vcb = dc.k_cb.clone(), dc.v_cb.clone()
        for tp in range(4):
            if tp != t:
                dc.k_cb[tp] = float("nan")
                dc.v_cb[tp] = float("nan")
        got = dc.decode(t)
        dc.k_cb.copy_(kcb)
        dc.v_cb.copy_(vcb)
        assert np.isfinite(got).all()
        assert rel_err_rows(got, clean) <= TOL


def test_page_lag_vq_len(lv):
    """vq_len above the exact-window count: the recent ring holds fewer than
    256 tokens and some of its slots are stale."""
    _note("page lag")
    lengths = (700, 1000, 3333)
    vq = [L - 320 + e for L, e in zip(lengths, (8, 5, 255))]
    c = make_cache(batch=3, n_heads=2, head_dim=64, group=16, lengths=lengths, seed=14,
                   codeword_tokens=True, vq_len=vq)
    dc = DeviceCache(lv, c)
    for t in (0, 2):
        _check(dc, t)


def test_sm_scale(lv):
    _note("sm_scale")
    c = make_cache(batch=1, n_heads=2, head_dim=128, group=16, lengths=(1500,), seed=15,
                   codeword_tokens=True)
    dc = DeviceCache(lv, c)
    _check(dc, 1, sm_scale=0.3)
    _check(dc, 1, sm_scale=1.0 / np.sqrt(128))   # 1/sqrt(d) applied a second time


def test_empty_context_and_repeat(lv):
    """L = 0 gives zeros; repeated calls on one workspace give identical bits
    (the blocks' epochs advance themselves, and the merge adds the split
    partials in slot order whichever workgroup merges)."""
    _note("empty + repeat")
    c = make_cache(batch=3, n_heads=2, head_dim=64, group=16, lengths=(1, 900, 1), seed=16,
                   codeword_tokens=True)
    c.lengths[0] = 0
    dc = DeviceCache(lv, c)
    a = dc.decode(0)
    assert np.all(a[0] == 0.0)
    ref = oracle_decode(oracle, c, 0)
    assert rel_err_rows(a, ref) <= TOL
    for _ in range(3):
        r = dc.decode(0)
        assert np.all(r[0] == 0.0)
        assert np.array_equal(r, a)
    b = dc.decode(3)
    assert rel_err_rows(b, oracle_decode(oracle, c, 3)) <= TOL


def test_max_ctx_len_bound(lv):
    """max_ctx_len larger than every L (it only sizes the launch)."""
    _note("max_ctx bound")
    c = make_cache(batch=2, n_heads=1, head_dim=64, group=16, lengths=(1000, 400), seed=17,
                   codeword_tokens=True, t_max=6000)
    dc = DeviceCache(lv, c)
    lv.lvq_decode_attn(dc.cfg, 1, dc.q[1].contiguous(), dc.ctx, 6000, dc.k_index, dc.v_index,
                       dc.k_cb, dc.v_cb, dc.k_win, dc.v_win, dc.ws, dc.out)
    torch.cuda.synchronize()
    got = dc.out.double().cpu().numpy()
    assert rel_err_rows(got, oracle_decode(oracle, c, 1)) <= TOL


# --- full-size grouped-query workload -----------------------------------------

def _full_size_cache(lv, H, d, G, lengths, seed, device="cuda", Hq=None):
    """Device-resident cache at full size (H KV heads, Hq query heads):
    windows from the loop-correlated generator, VQ indices drawn uniformly
    (drawn, so the oracle can take them as input)."""
    B = len(lengths)
    Tc = 4
    cg = G // Tc
    S = d // cg
    T = max(lengths)
    Hq = Hq or H
    cfg = lv.Config(batch=B, n_heads=Hq, head_dim=d, group=G, max_tokens=T,
                    n_kv_heads=H if Hq != H else 0)
    bufs = lv.allocate(cfg, device)
    kcb = synth.codebooks(H, d, Tc, G, seed + 1, device=device)
    vcb = synth.codebooks(H, d, Tc, G, seed + 2, device=device)
    q = synth.queries(B, Hq, d, Tc, seed + 3, device=device)
    for b, L in enumerate(lengths):
        ki = synth.random_indices((H, L, S), seed + 10 + 2 * b, device=device)
        vi = synth.random_indices((H, L, S), seed + 11 + 2 * b, device=device)
        bufs["k_index"][b, :, :L] = ki
        bufs["v_index"][b, :, :L] = vi
        # only the window tokens are needed in bf16
        sink, _, recent = synth.window_positions(L, 64, 256)
        win = list(sink) + list(recent)
        kt = synth.loop_correlated_kv(len(win), H, Tc, d, seed + 20 + 2 * b, device=device)
        vt = synth.loop_correlated_kv(len(win), H, Tc, d, seed + 21 + 2 * b, device=device)
        slots = torch.tensor([synth.window_slot(p, 64, 256) for p in win], device=device)
        bufs["k_window"][b][:, :, slots, :] = kt.permute(2, 1, 0, 3)
        bufs["v_window"][b][:, :, slots, :] = vt.permute(2, 1, 0, 3)
    ctx = torch.tensor(lengths, dtype=torch.int32, device=device)
    return cfg, bufs, kcb, vcb, q, ctx


def test_full_32k_gqa(lv):
    """32 query heads over 8 KV heads, one 32768-token sequence, 0.5 bit:
    every query head at every loop step against the oracle, in the launch
    configuration the benchmark's GQA workload times."""
    _note("32K GQA 32q/8kv")
    cfg, bufs, kcb, vcb, q, ctx = _full_size_cache(lv, 8, 128, 16, [32768], seed=500, Hq=32)
    for t in range(4):
        lv.lvq_decode_attn(cfg, t, q[t].contiguous(), ctx, 32768, bufs["k_index"],
                           bufs["v_index"], kcb, vcb, bufs["k_window"], bufs["v_window"],
                           bufs["workspace"], bufs["out"])
        torch.cuda.synchronize()
        got = bufs["out"].double().cpu().numpy()
        ref = oracle.decode_attn(loop_step=t, q=q[t].cpu(), ctx_len=[32768],
                                 k_index=bufs["k_index"].cpu(), v_index=bufs["v_index"].cpu(),
                                 k_codebook=kcb.cpu(), v_codebook=vcb.cpu(),
                                 k_window=bufs["k_window"].cpu(), v_window=bufs["v_window"].cpu(),
                                 n_sink=64, n_recent=256, group=16)
        err = rel_err_rows(got, ref)
        _note(f"  t={t} rel err {err:.2e}")
        assert err <= TOL

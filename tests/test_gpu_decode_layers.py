"""GPU parity of lvq_decode_attn_layers (several layers' caches attended in
one launch) against the CPU oracle, layer by layer (MI355X).

Each layer is an independent decode with its own query, caches, codebooks
and windows, sharing the sequence lengths and the loop step; the oracle is
the single-layer oracle applied to each.  Bar as for lvq_decode_attn: per
(b, h) row, max_ch |gpu - oracle| / max_ch |oracle| <= 2e-3.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from cases import DeviceCache, make_cache, oracle_decode, rel_err_rows, weight_rounding_bound
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


def _layers(lv, n, seed0=0, **kw):
    """n independently seeded caches of one shape and one set of lengths."""
    return [DeviceCache(lv, make_cache(seed=seed0 + 1000 * (i + 1), **kw)) for i in range(n)]


def _entries(dcs, t):
    return [dict(q=dc.q[t].contiguous(), k_index=dc.k_index, v_index=dc.v_index,
                 k_codebook=dc.k_cb, v_codebook=dc.v_cb, k_window=dc.k_win, v_window=dc.v_win,
                 out=dc.out) for dc in dcs]


def _workspace(lv, cfg, n):
    per = lv.lvq_cache_layout(cfg)["workspace_bytes"]
    return torch.zeros(n * per, dtype=torch.uint8, device="cuda")


def test_layers_match_oracle(lv):
    """3 layers, ragged batch (window-only and multi-split sequences), every
    loop step: each layer against the oracle and against its own
    single-layer call."""
    _note("3 layers, ragged")
    kw = dict(batch=5, n_heads=2, head_dim=128, group=16, lengths=(1, 40, 321, 2500, 5000),
              codeword_tokens=True)
    dcs = _layers(lv, 3, **kw)
    cfg = dcs[0].cfg
    ws = _workspace(lv, cfg, 3)
    for t in range(4):
        ents = _entries(dcs, t)
        lv.lvq_decode_attn_layers(cfg, t, ents, dcs[0].ctx, 5000, ws)
        torch.cuda.synchronize()
        got = [e["out"].double().cpu().numpy() for e in ents]
        for i, dc in enumerate(dcs):
            ref = oracle_decode(oracle, dc.c, t)
            err = rel_err_rows(got[i], ref)
            assert np.isfinite(got[i]).all()
            assert err <= TOL, f"layer {i} step {t}: rel err {err:.3e}"
            single = dc.decode(t)          # its own workspace and output buffer
            bound = weight_rounding_bound(dc.c, t, ref)
            assert (np.abs(got[i] - single) <= bound).all(), f"layer {i} step {t}"


def test_layers_beyond_one_launch(lv):
    """20 layers: more than one launch's 16; every layer against the oracle,
    twice in a row on the same workspace (the merge state carries over)."""
    _note("20 layers")
    kw = dict(batch=2, n_heads=2, head_dim=64, group=16, lengths=(700, 2000),
              codeword_tokens=True, seed0=7)
    dcs = _layers(lv, 20, **kw)
    cfg = dcs[0].cfg
    ws = _workspace(lv, cfg, 20)
    refs = [oracle_decode(oracle, dc.c, 2) for dc in dcs]
    for rep in range(2):
        for dc in dcs:
            dc.out.fill_(float("nan"))
        ents = _entries(dcs, 2)
        lv.lvq_decode_attn_layers(cfg, 2, ents, dcs[0].ctx, 2000, ws)
        torch.cuda.synchronize()
        for i, e in enumerate(ents):
            err = rel_err_rows(e["out"].double().cpu().numpy(), refs[i])
            assert err <= TOL, f"rep {rep} layer {i}: rel err {err:.3e}"


def test_layers_share_workspace_with_single_call(lv):
    """Layer 0 of a multi-layer call and lvq_decode_attn use the same
    workspace layout: alternating the two on one workspace stays correct."""
    _note("shared workspace")
    kw = dict(batch=1, n_heads=4, head_dim=128, group=32, lengths=(6000,),
              codeword_tokens=True, seed0=3)
    dcs = _layers(lv, 2, **kw)
    cfg = dcs[0].cfg
    ws = _workspace(lv, cfg, 2)
    dc0 = dcs[0]
    for t in (0, 1, 2, 3):
        ref0 = oracle_decode(oracle, dc0.c, t)
        lv.lvq_decode_attn(cfg, t, dc0.q[t].contiguous(), dc0.ctx, 6000, dc0.k_index,
                           dc0.v_index, dc0.k_cb, dc0.v_cb, dc0.k_win, dc0.v_win, ws, dc0.out)
        torch.cuda.synchronize()
        assert rel_err_rows(dc0.out.double().cpu().numpy(), ref0) <= TOL
        ents = _entries(dcs, t)
        lv.lvq_decode_attn_layers(cfg, t, ents, dc0.ctx, 6000, ws)
        torch.cuda.synchronize()
        for i, dc in enumerate(dcs):
            err = rel_err_rows(ents[i]["out"].double().cpu().numpy(), oracle_decode(oracle, dc.c, t))
            assert err <= TOL, f"step {t} layer {i}: rel err {err:.3e}"


def test_layers_full_32k(lv):
    """4 layers of the 32768-token, 16-head, 0.5-bit workload in the launch
    configuration the benchmark's multi-layer workload times: every head of
    every layer at loop step 1 against the oracle."""
    _note("4 layers x 32K")
    H, d, G, Tc, L = 16, 128, 16, 4, 32768
    S = d // (G // Tc)
    cfg = lv.Config(batch=1, n_heads=H, head_dim=d, group=G, max_tokens=L)
    ents = []
    for i in range(4):
        seed = 700 + 50 * i
        bufs = lv.allocate(cfg, "cuda")
        kcb = synth.codebooks(H, d, Tc, G, seed + 1, device="cuda")
        vcb = synth.codebooks(H, d, Tc, G, seed + 2, device="cuda")
        q = synth.queries(1, H, d, Tc, seed + 3, device="cuda")
        bufs["k_index"][0] = synth.random_indices((H, L, S), seed + 10, device="cuda")
        bufs["v_index"][0] = synth.random_indices((H, L, S), seed + 11, device="cuda")
        bufs["k_window"].normal_(generator=torch.Generator("cuda").manual_seed(seed + 20))
        bufs["v_window"].normal_(generator=torch.Generator("cuda").manual_seed(seed + 21))
        ents.append(dict(q=q[1].contiguous(), k_index=bufs["k_index"], v_index=bufs["v_index"],
                         k_codebook=kcb, v_codebook=vcb, k_window=bufs["k_window"],
                         v_window=bufs["v_window"], out=bufs["out"]))
    ctx = torch.tensor([L], dtype=torch.int32, device="cuda")
    ws = _workspace(lv, cfg, 4)
    lv.lvq_decode_attn_layers(cfg, 1, ents, ctx, L, ws)
    torch.cuda.synchronize()
    for i, e in enumerate(ents):
        ref = oracle.decode_attn(loop_step=1, q=e["q"].cpu(), ctx_len=[L],
                                 k_index=e["k_index"].cpu(), v_index=e["v_index"].cpu(),
                                 k_codebook=e["k_codebook"].cpu(), v_codebook=e["v_codebook"].cpu(),
                                 k_window=e["k_window"].cpu(), v_window=e["v_window"].cpu(),
                                 n_sink=64, n_recent=256, group=G)
        err = rel_err_rows(e["out"].double().cpu().numpy(), ref)
        _note(f"  layer {i}: rel err {err:.2e}")
        assert err <= TOL

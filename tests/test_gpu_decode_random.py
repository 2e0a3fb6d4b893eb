"""Seeded random sweep of lvq_decode_attn / lvq_decode_attn_layers against
the CPU oracle (MI355X).

Every case draws a supported shape (head_dim, G, codebook dtype), a batch of
ragged lengths mixing window-only, short and multi-split sequences (for some
cases 45-89 sequences, a grid beyond the chip taken one workgroup per (b, h)
in longest-first order), a grouped-query ratio, a loop-group count, an
optional page lag (vq_len), an optional explicit split count and window
workgroup count, sm_scale, the loop step and, for some cases, two layers in
one call.  Indices are drawn (exact codewords), so the oracle
takes the same cache.  Bar: per (b, h) row, max_ch |gpu - oracle| /
max_ch |oracle| <= 2e-3.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
from cases import DeviceCache, make_cache, merge_loop_groups, oracle_decode, rel_err_rows

pytestmark = pytest.mark.gpu
TOL = 2e-3
N_CASES = 32
SHAPES = [  # (head_dim, G, codebook dtype): every supported sub-vector shape
    (32, 8, torch.bfloat16), (32, 16, torch.bfloat16), (32, 16, torch.float32),
    (64, 8, torch.bfloat16), (64, 8, torch.float32), (64, 16, torch.bfloat16),
    (64, 16, torch.float32), (64, 32, torch.bfloat16), (128, 8, torch.bfloat16),
    (128, 16, torch.bfloat16), (128, 32, torch.bfloat16),
]


@pytest.fixture(scope="module")
def lv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sub_bit_vq_amd import loopvq
    loopvq.library()
    return loopvq


def _draw(seed):
    rng = np.random.default_rng(seed)
    d, G, dt = SHAPES[int(rng.integers(len(SHAPES)))]
    big = seed % 8 == 5                           # a grid beyond the chip: one workgroup per (b, h)
    B = int(rng.integers(45, 90)) if big else int(rng.integers(1, 5))
    kinds = rng.integers(0, 3 if big else 4, size=B)   # window-only, short, medium, long
    bounds = [(1, 320), (321, 900), (901, 4000), (4001, 9000)]
    lengths = [int(rng.integers(*bounds[k])) for k in kinds]
    Hk = 3 if big else int(rng.integers(1, 4))
    qpk = 1 if big else int(rng.choice([1, 2, 4]))
    groups = int(rng.choice([1, 1, 2]))
    lag = bool(rng.integers(0, 4) == 0)
    vq = None
    if lag:   # vq_len above the exact-window count by up to one page
        vq = [max(0, L - 320) + (int(rng.integers(0, 9)) if L > 320 else 0) for L in lengths]
        vq = [min(v, max(0, L - min(L, 64))) for v, L in zip(vq, lengths)]
    splits = int(rng.choice([0, 0, 0, int(rng.integers(1, 21))]))
    # with a forced split count, sometimes a forced number of window workgroups
    wgroups = int(rng.integers(1, min(4, splits - 1) + 1)) if splits > 1 and rng.integers(0, 2) else 0
    sm = float(rng.choice([1.0, 1.0 / np.sqrt(d)]))
    layers = int(rng.choice([1, 1, 2]))
    return dict(d=d, G=G, dt=dt, B=B, lengths=lengths, Hk=Hk, qpk=qpk, groups=groups, vq=vq,
                splits=splits, wgroups=wgroups, sm=sm, layers=layers, t=int(rng.integers(0, 4 * groups)))


def _cache(p, seed):
    parts = [make_cache(batch=p["B"], n_heads=p["Hk"], q_heads=p["Hk"] * p["qpk"] if p["qpk"] > 1 else None,
                        head_dim=p["d"], group=p["G"], lengths=p["lengths"], cb_dtype=p["dt"],
                        seed=seed + 31 * g, codeword_tokens=True, vq_len=p["vq"])
             for g in range(p["groups"])]
    return parts[0] if p["groups"] == 1 else merge_loop_groups(parts)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_decode(lv, case):
    p = _draw(9000 + case)
    print(f"[gpu] random case {case}: {p}", file=sys.stderr, flush=True)
    caches = [_cache(p, 5000 + 100 * case + 7 * i) for i in range(p["layers"])]
    dcs = [DeviceCache(lv, c) for c in caches]
    cfg = dcs[0].cfg
    if p["splits"]:
        cfg = dataclasses.replace(cfg, decode_splits=p["splits"], decode_window_groups=p["wgroups"])
    t, L = p["t"], max(p["lengths"])
    if p["layers"] == 1:
        got = [dcs[0].decode(t, p["sm"], cfg=cfg)]
    else:
        per = lv.lvq_cache_layout(cfg)["workspace_bytes"]
        ws = torch.zeros(p["layers"] * per, dtype=torch.uint8, device="cuda")
        ents = [dict(q=dc.q[t].contiguous(), k_index=dc.k_index, v_index=dc.v_index,
                     k_codebook=dc.k_cb, v_codebook=dc.v_cb, k_window=dc.k_win,
                     v_window=dc.v_win, out=dc.out) for dc in dcs]
        lv.lvq_decode_attn_layers(cfg, t, ents, dcs[0].ctx, L, ws, sm_scale=p["sm"],
                                  vq_len=dcs[0].vq)
        torch.cuda.synchronize()
        got = [dc.out.double().cpu().numpy() for dc in dcs]
    for i, c in enumerate(caches):
        ref = oracle_decode(oracle, c, t, p["sm"])
        assert np.isfinite(got[i]).all()
        err = rel_err_rows(got[i], ref)
        assert err <= TOL, f"layer {i}: rel err {err:.3e}"

"""C-ABI checks that need no GPU: the library loads, exports every function
``include/loopvq.h`` declares, computes layouts that reproduce the pages'
bit budgets, and rejects bad arguments before anything is launched."""
import ctypes
import json
import pathlib
import re

import numpy as np
import pytest

from sub_bit_vq_amd import loopvq as lv

ROOT = pathlib.Path(__file__).resolve().parents[1]
GOLDEN = json.loads((ROOT / "tests" / "golden" / "page_constants.json").read_text())

WORKLOADS = {  # (B, H, d, Tc, G, max_tokens, cb dtype)
    "tiny_0p5bit_fp32cb": (1, 1, 64, 4, 16, 512, lv.LVQ_F32),
    "ouro1p4b_layer_32k_0p5bit": (1, 16, 128, 4, 16, 32768, lv.LVQ_BF16),
    "ouro1p4b_layer_32k_0p25bit": (1, 16, 128, 4, 32, 32768, lv.LVQ_BF16),
    "batch64_ragged_0p5bit": (64, 16, 128, 4, 16, 18432, lv.LVQ_BF16),
}


def _cfg(B, H, d, Tc, G, T, dt, **kw):
    return lv.Config(batch=B, n_heads=H, head_dim=d, loop_steps=Tc, group=G, max_tokens=T,
                     codebook_dtype=dt, **kw)


def test_library_exports_header_symbols():
    declared = set()
    for header in sorted((ROOT / "include").glob("*.h")):
        declared |= set(re.findall(r"^\s*(?:const\s+char\s*\*|lvq_status|int32_t)\s*(lvq_\w+)\s*\(",
                                   header.read_text(), flags=re.M))
    assert declared == set(lv.EXPORTS)
    lib = lv.library()
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    for s in range(5):
        assert lv.lvq_status_string(s)
    assert "unknown" in lv.lvq_status_string(99)


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_layout_shapes(name):
    B, H, d, Tc, G, T, dt = WORKLOADS[name]
    lay = lv.lvq_cache_layout(_cfg(B, H, d, Tc, G, T, dt))
    cg = G // Tc
    S = d // cg
    assert lay["n_sub"] == S and lay["sub_channels"] == cg and lay["n_codes"] == 256
    assert lay["k_index"]["shape"] == (B, H, T, S) and lay["k_index"]["bytes"] == B * H * T * S
    assert lay["k_codebook"]["shape"] == (Tc, H, 256, S, cg)
    assert lay["k_codebook"]["bytes"] == Tc * H * S * 256 * cg * (2 if dt == lv.LVQ_BF16 else 4)
    assert lay["k_window"]["shape"] == (B, Tc, H, 64 + 256, d)
    assert lay["query"]["shape"] == (B, H, d) and lay["output"]["bytes"] == B * H * d * 4
    assert lay["workspace_bytes"] >= B * H * lv.LVQ_MAX_SPLITS * (d + 2) * 4


def test_layout_grouped_query_heads():
    """12 query heads over 4 KV heads: caches, codebooks and windows per KV
    head; query, output and workspace per query head."""
    B, H, Hk, d, Tc, G, T = 2, 12, 4, 128, 4, 16, 1000
    lay = lv.lvq_cache_layout(lv.Config(batch=B, n_heads=H, head_dim=d, loop_steps=Tc, group=G,
                                        max_tokens=T, n_kv_heads=Hk))
    mha = lv.lvq_cache_layout(lv.Config(batch=B, n_heads=H, head_dim=d, loop_steps=Tc, group=G,
                                        max_tokens=T))
    S = d // (G // Tc)
    assert lay["k_index"]["shape"] == (B, Hk, T, S)
    assert lay["v_codebook"]["shape"] == (Tc, Hk, 256, S, G // Tc)
    assert lay["k_window"]["shape"] == (B, Tc, Hk, 64 + 256, d)
    assert lay["query"]["shape"] == (B, H, d) and lay["output"]["shape"] == (B, H, d)
    assert lay["workspace_bytes"] == mha["workspace_bytes"]
    # n_kv_heads = n_heads is multi-head attention
    same = lv.lvq_cache_layout(lv.Config(batch=B, n_heads=H, head_dim=d, loop_steps=Tc, group=G,
                                         max_tokens=T, n_kv_heads=H))
    assert same == mha


def test_layout_loop_groups():
    """R = 12 loop steps over Tc = 4: three index rows per token, stored as
    three [B][H][T][S] blocks; codebooks and windows carry all 12 steps."""
    B, H, d, Tc, G, T, R = 2, 4, 64, 4, 16, 500, 12
    lay = lv.lvq_cache_layout(lv.Config(batch=B, n_heads=H, head_dim=d, loop_steps=Tc, group=G,
                                        max_tokens=T, n_loops=R))
    S = d // (G // Tc)
    assert lay["k_index"]["shape"] == (R // Tc, B, H, T, S)
    assert lay["k_index"]["bytes"] == (R // Tc) * B * H * T * S
    assert lay["k_codebook"]["shape"] == (R, H, 256, S, G // Tc)
    assert lay["v_window"]["shape"] == (B, R, H, 64 + 256, d)
    assert lay["bits_per_element"] == 8 / G
    # R = Tc is the single-group layout
    one = lv.lvq_cache_layout(lv.Config(batch=B, n_heads=H, head_dim=d, loop_steps=Tc, group=G,
                                        max_tokens=T, n_loops=Tc))
    assert one["k_index"]["shape"] == (B, H, T, S)


def test_layout_reproduces_page_bit_budgets():
    """bits/element, compression and bytes read per token and loop step, as
    the project page prints them (Highlights; Efficiency -- Latency), for the
    loop-step count of its redundancy figure."""
    Tc = GOLDEN["loop_steps_per_code"]["value"]
    for row in GOLDEN["bit_budgets"]:
        G = int(round(8 / row["bits_per_element"]))
        lay = lv.lvq_cache_layout(_cfg(1, 16, 128, Tc, G, 1024, lv.LVQ_BF16))
        assert lay["bits_per_element"] == row["bits_per_element"]
        assert lay["compression_vs_bf16"] == row["compression_vs_bf16"]
        assert lay["read_reduction_per_step"] == row["bytes_read_reduction_per_token_per_loop_step"]


def test_default_windows_match_pages():
    w = {e["name"]: e["value"] for e in GOLDEN["window"]}
    cfg = lv.Config(batch=1, n_heads=1, head_dim=64)
    assert (cfg.n_sink, cfg.n_recent) == (w["n_sink"], w["n_recent"])


@pytest.mark.parametrize("bad", [
    dict(batch=0), dict(n_heads=0), dict(head_dim=0), dict(loop_steps=0), dict(group=18),
    dict(group=16, head_dim=66), dict(n_sink=-1), dict(n_recent=0), dict(max_tokens=-1),
    dict(codebook_dtype=7), dict(decode_splits=65), dict(decode_splits=-1),
    dict(n_kv_heads=-1), dict(n_kv_heads=3), dict(n_heads=6, n_kv_heads=4),
    dict(n_loops=-4), dict(n_loops=6), dict(n_loops=68),
    dict(decode_window_groups=1), dict(decode_splits=8, decode_window_groups=-1),
    dict(decode_splits=8, decode_window_groups=5), dict(decode_splits=3, decode_window_groups=3),
    dict(n_sink=lv.LVQ_MAX_WINDOW_SLOTS // 2, n_recent=lv.LVQ_MAX_WINDOW_SLOTS // 2 + 1),
])
def test_layout_rejects_bad_config(bad):
    base = dict(batch=1, n_heads=2, head_dim=64, loop_steps=4, group=16, max_tokens=100)
    base.update(bad)
    with pytest.raises(lv.LoopVQError) as e:
        lv.lvq_cache_layout(lv.Config(**base))
    assert e.value.status == lv.LVQ_ERR_INVALID_ARG


def test_decode_splits():
    cfg = _cfg(*WORKLOADS["ouro1p4b_layer_32k_0p5bit"])
    splits = lambda c, L: (lv.lvq_decode_splits(c, L), lv.lvq_decode_window_groups(c, L))  # noqa: E731
    # Grid within the chip: VQ token chunks + window workgroups per (b, h).
    # A round costs its slowest workgroup: a VQ chunk in whole 384-token
    # batches, or a window range at 8 VQ tokens per slot (512 B against 64 B),
    # each plus a fixed start-up of 6 batches.  32448 VQ tokens in 15 chunks
    # of 2164 take 6 batches (4608 token-equivalents); one window workgroup
    # reads 320 slots (2304 + 2560 = 4864) and sets the round; 14 chunks of
    # 2318 would take 7 batches (4992).
    assert splits(cfg, 32768) == (16, 1)
    assert splits(cfg, 320) == (1, 0)                   # nothing VQ-coded: windows only
    # short contexts: the window rows outweigh the VQ chunks, so they are
    # split: 2 chunks of 550 (2 batches, 3072) and 4 window ranges of 80 slots
    # (2304 + 640)
    assert splits(cfg, 320 + 1100) == (6, 4)
    assert splits(cfg, 320 + 600) == (5, 4)            # splits stay >= 512 tokens
    assert splits(cfg, 2048) == (7, 4)                  # 3 chunks of 576
    assert lv.lvq_decode_splits(cfg, 40000) == 0        # beyond max_tokens
    assert lv.lvq_decode_window_groups(cfg, 40000) == -1
    # 0.25 bit (S = 16, 768-token batches, a window slot weighs 16 VQ tokens):
    # one window workgroup would cost 4608 + 5120; two cost 4608 + 2560, below
    # the 4 batches of any chunk count from 11 (2950 tokens) to 14 (2318), and
    # ties go to the fewest workgroups
    cfg2 = _cfg(*WORKLOADS["ouro1p4b_layer_32k_0p25bit"])
    assert splits(cfg2, 32768) == (13, 2)
    # Larger grids (1024 heads over 256 CUs): every split costs a workgroup
    # start-up in every round, so one workgroup per (b, h) takes its whole
    # context and its window slots.
    cfg3 = _cfg(*WORKLOADS["batch64_ragged_0p5bit"])
    assert splits(cfg3, 18432) == (1, 0)
    # forced plans: decode_splits alone takes one window workgroup when the
    # grid fits, decode_window_groups sets the count; a grid beyond the chip
    # spreads the window slots
    forced = lambda **kw: _cfg(1, 16, 128, 4, 16, 32768, lv.LVQ_BF16, **kw)  # noqa: E731
    assert splits(forced(decode_splits=7), 32768) == (7, 1)
    assert splits(forced(decode_splits=7, decode_window_groups=3), 32768) == (7, 3)
    assert splits(forced(decode_splits=17, decode_window_groups=3), 32768) == (17, 0)
    assert splits(forced(decode_splits=1), 32768) == (1, 0)


# --- argument validation: every case fails before any HIP call ---------------

_HOST = np.zeros(1 << 16, np.uint8)            # an aligned host address; never dereferenced
P = ctypes.c_void_p((_HOST.ctypes.data + 255) // 256 * 256)


def _decode(cfg, **over):
    lay = lv.lvq_cache_layout(cfg)
    a = dict(loop_step=0, q=P, ctx_len=P, vq_len=None, max_ctx_len=cfg.max_tokens, k_index=P,
             v_index=P, k_cb=P, v_cb=P, k_win=P, v_win=P, sm_scale=1.0, ws=P,
             ws_bytes=lay["workspace_bytes"], out=P)
    a.update(over)
    return lv.library().lvq_decode_attn(
        ctypes.byref(cfg.c()), a["loop_step"], a["q"], a["ctx_len"], a["vq_len"],
        a["max_ctx_len"], a["k_index"], a["v_index"], a["k_cb"], a["v_cb"], a["k_win"],
        a["v_win"], ctypes.c_float(a["sm_scale"]), a["ws"], ctypes.c_uint64(a["ws_bytes"]),
        a["out"], None)


def test_decode_validation():
    cfg = _cfg(1, 2, 64, 4, 16, 1024, lv.LVQ_BF16)
    INV, UNS, WS = lv.LVQ_ERR_INVALID_ARG, lv.LVQ_ERR_UNSUPPORTED, lv.LVQ_ERR_WORKSPACE
    assert _decode(cfg, q=None) == INV
    assert _decode(cfg, k_index=None) == INV
    assert _decode(cfg, out=None) == INV
    assert _decode(cfg, loop_step=4) == INV
    assert _decode(cfg, loop_step=-1) == INV
    assert _decode(cfg, max_ctx_len=1025) == INV
    assert _decode(cfg, sm_scale=float("nan")) == INV
    assert _decode(cfg, k_win=ctypes.c_void_p(P.value + 8)) == INV      # misaligned
    assert _decode(cfg, ws=None) == WS
    assert _decode(cfg, ws_bytes=lv.lvq_cache_layout(cfg)["workspace_bytes"] - 1) == WS
    assert _decode(_cfg(1, 2, 384, 4, 16, 1024, lv.LVQ_BF16)) == UNS     # S = 96
    assert _decode(_cfg(1, 2, 256, 4, 16, 1024, lv.LVQ_BF16)) == UNS     # tables exceed LDS
    assert _decode(_cfg(1, 2, 128, 4, 16, 1024, lv.LVQ_F32)) == UNS      # fp32 tables too big
    assert _decode(_cfg(1, 2, 64, 4, 16, 1024, lv.LVQ_BF16), k_cb=ctypes.c_void_p(P.value + 8)) == INV
    assert _decode(_cfg(1, 2, 64, 1, 1, 1024, lv.LVQ_BF16)) == UNS       # cg = 1
    bad = lv.Config(batch=1, n_heads=1, head_dim=64, group=18)
    assert lv.library().lvq_decode_attn(ctypes.byref(bad.c()), 0, *([P] * 2), None, 0,
                                        *([P] * 6), ctypes.c_float(1.0), P,
                                        ctypes.c_uint64(1 << 30), P, None) == INV


def _decode_noalloc(cfg, **over):
    a = dict(loop_step=0, q=P, ctx_len=P, vq_len=None, max_ctx_len=cfg.max_tokens, k_index=P,
             v_index=P, k_cb=P, v_cb=P, k_win=P, v_win=P, sm_scale=1.0, out=P)
    a.update(over)
    return lv.library().lvq_decode_attn_noalloc(
        ctypes.byref(cfg.c()), a["loop_step"], a["q"], a["ctx_len"], a["vq_len"],
        a["max_ctx_len"], a["k_index"], a["v_index"], a["k_cb"], a["v_cb"], a["k_win"],
        a["v_win"], ctypes.c_float(a["sm_scale"]), a["out"], None)


def test_decode_noalloc_validation():
    """The allocation-free entry point checks its arguments like
    lvq_decode_attn, and rejects a merging plan over more (b, h) pairs than
    its static workspace holds, before any HIP call."""
    cfg = _cfg(1, 2, 64, 4, 16, 1024, lv.LVQ_BF16)
    INV, UNS, WS = lv.LVQ_ERR_INVALID_ARG, lv.LVQ_ERR_UNSUPPORTED, lv.LVQ_ERR_WORKSPACE
    assert _decode_noalloc(cfg, q=None) == INV
    assert _decode_noalloc(cfg, out=None) == INV
    assert _decode_noalloc(cfg, loop_step=4) == INV
    assert _decode_noalloc(cfg, k_win=ctypes.c_void_p(P.value + 8)) == INV
    assert _decode_noalloc(_cfg(1, 2, 256, 4, 16, 1024, lv.LVQ_BF16)) == UNS
    limit = lv.LVQ_NOALLOC_MAX_HEADS
    big = _cfg(20, 16, 64, 4, 16, 1200, lv.LVQ_BF16, decode_splits=2)   # 320 > 256 pairs, merging
    assert 20 * 16 > limit and lv.lvq_decode_splits(big, 1200) == 2
    assert _decode_noalloc(big) == WS
    hdr = lv.WORKSPACE_HEADER_BYTES
    blk = lv.lvq_cache_layout(_cfg(1, 1, 64, 4, 16, 16, lv.LVQ_BF16))["workspace_bytes"] - hdr
    assert hdr + limit * blk == 17105152          # LVQ_NOALLOC_SCRATCH_BYTES


def _decode_layers(cfg, n_layers=3, layer_over=None, **over):
    lay = lv.lvq_cache_layout(cfg)
    arr = (lv._DecodeLayer * max(1, n_layers))()
    for i in range(n_layers):
        for key in lv.LAYER_KEYS:
            setattr(arr[i], key, P)
    for (i, key), v in (layer_over or {}).items():
        setattr(arr[i], key, v)
    a = dict(n_layers=n_layers, layers=arr, loop_step=0, ctx_len=P, vq_len=None,
             max_ctx_len=cfg.max_tokens, sm_scale=1.0, ws=P,
             ws_bytes=n_layers * lay["workspace_bytes"])
    a.update(over)
    return lv.library().lvq_decode_attn_layers(
        ctypes.byref(cfg.c()), a["n_layers"], a["loop_step"], a["layers"], a["ctx_len"],
        a["vq_len"], a["max_ctx_len"], ctypes.c_float(a["sm_scale"]), a["ws"],
        ctypes.c_uint64(a["ws_bytes"]), None)


def test_decode_layers_validation():
    """Every argument of the multi-layer call is checked before any launch:
    the layer count, each layer's buffers and the workspace of all layers."""
    cfg = _cfg(1, 2, 64, 4, 16, 1024, lv.LVQ_BF16)
    INV, UNS, WS = lv.LVQ_ERR_INVALID_ARG, lv.LVQ_ERR_UNSUPPORTED, lv.LVQ_ERR_WORKSPACE
    per = lv.lvq_cache_layout(cfg)["workspace_bytes"]
    assert _decode_layers(cfg, n_layers=0) == INV
    assert _decode_layers(cfg, n_layers=lv.LVQ_MAX_LAYERS + 1) == INV
    assert _decode_layers(cfg, layers=None) == INV
    assert _decode_layers(cfg, ctx_len=None) == INV
    for key in lv.LAYER_KEYS:                                           # any layer, any buffer
        assert _decode_layers(cfg, layer_over={(2, key): None}) == INV, key
    assert _decode_layers(cfg, layer_over={(1, "k_window"): P.value + 8}) == INV   # misaligned
    assert _decode_layers(cfg, layer_over={(0, "v_codebook"): P.value + 8}) == INV
    assert _decode_layers(cfg, loop_step=4) == INV
    assert _decode_layers(cfg, sm_scale=float("inf")) == INV
    hdr = lv.WORKSPACE_HEADER_BYTES
    assert _decode_layers(cfg, ws_bytes=hdr + 3 * (per - hdr) - 1) == WS   # one block set per layer
    assert _decode_layers(cfg, ws=None) == WS
    assert _decode_layers(_cfg(1, 2, 384, 4, 16, 1024, lv.LVQ_BF16)) == UNS


def _encode(cfg, **over):
    a = dict(x=P, strides=None, n=16, cb=P, index=P, seq=0, first=0)
    a.update(over)
    st = None if a["strides"] is None else (ctypes.c_int64 * 3)(*a["strides"])
    return lv.library().lvq_encode(ctypes.byref(cfg.c()), a["x"], st, a["n"], a["cb"], a["index"],
                                   a["seq"], a["first"], None)


def test_encode_validation():
    cfg = _cfg(2, 2, 64, 4, 16, 100, lv.LVQ_BF16)
    INV, UNS = lv.LVQ_ERR_INVALID_ARG, lv.LVQ_ERR_UNSUPPORTED
    assert _encode(cfg, x=None) == INV
    assert _encode(cfg, cb=None) == INV
    assert _encode(cfg, index=None) == INV
    assert _encode(cfg, seq=2) == INV
    assert _encode(cfg, seq=-1) == INV
    assert _encode(cfg, first=90, n=11) == INV
    assert _encode(cfg, n=-1) == INV
    assert _encode(cfg, strides=(512, 256, 63)) == INV                  # not a multiple of cg
    assert _encode(cfg, x=ctypes.c_void_p(P.value + 2)) == INV         # misaligned
    assert _encode(cfg, index=ctypes.c_void_p(P.value + 2)) == INV     # index rows written as 4-byte words
    assert _encode(_cfg(1, 1, 64, 4, 64, 100, lv.LVQ_BF16)) == UNS      # G = 64
    assert _encode(_cfg(1, 1, 128, 4, 32, 100, lv.LVQ_F32)) == UNS      # fp32, G = 32
    assert _encode(cfg, n=0) == lv.LVQ_OK                              # nothing to launch


# --- workspace grid and merge roles (host arithmetic) ---------------------------

def test_workspace_grid_is_fixed():
    """The workspace is a header plus one fixed-size block per (layer, b, h):
    its size is linear in B * H and does not depend on head_dim, group or
    context, so blocks keep their places when the batch changes."""
    size = lambda **kw: lv.lvq_cache_layout(_cfg(**{**dict(B=1, H=16, d=128, Tc=4, G=16,  # noqa: E731
                                                       T=4096, dt=lv.LVQ_BF16), **kw}))["workspace_bytes"]
    hdr = lv.WORKSPACE_HEADER_BYTES
    blk = size(B=1, H=1) - hdr
    assert blk % 256 == 0 and blk >= lv.LVQ_MAX_SPLITS * (128 + 2) * 8
    for B, H in ((1, 16), (32, 16), (64, 16), (3, 5)):
        assert size(B=B, H=H) == hdr + B * H * blk
    assert size(d=64) == size(d=128) == size(G=32) == size(T=40000)


def _roles(B, H, n, layers=1, L=32768):
    """role, (layer, seq, head) of every workgroup of a forced n-split launch"""
    cfg = _cfg(B, H, 128, 4, 16, max(L, 1), lv.LVQ_BF16, decode_splits=n)
    total = n * B * H * layers
    out = [lv.lvq_decode_role(cfg, layers, L, p) for p in range(total)]
    assert lv.lvq_decode_role(cfg, layers, L, total) is None
    assert lv.lvq_decode_role(cfg, layers, L, -1) is None
    return out


def test_merge_roles_follow_dispatch_order():
    """For every launch of at most 256 workgroups (every split count 1..64
    and number of (b, h) groups): each group gets roles 0..n-1 once, the
    member with role n - 1 (the merger of a window-workgroup launch) is the
    group's last in dispatch order, and a group that fits one XCD slab sits
    on one XCD (dispatch index mod 8)."""
    checked = 0
    for n in range(1, lv.LVQ_MAX_SPLITS + 1):
        for groups in range(1, 256 // n + 1):
            roles = _roles(groups, 1, n)
            members = {}
            for p, r in enumerate(roles):
                assert r is not None
                members.setdefault((r[1], r[2], r[3]), []).append((p, r[0]))
            assert len(members) == groups
            total = n * groups
            for key, ms in members.items():
                assert sorted(r for _, r in ms) == list(range(n)), (n, groups, key)
                last = max(ms)                   # highest dispatch index
                assert last[1] == n - 1, (n, groups, key, ms)
                # roles follow dispatch order within the group
                assert [r for _, r in sorted(ms)] == list(range(n)), (n, groups, key)
                if total % 8 == 0:
                    slab = total // 8
                    g = key[1]
                    if (g * n) // slab == (g * n + n - 1) // slab:
                        assert len({p % 8 for p, _ in ms}) == 1
            checked += 1
    assert checked > 1000


def test_merge_roles_multi_layer():
    """Layers are the outermost groups; roles still follow dispatch order."""
    for B, H, n, layers in ((1, 16, 5, 3), (2, 3, 7, 4), (1, 2, 16, 8)):
        roles = _roles(B, H, n, layers)
        members = {}
        for p, r in enumerate(roles):
            members.setdefault(r[1:], []).append((p, r[0]))
        assert set(members) == {(l, b, h) for l in range(layers) for b in range(B) for h in range(H)}
        for ms in members.values():
            assert [r for _, r in sorted(ms)] == list(range(n))

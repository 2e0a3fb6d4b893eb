"""Test infrastructure: drive a sanitizer build of the CPU oracle and of the
library's host code (C ABI with stand-in kernel launchers) through their
entry points.  Run by tests/test_sanitize_cpu.py in a subprocess with the
address sanitizer preloaded; any finding aborts the process.

usage: drive.py ORACLE_SO HOST_SO
"""
import ctypes
import pathlib
import sys
import types

ROOT = pathlib.Path(__file__).resolve().parents[2]
sys.path.insert(0, str(ROOT))

# The binding module imports torch only for its tensor helpers; the raw
# entry points used here need none of it, and an uninstrumented torch under
# the sanitizer runtime is slow to load.
if "torch" not in sys.modules:
    stub = types.ModuleType("torch")
    stub.Tensor = type("Tensor", (), {})
    sys.modules["torch"] = stub

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from sub_bit_vq_amd import loopvq as lv  # noqa: E402

rng = np.random.default_rng(7)


def bf16_bits(a):
    """round-to-nearest-even fp32 -> bf16 bit patterns (inputs only)"""
    u = np.asarray(a, np.float32).view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def drive_oracle(path):
    with oracle.use_library(path):
        for (H, d, Tc, G, R, bf16) in ((2, 64, 4, 16, 4, True), (1, 64, 4, 16, 4, False),
                                       (2, 128, 4, 32, 4, True), (1, 64, 4, 8, 4, False),
                                       (2, 64, 4, 16, 8, True)):
            n = 37
            S = d // (G // Tc)
            x = bf16_bits(rng.standard_normal((n, H, R, d)))
            cb = rng.standard_normal((R, H, 256, S, G // Tc)).astype(np.float32)
            cb = bf16_bits(cb) if bf16 else cb
            idx = oracle.encode(x, cb, n_heads=H, head_dim=d, loop_steps=Tc, group=G, n_loops=R,
                                t_max=n + 5, seq=1, first_token=3, threads=2)
            assert idx.shape[-1] == S
            # decode over window-only, wrapped-ring and page-lagged contexts
            B, Hq = 3, 2 * H
            T = 700
            shape = (B, H, T, S) if R == Tc else (R // Tc, B, H, T, S)
            ki = rng.integers(0, 256, shape, dtype=np.uint8)
            vi = rng.integers(0, 256, shape, dtype=np.uint8)
            win = bf16_bits(rng.standard_normal((B, R, H, 320, d)))
            win2 = bf16_bits(rng.standard_normal((B, R, H, 320, d)))
            q = bf16_bits(rng.standard_normal((B, Hq, d)) / 8)
            for lengths, vq in (([0, 40, 300], None), ([700, 321, 1], None), ([700, 400, 5], [390, 80, 0])):
                for t in (0, R - 1):
                    out, p = oracle.decode_attn(loop_step=t, q=q, ctx_len=lengths, k_index=ki, v_index=vi,
                                                k_codebook=cb, v_codebook=cb, k_window=win,
                                                v_window=win2, n_sink=64, n_recent=256, group=G,
                                                vq_len=vq, want_p=True, threads=2, loop_steps=Tc)
                    assert np.isfinite(out).all() and out.shape == (B, Hq, d)
            K = rng.standard_normal((50, d))
            oracle.attend(rng.standard_normal(d), K, K, 0.1)


P = None


def drive_host(path):
    global P
    lv.LIB_PATH = pathlib.Path(path)
    lib = lv.library()
    lib.lvq_stub_counts.restype = ctypes.c_int
    lib.lvq_stub_counts.argtypes = [ctypes.c_int]
    host = np.zeros(1 << 20, np.uint8)
    P = ctypes.c_void_p((host.ctypes.data + 255) // 256 * 256)   # never dereferenced
    OK = lv.LVQ_OK

    def cfg(**kw):
        base = dict(batch=2, n_heads=4, head_dim=128, loop_steps=4, group=16, max_tokens=5000)
        base.update(kw)
        return lv.Config(**base)

    # layouts, plans and roles over many shapes
    for c in (cfg(), cfg(group=32), cfg(head_dim=64, codebook_dtype=lv.LVQ_F32), cfg(n_kv_heads=2),
              cfg(n_loops=8), cfg(batch=64, n_heads=16, max_tokens=18432), cfg(n_sink=0, n_recent=1)):
        lay = lv.lvq_cache_layout(c)
        assert lay["workspace_bytes"] > 0
        for L in (0, 1, 320, 321, 2000, c.max_tokens):
            n = lv.lvq_decode_splits(c, L)
            assert n >= 1 and lv.lvq_decode_window_groups(c, L) >= 0
            nh = lv.lvq_decode_heads_per_workgroup(c, 1, L)
            assert nh in (1, 2)
            total = n * c.batch * (c.n_heads // nh)
            for p in (0, total // 2, total - 1):
                assert lv.lvq_decode_role(c, 1, L, p) is not None
    for n in range(1, 65):
        for groups in (1, 3, 256 // n):
            c = cfg(batch=groups, n_heads=1, decode_splits=n, max_tokens=32768)
            for p in range(n * groups):
                assert lv.lvq_decode_role(c, 1, 32768, p) is not None

    def decode(c, **over):
        try:
            wsb = lv.lvq_cache_layout(c)["workspace_bytes"]
        except lv.LoopVQError:                 # an invalid shape: the call must refuse it too
            wsb = 1 << 19
        a = dict(t=0, q=P, ctx=P, vq=None, L=c.max_tokens, ki=P, vi=P, kc=P, vc=P, kw=P, vw=P, sc=1.0,
                 ws=P, wsb=wsb, out=P)
        a.update(over)
        return lib.lvq_decode_attn(ctypes.byref(c.c()), a["t"], a["q"], a["ctx"], a["vq"], a["L"],
                                   a["ki"], a["vi"], a["kc"], a["vc"], a["kw"], a["vw"],
                                   ctypes.c_float(a["sc"]), a["ws"], ctypes.c_uint64(a["wsb"]), a["out"],
                                   None)

    launches = lib.lvq_stub_counts(0)
    for c in (cfg(), cfg(group=32), cfg(n_kv_heads=1), cfg(n_loops=8), cfg(decode_splits=17),
              cfg(decode_splits=5, decode_window_groups=3), cfg(batch=64, n_heads=16, max_tokens=18432),
              cfg(head_dim=64, codebook_dtype=lv.LVQ_F32), cfg(decode_poll_limit=1),
              cfg(n_kv_heads=2), cfg(n_kv_heads=2, decode_splits=1), cfg(n_kv_heads=2, decode_heads_per_group=1),
              cfg(n_kv_heads=2, decode_heads_per_group=2), cfg(n_kv_heads=2, decode_splits=64, batch=8)):
        for L in (1, 321, c.max_tokens):
            assert decode(c, L=L) == OK, (c, L, decode(c, L=L))
            assert decode(c, L=L, vq=P) == OK
            assert decode(c, t=c.loops - 1, L=L, sc=0.125) == OK
    assert lib.lvq_stub_counts(0) > launches
    # every rejection path
    c = cfg()
    for over in (dict(q=None), dict(ki=None), dict(out=None), dict(t=4), dict(t=-1), dict(L=5001),
                 dict(sc=float("nan")), dict(kw=ctypes.c_void_p(P.value + 8)), dict(q=ctypes.c_void_p(P.value + 8)),
                 dict(ws=None),
                 dict(wsb=0), dict(ws=ctypes.c_void_p(P.value + 64))):
        assert decode(c, **over) != OK, over
    for bad in (cfg(head_dim=256), cfg(head_dim=384), cfg(group=18), cfg(loop_steps=3),
                cfg(n_kv_heads=3), cfg(n_loops=6), cfg(decode_window_groups=2), cfg(decode_heads_per_group=3),
                cfg(decode_heads_per_group=2), cfg(n_kv_heads=2, group=32, decode_heads_per_group=2)):
        assert decode(bad) != OK, bad
    # layers: 20 layers are two launches
    arr = (lv._DecodeLayer * 20)()
    for i in range(20):
        for key in lv.LAYER_KEYS:
            setattr(arr[i], key, P)
    lay = lv.lvq_cache_layout(c)
    before = lib.lvq_stub_counts(0)
    assert lib.lvq_decode_attn_layers(ctypes.byref(c.c()), 20, 1, arr, P, None, 5000, ctypes.c_float(1.0), P,
                                      ctypes.c_uint64(20 * lay["workspace_bytes"]), None) == OK
    assert lib.lvq_stub_counts(0) == before + 2
    # allocation-free entry
    for cc, want in ((cfg(), OK), (cfg(batch=64, n_heads=16, max_tokens=18432), OK),
                     (cfg(batch=20, n_heads=16, max_tokens=1200, decode_splits=2), lv.LVQ_ERR_WORKSPACE)):
        st = lib.lvq_decode_attn_noalloc(ctypes.byref(cc.c()), 0, P, P, None, cc.max_tokens, P, P, P, P, P, P,
                                         ctypes.c_float(1.0), P, None)
        assert st == want, (cc, st)
    # status word read from (host) memory through the runtime stand-in
    flags = ctypes.c_uint32()
    ctypes.c_uint32.from_address(P.value).value = 3
    assert lib.lvq_decode_status(P, ctypes.byref(flags), 1, None) == OK and flags.value == 3
    assert lib.lvq_decode_status(P, ctypes.byref(flags), 0, None) == OK and flags.value == 0
    assert lib.lvq_decode_status(None, ctypes.byref(flags), 0, None) != OK
    # encoder entries
    for ce in (cfg(), cfg(group=32), cfg(head_dim=64, group=8, codebook_dtype=lv.LVQ_F32), cfg(n_loops=8)):
        for n in (0, 1, 32, 33, 3000):
            assert lib.lvq_encode(ctypes.byref(ce.c()), P, None, n, P, P, 1, 7, None) == OK
            assert lib.lvq_encode_kv(ctypes.byref(ce.c()), P, P, None, n, P, P, P, P, 0, 0, None) == OK
        st = (ctypes.c_int64 * 3)(9 * 512, 512, 128)
        assert lib.lvq_encode(ctypes.byref(ce.c()), P, st, 40, P, P, 0, 0, None) == OK
    sc = cfg()
    assert lib.lvq_encode_screen(ctypes.byref(sc.c()), P, None, 64, P, P, 0, 0, P, None) == OK
    assert lib.lvq_encode_screen(ctypes.byref(sc.c()), P, None, 64, P, P, 0, 0, None, None) != OK
    assert lib.lvq_encode(ctypes.byref(sc.c()), P, None, 4996, P, P, 0, 5, None) != OK
    assert lib.lvq_stub_counts(2) == 0, "a launch got arguments that break its invariants"


if __name__ == "__main__":
    drive_oracle(sys.argv[1])
    drive_host(sys.argv[2])
    print("sanitized drive ok", flush=True)

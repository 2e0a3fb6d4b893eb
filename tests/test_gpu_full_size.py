"""Full-size GPU parity at the workloads' own sizes (MI355X).

* prefill encode, 32768 tokens x 16 KV heads x 4 loop steps x 128 channels,
  K and V in one lvq_encode_kv launch: every index bit-exact against the CPU
  oracle's encoding of the same inputs (0.5 bit, G = 16, and 0.25 bit,
  G = 32);
* decode attention over those caches (a 32768-token context, 16 heads, the
  launch configuration the benchmark times) at every loop step, with the
  oracle fed the oracle's own index caches;
* batch 64 with ragged contexts (2048 + U{4096, 8192, 16384}): every one of
  the 64 x 16 (sequence, head) rows at every loop step.

Bars: bit-exact indices; decode rows within 2e-3 (max_ch |gpu - oracle| /
max_ch |oracle|).  The oracle runs with all host threads (OpenMP; each unit
of work keeps its fixed order).
"""
import sys
import time

import numpy as np
import pytest
import torch

import oracle
from cases import rel_err_rows
from sub_bit_vq_amd import synth

pytestmark = pytest.mark.gpu
TOL = 2e-3
N_SINK, N_RECENT = 64, 256


@pytest.fixture(scope="module")
def lv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sub_bit_vq_amd import loopvq
    loopvq.library()
    return loopvq


def _note(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def _fill_windows(bufs, b, k, v, L):
    """bf16 sink and recent tokens of sequence b from token-major K/V"""
    sink, _, recent = synth.window_positions(L, N_SINK, N_RECENT)
    win = list(sink) + list(recent)
    slots = torch.tensor([synth.window_slot(p, N_SINK, N_RECENT) for p in win], device=k.device)
    pos = torch.tensor(win, device=k.device)
    bufs["k_window"][b][:, :, slots, :] = k[pos].permute(2, 1, 0, 3)
    bufs["v_window"][b][:, :, slots, :] = v[pos].permute(2, 1, 0, 3)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("G", [16, 32])
def test_prefill_32k_bit_exact_then_decode(lv, G):
    """Prefill encode of a 32768-token, 16-head context (K and V in one
    launch) equals the oracle's encoding bit for bit; decode attention over
    the encoded cache matches the oracle at all four loop steps."""
    dev = torch.device("cuda")
    N, H, d, Tc = 32768, 16, 128, 4
    seed = 2000 + G
    cfg = lv.Config(batch=1, n_heads=H, head_dim=d, loop_steps=Tc, group=G, max_tokens=N)
    _note(f"prefill G={G}: generate and encode on the GPU")
    k = synth.loop_correlated_kv(N, H, Tc, d, seed + 1, device=dev)
    v = synth.loop_correlated_kv(N, H, Tc, d, seed + 2, device=dev)
    kcb = synth.codebooks(H, d, Tc, G, seed + 3, device=dev)
    vcb = synth.codebooks(H, d, Tc, G, seed + 4, device=dev)
    bufs = lv.allocate(cfg, dev)
    lv.lvq_encode_kv(cfg, k, v, kcb, vcb, bufs["k_index"], bufs["v_index"], 0, 0)
    torch.cuda.synchronize()
    kh, vh, kcb_h, vcb_h = k.cpu(), v.cpu(), kcb.cpu(), vcb.cpu()
    refs = {}
    for name, x, cb in (("K", kh, kcb_h), ("V", vh, vcb_h)):
        t0 = time.perf_counter()
        refs[name] = oracle.encode(x, cb, n_heads=H, head_dim=d, loop_steps=Tc, group=G, t_max=N)
        _note(f"  oracle {name}: {time.perf_counter() - t0:.1f} s on {oracle.max_threads()} threads")
    for name, key in (("K", "k_index"), ("V", "v_index")):
        got = bufs[key].cpu().numpy()
        diff = int((got != refs[name]).sum())
        assert diff == 0, f"{name}: {diff} of {got.size} indices differ"
    _note(f"  {2 * N * H * (d // (G // Tc))} indices bit-exact")

    _fill_windows(bufs, 0, k, v, N)
    q = synth.queries(1, H, d, Tc, seed + 5, device=dev)
    ctx = torch.tensor([N], dtype=torch.int32, device=dev)
    kw, vw = bufs["k_window"].cpu(), bufs["v_window"].cpu()
    del k, v, kh, vh
    for t in range(Tc):
        lv.lvq_decode_attn(cfg, t, q[t].contiguous(), ctx, N, bufs["k_index"], bufs["v_index"],
                           kcb, vcb, bufs["k_window"], bufs["v_window"], bufs["workspace"],
                           bufs["out"])
        torch.cuda.synchronize()
        got = bufs["out"].double().cpu().numpy()
        ref = oracle.decode_attn(loop_step=t, q=q[t].cpu(), ctx_len=[N], k_index=refs["K"],
                                 v_index=refs["V"], k_codebook=kcb_h, v_codebook=vcb_h,
                                 k_window=kw, v_window=vw, n_sink=N_SINK, n_recent=N_RECENT,
                                 group=G)
        err = rel_err_rows(got, ref)
        _note(f"  decode t={t}: rel err {err:.2e}")
        assert err <= TOL, t


@pytest.mark.timeout(600)
def test_batch64_ragged_every_row(lv):
    """Batch 64, L_b = 2048 + U{4096, 8192, 16384}, 16 heads, d = 128,
    0.5 bit: all 64 x 16 rows at every loop step.  The VQ indices are drawn
    (uniform) so that the oracle can take them as input; windows hold
    loop-correlated bf16 tokens."""
    dev = torch.device("cuda")
    H, d, Tc, G = 16, 128, 4, 16
    S = d // (G // Tc)
    lengths = synth.ragged_lengths(64, seed=1003)
    B, T = len(lengths), max(lengths)
    seed = 300
    cfg = lv.Config(batch=B, n_heads=H, head_dim=d, loop_steps=Tc, group=G, max_tokens=T)
    bufs = lv.allocate(cfg, dev)
    kcb = synth.codebooks(H, d, Tc, G, seed + 1, device=dev)
    vcb = synth.codebooks(H, d, Tc, G, seed + 2, device=dev)
    q = synth.queries(B, H, d, Tc, seed + 3, device=dev)
    _note(f"batch 64 ragged: {sum(lengths)} tokens")
    for b, L in enumerate(lengths):
        bufs["k_index"][b, :, :L] = synth.random_indices((H, L, S), seed + 10 + 2 * b, device=dev)
        bufs["v_index"][b, :, :L] = synth.random_indices((H, L, S), seed + 11 + 2 * b, device=dev)
        k = synth.loop_correlated_kv(L, H, Tc, d, seed + 20 + 2 * b, device=dev)
        v = synth.loop_correlated_kv(L, H, Tc, d, seed + 21 + 2 * b, device=dev)
        _fill_windows(bufs, b, k, v, L)
        del k, v
    ctx = torch.tensor(lengths, dtype=torch.int32, device=dev)
    host = {key: bufs[key].cpu() for key in ("k_index", "v_index", "k_window", "v_window")}
    kcb_h, vcb_h = kcb.cpu(), vcb.cpu()
    for t in range(Tc):
        lv.lvq_decode_attn(cfg, t, q[t].contiguous(), ctx, T, bufs["k_index"], bufs["v_index"],
                           kcb, vcb, bufs["k_window"], bufs["v_window"], bufs["workspace"],
                           bufs["out"])
        torch.cuda.synchronize()
        got = bufs["out"].double().cpu().numpy()
        t0 = time.perf_counter()
        ref = oracle.decode_attn(loop_step=t, q=q[t].cpu(), ctx_len=lengths,
                                 k_index=host["k_index"], v_index=host["v_index"],
                                 k_codebook=kcb_h, v_codebook=vcb_h, k_window=host["k_window"],
                                 v_window=host["v_window"], n_sink=N_SINK, n_recent=N_RECENT,
                                 group=G)
        err = rel_err_rows(got, ref)
        _note(f"  t={t}: {B * H} rows, rel err {err:.2e} (oracle {time.perf_counter() - t0:.1f} s)")
        assert np.isfinite(got).all()
        assert err <= TOL, t

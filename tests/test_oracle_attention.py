"""Pins for the oracle's decode attention (dequantise, then attend in fp64).

Independent references: torch's ``scaled_dot_product_attention`` in fp64 on
the original (un-quantised) tokens, the closed form for a zero query (the
mean of the values), probabilities summing to one, and slice isolation (NaN
in codebook slices of other loop steps never reaches the output).  The
end-to-end case builds its VQ tokens from exact codewords, encodes them with
the oracle and must then reproduce dense attention over the original tokens
at every loop step, with the recent window wrapping around its ring.
"""
import numpy as np
import pytest
import torch

import oracle
from cases import make_cache, merge_loop_groups, oracle_encoder, sdpa_fp64
from sub_bit_vq_amd import synth

TOL = 1e-10


def _decode(c, t, sm_scale=1.0, **kw):
    return oracle.decode_attn(loop_step=t, q=c.q[t], ctx_len=c.lengths, k_index=c.k_index,
                              v_index=c.v_index, k_codebook=c.k_codebook,
                              v_codebook=c.v_codebook, k_window=c.k_window,
                              v_window=c.v_window, n_sink=c.n_sink, n_recent=c.n_recent,
                              group=c.group, sm_scale=sm_scale, vq_len=c.vq_len,
                              loop_steps=c.loop_steps, **kw)


def _dense_reference(c, t, sm_scale):
    ref = np.zeros((c.batch, c.n_heads, c.head_dim))
    for b, L in enumerate(c.lengths):
        for h in range(c.n_heads):
            if L == 0:
                continue
            ref[b, h] = sdpa_fp64(c.q[t, b, h], c.k_tokens[b][:L, h, t],
                                  c.v_tokens[b][:L, h, t], sm_scale).numpy()
    return ref


def check_attend_matches_sdpa(seed=0):
    g = torch.Generator().manual_seed(seed)
    for L, d, scale in ((1, 8, 1.0), (7, 16, 0.3), (300, 64, 1.0 / 8), (1000, 128, 2.0)):
        q = torch.randn(d, generator=g, dtype=torch.float64)
        K = torch.randn((L, d), generator=g, dtype=torch.float64)
        V = torch.randn((L, d), generator=g, dtype=torch.float64)
        out, p = oracle.attend(q.numpy(), K.numpy(), V.numpy(), scale, want_p=True)
        ref = sdpa_fp64(q, K, V, scale).numpy()
        assert np.allclose(out, ref, rtol=0, atol=TOL * max(1.0, np.abs(ref).max()))
        assert abs(p.sum() - 1.0) < 1e-12 and (p >= 0).all()


def check_windows_only(seed=1):
    """Every token in the bf16 windows (L <= 64 + 256): decode equals dense
    attention over the tokens of loop step t."""
    c = make_cache(batch=5, n_heads=2, head_dim=64, lengths=(1, 40, 64, 200, 320), seed=seed)
    for t in range(4):
        for scale in (1.0, 0.125):
            got = _decode(c, t, scale)
            ref = _dense_reference(c, t, scale)
            assert np.abs(got - ref).max() < TOL, (t, scale)


def check_end_to_end(seed=2, group=16, head_dim=64, cb_dtype=torch.bfloat16, vq_len=None,
                     lengths=(512, 321, 700, 2000)):
    """VQ tokens are exact codewords; the oracle encodes them; decode at
    every loop step equals dense attention over the original tokens (recent
    ring wraps for L > 64 + 256 + ...)."""
    B = len(lengths)
    c = make_cache(batch=B, n_heads=2, head_dim=head_dim, group=group, lengths=lengths,
                   seed=seed, codeword_tokens=True, cb_dtype=cb_dtype, vq_len=vq_len)
    # discard the drawn indices and re-derive them with the oracle encoder
    truth_k, truth_v = c.k_index.clone(), c.v_index.clone()
    c.k_index.zero_()
    c.v_index.zero_()
    enc = oracle_encoder(oracle, c.n_heads, c.head_dim, c.loop_steps, c.group)
    for b in range(B):
        r = c.vq_range(b)
        if len(r):
            enc(c.k_tokens[b][r.start:r.stop], c.k_codebook, c.k_index, b, r.start)
            enc(c.v_tokens[b][r.start:r.stop], c.v_codebook, c.v_index, b, r.start)
    assert torch.equal(c.k_index, truth_k) and torch.equal(c.v_index, truth_v)
    for t in range(c.loop_steps):
        got, p = _decode(c, t, 0.5, want_p=True)
        ref = _dense_reference(c, t, 0.5)
        assert np.abs(got - ref).max() < TOL * max(1.0, np.abs(ref).max()), t
        for b, L in enumerate(c.lengths):
            assert np.allclose(p[b, :, :L].sum(-1), 1.0, rtol=0, atol=1e-12)


def check_zero_query_mean(seed=3):
    """q = 0: uniform softmax, out = mean of the values of loop step t."""
    c = make_cache(batch=2, n_heads=1, head_dim=64, lengths=(900, 333), seed=seed,
                   codeword_tokens=True)
    c.q.zero_()
    for t in range(4):
        got = _decode(c, t)
        for b, L in enumerate(c.lengths):
            ref = c.v_tokens[b][:L, 0, t].double().mean(0).numpy()
            assert np.abs(got[b, 0] - ref).max() < TOL


def check_slice_isolation(seed=4):
    """NaN in every codebook slice t' != t leaves the step-t output finite and
    unchanged."""
    c = make_cache(batch=1, n_heads=2, head_dim=64, lengths=(600,), seed=seed,
                   codeword_tokens=True, cb_dtype=torch.float32)
    for t in range(4):
        clean = _decode(c, t)
        kcb, vcb = c.k_codebook.clone(), c.v_codebook.clone()
        for tp in range(4):
            if tp != t:
                c.k_codebook[tp] = float("nan")
                c.v_codebook[tp] = float("nan")
        dirty = _decode(c, t)
        c.k_codebook.copy_(kcb)
        c.v_codebook.copy_(vcb)
        assert np.isfinite(dirty).all() and np.array_equal(clean, dirty), t


def check_empty_and_single(seed=5):
    c = make_cache(batch=2, n_heads=1, head_dim=64, lengths=(1, 1), seed=seed)
    c.lengths[0] = 0
    got = _decode(c, 2)
    assert np.all(got[0] == 0.0)
    want = c.v_tokens[1][0, 0, 2].double().numpy()
    assert np.abs(got[1, 0] - want).max() < TOL


def check_gqa_end_to_end(seed=8):
    """Grouped-query attention: 6 query heads over 2 KV heads.  VQ tokens are
    exact codewords encoded by the oracle; at every loop step the decode equals
    torch's fp64 SDPA with ``enable_gqa`` (query head h reads KV head h // 3)
    over the original tokens, for window-only and wrapped-ring contexts."""
    lengths = (200, 700, 1500)
    c = make_cache(batch=3, n_heads=2, q_heads=6, head_dim=64, lengths=lengths, seed=seed,
                   codeword_tokens=True)
    for t in range(c.loop_steps):
        got = _decode(c, t, 0.5)
        for b, L in enumerate(lengths):
            q = c.q[t, b].double()[None, :, None, :]                    # [1][6][1][d]
            K = c.k_tokens[b][:L, :, t].double().permute(1, 0, 2)[None]  # [1][2][L][d]
            V = c.v_tokens[b][:L, :, t].double().permute(1, 0, 2)[None]
            ref = torch.nn.functional.scaled_dot_product_attention(
                q, K, V, scale=0.5, enable_gqa=True)[0, :, 0].numpy()
            assert np.abs(got[b] - ref).max() < TOL * max(1.0, np.abs(ref).max()), (t, b)


def check_loop_groups_end_to_end(seed=9):
    """A model with R = 8 loop steps over Tc = 4 (two index rows per token):
    two independently drawn single-group caches joined along the loop axis.
    The oracle encoder, given every loop step of the VQ tokens, must recover
    both groups' drawn indices, and decoding loop step r = 0..7 must equal
    fp64 SDPA over the original tokens at step r."""
    lengths = (300, 900, 1700)
    parts = [make_cache(batch=3, n_heads=2, head_dim=64, lengths=lengths, seed=seed + 31 * g,
                        codeword_tokens=True) for g in range(2)]
    c = merge_loop_groups(parts)
    truth_k, truth_v = c.k_index.clone(), c.v_index.clone()
    c.k_index.zero_()
    c.v_index.zero_()
    for b in range(c.batch):
        r = c.vq_range(b)
        if len(r):
            for tok, cb, idx in ((c.k_tokens, c.k_codebook, c.k_index),
                                 (c.v_tokens, c.v_codebook, c.v_index)):
                oracle.encode(tok[b][r.start:r.stop], cb, n_heads=2, head_dim=64, loop_steps=4,
                              group=16, n_loops=8, index=idx.numpy(), seq=b, first_token=r.start)
    assert torch.equal(c.k_index, truth_k) and torch.equal(c.v_index, truth_v)
    for step in range(8):
        got = _decode(c, step, 0.5)
        ref = _dense_reference(c, step, 0.5)
        assert np.abs(got - ref).max() < TOL * max(1.0, np.abs(ref).max()), step


def test_loop_groups_end_to_end():
    check_loop_groups_end_to_end()


def test_gqa_end_to_end():
    check_gqa_end_to_end()


def test_attend_matches_sdpa():
    check_attend_matches_sdpa()


def test_windows_only():
    check_windows_only()


@pytest.mark.parametrize("group,head_dim,cb_dtype", [(16, 64, torch.bfloat16),
                                                      (32, 128, torch.bfloat16),
                                                      (16, 64, torch.float32)])
def test_end_to_end(group, head_dim, cb_dtype):
    check_end_to_end(group=group, head_dim=head_dim, cb_dtype=cb_dtype)


def check_end_to_end_page_lag():
    """vq_len larger than the exact-window count (a recent page already
    encoded): VQ = [64, 64 + vq_len), recent = the rest, fewer than 256."""
    lengths = (700, 1000)
    exact = [L - 64 - 256 for L in lengths]
    check_end_to_end(seed=6, lengths=lengths, vq_len=[exact[0] + 8, exact[1] + 5])


def test_end_to_end_page_lag():
    check_end_to_end_page_lag()


def test_zero_query_mean():
    check_zero_query_mean()


def test_slice_isolation():
    check_slice_isolation()


def test_empty_and_single():
    check_empty_and_single()


def test_rejects_bad_preconditions():
    c = make_cache(batch=1, n_heads=1, head_dim=64, lengths=(500,), seed=7)
    with pytest.raises(ValueError):   # recent window would exceed n_recent
        oracle.decode_attn(loop_step=0, q=c.q[0], ctx_len=c.lengths, k_index=c.k_index,
                           v_index=c.v_index, k_codebook=c.k_codebook, v_codebook=c.v_codebook,
                           k_window=c.k_window, v_window=c.v_window, n_sink=64, n_recent=256,
                           group=16, vq_len=[10])
    with pytest.raises(ValueError):   # loop step out of range
        oracle.decode_attn(loop_step=4, q=c.q[0], ctx_len=c.lengths, k_index=c.k_index,
                           v_index=c.v_index, k_codebook=c.k_codebook, v_codebook=c.v_codebook,
                           k_window=c.k_window, v_window=c.v_window, n_sink=64, n_recent=256,
                           group=16)

"""The pages' loop-axis claim on synthetic data, with the CPU oracle as the
k-means assignment step (LoopVQ project page, "Component 1 -- Loop-axis
vector quantization": at the same bits per element, a codeword spanning
channels at several loop steps reconstructs a looped model's keys better than
one spanning channels of a single step, because a token's keys at consecutive
steps are near-copies).  The synthetic generator has exactly that structure
(a shared base plus small per-step noise), so the loop-axis grouping must win
clearly; channel-only grouping gets its own codebooks per loop step.
"""
import numpy as np
import torch

import oracle
from sub_bit_vq_amd import kmeans, synth


def oracle_assign(x, cb, group):
    N, H, Tc, d = x.shape
    idx = oracle.encode(x, cb, n_heads=H, head_dim=d, loop_steps=Tc, group=group)
    return idx[0].transpose(1, 0, 2)                                   # [N][H][S]


def test_channel_view_holds_one_steps_channels():
    x = synth.loop_correlated_kv(5, 2, 4, 64, seed=1)
    for step in range(4):
        for G in (16, 32):
            sub = kmeans.natural_subvectors(kmeans.channel_view(x, step, G), G)   # [N][H][S][G]
            want = x[:, :, step, :].reshape(5, 2, 64 // G, G)
            assert torch.equal(sub, want)


def test_codebook_layout_round_trip():
    cb = synth.codebooks(2, 64, 4, 16, seed=2)
    assert torch.equal(kmeans.storage_codebook(kmeans.natural_codebook(cb), 4), cb)


def test_lloyd_iterations_do_not_increase_error():
    """Exact nearest-codeword assignment and fp64 means (fp32 codebooks):
    Lloyd's training error never rises (up to the fp32 rounding of codes)."""
    x = synth.loop_correlated_kv(600, 1, 4, 64, seed=3)
    _, hist = kmeans.fit_codebooks(x, 16, 6, seed=4, assign=oracle_assign, dtype=torch.float32)
    assert all(b <= a * (1 + 1e-6) for a, b in zip(hist, hist[1:])), hist
    assert hist[-1] < hist[0]


def test_loop_axis_beats_channels_at_equal_bits():
    """0.5 bit per element (G = 16): 4 channels x 4 loop steps against 16
    channels x 1 step, fitted on 1024 tokens, measured on 256 others."""
    x = synth.loop_correlated_kv(1280, 1, 4, 64, seed=5)
    r = kmeans.loop_axis_comparison(x[:1024], x[1024:], 16, 5, seed=6, assign=oracle_assign)
    assert r["bits_per_element"] == 0.5
    assert r["mse_loop_axis"] < 0.5 * r["mse_channels_only"], r

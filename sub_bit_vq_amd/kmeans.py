"""Codebook fitting for LoopVQ by k-means, with the encoder as the assignment step.

LoopVQ project page, "Component 1 -- Loop-axis vector quantization": a
codeword covers G/Tc channels at each of Tc consecutive loop steps, so that
the near-copies a looped model writes at consecutive steps share one index.
The pages learn their codebooks (and fine-tune the model, which is out of scope
here).  This module fits codebooks to a sample of keys or values with Lloyd's
k-means, which is enough to repeat the section's equal-bits comparison --
grouping along the loop axis against grouping along channels only -- on
synthetic data:

* assignment: the nearest codeword exactly as the encoder defines it, through
  an ``assign`` callable (by default :func:`device_assign`, i.e. ``lvq_encode``
  on the GPU);
* update: each code becomes the mean of the sub-vectors assigned to it,
  summed in fp64 on the host in token order and rounded once to the codebook
  dtype; a code with no sub-vector keeps its codeword;
* initialisation: 256 distinct training sub-vectors per (head, sub-vector),
  drawn with a seeded generator.

Given the inputs and the seed everything is deterministic, so two assignment
implementations that agree bit for bit produce identical codebooks.

Channel-only grouping (16 channels of one loop step per index at G = 16) is
run through the same encoder by viewing the step's 16 channels as 4 pseudo
steps of 4 channels (:func:`channel_view`): the sub-vector's elements are then
exactly those channels in order.
"""
from __future__ import annotations

import time

import numpy as np
import torch

N_CODES = 256


def natural_subvectors(x: torch.Tensor, group: int) -> torch.Tensor:
    """``[N][H][Tc][d]`` -> ``[N][H][S][G]``: entry ``i = t*cg + c`` of
    sub-vector j is ``x[n][h][t][j*cg + c]``."""
    N, H, Tc, d = x.shape
    cg = group // Tc
    S = d // cg
    return x.reshape(N, H, Tc, S, cg).permute(0, 1, 3, 2, 4).reshape(N, H, S, group)


def storage_codebook(nat: torch.Tensor, loop_steps: int) -> torch.Tensor:
    """Natural ``[H][S][256][G]`` -> the library's ``[Tc][H][256][S][cg]``."""
    H, S, K, G = nat.shape
    return nat.reshape(H, S, K, loop_steps, G // loop_steps).permute(3, 0, 2, 1, 4).contiguous()


def natural_codebook(cb: torch.Tensor) -> torch.Tensor:
    """The library's ``[Tc][H][256][S][cg]`` -> natural ``[H][S][256][G]``."""
    Tc, H, K, S, cg = cb.shape
    return cb.permute(1, 3, 2, 0, 4).reshape(H, S, K, Tc * cg)


def channel_view(x: torch.Tensor, step: int, channels: int, pieces: int = 4) -> torch.Tensor:
    """Loop step ``step`` of ``x [N][H][R][d]`` as ``[N][H][pieces][d/pieces]``
    such that sub-vector j of group ``channels`` (``pieces`` pseudo steps of
    ``channels/pieces`` channels) holds channels ``[j*channels, (j+1)*channels)``
    of that step in order."""
    N, H, R, d = x.shape
    cg = channels // pieces
    y = x[:, :, step, :].reshape(N, H, d // channels, pieces, cg)
    return y.permute(0, 1, 3, 2, 4).reshape(N, H, pieces, d // pieces).contiguous()


def device_assign(lv, device="cuda"):
    """Assignment step through ``lvq_encode``: ``assign(x, cb, group)`` with
    host ``x [N][H][Tc][d]`` bf16 and ``cb`` in the library layout returns the
    codes as a host ``uint8 [N][H][S]`` array."""
    def assign(x, cb, group):
        N, H, Tc, d = x.shape
        S = d // (group // Tc)
        cfg = lv.Config(batch=1, n_heads=H, head_dim=d, loop_steps=Tc, group=group,
                        max_tokens=N,
                        codebook_dtype=lv.LVQ_BF16 if cb.dtype == torch.bfloat16 else lv.LVQ_F32)
        idx = torch.empty((1, H, N, S), dtype=torch.uint8, device=device)
        lv.lvq_encode(cfg, x.to(device), cb.to(device), idx)
        return idx[0].permute(1, 0, 2).cpu().numpy()
    return assign


def _update(xs: np.ndarray, idx: np.ndarray, old: np.ndarray) -> np.ndarray:
    """Mean of the sub-vectors of every code (fp64, token order); codes with
    none keep ``old``.  xs [N][H][S][G], idx [N][H][S], old [H][S][256][G]."""
    N, H, S, G = xs.shape
    slot = ((np.arange(H)[None, :, None] * S + np.arange(S)[None, None, :]) * N_CODES
            + idx.astype(np.int64)).ravel()
    n_slots = H * S * N_CODES
    counts = np.bincount(slot, minlength=n_slots)
    flat = xs.reshape(-1, G)
    sums = np.stack([np.bincount(slot, weights=flat[:, i], minlength=n_slots) for i in range(G)], -1)
    new = old.reshape(n_slots, G).copy()
    used = counts > 0
    new[used] = sums[used] / counts[used, None]
    return new.reshape(H, S, N_CODES, G)


def fit_codebooks(x: torch.Tensor, group: int, iters: int, seed: int, assign,
                  dtype=torch.bfloat16):
    """Lloyd's k-means on host ``x [N][H][Tc][d]`` (bf16, N >= 256): returns
    the codebooks in the library layout (``dtype``) and the training error
    (mean squared error per element) after every assignment."""
    N, H, Tc, d = x.shape
    if N < N_CODES:
        raise ValueError("k-means needs at least 256 training tokens")
    xs = natural_subvectors(x.float(), group).double().numpy()     # [N][H][S][G]
    S = xs.shape[2]
    rng = np.random.default_rng(seed)
    pick = np.stack([rng.choice(N, N_CODES, replace=False) for _ in range(H * S)])
    nat = xs[pick.reshape(H, S, N_CODES), np.arange(H)[:, None, None], np.arange(S)[None, :, None]]
    nat_t = torch.from_numpy(nat).to(dtype)
    history = []
    for _ in range(iters):
        cb = storage_codebook(nat_t, Tc)
        idx = assign(x, cb, group)
        rec = nat_t.double().numpy()[np.arange(H)[None, :, None], np.arange(S)[None, None, :], idx]
        history.append(float(((rec - xs) ** 2).mean()))
        nat_t = torch.from_numpy(_update(xs, idx, nat_t.double().numpy())).to(dtype)
    return storage_codebook(nat_t, Tc), history


def reconstruction_mse(x: torch.Tensor, cb: torch.Tensor, group: int, assign) -> float:
    """Mean squared error per element of encoding ``x`` with ``cb`` and
    reading it back (every loop step of every sub-vector)."""
    xs = natural_subvectors(x.float(), group).double().numpy()
    N, H, S, G = xs.shape
    nat = natural_codebook(cb).double().numpy()
    idx = assign(x, cb, group)
    rec = nat[np.arange(H)[None, :, None], np.arange(S)[None, None, :], idx]
    return float(((rec - xs) ** 2).mean())


def loop_axis_comparison(x_train: torch.Tensor, x_test: torch.Tensor, group: int, iters: int,
                         seed: int, assign, dtype=torch.bfloat16) -> dict:
    """Equal bits per element (8 / group), two groupings of the same data
    ``[N][H][Tc][d]``:

    * loop axis: group/Tc channels at each of the Tc loop steps per index;
    * channels only: ``group`` channels of one loop step per index, with its
      own codebooks per loop step.

    Returns test-set errors (mean squared error per element), the training
    error histories and the wall time of the fits."""
    Tc = x_train.shape[2]
    t0 = time.perf_counter()
    cb_loop, hist_loop = fit_codebooks(x_train, group, iters, seed, assign, dtype)
    t1 = time.perf_counter()
    mse_loop = reconstruction_mse(x_test, cb_loop, group, assign)
    mse_ch, hist_ch = [], []
    t2 = time.perf_counter()
    for step in range(Tc):
        tr = channel_view(x_train, step, group)
        te = channel_view(x_test, step, group)
        cb, h = fit_codebooks(tr, group, iters, seed + 1 + step, assign, dtype)
        hist_ch.append(h)
        mse_ch.append(reconstruction_mse(te, cb, group, assign))
    t3 = time.perf_counter()
    return {
        "bits_per_element": 8.0 / group,
        "mse_loop_axis": mse_loop,
        "mse_channels_only": float(np.mean(mse_ch)),
        "mse_channels_only_per_step": mse_ch,
        "train_history_loop_axis": hist_loop,
        "train_history_channels_only": hist_ch,
        "fit_seconds_loop_axis": t1 - t0,
        "fit_seconds_channels_only": t3 - t2,
    }

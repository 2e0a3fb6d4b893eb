"""Seeded synthetic inputs for the LoopVQ decode-attention and encoder paths.

This module holds no LoopVQ arithmetic (no distances, no dequantisation, no
attention): only seeded random draws, rounding to bf16 and the storage layout
of the tensors the library consumes.  Both the HIP library and the CPU oracle
receive tensors produced here; the oracle always gets host copies of exactly
the tensors the device path sees.

Workload model (stand-in for the looped-LM caches the LoopVQ pages measure,
whose keys of one head look alike at every loop step -- LoopVQ project page,
"Method", redundancy figure):

* key/value of token n, head h, loop step l, channel ch:
  ``base[n][h][ch] + noise_l``, ``base ~ N(0, 1)`` shared by all loop steps of
  the token and ``noise_l ~ N(0, sigma_l^2)`` with ``sigma_l = 0.1 (l + 1)``
  (standard deviation), rounded to bf16 with round-to-nearest-even;
* codebooks: one 256 x G table per (head, sub-vector), entries ``N(0, 1)``,
  kept in fp32 or rounded to bf16;
* queries: ``N(0, 1) / sqrt(head_dim)`` in bf16, one independent draw per loop
  step;
* ragged batches: ``2048 + U{4096, 8192, 16384}`` context tokens per sequence.

Random streams come from ``torch.Generator`` seeded per (workload, tensor);
on the CPU for test-sized inputs, on the device for full-size workloads.
"""
from __future__ import annotations

import math

import torch

N_CODES = 256


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(int(seed))
    return g


def loop_correlated_kv(n_tokens: int, n_heads: int, loop_steps: int, head_dim: int,
                       seed: int, device="cpu") -> torch.Tensor:
    """bf16 tensor ``[n_tokens][n_heads][loop_steps][head_dim]``."""
    g = _gen(seed, device)
    base = torch.randn((n_tokens, n_heads, 1, head_dim), generator=g, device=device,
                       dtype=torch.float32)
    noise = torch.randn((n_tokens, n_heads, loop_steps, head_dim), generator=g,
                        device=device, dtype=torch.float32)
    sigma = 0.1 * torch.arange(1, loop_steps + 1, device=device, dtype=torch.float32)
    x = base + noise * sigma.view(1, 1, loop_steps, 1)
    return x.to(torch.bfloat16)


def codebooks(n_heads: int, head_dim: int, loop_steps: int, group: int, seed: int,
              dtype=torch.bfloat16, device="cpu") -> torch.Tensor:
    """Codebooks in the slice-major, code-major storage layout
    ``[loop_steps][n_heads][256][n_sub][group // loop_steps]``.

    Codeword k of (head h, sub-vector j) has ``group`` entries; entry
    ``i = t * cg + c`` (``cg = group // loop_steps``) is stored at
    ``[t][h][k][j][c]``: the part read at loop step t is contiguous, and within
    it row k holds code k of every sub-vector.  Draw order is the natural one,
    ``[h][j][k][i]``.
    """
    cg = group // loop_steps
    n_sub = head_dim // cg
    g = _gen(seed, device)
    nat = torch.randn((n_heads, n_sub, N_CODES, loop_steps, cg), generator=g,
                      device=device, dtype=torch.float32)
    return nat.to(dtype).permute(3, 0, 2, 1, 4).contiguous()


def queries(batch: int, n_heads: int, head_dim: int, loop_steps: int, seed: int,
            device="cpu") -> torch.Tensor:
    """bf16 ``[loop_steps][batch][n_heads][head_dim]``, ``N(0,1)/sqrt(head_dim)``."""
    g = _gen(seed, device)
    q = torch.randn((loop_steps, batch, n_heads, head_dim), generator=g, device=device,
                    dtype=torch.float32)
    return (q / math.sqrt(head_dim)).to(torch.bfloat16)


def ragged_lengths(batch: int, seed: int, prompt: int = 2048,
                   generated=(4096, 8192, 16384)) -> list[int]:
    """Per-sequence context lengths: prompt plus a generated length drawn
    uniformly from ``generated``."""
    g = _gen(seed, "cpu")
    pick = torch.randint(0, len(generated), (batch,), generator=g)
    return [prompt + generated[int(i)] for i in pick]


def random_indices(shape, seed: int, device="cpu") -> torch.Tensor:
    """Uniform random uint8 codes (used where a cache is drawn directly)."""
    g = _gen(seed, device)
    return torch.randint(0, N_CODES, tuple(shape), generator=g, device=device,
                         dtype=torch.uint8)


# --------------------------------------------------------------------------
# Window storage layout (bf16 sink + recent tokens).
#
# Window buffer: [batch][loop_steps][n_heads][n_sink + n_recent][head_dim].
# Sink token p (p < n_sink) lives in slot p.  Recent token p (p >= n_sink)
# lives in slot n_sink + ((p - n_sink) mod n_recent): a ring, so a slot is
# reused once the token it held has left the recent window.
# --------------------------------------------------------------------------

def window_slot(p: int, n_sink: int, n_recent: int) -> int:
    if p < n_sink:
        return p
    return n_sink + (p - n_sink) % n_recent


def window_positions(length: int, n_sink: int, n_recent: int, vq_len=None):
    """(sink positions, vq positions, recent positions) of a context of
    ``length`` tokens; ``vq_len=None`` means exact windows."""
    n_s = min(length, n_sink)
    if vq_len is None:
        n_v = max(0, length - n_sink - n_recent)
    else:
        n_v = int(vq_len)
    return (range(0, n_s), range(n_s, n_s + n_v), range(n_s + n_v, length))


def fill_window(window: torch.Tensor, b: int, tokens: torch.Tensor, length: int,
                n_sink: int, n_recent: int, vq_len=None) -> None:
    """Write the bf16 K or V of the sink and recent tokens of sequence ``b``.

    ``tokens``: ``[>= length][n_heads][loop_steps][head_dim]`` (token-major, as
    produced by :func:`loop_correlated_kv`); ``window``: the window buffer.
    """
    sink, _, recent = window_positions(length, n_sink, n_recent, vq_len)
    for rng in (sink, recent):
        if len(rng) == 0:
            continue
        pos = torch.tensor(list(rng), dtype=torch.long)
        slots = torch.tensor([window_slot(int(p), n_sink, n_recent) for p in rng],
                             dtype=torch.long)
        src = tokens[pos.to(tokens.device)]                 # [n][H][Tc][d]
        window[b][:, :, slots.to(window.device), :] = src.permute(2, 1, 0, 3).to(window.dtype)

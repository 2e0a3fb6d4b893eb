"""Test-case construction shared by the oracle pins and the GPU parity tests.

Nothing here computes an expected value: these helpers only assemble inputs
(seeded draws from ``sub_bit_vq_amd.synth`` plus plain indexing), and the
dense fp64 attention that pins the oracle comes from torch's own
``scaled_dot_product_attention``.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch
import torch.nn.functional as F

from sub_bit_vq_amd import synth

N_SINK, N_RECENT = 64, 256


def natural_codebook(cb: torch.Tensor) -> torch.Tensor:
    """[Tc][H][256][S][cg] storage -> [H][S][256][G] with entry i = t*cg + c."""
    Tc, H, K, S, cg = cb.shape
    return cb.permute(1, 3, 2, 0, 4).reshape(H, S, K, Tc * cg)


def natural_subvectors(x: torch.Tensor, group: int) -> torch.Tensor:
    """x [n][H][Tc][d] -> [n][H][S][G] with entry i = t*cg + c of sub-vector j
    taken from channel j*cg + c of loop step t."""
    n, H, Tc, d = x.shape
    cg = group // Tc
    S = d // cg
    return x.reshape(n, H, Tc, S, cg).permute(0, 1, 3, 2, 4).reshape(n, H, S, Tc * cg)


def kv_from_codewords(idx: torch.Tensor, cb: torch.Tensor) -> torch.Tensor:
    """Tokens whose every sub-vector is exactly a codeword.

    idx uint8 [n][H][S]; cb [Tc][H][256][S][cg] -> x [n][H][Tc][d] (cb dtype)."""
    Tc, H, K, S, cg = cb.shape
    n = idx.shape[0]
    hh = torch.arange(H).view(1, H, 1)
    jj = torch.arange(S).view(1, 1, S)
    rows = [cb[t][hh, idx.long(), jj] for t in range(Tc)]      # each [n][H][S][cg]
    return torch.stack(rows, dim=2).reshape(n, H, Tc, S * cg)


def bf16_representable_fp32(cb: torch.Tensor) -> torch.Tensor:
    """fp32 codebook whose entries are exactly bf16 values (so bf16 tokens can
    equal codewords)."""
    return cb.to(torch.bfloat16).to(torch.float32)


def sdpa_fp64(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, scale: float) -> torch.Tensor:
    """Dense attention from torch (CPU, fp64): q [d], K/V [L][d] -> [d]."""
    q64 = q.to(torch.float64).view(1, 1, 1, -1)
    K64 = K.to(torch.float64).view(1, 1, K.shape[0], -1)
    V64 = V.to(torch.float64).view(1, 1, V.shape[0], -1)
    return F.scaled_dot_product_attention(q64, K64, V64, scale=scale).view(-1)


@dataclass
class Cache:
    """A complete decode-attention test case (host tensors).  ``n_heads`` is the
    number of KV heads (index caches, codebooks, windows, tokens); the query has
    ``q_heads`` heads (0: as many), query head h reading KV head
    h // (q_heads // n_heads)."""
    batch: int
    n_heads: int
    head_dim: int
    loop_steps: int
    group: int
    t_max: int
    lengths: list
    vq_len: list | None
    q: torch.Tensor            # bf16 [Tc][B][Hq][d]
    k_tokens: list             # per sequence bf16 [L][H][Tc][d] (original tokens)
    v_tokens: list
    k_index: torch.Tensor      # uint8 [B][H][t_max][S]
    v_index: torch.Tensor
    k_codebook: torch.Tensor   # [Tc][H][256][S][cg]
    v_codebook: torch.Tensor
    k_window: torch.Tensor     # bf16 [B][Tc][H][n_sink+n_recent][d]
    v_window: torch.Tensor
    n_sink: int = N_SINK
    n_recent: int = N_RECENT
    extra: dict = field(default_factory=dict)
    q_heads: int = 0
    n_loops: int = 0          # R > loop_steps: index caches [R/Tc][B][H][t_max][S]

    @property
    def n_q_heads(self):
        return self.q_heads or self.n_heads

    @property
    def n_sub(self):
        return self.head_dim // (self.group // self.loop_steps)

    def vq_range(self, b):
        return synth.window_positions(self.lengths[b], self.n_sink, self.n_recent,
                                      None if self.vq_len is None else self.vq_len[b])[1]


def make_cache(*, batch=1, n_heads=1, head_dim=64, loop_steps=4, group=16, lengths=(512,),
               cb_dtype=torch.bfloat16, seed=0, codeword_tokens=False, vq_len=None,
               encode=None, t_max=None, n_sink=N_SINK, n_recent=N_RECENT, q_heads=None) -> Cache:
    """Seeded cache.  VQ tokens either come from the loop-correlated generator
    and are encoded with ``encode(x, codebook, index, seq, first_token)``, or
    (``codeword_tokens=True``) are drawn as exact codewords of random indices,
    in which case the index cache holds those indices directly."""
    lengths = list(lengths)
    assert len(lengths) == batch
    cg = group // loop_steps
    S = head_dim // cg
    t_max = t_max or max(max(lengths), 1)
    kcb = synth.codebooks(n_heads, head_dim, loop_steps, group, seed * 7919 + 1, dtype=cb_dtype)
    vcb = synth.codebooks(n_heads, head_dim, loop_steps, group, seed * 7919 + 2, dtype=cb_dtype)
    if cb_dtype == torch.float32 and codeword_tokens:
        kcb, vcb = bf16_representable_fp32(kcb), bf16_representable_fp32(vcb)
    q = synth.queries(batch, q_heads or n_heads, head_dim, loop_steps, seed * 7919 + 3)
    k_index = torch.zeros((batch, n_heads, t_max, S), dtype=torch.uint8)
    v_index = torch.zeros_like(k_index)
    W = n_sink + n_recent
    k_window = torch.zeros((batch, loop_steps, n_heads, W, head_dim), dtype=torch.bfloat16)
    v_window = torch.zeros_like(k_window)
    k_tokens, v_tokens = [], []
    for b, L in enumerate(lengths):
        kt = synth.loop_correlated_kv(L, n_heads, loop_steps, head_dim, seed * 7919 + 100 + 2 * b)
        vt = synth.loop_correlated_kv(L, n_heads, loop_steps, head_dim, seed * 7919 + 101 + 2 * b)
        vql = None if vq_len is None else vq_len[b]
        vq = synth.window_positions(L, n_sink, n_recent, vql)[1]
        if len(vq):
            lo, hi = vq.start, vq.stop
            if codeword_tokens:
                ik = synth.random_indices((hi - lo, n_heads, S), seed * 7919 + 500 + 2 * b)
                iv = synth.random_indices((hi - lo, n_heads, S), seed * 7919 + 501 + 2 * b)
                kt[lo:hi] = kv_from_codewords(ik, kcb).to(torch.bfloat16)
                vt[lo:hi] = kv_from_codewords(iv, vcb).to(torch.bfloat16)
                k_index[b, :, lo:hi] = ik.permute(1, 0, 2)
                v_index[b, :, lo:hi] = iv.permute(1, 0, 2)
            elif encode is not None:
                encode(kt[lo:hi], kcb, k_index, b, lo)
                encode(vt[lo:hi], vcb, v_index, b, lo)
        synth.fill_window(k_window, b, kt, L, n_sink, n_recent, vql)
        synth.fill_window(v_window, b, vt, L, n_sink, n_recent, vql)
        k_tokens.append(kt)
        v_tokens.append(vt)
    return Cache(batch, n_heads, head_dim, loop_steps, group, t_max, lengths, vq_len, q,
                 k_tokens, v_tokens, k_index, v_index, kcb, vcb, k_window, v_window,
                 n_sink, n_recent, q_heads=q_heads or 0)


def merge_loop_groups(caches) -> Cache:
    """One cache of a model with R = len(caches) * Tc loop steps from caches
    built for Tc steps each (same shapes and lengths): tokens, queries,
    codebooks and windows are joined along the loop axis, index caches are
    stacked as groups [R/Tc][B][H][t_max][S]."""
    c0 = caches[0]
    cat = lambda key, dim: torch.cat([getattr(c, key) for c in caches], dim)  # noqa: E731
    merged = Cache(c0.batch, c0.n_heads, c0.head_dim, c0.loop_steps, c0.group, c0.t_max,
                   list(c0.lengths), c0.vq_len, cat("q", 0),
                   [torch.cat([c.k_tokens[b] for c in caches], 2) for b in range(c0.batch)],
                   [torch.cat([c.v_tokens[b] for c in caches], 2) for b in range(c0.batch)],
                   torch.stack([c.k_index for c in caches]), torch.stack([c.v_index for c in caches]),
                   cat("k_codebook", 0), cat("v_codebook", 0), cat("k_window", 1),
                   cat("v_window", 1), c0.n_sink, c0.n_recent, q_heads=c0.q_heads,
                   n_loops=len(caches) * c0.loop_steps)
    return merged


def oracle_encoder(oracle_mod, n_heads, head_dim, loop_steps, group):
    """encode(x, cb, index, seq, first) callback running the CPU oracle in place."""
    def enc(x, cb, index, seq, first):
        arr = index.numpy()
        oracle_mod.encode(x, cb, n_heads=n_heads, head_dim=head_dim, loop_steps=loop_steps,
                          group=group, index=arr, seq=seq, first_token=first)
    return enc


def rel_err_rows(got: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of max_ch |got - ref| / max_ch |ref| (rows = leading dims)."""
    got = np.asarray(got, np.float64).reshape(-1, got.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    num = np.abs(got - ref).max(axis=1)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return float((num / den).max()) if num.size else 0.0


# ---------------------------------------------------------------------------
# Device-side helpers for the GPU parity tests (HIP library through the
# binding; expected values always come from the oracle on host copies).
# ---------------------------------------------------------------------------

def lvq_config(lv, c: Cache, **kw):
    kw.setdefault("n_kv_heads", c.n_heads if c.n_q_heads != c.n_heads else 0)
    kw.setdefault("n_loops", c.n_loops)
    return lv.Config(batch=c.batch, n_heads=c.n_q_heads, head_dim=c.head_dim,
                     loop_steps=c.loop_steps, group=c.group, n_sink=c.n_sink,
                     n_recent=c.n_recent, max_tokens=c.t_max,
                     codebook_dtype=lv.LVQ_BF16 if c.k_codebook.dtype == torch.bfloat16
                     else lv.LVQ_F32, **kw)


class DeviceCache:
    """Device copies of a :class:`Cache` plus output and workspace."""

    def __init__(self, lv, c: Cache, device="cuda", **cfg_kw):
        self.lv = lv
        self.c = c
        self.cfg = lvq_config(lv, c, **cfg_kw)
        d = device
        self.q = c.q.to(d)
        self.ctx = torch.tensor(c.lengths, dtype=torch.int32, device=d)
        self.vq = None if c.vq_len is None else torch.tensor(c.vq_len, dtype=torch.int32, device=d)
        self.k_index, self.v_index = c.k_index.to(d), c.v_index.to(d)
        self.k_cb, self.v_cb = c.k_codebook.to(d), c.v_codebook.to(d)
        self.k_win, self.v_win = c.k_window.to(d), c.v_window.to(d)
        bufs = lv.allocate(self.cfg, d)
        self.out, self.ws = bufs["out"], bufs["workspace"]

    def decode(self, t, sm_scale=1.0, cfg=None, max_ctx=None):
        cfg = cfg or self.cfg
        self.lv.lvq_decode_attn(cfg, t, self.q[t].contiguous(), self.ctx,
                                max(self.c.lengths) if max_ctx is None else max_ctx,
                                self.k_index, self.v_index, self.k_cb, self.v_cb, self.k_win,
                                self.v_win, self.ws, self.out, sm_scale=sm_scale, vq_len=self.vq)
        torch.cuda.synchronize()
        return self.out.double().cpu().numpy()


def oracle_decode(oracle_mod, c: Cache, t, sm_scale=1.0, heads=None):
    return oracle_mod.decode_attn(loop_step=t, q=c.q[t], ctx_len=c.lengths, k_index=c.k_index,
                                  v_index=c.v_index, k_codebook=c.k_codebook,
                                  v_codebook=c.v_codebook, k_window=c.k_window,
                                  v_window=c.v_window, n_sink=c.n_sink, n_recent=c.n_recent,
                                  group=c.group, sm_scale=sm_scale, vq_len=c.vq_len, heads=heads,
                                  loop_steps=c.loop_steps)


def rounding_order_case(H, d, Tc, G, n, cb_dtype, seed, n_base=4):
    """Codebooks whose 256 codes of each (head, sub-vector) are permutations
    of ``n_base`` base vectors, and inputs whose rows are constant (one level
    per token).  The exact distances of sibling codes coincide, so the winner
    is decided by the fp32 rounding of each term and by the summation order:
    an implementation that fuses the square into the add, or sums in another
    order, picks a different code on many sub-vectors.  Returns (x, cb)."""
    g = torch.Generator().manual_seed(seed)
    cg = G // Tc
    S = d // cg
    base = torch.randn((H, S, n_base, G), generator=g)
    if cb_dtype == torch.bfloat16:
        base = (0.25 * base).to(torch.bfloat16).float()
    rows = base[:, :, torch.arange(256) % n_base]                       # [H][S][256][G]
    perm = torch.argsort(torch.rand((H, S, 256, G), generator=g), dim=-1)
    nat = torch.gather(rows, -1, perm)
    cb = nat.reshape(H, S, 256, Tc, cg).permute(3, 0, 2, 1, 4).contiguous().to(cb_dtype)
    if cb_dtype == torch.bfloat16:
        levels = 1.0 + torch.arange(n, dtype=torch.float32) * 2.0 ** -7
    else:
        levels = torch.arange(n, dtype=torch.float32) * 2.0 ** -6
    x = levels[:, None, None, None].expand(n, H, Tc, d).to(torch.bfloat16).contiguous()
    return x, cb


def fp32_sequential_argmin(xs: np.ndarray, cn: np.ndarray, fused: bool = False) -> np.ndarray:
    """Nearest code by an independent numpy evaluation of the fp32 distance:
    xs [..., G] float32 sub-vectors, cn [256][G] float32 codes (broadcast over
    the leading axes of xs as [..., 256, G]).  Each step rounds to fp32;
    ``fused=True`` instead rounds e*e + acc once (what a fused multiply-add
    would give), to show that a case tells the two apart."""
    acc = np.zeros(xs.shape[:-1] + (cn.shape[-2],), np.float32)
    for i in range(xs.shape[-1]):
        e = (xs[..., i][..., None] - cn[..., i]).astype(np.float32)
        if fused:
            acc = (acc.astype(np.float64) + e.astype(np.float64) ** 2).astype(np.float32)
        else:
            acc = (acc + (e * e).astype(np.float32)).astype(np.float32)
    return acc.argmin(-1)          # numpy returns the first (lowest) index on ties


# fp16 rounding of a token weight (round to nearest: relative error <= 2^-11)
# plus the fp32 summation order of a token's score (which lane, and so which
# order, adds a token's table entries depends on the split: ~1e-6 relative)
WEIGHT_ROUNDING = 2.0 ** -11 + 2e-6


def weight_rounding_bound(c: Cache, t: int, ref: np.ndarray) -> np.ndarray:
    """Per (b, h, ch): how far two decodes of the same cache may differ when
    they split the tokens differently (split counts, token order).  The kernel
    rounds each token weight p_n to fp16 (relative error u) and divides by the
    sum of the same rounded weights, so its output is the exact weighted mean
    of the values with weights p_n (1 + d_n), |d_n| <= u:
        o - o* = sum_n p_n d_n (v_n - o*) / sum_n p_n (1 + d_n),
        |o - o*| <= u / (1 - u) * max_n |v_n - o*|,
    and two such outputs differ by at most twice that.  Needs a cache whose
    tokens are the values attended (exact windows; codeword VQ tokens), and
    the oracle's output ``ref`` for o*."""
    u = WEIGHT_ROUNDING
    Hq, Hk = c.n_q_heads, c.n_heads
    out = np.zeros(ref.shape, np.float64)
    for b, L in enumerate(c.lengths):
        if L == 0:
            continue
        V = c.v_tokens[b][:L, :, t, :].double().numpy()         # [L][Hk][d]
        for h in range(Hq):
            spread = np.abs(V[:, h // (Hq // Hk), :] - ref[b, h][None, :]).max(axis=0)
            out[b, h] = 2.0 * u / (1.0 - u) * spread + 1e-6 * np.abs(ref[b, h]).max()
    return out

"""Pins for the oracle's encoder (nearest codeword, lowest index on ties).

Each check is independent of the oracle's own loop: exact recovery of
codeword inputs, constructed exact ties, agreement with an fp64 brute-force
argmin away from near-ties, equivariance under a permutation of the codebook
rows, and correct placement in the index cache.  ``test_oracle_mutants.py``
re-runs these checks against deliberately broken copies of the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from cases import (kv_from_codewords, natural_codebook, natural_subvectors, bf16_representable_fp32,
                   rounding_order_case, fp32_sequential_argmin)
from sub_bit_vq_amd import synth

SHAPES = [  # (n_heads, head_dim, loop_steps, group)
    (2, 64, 4, 16),
    (1, 128, 4, 32),
    (2, 32, 2, 8),
]


def _enc(x, cb, H, d, Tc, G, **kw):
    idx = oracle.encode(x, cb, n_heads=H, head_dim=d, loop_steps=Tc, group=G, **kw)
    return torch.from_numpy(idx)


def check_codeword_inputs(H=2, d=64, Tc=4, G=16, cb_dtype=torch.bfloat16, n=96, seed=1):
    """x equal to a codeword (of N(0,1) codebooks, almost surely distinct rows)
    -> its index is returned and re-assembling the codewords gives x back."""
    cg = G // Tc
    S = d // cg
    cb = synth.codebooks(H, d, Tc, G, seed, dtype=cb_dtype)
    if cb_dtype == torch.float32:
        cb = bf16_representable_fp32(cb)
    idx = synth.random_indices((n, H, S), seed + 10)
    x = kv_from_codewords(idx, cb).to(torch.bfloat16)
    got = _enc(x, cb, H, d, Tc, G)[0].permute(1, 0, 2)        # [n][H][S]
    assert torch.equal(got, idx), "codeword inputs must map to their own index"
    assert torch.equal(kv_from_codewords(got, cb).to(torch.bfloat16), x)


def check_exact_ties(seed=2):
    """Integer codewords make every fp32 operation exact.  x = 0 and two or
    more codewords at the same minimal squared norm -> the lowest index."""
    H, d, Tc, G = 1, 4, 4, 16               # cg = 4 channels -> one sub-vector
    g = torch.Generator().manual_seed(seed)
    cases = [(3, 200), (0, 255), (17, 18), (254, 255), (40, 9, 41)]
    for tie in cases:
        nat = torch.randint(-3, 4, (H, 1, 256, G), generator=g).float()
        nat[..., 0] = 3.0                       # every other code: squared norm >= 9
        for k in tie:                           # tied codes: squared norm exactly 4
            nat[0, 0, k] = 0.0
            nat[0, 0, k, (k * 5) % G] = 2.0 if k % 2 else -2.0
        cb = nat.reshape(H, 1, 256, Tc, G // Tc).permute(3, 0, 2, 1, 4).contiguous()
        x = torch.zeros((1, H, Tc, d), dtype=torch.bfloat16)
        got = int(_enc(x, cb, H, d, Tc, G)[0, 0, 0, 0])
        assert got == min(tie), (tie, got)
    # a codeword tied with itself repeated at a lower index: lowest index wins
    nat = torch.randint(-3, 4, (H, 1, 256, G), generator=g).float()
    nat[0, 0, 77] = nat[0, 0, 200]
    cb = nat.reshape(H, 1, 256, Tc, G // Tc).permute(3, 0, 2, 1, 4).contiguous()
    x = nat[0, 0, 200].reshape(1, H, Tc, G // Tc).to(torch.bfloat16)
    assert int(_enc(x, cb, H, d, Tc, G)[0, 0, 0, 0]) == 77


def check_fp64_bruteforce(H=2, d=64, Tc=4, G=16, cb_dtype=torch.bfloat16, n=128, seed=3):
    """Nearest codeword computed independently in fp64 (numpy) agrees with
    the oracle wherever the fp64 gap between the two nearest codes exceeds
    the fp32 rounding of a G-term sum (relative 1e-5 is ~100x that bound)."""
    cb = synth.codebooks(H, d, Tc, G, seed, dtype=cb_dtype)
    x = synth.loop_correlated_kv(n, H, Tc, d, seed + 1)
    got = _enc(x, cb, H, d, Tc, G)[0].permute(1, 0, 2).numpy()        # [n][H][S]
    xs = natural_subvectors(x.float(), G).double().numpy()             # [n][H][S][G]
    cn = natural_codebook(cb.float()).double().numpy()                  # [H][S][256][G]
    D = ((xs[:, :, :, None, :] - cn[None]) ** 2).sum(-1)                # [n][H][S][256]
    ref = D.argmin(-1)
    Ds = np.sort(D, axis=-1)
    clear = (Ds[..., 1] - Ds[..., 0]) > 1e-5 * Ds[..., 1]
    assert clear.mean() > 0.99
    assert np.array_equal(got[clear], ref[clear])
    # near-ties may differ only between the two nearest codes
    amb = ~clear
    if amb.any():
        Dg = np.take_along_axis(D, got[..., None].astype(np.int64), -1)[..., 0]
        assert np.all(Dg[amb] <= Ds[..., 1][amb] * (1 + 1e-5))


def check_row_permutation(H=1, d=64, Tc=4, G=16, n=64, seed=4):
    """Permuting the rows of a codebook permutes the returned indices."""
    cb = synth.codebooks(H, d, Tc, G, seed)
    x = synth.loop_correlated_kv(n, H, Tc, d, seed + 1)
    base = _enc(x, cb, H, d, Tc, G)[0, 0]                              # [n][S]
    perm = torch.randperm(256, generator=torch.Generator().manual_seed(seed))
    inv = torch.argsort(perm)
    got = _enc(x, cb[:, :, perm].contiguous(), H, d, Tc, G)[0, 0]
    # new row r holds old code perm[r]: the old code k is now at row inv[k]
    assert torch.equal(got.long(), inv[base.long()])


def check_placement(seed=5):
    """Index rows land at [seq][h][first_token + n][j]; other rows untouched."""
    H, d, Tc, G = 2, 64, 4, 16
    S = d // (G // Tc)
    cb = synth.codebooks(H, d, Tc, G, seed)
    idx = synth.random_indices((10, H, S), seed + 1)
    x = kv_from_codewords(idx, cb).to(torch.bfloat16)
    cache = np.full((3, H, 40, S), 0xAB, np.uint8)
    oracle.encode(x, cb, n_heads=H, head_dim=d, loop_steps=Tc, group=G, index=cache,
                  seq=1, first_token=25)
    want = np.full_like(cache, 0xAB)
    want[1, :, 25:35] = idx.permute(1, 0, 2).numpy()
    assert np.array_equal(cache, want)


def check_rounding_order(seed=6):
    """The distance is a sequence of separately rounded fp32 operations in
    ascending entry order.  On codes that are permutations of each other the
    exact distances coincide, so the winner is decided by those roundings; an
    independent numpy evaluation step by step must agree with the oracle, and
    a fused multiply-add evaluation must not (so the case has teeth)."""
    for cb_dtype, (H, d, Tc, G) in ((torch.float32, (1, 64, 4, 16)), (torch.bfloat16, (1, 64, 4, 32)),
                                    (torch.float32, (1, 32, 2, 8))):
        x, cb = rounding_order_case(H, d, Tc, G, 48, cb_dtype, seed)
        got = _enc(x, cb, H, d, Tc, G)[0].permute(1, 0, 2).numpy()        # [n][H][S]
        xs = natural_subvectors(x.float(), G).numpy()
        cn = natural_codebook(cb.float()).numpy()
        want = fp32_sequential_argmin(xs, cn)
        assert np.array_equal(got, want), (cb_dtype, G, int((got != want).sum()))
        assert (fp32_sequential_argmin(xs, cn, fused=True) != want).any()


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("cb_dtype", [torch.bfloat16, torch.float32])
def test_codeword_inputs(shape, cb_dtype):
    H, d, Tc, G = shape
    check_codeword_inputs(H, d, Tc, G, cb_dtype)


def test_exact_ties():
    check_exact_ties()


def test_rounding_order():
    check_rounding_order()


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("cb_dtype", [torch.bfloat16, torch.float32])
def test_fp64_bruteforce(shape, cb_dtype):
    H, d, Tc, G = shape
    check_fp64_bruteforce(H, d, Tc, G, cb_dtype)


def test_row_permutation():
    check_row_permutation()


def test_placement():
    check_placement()


def test_rejects_bad_shapes():
    x = torch.zeros((1, 1, 4, 64), dtype=torch.bfloat16)
    cb = synth.codebooks(1, 64, 4, 16, 0)
    with pytest.raises(ValueError):
        oracle.encode(x, cb, n_heads=1, head_dim=64, loop_steps=4, group=18)

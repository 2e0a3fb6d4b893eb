"""The encoder's screen error, measured (MI355X).

The encoder screens all 256 codes of a sub-vector x with the MFMA value
S_k = |c_k|^2 - 2 x.c_k (fp32) and trusts the screen's winner when its two
smallest values are further apart than eps = E 2^-24 R^2, R = |x| + max_k |c_k|.
That is exact (the winner is the oracle's, bit for bit) as long as the screen
error stays within F (P G + 3) 2^-24 R^2 with

    2 * 32 + 2 (G + 2) + 2 F (P G + 3) <= E

(eps must exceed twice the sum of a mark, at most 32 units of 2^-24 R^2, the
exact distance's rounding and the screen's),
where P is the number of bf16 parts of each codebook entry (1 for bf16
codebooks, 3 for fp32) and F measures the matrix cores' accumulation against
the worst case of a sequential fp32 sum of the P G + 3 products.  The encoder
takes E = 256 where the bound then allows F >= 3 (every fp32 summation order
has F <= 2), else E = 512.  This test
reads every screen value through the diagnostic entry point
(``lvq_encode_screen``), evaluates S_k exactly in fp64 on the host and
records the largest F it implies, on the workloads' data (loop-correlated
tokens, N(0,1) codebooks), on near-tie constructions and on data with a large
common offset (heavy cancellation).  Each case must leave a margin of at
least 4x to the F the proof allows.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from cases import natural_codebook, natural_subvectors, rounding_order_case
from sub_bit_vq_amd import synth

pytestmark = pytest.mark.gpu
MARGIN = 4.0
MEASURED = {}


@pytest.fixture(scope="module")
def lv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sub_bit_vq_amd import loopvq
    loopvq.library()
    return loopvq


def _note(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def eps_units(G, P):
    """eps in units of 2^-24 R^2: the encoder's choice for this shape"""
    return 256 if 2 * 32 + 2 * (G + 2) + 2 * 3 * (P * G + 3) <= 256 else 512


def allowed_f(G, P):
    return (eps_units(G, P) - 2 * 32 - 2 * (G + 2)) / (2 * (P * G + 3))


def _offset_case(H, d, Tc, G, n, seed):
    """tokens and bf16 codewords around a common offset of 30: distances are
    small differences of large squared norms"""
    g = torch.Generator().manual_seed(seed)
    x = (30.0 + torch.randn((n, H, Tc, d), generator=g)).to(torch.bfloat16)
    cb = synth.codebooks(H, d, Tc, G, seed + 1, dtype=torch.float32)
    return x, (30.0 + cb).to(torch.bfloat16)


CASES = {
    # name: (H, d, Tc, G, codebook dtype, tokens, data)
    "prefill 0.5 bit": (16, 128, 4, 16, torch.bfloat16, 512, "loop"),
    "0.25 bit": (16, 128, 4, 32, torch.bfloat16, 512, "loop"),
    "G8 bf16": (4, 64, 4, 8, torch.bfloat16, 512, "loop"),
    "fp32 codebooks G16": (1, 64, 4, 16, torch.float32, 512, "loop"),
    "fp32 codebooks G8": (2, 64, 4, 8, torch.float32, 512, "loop"),
    "near ties bf16 G16": (2, 64, 4, 16, torch.bfloat16, 300, "ties"),
    "near ties bf16 G32": (2, 128, 4, 32, torch.bfloat16, 300, "ties"),
    "near ties fp32 G16": (2, 64, 4, 16, torch.float32, 300, "ties"),
    "offset 30 bf16 G16": (4, 128, 4, 16, torch.bfloat16, 512, "offset"),
    "offset 30 bf16 G32": (4, 128, 4, 32, torch.bfloat16, 512, "offset"),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_screen_error_factor(lv, name):
    H, d, Tc, G, cb_dtype, n, kind = CASES[name]
    P = 1 if cb_dtype == torch.bfloat16 else 3
    seed = 3000 + sum(map(ord, name))
    if kind == "loop":
        x = synth.loop_correlated_kv(n, H, Tc, d, seed)
        cb = synth.codebooks(H, d, Tc, G, seed + 1, dtype=cb_dtype)
    elif kind == "ties":
        x, cb = rounding_order_case(H, d, Tc, G, n, cb_dtype, seed)
    else:
        x, cb = _offset_case(H, d, Tc, G, n, seed)
    S = d // (G // Tc)
    dt = lv.LVQ_BF16 if cb_dtype == torch.bfloat16 else lv.LVQ_F32
    cfg = lv.Config(batch=1, n_heads=H, head_dim=d, loop_steps=Tc, group=G, max_tokens=n,
                    codebook_dtype=dt)
    idx = torch.zeros((1, H, n, S), dtype=torch.uint8, device="cuda")
    screen = torch.zeros((n, H, S, 256), dtype=torch.float32, device="cuda")
    lv.lvq_encode_screen(cfg, x.cuda(), cb.cuda(), idx, screen)
    torch.cuda.synchronize()
    got = screen.double().cpu().numpy()
    assert np.isfinite(got).all()
    # the indices written are lvq_encode's, bit for bit the oracle's
    ref_idx = oracle.encode(x, cb, n_heads=H, head_dim=d, loop_steps=Tc, group=G)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)

    # exact screen values: fp64 holds every product and sum of these bf16 /
    # fp32 inputs with error far below the fp32 rounding being measured
    xs = natural_subvectors(x.float(), G).double()                   # [n][H][S][G]
    cn = natural_codebook(cb.float()).double()                       # [H][S][256][G]
    c2 = (cn * cn).sum(-1)                                           # [H][S][256]
    exact = (c2[None] - 2.0 * torch.einsum("nhsg,hskg->nhsk", xs, cn)).numpy()
    R = (torch.sqrt((xs * xs).sum(-1)) + torch.sqrt(c2.max(-1).values)[None]).numpy()
    c2 = c2.numpy()
    unit = (P * G + 3) * 2.0 ** -24 * R * R
    F = np.abs(got - exact) / unit[..., None]
    f_obs = float(F.max())
    # how often the screen leaves two codes within eps (re-scored exactly)
    srt = np.sort(got, axis=-1)
    rescored = float(((srt[..., 1] - srt[..., 0]) <= eps_units(G, P) * 2.0 ** -24 * R * R).mean())
    MEASURED[name] = f_obs
    _note(f"{name}: largest F {f_obs:.4f} (allowed {allowed_f(G, P):.2f}); "
          f"max |error| {float(np.abs(got - exact).max()):.3e}; {rescored:.2%} within eps")
    assert f_obs * MARGIN <= allowed_f(G, P), name

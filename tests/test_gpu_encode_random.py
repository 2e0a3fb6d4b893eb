"""Seeded random sweep of lvq_encode against the CPU oracle (MI355X): every
supported (G, Tc, cg) with head_dims whose sub-vector count the encoder
tiles, bf16 and fp32 codebooks, run lengths on both sides of the short-run
switch, placement (sequence, first row) inside a larger cache, and strided
sources.  Bar: bit-exact indices."""
import sys

import numpy as np
import pytest
import torch

import oracle
from sub_bit_vq_amd import synth

pytestmark = pytest.mark.gpu
N_CASES = 20


@pytest.fixture(scope="module")
def lv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sub_bit_vq_amd import loopvq
    loopvq.library()
    return loopvq


def _draw(seed):
    rng = np.random.default_rng(seed)
    while True:
        G = int(rng.choice([8, 16, 32]))
        Tc = int(rng.choice([1, 2, 4]))
        cg = G // Tc
        d = int(rng.choice([32, 64, 128]))
        if cg not in (2, 4, 8) or d % cg or (d // cg) % 4:
            continue
        fp32 = bool(rng.integers(0, 3) == 0) and G <= 16
        break
    n = int(rng.choice([int(rng.integers(1, 33)), int(rng.integers(33, 3000)),
                        int(rng.integers(3000, 6000))]))
    return dict(G=G, Tc=Tc, d=d, fp32=fp32, n=n, H=int(rng.integers(1, 4)), B=int(rng.integers(1, 3)),
                first=int(rng.integers(0, 200)), strided=bool(rng.integers(0, 2)))


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_encode(lv, case):
    p = _draw(7000 + case)
    print(f"[gpu] random encode {case}: {p}", file=sys.stderr, flush=True)
    G, Tc, d, H, n, B = p["G"], p["Tc"], p["d"], p["H"], p["n"], p["B"]
    S = d // (G // Tc)
    dt = torch.float32 if p["fp32"] else torch.bfloat16
    x = synth.loop_correlated_kv(n, H, Tc, d, seed=8000 + case)
    cb = synth.codebooks(H, d, Tc, G, seed=8100 + case, dtype=dt)
    if p["strided"]:
        # the tokens as a view of a wider buffer: a padded head axis
        wide = torch.zeros((n, H + 1, Tc, d), dtype=torch.bfloat16)
        wide[:, :H] = x
        xg = wide.cuda()[:, :H]
    else:
        xg = x.cuda()
    seq = B - 1
    T = p["first"] + n + 5
    cfg = lv.Config(batch=B, n_heads=H, head_dim=d, loop_steps=Tc, group=G, max_tokens=T,
                    codebook_dtype=lv.LVQ_F32 if p["fp32"] else lv.LVQ_BF16)
    idx = torch.full((B, H, T, S), 7, dtype=torch.uint8, device="cuda")
    lv.lvq_encode(cfg, xg, cb.cuda(), idx, seq, p["first"])
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    ref = np.full((B, H, T, S), 7, np.uint8)
    oracle.encode(x, cb, n_heads=H, head_dim=d, loop_steps=Tc, group=G, index=ref, seq=seq,
                  first_token=p["first"])
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:5].tolist()}"

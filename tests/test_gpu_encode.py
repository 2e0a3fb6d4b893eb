"""GPU parity of lvq_encode against the CPU oracle (MI355X): bit-exact
indices, including constructed exact ties and near-ties that the MFMA screen
cannot separate, strided inputs, placement and a sampled full-size run."""
import sys

import numpy as np
import pytest
import torch

import oracle
from cases import kv_from_codewords, rounding_order_case
from sub_bit_vq_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sub_bit_vq_amd import loopvq
    loopvq.library()
    return loopvq


def _note(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def _gpu_encode(lv, x, cb, H, d, Tc, G, T=None, B=1, seq=0, first=0, fill=0):
    n = x.shape[0]
    T = T or first + n
    dt = lv.LVQ_BF16 if cb.dtype == torch.bfloat16 else lv.LVQ_F32
    cfg = lv.Config(batch=B, n_heads=H, head_dim=d, loop_steps=Tc, group=G, max_tokens=T,
                    codebook_dtype=dt)
    idx = torch.full((B, H, T, d // (G // Tc)), fill, dtype=torch.uint8, device="cuda")
    lv.lvq_encode(cfg, x.cuda() if x.device.type != "cuda" else x, cb.cuda(), idx, seq, first)
    torch.cuda.synchronize()
    return idx.cpu().numpy()


def _oracle_encode(x, cb, H, d, Tc, G, T=None, B=1, seq=0, first=0, fill=0):
    n = x.shape[0]
    T = T or first + n
    idx = np.full((B, H, T, d // (G // Tc)), fill, np.uint8)
    oracle.encode(x, cb, n_heads=H, head_dim=d, loop_steps=Tc, group=G, index=idx, seq=seq,
                  first_token=first)
    return idx


def _assert_same(got, ref, what):
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[:5].tolist()}"


def test_tiny_workload_fp32_codebooks(lv):
    """B1 H1 d64 Tc4 G16, fp32 N(0,1) codebooks, 512 loop-correlated tokens."""
    _note("tiny fp32")
    x = synth.loop_correlated_kv(512, 1, 4, 64, seed=2000)
    cb = synth.codebooks(1, 64, 4, 16, seed=2001, dtype=torch.float32)
    _assert_same(_gpu_encode(lv, x, cb, 1, 64, 4, 16), _oracle_encode(x, cb, 1, 64, 4, 16),
                 "tiny")


SHAPES = [  # (H, d, Tc, G, cb dtype)
    (2, 128, 4, 16, torch.bfloat16),
    (2, 128, 4, 32, torch.bfloat16),
    (3, 64, 4, 16, torch.bfloat16),
    (2, 64, 4, 8, torch.bfloat16),
    (2, 64, 2, 16, torch.bfloat16),
    (1, 64, 8, 16, torch.bfloat16),
    (1, 64, 4, 32, torch.bfloat16),
    (2, 64, 4, 16, torch.float32),
    (1, 64, 4, 8, torch.float32),
    (1, 64, 8, 16, torch.float32),
]


@pytest.mark.parametrize("H,d,Tc,G,cb_dtype", SHAPES)
def test_shapes_multi_chunk_ragged_tail(lv, H, d, Tc, G, cb_dtype):
    """4500 tokens: three 2048-token workgroups, the last one ragged."""
    _note(f"shape H={H} d={d} Tc={Tc} G={G} {cb_dtype}")
    seed = H * 1000 + d + Tc * 10 + G
    x = synth.loop_correlated_kv(4500, H, Tc, d, seed)
    cb = synth.codebooks(H, d, Tc, G, seed + 1, dtype=cb_dtype)
    _assert_same(_gpu_encode(lv, x, cb, H, d, Tc, G), _oracle_encode(x, cb, H, d, Tc, G),
                 "shape")


@pytest.mark.parametrize("n", [1, 8, 31, 32, 33, 64])
@pytest.mark.parametrize("H,d,Tc,G,cb_dtype", SHAPES)
def test_short_runs(lv, n, H, d, Tc, G, cb_dtype):
    """Runs of up to 32 tokens (a page of generated tokens) take the direct
    exact path, longer ones the MFMA screen; both sides of the switch."""
    _note(f"short run n={n} H={H} d={d} Tc={Tc} G={G} {cb_dtype}")
    seed = 7000 + n + H * 100 + d + Tc * 10 + G
    x = synth.loop_correlated_kv(n, H, Tc, d, seed)
    cb = synth.codebooks(H, d, Tc, G, seed + 1, dtype=cb_dtype)
    _assert_same(_gpu_encode(lv, x, cb, H, d, Tc, G, T=n + 5, first=5),
                 _oracle_encode(x, cb, H, d, Tc, G, T=n + 5, first=5), "short run")


def test_grouped_query_config(lv):
    """With grouped-query attention the encoder writes the KV heads' caches:
    x has n_kv_heads heads."""
    _note("GQA encode")
    Hk, Hq, d, Tc, G = 2, 8, 128, 4, 16
    for n in (8, 300):
        x = synth.loop_correlated_kv(n, Hk, Tc, d, seed=90 + n)
        cb = synth.codebooks(Hk, d, Tc, G, seed=91)
        cfg = lv.Config(batch=1, n_heads=Hq, n_kv_heads=Hk, head_dim=d, loop_steps=Tc, group=G,
                        max_tokens=n)
        idx = torch.zeros((1, Hk, n, d // (G // Tc)), dtype=torch.uint8, device="cuda")
        lv.lvq_encode(cfg, x.cuda(), cb.cuda(), idx)
        torch.cuda.synchronize()
        _assert_same(idx.cpu().numpy(), _oracle_encode(x, cb, Hk, d, Tc, G), "gqa encode")


@pytest.mark.parametrize("n", [8, 700])
def test_loop_groups(lv, n):
    """R = 8 loop steps over Tc = 4: x carries all 8 steps, and both groups'
    index blocks are written (group g from steps 4g..4g+3 and codebook
    slices 4g..4g+3)."""
    _note(f"loop groups encode n={n}")
    H, d, Tc, G, R = 2, 128, 4, 16, 8
    x = synth.loop_correlated_kv(n, H, R, d, seed=95 + n)
    S = d // (G // Tc)
    cb = synth.codebooks(H, d, Tc, G, seed=97)
    cb = torch.cat([cb, synth.codebooks(H, d, Tc, G, seed=98)], 0)   # [8][H][256][S][cg]
    cfg = lv.Config(batch=2, n_heads=H, head_dim=d, loop_steps=Tc, group=G, max_tokens=n + 3,
                    n_loops=R)
    idx = torch.full((R // Tc, 2, H, n + 3, S), 0x5A, dtype=torch.uint8, device="cuda")
    lv.lvq_encode(cfg, x.cuda(), cb.cuda(), idx, 1, 3)
    torch.cuda.synchronize()
    ref = np.full((R // Tc, 2, H, n + 3, S), 0x5A, np.uint8)
    oracle.encode(x, cb, n_heads=H, head_dim=d, loop_steps=Tc, group=G, n_loops=R, index=ref,
                  seq=1, first_token=3)
    _assert_same(idx.cpu().numpy(), ref, "loop groups encode")


def test_codeword_inputs(lv):
    _note("codeword inputs")
    H, d, Tc, G = 2, 128, 4, 16
    S = d // (G // Tc)
    cb = synth.codebooks(H, d, Tc, G, seed=31)
    idx = synth.random_indices((300, H, S), seed=32)
    x = kv_from_codewords(idx, cb).to(torch.bfloat16)
    got = _gpu_encode(lv, x, cb, H, d, Tc, G)
    assert np.array_equal(got[0].transpose(1, 0, 2), idx.numpy())


def _tie_codebook(H, d, Tc, G, seed):
    """Integer-valued codebooks (small range) so that many codes sit at
    exactly equal or nearly equal distances from integer-valued inputs."""
    g = torch.Generator().manual_seed(seed)
    cg = G // Tc
    S = d // cg
    nat = torch.randint(-2, 3, (H, S, 256, Tc, cg), generator=g).float()
    return nat.permute(3, 0, 2, 1, 4).contiguous()


@pytest.mark.parametrize("n", [700, 24])
@pytest.mark.parametrize("cb_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("G", [16, 32])
def test_exact_ties(lv, cb_dtype, G, n):
    """Integer codebooks and integer inputs: exact fp32 ties everywhere; the
    lowest index must win on every sub-vector."""
    if cb_dtype == torch.float32 and G == 32:
        pytest.skip("fp32 codebooks are supported for G <= 16")
    _note(f"exact ties G={G} {cb_dtype} n={n}")
    H, d, Tc = 2, 64, 4
    cb = _tie_codebook(H, d, Tc, G, seed=40 + G).to(cb_dtype)
    g = torch.Generator().manual_seed(41)
    x = torch.randint(-2, 3, (n, H, Tc, d), generator=g).to(torch.bfloat16)
    _assert_same(_gpu_encode(lv, x, cb, H, d, Tc, G), _oracle_encode(x, cb, H, d, Tc, G),
                 "ties")


def test_near_ties(lv):
    """Inputs at (or a few ulps from) the midpoint of two codewords: the two
    screen values are closer than the screen's error bound, so the exact
    re-score decides; it must reproduce the oracle bit for bit."""
    _note("near ties")
    H, d, Tc, G = 2, 128, 4, 16
    cg = G // Tc
    S = d // cg
    cb = synth.codebooks(H, d, Tc, G, seed=50)
    g = torch.Generator().manual_seed(51)
    n = 1200
    a = torch.randint(0, 256, (n, H, S), generator=g, dtype=torch.uint8)
    b = torch.randint(0, 256, (n, H, S), generator=g, dtype=torch.uint8)
    xa = kv_from_codewords(a, cb).float()
    xb = kv_from_codewords(b, cb).float()
    mid = 0.5 * (xa + xb)
    jitter = torch.randint(-2, 3, mid.shape, generator=g).float() * 2.0 ** -8 * mid.abs()
    x = (mid + jitter).to(torch.bfloat16)
    _assert_same(_gpu_encode(lv, x, cb, H, d, Tc, G), _oracle_encode(x, cb, H, d, Tc, G),
                 "near ties")


@pytest.mark.parametrize("cb_dtype,G", [(torch.float32, 16), (torch.float32, 8),
                                        (torch.bfloat16, 16), (torch.bfloat16, 32),
                                        (torch.bfloat16, 8)])
@pytest.mark.parametrize("n", [300, 30])
def test_rounding_order(lv, cb_dtype, G, n):
    """Codes that are permutations of each other: the screen cannot separate
    them, and the exact re-score must round every subtraction, square and add
    separately in ascending entry order, as the oracle does (a fused
    multiply-add picks another code on many of these sub-vectors)."""
    _note(f"rounding order G={G} {cb_dtype} n={n}")
    H, d, Tc = 2, 64, 4
    x, cb = rounding_order_case(H, d, Tc, G, n, cb_dtype, seed=80 + G)
    _assert_same(_gpu_encode(lv, x, cb, H, d, Tc, G), _oracle_encode(x, cb, H, d, Tc, G),
                 "rounding order")


def test_strided_input_from_window_buffer(lv):
    """Encode a page of 8 recent tokens straight from the bf16 window buffer
    ([b][t][h][slot][d]) into rows of sequence 1 (the eviction-page case)."""
    _note("strided window page")
    H, d, Tc, G, B = 2, 128, 4, 16, 2
    W = 320
    win = synth.loop_correlated_kv(B * W, H, Tc, d, seed=60).view(B, W, H, Tc, d)
    win = win.permute(0, 3, 2, 1, 4).contiguous()                 # [B][Tc][H][W][d]
    cb = synth.codebooks(H, d, Tc, G, seed=61)
    slots = slice(64 + 16, 64 + 24)
    dwin = win.cuda()
    x_dev = dwin[1][:, :, slots, :].permute(2, 1, 0, 3)           # [8][H][Tc][d] view
    assert not x_dev.is_contiguous()
    got = _gpu_encode(lv, x_dev, cb, H, d, Tc, G, T=500, B=B, seq=1, first=400, fill=0xAB)
    x_host = win[1][:, :, slots, :].permute(2, 1, 0, 3).contiguous()
    ref = _oracle_encode(x_host, cb, H, d, Tc, G, T=500, B=B, seq=1, first=400, fill=0xAB)
    _assert_same(got, ref, "strided")


@pytest.mark.parametrize("n", [8, 300])
def test_encode_kv_one_launch(lv, n):
    """lvq_encode_kv (K and V of a page in one launch, here from the strided
    window buffers) writes exactly what two lvq_encode calls and the oracle
    write, on both sides of the short-run switch."""
    _note(f"encode_kv n={n}")
    H, d, Tc, G, B = 2, 128, 4, 16, 2
    W = max(320, n)
    kwin = synth.loop_correlated_kv(B * W, H, Tc, d, seed=62).view(B, W, H, Tc, d)
    vwin = synth.loop_correlated_kv(B * W, H, Tc, d, seed=63).view(B, W, H, Tc, d)
    kwin = kwin.permute(0, 3, 2, 1, 4).contiguous().cuda()       # [B][Tc][H][W][d]
    vwin = vwin.permute(0, 3, 2, 1, 4).contiguous().cuda()
    kcb = synth.codebooks(H, d, Tc, G, seed=64).cuda()
    vcb = synth.codebooks(H, d, Tc, G, seed=65).cuda()
    T, first = n + 400, 400
    cfg = lv.Config(batch=B, n_heads=H, head_dim=d, loop_steps=Tc, group=G, max_tokens=T)
    S = d // (G // Tc)
    kx = kwin[1][:, :, :n, :].permute(2, 1, 0, 3)                  # [n][H][Tc][d] views
    vx = vwin[1][:, :, :n, :].permute(2, 1, 0, 3)
    ki = torch.full((B, H, T, S), 0xAB, dtype=torch.uint8, device="cuda")
    vi = torch.full_like(ki, 0xCD)
    lv.lvq_encode_kv(cfg, kx, vx, kcb, vcb, ki, vi, 1, first)
    ki2, vi2 = torch.full_like(ki, 0xAB), torch.full_like(vi, 0xCD)
    lv.lvq_encode(cfg, kx, kcb, ki2, 1, first)
    lv.lvq_encode(cfg, vx, vcb, vi2, 1, first)
    torch.cuda.synchronize()
    assert torch.equal(ki, ki2) and torch.equal(vi, vi2)
    ref_k = _oracle_encode(kx.cpu().contiguous(), kcb.cpu(), H, d, Tc, G, T=T, B=B, seq=1,
                           first=first, fill=0xAB)
    ref_v = _oracle_encode(vx.cpu().contiguous(), vcb.cpu(), H, d, Tc, G, T=T, B=B, seq=1,
                           first=first, fill=0xCD)
    _assert_same(ki.cpu().numpy(), ref_k, "encode_kv K")
    _assert_same(vi.cpu().numpy(), ref_v, "encode_kv V")


def test_placement_and_untouched_rows(lv):
    _note("placement")
    H, d, Tc, G = 2, 64, 4, 16
    x = synth.loop_correlated_kv(77, H, Tc, d, seed=70)
    cb = synth.codebooks(H, d, Tc, G, seed=71)
    got = _gpu_encode(lv, x, cb, H, d, Tc, G, T=300, B=3, seq=2, first=123, fill=0xCD)
    ref = _oracle_encode(x, cb, H, d, Tc, G, T=300, B=3, seq=2, first=123, fill=0xCD)
    _assert_same(got, ref, "placement")

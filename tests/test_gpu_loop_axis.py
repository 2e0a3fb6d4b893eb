"""k-means codebook fitting with the HIP encoder as the assignment step
(MI355X): identical codebooks to the same fit driven by the CPU oracle, and
the pages' loop-axis claim at a larger size (LoopVQ project page,
"Component 1 -- Loop-axis vector quantization")."""
import sys

import pytest
import torch

import oracle
from sub_bit_vq_amd import kmeans, synth

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


def oracle_assign(x, cb, group):
    N, H, Tc, d = x.shape
    return oracle.encode(x, cb, n_heads=H, head_dim=d, loop_steps=Tc, group=group)[0].transpose(1, 0, 2)


@pytest.mark.parametrize("group", [16, 32])
def test_device_fit_equals_oracle_fit(lv, group):
    """Bit-exact assignments give bit-identical codebooks after every
    iteration (the update step is the same deterministic fp64 mean)."""
    _note(f"k-means parity G={group}")
    x = synth.loop_correlated_kv(1500, 2, 4, 128, seed=10 + group)
    cb_dev, h_dev = kmeans.fit_codebooks(x, group, 4, seed=11, assign=kmeans.device_assign(lv))
    cb_ora, h_ora = kmeans.fit_codebooks(x, group, 4, seed=11, assign=oracle_assign)
    assert torch.equal(cb_dev.view(torch.int16), cb_ora.view(torch.int16))
    assert h_dev == h_ora


def test_loop_axis_claim(lv):
    """4 heads, d = 128, 8192 training and 2048 test tokens, 8 iterations:
    the loop-axis grouping has well under half the error of channel-only
    grouping at 0.5 and at 0.25 bit per element."""
    x = synth.loop_correlated_kv(10240, 4, 4, 128, seed=20)
    for group in (16, 32):
        r = kmeans.loop_axis_comparison(x[:8192], x[8192:], group, 8, seed=21,
                                        assign=kmeans.device_assign(lv))
        _note(f"  G={group}: loop axis {r['mse_loop_axis']:.4f}, "
              f"channels only {r['mse_channels_only']:.4f}")
        assert r["mse_loop_axis"] < 0.5 * r["mse_channels_only"]

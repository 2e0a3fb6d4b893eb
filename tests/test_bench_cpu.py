"""Host-side logic of bench.py (no GPU): the algorithmic bytes behind the
roofline figure, the counter-summary lookup behind its traffic figure, and
the one-GPU contract."""
import subprocess
import sys
import pathlib

import bench

ROOT = pathlib.Path(__file__).resolve().parents[1]


def test_cache_bytes_match_workload_sizes():
    # one 32768-token sequence, 16 heads, d 128: 32448 VQ tokens of 2 x S index
    # bytes per head, 320 window tokens of 2 x d bf16 values per head
    assert bench.cache_bytes(16, 128, 4, 16, [32768]) == 32448 * 16 * 2 * 32 + 320 * 16 * 2 * 128 * 2
    assert bench.cache_bytes(16, 128, 4, 16, [32768]) == 35_848_192      # 0.5 bit
    assert bench.cache_bytes(16, 128, 4, 32, [32768]) == 19_234_816      # 0.25 bit: S = 16
    # short sequences: only the tokens they have, no VQ tokens below 320
    assert bench.cache_bytes(1, 64, 4, 16, [100]) == 100 * 2 * 64 * 2
    assert bench.cache_bytes(1, 64, 4, 16, [64 + 256 + 10]) == 10 * 2 * 16 + 320 * 2 * 64 * 2
    # a batch sums its sequences
    assert bench.cache_bytes(2, 128, 4, 16, [4000, 900]) == (bench.cache_bytes(2, 128, 4, 16, [4000])
                                                            + bench.cache_bytes(2, 128, 4, 16, [900]))


def test_encode_workload_sizes():
    # 32768 tokens x 16 heads x 4 steps x 128 channels of bf16, one index byte
    # per sub-vector (32 per token and head), the bf16 codebook once
    assert bench.encode_bytes(32768, 16, 128, 4, 16) == 32768 * 16 * 4 * 128 * 2 + 32768 * 16 * 32 + 4 * 16 * 256 * 32 * 4 * 2
    assert bench.encode_bytes(32768, 16, 128, 4, 16, 2) == 1_115_684_864          # K and V
    # x . c over G = 16 products for 256 codes of each sub-vector: 274.9 GFLOP for K and V;
    # the matrix cores run an augmented axis of 32
    assert bench.encode_mfma_flops(32768, 16, 128, 4, 16, 2) == 2 * 2 * 32768 * 16 * 32 * 256 * 16
    assert abs(bench.encode_mfma_flops(32768, 16, 128, 4, 16, 2) / 1e9 - 274.9) < 0.1
    # issued: one 16x16x16 MFMA per 16 codes x 16 tokens at G = 16 (K = G),
    # one 16x16x32 at G = 32, K = 16 at G = 8 (half of it padding)
    assert bench.encode_mfma_flops(32768, 16, 128, 4, 16, 2, issued=True) == \
        bench.encode_mfma_flops(32768, 16, 128, 4, 16, 2)
    assert bench.encode_mfma_flops(1, 1, 128, 4, 32, issued=True) == 2 * 16 * 256 * 32
    assert bench.encode_mfma_flops(1, 1, 64, 4, 8, issued=True) == 2 * 32 * 256 * 16


def test_rel_err_rows():
    import numpy as np
    ref = np.array([[[1.0, -2.0], [0.5, 0.25]]])
    got = ref + np.array([[[0.0, 0.02], [0.0, 0.0]]])
    assert abs(bench.rel_err_rows(got, ref) - 0.01) < 1e-12


def test_counter_traffic_needs_matching_sources(monkeypatch):
    wl = "ouro1p4b_layer_32k_0p5bit"
    text = (ROOT / "profiles" / f"decode_attn_{wl}.md").read_text()
    assert "hbm_bytes_per_launch" in text
    # counters taken on other kernel sources are not reported
    monkeypatch.setattr(bench, "kernel_source_hash", lambda paths=bench.DECODE_SOURCES: "0" * 16)
    assert bench.counters_traffic(wl) is None
    assert bench.counters_traffic("no_such_workload") is None


def test_source_hash_covers_kernel_inputs():
    names = {pathlib.Path(p).name for p in bench.DECODE_SOURCES}
    assert {"decode_attn.hip", "kernels.h", "build.py"} <= names
    assert len(bench.kernel_source_hash()) == 16


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""

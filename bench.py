"""LoopVQ decode-attention throughput on one MI355X.

One step = one eviction period of the pages' serving loop (LoopVQ project
page, "Serving in SGLang"): 8 generated tokens, each decoded at the Tc = 4
loop steps of one Ouro-1.4B-like layer (16 heads, head_dim 128, 0.5 bit,
G = 16) over a 32768-token context, then the encoding of the oldest 8-token
recent page (its K and V) into the index cache.  The context is held at 32768
tokens for the 8 decodes.

Metric: context-token x loop-steps per second (sum over decode calls of the
context length).  Inputs are resident in HBM before the timed region; the
index caches and windows are rotated over distinct copies so that the working
set exceeds the 256 MB last-level cache twice.  The step is captured once in a
HIP graph and replayed.

Extra fields: ``roofline`` for the decode-attention kernel (algorithmic cache
bytes per launch / its mean duration from HIP events), ``cpu_baseline`` (the
C oracle on a bounded sample of the same workload) and ``workloads``: the
other configurations, each timed the same way (decode launches at 0.25 bit,
batch 64 with ragged contexts, grouped-query heads; the 32768-token K and V
prefill encode against HBM and MFMA peaks) with the largest error of a
sampled parity check against the oracle (run in the CPU-baseline leg).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import pathlib
import sys
import time

ROOT = pathlib.Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBS = 8000.0
LLC_BYTES = 256 << 20
WORKLOADS = {
    # name: (B, H, d, Tc, G, context; "ragged" = 2048 + U{4096, 8192, 16384}[, KV heads])
    "ouro1p4b_layer_32k_0p5bit": (1, 16, 128, 4, 16, 32768),
    "ouro1p4b_layer_32k_0p25bit": (1, 16, 128, 4, 32, 32768),
    "batch64_ragged_0p5bit": (64, 16, 128, 4, 16, "ragged"),
    # grouped-query attention: 32 query heads over 8 KV heads
    "gqa32q8kv_32k_0p5bit": (1, 32, 128, 4, 16, 32768, 8),
}
PAGE = 8          # tokens per eviction page
N_SINK, N_RECENT = 64, 256
METRIC = "VQ-KV decode attn: context-token·loop-steps/s at 32K; % HBM roofline"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cache_bytes(H, d, Tc, G, lengths):
    """Algorithmic bytes of one decode call: K and V index rows of every VQ
    token plus the bf16 K and V of the sink and recent tokens of the step,
    summed over the sequences of the batch (H = KV heads: query heads that
    share a KV head share its bytes)."""
    S = d // (G // Tc)
    total = 0
    for L in lengths:
        n_vq = max(0, L - N_SINK - N_RECENT)
        n_win = min(L, N_SINK) + min(max(L - N_SINK, 0), N_RECENT)
        total += n_vq * H * 2 * S + n_win * H * 2 * d * 2
    return total


MFMA_BF16_PEAK_TFLOPS = 2500.0      # dense bf16 matrix peak of MI355X
PREFILL_TOKENS = 32768


def encode_bytes(n, H, d, Tc, G, tensors=1):
    """Algorithmic bytes of encoding n tokens: bf16 input, one index byte per
    sub-vector, and the bf16 codebook read once, per tensor."""
    S = d // (G // Tc)
    return tensors * (n * H * Tc * d * 2 + n * H * S + Tc * H * 256 * S * (G // Tc) * 2)


def encode_mfma_flops(n, H, d, Tc, G, tensors=1, issued=False):
    """Algorithmic flops of the encoder's distance contraction: every
    sub-vector against all 256 codes, G products each (x . c_k).  With
    ``issued``: what the matrix cores execute for bf16 codebooks, the
    contraction axis padded to the MFMA's K (16 when G <= 16, else a multiple
    of 32; the squared norms enter as the accumulator, not as products)."""
    S = d // (G // Tc)
    k = (16 if G <= 16 else (G + 31) // 32 * 32) if issued else G
    return tensors * 2.0 * n * H * S * 256 * k


def cpu_model():
    try:
        for line in pathlib.Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def rel_err_rows(got, ref):
    """max over (b, h) rows of max_ch |got - ref| / max_ch |ref|"""
    import numpy as np
    got = np.asarray(got, np.float64).reshape(-1, got.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return float((np.abs(got - ref).max(axis=1) / den).max())


# everything the decode kernel's code depends on: its source, the header it
# shares with the host (workgroup shape, argument layout) and the build flags
DECODE_SOURCES = ("sub_bit_vq_amd/csrc/decode_attn.hip", "sub_bit_vq_amd/csrc/kernels.h",
                  "sub_bit_vq_amd/build.py")


def kernel_source_hash(paths=DECODE_SOURCES):
    h = hashlib.sha256()
    for rel in paths:
        h.update((ROOT / rel).read_bytes())
    return h.hexdigest()[:16]


def counters_traffic(workload):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE scaled by a plain copy), or None when it is
    missing or was taken on different kernel sources (DECODE_SOURCES)."""
    p = ROOT / "profiles" / f"decode_attn_{workload}.md"
    if not p.exists():
        return None
    fields = {}
    for line in p.read_text().splitlines():
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].split(": ", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("decode kernel sources (decode_attn.hip, kernels.h, build.py) sha256[:16]") != kernel_source_hash():
        return None
    return int(fields["hbm_bytes_per_launch"]) if "hbm_bytes_per_launch" in fields else None


class Setup:
    """Device-resident caches of one workload: index caches produced by the
    HIP encoder from loop-correlated K/V, bf16 windows, codebooks, queries,
    rotated over enough distinct copies to defeat the last-level cache."""

    def __init__(self, lv, synth, torch, workload, rotate, seed=1001):
        B, H, d, Tc, G, L = WORKLOADS[workload][:6]
        Hk = WORKLOADS[workload][6] if len(WORKLOADS[workload]) > 6 else H
        lengths = synth.ragged_lengths(B, seed=1003) if L == "ragged" else [L] * B
        self.B, self.H, self.Hk, self.d, self.Tc, self.G = B, H, Hk, d, Tc, G
        self.lengths = lengths
        self.L = max(lengths)
        dev = torch.device("cuda")
        T = self.L + PAGE
        self.cfg = lv.Config(batch=B, n_heads=H, head_dim=d, loop_steps=Tc, group=G,
                             max_tokens=T, n_kv_heads=Hk if Hk != H else 0)
        self.kcb = synth.codebooks(Hk, d, Tc, G, seed * 10 + 1, device=dev)
        self.vcb = synth.codebooks(Hk, d, Tc, G, seed * 10 + 2, device=dev)
        # one query per (token of the page, loop step)
        self.q = torch.stack([synth.queries(B, H, d, Tc, seed * 10 + 3 + i, device=dev)
                              for i in range(PAGE)])                 # [PAGE][Tc][B][H][d]
        base = lv.allocate(self.cfg, dev)
        for b, Lb in enumerate(lengths):
            k = synth.loop_correlated_kv(Lb + PAGE, Hk, Tc, d, seed * 10 + 5 + 2 * b, device=dev)
            v = synth.loop_correlated_kv(Lb + PAGE, Hk, Tc, d, seed * 10 + 6 + 2 * b, device=dev)
            lo, hi = N_SINK, Lb - N_RECENT
            if hi > lo:
                lv.lvq_encode(self.cfg, k[lo:hi], self.kcb, base["k_index"], b, lo)
                lv.lvq_encode(self.cfg, v[lo:hi], self.vcb, base["v_index"], b, lo)
            win = list(range(min(Lb, N_SINK))) + list(range(max(N_SINK, Lb - N_RECENT), Lb))
            slots = [p if p < N_SINK else N_SINK + (p - N_SINK) % N_RECENT for p in win]
            pos = torch.tensor(win, device=dev)
            sl = torch.tensor(slots, device=dev)
            base["k_window"][b][:, :, sl, :] = k[pos].permute(2, 1, 0, 3)
            base["v_window"][b][:, :, sl, :] = v[pos].permute(2, 1, 0, 3)
            if b == 0:
                # the page to encode in each step: the next 8 tokens of sequence 0
                self.page_k, self.page_v = k[Lb:Lb + PAGE].contiguous(), v[Lb:Lb + PAGE].contiguous()
                self.page_row = Lb
            del k, v
        torch.cuda.synchronize()
        self.ctx = torch.tensor(lengths, dtype=torch.int32, device=dev)
        self.out = base["out"]
        self.ws = base["workspace"]
        copy_bytes = (base["k_index"].numel() * 2 + base["k_window"].numel() * 4)
        self.rotate = rotate or max(2, math.ceil(2 * LLC_BYTES / copy_bytes))
        self.copies = []
        for r in range(self.rotate):
            c = {key: base[key].clone() for key in ("k_index", "v_index", "k_window", "v_window")}
            self.copies.append(c)
        del base
        torch.cuda.synchronize()
        self.calls = [lv.PreparedDecode(self.cfg, self.ctx, self.L, c["k_index"], c["v_index"],
                                        self.kcb, self.vcb, c["k_window"], c["v_window"],
                                        self.ws, self.out) for c in self.copies]
        self.lv = lv
        self.n_call = 0

    def decode(self, tok, t):
        call = self.calls[self.n_call % self.rotate]
        self.n_call += 1
        call(t, self.q[tok, t])

    def step(self, decode_only=False):
        for tok in range(PAGE):
            for t in range(self.Tc):
                self.decode(tok, t)
        if decode_only:
            return
        self.page_encode()

    def page_encode(self):
        """The K and V page encode of a step (8 tokens, one launch)."""
        c = self.copies[self.n_call % self.rotate]
        self.lv.lvq_encode_kv(self.cfg, self.page_k, self.page_v, self.kcb, self.vcb,
                              c["k_index"], c["v_index"], 0, self.page_row)

    @property
    def tokens_steps_per_step(self):
        return PAGE * self.Tc * sum(self.lengths)


class PrefillEncode:
    """Prefill encoder workload: 32768 tokens x 16 heads x 4 loop steps x 128
    channels of bf16 K (and V), G = 16, into a 32768-row index cache; ``run``
    encodes K, ``run_kv`` K and V in one lvq_encode_kv launch."""

    N = PREFILL_TOKENS

    def __init__(self, lv, synth, torch, setup, seed=1004):
        dev = torch.device("cuda")
        self.lv = lv
        self.H, self.d, self.Tc, self.G = setup.Hk, setup.d, setup.Tc, setup.G
        self.cfg = lv.Config(batch=1, n_heads=setup.Hk, head_dim=setup.d, loop_steps=setup.Tc,
                             group=setup.G, max_tokens=self.N)
        self.x = synth.loop_correlated_kv(self.N, setup.Hk, setup.Tc, setup.d, seed, device=dev)
        self.xv = synth.loop_correlated_kv(self.N, setup.Hk, setup.Tc, setup.d, seed + 1, device=dev)
        self.cb, self.vcb = setup.kcb, setup.vcb
        bufs = lv.allocate(self.cfg, dev)
        self.idx, self.vidx = bufs["k_index"], bufs["v_index"]

    def run(self):
        self.lv.lvq_encode(self.cfg, self.x, self.cb, self.idx, 0, 0)

    def run_kv(self):
        self.lv.lvq_encode_kv(self.cfg, self.x, self.xv, self.cb, self.vcb, self.idx, self.vidx, 0, 0)


def spin_cycles_for(torch, ms):
    """Cycles of torch's spin kernel that last about ``ms`` milliseconds."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    torch.cuda._sleep(1_000_000)
    b.record()
    torch.cuda.synchronize()
    per_ms = 1_000_000 / max(a.elapsed_time(b), 1e-3)
    return int(per_ms * ms)


def decode_kernel_time_ms(setup, torch, n=64, reps=8, spread=None):
    """Mean duration of one decode launch: HIP events on the launch stream
    around replays of a graph of ``n`` back-to-back launches (rotating over the
    cache copies), so the interval holds launches and nothing else.  With a
    dict ``spread``, each replay is also timed on its own and the median and
    minimum per-launch times of the replays are stored there."""
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(n):
            setup.decode(i % PAGE, i % setup.Tc)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        graph.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    if spread is not None:
        per = sorted(ev[i].elapsed_time(ev[i + 1]) / n for i in range(reps))
        spread["median_ms"] = per[len(per) // 2] if reps % 2 else 0.5 * (per[reps // 2 - 1] + per[reps // 2])
        spread["min_ms"] = per[0]
    return ev[0].elapsed_time(ev[reps]) / (n * reps)


def prefill_encode_time_ms(enc, torch, n=10, kv=False):
    """Mean duration of one 32768-token prefill encode (one tensor, or K and
    V in one launch): HIP events around ``n`` back-to-back launches on the
    current stream, after ten untimed ones (the clock ramps up over the first
    few)."""
    run = enc.run_kv if kv else enc.run
    for _ in range(10):
        run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n):
        run()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def cpu_baseline(setup, torch, checks=(), budget_s=15.0):
    """The C oracle on a bounded sample of the same workload: whole decode
    calls (all heads, loop step 0) repeated for about ``budget_s`` seconds, and
    one page encode, combined into the time of one step.  Also the parity
    samples of ``checks`` (see ``parity_checks``): the oracle's output for the
    sampled rows next to the device's, as the largest row error (decode) or
    the number of differing indices (encode)."""
    import oracle
    c = setup.copies[0]
    kidx, vidx = c["k_index"].cpu(), c["v_index"].cpu()
    kw, vw = c["k_window"].cpu(), c["v_window"].cpu()
    kcb, vcb = setup.kcb.cpu(), setup.vcb.cpu()
    q = setup.q[0, 0].cpu()
    threads = oracle.max_threads()
    calls = 0
    t0 = time.perf_counter()
    while calls < 1 or time.perf_counter() - t0 < budget_s:
        oracle.decode_attn(loop_step=0, q=q, ctx_len=[setup.L] * setup.B, k_index=kidx,
                           v_index=vidx, k_codebook=kcb, v_codebook=vcb, k_window=kw,
                           v_window=vw, n_sink=N_SINK, n_recent=N_RECENT, group=setup.G,
                           threads=threads)
        calls += 1
    t_dec = (time.perf_counter() - t0) / calls
    t1 = time.perf_counter()
    oracle.encode(setup.page_k.cpu(), kcb, n_heads=setup.Hk, head_dim=setup.d,
                  loop_steps=setup.Tc, group=setup.G, threads=threads)
    t_enc = time.perf_counter() - t1
    t_step = PAGE * setup.Tc * t_dec + 2 * t_enc
    # the same on one core: one whole decode call and the page encode
    t2 = time.perf_counter()
    oracle.decode_attn(loop_step=0, q=q, ctx_len=[setup.L] * setup.B, k_index=kidx,
                       v_index=vidx, k_codebook=kcb, v_codebook=vcb, k_window=kw,
                       v_window=vw, n_sink=N_SINK, n_recent=N_RECENT, group=setup.G, threads=1)
    t_dec1 = time.perf_counter() - t2
    t3 = time.perf_counter()
    oracle.encode(setup.page_k.cpu(), kcb, n_heads=setup.Hk, head_dim=setup.d,
                  loop_steps=setup.Tc, group=setup.G, threads=1)
    t_enc1 = time.perf_counter() - t3
    parity = {}
    for chk in checks:
        if chk["kind"] == "decode":
            ref = oracle.decode_attn(threads=threads, **chk["oracle"])
            if chk.get("heads"):
                h0, h1 = chk["heads"]
                ref = ref[:, h0:h1]
            parity[chk["name"]] = {"max_rel_err": rel_err_rows(chk["gpu"], ref), "rows": chk["rows"]}
        else:
            import numpy as np
            ref = oracle.encode(threads=threads, **chk["oracle"])
            parity[chk["name"]] = {"indices_differing": int((np.asarray(chk["gpu"]) != ref).sum()),
                                   "indices": int(ref.size), "rows": chk["rows"]}
    return {
        "value": setup.tokens_steps_per_step / t_step,
        "unit": "ctx-token*loop-steps/s",
        "cores": threads,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"{calls} whole decode calls ({setup.H} heads, {setup.L}-token context, loop step 0, "
                   f"{t_dec * 1e3:.1f} ms each) and one 8-token page encode ({t_enc * 1e3:.1f} ms, "
                   f"counted for K and V), combined as one step of 32 decodes + 2 encodes; "
                   f"OpenMP threads {threads} of {os.cpu_count()} logical CPUs"),
        "value_1core": setup.tokens_steps_per_step / (PAGE * setup.Tc * t_dec1 + 2 * t_enc1),
        "sample_1core": (f"one whole decode call ({t_dec1 * 1e3:.0f} ms) and one page encode "
                         f"({t_enc1 * 1e3:.1f} ms) on one thread, combined the same way"),
        "parity": parity,
    }


def parity_checks(setup, torch, name, heads=None, seqs=None):
    """One device decode call of loop step 0 on the workload's first cache
    copy and the oracle's arguments for the same rows: ``heads`` (h0, h1) of
    every sequence, or the sequences ``seqs`` (all heads)."""
    c = setup.copies[0]
    setup.lv.lvq_decode_attn(setup.cfg, 0, setup.q[0, 0].contiguous(), setup.ctx, setup.L,
                             c["k_index"], c["v_index"], setup.kcb, setup.vcb, c["k_window"],
                             c["v_window"], setup.ws, setup.out)
    torch.cuda.synchronize()
    out = setup.out.double().cpu().numpy()
    common = dict(loop_step=0, k_codebook=setup.kcb.cpu(), v_codebook=setup.vcb.cpu(),
                  n_sink=N_SINK, n_recent=N_RECENT, group=setup.G)
    if seqs is None:
        h0, h1 = heads
        return {"name": name, "kind": "decode", "heads": heads, "gpu": out[:, h0:h1],
                "rows": f"heads {h0}..{h1 - 1} of every sequence",
                "oracle": dict(common, q=setup.q[0, 0].cpu(), ctx_len=setup.lengths,
                               k_index=c["k_index"].cpu(), v_index=c["v_index"].cpu(),
                               k_window=c["k_window"].cpu(), v_window=c["v_window"].cpu(),
                               heads=heads)}
    sel = list(seqs)
    idx = torch.tensor(sel, device=c["k_index"].device)
    return {"name": name, "kind": "decode", "gpu": out[sel],
            "rows": f"sequences {sel} (lengths {[setup.lengths[b] for b in sel]}), every head",
            "oracle": dict(common, q=setup.q[0, 0][idx].cpu(), ctx_len=[setup.lengths[b] for b in sel],
                           k_index=c["k_index"][idx].cpu(), v_index=c["v_index"][idx].cpu(),
                           k_window=c["k_window"][idx].cpu(), v_window=c["v_window"][idx].cpu())}


def stream_rates(torch, reps=10):
    """HBM rates of plain torch kernels on this GPU, for reference beside the
    roofline: a read-bound reduction over 1 GiB of fp32 (bytes read per
    second) and a 512 MiB device copy (bytes read + written per second)."""
    big = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    src = torch.ones(1 << 29, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    out = {}
    for name, fn, nbytes in (("read_GBps", lambda: big.sum(), big.numel() * 4),
                             ("copy_GBps", lambda: dst.copy_(src), 2 * src.numel())):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        out[name] = nbytes * reps / (a.elapsed_time(b) / 1e3) / 1e9
    del big, src, dst
    return out


def layers_experiment(lv, synth, torch, workload, n_layers, reps=8, n_calls=16):
    """Decode attention of ``n_layers`` layers per launch (lvq_decode_attn_layers)
    against one layer per launch, on the same caches: each layer is one of
    the workload's rotated cache copies with its own codebooks and query;
    sets of layers rotate so that every call reads cold caches.  Prints one
    JSON line."""
    B, H, d, Tc, G, L = WORKLOADS[workload][:6]
    Hk = WORKLOADS[workload][6] if len(WORKLOADS[workload]) > 6 else H
    T = (max(synth.ragged_lengths(B, seed=1003)) if L == "ragged" else L) + PAGE
    lay0 = lv.lvq_cache_layout(lv.Config(batch=B, n_heads=H, head_dim=d, loop_steps=Tc, group=G,
                                         max_tokens=T, n_kv_heads=Hk if Hk != H else 0))
    per_copy = 2 * lay0["k_index"]["bytes"] + 2 * lay0["k_window"]["bytes"]
    sets = max(2, math.ceil(2 * LLC_BYTES / (per_copy * n_layers)))
    setup = Setup(lv, synth, torch, workload, sets * n_layers)
    dev = torch.device("cuda")
    lay = lv.lvq_cache_layout(setup.cfg)
    layers = []
    for i, c in enumerate(setup.copies):
        layers.append(dict(
            q=setup.q[0, i % setup.Tc].clone(), k_index=c["k_index"], v_index=c["v_index"],
            k_codebook=synth.codebooks(setup.Hk, setup.d, setup.Tc, setup.G, 9000 + 2 * i, device=dev),
            v_codebook=synth.codebooks(setup.Hk, setup.d, setup.Tc, setup.G, 9001 + 2 * i, device=dev),
            k_window=c["k_window"], v_window=c["v_window"],
            out=torch.empty(lay["output"]["shape"], dtype=torch.float32, device=dev)))
    ws = torch.zeros(n_layers * lay["workspace_bytes"], dtype=torch.uint8, device=dev)

    def timed(call):
        """mean per-call time over graph replays of n_calls calls"""
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for k in range(n_calls):
                call(k)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            graph.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / (reps * n_calls)

    def multi(k):
        s = (k % sets) * n_layers
        lv.lvq_decode_attn_layers(setup.cfg, k % setup.Tc, layers[s:s + n_layers], setup.ctx,
                                  setup.L, ws)

    def single(k):
        ly = layers[k % len(layers)]
        lv.lvq_decode_attn(setup.cfg, k % setup.Tc, ly["q"], setup.ctx, setup.L, ly["k_index"],
                           ly["v_index"], ly["k_codebook"], ly["v_codebook"], ly["k_window"],
                           ly["v_window"], ws, ly["out"])

    for _ in range(3):
        multi(0)
        single(0)
    torch.cuda.synchronize()
    ms_multi = timed(multi)
    ms_single = timed(single)
    bpl = cache_bytes(setup.Hk, setup.d, setup.Tc, setup.G, setup.lengths)
    per_layer_us = ms_multi * 1e3 / n_layers
    achieved = bpl / (per_layer_us * 1e-6) / 1e9
    log(f"{n_layers} layers per launch: {ms_multi * 1e3:.2f} us per call, {per_layer_us:.2f} us "
        f"per layer ({achieved:.0f} GB/s); one layer per launch: {ms_single * 1e3:.2f} us")
    rec = {
        "metric": f"VQ-KV decode attn, {n_layers} layers per launch: context-token*loop-steps/s",
        "value": sum(setup.lengths) * n_layers / (ms_multi / 1e3),
        "unit": "ctx-token*loop-steps/s",
        "n_gpus": 1,
        "higher_is_better": True,
        "dtype": "bf16/fp16->fp32",
        "data": "synthetic (seeded loop-correlated K/V encoded by the HIP encoder, N(0,1) codebooks per layer)",
        "config": {"workload": workload, "layers_per_call": n_layers, "cache_sets": sets,
                   "heads": setup.H, "head_dim": setup.d, "group": setup.G,
                   "context": sum(setup.lengths)},
        "per_call_us": ms_multi * 1e3,
        "per_layer_us": per_layer_us,
        "single_layer_call_us": ms_single * 1e3,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "bytes_per_layer": bpl},
    }
    print(json.dumps(rec), flush=True)


def loop_axis_experiment(lv, synth, torch, heads=8, d=128, n_train=8192, n_test=2048,
                         iters=8, seed=2024):
    """The equal-bits comparison of the LoopVQ project page ("Component 1 --
    Loop-axis vector quantization") on the synthetic looped-model keys: k-means
    codebooks with the HIP encoder as the assignment step, test-set error per
    element for 4-step loop-axis grouping and for channel-only grouping."""
    from sub_bit_vq_amd import kmeans
    x = synth.loop_correlated_kv(n_train + n_test, heads, 4, d, seed)
    assign = kmeans.device_assign(lv)
    rows = []
    for group in (16, 32):
        t0 = time.perf_counter()
        r = kmeans.loop_axis_comparison(x[:n_train], x[n_train:], group, iters, seed + group,
                                        assign)
        log(f"G={group}: loop axis {r['mse_loop_axis']:.5f}, channels only "
            f"{r['mse_channels_only']:.5f} ({time.perf_counter() - t0:.1f} s)")
        rows.append({k: v for k, v in r.items() if not k.startswith("train_history")}
                    | {"group": group})
    print(json.dumps({"experiment": "loop_axis_vs_channels_equal_bits", "heads": heads,
                      "head_dim": d, "loop_steps": 4, "train_tokens": n_train,
                      "test_tokens": n_test, "iterations": iters,
                      "data": "synthetic loop-correlated keys (base N(0,1) + N(0, (0.1(l+1))^2))",
                      "results": rows}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="ouro1p4b_layer_32k_0p5bit", choices=sorted(WORKLOADS))
    ap.add_argument("--rotate", type=int, default=0, help="cache copies (0 = auto, >= 2x LLC)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="time only the main workload (not the other configurations)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying")
    ap.add_argument("--decode-only", action="store_true",
                    help="time the 32 decode calls of a step without the page encode")
    ap.add_argument("--profile-decode", type=int, default=0,
                    help="only run N decode launches (for rocprofv3 runs) and exit")
    ap.add_argument("--profile-encode", type=int, default=0,
                    help="only run N prefill encodes of 32768 tokens (for rocprofv3 runs) and exit")
    ap.add_argument("--profile-encode-kv", type=int, default=0,
                    help="only run N prefill encodes of 32768 tokens, K and V in one launch (for "
                         "rocprofv3 runs) and exit")
    ap.add_argument("--profile-page", type=int, default=0,
                    help="only run N page encodes (8 tokens, K and V in one launch; for "
                         "rocprofv3 runs) and exit")
    ap.add_argument("--layers", type=int, default=0,
                    help="time lvq_decode_attn_layers with this many layers per launch "
                         "(prints its own JSON line)")
    ap.add_argument("--loop-axis", action="store_true",
                    help="instead of the benchmark: the equal-bits loop-axis vs channel-only "
                         "k-means comparison (encoder as the assignment step); prints one JSON line")
    ap.add_argument("--copy-calibrate", action="store_true",
                    help="with --profile-*: also run plain 512 MiB device copies, whose HBM "
                         "counters give the scale of FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the LoopVQ path shards by heads or sequences with no exchange).", file=sys.stderr)
        sys.exit(2)

    import torch
    from sub_bit_vq_amd import loopvq as lv
    from sub_bit_vq_amd import synth

    lv.library()
    if args.loop_axis:
        loop_axis_experiment(lv, synth, torch)
        return
    if args.layers:
        layers_experiment(lv, synth, torch, args.workload, args.layers)
        return
    log(f"workload {args.workload}: setup")
    setup = Setup(lv, synth, torch, args.workload, args.rotate)
    log(f"rotation over {setup.rotate} cache copies, "
        f"{lv.lvq_decode_splits(setup.cfg, setup.L)} workgroups per (sequence, head), "
        f"{lv.lvq_decode_window_groups(setup.cfg, setup.L)} of them on the window slots")

    if args.profile_decode or args.profile_encode or args.profile_page or args.profile_encode_kv:
        if args.copy_calibrate:
            src = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
            dst = torch.empty_like(src)
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
            log("ran 3 copies of 536870912 bytes")
            del src, dst
        for i in range(args.profile_decode):
            setup.decode(i % PAGE, i % setup.Tc)
        if args.profile_encode or args.profile_encode_kv:
            enc = PrefillEncode(lv, synth, torch, setup)
            for _ in range(args.profile_encode):
                enc.run()
            for _ in range(args.profile_encode_kv):
                enc.run_kv()
        for _ in range(args.profile_page):
            setup.page_encode()
        torch.cuda.synchronize()
        log(f"ran {args.profile_decode} decode launches, {args.profile_encode} prefill encodes, "
            f"{args.profile_encode_kv} K+V prefill encodes, {args.profile_page} page encodes")
        return

    # warmup (eager), then capture exactly the timed steps in one graph (the
    # cache copies keep rotating from call to call)
    for _ in range(max(1, args.warmup)):
        setup.step(args.decode_only)
    torch.cuda.synchronize()
    steps = max(1, args.steps)
    graph = None
    if not args.no_graph:
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for _ in range(steps):
                setup.step(args.decode_only)
        torch.cuda.synchronize()
        graph.replay()                                # untimed: first replay
        torch.cuda.synchronize()
        log(f"graph: {steps} steps")
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    if graph is not None:
        graph.replay()
    else:
        for _ in range(steps):
            setup.step(args.decode_only)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    ms_per_step = ms / steps
    value = setup.tokens_steps_per_step / (ms_per_step / 1e3)
    log(f"{steps} steps in {ms:.3f} ms ({ms_per_step * 1e3:.1f} us/step)")

    spread = {}
    mean_ms = decode_kernel_time_ms(setup, torch, spread=spread)
    bpl = cache_bytes(setup.Hk, setup.d, setup.Tc, setup.G, setup.lengths)
    achieved = bpl / (mean_ms / 1e3) / 1e9
    log(f"decode launch: mean {mean_ms * 1e3:.2f} us (replay median {spread['median_ms'] * 1e3:.2f}, "
        f"min {spread['min_ms'] * 1e3:.2f}), {achieved:.0f} GB/s on {bpl} cache bytes")

    checks = [] if args.no_cpu_baseline else [parity_checks(setup, torch, args.workload, heads=(0, 2))]
    workloads = {}
    if not args.no_secondary:
        workloads, more = secondary_workloads(lv, synth, torch, args.workload, setup,
                                              with_checks=not args.no_cpu_baseline)
        checks += more

    streams = stream_rates(torch)
    cb_bytes = 2 * setup.Hk * 256 * setup.d * 2     # the K and V slices of step t, bf16
    log(f"stream rates on this GPU: read {streams['read_GBps']:.0f} GB/s, copy {streams['copy_GBps']:.0f} GB/s")

    cpu = None if args.no_cpu_baseline else cpu_baseline(setup, torch, checks)
    if cpu is not None:
        for name, res in cpu["parity"].items():
            if name in workloads:
                workloads[name]["parity"] = res
        log("parity samples: " + ", ".join(
            f"{k}: {v.get('max_rel_err', v.get('indices_differing'))}" for k, v in cpu["parity"].items()))
    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "ctx-token*loop-steps/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16/fp16->fp32",
        "data": "synthetic (seeded loop-correlated K/V, N(0,1) codebooks)",
        "config": {
            "workload": args.workload,
            "batch": setup.B, "heads": setup.H, "kv_heads": setup.Hk, "head_dim": setup.d,
            "loop_steps": setup.Tc,
            "group": setup.G, "context": setup.L if setup.B == 1 else sum(setup.lengths),
            "n_sink": N_SINK, "n_recent": N_RECENT,
            "step": ("8 tokens x 4 loop-step decodes" if args.decode_only else
                     "8 tokens x 4 loop-step decodes + 8-token page encode (K and V, one launch)"),
            "cache_copies": setup.rotate, "graph": graph is not None,
            "arithmetic": ("uint8 indices; score tables fp32 from bf16 products; value terms "
                           "fp16 codewords x fp16 weights; fp32 accumulation and output"),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": ("lvq_decode_attn: decode_main<S=%d,cg=%d,bf16>, one launch per call"
                       % (setup.d // (setup.G // setup.Tc), setup.G // setup.Tc)),
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": counters_traffic(args.workload),
            "bytes_per_launch": bpl,
            "mean_launch_us": mean_ms * 1e3,
            "median_launch_us": spread["median_ms"] * 1e3,     # over the timed replays
            "min_launch_us": spread["min_ms"] * 1e3,
            # secondary: with the codebook slices of step t counted, and
            # against the HBM rates of plain torch kernels measured here (a
            # device copy moves the most bytes per second of the two)
            "achieved_with_codebook_slices": (bpl + cb_bytes) / (mean_ms / 1e3) / 1e9,
            "measured_read_GBps": streams["read_GBps"],
            "measured_copy_GBps": streams["copy_GBps"],
            "frac_of_measured_copy": achieved / streams["copy_GBps"],
        },
        "cpu_baseline": cpu,
        "parity": None if cpu is None else cpu["parity"].get(args.workload),
        "workloads": workloads,
    }
    print(json.dumps(rec), flush=True)


SECONDARY = ("ouro1p4b_layer_32k_0p25bit", "batch64_ragged_0p5bit", "gqa32q8kv_32k_0p5bit")


def secondary_workloads(lv, synth, torch, main_workload, setup, with_checks=True):
    """The other configurations, each timed like the main one (mean decode
    launch over graph replays of 64 back-to-back launches on rotated cache
    copies) and the K + V prefill encode of 32768 tokens; with their parity
    samples for the CPU-baseline leg."""
    out, checks = {}, []
    for wl in SECONDARY:
        if wl == main_workload:
            continue
        log(f"workload {wl}: setup")
        s2 = Setup(lv, synth, torch, wl, 0)
        spread = {}
        ms = decode_kernel_time_ms(s2, torch, spread=spread)
        nbytes = cache_bytes(s2.Hk, s2.d, s2.Tc, s2.G, s2.lengths)
        gbs = nbytes / (ms / 1e3) / 1e9
        out[wl] = {
            "metric": "context-token*loop-steps/s per decode call", "value": sum(s2.lengths) / (ms / 1e3),
            "mean_launch_us": ms * 1e3, "median_launch_us": spread["median_ms"] * 1e3,
            "min_launch_us": spread["min_ms"] * 1e3, "bytes_per_launch": nbytes, "GBps": gbs,
            "frac": gbs / HBM_PEAK_GBS, "batch": s2.B, "heads": s2.H, "kv_heads": s2.Hk, "group": s2.G,
            "context": sum(s2.lengths),
            # workgroups per (sequence, head group) and query heads per workgroup
            "workgroups_per_head_group": lv.lvq_decode_splits(s2.cfg, s2.L),
            "heads_per_workgroup": lv.lvq_decode_heads_per_workgroup(s2.cfg, 1, s2.L),
            "cache_copies": s2.rotate,
        }
        log(f"  decode launch {ms * 1e3:.2f} us, {gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.3f} of peak)")
        if with_checks:
            if s2.B > 1:
                picked = {}
                for b, L in enumerate(s2.lengths):
                    picked.setdefault(L, b)
                checks.append(parity_checks(s2, torch, wl, seqs=sorted(picked.values())))
            else:
                checks.append(parity_checks(s2, torch, wl, heads=(0, 2)))
        del s2
        torch.cuda.empty_cache()
    # prefill encode: 32768 tokens of K and V in one launch, and one tensor
    enc = PrefillEncode(lv, synth, torch, setup)
    ms_kv = prefill_encode_time_ms(enc, torch, kv=True)
    ms_k = prefill_encode_time_ms(enc, torch)
    nb = encode_bytes(enc.N, enc.H, enc.d, enc.Tc, enc.G, 2)
    fl = encode_mfma_flops(enc.N, enc.H, enc.d, enc.Tc, enc.G, 2)
    fl_issued = encode_mfma_flops(enc.N, enc.H, enc.d, enc.Tc, enc.G, 2, issued=True)
    gbs = nb / (ms_kv / 1e3) / 1e9
    tfl = fl / (ms_kv / 1e3) / 1e12
    out["prefill_encode_kv_32k_0p5bit"] = {
        "metric": "tokens/s (K and V, 16 KV heads, 4 loop steps, d 128)", "value": enc.N / (ms_kv / 1e3),
        "mean_launch_us": ms_kv * 1e3, "bytes_per_launch": nb, "GBps": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
        "mfma_flops_per_launch": fl, "TFLOPs": tfl, "frac_mfma_bf16": tfl / MFMA_BF16_PEAK_TFLOPS,
        "mfma_flops_issued_per_launch": fl_issued,
        "frac_mfma_bf16_issued": fl_issued / (ms_kv / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "one_tensor_us": ms_k * 1e3, "tokens": enc.N,
    }
    log(f"prefill encode K+V ({enc.N} tokens): {ms_kv * 1e3:.1f} us, {gbs:.0f} GB/s "
        f"({gbs / HBM_PEAK_GBS:.3f} of HBM), {tfl:.0f} TFLOP/s ({tfl / MFMA_BF16_PEAK_TFLOPS:.3f} of bf16 MFMA); "
        f"one tensor {ms_k * 1e3:.1f} us")
    if with_checks:
        # bit-exact sample: the first 64 tokens of K (every head and sub-vector)
        n = 64
        checks.append({"name": "prefill_encode_kv_32k_0p5bit", "kind": "encode",
                       "gpu": enc.idx[:, :, :n].cpu().numpy(), "rows": f"tokens 0..{n - 1} of K, every head",
                       "oracle": dict(x=enc.x[:n].cpu(), codebook=enc.cb.cpu(), n_heads=enc.H,
                                      head_dim=enc.d, loop_steps=enc.Tc, group=enc.G)})
    del enc
    torch.cuda.empty_cache()
    return out, checks


if __name__ == "__main__":
    main()

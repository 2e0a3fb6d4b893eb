"""CPU oracle for LoopVQ -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It wraps ``loopvq_oracle.c`` (plain C,
built with ``gcc -O2 -ffp-contract=off``) through ctypes and takes numpy
arrays or CPU torch tensors; bf16 data is passed as its raw 16-bit patterns.

Functions (each cites the LoopVQ passage it follows in the C source):

* :func:`encode` -- brute-force nearest codeword, fp32 sequential sums,
  lowest index on ties (E1-E4);
* :func:`decode_attn` -- dequantise the VQ tokens through slice t of the
  codebooks, add the bf16 sink/recent windows, dense fp64 attention (D1-D5);
* :func:`attend` -- the dense fp64 attention alone (D3-D5).
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import pathlib
import subprocess

import numpy as np

_HERE = pathlib.Path(__file__).resolve().parent
_SRC = _HERE / "loopvq_oracle.c"
_LIB_PATH = _HERE / "liboracle.so"
_lib = None

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-fPIC", "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(force: bool = True) -> pathlib.Path:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    global _lib
    if force or not _LIB_PATH.exists():
        tmp = _LIB_PATH.with_suffix(".so.tmp")
        subprocess.run(["gcc", *CFLAGS, str(_SRC), "-o", str(tmp), "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
        _lib = None
    return _LIB_PATH


def _bind(path):
    lib = ctypes.CDLL(str(path))
    i32, i64, vp, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
    lib.lvqo_encode.restype = i32
    lib.lvqo_encode.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, i64, i64, i64, i64,
                                vp, i64, i64, i64, i64, i32]
    lib.lvqo_attend.restype = None
    lib.lvqo_attend.argtypes = [i64, i32, vp, vp, vp, dbl, vp, vp]
    lib.lvqo_decode_attn.restype = i32
    lib.lvqo_decode_attn.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32, i64, i32, i32,
                                     vp, vp, vp, vp, vp, vp, vp, vp, vp, dbl, vp, vp,
                                     i32, i32, i32]
    lib.lvqo_max_threads.restype = i32
    lib.lvqo_max_threads.argtypes = []
    return lib


def _load():
    global _lib
    if _lib is None:
        if not _LIB_PATH.exists() or _LIB_PATH.stat().st_mtime < _SRC.stat().st_mtime:
            build(force=True)
        _lib = _bind(_LIB_PATH)
    return _lib


@contextlib.contextmanager
def use_library(path):
    """Temporarily route every call to another build of the oracle source
    (the mutation tests load deliberately broken copies this way)."""
    global _lib
    saved = _load()
    _lib = _bind(path)
    try:
        yield
    finally:
        _lib = saved


def max_threads() -> int:
    return int(_load().lvqo_max_threads())


def _np(a, dtype=None):
    """numpy view of an array or CPU torch tensor; bf16 tensors -> uint16 bits."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().contiguous()
            if a.dtype == torch.bfloat16:
                a = a.view(torch.int16).numpy().view(np.uint16)
            else:
                a = a.numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(a)
    if dtype is not None and a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _codebook(cb):
    a = _np(cb)
    if a.dtype == np.uint16:
        return a, 1
    if a.dtype == np.float32:
        return a, 0
    raise TypeError("codebook must be bf16 (uint16 bits) or float32")


def encode(x, codebook, *, n_heads, head_dim, loop_steps, group, n_loops=None, index=None,
           t_max=None, seq=0, first_token=0, threads=None):
    """Encode ``x`` (bf16 ``[n][H][R][d]``, R = ``n_loops`` or ``loop_steps``)
    into ``index`` (uint8 ``[B][H][t_max][S]``, or ``[R/Tc][B][H][t_max][S]``
    when R > Tc; allocated with B = seq + 1 and t_max = first_token + n if
    None).  Returns the index array."""
    xa = _np(x, np.uint16)
    n = xa.shape[0]
    cb, is_bf16 = _codebook(codebook)
    cg = group // loop_steps
    S = head_dim // cg
    R = n_loops or loop_steps
    NG = R // loop_steps
    if index is None:
        t_max = first_token + n if t_max is None else t_max
        shape = (seq + 1, n_heads, t_max, S)
        index = np.zeros(shape if NG == 1 else (NG,) + shape, np.uint8)
    else:
        index = _np(index, np.uint8)
        if index.ndim != (4 if NG == 1 else 5):
            raise ValueError(f"index: expected {4 if NG == 1 else 5} dimensions")
    batch, t_max = index.shape[-4], index.shape[-2]
    assert xa.shape == (n, n_heads, R, head_dim), xa.shape
    st = (n_heads * R * head_dim, R * head_dim, head_dim)
    rc = _load().lvqo_encode(n_heads, head_dim, loop_steps, R, group, is_bf16, _ptr(cb), _ptr(xa),
                             n, st[0], st[1], st[2], _ptr(index), batch, t_max, seq, first_token,
                             threads or max_threads())
    if rc != 0:
        raise ValueError(f"lvqo_encode rejected its arguments ({rc})")
    return index


def attend(q, K, V, sm_scale, want_p=False):
    """Dense fp64 attention of one query ``q[d]`` over ``K, V [L][d]``."""
    qa = np.ascontiguousarray(q, np.float64)
    Ka = np.ascontiguousarray(K, np.float64)
    Va = np.ascontiguousarray(V, np.float64)
    L, d = Ka.shape
    out = np.zeros(d, np.float64)
    p = np.zeros(max(L, 1), np.float64) if want_p else None
    _load().lvqo_attend(L, d, _ptr(qa), _ptr(Ka), _ptr(Va), float(sm_scale), _ptr(out), _ptr(p))
    return (out, p[:L]) if want_p else out


def decode_attn(*, loop_step, q, ctx_len, k_index, v_index, k_codebook, v_codebook,
                k_window, v_window, n_sink, n_recent, group, sm_scale=1.0, vq_len=None,
                want_p=False, heads=None, threads=None, loop_steps=None):
    """fp64 decode attention (D1-D5).  Shapes: q bf16 [B][H][d]; ctx_len int32 [B];
    index uint8 [B][Hk][t_max][S]; codebooks [Tc][Hk][256][S][cg]; windows bf16
    [B][Tc][Hk][n_sink+n_recent][d], where Hk (taken from the index cache)
    divides H and query head h reads KV head h // (H // Hk).  A model with R
    loop steps (codebooks and windows with R slices, R a multiple of
    ``loop_steps``) has index caches [R/Tc][B][Hk][t_max][S] and decodes
    loop_step in [0, R).  Returns out fp64 [B][H][d] (and p fp64
    [B][H][t_max] when ``want_p``)."""
    qa = _np(q, np.uint16)
    B, H, d = qa.shape
    ki, vi = _np(k_index, np.uint8), _np(v_index, np.uint8)
    Hk, t_max = ki.shape[-3], ki.shape[-2]
    kcb, kb = _codebook(k_codebook)
    vcb, vb = _codebook(v_codebook)
    if kb != vb:
        raise TypeError("K and V codebooks must share a dtype")
    R = kcb.shape[0]
    Tc = loop_steps or R
    kw, vw = _np(k_window, np.uint16), _np(v_window, np.uint16)
    cl = np.ascontiguousarray(np.asarray(ctx_len, np.int32))
    vl = None if vq_len is None else np.ascontiguousarray(np.asarray(vq_len, np.int32))
    out = np.zeros((B, H, d), np.float64)
    p = np.zeros((B, H, t_max), np.float64) if want_p else None
    h0, h1 = (0, H) if heads is None else heads
    rc = _load().lvqo_decode_attn(B, H, Hk, d, Tc, R, group, n_sink, n_recent, t_max, kb, loop_step,
                                  _ptr(qa), _ptr(cl), _ptr(vl), _ptr(ki), _ptr(vi), _ptr(kcb),
                                  _ptr(vcb), _ptr(kw), _ptr(vw), float(sm_scale), _ptr(out),
                                  _ptr(p), h0, h1, threads or max_threads())
    if rc != 0:
        raise ValueError(f"lvqo_decode_attn rejected its arguments ({rc})")
    return (out, p) if want_p else out

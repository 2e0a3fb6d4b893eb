"""Thin Python binding of libloopvq (``include/loopvq.h``).

Argument marshalling only: torch tensors are checked against the layout the
library documents and passed as raw device pointers on torch's current HIP
stream.  Every step of the computation runs in the library's kernels; there is
no fallback, and a missing ``libloopvq.so`` raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import pathlib

import torch

_HERE = pathlib.Path(__file__).resolve().parent
LIB_PATH = _HERE / "libloopvq.so"

LVQ_OK, LVQ_ERR_INVALID_ARG, LVQ_ERR_UNSUPPORTED, LVQ_ERR_WORKSPACE, LVQ_ERR_HIP = range(5)
LVQ_F32, LVQ_BF16 = 0, 1
LVQ_MAX_SPLITS = 64
LVQ_MAX_WINDOW_GROUPS = 4
LVQ_MAX_WINDOW_SLOTS = 1 << 24
LVQ_MAX_LAYERS = 4096
N_CODES = 256

LVQ_STATUS_MERGE_TIMEOUT, LVQ_STATUS_VALUE_RANGE = 1, 2
# the workspace opens with a 256-byte header (the status word) followed by
# one fixed-size block per (layer, b, h)
WORKSPACE_HEADER_BYTES = 256

LVQ_NOALLOC_MAX_HEADS = 256

EXPORTS = ("lvq_cache_layout", "lvq_encode", "lvq_encode_kv", "lvq_decode_attn",
           "lvq_decode_attn_noalloc", "lvq_decode_attn_layers", "lvq_decode_status", "lvq_decode_role",
           "lvq_decode_splits", "lvq_decode_window_groups", "lvq_decode_heads_per_workgroup",
           "lvq_status_string",
           "lvq_encode_screen")


class LoopVQError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {lvq_status_string(status)} (status {status})")


class _Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_heads", "head_dim", "loop_steps", "group", "n_sink", "n_recent",
        "max_tokens", "codebook_dtype", "decode_splits", "n_kv_heads", "n_loops",
        "decode_window_groups", "decode_poll_limit", "decode_heads_per_group")]


class _DecodeLayer(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "q", "k_index", "v_index", "k_codebook", "v_codebook", "k_window", "v_window", "out")]


class _Tensor(ctypes.Structure):
    _fields_ = [("ndim", ctypes.c_int32), ("shape", ctypes.c_int64 * 6),
                ("stride", ctypes.c_int64 * 6), ("bytes", ctypes.c_uint64)]


class _Layout(ctypes.Structure):
    _fields_ = [("n_sub", ctypes.c_int32), ("sub_channels", ctypes.c_int32),
                ("n_codes", ctypes.c_int32), ("window_slots", ctypes.c_int32),
                ("bits_per_element", ctypes.c_double), ("compression_vs_bf16", ctypes.c_double),
                ("read_reduction_per_step", ctypes.c_double),
                ("k_index", _Tensor), ("v_index", _Tensor), ("k_codebook", _Tensor),
                ("v_codebook", _Tensor), ("k_window", _Tensor), ("v_window", _Tensor),
                ("query", _Tensor), ("output", _Tensor), ("workspace_bytes", ctypes.c_uint64)]


@dataclasses.dataclass(frozen=True)
class Config:
    """Mirror of ``lvq_config``."""
    batch: int
    n_heads: int
    head_dim: int
    loop_steps: int = 4
    group: int = 16
    n_sink: int = 64
    n_recent: int = 256
    max_tokens: int = 0
    codebook_dtype: int = LVQ_BF16
    decode_splits: int = 0
    n_kv_heads: int = 0          # 0: as many KV heads as query heads
    n_loops: int = 0             # 0: the model has loop_steps loop steps
    decode_window_groups: int = 0  # with decode_splits: workgroups taking window slots
    decode_poll_limit: int = 0     # 0: the library's bound of a merger's wait
    decode_heads_per_group: int = 0  # query heads per decode workgroup: 0 library's choice, 1, 2

    @property
    def kv_heads(self) -> int:
        return self.n_kv_heads or self.n_heads

    @property
    def loops(self) -> int:
        return self.n_loops or self.loop_steps

    def c(self) -> _Config:
        return _Config(*(int(getattr(self, f.name)) for f in dataclasses.fields(self)))

    @property
    def torch_codebook_dtype(self):
        return torch.bfloat16 if self.codebook_dtype == LVQ_BF16 else torch.float32


_lib = None


def library() -> ctypes.CDLL:
    """Load libloopvq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m sub_bit_vq_amd.build`")
        lib = ctypes.CDLL(str(LIB_PATH))
        vp, i32, i64, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
        cfgp = ctypes.POINTER(_Config)
        lib.lvq_cache_layout.restype = i32
        lib.lvq_cache_layout.argtypes = [cfgp, ctypes.POINTER(_Layout)]
        lib.lvq_encode.restype = i32
        lib.lvq_encode.argtypes = [cfgp, vp, ctypes.POINTER(i64), i64, vp, vp, i32, i64, vp]
        lib.lvq_encode_screen.restype = i32
        lib.lvq_encode_screen.argtypes = [cfgp, vp, ctypes.POINTER(i64), i64, vp, vp, i32, i64, vp, vp]
        lib.lvq_encode_kv.restype = i32
        lib.lvq_encode_kv.argtypes = [cfgp, vp, vp, ctypes.POINTER(i64), i64, vp, vp, vp, vp,
                                      i32, i64, vp]
        lib.lvq_decode_attn.restype = i32
        lib.lvq_decode_attn.argtypes = [cfgp, i32, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp,
                                        ctypes.c_float, vp, u64, vp, vp]
        lib.lvq_decode_attn_noalloc.restype = i32
        lib.lvq_decode_attn_noalloc.argtypes = [cfgp, i32, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp,
                                                ctypes.c_float, vp, vp]
        lib.lvq_decode_attn_layers.restype = i32
        lib.lvq_decode_attn_layers.argtypes = [cfgp, i32, i32, ctypes.POINTER(_DecodeLayer), vp, vp,
                                               i32, ctypes.c_float, vp, u64, vp]
        lib.lvq_decode_status.restype = i32
        lib.lvq_decode_status.argtypes = [vp, ctypes.POINTER(ctypes.c_uint32), i32, vp]
        lib.lvq_decode_role.restype = i32
        lib.lvq_decode_role.argtypes = [cfgp, i32, i32, i32, ctypes.POINTER(i32),
                                        ctypes.POINTER(i32), ctypes.POINTER(i32)]
        lib.lvq_decode_splits.restype = i32
        lib.lvq_decode_splits.argtypes = [cfgp, i32]
        lib.lvq_decode_window_groups.restype = i32
        lib.lvq_decode_window_groups.argtypes = [cfgp, i32]
        lib.lvq_decode_heads_per_workgroup.restype = i32
        lib.lvq_decode_heads_per_workgroup.argtypes = [cfgp, i32, i32]
        lib.lvq_status_string.restype = ctypes.c_char_p
        lib.lvq_status_string.argtypes = [i32]
        _lib = lib
    return _lib


def lvq_status_string(status: int) -> str:
    return library().lvq_status_string(int(status)).decode()


def _tensor_dict(t: _Tensor) -> dict:
    return {"shape": tuple(t.shape[: t.ndim]), "stride": tuple(t.stride[: t.ndim]),
            "bytes": int(t.bytes)}


def lvq_cache_layout(cfg: Config) -> dict:
    """Sizes and shapes of every buffer (host arithmetic only)."""
    lay = _Layout()
    st = library().lvq_cache_layout(ctypes.byref(cfg.c()), ctypes.byref(lay))
    if st != LVQ_OK:
        raise LoopVQError("lvq_cache_layout", st)
    out = {f: getattr(lay, f) for f in ("n_sub", "sub_channels", "n_codes", "window_slots",
                                         "bits_per_element", "compression_vs_bf16",
                                         "read_reduction_per_step", "workspace_bytes")}
    for f in ("k_index", "v_index", "k_codebook", "v_codebook", "k_window", "v_window", "query",
              "output"):
        out[f] = _tensor_dict(getattr(lay, f))
    return out


def lvq_decode_splits(cfg: Config, max_ctx_len: int) -> int:
    return int(library().lvq_decode_splits(ctypes.byref(cfg.c()), int(max_ctx_len)))


def lvq_decode_window_groups(cfg: Config, max_ctx_len: int) -> int:
    return int(library().lvq_decode_window_groups(ctypes.byref(cfg.c()), int(max_ctx_len)))


def lvq_decode_heads_per_workgroup(cfg: Config, n_layers: int, max_ctx_len: int) -> int:
    return int(library().lvq_decode_heads_per_workgroup(ctypes.byref(cfg.c()), int(n_layers),
                                                        int(max_ctx_len)))


def lvq_decode_role(cfg: Config, n_layers: int, max_ctx_len: int, workgroup: int):
    """(role, layer, seq, head) of a decode workgroup (host arithmetic), or
    None for an invalid workgroup index or config."""
    ly, sq, hd = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    r = library().lvq_decode_role(ctypes.byref(cfg.c()), int(n_layers), int(max_ctx_len),
                                  int(workgroup), ctypes.byref(ly), ctypes.byref(sq),
                                  ctypes.byref(hd))
    return None if r < 0 else (int(r), ly.value, sq.value, hd.value)


def lvq_decode_status(workspace: torch.Tensor, clear: bool = False, stream=None) -> int:
    """Status flags (``LVQ_STATUS_*``) the decode calls set in ``workspace``;
    waits for the stream.  ``clear`` zeroes them."""
    flags = ctypes.c_uint32()
    st = library().lvq_decode_status(_dev_ptr(workspace, "workspace"), ctypes.byref(flags),
                                     int(bool(clear)), _stream(stream))
    if st != LVQ_OK:
        raise LoopVQError("lvq_decode_status", st)
    return int(flags.value)


def _dev_ptr(t, name, dtype=None, shape=None, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def lvq_encode(cfg: Config, x: torch.Tensor, codebook: torch.Tensor, index_cache: torch.Tensor,
               seq: int = 0, first_token: int = 0, stream=None) -> None:
    """Encode bf16 ``x`` ``[n][Hk][R][d]`` (KV heads, every loop step of the
    model; any element strides with contiguous channels) into rows
    ``[first_token, first_token + n)`` of sequence ``seq`` of every group."""
    lay = lvq_cache_layout(cfg)
    xp = _encode_input(cfg, x, "x")
    strides = (ctypes.c_int64 * 3)(x.stride(0), x.stride(1), x.stride(2))
    cbp = _dev_ptr(codebook, "codebook", cfg.torch_codebook_dtype, lay["k_codebook"]["shape"])
    ip = _dev_ptr(index_cache, "index_cache", torch.uint8, lay["k_index"]["shape"])
    st = library().lvq_encode(ctypes.byref(cfg.c()), xp, strides, int(x.shape[0]), cbp, ip,
                              int(seq), int(first_token), _stream(stream))
    if st != LVQ_OK:
        raise LoopVQError("lvq_encode", st)


def lvq_encode_screen(cfg: Config, x: torch.Tensor, codebook: torch.Tensor,
                      index_cache: torch.Tensor, screen: torch.Tensor, seq: int = 0,
                      first_token: int = 0, stream=None) -> None:
    """:func:`lvq_encode` through the MFMA screen at any length, also storing
    every screen value ``|c_k|^2 - 2 x.c_k`` into fp32 ``screen``
    ``[n][Hk][S][256]`` (diagnostic, ``include/loopvq_diag.h``)."""
    lay = lvq_cache_layout(cfg)
    xp = _encode_input(cfg, x, "x")
    strides = (ctypes.c_int64 * 3)(x.stride(0), x.stride(1), x.stride(2))
    cbp = _dev_ptr(codebook, "codebook", cfg.torch_codebook_dtype, lay["k_codebook"]["shape"])
    ip = _dev_ptr(index_cache, "index_cache", torch.uint8, lay["k_index"]["shape"])
    sp = _dev_ptr(screen, "screen", torch.float32,
                  (x.shape[0], cfg.kv_heads, lay["n_sub"], N_CODES))
    st = library().lvq_encode_screen(ctypes.byref(cfg.c()), xp, strides, int(x.shape[0]), cbp, ip,
                                     int(seq), int(first_token), sp, _stream(stream))
    if st != LVQ_OK:
        raise LoopVQError("lvq_encode_screen", st)


def _encode_input(cfg: Config, x: torch.Tensor, name: str):
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda" or x.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be a bf16 device tensor")
    if x.dim() != 4 or tuple(x.shape[1:]) != (cfg.kv_heads, cfg.loops, cfg.head_dim):
        raise ValueError(f"{name}: expected [n][{cfg.kv_heads}][{cfg.loops}][{cfg.head_dim}]")
    if x.stride(3) != 1:
        raise ValueError(f"{name}: channels must be contiguous")
    return ctypes.c_void_p(x.data_ptr())


def lvq_encode_kv(cfg: Config, k_x: torch.Tensor, v_x: torch.Tensor, k_codebook: torch.Tensor,
                  v_codebook: torch.Tensor, k_index: torch.Tensor, v_index: torch.Tensor,
                  seq: int = 0, first_token: int = 0, stream=None) -> None:
    """Encode the K and V of one run of tokens in one launch (same shapes and
    strides for both inputs, as for a page of the bf16 window buffers)."""
    lay = lvq_cache_layout(cfg)
    kx, vx = _encode_input(cfg, k_x, "k_x"), _encode_input(cfg, v_x, "v_x")
    if tuple(k_x.shape) != tuple(v_x.shape) or k_x.stride() != v_x.stride():
        raise ValueError("k_x and v_x must have the same shape and strides")
    strides = (ctypes.c_int64 * 3)(k_x.stride(0), k_x.stride(1), k_x.stride(2))
    args = [_dev_ptr(k_codebook, "k_codebook", cfg.torch_codebook_dtype, lay["k_codebook"]["shape"]),
            _dev_ptr(v_codebook, "v_codebook", cfg.torch_codebook_dtype, lay["v_codebook"]["shape"]),
            _dev_ptr(k_index, "k_index", torch.uint8, lay["k_index"]["shape"]),
            _dev_ptr(v_index, "v_index", torch.uint8, lay["v_index"]["shape"])]
    st = library().lvq_encode_kv(ctypes.byref(cfg.c()), kx, vx, strides, int(k_x.shape[0]), *args,
                                 int(seq), int(first_token), _stream(stream))
    if st != LVQ_OK:
        raise LoopVQError("lvq_encode_kv", st)


def lvq_decode_attn(cfg: Config, loop_step: int, q: torch.Tensor, ctx_len: torch.Tensor,
                    max_ctx_len: int, k_index, v_index, k_codebook, v_codebook, k_window,
                    v_window, workspace: torch.Tensor, out: torch.Tensor, sm_scale: float = 1.0,
                    vq_len: torch.Tensor | None = None, stream=None) -> None:
    """Decode attention of ``loop_step``; writes fp32 ``out`` ``[B][H][d]``."""
    lay = lvq_cache_layout(cfg)
    B = cfg.batch
    args = [
        _dev_ptr(q, "q", torch.bfloat16, lay["query"]["shape"]),
        _dev_ptr(ctx_len, "ctx_len", torch.int32, (B,)),
        _dev_ptr(vq_len, "vq_len", torch.int32, (B,), allow_none=True),
        int(max_ctx_len),
        _dev_ptr(k_index, "k_index", torch.uint8, lay["k_index"]["shape"]),
        _dev_ptr(v_index, "v_index", torch.uint8, lay["v_index"]["shape"]),
        _dev_ptr(k_codebook, "k_codebook", cfg.torch_codebook_dtype, lay["k_codebook"]["shape"]),
        _dev_ptr(v_codebook, "v_codebook", cfg.torch_codebook_dtype, lay["v_codebook"]["shape"]),
        _dev_ptr(k_window, "k_window", torch.bfloat16, lay["k_window"]["shape"]),
        _dev_ptr(v_window, "v_window", torch.bfloat16, lay["v_window"]["shape"]),
        ctypes.c_float(sm_scale),
        _dev_ptr(workspace, "workspace"),
        ctypes.c_uint64(workspace.numel() * workspace.element_size()),
        _dev_ptr(out, "out", torch.float32, lay["output"]["shape"]),
    ]
    st = library().lvq_decode_attn(ctypes.byref(cfg.c()), int(loop_step), *args, _stream(stream))
    if st != LVQ_OK:
        raise LoopVQError("lvq_decode_attn", st)


def lvq_decode_attn_noalloc(cfg: Config, loop_step: int, q: torch.Tensor, ctx_len: torch.Tensor,
                            max_ctx_len: int, k_index, v_index, k_codebook, v_codebook, k_window,
                            v_window, out: torch.Tensor, sm_scale: float = 1.0,
                            vq_len: torch.Tensor | None = None, stream=None) -> None:
    """:func:`lvq_decode_attn` with the library's static device workspace
    (allocates nothing; calls on one device must not overlap)."""
    lay = lvq_cache_layout(cfg)
    B = cfg.batch
    args = [
        _dev_ptr(q, "q", torch.bfloat16, lay["query"]["shape"]),
        _dev_ptr(ctx_len, "ctx_len", torch.int32, (B,)),
        _dev_ptr(vq_len, "vq_len", torch.int32, (B,), allow_none=True),
        int(max_ctx_len),
        _dev_ptr(k_index, "k_index", torch.uint8, lay["k_index"]["shape"]),
        _dev_ptr(v_index, "v_index", torch.uint8, lay["v_index"]["shape"]),
        _dev_ptr(k_codebook, "k_codebook", cfg.torch_codebook_dtype, lay["k_codebook"]["shape"]),
        _dev_ptr(v_codebook, "v_codebook", cfg.torch_codebook_dtype, lay["v_codebook"]["shape"]),
        _dev_ptr(k_window, "k_window", torch.bfloat16, lay["k_window"]["shape"]),
        _dev_ptr(v_window, "v_window", torch.bfloat16, lay["v_window"]["shape"]),
        ctypes.c_float(sm_scale),
        _dev_ptr(out, "out", torch.float32, lay["output"]["shape"]),
    ]
    st = library().lvq_decode_attn_noalloc(ctypes.byref(cfg.c()), int(loop_step), *args,
                                           _stream(stream))
    if st != LVQ_OK:
        raise LoopVQError("lvq_decode_attn_noalloc", st)


LAYER_KEYS = ("q", "k_index", "v_index", "k_codebook", "v_codebook", "k_window", "v_window", "out")


def _layers_array(cfg: Config, layers):
    lay = lvq_cache_layout(cfg)
    specs = {"q": (torch.bfloat16, lay["query"]["shape"]),
             "k_index": (torch.uint8, lay["k_index"]["shape"]),
             "v_index": (torch.uint8, lay["v_index"]["shape"]),
             "k_codebook": (cfg.torch_codebook_dtype, lay["k_codebook"]["shape"]),
             "v_codebook": (cfg.torch_codebook_dtype, lay["v_codebook"]["shape"]),
             "k_window": (torch.bfloat16, lay["k_window"]["shape"]),
             "v_window": (torch.bfloat16, lay["v_window"]["shape"]),
             "out": (torch.float32, lay["output"]["shape"])}
    arr = (_DecodeLayer * max(1, len(layers)))()
    for i, ly in enumerate(layers):
        for key in LAYER_KEYS:
            dt, shape = specs[key]
            setattr(arr[i], key, _dev_ptr(ly[key], f"layers[{i}].{key}", dt, shape))
    return arr


def lvq_decode_attn_layers(cfg: Config, loop_step: int, layers, ctx_len: torch.Tensor,
                           max_ctx_len: int, workspace: torch.Tensor, sm_scale: float = 1.0,
                           vq_len: torch.Tensor | None = None, stream=None) -> None:
    """Decode attention of ``loop_step`` for several layers at once: each entry
    of ``layers`` maps the keys of ``LAYER_KEYS`` to that layer's buffers (as
    :func:`lvq_decode_attn` takes them); ``workspace`` holds at least
    ``len(layers)`` single-layer workspaces."""
    arr = _layers_array(cfg, layers)
    B = cfg.batch
    st = library().lvq_decode_attn_layers(
        ctypes.byref(cfg.c()), len(layers), int(loop_step), arr,
        _dev_ptr(ctx_len, "ctx_len", torch.int32, (B,)),
        _dev_ptr(vq_len, "vq_len", torch.int32, (B,), allow_none=True), int(max_ctx_len),
        ctypes.c_float(sm_scale), _dev_ptr(workspace, "workspace"),
        ctypes.c_uint64(workspace.numel() * workspace.element_size()), _stream(stream))
    if st != LVQ_OK:
        raise LoopVQError("lvq_decode_attn_layers", st)


def allocate(cfg: Config, device="cuda") -> dict:
    """Zero-filled device buffers for a configuration (index caches, windows,
    workspace and output); codebooks, queries and lengths are the caller's."""
    lay = lvq_cache_layout(cfg)
    z = lambda key, dt: torch.zeros(lay[key]["shape"], dtype=dt, device=device)  # noqa: E731
    return {
        "k_index": z("k_index", torch.uint8), "v_index": z("v_index", torch.uint8),
        "k_window": z("k_window", torch.bfloat16), "v_window": z("v_window", torch.bfloat16),
        "out": z("output", torch.float32),
        "workspace": torch.zeros(int(lay["workspace_bytes"]), dtype=torch.uint8, device=device),
    }


class PreparedDecode:
    """``lvq_decode_attn`` with every buffer marshalled once, for tight serving
    or benchmark loops: a call costs one ctypes transition.  Buffers are
    validated here exactly as :func:`lvq_decode_attn` validates them."""

    def __init__(self, cfg: Config, ctx_len, max_ctx_len, k_index, v_index, k_codebook,
                 v_codebook, k_window, v_window, workspace, out, sm_scale=1.0, vq_len=None):
        lay = lvq_cache_layout(cfg)
        B = cfg.batch
        self._cfg = cfg.c()
        self._qshape = lay["query"]["shape"]
        self._lib = library()
        self._args = (
            _dev_ptr(ctx_len, "ctx_len", torch.int32, (B,)),
            _dev_ptr(vq_len, "vq_len", torch.int32, (B,), allow_none=True),
            int(max_ctx_len),
            _dev_ptr(k_index, "k_index", torch.uint8, lay["k_index"]["shape"]),
            _dev_ptr(v_index, "v_index", torch.uint8, lay["v_index"]["shape"]),
            _dev_ptr(k_codebook, "k_codebook", cfg.torch_codebook_dtype, lay["k_codebook"]["shape"]),
            _dev_ptr(v_codebook, "v_codebook", cfg.torch_codebook_dtype, lay["v_codebook"]["shape"]),
            _dev_ptr(k_window, "k_window", torch.bfloat16, lay["k_window"]["shape"]),
            _dev_ptr(v_window, "v_window", torch.bfloat16, lay["v_window"]["shape"]),
            ctypes.c_float(sm_scale),
            _dev_ptr(workspace, "workspace"),
            ctypes.c_uint64(workspace.numel() * workspace.element_size()),
            _dev_ptr(out, "out", torch.float32, lay["output"]["shape"]),
        )
        self._keep = (ctx_len, vq_len, k_index, v_index, k_codebook, v_codebook, k_window,
                      v_window, workspace, out)

    def __call__(self, loop_step: int, q: torch.Tensor, stream=None) -> None:
        qp = _dev_ptr(q, "q", torch.bfloat16, self._qshape)
        st = self._lib.lvq_decode_attn(ctypes.byref(self._cfg), int(loop_step), qp, *self._args,
                                       _stream(stream))
        if st != LVQ_OK:
            raise LoopVQError("lvq_decode_attn", st)

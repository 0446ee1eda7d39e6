"""Thin ctypes binding of libswa (include/swa.h).

Argument marshalling only: torch tensors are turned into device pointers and
the current HIP stream; every step of the decode path runs in libswa's
kernels.  There is no fallback of any kind: if libswa.so has not been built
the import of this module raises.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libswa.so")

SWA_OK = 0
SWA_ERR_INVALID_ARG = -1
SWA_ERR_UNSUPPORTED = -2
SWA_ERR_WORKSPACE = -3
SWA_ERR_HIP = -4

SWA_F32 = 0
SWA_BF16 = 1
SWA_I8 = 2
SWA_ROPE_INTERLEAVED = 0
SWA_ROPE_HALF = 1

_DTYPE_CODE = {torch.float32: SWA_F32, torch.bfloat16: SWA_BF16}
_DTYPE_NAME = {"f32": SWA_F32, "bf16": SWA_BF16, "i8": SWA_I8}
# torch dtype of the cache buffers: int8 caches are raw bytes (codes, then scales)
_BUFFER_DTYPE = {SWA_F32: torch.float32, SWA_BF16: torch.bfloat16, SWA_I8: torch.uint8}
_STYLE_CODE = {"interleaved": SWA_ROPE_INTERLEAVED, "half": SWA_ROPE_HALF}


class SwaCacheConfig(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("window", ctypes.c_int32),
                ("num_sinks", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("rope_base", ctypes.c_float), ("rope_style", ctypes.c_int32)]


class SwaPagedDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("num_phys_blocks", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class SwaPagerConfig(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("logical_blocks", ctypes.c_int32), ("slots_per_seq", ctypes.c_int32),
                ("num_phys_blocks", ctypes.c_int32), ("dtype", ctypes.c_int32)]


_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_PROTOS = {
    "swa_cache_required_bytes": (ctypes.c_int, [ctypes.POINTER(SwaCacheConfig),
                                                ctypes.POINTER(ctypes.c_size_t),
                                                ctypes.POINTER(ctypes.c_size_t)]),
    "swa_cache_create": (ctypes.c_int, [ctypes.POINTER(SwaCacheConfig), _vp, _vp, _vp,
                                        ctypes.POINTER(_vp)]),
    "swa_cache_reset": (ctypes.c_int, [_vp, _vp]),
    "swa_cache_destroy": (None, [_vp]),
    "kv_append_rope": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _vp, _i32, _vp]),
    "decode_attn_workspace_bytes": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32,
                                                   ctypes.POINTER(ctypes.c_size_t)]),
    "decode_attn_ring": (ctypes.c_int, [_vp, _vp, _i32, ctypes.c_float, _vp, _i32, _vp, _vp,
                                        ctypes.c_size_t, _vp]),
    "decode_step_ring": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, ctypes.c_float, _vp, _i32,
                                        _vp, _vp, ctypes.c_size_t, _vp]),
    "decode_step_ring_shifted": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, ctypes.c_float, _vp,
                                                _i32, _vp, _vp, ctypes.c_size_t, _vp]),
    "swa_pos_advance": (ctypes.c_int, [_vp, _i32, _i32, _vp]),
    "swa_stream_read": (ctypes.c_int, [_vp, ctypes.c_size_t, _vp, ctypes.c_size_t, _vp]),
    "prefill_attn_workspace_bytes": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32,
                                                    ctypes.POINTER(ctypes.c_size_t)]),
    "prefill_attn_ring": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _vp, _i32, ctypes.c_float, _vp,
                                         _i32, _vp, _vp, ctypes.c_size_t, _vp]),
    "swa_pool_required_bytes": (ctypes.c_int, [ctypes.POINTER(SwaPagedDesc),
                                               ctypes.POINTER(ctypes.c_size_t)]),
    "decode_attn_paged": (ctypes.c_int, [ctypes.POINTER(SwaPagedDesc), _vp, _vp, _vp, _vp, _vp,
                                         _vp, ctypes.c_float, _vp, _i32, _vp, _vp,
                                         ctypes.c_size_t, _vp]),
    "decode_attn_paged_noalloc": (ctypes.c_int, [ctypes.POINTER(SwaPagedDesc), _vp, _vp, _vp, _vp,
                                                 _vp, _vp, ctypes.c_float, _vp, _i32, _vp, _vp]),
    "kv_write_paged": (ctypes.c_int, [ctypes.POINTER(SwaPagedDesc), _vp, _vp, _vp, _vp, _vp, _vp,
                                      _i32, ctypes.c_float, _i32, _vp]),
    "swa_blocks_create": (ctypes.c_int, [_i32, _i32, _i32, _i32, ctypes.POINTER(_vp)]),
    "swa_blocks_destroy": (None, [_vp]),
    "swa_blocks_reset": (ctypes.c_int, [_vp]),
    "swa_blocks_sync": (ctypes.c_int, [_vp, _vp, _vp, _vp]),
    "swa_blocks_share_prefix": (ctypes.c_int, [_vp, _i32, _i32, _i32, _vp, _vp, _vp]),
    "swa_blocks_free": (ctypes.c_int, [_vp, _i32, _vp, _vp]),
    "swa_blocks_state": (ctypes.c_int, [_vp, _vp, _vp, _vp, ctypes.POINTER(_i32)]),
    "kv_append_paged": (ctypes.c_int, [_vp, ctypes.POINTER(SwaPagedDesc), _vp, _vp, _vp, _vp, _vp,
                                       _i32, _i32, _vp, _vp, _i32, ctypes.c_float, _i32, _vp]),
    "swa_pager_create": (ctypes.c_int, [ctypes.POINTER(SwaPagerConfig), _vp, _vp, _vp, _vp, _vp,
                                        _vp, _vp, ctypes.POINTER(_vp)]),
    "swa_pager_reset": (ctypes.c_int, [_vp, _vp]),
    "swa_pager_advance": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, ctypes.POINTER(_i32)]),
    "swa_pager_commit": (ctypes.c_int, [_vp, _vp]),
    "swa_pager_stage": (ctypes.c_int, [_vp, _vp, _vp, ctypes.POINTER(_i32)]),
    "swa_pager_decode": (ctypes.c_int, [_vp, _vp, _i32, _vp, ctypes.c_float, _vp, _i32, _vp, _vp,
                                        ctypes.c_size_t, _vp]),
    "swa_pager_workspace_bytes": (ctypes.c_int, [_vp, _i32, ctypes.POINTER(ctypes.c_size_t)]),
    "swa_pager_slot_blocks": (ctypes.c_int, [_vp, _i32, _vp]),
    "swa_pager_destroy": (None, [_vp]),
    "swa_last_error": (ctypes.c_char_p, []),
}
EXPORTED = tuple(_PROTOS)


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m decode_attention_fixed_amd.build`"
                          " (there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _PROTOS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()


class SwaError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn} failed ({code}): {swa_last_error()}")


def _check(fn: str, code: int) -> None:
    if code != SWA_OK:
        raise SwaError(fn, code)


def _invoke(name: str, args: tuple, keep: tuple, prepare: bool):
    """Calls LIB.<name>(*args), or with prepare=True returns a function of no
    arguments that makes that call (the arguments marshalled once, for loops
    that repeat one call on the same buffers; the tensors in `keep` stay alive
    as long as the function)."""
    fn = getattr(LIB, name)
    if not prepare:
        _check(name, fn(*args))
        return None

    def call() -> None:
        code = fn(*args)
        if code != SWA_OK:
            raise SwaError(name, code)
    call.keep = keep
    return call


def swa_last_error() -> str:
    return LIB.swa_last_error().decode()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: torch.Tensor | None, name: str, dtype=None) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


# The C ABI takes bare pointers and cannot see a tensor's extent, so the
# binding checks every tensor against the sizes the call will touch before
# handing its pointer over; a mismatch raises ValueError and nothing runs.

def _expect(t: torch.Tensor | None, name: str, shape: tuple, dtypes) -> None:
    """t (if given) has exactly `shape` and one of `dtypes`."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must be one of {list(dtypes)}, got {t.dtype}")


def _expect_numel(t: torch.Tensor | None, name: str, numel: int, dtype) -> None:
    """t (if given) holds at least `numel` elements of `dtype` (flat views)."""
    if t is None:
        return
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() < numel:
        raise ValueError(f"{name} must hold at least {numel} elements, got {t.numel()}")


def _expect_bytes(t: torch.Tensor | None, name: str, nbytes: int) -> None:
    if t is None:
        return
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name} must hold at least {nbytes} bytes, got {have}")


_OUT_DTYPES = (torch.float32, torch.bfloat16)


def _row_dtype(code: int):
    """torch dtype of the rows and queries handed to a call on a cache or
    pool of element type `code` (int8 caches take bf16 rows)."""
    return torch.float32 if code == SWA_F32 else torch.bfloat16


# ring-cache handle -> its config, recorded by swa_cache_create so that the
# calls on the handle can check their tensors' shapes
_RING_CFG: dict = {}


def _ring_cfg(handle: int):
    return _RING_CFG.get(handle)


# ---------------------------------------------------------------------------
# ring cache
# ---------------------------------------------------------------------------

def make_config(batch: int, num_kv_heads: int, head_dim: int, window: int, num_sinks: int,
                dtype: str = "bf16", rope_base: float = 10000.0,
                rope_style: str = "interleaved") -> SwaCacheConfig:
    return SwaCacheConfig(batch, num_kv_heads, head_dim, window, num_sinks, _DTYPE_NAME[dtype],
                          rope_base, _STYLE_CODE[rope_style])


def swa_cache_required_bytes(cfg: SwaCacheConfig) -> tuple:
    kv, sp = ctypes.c_size_t(), ctypes.c_size_t()
    _check("swa_cache_required_bytes",
           LIB.swa_cache_required_bytes(ctypes.byref(cfg), ctypes.byref(kv), ctypes.byref(sp)))
    return kv.value, sp.value


def swa_cache_create(cfg: SwaCacheConfig, k_cache: torch.Tensor, v_cache: torch.Tensor,
                     slot_pos: torch.Tensor) -> int:
    handle = _vp()
    dt = _BUFFER_DTYPE[cfg.dtype]
    kv_bytes, sp_bytes = swa_cache_required_bytes(cfg)
    _expect_bytes(k_cache, "k_cache", kv_bytes)
    _expect_bytes(v_cache, "v_cache", kv_bytes)
    _expect_bytes(slot_pos, "slot_pos", sp_bytes)
    _check("swa_cache_create",
           LIB.swa_cache_create(ctypes.byref(cfg), _ptr(k_cache, "k_cache", dt),
                                _ptr(v_cache, "v_cache", dt), _ptr(slot_pos, "slot_pos", torch.int32),
                                ctypes.byref(handle)))
    _RING_CFG[handle.value] = SwaCacheConfig(cfg.batch, cfg.num_kv_heads, cfg.head_dim, cfg.window,
                                             cfg.num_sinks, cfg.dtype, cfg.rope_base,
                                             cfg.rope_style)
    return handle.value


def swa_cache_reset(handle: int, stream=None) -> None:
    _check("swa_cache_reset", LIB.swa_cache_reset(handle, _stream(stream)))


def swa_cache_destroy(handle: int | None) -> None:
    _RING_CFG.pop(handle, None)
    LIB.swa_cache_destroy(handle)


def kv_append_rope(handle: int, k_new: torch.Tensor, v_new: torch.Tensor, pos: torch.Tensor,
                   q_inout: torch.Tensor | None = None, stream=None, prepare: bool = False):
    """k_new, v_new [B, T, Hkv, d]; pos [B] int32 (position of token 0);
    q_inout [B, T, Hq, d] or None, rotated in place.  prepare=True: return the
    call marshalled once instead of making it."""
    n_tokens = k_new.shape[1]
    hq = q_inout.shape[2] if q_inout is not None else 0
    cfg = _ring_cfg(handle)
    if cfg is not None:
        rt = (_row_dtype(cfg.dtype),)
        _expect(k_new, "k_new", (cfg.batch, n_tokens, cfg.num_kv_heads, cfg.head_dim), rt)
        _expect(v_new, "v_new", (cfg.batch, n_tokens, cfg.num_kv_heads, cfg.head_dim), rt)
        _expect(pos, "pos", (cfg.batch,), (torch.int32,))
        _expect(q_inout, "q_inout", (cfg.batch, n_tokens, hq, cfg.head_dim), rt)
    args = (handle, _ptr(k_new, "k_new"), _ptr(v_new, "v_new"), _ptr(pos, "pos", torch.int32),
            n_tokens, _ptr(q_inout, "q_inout"), hq, _stream(stream))
    return _invoke("kv_append_rope", args, (k_new, v_new, pos, q_inout), prepare)


def decode_attn_workspace_bytes(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                                max_kv_tokens: int) -> int:
    n = ctypes.c_size_t()
    _check("decode_attn_workspace_bytes",
           LIB.decode_attn_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim,
                                           max_kv_tokens, ctypes.byref(n)))
    return n.value


def new_workspace(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                  max_kv_tokens: int, device="cuda") -> torch.Tensor:
    """A decode workspace for these sizes (no initialisation needed)."""
    n = decode_attn_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, max_kv_tokens)
    return torch.empty(n, dtype=torch.uint8, device=device)


def _check_ring_decode(handle: int, q: torch.Tensor, out: torch.Tensor,
                       lse: torch.Tensor | None, k_new=None, v_new=None, pos=None) -> None:
    cfg = _ring_cfg(handle)
    if cfg is None:
        return
    hq = q.shape[1] if q.dim() == 3 else -1
    rt = (_row_dtype(cfg.dtype),)
    _expect(q, "q", (cfg.batch, hq, cfg.head_dim), rt)
    _expect(out, "out", (cfg.batch, hq, cfg.head_dim), _OUT_DTYPES)
    _expect(lse, "lse", (cfg.batch, hq), (torch.float32,))
    _expect(k_new, "k_new", (cfg.batch, cfg.num_kv_heads, cfg.head_dim), rt)
    _expect(v_new, "v_new", (cfg.batch, cfg.num_kv_heads, cfg.head_dim), rt)
    _expect(pos, "pos", (cfg.batch,), (torch.int32,))


def decode_attn_ring(handle: int, q: torch.Tensor, out: torch.Tensor,
                     workspace: torch.Tensor, lse: torch.Tensor | None = None,
                     scale: float = 0.0, stream=None, prepare: bool = False):
    """q [B, Hq, d] (rotated); out [B, Hq, d] float32 or bf16; lse [B, Hq] float32 or None.
    prepare=True: return the call marshalled once instead of making it."""
    _check_ring_decode(handle, q, out, lse)
    args = (handle, _ptr(q, "q"), q.shape[1], scale, _ptr(out, "out"), _DTYPE_CODE[out.dtype],
            _ptr(lse, "lse", torch.float32), _ptr(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _stream(stream))
    return _invoke("decode_attn_ring", args, (q, out, lse, workspace), prepare)


def _step_args(handle, k_new, v_new, pos, q, out, workspace, lse, scale, stream) -> tuple:
    _check_ring_decode(handle, q, out, lse, k_new, v_new, pos)
    return (handle, _ptr(k_new, "k_new"), _ptr(v_new, "v_new"), _ptr(pos, "pos", torch.int32),
            _ptr(q, "q"), q.shape[1], scale, _ptr(out, "out"), _DTYPE_CODE[out.dtype],
            _ptr(lse, "lse", torch.float32), _ptr(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _stream(stream))


def decode_step_ring(handle: int, k_new: torch.Tensor, v_new: torch.Tensor, pos: torch.Tensor,
                     q: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor,
                     lse: torch.Tensor | None = None, scale: float = 0.0, stream=None,
                     prepare: bool = False):
    """Append of one token per sequence + decode in one call.  k_new, v_new
    [B, Hkv, d]; pos [B] int32; q [B, Hq, d] NOT rotated (left unchanged);
    out [B, Hq, d] float32 or bf16; lse [B, Hq] float32 or None.
    prepare=True: return the call marshalled once instead of making it."""
    args = _step_args(handle, k_new, v_new, pos, q, out, workspace, lse, scale, stream)
    return _invoke("decode_step_ring", args, (k_new, v_new, pos, q, out, workspace, lse), prepare)


def pos_advance(pos: torch.Tensor, delta: int = 1, stream=None) -> None:
    """pos += delta on the stream (int32 device tensor): lets a captured HIP
    graph of decode steps replay at advancing positions."""
    _check("swa_pos_advance",
           LIB.swa_pos_advance(_ptr(pos, "pos", torch.int32), pos.numel(), delta,
                               _stream(stream)))


STREAM_READ_SINK_BYTES = 32768


def stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Reads all of src (device, contiguous, a multiple of 16 bytes) once:
    the measuring aid for the achievable HBM read rate."""
    _expect_bytes(sink, "sink", STREAM_READ_SINK_BYTES)
    _check("swa_stream_read",
           LIB.swa_stream_read(_ptr(src, "src"), src.numel() * src.element_size(),
                               _ptr(sink, "sink"), sink.numel() * sink.element_size(),
                               _stream(stream)))


def decode_step_ring_shifted(handle: int, k_new: torch.Tensor, v_new: torch.Tensor,
                             pos: torch.Tensor, q: torch.Tensor, out: torch.Tensor,
                             workspace: torch.Tensor, lse: torch.Tensor | None = None,
                             scale: float = 0.0, stream=None, prepare: bool = False):
    """decode_step_ring with positions taken inside the cache (sinks scored
    against the query rotated at its cache position)."""
    args = _step_args(handle, k_new, v_new, pos, q, out, workspace, lse, scale, stream)
    return _invoke("decode_step_ring_shifted", args, (k_new, v_new, pos, q, out, workspace, lse),
                   prepare)


def prefill_attn_workspace_bytes(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                                 n_tokens: int) -> int:
    n = ctypes.c_size_t()
    _check("prefill_attn_workspace_bytes",
           LIB.prefill_attn_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, n_tokens,
                                            ctypes.byref(n)))
    return n.value


def new_prefill_workspace(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                          n_tokens: int, device="cuda") -> torch.Tensor:
    n = prefill_attn_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, n_tokens)
    return torch.empty(n, dtype=torch.uint8, device=device)


def prefill_attn_ring(handle: int, k_new: torch.Tensor, v_new: torch.Tensor, pos: torch.Tensor,
                      q: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor,
                      lse: torch.Tensor | None = None, scale: float = 0.0, stream=None,
                      prepare: bool = False):
    """Chunked prefill: k_new, v_new [B, T, Hkv, d]; pos [B] int32 (position of
    token 0); q [B, T, Hq, d] NOT rotated (left unchanged); out [B, T, Hq, d]
    float32 or bf16; lse [B, T, Hq] float32 or None."""
    cfg = _ring_cfg(handle)
    if cfg is not None:
        T = k_new.shape[1] if k_new.dim() == 4 else -1
        hq = q.shape[2] if q.dim() == 4 else -1
        rt = (_row_dtype(cfg.dtype),)
        _expect(k_new, "k_new", (cfg.batch, T, cfg.num_kv_heads, cfg.head_dim), rt)
        _expect(v_new, "v_new", (cfg.batch, T, cfg.num_kv_heads, cfg.head_dim), rt)
        _expect(pos, "pos", (cfg.batch,), (torch.int32,))
        _expect(q, "q", (cfg.batch, T, hq, cfg.head_dim), rt)
        _expect(out, "out", (cfg.batch, T, hq, cfg.head_dim), _OUT_DTYPES)
        _expect(lse, "lse", (cfg.batch, T, hq), (torch.float32,))
    args = (handle, _ptr(k_new, "k_new"), _ptr(v_new, "v_new"), _ptr(pos, "pos", torch.int32),
            k_new.shape[1], _ptr(q, "q"), q.shape[2], scale, _ptr(out, "out"),
            _DTYPE_CODE[out.dtype], _ptr(lse, "lse", torch.float32),
            _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
            _stream(stream))
    return _invoke("prefill_attn_ring", args, (k_new, v_new, pos, q, out, workspace, lse),
                   prepare)


# ---------------------------------------------------------------------------
# paged pool
# ---------------------------------------------------------------------------

def make_paged_desc(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                    block_size: int, max_blocks_per_seq: int, num_phys_blocks: int,
                    dtype: str = "bf16") -> SwaPagedDesc:
    return SwaPagedDesc(batch, num_q_heads, num_kv_heads, head_dim, block_size,
                        max_blocks_per_seq, num_phys_blocks, _DTYPE_NAME[dtype])


def swa_pool_required_bytes(desc: SwaPagedDesc) -> int:
    n = ctypes.c_size_t()
    _check("swa_pool_required_bytes", LIB.swa_pool_required_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def new_pool(desc: SwaPagedDesc, device="cuda") -> tuple:
    """(k_pool, v_pool) device buffers for `desc`: [Nphys, Hkv, bs, d] tensors
    of the element type, or flat byte buffers for int8 pools."""
    if desc.dtype == SWA_I8:
        n = swa_pool_required_bytes(desc)
        return (torch.empty(n, dtype=torch.uint8, device=device),
                torch.empty(n, dtype=torch.uint8, device=device))
    shape = (desc.num_phys_blocks, desc.num_kv_heads, desc.block_size, desc.head_dim)
    dt = _BUFFER_DTYPE[desc.dtype]
    return torch.empty(shape, dtype=dt, device=device), torch.empty(shape, dtype=dt, device=device)


def _check_paged_decode(desc: SwaPagedDesc, q, k_pool, v_pool, block_table, seq_lens,
                        block_valid, out, lse) -> None:
    B_, hq, d = desc.batch, desc.num_q_heads, desc.head_dim
    _expect(q, "q", (B_, hq, d), (_row_dtype(desc.dtype),))
    _expect(out, "out", (B_, hq, d), _OUT_DTYPES)
    _expect(lse, "lse", (B_, hq), (torch.float32,))
    pool_bytes = swa_pool_required_bytes(desc)
    _expect_bytes(k_pool, "k_pool", pool_bytes)
    _expect_bytes(v_pool, "v_pool", pool_bytes)
    _expect_numel(block_table, "block_table", B_ * desc.max_blocks_per_seq, torch.int32)
    _expect_numel(seq_lens, "seq_lens", B_, torch.int32)
    _expect_numel(block_valid, "block_valid", B_ * desc.max_blocks_per_seq, torch.uint8)


def decode_attn_paged(desc: SwaPagedDesc, q: torch.Tensor, k_pool: torch.Tensor,
                      v_pool: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                      block_valid: torch.Tensor | None, out: torch.Tensor,
                      workspace: torch.Tensor, lse: torch.Tensor | None = None,
                      scale: float = 0.0, stream=None, prepare: bool = False):
    """prepare=True: return the call marshalled once instead of making it."""
    _check_paged_decode(desc, q, k_pool, v_pool, block_table, seq_lens, block_valid, out, lse)
    args = (ctypes.byref(desc), _ptr(q, "q"), _ptr(k_pool, "k_pool"), _ptr(v_pool, "v_pool"),
            _ptr(block_table, "block_table", torch.int32), _ptr(seq_lens, "seq_lens", torch.int32),
            _ptr(block_valid, "block_valid", torch.uint8), scale, _ptr(out, "out"),
            _DTYPE_CODE[out.dtype], _ptr(lse, "lse", torch.float32), _ptr(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _stream(stream))
    keep = (desc, q, k_pool, v_pool, block_table, seq_lens, block_valid, out, workspace, lse)
    return _invoke("decode_attn_paged", args, keep, prepare)


NOALLOC_SCRATCH_BYTES = 32 << 20  # SWA_NOALLOC_SCRATCH_BYTES of include/swa.h


def decode_attn_paged_noalloc(desc: SwaPagedDesc, q: torch.Tensor, k_pool: torch.Tensor,
                              v_pool: torch.Tensor, block_table: torch.Tensor,
                              seq_lens: torch.Tensor, block_valid: torch.Tensor | None,
                              out: torch.Tensor, lse: torch.Tensor | None = None,
                              scale: float = 0.0, stream=None, prepare: bool = False):
    """decode_attn_paged without a workspace: the partial results go to the
    library's fixed per-device array (calls on one device must not overlap)."""
    _check_paged_decode(desc, q, k_pool, v_pool, block_table, seq_lens, block_valid, out, lse)
    args = (ctypes.byref(desc), _ptr(q, "q"), _ptr(k_pool, "k_pool"), _ptr(v_pool, "v_pool"),
            _ptr(block_table, "block_table", torch.int32), _ptr(seq_lens, "seq_lens", torch.int32),
            _ptr(block_valid, "block_valid", torch.uint8), scale, _ptr(out, "out"),
            _DTYPE_CODE[out.dtype], _ptr(lse, "lse", torch.float32), _stream(stream))
    keep = (desc, q, k_pool, v_pool, block_table, seq_lens, block_valid, out, lse)
    return _invoke("decode_attn_paged_noalloc", args, keep, prepare)


def prepare_decode_attn_paged(desc: SwaPagedDesc, q: torch.Tensor, k_pool: torch.Tensor,
                              v_pool: torch.Tensor, block_table: torch.Tensor,
                              seq_lens: torch.Tensor, block_valid: torch.Tensor | None,
                              out: torch.Tensor, workspace: torch.Tensor,
                              lse: torch.Tensor | None = None, scale: float = 0.0, stream=None):
    """decode_attn_paged's arguments marshalled once (stream included);
    returns a function of no arguments that makes the call."""
    return decode_attn_paged(desc, q, k_pool, v_pool, block_table, seq_lens, block_valid, out,
                             workspace, lse, scale, stream, prepare=True)


def kv_write_paged(desc: SwaPagedDesc, k_pool: torch.Tensor, v_pool: torch.Tensor,
                   k_src: torch.Tensor, v_src: torch.Tensor, dst_rows: torch.Tensor,
                   pos: torch.Tensor | None = None, rope_base: float = 10000.0,
                   rope_style: str = "interleaved", stream=None) -> None:
    """k_src, v_src [N, Hkv, d]; dst_rows [N] int32 physical token rows; pos [N] int32 or None."""
    n = k_src.shape[0]
    rt = (_row_dtype(desc.dtype),)
    _expect(k_src, "k_src", (n, desc.num_kv_heads, desc.head_dim), rt)
    _expect(v_src, "v_src", (n, desc.num_kv_heads, desc.head_dim), rt)
    _expect(dst_rows, "dst_rows", (n,), (torch.int32,))
    _expect(pos, "pos", (n,), (torch.int32,))
    pool_bytes = swa_pool_required_bytes(desc)
    _expect_bytes(k_pool, "k_pool", pool_bytes)
    _expect_bytes(v_pool, "v_pool", pool_bytes)
    _check("kv_write_paged",
           LIB.kv_write_paged(ctypes.byref(desc), _ptr(k_pool, "k_pool"), _ptr(v_pool, "v_pool"),
                              _ptr(k_src, "k_src"), _ptr(v_src, "v_src"),
                              _ptr(dst_rows, "dst_rows", torch.int32), _ptr(pos, "pos", torch.int32),
                              k_src.shape[0], rope_base, _STYLE_CODE[rope_style], _stream(stream)))


# ---------------------------------------------------------------------------
# block manager (refcounted blocks, prefix sharing, copy-on-write)
# ---------------------------------------------------------------------------

def swa_blocks_create(num_blocks: int, block_size: int, max_seqs: int,
                      max_blocks_per_seq: int) -> int:
    handle = _vp()
    _check("swa_blocks_create", LIB.swa_blocks_create(num_blocks, block_size, max_seqs,
                                                      max_blocks_per_seq, ctypes.byref(handle)))
    return handle.value


def swa_blocks_destroy(handle: int | None) -> None:
    LIB.swa_blocks_destroy(handle)


def swa_blocks_reset(handle: int) -> None:
    _check("swa_blocks_reset", LIB.swa_blocks_reset(handle))


def swa_blocks_sync(handle: int, block_table: torch.Tensor, seq_lens: torch.Tensor,
                    stream=None) -> None:
    _check("swa_blocks_sync",
           LIB.swa_blocks_sync(handle, _ptr(block_table, "block_table", torch.int32),
                               _ptr(seq_lens, "seq_lens", torch.int32), _stream(stream)))


def swa_blocks_share_prefix(handle: int, src: int, dst: int, prefix_len: int,
                            block_table: torch.Tensor, seq_lens: torch.Tensor,
                            stream=None) -> None:
    _check("swa_blocks_share_prefix",
           LIB.swa_blocks_share_prefix(handle, src, dst, prefix_len,
                                       _ptr(block_table, "block_table", torch.int32),
                                       _ptr(seq_lens, "seq_lens", torch.int32), _stream(stream)))


def swa_blocks_free(handle: int, seq: int, seq_lens: torch.Tensor, stream=None) -> None:
    _check("swa_blocks_free",
           LIB.swa_blocks_free(handle, seq, _ptr(seq_lens, "seq_lens", torch.int32),
                               _stream(stream)))


def swa_blocks_state(handle: int, max_seqs: int, max_blocks: int, num_blocks: int) -> dict:
    table = (_i32 * (max_seqs * max_blocks))()
    lens = (_i32 * max_seqs)()
    refs = (_i32 * num_blocks)()
    free = _i32()
    _check("swa_blocks_state",
           LIB.swa_blocks_state(handle, ctypes.cast(table, _vp), ctypes.cast(lens, _vp),
                                ctypes.cast(refs, _vp), ctypes.byref(free)))
    t = list(table)
    return {"table": [t[i * max_blocks:(i + 1) * max_blocks] for i in range(max_seqs)],
            "lens": list(lens), "refs": list(refs), "free": free.value}


def kv_append_paged(handle: int, desc: SwaPagedDesc, k_pool: torch.Tensor, v_pool: torch.Tensor,
                    block_table: torch.Tensor, seq_lens: torch.Tensor, seqs,
                    k_new: torch.Tensor, v_new: torch.Tensor, rotate: bool = False,
                    rope_base: float = 10000.0, rope_style: str = "interleaved",
                    stream=None) -> None:
    """k_new, v_new [n_seqs, n_tokens, Hkv, d]; seqs: the n_seqs sequences
    (a list, or a C int32 array made once for a loop)."""
    if isinstance(seqs, ctypes.Array):
        arr, n = seqs, len(seqs)
    else:
        n = len(seqs)
        arr = (_i32 * max(1, n))(*[int(x) for x in seqs])
    T = k_new.shape[1] if k_new.dim() == 4 else -1
    rt = (_row_dtype(desc.dtype),)
    _expect(k_new, "k_new", (n, T, desc.num_kv_heads, desc.head_dim), rt)
    _expect(v_new, "v_new", (n, T, desc.num_kv_heads, desc.head_dim), rt)
    if desc.dtype != SWA_I8:  # (int8 pools are refused by the library itself)
        pool_bytes = swa_pool_required_bytes(desc)
        _expect_bytes(k_pool, "k_pool", pool_bytes)
        _expect_bytes(v_pool, "v_pool", pool_bytes)
    _expect_numel(block_table, "block_table", desc.batch * desc.max_blocks_per_seq, torch.int32)
    _expect_numel(seq_lens, "seq_lens", desc.batch, torch.int32)
    _check("kv_append_paged",
           LIB.kv_append_paged(handle, ctypes.byref(desc), _ptr(k_pool, "k_pool"),
                               _ptr(v_pool, "v_pool"),
                               _ptr(block_table, "block_table", torch.int32),
                               _ptr(seq_lens, "seq_lens", torch.int32), ctypes.cast(arr, _vp), n,
                               k_new.shape[1], _ptr(k_new, "k_new"), _ptr(v_new, "v_new"),
                               1 if rotate else 0, rope_base, _STYLE_CODE[rope_style],
                               _stream(stream)))


# ---------------------------------------------------------------------------
# host-pool pager
# ---------------------------------------------------------------------------

def make_pager_config(batch: int, num_kv_heads: int, head_dim: int, block_size: int,
                      logical_blocks: int, slots_per_seq: int, num_phys_blocks: int,
                      dtype: str = "bf16") -> SwaPagerConfig:
    return SwaPagerConfig(batch, num_kv_heads, head_dim, block_size, logical_blocks,
                          slots_per_seq, num_phys_blocks, _DTYPE_NAME[dtype])


def _host_ptr(t: torch.Tensor, name: str) -> int:
    if t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous host tensor")
    return t.data_ptr()


def swa_pager_create(cfg: SwaPagerConfig, host_k: torch.Tensor, host_v: torch.Tensor,
                     k_pool: torch.Tensor, v_pool: torch.Tensor, slot_phys,
                     block_table: torch.Tensor, block_valid: torch.Tensor) -> int:
    """host_k, host_v: pinned host [B, L, Hkv, bs, d]; k_pool, v_pool: device
    [Nphys, Hkv, bs, d]; slot_phys: [B, C] int32 host array (copied);
    block_table [B, C] int32 and block_valid [B, C] uint8 on the device."""
    flat = [int(x) for row in slot_phys for x in row]
    B_, C = cfg.batch, cfg.slots_per_seq
    if len(flat) != B_ * C:
        raise ValueError(f"slot_phys must hold {B_} x {C} entries, got {len(flat)}")
    blk = cfg.num_kv_heads * cfg.block_size * cfg.head_dim * (4 if cfg.dtype == SWA_F32 else 2)
    _expect_bytes(host_k, "host_k", B_ * cfg.logical_blocks * blk)
    _expect_bytes(host_v, "host_v", B_ * cfg.logical_blocks * blk)
    _expect_bytes(k_pool, "k_pool", cfg.num_phys_blocks * blk)
    _expect_bytes(v_pool, "v_pool", cfg.num_phys_blocks * blk)
    _expect_numel(block_table, "block_table", B_ * C, torch.int32)
    _expect_numel(block_valid, "block_valid", B_ * C, torch.uint8)
    sp = (_i32 * len(flat))(*flat)
    handle = _vp()
    _check("swa_pager_create",
           LIB.swa_pager_create(ctypes.byref(cfg), _host_ptr(host_k, "host_k"),
                                _host_ptr(host_v, "host_v"), _ptr(k_pool, "k_pool"),
                                _ptr(v_pool, "v_pool"), ctypes.cast(sp, _vp),
                                _ptr(block_table, "block_table", torch.int32),
                                _ptr(block_valid, "block_valid", torch.uint8),
                                ctypes.byref(handle)))
    return handle.value


def swa_pager_reset(handle: int, stream=None) -> None:
    _check("swa_pager_reset", LIB.swa_pager_reset(handle, _stream(stream)))


def pack_requests(requests) -> tuple:
    """(offsets, blocks) C arrays of one request per sequence, for
    swa_pager_advance (packing ahead of time keeps it off a timed loop)."""
    flat = [int(b) for r in requests for b in r]
    offsets = [0]
    for r in requests:
        offsets.append(offsets[-1] + len(r))
    return (_i32 * len(offsets))(*offsets), (_i32 * max(1, len(flat)))(*flat)


def swa_pager_advance(handle: int, requests, stream=None, copy_stream=None) -> int:
    """requests: one list of logical blocks per sequence, or what
    pack_requests returned.  Returns the number of blocks whose copies this
    call starts."""
    off, blocks = requests if isinstance(requests, tuple) else pack_requests(requests)
    n = _i32()
    cs = _stream(copy_stream) if copy_stream is not None else _stream(stream)
    _check("swa_pager_advance",
           LIB.swa_pager_advance(handle, ctypes.cast(off, _vp), ctypes.cast(blocks, _vp),
                                 _stream(stream), cs, ctypes.byref(n)))
    return n.value


def swa_pager_commit(handle: int, stream=None) -> None:
    _check("swa_pager_commit", LIB.swa_pager_commit(handle, _stream(stream)))


def swa_pager_stage(handle: int, requests) -> int:
    """The LRU decisions of swa_pager_advance for the next step's requests,
    with the copies left to the next swa_pager_decode.  Returns the number
    of blocks staged."""
    off, blocks = requests if isinstance(requests, tuple) else pack_requests(requests)
    n = _i32()
    _check("swa_pager_stage", LIB.swa_pager_stage(handle, ctypes.cast(off, _vp),
                                                  ctypes.cast(blocks, _vp), ctypes.byref(n)))
    return n.value


def swa_pager_decode(handle: int, desc: SwaPagedDesc, q: torch.Tensor, k_pool: torch.Tensor,
                     v_pool: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                     block_valid: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor,
                     lse: torch.Tensor | None = None, scale: float = 0.0, stream=None,
                     prepare: bool = False):
    """decode_attn_paged over the pager's pool, then the staged copies in the
    same launches.  desc and the pool tensors are the ones the pager was made
    with (their extents are checked here; the library uses its own pointers).
    prepare=True: return the call marshalled once instead of making it."""
    _check_paged_decode(desc, q, k_pool, v_pool, block_table, seq_lens, block_valid, out, lse)
    args = (handle, _ptr(q, "q"), desc.num_q_heads, _ptr(seq_lens, "seq_lens", torch.int32),
            scale, _ptr(out, "out"), _DTYPE_CODE[out.dtype], _ptr(lse, "lse", torch.float32),
            _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
            _stream(stream))
    keep = (desc, q, k_pool, v_pool, block_table, seq_lens, block_valid, out, workspace, lse)
    return _invoke("swa_pager_decode", args, keep, prepare)


def swa_pager_workspace_bytes(handle: int, num_q_heads: int) -> int:
    n = ctypes.c_size_t()
    _check("swa_pager_workspace_bytes",
           LIB.swa_pager_workspace_bytes(handle, num_q_heads, ctypes.byref(n)))
    return n.value


def swa_pager_slot_blocks(handle: int, seq: int, slots_per_seq: int) -> list:
    out = (_i32 * slots_per_seq)()
    _check("swa_pager_slot_blocks", LIB.swa_pager_slot_blocks(handle, seq, ctypes.cast(out, _vp)))
    return list(out)


def swa_pager_destroy(handle: int | None) -> None:
    LIB.swa_pager_destroy(handle)


# ---------------------------------------------------------------------------
# convenience owner of a ring cache's device buffers
# ---------------------------------------------------------------------------

@dataclass
class RingCache:
    """Device buffers of one ring cache (allocated with torch) plus its handle."""
    cfg: SwaCacheConfig
    k: torch.Tensor
    v: torch.Tensor
    slot_pos: torch.Tensor
    handle: int

    @classmethod
    def allocate(cls, batch: int, num_kv_heads: int, head_dim: int, window: int, num_sinks: int,
                 dtype: str = "bf16", rope_base: float = 10000.0,
                 rope_style: str = "interleaved", device="cuda", stream=None) -> "RingCache":
        cfg = make_config(batch, num_kv_heads, head_dim, window, num_sinks, dtype, rope_base,
                          rope_style)
        slots = num_sinks + window
        if cfg.dtype == SWA_I8:  # raw bytes: codes, then one float32 scale per row
            kv_bytes, _ = swa_cache_required_bytes(cfg)
            k = torch.empty(kv_bytes, dtype=torch.uint8, device=device)
        else:
            k = torch.empty((batch, num_kv_heads, slots, head_dim), dtype=_BUFFER_DTYPE[cfg.dtype],
                            device=device)
        v = torch.empty_like(k)
        slot_pos = torch.empty((batch, slots), dtype=torch.int32, device=device)
        handle = swa_cache_create(cfg, k, v, slot_pos)
        swa_cache_reset(handle, stream)
        return cls(cfg, k, v, slot_pos, handle)

    @property
    def slots(self) -> int:
        return self.cfg.num_sinks + self.cfg.window

    def workspace(self, num_q_heads: int) -> torch.Tensor:
        return new_workspace(self.cfg.batch, num_q_heads, self.cfg.num_kv_heads,
                             self.cfg.head_dim, self.slots, self.k.device)

    def close(self) -> None:
        if self.handle:
            swa_cache_destroy(self.handle)
            self.handle = 0

    def __del__(self):  # pragma: no cover - best effort
        try:
            self.close()
        except Exception:
            pass

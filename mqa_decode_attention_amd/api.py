"""Python binding of libkvc: argument marshalling only.

Each function checks the torch tensors it is given (device, dtype, layout,
shape), passes their device pointers and the current HIP stream to the C ABI,
and raises KvcError on a non-OK status.  All computation happens in the HIP
kernels; nothing here touches tensor values.
"""
from __future__ import annotations

import functools

from typing import Dict, Optional, Tuple

import torch

from . import _lib

KVC_F32, KVC_BF16, KVC_U8, KVC_FP8_E4M3, KVC_FP8_E5M2 = 0, 1, 2, 3, 4
# FP8 cache formats of the *_fp8 calls
FP8_FORMATS = {"e4m3": KVC_FP8_E4M3, "e5m2": KVC_FP8_E5M2}
ROPE_STYLES = {"interleaved": 0, "half": 1}


class KvcError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"kvc status {status}: {message}")
        self.status = status


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KVC_BF16
    if t.dtype == torch.float32:
        return KVC_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None) -> int:
    # (is_cuda and a direct Size comparison: half the host time of building
    # device objects and tuples, which matters for the smallest steps)
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and t.shape != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _stream(device: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _check(status: int) -> None:
    if status != 0:
        lib = _lib.load()
        raise KvcError(status, lib.kvc_last_error().decode() or lib.kvc_status_string(status).decode())


def append(k_cache: torch.Tensor, v_cache: torch.Tensor, positions: torch.Tensor,
           k_new: torch.Tensor, v_new: torch.Tensor, rope_cos: torch.Tensor,
           rope_sin: torch.Tensor, q: Optional[torch.Tensor] = None,
           block_table: Optional[torch.Tensor] = None, rope_style: str = "interleaved",
           stream=None) -> None:
    """kvc_append: rotate and store the new token's key, store its value, rotate q in place.

    Contiguous caches are [B, H_kv, T_max, d]; with a block_table [B, max_blocks]
    (int32) they are pools [num_blocks, H_kv, block_size, d].
    """
    lib = _lib.load()
    dt = _dtype_code(k_new)
    B, H_kv, d = k_new.shape
    H_q = q.shape[1] if q is not None else H_kv
    if rope_cos.dim() != 2 or rope_cos.shape[1] != d // 2:
        raise ValueError(f"rope_cos must be [rows, {d // 2}], got {tuple(rope_cos.shape)}")
    if block_table is not None:
        num_blocks, _, block_size, _ = k_cache.shape
        T_max = 0
        mb = block_table.shape[1]
        tbl = _dev(block_table, "block_table", torch.int32, (B, mb))
        shape = (num_blocks, H_kv, block_size, d)
    else:
        T_max = k_cache.shape[2]
        tbl, block_size, mb, num_blocks = None, 0, 0, 0
        shape = (B, H_kv, T_max, d)
    _check(lib.kvc_append(
        dt, B, H_q, H_kv, d,
        _dev(k_cache, "k_cache", k_new.dtype, shape), _dev(v_cache, "v_cache", k_new.dtype, shape), T_max,
        tbl, block_size, mb, num_blocks,
        _dev(positions, "positions", torch.int32, (B,)),
        _dev(k_new, "k_new", k_new.dtype), _dev(v_new, "v_new", k_new.dtype, (B, H_kv, d)),
        _dev(q, "q", k_new.dtype, (B, H_q, d)) if q is not None else None,
        _dev(rope_cos, "rope_cos", torch.float32), _dev(rope_sin, "rope_sin", torch.float32, rope_cos.shape),
        rope_cos.shape[0], ROPE_STYLES[rope_style], _stream(k_new.device, stream)))


def _cache_code(dtype) -> int:
    """dtype of the cache: torch.bfloat16, torch.float32, torch.uint8 (uint8
    codes), or torch.float8_e4m3fn / torch.float8_e5m2 (FP8 codes)."""
    if dtype == torch.uint8:
        return KVC_U8
    if dtype == torch.float8_e4m3fn:
        return KVC_FP8_E4M3
    if dtype == torch.float8_e5m2:
        return KVC_FP8_E5M2
    return KVC_BF16 if dtype == torch.bfloat16 else KVC_F32


def _q8_fn(lib, name: str, fmt: Optional[str]):
    """The uint8 call kvc_<name>_u8, or (fmt "e4m3" / "e5m2") kvc_<name>_fp8
    with its format argument bound."""
    if fmt is None:
        return getattr(lib, f"kvc_{name}_u8")
    if fmt not in FP8_FORMATS:
        raise ValueError(f"FP8 format must be one of {sorted(FP8_FORMATS)}, got {fmt!r}")
    return functools.partial(getattr(lib, f"kvc_{name}_fp8"), FP8_FORMATS[fmt])


def _q8_dtype(fmt: Optional[str]):
    return torch.uint8 if fmt is None else {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}[fmt]


def workspace_bytes(dtype: torch.dtype, B: int, H_q: int, H_kv: int, d: int, max_seq_len: int,
                    split_tokens: int = 0, pool_tokens: int = 0) -> int:
    """kvc_decode_workspace_bytes; pool_tokens = num_blocks * block_size for a paged
    cache; dtype torch.uint8 for the quantized cache."""
    lib = _lib.load()
    code = _cache_code(dtype)
    n = lib.kvc_decode_workspace_bytes(code, B, H_q, H_kv, d, max_seq_len, pool_tokens, split_tokens)
    if n == (1 << 64) - 1:
        raise KvcError(2, lib.kvc_last_error().decode() or "invalid sizes for the decode workspace")
    return n


def merge_launch(dtype: torch.dtype, B: int, H_q: int, H_kv: int, d: int, max_seq_len: int,
                 split_tokens: int = 0, pool_tokens: int = 0) -> bool:
    """kvc_decode_merge_launch: True when a decode with these sizes launches a
    separate merge kernel after the streaming kernel."""
    lib = _lib.load()
    n = lib.kvc_decode_merge_launch(_cache_code(dtype), B, H_q, H_kv, d, max_seq_len, pool_tokens, split_tokens)
    if n < 0:
        raise KvcError(2, lib.kvc_last_error().decode() or "invalid sizes")
    return bool(n)


def balanced(dtype: torch.dtype, B: int, H_q: int, H_kv: int, d: int, max_seq_len: int,
             split_tokens: int = 0, pool_tokens: int = 0) -> bool:
    """kvc_decode_balanced: True when a single-token decode with these sizes
    runs the balanced schedule (workgroups streaming equal shares of all
    sequences' steps) rather than fixed-length splits."""
    lib = _lib.load()
    n = lib.kvc_decode_balanced(_cache_code(dtype), B, H_q, H_kv, d, max_seq_len, pool_tokens, split_tokens)
    if n < 0:
        raise KvcError(2, lib.kvc_last_error().decode() or "invalid sizes")
    return bool(n)


def compact(dtype: torch.dtype, B: int, H_q: int, H_kv: int, d: int, max_seq_len: int,
            split_tokens: int = 0, pool_tokens: int = 0) -> bool:
    """kvc_decode_compact: True when a single-token decode with these sizes
    runs the compacted schedule (split length picked on the device from the
    lengths, the existing splits numbered first, merged in the same launch)."""
    lib = _lib.load()
    n = lib.kvc_decode_compact(_cache_code(dtype), B, H_q, H_kv, d, max_seq_len, pool_tokens, split_tokens)
    if n < 0:
        raise KvcError(2, lib.kvc_last_error().decode() or "invalid sizes")
    return bool(n)


def workspace_zeroed_bytes() -> int:
    """kvc_workspace_zeroed_bytes: the prefix of a caller's `workspace` tensor
    that must be zero before its first use (every completed call leaves it so)."""
    return _lib.load().kvc_workspace_zeroed_bytes()


def split_tokens(dtype: torch.dtype, B: int, H_q: int, H_kv: int, d: int, max_seq_len: int,
                 split_tokens: int = 0, pool_tokens: int = 0) -> int:
    """kvc_decode_split_tokens: the split length a decode call with these sizes uses."""
    lib = _lib.load()
    code = _cache_code(dtype)
    n = lib.kvc_decode_split_tokens(code, B, H_q, H_kv, d, max_seq_len, pool_tokens, split_tokens)
    if n < 0:
        raise KvcError(2, lib.kvc_last_error().decode() or "invalid sizes")
    return n


# Workspaces kept per (device, stream); calls on one stream run one at a time,
# so they can share one buffer.  Each is allocated with its stream current, so
# the caching allocator ties its memory to that stream: when a larger one
# replaces it, the old block is handed out again only in that stream's order,
# never while a kernel still queued there uses it.
_WORKSPACES: Dict[Tuple[int, int], torch.Tensor] = {}


def _workspace(device: torch.device, stream_handle: int, nbytes: int) -> Tuple[Optional[int], int]:
    if nbytes == 0:
        return None, 0
    key = (device.index if device.index is not None else torch.cuda.current_device(), stream_handle)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        # (zeroed once: its first bytes hold the split kernels' arrival
        # counters, which every completed call leaves at zero)
        with torch.cuda.stream(torch.cuda.ExternalStream(stream_handle, device=device)):
            ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _WORKSPACES[key] = ws
    return ws.data_ptr(), ws.numel()


def profile_next_decode(start: Optional["torch.cuda.Event"], stop: Optional["torch.cuda.Event"]) -> None:
    """Have the next decode call on this thread record `start`/`stop` around its
    streaming kernel (kvc_profile_next_decode; either may be None).  The events
    must exist already (record them once before the first use)."""
    _lib.load().kvc_profile_next_decode(start.cuda_event if start is not None else None,
                                        stop.cuda_event if stop is not None else None)


def _decode_args(q, out):
    dt = _dtype_code(q)
    B, H_q, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    return dt, B, H_q, d, out


def decode_attn(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                seq_lens: torch.Tensor, max_seq_len: int, out: Optional[torch.Tensor] = None,
                scale: Optional[float] = None, split_tokens: int = 0,
                workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """kvc_decode_attn over a contiguous cache [B, H_kv, T_max, d]; returns out [B, H_q, d]."""
    lib = _lib.load()
    dt, B, H_q, d, out = _decode_args(q, out)
    _, H_kv, T_max, _ = k_cache.shape
    st = _stream(q.device, stream)
    need = workspace_bytes(q.dtype, B, H_q, H_kv, d, max_seq_len, split_tokens)
    if workspace is not None:
        ws, wsn = _dev(workspace, "workspace", torch.uint8), workspace.numel()
    else:
        ws, wsn = _workspace(q.device, st, need)
    _check(lib.kvc_decode_attn(
        dt, B, H_q, H_kv, d, _dev(q, "q", q.dtype),
        _dev(k_cache, "k_cache", q.dtype, (B, H_kv, T_max, d)),
        _dev(v_cache, "v_cache", q.dtype, (B, H_kv, T_max, d)), T_max,
        _dev(seq_lens, "seq_lens", torch.int32, (B,)), int(max_seq_len),
        float(scale) if scale else 0.0, _dev(out, "out", q.dtype, (B, H_q, d)),
        int(split_tokens), ws, wsn, st))
    return out


def decode_attn_paged(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                      block_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                      out: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                      split_tokens: int = 0, workspace: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """kvc_decode_attn_paged over pools [num_blocks, H_kv, block_size, d]."""
    lib = _lib.load()
    dt, B, H_q, d, out = _decode_args(q, out)
    num_blocks, H_kv, block_size, _ = k_pool.shape
    st = _stream(q.device, stream)
    need = workspace_bytes(q.dtype, B, H_q, H_kv, d, max_seq_len, split_tokens,
                           pool_tokens=num_blocks * block_size)
    if workspace is not None:
        ws, wsn = _dev(workspace, "workspace", torch.uint8), workspace.numel()
    else:
        ws, wsn = _workspace(q.device, st, need)
    _check(lib.kvc_decode_attn_paged(
        dt, B, H_q, H_kv, d, _dev(q, "q", q.dtype),
        _dev(k_pool, "k_pool", q.dtype, (num_blocks, H_kv, block_size, d)),
        _dev(v_pool, "v_pool", q.dtype, (num_blocks, H_kv, block_size, d)),
        num_blocks, block_size, _dev(block_table, "block_table", torch.int32, (B, block_table.shape[1])),
        block_table.shape[1], _dev(seq_lens, "seq_lens", torch.int32, (B,)), int(max_seq_len),
        float(scale) if scale else 0.0, _dev(out, "out", q.dtype, (B, H_q, d)),
        int(split_tokens), ws, wsn, st))
    return out


def decode_step(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                positions: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                rope_cos: torch.Tensor, rope_sin: torch.Tensor, max_seq_len: int,
                block_table: Optional[torch.Tensor] = None, rope_style: str = "interleaved",
                q_rot_out: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                scale: Optional[float] = None, split_tokens: int = 0,
                workspace: Optional[torch.Tensor] = None, stream=None):
    """kvc_decode_step: append the new token and attend, in one call.

    q is the raw query (left unchanged); returns (out, q_rot_out).
    """
    fn, args, out, q_rot_out = _step_call(q, k_cache, v_cache, positions, k_new, v_new, rope_cos, rope_sin,
                                          max_seq_len, block_table, rope_style, q_rot_out, out, scale, split_tokens,
                                          workspace, stream)
    _check(fn(*args))
    return out, q_rot_out


class PreparedCall:
    """A library call whose arguments were checked and converted once: each
    call of this object makes that one foreign call again, on the same
    buffers and stream, with no other host work (the form a serving loop that
    reuses its buffers every step wants).  Returns what the call returns."""

    __slots__ = ("_fn", "_args", "_result", "_keep")

    def __init__(self, fn, args, result, keep=()):
        self._fn = fn
        # (values already of the declared ctypes types pass through the
        # foreign call without conversion)
        self._args = tuple(a if a is None else t(a) for t, a in zip(fn.argtypes, args))
        self._result = result
        self._keep = keep          # the tensors whose addresses the arguments hold

    def __call__(self):
        status = self._fn(*self._args)
        if status:
            _check(status)
        return self._result


def prepare_decode_step(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                        positions: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                        rope_cos: torch.Tensor, rope_sin: torch.Tensor, max_seq_len: int,
                        block_table: Optional[torch.Tensor] = None, rope_style: str = "interleaved",
                        q_rot_out: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                        scale: Optional[float] = None, split_tokens: int = 0,
                        workspace: Optional[torch.Tensor] = None, stream=None) -> PreparedCall:
    """decode_step's checks and argument conversion done once, the launch left
    for later: returns a PreparedCall that runs kvc_decode_step on these
    buffers (their contents at that time) and returns (out, q_rot_out).  The
    tensors must stay alive and in place while it is used."""
    fn, args, out, q_rot_out = _step_call(q, k_cache, v_cache, positions, k_new, v_new, rope_cos, rope_sin,
                                          max_seq_len, block_table, rope_style, q_rot_out, out, scale, split_tokens,
                                          workspace, stream)
    if workspace is None:       # the library's own workspace for this stream, held for the call object's life
        workspace = _WORKSPACES.get((q.device.index if q.device.index is not None else torch.cuda.current_device(),
                                     args[-1]))
    return PreparedCall(fn, args, (out, q_rot_out),
                        (q, k_cache, v_cache, positions, k_new, v_new, rope_cos, rope_sin, block_table, workspace))


def _step_call(q, k_cache, v_cache, positions, k_new, v_new, rope_cos, rope_sin, max_seq_len, block_table,
               rope_style, q_rot_out, out, scale, split_tokens, workspace, stream):
    lib = _lib.load()
    dt, B, H_q, d, out = _decode_args(q, out)
    H_kv = k_new.shape[1]
    if q_rot_out is None:
        q_rot_out = torch.empty_like(q)
    if rope_cos.dim() != 2 or rope_cos.shape[1] != d // 2:
        raise ValueError(f"rope_cos must be [rows, {d // 2}], got {tuple(rope_cos.shape)}")
    if block_table is not None:
        num_blocks, _, block_size, _ = k_cache.shape
        T_max, mb = 0, block_table.shape[1]
        tbl = _dev(block_table, "block_table", torch.int32, (B, mb))
        shape = (num_blocks, H_kv, block_size, d)
    else:
        T_max = k_cache.shape[2]
        tbl, block_size, mb, num_blocks = None, 0, 0, 0
        shape = (B, H_kv, T_max, d)
    st = _stream(q.device, stream)
    need = workspace_bytes(q.dtype, B, H_q, H_kv, d, max_seq_len, split_tokens,
                           pool_tokens=num_blocks * block_size if block_table is not None else 0)
    if workspace is not None:
        ws, wsn = _dev(workspace, "workspace", torch.uint8), workspace.numel()
    else:
        ws, wsn = _workspace(q.device, st, need)
    args = (dt, B, H_q, H_kv, d, _dev(q, "q", q.dtype, (B, H_q, d)),
            _dev(q_rot_out, "q_rot_out", q.dtype, (B, H_q, d)),
            _dev(k_cache, "k_cache", q.dtype, shape), _dev(v_cache, "v_cache", q.dtype, shape), T_max,
            tbl, block_size, mb, num_blocks, _dev(positions, "positions", torch.int32, (B,)),
            _dev(k_new, "k_new", q.dtype, (B, H_kv, d)), _dev(v_new, "v_new", q.dtype, (B, H_kv, d)),
            _dev(rope_cos, "rope_cos", torch.float32), _dev(rope_sin, "rope_sin", torch.float32, rope_cos.shape),
            rope_cos.shape[0], ROPE_STYLES[rope_style], int(max_seq_len), float(scale) if scale else 0.0,
            _dev(out, "out", q.dtype, (B, H_q, d)), int(split_tokens), ws, wsn, st)
    return lib.kvc_decode_step, args, out, q_rot_out


def decode_step_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                        positions: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                        rope_cos: torch.Tensor, rope_sin: torch.Tensor, max_seq_len: int,
                        q_rot_out: torch.Tensor, out: torch.Tensor,
                        block_table: Optional[torch.Tensor] = None, rope_style: str = "interleaved",
                        scale: Optional[float] = None, split_tokens: int = 0, stream=None) -> None:
    """kvc_decode_step_noalloc: kvc_decode_step with the split partials in the
    library's fixed device array; allocates nothing (out and q_rot_out are the
    caller's).  Calls that overlap on one device race on that array."""
    lib = _lib.load()
    if out is None or q_rot_out is None:
        raise ValueError("decode_step_noalloc allocates nothing: pass out and q_rot_out")
    dt, B, H_q, d, out = _decode_args(q, out)
    H_kv = k_new.shape[1]
    if rope_cos.dim() != 2 or rope_cos.shape[1] != d // 2:
        raise ValueError(f"rope_cos must be [rows, {d // 2}], got {tuple(rope_cos.shape)}")
    if block_table is not None:
        num_blocks, _, block_size, _ = k_cache.shape
        T_max, mb = 0, block_table.shape[1]
        tbl = _dev(block_table, "block_table", torch.int32, (B, mb))
        shape = (num_blocks, H_kv, block_size, d)
    else:
        T_max = k_cache.shape[2]
        tbl, block_size, mb, num_blocks = None, 0, 0, 0
        shape = (B, H_kv, T_max, d)
    _check(lib.kvc_decode_step_noalloc(
        dt, B, H_q, H_kv, d, _dev(q, "q", q.dtype, (B, H_q, d)),
        _dev(q_rot_out, "q_rot_out", q.dtype, (B, H_q, d)),
        _dev(k_cache, "k_cache", q.dtype, shape), _dev(v_cache, "v_cache", q.dtype, shape), T_max,
        tbl, block_size, mb, num_blocks, _dev(positions, "positions", torch.int32, (B,)),
        _dev(k_new, "k_new", q.dtype, (B, H_kv, d)), _dev(v_new, "v_new", q.dtype, (B, H_kv, d)),
        _dev(rope_cos, "rope_cos", torch.float32), _dev(rope_sin, "rope_sin", torch.float32, rope_cos.shape),
        rope_cos.shape[0], ROPE_STYLES[rope_style], int(max_seq_len), float(scale) if scale else 0.0,
        _dev(out, "out", q.dtype, (B, H_q, d)), int(split_tokens), _stream(q.device, stream)))


def noalloc_max_bytes() -> int:
    """kvc_decode_step_noalloc_max_bytes: size of the library's fixed partials array."""
    return int(_lib.load().kvc_decode_step_noalloc_max_bytes())


# ---------------------------------------------------------------------------
# sliding window: attend the last `window` tokens (full cache or a ring)
# ---------------------------------------------------------------------------


def window_span(max_seq_len: int, window: int, ring: bool = False, T_max: int = 0) -> int:
    """kvc_window_span: the max_seq_len that sizes a windowed call's splits and workspace."""
    n = _lib.load().kvc_window_span(int(max_seq_len), int(window), int(bool(ring)), int(T_max))
    if n < 0:
        raise KvcError(2, "invalid window sizes")
    return n


def append_ring(k_ring: torch.Tensor, v_ring: torch.Tensor, positions: torch.Tensor, k_new: torch.Tensor,
                v_new: torch.Tensor, rope_cos: torch.Tensor, rope_sin: torch.Tensor,
                q: Optional[torch.Tensor] = None, rope_style: str = "interleaved", stream=None) -> None:
    """kvc_append_ring: position p goes to slot p % T_max of a ring [B, H_kv, T_max, d]."""
    lib = _lib.load()
    dt = _dtype_code(k_new)
    B, H_kv, d = k_new.shape
    H_q = q.shape[1] if q is not None else H_kv
    if rope_cos.dim() != 2 or rope_cos.shape[1] != d // 2:
        raise ValueError(f"rope_cos must be [rows, {d // 2}], got {tuple(rope_cos.shape)}")
    T_max = k_ring.shape[2]
    shape = (B, H_kv, T_max, d)
    _check(lib.kvc_append_ring(
        dt, B, H_q, H_kv, d, _dev(k_ring, "k_ring", k_new.dtype, shape), _dev(v_ring, "v_ring", k_new.dtype, shape),
        T_max, _dev(positions, "positions", torch.int32, (B,)),
        _dev(k_new, "k_new", k_new.dtype), _dev(v_new, "v_new", k_new.dtype, (B, H_kv, d)),
        _dev(q, "q", k_new.dtype, (B, H_q, d)) if q is not None else None,
        _dev(rope_cos, "rope_cos", torch.float32), _dev(rope_sin, "rope_sin", torch.float32, rope_cos.shape),
        rope_cos.shape[0], ROPE_STYLES[rope_style], _stream(k_new.device, stream)))


def _cache_geometry(k_cache, block_table, B, H_kv, d):
    if block_table is not None:
        num_blocks, _, block_size, _ = k_cache.shape
        mb = block_table.shape[1]
        return (0, _dev(block_table, "block_table", torch.int32, (B, mb)), block_size, mb, num_blocks,
                (num_blocks, H_kv, block_size, d))
    T_max = k_cache.shape[2]
    return T_max, None, 0, 0, 0, (B, H_kv, T_max, d)


def decode_attn_window(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, seq_lens: torch.Tensor,
                       max_seq_len: int, window: int, ring: bool = False,
                       block_table: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                       scale: Optional[float] = None, split_tokens: int = 0,
                       workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """kvc_decode_attn_window: attention over the last `window` tokens of a full
    cache (contiguous, or pools with a block_table), or over a ring (ring=True)."""
    lib = _lib.load()
    dt, B, H_q, d, out = _decode_args(q, out)
    H_kv = k_cache.shape[1]
    T_max, tbl, block_size, mb, num_blocks, shape = _cache_geometry(k_cache, block_table, B, H_kv, d)
    st = _stream(q.device, stream)
    need = workspace_bytes(q.dtype, B, H_q, H_kv, d, window_span(max_seq_len, window, ring, T_max), split_tokens,
                           pool_tokens=num_blocks * block_size)
    if workspace is not None:
        ws, wsn = _dev(workspace, "workspace", torch.uint8), workspace.numel()
    else:
        ws, wsn = _workspace(q.device, st, need)
    _check(lib.kvc_decode_attn_window(
        dt, B, H_q, H_kv, d, _dev(q, "q", q.dtype),
        _dev(k_cache, "k_cache", q.dtype, shape), _dev(v_cache, "v_cache", q.dtype, shape), T_max,
        tbl, block_size, mb, num_blocks, _dev(seq_lens, "seq_lens", torch.int32, (B,)), int(max_seq_len),
        int(window), int(bool(ring)), float(scale) if scale else 0.0, _dev(out, "out", q.dtype, (B, H_q, d)),
        int(split_tokens), ws, wsn, st))
    return out


def decode_step_window(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, positions: torch.Tensor,
                       k_new: torch.Tensor, v_new: torch.Tensor, rope_cos: torch.Tensor, rope_sin: torch.Tensor,
                       max_seq_len: int, window: int, ring: bool = False,
                       block_table: Optional[torch.Tensor] = None, rope_style: str = "interleaved",
                       q_rot_out: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                       scale: Optional[float] = None, split_tokens: int = 0,
                       workspace: Optional[torch.Tensor] = None, stream=None):
    """kvc_decode_step_window: append the new token (ring slot when ring=True)
    and attend over its window, in one call; returns (out, q_rot_out)."""
    lib = _lib.load()
    dt, B, H_q, d, out = _decode_args(q, out)
    H_kv = k_new.shape[1]
    if q_rot_out is None:
        q_rot_out = torch.empty_like(q)
    if rope_cos.dim() != 2 or rope_cos.shape[1] != d // 2:
        raise ValueError(f"rope_cos must be [rows, {d // 2}], got {tuple(rope_cos.shape)}")
    T_max, tbl, block_size, mb, num_blocks, shape = _cache_geometry(k_cache, block_table, B, H_kv, d)
    st = _stream(q.device, stream)
    need = workspace_bytes(q.dtype, B, H_q, H_kv, d, window_span(max_seq_len, window, ring, T_max), split_tokens,
                           pool_tokens=num_blocks * block_size)
    if workspace is not None:
        ws, wsn = _dev(workspace, "workspace", torch.uint8), workspace.numel()
    else:
        ws, wsn = _workspace(q.device, st, need)
    _check(lib.kvc_decode_step_window(
        dt, B, H_q, H_kv, d, _dev(q, "q", q.dtype, (B, H_q, d)),
        _dev(q_rot_out, "q_rot_out", q.dtype, (B, H_q, d)),
        _dev(k_cache, "k_cache", q.dtype, shape), _dev(v_cache, "v_cache", q.dtype, shape), T_max,
        tbl, block_size, mb, num_blocks, _dev(positions, "positions", torch.int32, (B,)),
        _dev(k_new, "k_new", q.dtype, (B, H_kv, d)), _dev(v_new, "v_new", q.dtype, (B, H_kv, d)),
        _dev(rope_cos, "rope_cos", torch.float32), _dev(rope_sin, "rope_sin", torch.float32, rope_cos.shape),
        rope_cos.shape[0], ROPE_STYLES[rope_style], int(max_seq_len), int(window), int(bool(ring)),
        float(scale) if scale else 0.0, _dev(out, "out", q.dtype, (B, H_q, d)), int(split_tokens), ws, wsn, st))
    return out, q_rot_out


# ---------------------------------------------------------------------------
# several new tokens per sequence (speculative verification, chunked prefill):
# k_new / v_new [B, n, H_kv, d], q / out [B, n, H_q, d]
# ---------------------------------------------------------------------------


def append_multi(k_cache: torch.Tensor, v_cache: torch.Tensor, positions: torch.Tensor, k_new: torch.Tensor,
                 v_new: torch.Tensor, rope_cos: torch.Tensor, rope_sin: torch.Tensor,
                 q: Optional[torch.Tensor] = None, block_table: Optional[torch.Tensor] = None,
                 rope_style: str = "interleaved", stream=None) -> None:
    """kvc_append_multi: token i of sequence b at slot positions[b] + i."""
    lib = _lib.load()
    dt = _dtype_code(k_new)
    B, n, H_kv, d = k_new.shape
    H_q = q.shape[2] if q is not None else H_kv
    if rope_cos.dim() != 2 or rope_cos.shape[1] != d // 2:
        raise ValueError(f"rope_cos must be [rows, {d // 2}], got {tuple(rope_cos.shape)}")
    T_max, tbl, block_size, mb, num_blocks, shape = _cache_geometry(k_cache, block_table, B, H_kv, d)
    _check(lib.kvc_append_multi(
        dt, B, n, H_q, H_kv, d,
        _dev(k_cache, "k_cache", k_new.dtype, shape), _dev(v_cache, "v_cache", k_new.dtype, shape), T_max,
        tbl, block_size, mb, num_blocks, _dev(positions, "positions", torch.int32, (B,)),
        _dev(k_new, "k_new", k_new.dtype), _dev(v_new, "v_new", k_new.dtype, (B, n, H_kv, d)),
        _dev(q, "q", k_new.dtype, (B, n, H_q, d)) if q is not None else None,
        _dev(rope_cos, "rope_cos", torch.float32), _dev(rope_sin, "rope_sin", torch.float32, rope_cos.shape),
        rope_cos.shape[0], ROPE_STYLES[rope_style], _stream(k_new.device, stream)))


def multi_workspace_bytes(dtype: torch.dtype, B: int, n: int, H_q: int, H_kv: int, d: int, max_seq_len: int,
                          window: int = 0, split_tokens: int = 0, pool_tokens: int = 0) -> int:
    """kvc_decode_multi_workspace_bytes."""
    lib = _lib.load()
    nb = lib.kvc_decode_multi_workspace_bytes(_cache_code(dtype), B, n, H_q, H_kv, d, max_seq_len, window,
                                              pool_tokens, split_tokens)
    if nb == (1 << 64) - 1:
        raise KvcError(3, lib.kvc_last_error().decode() or "unsupported sizes")
    return nb


def multi_split_tokens(dtype: torch.dtype, B: int, n: int, H_q: int, H_kv: int, d: int, max_seq_len: int,
                       window: int = 0, split_tokens: int = 0, pool_tokens: int = 0) -> int:
    """kvc_decode_multi_split_tokens."""
    lib = _lib.load()
    ts = lib.kvc_decode_multi_split_tokens(_cache_code(dtype), B, n, H_q, H_kv, d, max_seq_len, window,
                                           pool_tokens, split_tokens)
    if ts < 0:
        raise KvcError(3, lib.kvc_last_error().decode() or "unsupported sizes")
    return ts


def decode_attn_multi(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, seq_lens: torch.Tensor,
                      max_seq_len: int, window: int = 0, block_table: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None, scale: Optional[float] = None, split_tokens: int = 0,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """kvc_decode_attn_multi: q [B, n, H_q, d] (rotated), seq_lens after the append;
    returns out [B, n, H_q, d]."""
    lib = _lib.load()
    dt = _dtype_code(q)
    B, n, H_q, d = q.shape
    out = torch.empty_like(q) if out is None else out
    H_kv = k_cache.shape[1]
    T_max, tbl, block_size, mb, num_blocks, shape = _cache_geometry(k_cache, block_table, B, H_kv, d)
    st = _stream(q.device, stream)
    need = multi_workspace_bytes(q.dtype, B, n, H_q, H_kv, d, max_seq_len, window, split_tokens,
                                 pool_tokens=num_blocks * block_size)
    if workspace is not None:
        ws, wsn = _dev(workspace, "workspace", torch.uint8), workspace.numel()
    else:
        ws, wsn = _workspace(q.device, st, need)
    _check(lib.kvc_decode_attn_multi(
        dt, B, n, H_q, H_kv, d, _dev(q, "q", q.dtype, (B, n, H_q, d)),
        _dev(k_cache, "k_cache", q.dtype, shape), _dev(v_cache, "v_cache", q.dtype, shape), T_max,
        tbl, block_size, mb, num_blocks, _dev(seq_lens, "seq_lens", torch.int32, (B,)), int(max_seq_len),
        int(window), float(scale) if scale else 0.0, _dev(out, "out", q.dtype, (B, n, H_q, d)),
        int(split_tokens), ws, wsn, st))
    return out


# ---------------------------------------------------------------------------
# quantized cache: uint8 codes [.., d] with a float32 (step, zero point) pair
# [.., 2] per cached vector
# ---------------------------------------------------------------------------


def append_u8(k_codes: torch.Tensor, k_sz: torch.Tensor, v_codes: torch.Tensor, v_sz: torch.Tensor,
              positions: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, rope_cos: torch.Tensor,
              rope_sin: torch.Tensor, q: Optional[torch.Tensor] = None,
              block_table: Optional[torch.Tensor] = None, rope_style: str = "interleaved",
              stream=None, fmt: Optional[str] = None) -> None:
    """kvc_append_u8 (fmt None) or kvc_append_fp8 (fmt "e4m3" / "e5m2"):
    quantize the rotated new key and the new value into the code / pair
    arrays; rotate q (bf16 or f32, as k_new) in place if given."""
    lib = _lib.load()
    dt = _dtype_code(k_new)
    B, H_kv, d = k_new.shape
    H_q = q.shape[1] if q is not None else H_kv
    if rope_cos.dim() != 2 or rope_cos.shape[1] != d // 2:
        raise ValueError(f"rope_cos must be [rows, {d // 2}], got {tuple(rope_cos.shape)}")
    if block_table is not None:
        num_blocks, _, block_size, _ = k_codes.shape
        T_max, mb = 0, block_table.shape[1]
        tbl = _dev(block_table, "block_table", torch.int32, (B, mb))
        lead = (num_blocks, H_kv, block_size)
    else:
        T_max = k_codes.shape[2]
        tbl, block_size, mb, num_blocks = None, 0, 0, 0
        lead = (B, H_kv, T_max)
    _check(_q8_fn(lib, "append", fmt)(
        dt, B, H_q, H_kv, d,
        _dev(k_codes, "k_codes", torch.uint8, lead + (d,)), _dev(k_sz, "k_sz", torch.float32, lead + (2,)),
        _dev(v_codes, "v_codes", torch.uint8, lead + (d,)), _dev(v_sz, "v_sz", torch.float32, lead + (2,)), T_max,
        tbl, block_size, mb, num_blocks,
        _dev(positions, "positions", torch.int32, (B,)),
        _dev(k_new, "k_new", k_new.dtype), _dev(v_new, "v_new", k_new.dtype, (B, H_kv, d)),
        _dev(q, "q", k_new.dtype, (B, H_q, d)) if q is not None else None,
        _dev(rope_cos, "rope_cos", torch.float32), _dev(rope_sin, "rope_sin", torch.float32, rope_cos.shape),
        rope_cos.shape[0], ROPE_STYLES[rope_style], _stream(k_new.device, stream)))


def decode_attn_u8(q: torch.Tensor, k_codes: torch.Tensor, k_sz: torch.Tensor, v_codes: torch.Tensor,
                   v_sz: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                   out: Optional[torch.Tensor] = None, scale: Optional[float] = None, split_tokens: int = 0,
                   workspace: Optional[torch.Tensor] = None, stream=None,
                   fmt: Optional[str] = None) -> torch.Tensor:
    """kvc_decode_attn_u8 (fmt None) or kvc_decode_attn_fp8 (fmt "e4m3" /
    "e5m2") over an 8-bit contiguous cache [B, H_kv, T_max, d]; q and out bf16
    [B, H_q, d]."""
    lib = _lib.load()
    B, H_q, d = q.shape
    out = torch.empty_like(q) if out is None else out
    _, H_kv, T_max, _ = k_codes.shape
    st = _stream(q.device, stream)
    need = workspace_bytes(_q8_dtype(fmt), B, H_q, H_kv, d, max_seq_len, split_tokens)
    if workspace is not None:
        ws, wsn = _dev(workspace, "workspace", torch.uint8), workspace.numel()
    else:
        ws, wsn = _workspace(q.device, st, need)
    lead = (B, H_kv, T_max)
    _check(_q8_fn(lib, "decode_attn", fmt)(
        B, H_q, H_kv, d, _dev(q, "q", torch.bfloat16),
        _dev(k_codes, "k_codes", torch.uint8, lead + (d,)), _dev(k_sz, "k_sz", torch.float32, lead + (2,)),
        _dev(v_codes, "v_codes", torch.uint8, lead + (d,)), _dev(v_sz, "v_sz", torch.float32, lead + (2,)), T_max,
        _dev(seq_lens, "seq_lens", torch.int32, (B,)), int(max_seq_len), float(scale) if scale else 0.0,
        _dev(out, "out", torch.bfloat16, (B, H_q, d)), int(split_tokens), ws, wsn, st))
    return out


def decode_attn_paged_u8(q: torch.Tensor, k_codes: torch.Tensor, k_sz: torch.Tensor, v_codes: torch.Tensor,
                         v_sz: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                         out: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                         split_tokens: int = 0, workspace: Optional[torch.Tensor] = None,
                         stream=None, fmt: Optional[str] = None) -> torch.Tensor:
    """kvc_decode_attn_paged_u8 (fmt None) or kvc_decode_attn_paged_fp8 over
    8-bit pools [num_blocks, H_kv, block_size, d]."""
    lib = _lib.load()
    B, H_q, d = q.shape
    out = torch.empty_like(q) if out is None else out
    num_blocks, H_kv, block_size, _ = k_codes.shape
    st = _stream(q.device, stream)
    need = workspace_bytes(_q8_dtype(fmt), B, H_q, H_kv, d, max_seq_len, split_tokens,
                           pool_tokens=num_blocks * block_size)
    if workspace is not None:
        ws, wsn = _dev(workspace, "workspace", torch.uint8), workspace.numel()
    else:
        ws, wsn = _workspace(q.device, st, need)
    lead = (num_blocks, H_kv, block_size)
    _check(_q8_fn(lib, "decode_attn_paged", fmt)(
        B, H_q, H_kv, d, _dev(q, "q", torch.bfloat16),
        _dev(k_codes, "k_codes", torch.uint8, lead + (d,)), _dev(k_sz, "k_sz", torch.float32, lead + (2,)),
        _dev(v_codes, "v_codes", torch.uint8, lead + (d,)), _dev(v_sz, "v_sz", torch.float32, lead + (2,)),
        num_blocks, block_size, _dev(block_table, "block_table", torch.int32, (B, block_table.shape[1])),
        block_table.shape[1], _dev(seq_lens, "seq_lens", torch.int32, (B,)), int(max_seq_len),
        float(scale) if scale else 0.0, _dev(out, "out", torch.bfloat16, (B, H_q, d)),
        int(split_tokens), ws, wsn, st))
    return out


def decode_step_u8(q: torch.Tensor, k_codes: torch.Tensor, k_sz: torch.Tensor, v_codes: torch.Tensor,
                   v_sz: torch.Tensor, positions: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                   rope_cos: torch.Tensor, rope_sin: torch.Tensor, max_seq_len: int,
                   block_table: Optional[torch.Tensor] = None, rope_style: str = "interleaved",
                   q_rot_out: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                   scale: Optional[float] = None, split_tokens: int = 0,
                   workspace: Optional[torch.Tensor] = None, stream=None, fmt: Optional[str] = None):
    """kvc_decode_step_u8 (fmt None) or kvc_decode_step_fp8 (fmt "e4m3" /
    "e5m2"): the decode step over an 8-bit cache (contiguous codes
    [B, H_kv, T_max, d] or pools [num_blocks, H_kv, block_size, d] with a block
    table), append and attention in one launch; returns (out, q_rot_out)."""
    fn, args, out, q_rot_out = _step_u8_call(q, k_codes, k_sz, v_codes, v_sz, positions, k_new, v_new, rope_cos,
                                             rope_sin, max_seq_len, block_table, rope_style, q_rot_out, out, scale,
                                             split_tokens, workspace, stream, fmt)
    _check(fn(*args))
    return out, q_rot_out


def prepare_decode_step_u8(q: torch.Tensor, k_codes: torch.Tensor, k_sz: torch.Tensor, v_codes: torch.Tensor,
                           v_sz: torch.Tensor, positions: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                           rope_cos: torch.Tensor, rope_sin: torch.Tensor, max_seq_len: int,
                           block_table: Optional[torch.Tensor] = None, rope_style: str = "interleaved",
                           q_rot_out: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                           scale: Optional[float] = None, split_tokens: int = 0,
                           workspace: Optional[torch.Tensor] = None, stream=None,
                           fmt: Optional[str] = None) -> PreparedCall:
    """decode_step_u8 checked once, launched per call (as prepare_decode_step)."""
    fn, args, out, q_rot_out = _step_u8_call(q, k_codes, k_sz, v_codes, v_sz, positions, k_new, v_new, rope_cos,
                                             rope_sin, max_seq_len, block_table, rope_style, q_rot_out, out, scale,
                                             split_tokens, workspace, stream, fmt)
    if workspace is None:
        workspace = _WORKSPACES.get((q.device.index if q.device.index is not None else torch.cuda.current_device(),
                                     args[-1]))
    return PreparedCall(fn, args, (out, q_rot_out),
                        (q, k_codes, k_sz, v_codes, v_sz, positions, k_new, v_new, rope_cos, rope_sin, block_table,
                         workspace))


def _step_u8_call(q, k_codes, k_sz, v_codes, v_sz, positions, k_new, v_new, rope_cos, rope_sin, max_seq_len,
                  block_table, rope_style, q_rot_out, out, scale, split_tokens, workspace, stream, fmt=None):
    lib = _lib.load()
    B, H_q, d = q.shape
    H_kv = k_new.shape[1]
    out = torch.empty_like(q) if out is None else out
    q_rot_out = torch.empty_like(q) if q_rot_out is None else q_rot_out
    if rope_cos.dim() != 2 or rope_cos.shape[1] != d // 2:
        raise ValueError(f"rope_cos must be [rows, {d // 2}], got {tuple(rope_cos.shape)}")
    if block_table is not None:
        num_blocks, _, block_size, _ = k_codes.shape
        T_max, mb = 0, block_table.shape[1]
        tbl = _dev(block_table, "block_table", torch.int32, (B, mb))
        lead = (num_blocks, H_kv, block_size)
        pool_tokens = num_blocks * block_size
    else:
        T_max = k_codes.shape[2]
        tbl, block_size, mb, num_blocks = None, 0, 0, 0
        lead = (B, H_kv, T_max)
        pool_tokens = 0
    st = _stream(q.device, stream)
    need = workspace_bytes(_q8_dtype(fmt), B, H_q, H_kv, d, max_seq_len, split_tokens, pool_tokens=pool_tokens)
    if workspace is not None:
        ws, wsn = _dev(workspace, "workspace", torch.uint8), workspace.numel()
    else:
        ws, wsn = _workspace(q.device, st, need)
    args = (B, H_q, H_kv, d, _dev(q, "q", torch.bfloat16, (B, H_q, d)),
            _dev(q_rot_out, "q_rot_out", torch.bfloat16, (B, H_q, d)),
            _dev(k_codes, "k_codes", torch.uint8, lead + (d,)), _dev(k_sz, "k_sz", torch.float32, lead + (2,)),
            _dev(v_codes, "v_codes", torch.uint8, lead + (d,)), _dev(v_sz, "v_sz", torch.float32, lead + (2,)),
            T_max, tbl, block_size, mb, num_blocks, _dev(positions, "positions", torch.int32, (B,)),
            _dev(k_new, "k_new", torch.bfloat16, (B, H_kv, d)), _dev(v_new, "v_new", torch.bfloat16, (B, H_kv, d)),
            _dev(rope_cos, "rope_cos", torch.float32), _dev(rope_sin, "rope_sin", torch.float32, rope_cos.shape),
            rope_cos.shape[0], ROPE_STYLES[rope_style], int(max_seq_len), float(scale) if scale else 0.0,
            _dev(out, "out", torch.bfloat16, (B, H_q, d)), int(split_tokens), ws, wsn, st)
    if fmt is not None:
        if fmt not in FP8_FORMATS:
            raise ValueError(f"FP8 format must be one of {sorted(FP8_FORMATS)}, got {fmt!r}")
        return lib.kvc_decode_step_fp8, (FP8_FORMATS[fmt],) + args, out, q_rot_out
    return lib.kvc_decode_step_u8, args, out, q_rot_out


def append_fp8(*args, fmt: str = "e4m3", **kw) -> None:
    """kvc_append_fp8: append_u8's arguments, FP8 codes of format fmt."""
    return append_u8(*args, fmt=fmt, **kw)


def decode_attn_fp8(*args, fmt: str = "e4m3", **kw) -> torch.Tensor:
    """kvc_decode_attn_fp8: decode_attn_u8's arguments over FP8 codes of format fmt."""
    return decode_attn_u8(*args, fmt=fmt, **kw)


def decode_attn_paged_fp8(*args, fmt: str = "e4m3", **kw) -> torch.Tensor:
    """kvc_decode_attn_paged_fp8: decode_attn_paged_u8's arguments over FP8 codes."""
    return decode_attn_paged_u8(*args, fmt=fmt, **kw)


def decode_step_fp8(*args, fmt: str = "e4m3", **kw):
    """kvc_decode_step_fp8: decode_step_u8's arguments over FP8 codes of format fmt."""
    return decode_step_u8(*args, fmt=fmt, **kw)


def prepare_decode_step_fp8(*args, fmt: str = "e4m3", **kw) -> PreparedCall:
    """prepare_decode_step_u8 for FP8 codes of format fmt."""
    return prepare_decode_step_u8(*args, fmt=fmt, **kw)


# ---------------------------------------------------------------------------
# Latent cache (multi-head latent attention): cache [B, T_max, d_latent + rope_dim]
# ---------------------------------------------------------------------------

def append_mla(cache: torch.Tensor, positions: torch.Tensor, c_kv_new: torch.Tensor,
               k_rope_new: Optional[torch.Tensor] = None, stream=None) -> None:
    """kvc_append_mla: store [c_kv_new[b] | k_rope_new[b]] at slot positions[b] of each sequence."""
    lib = _lib.load()
    dt = _dtype_code(cache)
    B, T_max, row = cache.shape
    d_latent = c_kv_new.shape[-1]
    rope_dim = row - d_latent
    st = _stream(cache.device, stream)
    _check(lib.kvc_append_mla(
        dt, B, d_latent, rope_dim, _dev(cache, "cache", cache.dtype), T_max,
        _dev(positions, "positions", torch.int32, (B,)),
        _dev(c_kv_new, "c_kv_new", cache.dtype, (B, d_latent)),
        _dev(k_rope_new, "k_rope_new", cache.dtype, (B, rope_dim)) if rope_dim > 0 else None, st))


def mla_workspace_bytes(B: int, H: int, d_latent: int, max_seq_len: int, split_tokens: int = 0) -> int:
    """kvc_decode_mla_workspace_bytes."""
    lib = _lib.load()
    n = lib.kvc_decode_mla_workspace_bytes(B, H, d_latent, max_seq_len, split_tokens)
    if n == (1 << 64) - 1:
        raise KvcError(2, lib.kvc_last_error().decode() or "invalid sizes for the latent-cache workspace")
    return int(n)


def mla_split_tokens(B: int, H: int, d_latent: int, max_seq_len: int, split_tokens: int = 0) -> int:
    """kvc_decode_mla_split_tokens: tokens per split the latent-cache decode uses."""
    lib = _lib.load()
    n = lib.kvc_decode_mla_split_tokens(B, H, d_latent, max_seq_len, split_tokens)
    if n < 0:
        raise KvcError(2, lib.kvc_last_error().decode() or "invalid sizes for the latent-cache decode")
    return int(n)


def _mla_args(q, cache, w_uk, w_uv, b_uv, out):
    B, H, d_k = q.shape
    _, T_max, row = cache.shape
    d_latent = w_uk.shape[1]
    if out is None:
        out = torch.empty((B, H, d_k), dtype=torch.float32, device=q.device)
    ptrs = (_dev(w_uk, "w_uk", torch.bfloat16, (H * d_k, d_latent)),
            _dev(w_uv, "w_uv", torch.bfloat16, (H * d_k, d_latent)),
            _dev(b_uv, "b_uv", torch.bfloat16, (H * d_k,)) if b_uv is not None else None)
    return B, H, d_k, d_latent, row - d_latent, T_max, out, ptrs


def decode_attn_mla(q: torch.Tensor, cache: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                    w_uk: torch.Tensor, w_uv: torch.Tensor, b_uv: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, scale: Optional[float] = None, split_tokens: int = 0,
                    workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """kvc_decode_attn_mla: q bf16 [B, H, d_k] over a latent cache [B, T_max, d_latent + rope_dim];
    returns out float32 [B, H, d_k]."""
    lib = _lib.load()
    B, H, d_k, d_latent, rope_dim, T_max, out, (wk, wv, bv) = _mla_args(q, cache, w_uk, w_uv, b_uv, out)
    st = _stream(q.device, stream)
    need = mla_workspace_bytes(B, H, d_latent, max_seq_len, split_tokens)
    if workspace is not None:
        ws, wsn = _dev(workspace, "workspace", torch.uint8), workspace.numel()
    else:
        ws, wsn = _workspace(q.device, st, need)
    _check(lib.kvc_decode_attn_mla(
        B, H, d_k, d_latent, rope_dim, _dev(q, "q", torch.bfloat16), _dev(cache, "cache", torch.bfloat16), T_max,
        _dev(seq_lens, "seq_lens", torch.int32, (B,)), int(max_seq_len), wk, wv, bv,
        float(scale) if scale else 0.0, _dev(out, "out", torch.float32, (B, H, d_k)), int(split_tokens),
        ws, wsn, st))
    return out


def decode_step_mla(q: torch.Tensor, cache: torch.Tensor, positions: torch.Tensor, c_kv_new: torch.Tensor,
                    k_rope_new: Optional[torch.Tensor], max_seq_len: int, w_uk: torch.Tensor, w_uv: torch.Tensor,
                    b_uv: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                    scale: Optional[float] = None, split_tokens: int = 0,
                    workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """kvc_decode_step_mla: append the new rows, then attend positions[b] + 1 tokens."""
    lib = _lib.load()
    B, H, d_k, d_latent, rope_dim, T_max, out, (wk, wv, bv) = _mla_args(q, cache, w_uk, w_uv, b_uv, out)
    st = _stream(q.device, stream)
    need = mla_workspace_bytes(B, H, d_latent, max_seq_len, split_tokens)
    if workspace is not None:
        ws, wsn = _dev(workspace, "workspace", torch.uint8), workspace.numel()
    else:
        ws, wsn = _workspace(q.device, st, need)
    _check(lib.kvc_decode_step_mla(
        B, H, d_k, d_latent, rope_dim, _dev(q, "q", torch.bfloat16), _dev(cache, "cache", torch.bfloat16), T_max,
        _dev(positions, "positions", torch.int32, (B,)),
        _dev(c_kv_new, "c_kv_new", torch.bfloat16, (B, d_latent)),
        _dev(k_rope_new, "k_rope_new", torch.bfloat16, (B, rope_dim)) if rope_dim > 0 else None,
        int(max_seq_len), wk, wv, bv, float(scale) if scale else 0.0,
        _dev(out, "out", torch.float32, (B, H, d_k)), int(split_tokens), ws, wsn, st))
    return out

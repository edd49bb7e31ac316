"""ctypes binding of libpkv (include/pkv.h).

Argument marshalling only: every call checks the torch tensors it is handed
(device, dtype, contiguity, shape), passes raw pointers, sizes and the current
HIP stream to the C ABI, and turns a negative status into an exception.  No
computation happens here, and there is no fallback: if libpkv.so is missing
the first call raises.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

PKV_F32, PKV_BF16, PKV_FP8_E4M3 = 0, 1, 2
PKV_SEG_CAUSAL, PKV_SEG_FULL = 0, 1
PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EHIP, PKV_ERANGE, PKV_EWINDOW = 0, -1, -2, -3, -4, -5

_TORCH_DTYPE = {
    torch.float32: PKV_F32,
    torch.bfloat16: PKV_BF16,
    torch.uint8: PKV_FP8_E4M3,
    torch.float8_e4m3fn: PKV_FP8_E4M3,
}


class PkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"pkv status {status}: {message}")
        self.status = status


class PkvValueError(PkvError, ValueError):
    """Bad arguments (the pages raise ValueError for these)."""


class _Pools(ctypes.Structure):
    _fields_ = [
        ("key", ctypes.c_void_p),
        ("value", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int64),
        ("block_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
        ("k_inv_scale", ctypes.c_float),
        ("v_inv_scale", ctypes.c_float),
    ]


class _AttnMeta(ctypes.Structure):
    _fields_ = [
        ("block_table", ctypes.c_void_p),
        ("query_start_loc", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("segments", ctypes.c_void_p),
        ("segment_start_loc", ctypes.c_void_p),
        ("seq_order", ctypes.c_void_p),
        ("host_seq_lens", ctypes.c_void_p),
        ("query_pos", ctypes.c_void_p),
        ("table_width", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("max_query_len", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
    ]


class _WindowConfig(ctypes.Structure):
    _fields_ = [
        ("num_blocks", ctypes.c_int64),
        ("block_size", ctypes.c_int32),
        ("chunk_size", ctypes.c_int32),
        ("sink_chunks", ctypes.c_int32),
        ("window_chunks", ctypes.c_int32),
        ("chunks_per_block", ctypes.c_int32),
        ("reset_at_boundary", ctypes.c_int32),
        ("scratch_blocks", ctypes.c_int32),
        ("compact", ctypes.c_int32),
    ]


class _Staging(ctypes.Structure):
    _fields_ = [
        ("stage_key", ctypes.c_void_p),
        ("stage_value", ctypes.c_void_p),
        ("capacity_tokens", ctypes.c_int64),
        ("first_block", ctypes.c_int32),
    ]


class _StagingState(ctypes.Structure):
    _fields_ = [
        ("session", ctypes.c_int64),
        ("history_tokens", ctypes.c_int64),
        ("chunk_tokens", ctypes.c_int64),
        ("max_seq_len", ctypes.c_int32),
        ("num_history_blocks", ctypes.c_int32),
        ("history_blocks", ctypes.POINTER(ctypes.c_int32)),
        ("block_capacity", ctypes.c_int32),
    ]


_lib = None

_P = ctypes.c_void_p
_I32, _I64, _F32, _SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_PI32 = ctypes.POINTER(ctypes.c_int32)
_PI64 = ctypes.POINTER(ctypes.c_int64)
_PPOOLS = ctypes.POINTER(_Pools)

_ATTN_ARGS = [_P, _I32, _I64, _I32, _PPOOLS, _P, _I32, _P, _P, _I32, _I32, _I32, _P, _P, _P, _P, _F32, _P, _P, _SZ, _P]

_SIGNATURES = {
    "pkv_paged_write": (ctypes.c_int, [_P, _P, _I32, _I64, _P, _PPOOLS, _P]),
    "pkv_gather": (ctypes.c_int, [_PPOOLS, _P, _I32, _I32, _P, _P, _P]),
    "pkv_paged_attn": (ctypes.c_int, _ATTN_ARGS),
    "pkv_paged_attn_main": (ctypes.c_int, _ATTN_ARGS),
    "pkv_paged_attn_merge": (ctypes.c_int, _ATTN_ARGS),
    "pkv_paged_attn_noalloc": (ctypes.c_int, _ATTN_ARGS[:-3] + [_P]),  # no workspace, workspace_bytes
    "pkv_paged_write_attn": (
        ctypes.c_int,
        [_P, _I32, _I64, _I32, _P, _P, _I32, _I64, _P, _P, _P, _I64, _P, _PPOOLS,
         ctypes.POINTER(_AttnMeta), ctypes.POINTER(_Staging), _F32, _P, _P, _SZ, _P],
    ),
    "pkv_paged_attn_workspace_size": (_SZ, [_I64, _I32, _I32, _I32, _I32, _I32, _I32]),
    "pkv_slot_mapping": (ctypes.c_int, [_PI32, _I64, _I64, _I64, _I32, _PI64]),
    "pkv_window_table": (ctypes.c_int, [_PI32, _I64, _I64, _I64, _I64, _I64, _I32, _PI32, _I32, _PI32, _PI32]),
    "pkv_action_table": (ctypes.c_int, [_PI32, _I32, _PI32, _PI32, _PI32, _I32, _I64, _I32]),
    "pkv_build_segments": (ctypes.c_int, [_PI32, _I32, _I32, _I32, _PI32, _I32, _PI32]),
    "pkv_staging_decide": (
        ctypes.c_int,
        [ctypes.POINTER(_StagingState), _I64, _PI32, _I32, _I64, _I64, _I32, _I32, _I64, _PI32, _PI32],
    ),
    "pkv_validate_metadata_host": (
        ctypes.c_int,
        [_PI32, _PI32, _I32, _PI32, _I32, _I64, _I32, _I32, _I32, _PI32, _PI32, _PI32],
    ),
    "pkv_wm_max_video_blocks": (ctypes.c_int32, [ctypes.POINTER(_WindowConfig)]),
    "pkv_wm_create": (ctypes.c_int, [ctypes.POINTER(_WindowConfig), ctypes.POINTER(ctypes.c_void_p)]),
    "pkv_wm_destroy": (None, [_P]),
    "pkv_wm_begin_request": (ctypes.c_int, [_P, _PI32]),
    "pkv_wm_end_request": (ctypes.c_int, [_P, _I32]),
    "pkv_wm_prepare": (ctypes.c_int, [_P, _I32, _I64, _I32, _I64, _PI64, _PI64]),
    "pkv_wm_window_table": (ctypes.c_int, [_P, _I32, _PI32, _I32, _PI32, _PI32, _PI32]),
    "pkv_wm_commit": (ctypes.c_int, [_P, _I32]),
    "pkv_wm_info": (ctypes.c_int, [_P, _I32, _PI64]),
    "pkv_wm_block_table": (ctypes.c_int, [_P, _I32, _PI32, _I32, _PI32]),
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_window_capacity": (
        ctypes.c_int,
        [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)],
    ),
    "pkv_last_attn_plan": (ctypes.c_char_p, []),
    "pkv_probe_mfma": (ctypes.c_int, [ctypes.c_int64, _P, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64), _P]),
    "pkv_probe_stream": (ctypes.c_int, [_P, ctypes.c_int64, _P, _P]),
    "pkv_version": (ctypes.c_char_p, []),
}

EXPORTED = tuple(_SIGNATURES)


def lib():
    """The loaded libpkv.so.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_174_amd.build` "
                "(there is no non-HIP fallback)"
            )
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int) -> None:
    if status != PKV_OK:
        msg = lib().pkv_last_error().decode()
        if status == PKV_EINVAL:
            raise PkvValueError(status, msg)
        raise PkvError(status, msg)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    return t.data_ptr()


def _host_i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


class Pools:
    """One layer's K and V pools: two device tensors of shape
    ``[num_blocks * block_size, num_kv_heads, head_dim]`` (float32, bfloat16, or
    uint8 / float8_e4m3fn storage for fp8), plus the fp8 scales."""

    def __init__(self, key, value, block_size=16, k_scale=1.0, v_scale=1.0, k_inv_scale=1.0, v_inv_scale=1.0):
        if key.shape != value.shape or key.dtype != value.dtype:
            raise ValueError("key and value pools must match in shape and dtype")
        if key.dim() != 3 or key.shape[0] % block_size:
            raise ValueError("pools must be [num_blocks * block_size, num_kv_heads, head_dim]")
        if key.dtype not in _TORCH_DTYPE:
            raise ValueError(f"unsupported pool dtype {key.dtype}")
        _dev(key, "key pool")
        _dev(value, "value pool")
        self.key, self.value = key, value
        self.block_size = int(block_size)
        self.num_blocks = key.shape[0] // block_size
        self.num_kv_heads, self.head_dim = int(key.shape[1]), int(key.shape[2])
        self.dtype = _TORCH_DTYPE[key.dtype]
        self.k_scale, self.v_scale = float(k_scale), float(v_scale)
        self.k_inv_scale, self.v_inv_scale = float(k_inv_scale), float(v_inv_scale)

    def c_struct(self) -> _Pools:
        return _Pools(
            self.key.data_ptr(),
            self.value.data_ptr(),
            self.num_blocks,
            self.block_size,
            self.num_kv_heads,
            self.head_dim,
            self.dtype,
            self.k_scale,
            self.v_scale,
            self.k_inv_scale,
            self.v_inv_scale,
        )


# ----------------------------------------------------------------- device calls


def pkv_paged_write(key: torch.Tensor, value: torch.Tensor, slot_mapping: torch.Tensor, pools: Pools, stream=None):
    if key.shape != value.shape or key.dtype != value.dtype:
        raise ValueError("key and value must match")
    if key.dim() != 3 or key.shape[1:] != (pools.num_kv_heads, pools.head_dim):
        raise ValueError("key/value must be [tokens, num_kv_heads, head_dim] matching the pools")
    if slot_mapping.numel() != key.shape[0]:
        raise ValueError("slot_mapping needs one entry per token")
    src = _TORCH_DTYPE.get(key.dtype, -1)
    ps = pools.c_struct()
    _check(
        lib().pkv_paged_write(
            _dev(key, "key"),
            _dev(value, "value"),
            src,
            key.shape[0],
            _dev(slot_mapping, "slot_mapping", torch.int64),
            ctypes.byref(ps),
            _stream(stream),
        )
    )


def pkv_gather(pools: Pools, block_ids: torch.Tensor, n_blocks: int, first_block: int, stage_key, stage_value, stream=None):
    need = n_blocks * pools.block_size
    for name, t in (("stage_key", stage_key), ("stage_value", stage_value)):
        if t.dtype != pools.key.dtype or t.dim() != 3 or t.shape[1:] != pools.key.shape[1:] or t.shape[0] < need:
            raise ValueError(f"{name} must be [>= {need}, num_kv_heads, head_dim] of the pool dtype")
    if block_ids.numel() < n_blocks:
        raise ValueError("block_ids shorter than n_blocks")
    ps = pools.c_struct()
    _check(
        lib().pkv_gather(
            ctypes.byref(ps),
            _dev(block_ids, "block_ids", torch.int32),
            int(n_blocks),
            int(first_block),
            _dev(stage_key, "stage_key"),
            _dev(stage_value, "stage_value"),
            _stream(stream),
        )
    )


def pkv_paged_attn_workspace_size(num_q_tokens, num_q_heads, num_kv_heads, head_dim, num_seqs, max_query_len, max_seq_len) -> int:
    return int(
        lib().pkv_paged_attn_workspace_size(
            num_q_tokens, num_q_heads, num_kv_heads, head_dim, num_seqs, max_query_len, max_seq_len
        )
    )


def pkv_paged_attn(
    q: torch.Tensor,
    pools: Pools,
    block_table: torch.Tensor,
    query_start_loc: torch.Tensor,
    seq_lens: torch.Tensor,
    segments: torch.Tensor,
    segment_start_loc: torch.Tensor,
    softmax_scale: float,
    max_query_len: int,
    max_seq_len: int,
    out: torch.Tensor | None = None,
    workspace: torch.Tensor | None = None,
    stream=None,
    seq_order: torch.Tensor | None = None,
    host_seq_lens=None,
    _entry: str = "pkv_paged_attn",
) -> torch.Tensor:
    """Paged attention (see include/pkv.h).  ``seq_order`` (int32 [num_seqs], a
    permutation) is the order the sequences' work is dispatched in, e.g.
    ForwardPlan.seq_order (longest first); ``host_seq_lens`` (host ints, e.g.
    ForwardPlan.kv_lens) lets the library plan the work split from the
    sequences' own lengths.  Neither changes the result beyond rounding."""
    if q.dim() != 3 or q.shape[2] != pools.head_dim:
        raise ValueError("q must be [tokens, num_q_heads, head_dim]")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if block_table.dim() != 2:
        raise ValueError("block_table must be [num_seqs, width]")
    num_seqs = block_table.shape[0]
    if query_start_loc.numel() != num_seqs + 1 or seq_lens.numel() != num_seqs or segment_start_loc.numel() != num_seqs + 1:
        raise ValueError("query_start_loc, seq_lens and segment_start_loc must match block_table's rows")
    order_ptr = None
    if seq_order is not None:
        if seq_order.numel() != num_seqs:
            raise ValueError("seq_order must hold one entry per sequence")
        order_ptr = _dev(seq_order, "seq_order", torch.int32)
    hl = _host_lens(host_seq_lens, num_seqs)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    ws_args = (ws_ptr, ws_bytes)
    if _entry == "pkv_paged_attn_noalloc":
        if workspace is not None:
            raise ValueError("pkv_paged_attn_noalloc takes no workspace")
        ws_args = ()
    ps = pools.c_struct()
    _check(
        getattr(lib(), _entry)(
            _dev(q, "q"),
            _TORCH_DTYPE.get(q.dtype, -1),
            q.shape[0],
            q.shape[1],
            ctypes.byref(ps),
            _dev(block_table, "block_table", torch.int32),
            block_table.shape[1],
            _dev(query_start_loc, "query_start_loc", torch.int32),
            _dev(seq_lens, "seq_lens", torch.int32),
            num_seqs,
            int(max_query_len),
            int(max_seq_len),
            _dev(segments, "segments", torch.int32),
            _dev(segment_start_loc, "segment_start_loc", torch.int32),
            order_ptr,
            None if hl is None else _ptr(hl, ctypes.c_int32),
            float(softmax_scale),
            _dev(out, "out"),
            *ws_args,
            _stream(stream),
        )
    )
    return out


def pkv_paged_attn_noalloc(*args, **kwargs) -> torch.Tensor:
    """pkv_paged_attn without a workspace: the split partials go to the
    library's static per-device scratch (see include/pkv.h)."""
    return pkv_paged_attn(*args, _entry="pkv_paged_attn_noalloc", **kwargs)


def pkv_paged_attn_main(*args, **kwargs) -> torch.Tensor:
    """The attention-kernel half of pkv_paged_attn (same arguments)."""
    return pkv_paged_attn(*args, _entry="pkv_paged_attn_main", **kwargs)


def pkv_paged_attn_merge(*args, **kwargs) -> torch.Tensor:
    """The split-merge half of pkv_paged_attn (same arguments; `out` required)."""
    if kwargs.get("out") is None:
        raise ValueError("pkv_paged_attn_merge needs the `out` its pkv_paged_attn_main call wrote")
    return pkv_paged_attn(*args, _entry="pkv_paged_attn_merge", **kwargs)


def _host_lens(lens, num_seqs):
    if lens is None:
        return None
    a = _host_i32(lens)
    if a.size != num_seqs:
        raise ValueError("host_seq_lens needs one entry per sequence")
    return a


def _kv_rows(key, value, slot_mapping, pools, what):
    """(key ptr, value ptr, tokens, slot ptr) of one write, or nulls for none."""
    if key is None and value is None and slot_mapping is None:
        return None, None, 0, None
    if key is None or value is None or slot_mapping is None:
        raise ValueError(f"{what}: key, value and slot_mapping go together")
    if key.shape != value.shape or key.dtype != value.dtype:
        raise ValueError(f"{what}: key and value must match")
    if key.dim() != 3 or key.shape[1:] != (pools.num_kv_heads, pools.head_dim):
        raise ValueError(f"{what}: key/value must be [tokens, num_kv_heads, head_dim] matching the pools")
    if slot_mapping.numel() != key.shape[0]:
        raise ValueError(f"{what}: slot_mapping needs one entry per token")
    if key.shape[0] == 0:
        return None, None, 0, None
    return (_dev(key, f"{what} key"), _dev(value, f"{what} value"), key.shape[0],
            _dev(slot_mapping, f"{what} slot_mapping", torch.int64))


def pkv_paged_write_attn(
    q: torch.Tensor,
    key: torch.Tensor,
    value: torch.Tensor,
    slot_mapping: torch.Tensor,
    pools: Pools,
    meta,
    softmax_scale: float,
    *,
    action_key: torch.Tensor | None = None,
    action_value: torch.Tensor | None = None,
    action_slot_mapping: torch.Tensor | None = None,
    stage_key: torch.Tensor | None = None,
    stage_value: torch.Tensor | None = None,
    first_block: int = 0,
    out: torch.Tensor | None = None,
    workspace: torch.Tensor | None = None,
    stream=None,
) -> torch.Tensor:
    """One layer of the fused op (see include/pkv.h): writes the current video
    K/V and the action K/V through their slot mappings, optionally stages the
    window into ``stage_key``/``stage_value`` from ``first_block`` on, and
    attends.  ``meta`` is any object with the attention metadata as device
    tensors (block_table, query_start_loc, seq_lens, segments,
    segment_start_loc, seq_order or None, query_pos or None), the host ints
    max_query_len and max_seq_len, and optionally kv_lens (host sequence
    lengths, a planning hint) -- a ForwardPlan is one."""
    if q.dim() != 3 or q.shape[2] != pools.head_dim:
        raise ValueError("q must be [tokens, num_q_heads, head_dim]")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    kp, vp, n, sp = _kv_rows(key, value, slot_mapping, pools, "video")
    akp, avp, an, asp = _kv_rows(action_key, action_value, action_slot_mapping, pools, "action")
    kv_dtype = _TORCH_DTYPE.get(key.dtype, -1) if key is not None else _TORCH_DTYPE.get(q.dtype, -1)
    if an and action_key.dtype != key.dtype:
        raise ValueError("action K/V must have the video K/V's dtype")
    bt = meta.block_table
    if bt.dim() != 2:
        raise ValueError("block_table must be [num_seqs, width]")
    num_seqs = bt.shape[0]
    if (meta.query_start_loc.numel() != num_seqs + 1 or meta.seq_lens.numel() != num_seqs
            or meta.segment_start_loc.numel() != num_seqs + 1):
        raise ValueError("query_start_loc, seq_lens and segment_start_loc must match block_table's rows")
    order = getattr(meta, "seq_order", None)
    if order is not None and order.numel() != num_seqs:
        raise ValueError("seq_order must hold one entry per sequence")
    qpos = getattr(meta, "query_pos", None)
    if qpos is not None and qpos.numel() != num_seqs:
        raise ValueError("query_pos must hold one entry per sequence")
    hl = _host_lens(getattr(meta, "kv_lens", None), num_seqs)
    m = _AttnMeta(
        _dev(bt, "block_table", torch.int32),
        _dev(meta.query_start_loc, "query_start_loc", torch.int32),
        _dev(meta.seq_lens, "seq_lens", torch.int32),
        _dev(meta.segments, "segments", torch.int32),
        _dev(meta.segment_start_loc, "segment_start_loc", torch.int32),
        None if order is None else _dev(order, "seq_order", torch.int32),
        None if hl is None else hl.ctypes.data,
        None if qpos is None else _dev(qpos, "query_pos", torch.int32),
        bt.shape[1],
        num_seqs,
        int(meta.max_query_len),
        int(meta.max_seq_len),
    )
    st_ptr = None
    if stage_key is not None or stage_value is not None:
        for name, t in (("stage_key", stage_key), ("stage_value", stage_value)):
            if t is None or t.dtype != pools.key.dtype or t.dim() != 3 or t.shape[1:] != pools.key.shape[1:]:
                raise ValueError(f"{name} must be [capacity, num_kv_heads, head_dim] of the pool dtype")
        if stage_key.shape[0] != stage_value.shape[0]:
            raise ValueError("stage_key and stage_value must have the same capacity")
        st = _Staging(_dev(stage_key, "stage_key"), _dev(stage_value, "stage_value"), stage_key.shape[0],
                      int(first_block))
        st_ptr = ctypes.byref(st)
    elif first_block:
        raise ValueError("first_block needs staging buffers")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    ps = pools.c_struct()
    _check(
        lib().pkv_paged_write_attn(
            _dev(q, "q"), _TORCH_DTYPE.get(q.dtype, -1), q.shape[0], q.shape[1],
            kp, vp, kv_dtype, n, sp, akp, avp, an, asp,
            ctypes.byref(ps), ctypes.byref(m), st_ptr, float(softmax_scale),
            _dev(out, "out"), ws_ptr, ws_bytes, _stream(stream),
        )
    )
    return out


# ----------------------------------------------------------------- host metadata


def pkv_action_table(table, kv_len: int, action_block_ids, action_tokens: int, block_size: int = 16):
    """Appends the action scratch blocks to a visible-window table (include/pkv.h).
    Returns (table, kv_len)."""
    t = _host_i32(table)
    ids = _host_i32(action_block_ids)
    cap = t.size + max(0, -(-int(action_tokens) // block_size))
    out = np.zeros(cap, dtype=np.int32)
    out[: t.size] = t
    count, kl = ctypes.c_int32(t.size), ctypes.c_int32(int(kv_len))
    _check(lib().pkv_action_table(_ptr(out, ctypes.c_int32), cap, ctypes.byref(count), ctypes.byref(kl),
                                  _ptr(ids, ctypes.c_int32), ids.size, int(action_tokens), block_size))
    return out[: count.value], int(kl.value)



def pkv_slot_mapping(block_ids, first_position: int, num_tokens: int, block_size: int = 16) -> np.ndarray:
    ids = _host_i32(block_ids)
    out = np.empty(max(num_tokens, 0), dtype=np.int64)
    _check(lib().pkv_slot_mapping(_ptr(ids, ctypes.c_int32), ids.size, first_position, num_tokens, block_size, _ptr(out, ctypes.c_int64)))
    return out


def pkv_window_table(block_ids, history_tokens, query_tokens, sink_tokens, window_tokens, block_size=16):
    ids = _host_i32(block_ids)
    table = np.empty(ids.size, dtype=np.int32)
    count, kv_len = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(
        lib().pkv_window_table(
            _ptr(ids, ctypes.c_int32),
            ids.size,
            history_tokens,
            query_tokens,
            min(int(sink_tokens), 1 << 62),
            min(int(window_tokens), 1 << 62),
            block_size,
            _ptr(table, ctypes.c_int32),
            table.size,
            ctypes.byref(count),
            ctypes.byref(kv_len),
        )
    )
    return table[: count.value].copy(), int(kv_len.value)


def pkv_window_capacity(sink_tokens, window_tokens, chunk_size, block_size=16, action_tokens=0) -> int:
    out = ctypes.c_int64(0)
    _check(lib().pkv_window_capacity(int(sink_tokens), int(window_tokens), int(chunk_size), int(block_size),
                                     int(action_tokens), ctypes.byref(out)))
    return int(out.value)


def pkv_build_segments(full_spans, query_offset: int, query_len: int) -> np.ndarray:
    spans = _host_i32(full_spans).reshape(-1, 2) if len(full_spans) else np.zeros((0, 2), dtype=np.int32)
    cap = 2 * len(spans) + 1
    out = np.zeros((cap, 4), dtype=np.int32)
    count = ctypes.c_int32(0)
    _check(
        lib().pkv_build_segments(
            _ptr(spans, ctypes.c_int32), len(spans), query_offset, query_len, _ptr(out, ctypes.c_int32), cap, ctypes.byref(count)
        )
    )
    return out[: count.value].copy()


class StagingState:
    """Caller-owned pkv_staging_state with room for ``block_capacity`` history block ids."""

    def __init__(self, block_capacity: int):
        self.blocks = np.zeros(max(int(block_capacity), 1), dtype=np.int32)
        self.c = _StagingState(-1, 0, 0, 0, 0, self.blocks.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                               int(block_capacity))


def pkv_staging_decide(state: StagingState, session: int, table, history_tokens: int, chunk_tokens: int,
                       max_seq_len: int, block_size: int, capacity_tokens: int) -> tuple[bool, int]:
    """(reuse, first_block) of one staged forward; see include/pkv.h."""
    t = _host_i32(table)
    reuse, first = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(
        lib().pkv_staging_decide(ctypes.byref(state.c), int(session), _ptr(t, ctypes.c_int32), t.size,
                                 int(history_tokens), int(chunk_tokens), int(max_seq_len), int(block_size),
                                 int(capacity_tokens), ctypes.byref(reuse), ctypes.byref(first))
    )
    return bool(reuse.value), int(first.value)


def pkv_validate_metadata_host(query_start_loc, seq_lens, block_table, num_blocks, block_size, max_query_len, max_seq_len,
                               segments, segment_start_loc, query_pos=None):
    qsl, sl, bt = _host_i32(query_start_loc), _host_i32(seq_lens), _host_i32(block_table)
    qp = None if query_pos is None else _host_i32(query_pos)
    if qp is not None and qp.size != sl.size:
        raise ValueError("query_pos needs one entry per sequence")
    seg, sloc = _host_i32(segments).reshape(-1, 4), _host_i32(segment_start_loc)
    if bt.ndim != 2:
        raise ValueError("block_table must be 2-D")
    _check(
        lib().pkv_validate_metadata_host(
            _ptr(qsl, ctypes.c_int32),
            _ptr(sl, ctypes.c_int32),
            sl.size,
            _ptr(bt, ctypes.c_int32),
            bt.shape[1],
            num_blocks,
            block_size,
            max_query_len,
            max_seq_len,
            _ptr(seg, ctypes.c_int32),
            _ptr(sloc, ctypes.c_int32),
            None if qp is None else _ptr(qp, ctypes.c_int32),
        )
    )


def pkv_last_error() -> str:
    return lib().pkv_last_error().decode()


def pkv_probe_mfma(iters: int, sink: torch.Tensor, stream=None) -> int:
    """Enqueues the matrix-core peak probe; returns the FLOP it performs.
    sink: a float32 device tensor of at least 512 x CU-count elements."""
    flop = ctypes.c_int64(0)
    _check(lib().pkv_probe_mfma(int(iters), _dev(sink, "sink", torch.float32), sink.numel(), ctypes.byref(flop),
                                _stream(stream)))
    return int(flop.value)


def pkv_probe_stream(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Enqueues one read of src's bytes (the HBM read-rate probe); sink: a
    device tensor of at least 4 KB."""
    if sink.numel() * sink.element_size() < 4096:
        raise ValueError("sink must hold at least 4 KB")
    _check(lib().pkv_probe_stream(_dev(src, "src"), src.numel() * src.element_size(), _dev(sink, "sink"),
                                  _stream(stream)))


def pkv_last_attn_plan() -> str:
    return lib().pkv_last_attn_plan().decode()


def pkv_version() -> str:
    return lib().pkv_version().decode()

"""Host window manager (ctypes binding of the pkv_wm_* calls in include/pkv.h).

The block allocator, per-request block tables, chunk-granular eviction,
compaction and visible-window tables live in the C library; this class only
marshals arguments.  Pages cited by tag and function: P1
"vllm_omni/experimental/ar_diffusion/kv_cache/paged_attention.py", P2
"tests/diffusion/ar_diffusion/test_paged_attention.py".
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np

from . import _lib as L


@dataclass(frozen=True)
class WindowConfig:
    num_blocks: int
    chunk_size: int
    window_chunks: int
    sink_chunks: int = 0
    block_size: int = 16
    chunks_per_block: int = 1
    reset_at_boundary: bool = False
    scratch_blocks: int = 0
    compact: bool = True

    def c_struct(self):
        return L._WindowConfig(self.num_blocks, self.block_size, self.chunk_size, self.sink_chunks,
                               self.window_chunks, self.chunks_per_block, int(self.reset_at_boundary),
                               self.scratch_blocks, int(self.compact))

    @property
    def max_video_blocks(self) -> int:
        """The constant width of a visible window in blocks (P1 max_video_blocks)."""
        n = L.lib().pkv_wm_max_video_blocks(ctypes.byref(self.c_struct()))
        if n < 0:
            raise ValueError("bad window configuration")
        return int(n)


class WindowManager:
    """Blocks of one KV branch's pools and the requests that use them."""

    def __init__(self, cfg: WindowConfig):
        self.cfg = cfg
        handle = ctypes.c_void_p()
        L._check(L.lib().pkv_wm_create(ctypes.byref(cfg.c_struct()), ctypes.byref(handle)))
        self._h = handle

    def close(self) -> None:
        if self._h:
            L.lib().pkv_wm_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:  # interpreter shutdown
            pass

    def begin_request(self) -> int:
        rid = ctypes.c_int32()
        L._check(L.lib().pkv_wm_begin_request(self._h, ctypes.byref(rid)))
        return int(rid.value)

    def end_request(self, request: int) -> None:
        L._check(L.lib().pkv_wm_end_request(self._h, int(request)))

    def prepare(self, request: int, tokens: int, commit: bool, action_tokens: int = 0):
        """Slots (int64) of the forward's video tokens and of its action tokens."""
        slots = np.empty(int(tokens), dtype=np.int64)
        act = np.empty(max(int(action_tokens), 1), dtype=np.int64)
        L._check(L.lib().pkv_wm_prepare(self._h, int(request), int(tokens), int(bool(commit)), int(action_tokens),
                                        L._ptr(slots, ctypes.c_int64), L._ptr(act, ctypes.c_int64)))
        return slots, act[: int(action_tokens)]

    def window_table(self, request: int, capacity: int | None = None):
        """(table int32, kv_len, table entries looked up) of the prepared forward."""
        cap = int(capacity or (self.cfg.max_video_blocks + 64))
        table = np.empty(cap, dtype=np.int32)
        count, kv_len, reads = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        L._check(L.lib().pkv_wm_window_table(self._h, int(request), L._ptr(table, ctypes.c_int32), cap,
                                            ctypes.byref(count), ctypes.byref(kv_len), ctypes.byref(reads)))
        return table[: count.value].copy(), int(kv_len.value), int(reads.value)

    def commit(self, request: int) -> None:
        L._check(L.lib().pkv_wm_commit(self._h, int(request)))

    def info(self, request: int) -> dict:
        out = np.zeros(6, dtype=np.int64)
        L._check(L.lib().pkv_wm_info(self._h, int(request), L._ptr(out, ctypes.c_int64)))
        keys = ("num_computed_tokens", "absolute_num_computed_tokens", "compacted_tokens", "table_len",
                "free_blocks", "evicted_entries")
        return {k: int(v) for k, v in zip(keys, out)}

    def block_table(self, request: int) -> np.ndarray:
        """The storage block table, -1 for evicted blocks."""
        cap = self.info(request)["table_len"]
        out = np.empty(max(cap, 1), dtype=np.int32)
        count = ctypes.c_int32()
        L._check(L.lib().pkv_wm_block_table(self._h, int(request), L._ptr(out, ctypes.c_int32), max(cap, 1),
                                           ctypes.byref(count)))
        return out[: count.value].copy()

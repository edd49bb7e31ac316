"""Runs the oracle over a generated workload (test infrastructure only).

Turns ``workloads`` geometry + tensors into the oracle's own metadata (block
tables from the visible-window rule, slot mappings, segments), its own pools
(written with its own cast), and its float64 attention output.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import pkv_oracle as O

_NP_BITS = {O.F32: np.float32, O.BF16: np.uint16, O.FP8: np.uint8}
# Poison for slots nobody wrote: NaN in every storage format.
POISON = {O.F32: np.float32(np.nan), O.BF16: np.uint16(0x7FC0), O.FP8: np.uint8(0x7F)}


def storage_bits(t) -> np.ndarray:
    """A torch tensor (any device) as numpy storage bits."""
    import torch

    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.float32:
        return t.numpy().copy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return t.view(torch.uint8).numpy().copy()
    raise TypeError(f"unsupported dtype {t.dtype}")


@dataclass
class OracleMeta:
    tables: list[list[int]]
    kv_lens: list[int]
    positions: list[list[int]]
    hist_slots: list[np.ndarray]
    cur_slots: list[np.ndarray]
    act_slots: list[np.ndarray]
    segments: list[list[O.Segment]]
    block_table: np.ndarray  # [num_seqs, width] int32, tail-padded with block 0
    query_start_loc: np.ndarray  # [num_seqs + 1] int32
    seq_lens: np.ndarray  # [num_seqs] int32


def metadata(wl) -> OracleMeta:
    g = wl.geom
    B = g.block_size
    tables, kv_lens, positions, hist_slots, cur_slots, act_slots = [], [], [], [], [], []
    rows = []
    for b in range(g.num_seqs):
        h, q = g.history_lens[b], g.query_lens[b]
        a = g.action_lens[b] if g.action_lens else 0
        win = O.visible_window(wl.block_ids[b], h + q, g.sink_tokens[b], g.window_tokens[b], B)
        if a:
            win = O.with_action_tokens(win, wl.action_block_ids[b], a, B)
        tables.append(win.table)
        kv_lens.append(win.kv_len)
        positions.append(win.positions)
        hist_slots.append(O.slot_mapping(wl.block_ids[b], np.arange(h), B))
        cur_slots.append(O.slot_mapping(wl.block_ids[b], np.arange(h, h + q), B))
        act_slots.append(O.slot_mapping(wl.action_block_ids[b], np.arange(a), B) if a else np.zeros(0, np.int64))
        rows.append(q + a)  # the query: video chunk, then action tokens
    segs = O.segments_for_rows(g.full_spans, rows, kv_lens, g.causal_default)
    width = max(len(t) for t in tables)
    bt = np.zeros((g.num_seqs, width), dtype=np.int32)  # padding block id 0, as the pages pad
    for b, t in enumerate(tables):
        bt[b, : len(t)] = t
    qsl = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    return OracleMeta(
        tables=tables,
        kv_lens=kv_lens,
        positions=positions,
        hist_slots=hist_slots,
        cur_slots=cur_slots,
        act_slots=act_slots,
        segments=segs,
        block_table=bt,
        query_start_loc=qsl,
        seq_lens=np.asarray(kv_lens, dtype=np.int32),
    )


def empty_pool(geom) -> np.ndarray:
    shape = (geom.pool_blocks() * geom.block_size, geom.num_kv_heads, geom.head_dim)
    return np.full(shape, POISON[geom.pool_dtype], dtype=_NP_BITS[geom.pool_dtype])


def _seq_list(geom, seqs):
    return range(geom.num_seqs) if seqs is None else sorted(set(int(b) for b in seqs))


def write_history(geom, meta: OracleMeta, li, k_pool, v_pool, seqs=None) -> None:
    """Writes the history of the given sequences (all by default) into the pools."""
    src = O.F32 if geom.q_dtype == O.F32 else O.BF16
    offs = np.concatenate([[0], np.cumsum(geom.history_lens)])
    for b in _seq_list(geom, seqs):
        lo, hi = int(offs[b]), int(offs[b + 1])
        if hi == lo:
            continue
        kb, vb = storage_bits(li.k_hist[lo:hi]), storage_bits(li.v_hist[lo:hi])
        O.paged_write(k_pool, kb, meta.hist_slots[b], src, geom.pool_dtype, li.k_inv_scale)
        O.paged_write(v_pool, vb, meta.hist_slots[b], src, geom.pool_dtype, li.v_inv_scale)


def write_current(geom, meta: OracleMeta, li, k_pool, v_pool, seqs=None) -> None:
    src = O.F32 if geom.q_dtype == O.F32 else O.BF16
    offs = np.concatenate([[0], np.cumsum(geom.query_lens)])
    for b in _seq_list(geom, seqs):
        lo, hi = int(offs[b]), int(offs[b + 1])
        kb, vb = storage_bits(li.k_cur[lo:hi]), storage_bits(li.v_cur[lo:hi])
        O.paged_write(k_pool, kb, meta.cur_slots[b], src, geom.pool_dtype, li.k_inv_scale)
        O.paged_write(v_pool, vb, meta.cur_slots[b], src, geom.pool_dtype, li.v_inv_scale)


def write_actions(geom, meta: OracleMeta, li, k_pool, v_pool, seqs=None) -> None:
    """Writes the action K/V of the given sequences into their scratch blocks."""
    if not geom.action_lens:
        return
    src = O.F32 if geom.q_dtype == O.F32 else O.BF16
    offs = np.concatenate([[0], np.cumsum(geom.action_lens)])
    for b in _seq_list(geom, seqs):
        lo, hi = int(offs[b]), int(offs[b + 1])
        if hi == lo:
            continue
        kb, vb = storage_bits(li.k_act[lo:hi]), storage_bits(li.v_act[lo:hi])
        O.paged_write(k_pool, kb, meta.act_slots[b], src, geom.pool_dtype, li.k_inv_scale)
        O.paged_write(v_pool, vb, meta.act_slots[b], src, geom.pool_dtype, li.v_inv_scale)


def softmax_scale(head_dim: int) -> float:
    """head_dim^-0.5 computed in float64 and rounded once to fp32 (the value both
    sides receive)."""
    return float(np.float32(head_dim ** -0.5))


def attention(geom, meta: OracleMeta, li, k_pool, v_pool, heads=None, rows=None) -> np.ndarray:
    return O.paged_attention(
        storage_bits(li.q),
        geom.q_dtype,
        k_pool,
        v_pool,
        geom.pool_dtype,
        meta.block_table,
        meta.query_start_loc,
        meta.seq_lens,
        meta.segments,
        softmax_scale(geom.head_dim),
        geom.block_size,
        k_scale=li.k_scale,
        v_scale=li.v_scale,
        heads=heads,
        rows=rows,
    )


def run_layer(wl, layer: int = 0, heads=None, rows=None, li=None, seqs=None):
    """Full oracle pass for one layer: pools written (history, then the current
    chunk, then the action tokens) and attention over them.  Returns (meta, k_pool, v_pool, out).

    ``seqs`` restricts the pool writes to some sequences (sampled checks of
    large workloads); ``rows`` must then lie in those sequences."""
    geom = wl.geom
    li = wl.layer(layer) if li is None else li
    meta = metadata(wl)
    k_pool, v_pool = empty_pool(geom), empty_pool(geom)
    write_history(geom, meta, li, k_pool, v_pool, seqs)
    write_current(geom, meta, li, k_pool, v_pool, seqs)
    write_actions(geom, meta, li, k_pool, v_pool, seqs)
    out = attention(geom, meta, li, k_pool, v_pool, heads=heads, rows=rows)
    return meta, k_pool, v_pool, out

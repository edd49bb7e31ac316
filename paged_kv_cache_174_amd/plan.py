"""Per-forward host metadata, built once and shared by every layer.

For each sequence this asks the C library for the visible-window block table
(sink + recent window, whole blocks), the slot mappings of the history and of
the current chunk, and the piecewise segments; it then pads the table to one
width and uploads everything once (P1 ``ARDiffusionPagedForwardContext.prepare``
builds the same metadata once per KV branch for all layers).  Python only
moves arrays between the C calls and the device.
Pages cited by tag and function: P1 "vllm_omni/experimental/ar_diffusion/kv_cache/paged_attention.py",
P2 "tests/diffusion/ar_diffusion/test_paged_attention.py",
P3 "vllm_omni/diffusion/attention/backends/utils/piecewise_attn.py",
P4 "vllm_omni/diffusion/diffusion_kv/paged_attention_adapter.py".
"""

from __future__ import annotations

import weakref
from dataclasses import dataclass, field

import numpy as np
import torch

from . import _lib as L

# A fixed-capacity table wider than this many blocks (4M tokens of 16) is a
# window that does not bound the history, not a capacity.
MAX_FIXED_CAPACITY_BLOCKS = 1 << 18


@dataclass
class ForwardPlan:
    num_seqs: int
    block_size: int
    query_lens: list[int]
    history_lens: list[int]
    kv_lens: list[int]
    tables: list[np.ndarray]
    segments_host: np.ndarray  # [num_segments, 4]
    segment_start_host: np.ndarray  # [num_seqs + 1]
    block_table_host: np.ndarray  # [num_seqs, width]
    query_start_host: np.ndarray  # [num_seqs + 1]
    cur_slots_host: np.ndarray  # [sum q] int64
    hist_slots_host: np.ndarray  # [sum h] int64
    max_query_len: int
    max_seq_len: int
    # Action tokens (P1 ensure_action_slots): per sequence, rows after the
    # current video chunk in both the query and the keys.
    chunk_lens: list[int] = field(default_factory=list)  # current video tokens per sequence
    action_lens: list[int] = field(default_factory=list)
    act_slots_host: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))  # [sum a] int64
    # Full-attention spans each sequence's segments were built from (the AR
    # default resolved), kept for shard().
    spans: list = field(default_factory=list)
    # Query shards (shard()): key position of each entry's first query row,
    # and the sequence each entry reads.  None: one entry per sequence, its
    # query at the end of its keys.
    query_pos_host: np.ndarray | None = None
    entry_seq: np.ndarray | None = None
    # device copies
    block_table: torch.Tensor | None = None
    query_start_loc: torch.Tensor | None = None
    seq_lens: torch.Tensor | None = None
    segments: torch.Tensor | None = None
    segment_start_loc: torch.Tensor | None = None
    seq_order: torch.Tensor | None = None
    slot_mapping: torch.Tensor | None = None
    history_slot_mapping: torch.Tensor | None = None
    action_slot_mapping: torch.Tensor | None = None
    query_pos: torch.Tensor | None = None

    @classmethod
    def build(
        cls,
        block_ids,
        history_lens,
        query_lens,
        sink_tokens,
        window_tokens,
        full_spans,
        causal_default: bool = False,
        block_size: int = 16,
        table_width: int | None = None,
        max_seq_len: int | None = None,
        device=None,
        action_lens=None,
        action_block_ids=None,
        fixed_capacity: bool = False,
    ) -> "ForwardPlan":
        """``query_lens`` are the current video chunks.  With ``action_lens``
        (per sequence) and ``action_block_ids`` (each sequence's scratch
        blocks), the action K/V is listed after the window and the query of a
        sequence is its video chunk followed by its action tokens (P1
        build_block_table, P2 action tests).

        ``fixed_capacity`` sizes the metadata as P1 ``build_block_table`` does:
        the table width is the window's capacity in blocks (pkv_window_capacity:
        sink and recent range rounded separately, plus the action scratch) and
        ``max_seq_len`` that capacity in tokens, so both stay constant while the
        window fills; the real lengths go to the library as its planning hint
        (``kv_lens``).  Otherwise the width is the longest table and
        ``max_seq_len`` the longest sequence."""
        n = len(query_lens)
        acts = [0] * n if action_lens is None else [int(a) for a in action_lens]
        tables, kv_lens, segs, seg_start = [], [], [], [0]
        cur_slots, hist_slots, act_slots, used_spans = [], [], [], []
        for b in range(n):
            h, q, a = int(history_lens[b]), int(query_lens[b]), acts[b]
            table, kv_len = L.pkv_window_table(block_ids[b], h, q, sink_tokens[b], window_tokens[b], block_size)
            if a:
                table, kv_len = L.pkv_action_table(table, kv_len, action_block_ids[b], a, block_size)
                act_slots.append(L.pkv_slot_mapping(action_block_ids[b], 0, a, block_size))
            tables.append(table)
            kv_lens.append(kv_len)
            hist_slots.append(L.pkv_slot_mapping(block_ids[b], 0, h, block_size))
            cur_slots.append(L.pkv_slot_mapping(block_ids[b], h, q, block_size))
            rows = q + a  # the query is the suffix of the keys: video chunk, then actions
            spans = full_spans[b]
            if spans is None:
                spans = [] if causal_default else [(kv_len - rows, kv_len)]
            used_spans.append([(int(a_), int(b_)) for a_, b_ in spans])
            sg = L.pkv_build_segments(list(spans), kv_len - rows, rows)
            segs.append(sg)
            seg_start.append(seg_start[-1] + len(sg))
        rows_per_seq = [int(q) + a for q, a in zip(query_lens, acts)]
        if fixed_capacity:
            caps = [L.pkv_window_capacity(sink_tokens[b], window_tokens[b], query_lens[b], block_size, acts[b])
                    for b in range(n)]
            if max(caps) > MAX_FIXED_CAPACITY_BLOCKS:
                raise ValueError(
                    f"fixed_capacity needs a bounded window: sequence {int(np.argmax(caps))} would take a "
                    f"{max(caps)}-entry table (at most {MAX_FIXED_CAPACITY_BLOCKS})")
            width = max(max(caps), max(len(t) for t in tables))
            if table_width is None:
                table_width = width
            if max_seq_len is None:
                max_seq_len = max(caps) * block_size
        width = max(len(t) for t in tables) if table_width is None else int(table_width)
        bt = np.zeros((n, width), dtype=np.int32)  # tail padding with block 0, never read
        for b, t in enumerate(tables):
            if len(t) > width:
                raise ValueError(f"sequence {b} needs {len(t)} table entries, width is {width}")
            bt[b, : len(t)] = t
        qsl = np.concatenate([[0], np.cumsum(rows_per_seq)]).astype(np.int32)
        plan = cls(
            num_seqs=n,
            block_size=block_size,
            query_lens=rows_per_seq,
            history_lens=[int(h) for h in history_lens],
            kv_lens=kv_lens,
            tables=tables,
            segments_host=np.concatenate(segs).astype(np.int32),
            segment_start_host=np.asarray(seg_start, dtype=np.int32),
            block_table_host=bt,
            query_start_host=qsl,
            cur_slots_host=np.concatenate(cur_slots).astype(np.int64),
            hist_slots_host=np.concatenate(hist_slots).astype(np.int64) if hist_slots else np.zeros(0, np.int64),
            max_query_len=int(max(rows_per_seq)),
            max_seq_len=int(max(kv_lens) if max_seq_len is None else max_seq_len),
            chunk_lens=[int(q) for q in query_lens],
            action_lens=acts,
            act_slots_host=np.concatenate(act_slots).astype(np.int64) if act_slots else np.zeros(0, np.int64),
            spans=used_spans,
        )
        if device is not None:
            plan.to(device)
        return plan

    def to(self, device) -> "ForwardPlan":
        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(device)

        self.block_table = up(self.block_table_host)
        self.query_start_loc = up(self.query_start_host)
        self.seq_lens = up(np.asarray(self.kv_lens, dtype=np.int32))
        self.segments = up(self.segments_host.reshape(-1))
        self.segment_start_loc = up(self.segment_start_host)
        self.seq_order = up(self.seq_order_host)
        self.slot_mapping = up(self.cur_slots_host)
        self.history_slot_mapping = up(self.hist_slots_host)
        self.action_slot_mapping = up(self.act_slots_host)
        self.query_pos = None if self.query_pos_host is None else up(self.query_pos_host)
        return self

    def shard(self, query_ranges, device=None) -> "ForwardPlan":
        """Attention metadata for local query shards (P3 ``piecewise_attn``
        with ``query_ranges``): ``query_ranges[b]`` lists ``(local_start,
        local_end, global_start)`` triples covering sequence b's local query
        rows in order from 0; each range becomes one attention entry over
        sequence b's keys with its rows at key positions ``[global_start,
        global_start + local_end - local_start)``, its segments cut from the
        sequence's full spans at that start (a full segment keeps its span's
        end, so a shard's rows attend past the shard).  The write metadata
        (slot mappings) is the original plan's."""
        if len(query_ranges) != self.num_seqs or self.entry_seq is not None:
            raise ValueError("shard() takes one list of ranges per sequence of an unsharded plan")
        tables, kv_lens, rows, qpos, entry, segs, seg_start = [], [], [], [], [], [], [0]
        for b, ranges in enumerate(query_ranges):
            covered = 0
            for local_start, local_end, global_start in ranges:
                n = int(local_end) - int(local_start)
                if int(local_start) != covered or n < 0:
                    raise ValueError("query_ranges must cover local query contiguously")
                covered = int(local_end)
                if n == 0:
                    continue
                if int(global_start) < 0 or int(global_start) + n > self.kv_lens[b]:
                    raise ValueError(f"sequence {b}: rows [{global_start}, {int(global_start) + n}) lie outside "
                                     f"its {self.kv_lens[b]} keys")
                sg = L.pkv_build_segments(self.spans[b], int(global_start), n)
                tables.append(self.tables[b])
                kv_lens.append(self.kv_lens[b])
                rows.append(n)
                qpos.append(int(global_start))
                entry.append(b)
                segs.append(sg)
                seg_start.append(seg_start[-1] + len(sg))
        if not rows:
            raise ValueError("the shards hold no query rows")
        bt = np.zeros((len(rows), self.block_table_host.shape[1]), dtype=np.int32)
        for e, b in enumerate(entry):
            bt[e] = self.block_table_host[b]
        out = ForwardPlan(
            num_seqs=len(rows),
            block_size=self.block_size,
            query_lens=rows,
            history_lens=self.history_lens,
            kv_lens=kv_lens,
            tables=tables,
            segments_host=np.concatenate(segs).astype(np.int32),
            segment_start_host=np.asarray(seg_start, dtype=np.int32),
            block_table_host=bt,
            query_start_host=np.concatenate([[0], np.cumsum(rows)]).astype(np.int32),
            cur_slots_host=self.cur_slots_host,
            hist_slots_host=self.hist_slots_host,
            max_query_len=int(max(rows)),
            max_seq_len=self.max_seq_len,
            chunk_lens=self.chunk_lens,
            action_lens=self.action_lens,
            act_slots_host=self.act_slots_host,
            spans=self.spans,
            query_pos_host=np.asarray(qpos, dtype=np.int32),
            entry_seq=np.asarray(entry, dtype=np.int32),
        )
        if device is not None:
            out.to(device)
        return out

    @property
    def seq_order_host(self) -> np.ndarray:
        """Dispatch order for the attention kernel: longest sequence first
        (ties in index order), so that short sequences fill in behind long ones."""
        return np.argsort(-np.asarray(self.kv_lens, dtype=np.int64), kind="stable").astype(np.int32)

    def validate(self, num_blocks: int) -> None:
        order = self.seq_order_host
        if sorted(order.tolist()) != list(range(self.num_seqs)):
            raise ValueError("seq_order is not a permutation of the sequences")
        L.pkv_validate_metadata_host(
            self.query_start_host,
            np.asarray(self.kv_lens, dtype=np.int32),
            self.block_table_host,
            num_blocks,
            self.block_size,
            self.max_query_len,
            self.max_seq_len,
            self.segments_host,
            self.segment_start_host,
            self.query_pos_host,
        )

    def attn_flops(self, num_q_heads: int, head_dim: int) -> float:
        """Algorithmic FLOPs of one attention call: 4 * D * Hq * (visible
        query-key pairs), counting each multiply-add of QK^T and PV as 2."""
        pairs = 0
        for b in range(self.num_seqs):
            lo, hi = self.segment_start_host[b], self.segment_start_host[b + 1]
            for qs, qe, kv, mode in self.segments_host[lo:hi]:
                if mode == L.PKV_SEG_FULL:
                    pairs += int(qe - qs) * int(kv)
                else:  # rows g in [qs, qe) see g + 1 keys
                    pairs += int((qs + 1 + qe) * (qe - qs) // 2)
        return 4.0 * head_dim * num_q_heads * pairs


@dataclass(frozen=True)
class StagingDecision:
    """Whether a forward stages its window, and from which block row on."""

    enabled: bool
    reuse: bool
    first_block: int


class HistoryStaging:
    """Reuse state of one KV branch's staging buffers (P1
    ``_prepare_history_staging``); the decision itself is the C library's
    ``pkv_staging_decide``.

    A forward keeps the staged history when the buffers were last filled for
    the same session (compared by identity) and its history, extent and chunk
    length are unchanged, and the chunk fills whole blocks from a block edge;
    then only the chunk's blocks are gathered again, from the visible
    history's block count on.  Otherwise ``first_block`` is 0: everything is
    restaged.  The decision is a host value, the same for all layers of a
    forward.  One sequence and no action tokens only.
    """

    def __init__(self, capacity_tokens: int):
        self.capacity_tokens = int(capacity_tokens)
        self._session = None  # weak reference to the session staged last
        self._session_id = -1
        self._next_id = 0
        self._state = None
        self._block_size = None

    def _id_of(self, session) -> int:
        last = self._session() if self._session is not None else None
        if last is None or last is not session:
            self._session_id, self._next_id = self._next_id, self._next_id + 1
            try:
                self._session = weakref.ref(session)
            except TypeError:  # not weakly referenceable: keep it alive instead
                self._session = (lambda s: (lambda: s))(session)
        return self._session_id

    def decide(self, session, plan: ForwardPlan) -> StagingDecision:
        """``session`` identifies the request (compared by identity)."""
        if plan.num_seqs != 1 or any(plan.action_lens):
            return StagingDecision(False, False, 0)
        B = plan.block_size
        if self._state is None or self._block_size != B:
            self._state = L.StagingState(self.capacity_tokens // B + 1)
            self._block_size = B
        reuse, first = L.pkv_staging_decide(
            self._state, self._id_of(session), plan.tables[0], plan.history_lens[0], plan.chunk_lens[0],
            plan.max_seq_len, B, self.capacity_tokens,
        )
        return StagingDecision(True, reuse, first)

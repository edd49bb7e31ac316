"""Float64 reference for AR-diffusion paged self-attention (test infrastructure only).

Storage convention: pools and activations are handled as their raw storage
bits -- ``uint16`` for bfloat16, ``uint8`` for OCP float8 e4m3fn and
``float32`` for fp32 -- so that a bit-exact comparison against device memory
is a plain ``array_equal``.  All arithmetic on values is float64.

Page tags used in the citations:
  P1 = vllm_omni/experimental/ar_diffusion/kv_cache/paged_attention.py
  P2 = tests/diffusion/ar_diffusion/test_paged_attention.py
  P3 = vllm_omni/diffusion/attention/backends/utils/piecewise_attn.py
  P4 = vllm_omni/diffusion/diffusion_kv/paged_attention_adapter.py
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "F32",
    "BF16",
    "FP8",
    "bf16_bits_to_f64",
    "e4m3_code_values",
    "e4m3_decode",
    "e4m3_encode",
    "decode_storage",
    "encode_for_pool",
    "slot_mapping",
    "WindowRead",
    "visible_window",
    "with_action_tokens",
    "WindowModel",
    "StagingState",
    "staging_decision",
    "Segment",
    "build_segments",
    "segments_for_rows",
    "row_limits",
    "paged_write",
    "gather",
    "kernel_view",
    "paged_attention",
    "piecewise_attention",
    "dense_attention",
    "attention_bruteforce",
]

F32, BF16, FP8 = "f32", "bf16", "fp8"

# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the upper half of an IEEE binary32: shift the 16 bits into place."""
    wide = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return wide.view(np.float32).astype(np.float64)


def _e4m3_code_value(code: int) -> float:
    """Value of one OCP float8 e4m3fn code, from the format definition.

    One sign bit, four exponent bits with bias 7, three mantissa bits.  A zero
    exponent field encodes subnormals m/8 * 2^(1-7); exponent 15 with mantissa 7
    is NaN (the format has no infinities); everything else is normal
    (1 + m/8) * 2^(e-7).  The largest finite magnitude is 1.75 * 2^8 = 448.
    """
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3_TABLE = np.array([_e4m3_code_value(c) for c in range(256)], dtype=np.float64)
# Codes 0x00..0x7E are the non-negative finite values, in increasing order.
_E4M3_POS = _E4M3_TABLE[:0x7F].copy()
E4M3_MAX = 448.0


def e4m3_code_values() -> np.ndarray:
    """All 256 code values (float64, NaN for the two NaN codes)."""
    return _E4M3_TABLE.copy()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return _E4M3_TABLE[np.asarray(codes).astype(np.uint8)]


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round float64 values to e4m3fn codes: nearest value, ties to the even code,
    saturating at +-448, sign of zero kept, NaN to the NaN code.

    The rounding is done by search over the code table, not by bit tricks, so
    it follows the definition directly: of the two representable magnitudes
    around |x|, take the nearer; on an exact tie take the one whose code is
    even (mantissa LSB 0).  Magnitudes above 448 clamp to 448.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    a = np.abs(x)
    nan = np.isnan(x)
    a_clamped = np.minimum(np.where(nan, 0.0, a), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, a_clamped, side="left")  # first code with value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    v_hi = _E4M3_POS[hi]
    v_lo = _E4M3_POS[lo]
    d_hi = v_hi - a_clamped
    d_lo = a_clamped - v_lo
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(a_clamped == v_hi, hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    sign = np.signbit(x).astype(np.uint8) << np.uint8(7)
    out[...] = code | sign
    out[nan] = 0x7F | (np.signbit(x[nan]).astype(np.uint8) << np.uint8(7))
    return out


def decode_storage(bits: np.ndarray, dtype: str, scale: float = 1.0) -> np.ndarray:
    """Storage bits -> float64 values.  fp8 values are multiplied by their
    per-tensor dequantisation scale exactly (float64 holds the product)."""
    if dtype == F32:
        return np.asarray(bits, dtype=np.float32).astype(np.float64)
    if dtype == BF16:
        return bf16_bits_to_f64(bits)
    if dtype == FP8:
        return e4m3_decode(bits) * float(scale)
    raise ValueError(f"unknown dtype {dtype!r}")


def encode_for_pool(src_bits: np.ndarray, src_dtype: str, pool_dtype: str, inv_scale: float = 1.0) -> np.ndarray:
    """The cast a pool write applies (P1 ``_paged_write_attn_impl``: the source is
    converted to the pool's dtype before the scatter).

    Same dtype: the bits are copied unchanged.  bf16 -> fp8: the bf16 value is
    widened to fp32, multiplied by the fp32 quantisation multiplier with one
    round-to-nearest-even to fp32, then rounded to e4m3 (``e4m3_encode``).
    The float64 product of two fp32 numbers is exact, so casting it to float32
    is that single fp32 rounding.
    """
    if src_dtype == pool_dtype:
        return np.array(src_bits, copy=True)
    if src_dtype == BF16 and pool_dtype == FP8:
        x = bf16_bits_to_f64(src_bits) * float(np.float32(inv_scale))
        with np.errstate(over="ignore", invalid="ignore"):
            x32 = x.astype(np.float32).astype(np.float64)  # an fp32 overflow is inf, which saturates
        return e4m3_encode(x32)
    raise ValueError(f"unsupported cast {src_dtype} -> {pool_dtype}")


# ---------------------------------------------------------------------------
# Host metadata: slot mapping, visible window, segments
# ---------------------------------------------------------------------------


def slot_mapping(block_ids, positions, block_size: int) -> np.ndarray:
    """Physical slot of each token position (P1 ``_reference_paged_attention`` and
    ``ensure_video_slots``): the block listed for ``position // block_size``,
    times the block size, plus ``position % block_size``."""
    ids = np.asarray(block_ids, dtype=np.int64)
    pos = np.asarray(positions, dtype=np.int64)
    return ids[pos // block_size] * block_size + pos % block_size


@dataclass
class WindowRead:
    table: list[int]  # physical block ids, in the order the kernel reads them
    kv_len: int  # tokens the kernel reads from that run of blocks
    positions: list[int]  # model position held by each token read, in order


def visible_window(
    block_ids, end: int, sink_tokens: int, window_tokens: int, block_size: int
) -> WindowRead:
    """Blocks attention reads for a sink + sliding window, and how many tokens.

    Restates the visible-window rule of P1 ``video_block_table`` in the
    set-of-positions form that P2's ``_window_positions`` helper states it:

    * positions ``[0, end)`` have been written; ``block_ids[i]`` holds positions
      ``[i*B, (i+1)*B)``, or is negative when that block is no longer resident;
    * the window keeps the sink ``[0, min(S, end))`` and the most recent
      ``window_tokens`` positions ``[max(end - W, 0), end)`` (P1: the recent
      range counts the current chunk);
    * every resident block that holds a kept position is read *whole* -- all of
      its written positions, including ones the window has let go of -- in
      position order;
    * the kernel reads the listed blocks as one run, so only the last one may be
      partly written (P1 raises ``RuntimeError`` otherwise).
    """
    B = int(block_size)
    if end <= 0:
        raise ValueError("the window needs at least one written token")
    kept = {p // B for p in range(min(sink_tokens, end))}
    kept |= {p // B for p in range(max(end - window_tokens, 0), end)}
    ids = list(block_ids)
    order = sorted(i for i in kept if i < len(ids) and ids[i] >= 0)
    table: list[int] = []
    positions: list[int] = []
    for n, i in enumerate(order):
        first = i * B
        count = min(B, end - first)
        if n + 1 < len(order) and count < B:
            raise RuntimeError(f"block {ids[i]} is partly written but another block follows it")
        table.append(int(ids[i]))
        positions.extend(range(first, first + count))
    return WindowRead(table=table, kv_len=len(positions), positions=positions)


def with_action_tokens(window: WindowRead, action_block_ids, action_len: int, block_size: int) -> WindowRead:
    """Action K/V after the video window (P1 ``build_block_table`` with
    ``ensure_action_slots``; P2's dense reference appends the action K/V to
    the windowed video K/V).

    The ``action_len`` action tokens occupy positions ``[0, action_len)`` of
    their own scratch blocks.  Those blocks are listed after the video blocks
    and the run grows by ``action_len`` tokens.  The kernel reads the list as
    one run, so a video run that stops inside a block would have its unwritten
    slots read as action tokens: P1 raises ``ValueError`` for it.  Action
    tokens get the position labels ``-1, -2, ...`` in the returned window.
    """
    a = int(action_len)
    if a <= 0:
        return window
    B = int(block_size)
    if window.kv_len % B:
        raise ValueError("action tokens cannot follow a partly written video block")
    needed = (a + B - 1) // B
    ids = [int(x) for x in action_block_ids]
    if len(ids) < needed:
        raise ValueError("too few action scratch blocks")
    return WindowRead(
        table=list(window.table) + ids[:needed],
        kv_len=window.kv_len + a,
        positions=list(window.positions) + [-(1 + i) for i in range(a)],
    )


class WindowModel:
    """Which tokens a request keeps, in model positions only (no physical
    blocks, no compaction): the rules the pages' eviction and reset tests
    state (P2 ``test_attention_after_eviction_reads_every_kept_token_and_nothing_unwritten``,
    ``test_compaction_does_not_change_which_tokens_stay_resident``; P1
    ``video_block_table``), taken as this model:

    * the sink is the first ``sink_chunks`` chunks, the recent window the last
      ``window_chunks`` chunks including the current one;
    * after a commit that ends at E, no later window starts before E - W, so
      the whole chunks before that point, past the sink, are dead; with
      ``reset_at_boundary``, a commit completing ``chunks_per_block`` chunks
      kills everything past the sink;
    * a block stays while any token written in it is alive, and a partly
      written last block stays in any case (the next chunk continues it);
    * a forward reads the visible window (``visible_window``) over the blocks
      that stay plus the blocks its own tokens occupy.
    """

    def __init__(self, block_size: int, chunk_size: int, sink_chunks: int, window_chunks: int,
                 reset_at_boundary: bool = False, chunks_per_block: int = 1):
        self.B, self.C = int(block_size), int(chunk_size)
        self.S = int(sink_chunks) * self.C
        self.W = int(window_chunks) * self.C
        self.reset = bool(reset_at_boundary)
        self.per_block = int(chunks_per_block)
        self.end = 0  # committed tokens
        self.chunks = 0
        self.kept = set()  # model block indices that stay

    def window(self, tokens: int, action_tokens: int = 0) -> WindowRead:
        """Positions a forward of ``tokens`` tokens after the history reads,
        then its action tokens (labelled -1, -2, ...)."""
        B = self.B
        end = self.end + int(tokens)
        ids = [k if (k in self.kept or (k + 1) * B > self.end) else -1 for k in range(-(-end // B))]
        win = visible_window(ids, end, self.S, self.W, B)
        if action_tokens:
            win = with_action_tokens(win, list(range(10**6, 10**6 + -(-int(action_tokens) // B))), action_tokens, B)
        return win

    def commit(self, tokens: int) -> None:
        B, C = self.B, self.C
        start = self.end
        self.end += int(tokens)
        self.chunks += int(tokens) // C
        self.kept |= set(range(start // B, -(-self.end // B)))
        if self.reset and self.chunks % self.per_block == 0:
            dead_end = self.end
        else:
            dead_end = max(self.end - self.W, 0) // C * C
        tail = (self.end - 1) // B if self.end % B else None
        for k in sorted(self.kept):
            first, last = k * B, min((k + 1) * B, self.end)
            if first >= self.S and last <= dead_end and k != tail:
                self.kept.discard(k)


@dataclass
class StagingState:
    """What the staging buffers of one KV branch last held (P1
    ``history_staging_state``): the session and the window signature."""

    session: object = None
    signature: tuple | None = None


def staging_decision(
    state: StagingState,
    session,
    *,
    num_seqs: int,
    action_len: int,
    capacity_tokens: int,
    history_tokens: int,
    window: WindowRead,
    max_seq_len: int,
    chunk_tokens: int,
    block_size: int,
) -> tuple[bool, bool, int]:
    """P1 ``_prepare_history_staging``: (staging enabled, reuse the staged
    history, first block row to gather).

    * Staging covers one sequence without action tokens; otherwise it is off
      and the state is left alone.
    * A window longer than the buffers is an error (``RuntimeError``).
    * The staged history is reused when the session is the same object as last
      time, the signature (history length, the visible history's blocks,
      ``max_seq_len``, chunk length) is unchanged, and the chunk starts on a
      block edge and is whole blocks.  The state then records this forward.
    * The blocks to refresh start after the visible history: the window's
      block count minus the blocks the current chunk touches (counted from its
      offset inside its first block).

    The visible history's blocks are read off the window: a table entry is
    history when its first position lies in a block that ends at or before
    the chunk's first block.
    """
    if action_len or num_seqs != 1:
        return False, False, 0
    if max_seq_len > capacity_tokens:
        raise RuntimeError("the history staging buffers are smaller than the window")
    B = int(block_size)
    firsts, seen = [], set()
    for pos in window.positions:  # first position of every listed block, in order
        blk = pos // B
        if pos >= 0 and blk not in seen:
            seen.add(blk)
            firsts.append(pos)
    chunk_first_block = int(history_tokens) // B
    history_ids = tuple(int(window.table[n]) for n, pos in enumerate(firsts) if pos // B < chunk_first_block)
    signature = (int(history_tokens), history_ids, int(max_seq_len), int(chunk_tokens))
    offset = int(history_tokens) % B
    aligned = offset == 0 and int(chunk_tokens) % B == 0
    reuse = state.session is not None and state.session is session and state.signature == signature and aligned
    state.session = session
    state.signature = signature
    touched = -(-(offset + int(chunk_tokens)) // B)
    # without reuse the whole window is staged again: from block row 0
    return True, bool(reuse), window.kv_len // B - touched if reuse else 0


@dataclass(frozen=True)
class Segment:
    """One run of query rows with one masking rule (P3 ``Segment``), in the
    key (global) coordinates of the sequence."""

    q_start: int
    q_end: int
    kv_end: int
    mode: str  # "causal" or "full"


def build_segments(full_spans, query_offset: int, query_len: int) -> list[Segment]:
    """P3 ``build_segments``, from the rule of P3's module docstring: rows of
    the query range ``[o, o + n)`` that lie in a full span ``[a, b)`` attend
    ``K[:b]`` with no mask (``b`` is the span's own end, even where the query
    stops inside the span); the other rows are cut into causal segments
    ``[s, e)`` that attend ``K[:e]`` aligned at the bottom-right corner, so
    their ``kv_end`` is ``e``.

    Written row by row: each row gets its rule -- the end of the span holding
    it, or none -- and consecutive rows with the same rule form one segment.
    The spans are sorted and disjoint (P3 ``build_paged_piecewise_plan``
    refuses anything else).
    """
    lo, hi = int(query_offset), int(query_offset) + int(query_len)
    spans = [(int(a), int(b)) for a, b in full_spans]
    if any(b0 > a1 for (_, b0), (a1, _) in zip(spans, spans[1:])):
        raise ValueError("full spans must be sorted and disjoint")

    def span_end(g):
        for a, b in spans:
            if a <= g < b:
                return b
        return None

    runs: list[list] = []  # [first row, end row, span end or None]
    for g in range(lo, hi):
        rule = span_end(g)
        if runs and runs[-1][2] == rule:
            runs[-1][1] = g + 1
        else:
            runs.append([g, g + 1, rule])
    return [Segment(s, e, r, "full") if r is not None else Segment(s, e, e, "causal") for s, e, r in runs]


def segments_for_rows(full_spans_per_seq, query_lens, seq_lens, causal_default: bool = False):
    """Segments of every sequence for suffix queries.

    The query is the suffix of its sequence: its first row sits at key position
    ``seq_len - query_len`` (P3 ``piecewise_attn`` takes ``Sk - Sq`` as the
    query's global start; P4 refuses causal or piecewise rows that do not end
    at ``seq_len``).  ``full_spans_per_seq[b] is None`` means the AR default of
    P1 (``causal=False``): one full run over the whole query with
    ``kv_end = seq_len``.  With ``causal_default`` and no spans, the whole query
    is one causal run.
    """
    out = []
    for spans, q, s in zip(full_spans_per_seq, query_lens, seq_lens):
        if spans is None:
            spans = [] if causal_default else [(s - q, s)]
        out.append(build_segments(spans, s - q, q))
    return out


def row_limits(segments: list[Segment], seq_len: int, query_len: int) -> np.ndarray:
    """Exclusive key bound L(g) of each query row g = seq_len - query_len + i.

    P3's module docstring fixes FlashAttention's bottom-right convention: a
    causal run ``[s, e)`` attends ``K[:e]`` causally, so row g sees keys j <= g,
    i.e. L(g) = g + 1; a full run attends ``K[:kv_end]`` without a mask, so
    L(g) = kv_end.  P4 builds one native call per run with ``seq_lens =
    kv_end``, which is the same key-prefix limit.
    """
    limits = np.full(query_len, -1, dtype=np.int64)
    g0 = seq_len - query_len
    for seg in segments:
        for g in range(seg.q_start, seg.q_end):
            i = g - g0
            if not 0 <= i < query_len:
                raise ValueError("segment outside the query range")
            limits[i] = seg.kv_end if seg.mode == "full" else g + 1
    if (limits < 0).any():
        raise ValueError("segments do not cover the query")
    return limits


# ---------------------------------------------------------------------------
# Write and gather
# ---------------------------------------------------------------------------


def paged_write(pool: np.ndarray, src: np.ndarray, slots, src_dtype: str, pool_dtype: str, inv_scale=1.0) -> None:
    """Scatter ``src[t]`` (a ``[H_kv, D]`` row) into ``pool[slots[t]]`` after the
    pool cast (P1 ``_paged_write_attn_impl``: the pool indexed by the slot
    mapping is assigned the converted current K/V).  In place."""
    slots = np.asarray(slots, dtype=np.int64)
    if len(np.unique(slots)) != len(slots):
        raise ValueError("slot mapping has duplicate slots")
    pool[slots] = encode_for_pool(src, src_dtype, pool_dtype, inv_scale)


def gather(pool: np.ndarray, block_ids, n_blocks: int, first_block: int, stage: np.ndarray, block_size: int) -> None:
    """History staging (P1 ``_stage_window``): the staging buffer, seen as
    ``[n_blocks, B, ...]``, receives block ``block_ids[i]`` of the pool at row
    ``i`` for every ``first_block <= i < n_blocks``; other rows keep their
    contents.  In place."""
    B = int(block_size)
    for i in range(int(first_block), int(n_blocks)):
        b = int(block_ids[i])
        stage[i * B : (i + 1) * B] = pool[b * B : (b + 1) * B]


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------


def kernel_view(pool: np.ndarray, table_row, seq_len: int, block_size: int, dtype: str, scale=1.0) -> np.ndarray:
    """The key (or value) sequence one row of the block table describes (P1
    ``_reference_paged_attention``): token j comes from slot
    ``table[j // B] * B + j % B``; only ``seq_len`` tokens are read, so table
    entries past ``ceil(seq_len / B)`` are never touched.  Returns float64."""
    j = np.arange(int(seq_len), dtype=np.int64)
    slots = slot_mapping(np.asarray(table_row, dtype=np.int64), j, block_size)
    return decode_storage(pool[slots], dtype, scale)


def _softmax_attend(qh: np.ndarray, k: np.ndarray, v: np.ndarray, limits: np.ndarray, scale: float) -> np.ndarray:
    """Masked softmax attention for one head: row i sees keys j < limits[i]."""
    out = np.empty((qh.shape[0], v.shape[1]), dtype=np.float64)
    step = 256
    for r0 in range(0, qh.shape[0], step):
        r1 = min(r0 + step, qh.shape[0])
        z = (qh[r0:r1] @ k.T) * scale
        mask = np.arange(k.shape[0])[None, :] >= limits[r0:r1, None]
        z[mask] = -np.inf
        z -= z.max(axis=1, keepdims=True)
        p = np.exp(z)
        p /= p.sum(axis=1, keepdims=True)
        out[r0:r1] = p @ v
    return out


def paged_attention(
    q: np.ndarray,
    q_dtype: str,
    k_pool: np.ndarray,
    v_pool: np.ndarray,
    pool_dtype: str,
    block_table: np.ndarray,
    query_start_loc,
    seq_lens,
    segments,
    softmax_scale: float,
    block_size: int,
    k_scale: float = 1.0,
    v_scale: float = 1.0,
    heads=None,
    rows=None,
) -> np.ndarray:
    """Varlen paged attention, float64 throughout.

    For sequence b with query rows ``q[qsl[b]:qsl[b+1]]`` and ``seq_lens[b]``
    visible keys: the keys and values are the kernel view of the pools through
    ``block_table[b]``; query head h uses KV head ``h // (Hq // Hkv)``; row i
    (key position g = s - q + i) sees keys ``j < L(g)`` from its segment;
    ``O = softmax(scale * q k^T) v`` (P1 ``_reference_paged_attention``, with the
    P3 mask).  No intermediate rounding: the pages cast probabilities to the
    value dtype before the product, which the comparison tolerance absorbs.

    ``heads`` / ``rows`` (global token indices) restrict the computation to a
    sample; the result is then ``[len(rows), len(heads), D]``.
    """
    qf = decode_storage(q, q_dtype)
    T, Hq, D = qf.shape
    Hkv = k_pool.shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    group = Hq // Hkv
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    sl = np.asarray(seq_lens, dtype=np.int64)
    heads = list(range(Hq)) if heads is None else list(heads)
    want_rows = None if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((T if want_rows is None else len(want_rows), len(heads), D), dtype=np.float64)
    for b in range(len(sl)):
        t0, t1 = int(qsl[b]), int(qsl[b + 1])
        s = int(sl[b])
        ql = t1 - t0
        if want_rows is None:
            local = np.arange(ql)
            dest = np.arange(t0, t1)
        else:
            sel = (want_rows >= t0) & (want_rows < t1)
            if not sel.any():
                continue
            local = want_rows[sel] - t0
            dest = np.nonzero(sel)[0]
        limits = row_limits(segments[b], s, ql)[local]
        k_all = kernel_view(k_pool, block_table[b], s, block_size, pool_dtype, k_scale)
        v_all = kernel_view(v_pool, block_table[b], s, block_size, pool_dtype, v_scale)
        for hi, h in enumerate(heads):
            hk = h // group
            out[dest, hi] = _softmax_attend(qf[t0 + local, h], k_all[:, hk], v_all[:, hk], limits, float(softmax_scale))
    return out


def piecewise_attention(q_f64: np.ndarray, k_f64: np.ndarray, v_f64: np.ndarray, full_spans, scale: float,
                        query_ranges=None) -> np.ndarray:
    """P3 ``piecewise_attn`` for one sequence, float64.

    ``q_f64`` is the local query ``[rows, Hq, D]``; ``k_f64`` / ``v_f64`` the
    whole key sequence ``[S, Hkv, D]``; ``full_spans`` the full-attention spans
    in key coordinates.  ``query_ranges`` lists ``(local_start, local_end,
    global_start)`` triples that must cover the local rows in order (P3 raises
    ``ValueError`` otherwise); without it the query is the suffix of the keys.
    Each range is cut into segments by ``build_segments`` at its own global
    start, and each segment is one attention call as P3 dispatches it: a
    causal segment ``[s, e)`` attends ``K[:e]`` with the bottom-right causal
    mask (row at position g sees keys ``j <= g``), a full segment attends
    ``K[:kv_end]`` unmasked -- ``kv_end`` being the unclipped span end, so a
    shard's full rows see keys past the shard's own end.  GQA maps query head
    h to KV head ``h // (Hq // Hkv)``.
    """
    rows, Hq, D = q_f64.shape
    Hkv = k_f64.shape[1]
    group = Hq // Hkv
    if query_ranges is None:
        query_ranges = [(0, rows, k_f64.shape[0] - rows)]
    out = np.zeros((rows, Hq, D), dtype=np.float64)
    covered = 0
    for local_start, local_end, global_start in query_ranges:
        n = int(local_end) - int(local_start)
        if int(local_start) != covered or n < 0:
            raise ValueError("query_ranges must cover local query contiguously")
        for seg in build_segments(full_spans, int(global_start), n):
            lo = int(local_start) + seg.q_start - int(global_start)
            hi = int(local_start) + seg.q_end - int(global_start)
            keys = seg.kv_end
            for h in range(Hq):
                z = (q_f64[lo:hi, h] @ k_f64[:keys, h // group].T) * scale
                if seg.mode == "causal":
                    g = np.arange(seg.q_start, seg.q_end)[:, None]
                    z = np.where(np.arange(keys)[None, :] <= g, z, -np.inf)
                z = z - z.max(axis=1, keepdims=True)
                p = np.exp(z)
                out[lo:hi, h] = (p / p.sum(axis=1, keepdims=True)) @ v_f64[:keys, h // group]
        covered = int(local_end)
    if covered != rows:
        raise ValueError("query_ranges must cover the full local query")
    return out


def dense_attention(q_f64: np.ndarray, k_f64: np.ndarray, v_f64: np.ndarray, limits: np.ndarray, scale: float):
    """Dense masked attention for one sequence on already-decoded contiguous
    K/V ``[s, Hkv, D]`` (P2 ``_dense_attention``, with a key-prefix limit per
    row).  Returns ``[q, Hq, D]``."""
    q_len, Hq, D = q_f64.shape
    Hkv = k_f64.shape[1]
    group = Hq // Hkv
    out = np.empty((q_len, Hq, D), dtype=np.float64)
    for h in range(Hq):
        out[:, h] = _softmax_attend(q_f64[:, h], k_f64[:, h // group], v_f64[:, h // group], limits, scale)
    return out


def attention_bruteforce(q_f64, k_f64, v_f64, limits, scale):
    """Scalar loops with ``math.exp`` -- for tiny cases only.  Same contract as
    ``dense_attention``."""
    q_len, Hq, D = q_f64.shape
    Hkv = k_f64.shape[1]
    group = Hq // Hkv
    out = np.zeros((q_len, Hq, D), dtype=np.float64)
    for i in range(q_len):
        for h in range(Hq):
            hk = h // group
            logits = []
            for j in range(int(limits[i])):
                acc = 0.0
                for d in range(D):
                    acc += float(q_f64[i, h, d]) * float(k_f64[j, hk, d])
                logits.append(acc * scale)
            top = max(logits)
            weights = [math.exp(z - top) for z in logits]
            total = sum(weights)
            for d in range(D):
                acc = 0.0
                for j, w in enumerate(weights):
                    acc += w * float(v_f64[j, hk, d])
                out[i, h, d] = acc / total
    return out

"""Workload geometries and seeded tensors.

Geometry follows the AR-diffusion setting of the pages: one 832x480 latent
frame is (480/16)*(832/16) = 1560 tokens, K/V is paged in 16-token blocks, a
DiT has 40 blocks (layers), and classifier-free guidance runs a positive and a
negative branch as two sequences.

Random draws:
  * integers (sequence lengths, query lengths, the block permutation) come
    from ``numpy.random.default_rng(seed)`` in a fixed order;
  * activations are float32 N(0, 1) from a ``torch.Generator`` seeded with
    ``seed * 1000 + layer`` on the requested device, converted to the
    activation dtype by torch's round-to-nearest-even cast.  CPU and GPU
    generators give different (but each reproducible) bits; a GPU test copies
    the generated inputs to the host for the oracle.
  * fp8 pools get a per-tensor scale: the largest |K| (or |V|) over every
    token the layer writes, divided by 448, rounded to fp32; the quantisation
    multiplier is the fp32 reciprocal of that scale.  Both are inputs.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

FRAME_TOKENS = (480 // 16) * (832 // 16)  # 1560
BLOCK = 16


@dataclass(frozen=True)
class Geometry:
    name: str
    pool_dtype: str  # "f32" | "bf16" | "fp8"
    q_dtype: str  # "f32" | "bf16"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    history_lens: tuple[int, ...]  # tokens already written before this chunk, per sequence
    query_lens: tuple[int, ...]  # tokens of the current chunk, per sequence
    sink_tokens: tuple[int, ...]  # leading tokens the window always keeps
    window_tokens: tuple[int, ...]  # most recent tokens kept, current chunk included
    # Full-attention spans per sequence in key coordinates, or None for the
    # AR default (the whole chunk attends everything visible).
    full_spans: tuple[tuple[tuple[int, int], ...] | None, ...]
    causal_default: bool = False  # no spans at all -> causal within the chunk
    num_layers: int = 1
    block_size: int = BLOCK
    num_blocks: int = 0  # pool size in blocks; 0 -> ceil(1.25 * blocks needed)
    seed: int = 0
    note: str = ""
    # Action tokens per sequence (empty: none).  They follow the video chunk
    # in the query and sit in scratch blocks of their own after the window.
    action_lens: tuple[int, ...] = ()

    @property
    def num_seqs(self) -> int:
        return len(self.query_lens)

    def action_len(self, b: int) -> int:
        return self.action_lens[b] if self.action_lens else 0

    def action_blocks(self, b: int) -> int:
        return -(-self.action_len(b) // self.block_size)

    @property
    def query_rows(self) -> tuple[int, ...]:
        """Query rows per sequence: the video chunk, then the action tokens."""
        return tuple(q + self.action_len(b) for b, q in enumerate(self.query_lens))

    @property
    def ends(self) -> tuple[int, ...]:
        return tuple(h + q for h, q in zip(self.history_lens, self.query_lens))

    def logical_blocks(self, b: int) -> int:
        return -(-self.ends[b] // self.block_size)

    def pool_blocks(self) -> int:
        if self.num_blocks:
            return self.num_blocks
        need = sum(self.logical_blocks(b) + self.action_blocks(b) for b in range(self.num_seqs))
        return int(math.ceil(1.25 * need))


def _all_visible(n):
    return tuple([0] * n), tuple([1 << 30] * n)


def _c1() -> Geometry:
    sink, win = _all_visible(1)
    return Geometry(
        name="tiny_f32",
        pool_dtype="f32",
        q_dtype="f32",
        num_q_heads=4,
        num_kv_heads=4,
        head_dim=64,
        history_lens=(32,),
        query_lens=(16,),
        sink_tokens=sink,
        window_tokens=win,
        full_spans=(None,),
        num_blocks=64,
        seed=1001,
        note="1 seq, 2 history chunks of 16 + a 16-token chunk, full attention, 64-block permuted pool",
    )


def _c2() -> Geometry:
    return Geometry(
        name="frame_bf16",
        pool_dtype="bf16",
        q_dtype="bf16",
        num_q_heads=12,
        num_kv_heads=12,
        head_dim=128,
        history_lens=(3 * FRAME_TOKENS,) * 2,
        query_lens=(FRAME_TOKENS,) * 2,
        sink_tokens=(FRAME_TOKENS,) * 2,
        window_tokens=(3 * FRAME_TOKENS,) * 2,
        full_spans=(None, None),
        seed=1002,
        note="2 CFG branches, 1560-token chunk over 1 sink + 2 window chunks (history ends mid-block)",
    )


def _c3() -> Geometry:
    sink, win = _all_visible(1)
    return Geometry(
        name="piecewise_gqa_bf16",
        pool_dtype="bf16",
        q_dtype="bf16",
        num_q_heads=40,
        num_kv_heads=8,
        head_dim=128,
        history_lens=(FRAME_TOKENS,),
        query_lens=(3 * FRAME_TOKENS,),
        sink_tokens=sink,
        window_tokens=win,
        full_spans=(((FRAME_TOKENS, 2 * FRAME_TOKENS), (3 * FRAME_TOKENS, 4 * FRAME_TOKENS)),),
        seed=1003,
        note="query [1560, 6240) over keys [0, 6240); full spans [1560,3120) and [4680,6240), causal between",
    )


def _c4() -> Geometry:
    return Geometry(
        name="ar_step_40L_bf16",
        pool_dtype="bf16",
        q_dtype="bf16",
        num_q_heads=40,
        num_kv_heads=40,
        head_dim=128,
        history_lens=(5 * FRAME_TOKENS,) * 2,
        query_lens=(FRAME_TOKENS,) * 2,
        sink_tokens=(FRAME_TOKENS,) * 2,
        window_tokens=(5 * FRAME_TOKENS,) * 2,
        full_spans=(None, None),
        num_layers=40,
        seed=1004,
        note="40 layers, 2 CFG branches, 1560-token chunk over 1 sink + 4 window chunks (7800 history)",
    )


def _c5() -> Geometry:
    rng = np.random.default_rng(1005)
    seq_lens = rng.integers(2048, 32768, size=16, endpoint=True)
    q_lens = rng.choice(np.array([16, FRAME_TOKENS]), size=16)
    sink, win = _all_visible(16)
    return Geometry(
        name="varlen_fp8",
        pool_dtype="fp8",
        q_dtype="bf16",
        num_q_heads=32,
        num_kv_heads=8,
        head_dim=128,
        history_lens=tuple(int(s - q) for s, q in zip(seq_lens, q_lens)),
        query_lens=tuple(int(q) for q in q_lens),
        sink_tokens=sink,
        window_tokens=win,
        full_spans=(None,) * 16,
        causal_default=True,
        seed=1005,
        note="16 seqs, seq_len ~ U[2048, 32768], query len 16 or 1560, causal, fp8 e4m3 K/V pool",
    )


def _c5_short_queries(layers: int = 4) -> Geometry:
    """The 16-token-query sequences of the varlen batch on their own: the
    KV-bound half (each visible K/V byte feeds only 16 queries x 4 heads).
    ``layers`` independent pools are rotated through so that successive calls
    do not find their K/V in the last-level cache."""
    c5 = _c5()
    keep = [b for b, q in enumerate(c5.query_lens) if q == 16]
    pick = lambda t: tuple(t[b] for b in keep)  # noqa: E731
    return replace(
        c5,
        name="varlen_fp8_q16",
        history_lens=pick(c5.history_lens),
        query_lens=pick(c5.query_lens),
        sink_tokens=pick(c5.sink_tokens),
        window_tokens=pick(c5.window_tokens),
        full_spans=pick(c5.full_spans),
        num_layers=layers,
        note="the query-length-16 sequences of varlen_fp8, over several rotating pools",
    )


CONFIGS = {g.name: g for g in (_c1(), _c2(), _c3(), _c4(), _c5(), _c5_short_queries())}


def small_variant(geom: Geometry, **overrides) -> Geometry:
    """A copy of a geometry with some fields replaced (tests use it to shrink
    configurations while keeping their structure)."""
    if "num_blocks" not in overrides:
        overrides["num_blocks"] = 0
    return replace(geom, **overrides)


@dataclass
class LayerInputs:
    """Activations of one layer: history K/V (written before the step), the
    current chunk's K/V and the queries.  Token-major, ``[tokens, heads, D]``."""

    k_hist: torch.Tensor
    v_hist: torch.Tensor
    k_cur: torch.Tensor
    v_cur: torch.Tensor
    q: torch.Tensor
    k_scale: float = 1.0
    k_inv_scale: float = 1.0
    v_scale: float = 1.0
    v_inv_scale: float = 1.0
    k_act: torch.Tensor | None = None  # action K/V, [sum of action tokens, heads, D]
    v_act: torch.Tensor | None = None


@dataclass
class Workload:
    geom: Geometry
    device: str
    # block_ids[b][i]: physical block holding positions [16 i, 16 i + 16) of seq b
    block_ids: list[np.ndarray] = field(default_factory=list)
    # action_block_ids[b][i]: scratch block holding action tokens [16 i, 16 i + 16) of seq b
    action_block_ids: list[np.ndarray] = field(default_factory=list)

    def layer(self, layer: int) -> LayerInputs:
        g = self.geom
        act = torch.float32 if g.q_dtype == "f32" else torch.bfloat16
        gen = torch.Generator(device=self.device)
        gen.manual_seed(g.seed * 1000 + layer)
        H, Hq, D = g.num_kv_heads, g.num_q_heads, g.head_dim
        hist, cur = sum(g.history_lens), sum(g.query_lens)

        def draw(tokens, heads):
            x = torch.randn((tokens, heads, D), generator=gen, device=self.device, dtype=torch.float32)
            return x.to(act)

        acts = sum(g.action_len(b) for b in range(g.num_seqs))
        # Query rows in sequence order; each sequence's video rows come before
        # its action rows.
        q = draw(cur + acts, Hq)
        k_cur = draw(cur, H)
        v_cur = draw(cur, H)
        k_hist = draw(hist, H)
        v_hist = draw(hist, H)
        li = LayerInputs(k_hist=k_hist, v_hist=v_hist, k_cur=k_cur, v_cur=v_cur, q=q)
        if acts:
            li.k_act = draw(acts, H)
            li.v_act = draw(acts, H)
        if g.pool_dtype == "fp8":
            extra = (li.k_act,) if acts else ()
            li.k_scale, li.k_inv_scale = _fp8_scale(k_hist, k_cur, *extra)
            extra = (li.v_act,) if acts else ()
            li.v_scale, li.v_inv_scale = _fp8_scale(v_hist, v_cur, *extra)
        return li


def _fp8_scale(*parts: torch.Tensor) -> tuple[float, float]:
    amax = max(float(p.float().abs().max()) if p.numel() else 0.0 for p in parts)
    scale = np.float32(amax / 448.0) if amax > 0 else np.float32(1.0)
    inv = np.float32(1.0) / scale
    return float(scale), float(np.float32(inv))


def make_workload(geom: Geometry, device: str = "cpu") -> Workload:
    """Draw the block assignment: a seeded permutation of the pool's blocks,
    handed out to the sequences in order, so no two sequences share a block."""
    rng = np.random.default_rng(geom.seed)
    perm = rng.permutation(geom.pool_blocks())
    ids = []
    off = 0
    for b in range(geom.num_seqs):
        n = geom.logical_blocks(b)
        if off + n > len(perm):
            raise ValueError(f"pool of {len(perm)} blocks is too small for {geom.name}")
        ids.append(perm[off : off + n].astype(np.int64))
        off += n
    act_ids = []
    for b in range(geom.num_seqs):  # scratch blocks for action tokens come after every video block
        n = geom.action_blocks(b)
        if off + n > len(perm):
            raise ValueError(f"pool of {len(perm)} blocks is too small for {geom.name}")
        act_ids.append(perm[off : off + n].astype(np.int64))
        off += n
    return Workload(geom=geom, device=device, block_ids=ids, action_block_ids=act_ids)

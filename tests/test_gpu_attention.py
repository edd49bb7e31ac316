"""Paged attention on the GPU against the float64 oracle.

Tolerances (max |O_gpu - O_oracle|): 1e-4 for fp32, 2e-2 for bf16, 6e-2 for
fp8 K/V pools.  Small variants span several row and key tiles with ragged
tails; the configurations at full size are checked in full where the oracle
takes seconds and on sampled rows otherwise."""

import numpy as np
import pytest
import torch

import paged_kv_cache_174_amd as pkv
from oracle import harness as H
from workloads import CONFIGS, make_workload, small_variant

from . import gpu_harness as G

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    G.ensure_built()


def _check(geom, out, ref, rows=None, heads=None):
    got = G.as_f64(out)
    if rows is not None:
        got = got[np.asarray(rows)]
    if heads is not None:
        got = got[:, np.asarray(heads)]
    assert np.isfinite(got).all(), "non-finite output (an unwritten slot was read?)"
    err = np.max(np.abs(got - ref))
    assert err <= TOL[geom.pool_dtype], f"{geom.name}: max abs error {err:.3e} > {TOL[geom.pool_dtype]}"
    return err


SMALL = [
    CONFIGS["tiny_f32"],
    small_variant(CONFIGS["tiny_f32"], name="f32_d128_ragged", head_dim=128, num_q_heads=6, num_kv_heads=2,
                  history_lens=(70, 5), query_lens=(33, 90), sink_tokens=(0, 0), window_tokens=(1 << 30,) * 2,
                  full_spans=(((70, 90),), None)),
    small_variant(CONFIGS["frame_bf16"], name="frame_small_bf16", num_q_heads=3, num_kv_heads=3,
                  history_lens=(600, 600), query_lens=(300, 300), sink_tokens=(300, 300),
                  window_tokens=(900, 900)),
    small_variant(CONFIGS["frame_bf16"], name="slid_window_bf16", num_q_heads=2, num_kv_heads=2,
                  history_lens=(24 * 9, 24 * 5), query_lens=(24, 24), sink_tokens=(24, 48),
                  window_tokens=(72, 48)),
    small_variant(CONFIGS["piecewise_gqa_bf16"], name="piecewise_small_bf16", num_q_heads=10, num_kv_heads=2,
                  history_lens=(100,), query_lens=(300,), full_spans=(((100, 180), (250, 400)),)),
    small_variant(CONFIGS["piecewise_gqa_bf16"], name="piecewise_causal_only_bf16", num_q_heads=4, num_kv_heads=4,
                  history_lens=(0,), query_lens=(333,), full_spans=((),)),
    small_variant(CONFIGS["varlen_fp8"], name="varlen_small_fp8", num_q_heads=8, num_kv_heads=2,
                  history_lens=(100, 40, 777, 0, 5), query_lens=(16, 100, 16, 50, 1), sink_tokens=(0,) * 5,
                  window_tokens=(1 << 30,) * 5, full_spans=(None,) * 5),
    small_variant(CONFIGS["varlen_fp8"], name="varlen_small_bf16", pool_dtype="bf16", num_q_heads=4,
                  num_kv_heads=1, history_lens=(1000, 3), query_lens=(64, 1), sink_tokens=(0,) * 2,
                  window_tokens=(1 << 30,) * 2, full_spans=(None,) * 2),
    small_variant(CONFIGS["frame_bf16"], name="single_key_bf16", num_q_heads=2, num_kv_heads=1,
                  history_lens=(0,), query_lens=(1,), sink_tokens=(0,), window_tokens=(1 << 30,),
                  full_spans=(None,)),
    small_variant(CONFIGS["frame_bf16"], name="block_aligned_bf16", num_q_heads=2, num_kv_heads=2,
                  history_lens=(128,), query_lens=(64,), sink_tokens=(0,), window_tokens=(1 << 30,),
                  full_spans=(None,)),
    # Long causal chunks: the key range is split, and early row tiles see fewer
    # keys than one split holds (later splits are empty for them) while later
    # ones span several splits (merged by the separate merge launch).
    small_variant(CONFIGS["piecewise_gqa_bf16"], name="causal_long_split_bf16", num_q_heads=2, num_kv_heads=2,
                  history_lens=(0,), query_lens=(1200,), full_spans=((),)),
    # Short query chunks (at most 64 rows per KV head): the kernel that splits
    # the keys four ways inside the workgroup and merges them in LDS.
    small_variant(CONFIGS["varlen_fp8"], name="short_fp8_gqa", num_q_heads=8, num_kv_heads=2,
                  history_lens=(3000, 700, 90, 5000), query_lens=(16, 16, 3, 16), sink_tokens=(0,) * 4,
                  window_tokens=(1 << 30,) * 4, full_spans=(None,) * 4),
    small_variant(CONFIGS["frame_bf16"], name="short_window_bf16", num_q_heads=4, num_kv_heads=2,
                  history_lens=(1000, 37), query_lens=(32, 7), sink_tokens=(300, 0), window_tokens=(600, 1 << 30)),
    small_variant(CONFIGS["piecewise_gqa_bf16"], name="short_piecewise_bf16", num_q_heads=2, num_kv_heads=2,
                  history_lens=(200,), query_lens=(60,), full_spans=(((210, 240),),)),
    # More than 64 sequences (the kernels then read each workgroup's sequence entries
    # directly instead of across the lanes) and more than 8 segments in a sequence
    # (row limits then come from the segment walk instead of the register copy).
    small_variant(CONFIGS["frame_bf16"], name="many_seqs_long_bf16", num_q_heads=2, num_kv_heads=1,
                  history_lens=tuple(20 + 7 * (i % 5) for i in range(70)), query_lens=(40,) * 70,
                  sink_tokens=(0,) * 70, window_tokens=(1 << 30,) * 70, full_spans=(None,) * 70),
    small_variant(CONFIGS["varlen_fp8"], name="many_seqs_fp8", num_q_heads=4, num_kv_heads=1,
                  history_lens=tuple(30 + 11 * (i % 7) for i in range(66)), query_lens=(16,) * 33 + (90,) * 33,
                  sink_tokens=(0,) * 66, window_tokens=(1 << 30,) * 66, full_spans=(None,) * 66),
    small_variant(CONFIGS["piecewise_gqa_bf16"], name="many_segments_bf16", num_q_heads=4, num_kv_heads=2,
                  history_lens=(100,), query_lens=(500,),
                  full_spans=(((110, 130), (160, 170), (200, 260), (300, 310), (350, 400), (450, 520)),)),
    # head_dim 64 (P2's geometry: 4 heads, D 64, 16-token blocks) on each MFMA kernel:
    # bf16 long chunks, bf16 short chunks, fp8 long and short chunks, piecewise GQA.
    small_variant(CONFIGS["frame_bf16"], name="d64_bf16_long", head_dim=64, num_q_heads=4, num_kv_heads=4,
                  history_lens=(3000, 37), query_lens=(300, 90), sink_tokens=(0, 0), window_tokens=(1 << 30,) * 2),
    small_variant(CONFIGS["frame_bf16"], name="d64_bf16_short", head_dim=64, num_q_heads=4, num_kv_heads=4,
                  history_lens=(2000, 32), query_lens=(16, 16), sink_tokens=(0, 0), window_tokens=(1 << 30,) * 2),
    small_variant(CONFIGS["varlen_fp8"], name="d64_fp8_long", head_dim=64, num_q_heads=8, num_kv_heads=2,
                  history_lens=(900, 5), query_lens=(200, 70), sink_tokens=(0,) * 2,
                  window_tokens=(1 << 30,) * 2, full_spans=(None,) * 2),
    small_variant(CONFIGS["varlen_fp8"], name="d64_fp8_short", head_dim=64, num_q_heads=8, num_kv_heads=2,
                  history_lens=(3000, 40), query_lens=(16, 16), sink_tokens=(0,) * 2,
                  window_tokens=(1 << 30,) * 2, full_spans=(None,) * 2),
    small_variant(CONFIGS["piecewise_gqa_bf16"], name="d64_piecewise_gqa", head_dim=64, num_q_heads=8,
                  num_kv_heads=2, history_lens=(100,), query_lens=(300,), full_spans=(((100, 180), (250, 400)),)),
    small_variant(CONFIGS["piecewise_gqa_bf16"], name="causal_hist_split_bf16", num_q_heads=4, num_kv_heads=2,
                  history_lens=(3000, 100), query_lens=(600, 700), full_spans=((), ((100, 500),)), sink_tokens=(0, 0), window_tokens=(1 << 30,) * 2),
    # Long chunks with 3, 4, 6 and 8 query heads per KV head: a workgroup's and
    # a wave's rows start mid-token and cross token boundaries in every pattern
    # (Q is loaded and the output stored four rows at a time).
    small_variant(CONFIGS["frame_bf16"], name="gqa3_long_bf16", num_q_heads=6, num_kv_heads=2,
                  history_lens=(500, 40), query_lens=(150, 31), sink_tokens=(0, 0), window_tokens=(1 << 30,) * 2),
    small_variant(CONFIGS["frame_bf16"], name="gqa4_long_bf16", num_q_heads=8, num_kv_heads=2,
                  history_lens=(700, 0), query_lens=(77, 130), sink_tokens=(0, 0), window_tokens=(1 << 30,) * 2),
    small_variant(CONFIGS["piecewise_gqa_bf16"], name="gqa6_long_bf16", num_q_heads=12, num_kv_heads=2,
                  history_lens=(300,), query_lens=(53,), full_spans=(((310, 330),),)),
    small_variant(CONFIGS["frame_bf16"], name="gqa8_long_bf16", num_q_heads=16, num_kv_heads=2,
                  history_lens=(1000, 64), query_lens=(40, 9), sink_tokens=(0, 0), window_tokens=(1 << 30,) * 2),
]


PLAN_KERNEL = {
    "tiny_f32": "f32",
    "frame_small_bf16": "long",
    "gqa3_long_bf16": "long",
    "gqa8_long_bf16": "long",
    "short_window_bf16": "short",
    "short_fp8_gqa": "short",
    "varlen_small_fp8": "fp8",
}


@pytest.mark.parametrize("name", sorted(PLAN_KERNEL))
def test_plan_names_the_kernel(name):
    """pkv_last_attn_plan reports the kernel family the call ran: the long-chunk
    bf16 kernel, the short-chunk kernel, the fp8 kernel or the fp32 path."""
    geom = next(g for g in SMALL if g.name == name)
    wl = make_workload(geom, device="cuda")
    G.run(wl)
    plan = pkv.pkv_last_attn_plan()
    assert plan.split()[0] == PLAN_KERNEL[name], plan


@pytest.mark.parametrize("geom", SMALL, ids=[g.name for g in SMALL])
@pytest.mark.parametrize("workspace", ["auto", None], ids=["split", "nosplit"])
def test_small_configs_match_oracle(geom, workspace):
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    G.say("attn", geom.name, workspace)
    _, _, _, out = G.run(wl, li=li, workspace=workspace)
    _, _, _, ref = H.run_layer(wl, li=li)
    _check(geom, out, ref)


def test_frame_bf16_full_size_matches_oracle():
    """The 1560-token frame over 1 sink + 2 window chunks, every output."""
    geom = CONFIGS["frame_bf16"]
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    G.say("attn full", geom.name)
    plan, _, _, out = G.run(wl, li=li)
    assert plan.kv_lens == [6240, 6240]
    _, _, _, ref = H.run_layer(wl, li=li)
    _check(geom, out, ref)


def _sample_rows(geom, rng, per_seq=24, seqs=None):
    qsl = np.concatenate([[0], np.cumsum(geom.query_lens)])
    rows = []
    for b in range(geom.num_seqs) if seqs is None else seqs:
        lo, hi = int(qsl[b]), int(qsl[b + 1])
        picks = {lo, hi - 1, min(lo + 255, hi - 1), min(lo + 256, hi - 1)}
        picks |= set(rng.integers(lo, hi, size=per_seq).tolist())
        rows.extend(sorted(picks))
    return rows


def test_piecewise_gqa_full_size_sampled_rows():
    geom = CONFIGS["piecewise_gqa_bf16"]
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    G.say("attn full", geom.name)
    _, _, _, out = G.run(wl, li=li)
    # rows at and around every segment boundary plus random ones
    edges = [0, 1, 1559, 1560, 1561, 3119, 3120, 3121, 4679]
    rows = sorted(set(edges) | set(np.random.default_rng(0).integers(0, 4680, 40).tolist()))
    _, _, _, ref = H.run_layer(wl, li=li, rows=rows)
    _check(geom, out, ref, rows=rows)


def test_varlen_fp8_full_size_sampled_rows():
    geom = CONFIGS["varlen_fp8"]
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    G.say("attn full", geom.name)
    _, _, _, out = G.run(wl, li=li)
    q = np.asarray(geom.query_lens)
    s = np.asarray(geom.history_lens) + q
    long_q = int(np.argmax(np.where(q == 1560, s, -1)))
    short_q = int(np.argmax(np.where(q == 16, s, -1)))
    seqs = sorted({long_q, short_q, int(np.argmin(s))})
    rows = _sample_rows(geom, np.random.default_rng(1), per_seq=12, seqs=seqs)
    heads = [0, 3, 4, 31]
    _, _, _, ref = H.run_layer(wl, li=li, rows=rows, heads=heads, seqs=seqs)
    _check(geom, out, ref, rows=rows, heads=heads)


def test_varlen_fp8_short_queries_full_size():
    """The KV-bound half of the varlen batch (query length 16, 32/8 heads, up to
    32k keys) through the short-query kernel: every row of the longest and the
    shortest sequence on four heads."""
    geom = CONFIGS["varlen_fp8_q16"]
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    G.say("attn full", geom.name)
    plan, _, _, out = G.run(wl, li=li)
    s = np.asarray(plan.kv_lens)
    seqs = sorted({int(np.argmax(s)), int(np.argmin(s))})
    qsl = np.concatenate([[0], np.cumsum(geom.query_lens)])
    rows = [r for b in seqs for r in range(int(qsl[b]), int(qsl[b + 1]))]
    heads = [0, 5, 17, 31]
    _, _, _, ref = H.run_layer(wl, li=li, rows=rows, heads=heads, seqs=seqs)
    _check(geom, out, ref, rows=rows, heads=heads)


def test_ar_step_layers_sampled():
    """The 40-layer step's shape (2 x 40 heads, 9360 visible keys): write + attend
    on a few layers, each with its own pools, shared metadata."""
    geom = CONFIGS["ar_step_40L_bf16"]
    wl = make_workload(geom, device="cuda")
    plan = G.make_plan(wl)
    assert plan.kv_lens == [9360, 9360]
    for layer in (0, 39):
        li = wl.layer(layer)
        G.say("attn layer", layer)
        pools = G.make_pools(geom, li)
        G.write_layer(plan, pools, li)
        out = G.attend(plan, pools, li, geom)
        torch.cuda.synchronize()
        rows = _sample_rows(geom, np.random.default_rng(layer), per_seq=6)
        heads = [0, 17, 39]
        _, _, _, ref = H.run_layer(wl, li=li, rows=rows, heads=heads)
        _check(geom, out, ref, rows=rows, heads=heads)
        del pools, out


@pytest.mark.parametrize("name,layer,capacity", [("ar_step_40L_bf16", 7, 587), ("frame_bf16", 0, 392)])
def test_fused_call_all_heads_at_tile_edges(name, layer, capacity):
    """One layer of the 40-layer step, and the frame layer, through the fused
    per-layer call (pkv_paged_write_attn: the current chunk's slot writes,
    then attention and the merge of its key splits) at full size and with the
    metadata P1 build_block_table passes (table width and max_seq_len fixed
    at the window's capacity; the bench times the same): every query head, on
    rows at each 256-row tile edge of both sequences (the last tile holds the
    24-row tail), the first and last rows, and random ones.  Every row here
    sees all keys, so each one spans every key split."""
    geom = CONFIGS[name]
    wl = make_workload(geom, device="cuda")
    plan = G.make_plan(wl, fixed_capacity=True)
    assert plan.block_table.shape[1] == capacity and plan.max_seq_len == 16 * capacity
    li = wl.layer(layer)
    pools = G.make_pools(geom, li)
    G.P.pkv_paged_write(li.k_hist, li.v_hist, plan.history_slot_mapping, pools)
    G.say("fused call", geom.name, "layer", layer)
    out = G.write_attend(plan, pools, li, geom)
    torch.cuda.synchronize()
    assert G.workspace_for(plan, geom) is not None  # the keys are split
    qsl = np.concatenate([[0], np.cumsum(geom.query_lens)])
    rng = np.random.default_rng(layer)
    rows = set()
    for b in range(geom.num_seqs):
        lo, hi = int(qsl[b]), int(qsl[b + 1])
        for edge in range(0, hi - lo, 256):
            rows |= {lo + max(edge - 1, 0), lo + edge}
        rows |= {hi - 1} | set(rng.integers(lo, hi, size=4).tolist())
    rows = sorted(rows)
    _, _, _, ref = H.run_layer(wl, li=li, rows=rows)
    _check(geom, out, ref, rows=rows)


def test_varlen_fp8_a_row_block_of_every_sequence():
    """The whole varlen fp8 batch (16 sequences, 2k..32k keys, chunks of 16
    and 1560 queries, causal): for every sequence, the rows of one workgroup
    -- 64 consecutive query tokens (all of a 16-token chunk) times the 4 query
    heads of a KV head -- for the first and the last KV head."""
    geom = CONFIGS["varlen_fp8"]
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    G.say("attn full", geom.name, "row block per sequence")
    _, _, _, out = G.run(wl, li=li)
    qsl = np.concatenate([[0], np.cumsum(geom.query_lens)])
    rng = np.random.default_rng(5)
    rows = []
    for b in range(geom.num_seqs):
        lo, hi = int(qsl[b]), int(qsl[b + 1])
        start = lo if hi - lo <= 64 else lo + 64 * int(rng.integers(0, (hi - lo) // 64))
        rows.extend(range(start, min(start + 64, hi)))
    heads = [0, 1, 2, 3, 28, 29, 30, 31]
    _, _, _, ref = H.run_layer(wl, li=li, rows=rows, heads=heads)
    _check(geom, out, ref, rows=rows, heads=heads)


UNEVEN = [
    small_variant(CONFIGS["frame_bf16"], name="uneven_splits_full_bf16", num_q_heads=24, num_kv_heads=24,
                  history_lens=(1720, 1720), query_lens=(280, 280), sink_tokens=(0, 0),
                  window_tokens=(1 << 30, 1 << 30), full_spans=(None, None)),
    small_variant(CONFIGS["frame_bf16"], name="uneven_splits_causal_bf16", num_q_heads=24, num_kv_heads=24,
                  history_lens=(1720, 1720), query_lens=(280, 280), sink_tokens=(0, 0),
                  window_tokens=(1 << 30, 1 << 30), full_spans=((), ()), causal_default=True),
]


@pytest.mark.parametrize("geom", UNEVEN, ids=[g.name for g in UNEVEN])
def test_key_splits_of_unequal_length(geom):
    """The long kernel's planner cuts this launch's 2000 keys into splits of
    896, 896 and 208 keys (the short one fills in behind the others), and
    each head's 280 rows are a full row tile and a 24-row tail.  Every row of
    every head against the oracle; with causal rows the last split is empty
    for the chunk's early rows, which write an empty partial."""
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    G.say("uneven splits", geom.name)
    _, _, _, out = G.run(wl, li=li)
    assert "splits=3" in pkv.pkv_last_attn_plan() and "cut=896,1792" in pkv.pkv_last_attn_plan()
    _, _, _, ref = H.run_layer(wl, li=li)
    _check(geom, out, ref)


@pytest.mark.parametrize("gain", [30.0, 8.0])
def test_scores_far_above_the_first_subtile(gain):
    """The long-chunk kernel fixes each row's running max after its first
    32 keys and reruns a workgroup exactly (max moving per sub-tile) when a
    row's probability sum passes 2^64 or is not finite.  Keys from position
    500 on are scaled up: with gain 30 their scores (log2 units, std ~40)
    overflow against the first keys' max and force the rerun; with gain 8
    (std ~11) the fast path absorbs them.  Both must match the oracle."""
    geom = small_variant(CONFIGS["frame_bf16"], name=f"rising_scores_{int(gain)}", num_q_heads=2, num_kv_heads=2,
                         history_lens=(1000,), query_lens=(300,), sink_tokens=(0,), window_tokens=(1 << 30,),
                         full_spans=(None,))
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    li.k_hist = li.k_hist.clone()
    li.k_hist[500:] = (li.k_hist[500:].float() * gain).to(li.k_hist.dtype)
    G.say("rising scores", gain)
    _, _, _, out = G.run(wl, li=li)
    _, _, _, ref = H.run_layer(wl, li=li)
    _check(geom, out, ref)


def test_bad_arguments_raise_before_launch():
    geom = SMALL[2]
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    plan = G.make_plan(wl)
    pools = G.make_pools(geom, li)
    with pytest.raises(ValueError):  # q dtype does not go with a bf16 pool
        G.P.pkv_paged_attn(li.q.float(), pools, plan.block_table, plan.query_start_loc, plan.seq_lens,
                           plan.segments, plan.segment_start_loc, 0.1, plan.max_query_len, plan.max_seq_len)
    with pytest.raises(ValueError):  # max_query_len > max_seq_len
        G.P.pkv_paged_attn(li.q, pools, plan.block_table, plan.query_start_loc, plan.seq_lens,
                           plan.segments, plan.segment_start_loc, 0.1, 10_000, plan.max_seq_len)
    with pytest.raises(ValueError):  # heads not a multiple of KV heads
        G.P.pkv_paged_attn(li.q[:, :2].contiguous(), pools, plan.block_table, plan.query_start_loc,
                           plan.seq_lens, plan.segments, plan.segment_start_loc, 0.1, plan.max_query_len,
                           plan.max_seq_len)

"""Pins of the CPU oracle to things other than itself: values the pages and the
OCP fp8 spec fix, library routines, closed forms, brute force, and invariants
the pages state.  No GPU.
Pages cited by tag and function: P1 "vllm_omni/experimental/ar_diffusion/kv_cache/paged_attention.py",
P2 "tests/diffusion/ar_diffusion/test_paged_attention.py",
P3 "vllm_omni/diffusion/attention/backends/utils/piecewise_attn.py",
P4 "vllm_omni/diffusion/diffusion_kv/paged_attention_adapter.py"."""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from oracle import harness as H
from workloads import CONFIGS, make_workload, small_variant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------- formats


def test_bf16_decode_matches_torch_on_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = O.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_e4m3_code_values_match_the_ocp_table():
    g = _golden("e4m3_codes.json")
    vals = O.e4m3_code_values()
    for code, want in g["codes"].items():
        got = vals[int(code, 16)]
        assert got == want and math.copysign(1, got) == math.copysign(1, want), code
    for code in g["nan_codes"]:
        assert math.isnan(vals[int(code, 16)])
    finite = vals[~np.isnan(vals)]
    assert len(finite) == 254 and finite.max() == 448.0 and finite.min() == -448.0


def test_e4m3_encode_golden_cases():
    g = _golden("e4m3_codes.json")
    for case in g["encode_cases"]:
        x = float(case["x"])
        assert int(O.e4m3_encode(np.array([x]))[0]) == int(case["code"], 16), case["why"]
    assert int(O.e4m3_encode(np.array([np.nan]))[0]) & 0x7F == 0x7F


def test_e4m3_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = O.e4m3_decode(codes)
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


@pytest.mark.parametrize("inv_scale", [1.0, 1.0 / 3.7, 448.0 / 4.5, 0.001, 37.0])
def test_e4m3_quantiser_matches_torch_cast_on_all_bf16_inputs(inv_scale):
    """The pool cast (bf16 -> fp32 * inv_scale -> e4m3, RNE, saturating) against
    torch's float8_e4m3fn cast of the same fp32 product.  torch does not
    saturate (beyond the rounding range it yields NaN), so the comparison is
    restricted to products that round to a finite value, and saturation is
    pinned separately above."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = O.bf16_bits_to_f64(bits)
    keep = np.isfinite(x)
    bits, x = bits[keep], x[keep]
    prod32 = (torch.from_numpy(x).to(torch.float32) * torch.tensor(np.float32(inv_scale))).to(torch.float32)
    in_range = prod32.abs() < 464.0
    ref = prod32[in_range].to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = O.encode_for_pool(bits, O.BF16, O.FP8, inv_scale)[in_range.numpy()]
    assert np.array_equal(ours, ref)
    sat = O.encode_for_pool(bits, O.BF16, O.FP8, inv_scale)[~in_range.numpy()]
    assert np.all((sat & 0x7F) == 0x7E)


# --------------------------------------------------------------------------- metadata


def test_slot_mapping_ragged_chunk_worked_example():
    """P2: after one 24-token chunk in 16-token blocks, the next chunk's first
    slot is the history's tail block * 16 + 8."""
    g = _golden("window_geometry.json")["ragged_chunk"]
    ids = [5, 9, 2]  # any physical blocks for logical blocks 0, 1, 2
    first = int(O.slot_mapping(ids, [g["chunk"]], g["block"])[0])
    assert first == ids[1] * 16 + 8
    # and the whole chunk is contiguous with its history
    slots = O.slot_mapping(ids, np.arange(24, 48), 16)
    assert list(slots[:8]) == [9 * 16 + o for o in range(8, 16)]
    assert list(slots[8:24]) == [2 * 16 + o for o in range(16)]


def test_frame_geometry_numbers():
    g = _golden("window_geometry.json")
    assert (480 // 16) * (832 // 16) == g["frame_tokens"]
    assert g["frame_tokens"] % 16 == g["frame_mod_block"]
    assert -(-g["frame_tokens"] // 16) == g["blocks_per_frame"]


def test_visible_window_slid_worked_example():
    g = _golden("window_geometry.json")["slid_window"]
    end = g["history"] + g["query"]
    ids = np.arange(10_000, 10_000 + -(-end // 16))
    win = O.visible_window(ids, end, g["sink_chunks"] * g["chunk"], g["window_tokens"], g["block"])
    assert win.kv_len == g["expected_kv_len"]
    assert len(win.table) == g["expected_table_len"]
    lo, hi = g["expected_sink_blocks"]
    assert win.table[: hi + 1] == list(ids[lo : hi + 1])
    assert win.table[hi + 1] == ids[g["expected_recent_first_block"]]
    assert win.positions[1567] == 1567 and win.positions[1568] == 487 * 16


def _index_range_window(ids, history, q, sink, window, B):
    """P1 ``video_block_table`` in its own (index-range) formulation, as a second
    statement of the rule: sink blocks and blocks from the recent start onward,
    the current chunk's blocks always listed, blocks wholly between the two
    ranges skipped, lengths ``min(B, end - first)``."""
    end = history + q
    recent_start = end - window
    hist_blocks = -(-history // B)
    sink_blocks = min(-(-sink // B), hist_blocks)
    recent_first = max(max(recent_start, 0) // B, sink_blocks)
    first_pos = {}
    for i in [*range(sink_blocks), *range(recent_first, hist_blocks)]:
        if ids[i] >= 0:
            first_pos.setdefault(ids[i], i * B)
    cur_first = history - history % B
    for n in range(-(-(history % B + q) // B)):
        first_pos.setdefault(ids[cur_first // B + n], cur_first + n * B)
    table, length = [], 0
    for blk, first in sorted(first_pos.items(), key=lambda kv: kv[1]):
        if first >= sink and first + B <= recent_start:
            continue
        table.append(int(blk))
        length += min(B, end - first)
    return table, length


@pytest.mark.parametrize("chunk,sink_chunks,window_chunks", [(24, 1, 2), (24, 0, 2), (24, 1, 3), (1560, 9, 9), (16, 1, 2), (40, 2, 3)])
def test_visible_window_agrees_with_index_range_rule_and_page_invariants(chunk, sink_chunks, window_chunks):
    B = 16
    rng = np.random.default_rng(chunk * 31 + sink_chunks)
    frames_per_tick = 3 if chunk == 1560 else 1
    sink, window = sink_chunks * chunk, window_chunks * chunk
    total_ticks = 12
    ids = rng.permutation(10 * (total_ticks * frames_per_tick * chunk // B + 4))
    widths = set()
    for tick in range(total_ticks):
        q = frames_per_tick * chunk
        history = tick * q
        end = history + q
        win = O.visible_window(ids, end, sink, window, B)
        ref_table, ref_len = _index_range_window(ids, history, q, sink, window, B)
        assert win.table == ref_table and win.kv_len == ref_len
        # every kept token is read, in order, and each read slot holds its position
        kept = set(range(min(sink, end))) | set(range(max(end - window, 0), end))
        assert kept <= set(win.positions)
        assert win.positions == sorted(win.positions)
        assert win.kv_len == len(win.positions)
        # whole blocks: at most B - 1 extra tokens at each of the two boundaries (P2)
        assert win.kv_len <= min(end, sink + window) + 2 * (B - 1)
        for n, p in enumerate(win.positions):
            assert win.table[n // B] == ids[p // B] and n % B == p % B
        widths.add(len(win.table))
    assert max(widths) <= -(-sink // B) + -(-window // B) + 1


def test_segments_golden():
    for case in _golden("segments.json")["cases"]:
        segs = O.build_segments([tuple(s) for s in case["spans"]], case["query_offset"], case["query_len"])
        assert [[s.q_start, s.q_end, s.kv_end, s.mode] for s in segs] == case["segments"], case["why"]


def test_segments_of_touching_spans_stay_apart():
    """Two full spans that touch, [2, 5) and [5, 9), over the query [0, 12):
    their rows attend K[:5] and K[:9] respectively (P3 module docstring), so
    they are two full segments, between causal runs [0, 2) and [9, 12)."""
    segs = O.build_segments([(2, 5), (5, 9)], 0, 12)
    assert [(g.q_start, g.q_end, g.kv_end, g.mode) for g in segs] == [
        (0, 2, 2, "causal"), (2, 5, 5, "full"), (5, 9, 9, "full"), (9, 12, 12, "causal")]
    # a span that starts before the query and one that ends past it keep their own ends
    segs = O.build_segments([(0, 4), (10, 20)], 3, 9)
    assert [(g.q_start, g.q_end, g.kv_end, g.mode) for g in segs] == [
        (3, 4, 4, "full"), (4, 10, 10, "causal"), (10, 12, 20, "full")]


def test_row_limits_against_the_docstring_rule_by_enumeration():
    """P3's docstring: a row inside a full span [a, b) sees keys < b; any other
    row is causal and sees keys <= its own position.  Enumerate random span sets
    and compare every row."""
    rng = np.random.default_rng(7)
    for _ in range(300):
        s = int(rng.integers(1, 60))
        q = int(rng.integers(1, s + 1))
        cuts = sorted(set(rng.integers(0, s + 1, size=int(rng.integers(0, 7))).tolist()))
        spans = [(cuts[i], cuts[i + 1]) for i in range(0, len(cuts) - 1, 2) if cuts[i] < cuts[i + 1]]
        segs = O.build_segments(spans, s - q, q)
        # tiling
        assert segs[0].q_start == s - q and segs[-1].q_end == s
        assert all(a.q_end == b.q_start for a, b in zip(segs, segs[1:]))
        lim = O.row_limits(segs, s, q)
        for i in range(q):
            g = s - q + i
            inside = [b for a, b in spans if a <= g < b]
            want = inside[0] if inside else g + 1
            assert lim[i] == want
        assert np.all(np.diff(lim) >= 0) or spans  # causal-only limits are increasing


# --------------------------------------------------------------------------- write / gather


def test_write_is_a_bit_exact_scatter_and_leaves_other_slots():
    rng = np.random.default_rng(3)
    pool = np.full((64 * 16, 2, 8), np.uint16(0x7FC0), dtype=np.uint16)
    src = rng.integers(0, 1 << 16, size=(40, 2, 8)).astype(np.uint16)
    slots = rng.permutation(64 * 16)[:40]
    O.paged_write(pool, src, slots, O.BF16, O.BF16)
    assert np.array_equal(pool[slots], src)
    others = np.setdiff1d(np.arange(64 * 16), slots)
    assert np.all(pool[others] == 0x7FC0)
    with pytest.raises(ValueError):
        O.paged_write(pool, src[:2], [1, 1], O.BF16, O.BF16)


def test_gather_matches_index_select_and_keeps_sentinel():
    """P2 history-staging test: staging equals torch.index_select of the blocks,
    and rows outside the restaged range keep a -7 sentinel."""
    rng = np.random.default_rng(4)
    B = 16
    pool = rng.standard_normal((50 * B, 3, 8)).astype(np.float32)
    ids = rng.permutation(50)[:12]
    stage = np.full((15 * B, 3, 8), -7.0, dtype=np.float32)
    O.gather(pool, ids, 12, 4, stage, B)
    ref = torch.index_select(torch.from_numpy(pool).view(50, B, 3, 8), 0, torch.from_numpy(ids[4:12])).reshape(-1, 3, 8)
    assert np.array_equal(stage[4 * B : 12 * B], ref.numpy())
    assert np.all(stage[: 4 * B] == -7.0) and np.all(stage[12 * B :] == -7.0)


# --------------------------------------------------------------------------- attention


def _tiny_case(seed, q_len, s, Hq, Hkv, D):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((q_len, Hq, D))
    k = rng.standard_normal((s, Hkv, D))
    v = rng.standard_normal((s, Hkv, D))
    return q, k, v


@pytest.mark.parametrize("spans", [None, [], [(2, 9)], [(0, 5), (7, 12)]])
def test_attention_matches_scalar_bruteforce(spans):
    s, q_len = 14, 8
    q, k, v = _tiny_case(1, q_len, s, 4, 2, 5)
    segs = O.segments_for_rows([spans], [q_len], [s])[0]
    lim = O.row_limits(segs, s, q_len)
    scale = 5 ** -0.5
    fast = O.dense_attention(q, k, v, lim, scale)
    slow = O.attention_bruteforce(q, k, v, lim, scale)
    assert np.max(np.abs(fast - slow)) < 1e-12


def test_attention_reduces_to_torch_sdpa_with_explicit_mask():
    s, q_len, Hq, Hkv, D = 70, 33, 6, 3, 16
    q, k, v = _tiny_case(2, q_len, s, Hq, Hkv, D)
    segs = O.segments_for_rows([[(40, 50), (60, 66)]], [q_len], [s])[0]
    lim = O.row_limits(segs, s, q_len)
    scale = D ** -0.5
    ours = O.dense_attention(q, k, v, lim, scale)
    mask = torch.arange(s)[None, :] < torch.from_numpy(lim)[:, None]
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(k).repeat_interleave(Hq // Hkv, dim=1).permute(1, 0, 2)
    tv = torch.from_numpy(v).repeat_interleave(Hq // Hkv, dim=1).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    assert np.max(np.abs(ours - ref.permute(1, 0, 2).numpy())) < 1e-12


def test_attention_closed_forms():
    s, q_len, D = 30, 10, 8
    _, k, v = _tiny_case(3, q_len, s, 2, 2, D)
    segs = O.segments_for_rows([[(22, 26)]], [q_len], [s])[0]
    lim = O.row_limits(segs, s, q_len)
    # Q = 0: uniform weights -> each row is the mean of the values it may see
    zero = O.dense_attention(np.zeros((q_len, 2, D)), k, v, lim, 1.0)
    for i in range(q_len):
        assert np.allclose(zero[i], v[: lim[i]].mean(axis=0), atol=1e-14)
    # one visible key -> the output is that value
    one = O.dense_attention(np.ones((1, 2, D)), k[:1], v[:1], np.array([1]), 0.3)
    assert np.array_equal(one[0], v[0])
    # identical keys -> mean of values whatever the query
    same_k = np.repeat(k[:1], s, axis=0)
    qq = np.random.default_rng(9).standard_normal((q_len, 2, D))
    out = O.dense_attention(qq, same_k, v, np.full(q_len, s), 0.7)
    assert np.allclose(out, v.mean(axis=0)[None], atol=1e-12)


def test_causal_row_ignores_later_keys_and_full_row_sees_its_span():
    s, q_len = 24, 12
    q, k, v = _tiny_case(5, q_len, s, 2, 2, 4)
    segs = O.segments_for_rows([[(16, 20)]], [q_len], [s])[0]
    lim = O.row_limits(segs, s, q_len)
    base = O.dense_attention(q, k, v, lim, 0.5)
    k2, v2 = k.copy(), v.copy()
    k2[21:] += 3.0
    v2[21:] -= 2.0
    moved = O.dense_attention(q, k2, v2, lim, 0.5)
    g = np.arange(s - q_len, s)
    causal_rows = np.nonzero(lim <= 21)[0]
    assert np.array_equal(base[causal_rows], moved[causal_rows])
    # full rows of span [16, 20) see keys < 20 only, so changing key 19 moves them
    k3 = k.copy()
    k3[19] += 1.0
    moved3 = O.dense_attention(q, k3, v, lim, 0.5)
    full_rows = np.nonzero((g >= 16) & (g < 20))[0]
    assert np.all(np.abs(moved3[full_rows] - base[full_rows]).max(axis=(1, 2)) > 0)


def test_paged_view_equals_dense_over_window_positions():
    """P2's pattern: paged attention over a permuted pool equals dense attention
    over the K/V of the positions the window keeps (here with a slid window,
    ragged chunks and a history ending mid-block)."""
    geom = small_variant(
        CONFIGS["frame_bf16"],
        name="ragged_window",
        num_q_heads=4,
        num_kv_heads=2,
        head_dim=16,
        history_lens=(7 * 24, 5 * 24),
        query_lens=(24, 24),
        sink_tokens=(24, 24),
        window_tokens=(72, 48),
        full_spans=(None, None),
    )
    wl = make_workload(geom)
    li = wl.layer(0)
    meta, kp, vp, out = H.run_layer(wl, li=li)
    k_all = torch.cat([li.k_hist[: geom.history_lens[0]], li.k_cur[:24]]).float().double().numpy()
    v_all = torch.cat([li.v_hist[: geom.history_lens[0]], li.v_cur[:24]]).float().double().numpy()
    pos = meta.positions[0]
    lim = np.full(24, len(pos))
    ref = O.dense_attention(li.q[:24].float().double().numpy(), k_all[pos], v_all[pos], lim, H.softmax_scale(16))
    assert np.max(np.abs(out[:24] - ref)) < 1e-12
    assert meta.kv_lens[0] < geom.history_lens[0] + 24  # the window actually slid


def test_unwritten_slots_never_reach_the_output():
    """The oracle pool starts as NaN everywhere; a finite output shows only
    written slots were read (P2's NaN-poisoning test)."""
    wl = make_workload(CONFIGS["tiny_f32"])
    _, _, _, out = H.run_layer(wl)
    assert np.isfinite(out).all()


# --------------------------------------------------------------------------- action tokens


def test_action_tokens_follow_the_window_like_the_pages_dense_reference():
    """P2 ``test_paged_attention_matches_dense_reference_cpu`` with actions: the
    paged result over video window + action scratch blocks equals dense
    attention over the windowed video K/V with the action K/V appended, the
    query being the chunk's rows followed by the action rows (full attention)."""
    rng = np.random.default_rng(7)
    B, H, D, a = 16, 2, 8, 3
    history, chunk, window = 3 * B, B, 2 * B
    end = history + chunk
    video_ids = [5, 9, 2, 7]  # positions [16 i, 16 i + 16) live in block video_ids[i]
    action_ids = [11]
    k_vid = rng.standard_normal((end, H, D)).astype(np.float32)
    v_vid = rng.standard_normal((end, H, D)).astype(np.float32)
    k_act = rng.standard_normal((a, H, D)).astype(np.float32)
    v_act = rng.standard_normal((a, H, D)).astype(np.float32)
    q = rng.standard_normal((chunk + a, H, D)).astype(np.float32)
    kp = np.full((16 * B, H, D), np.nan, np.float32)
    vp = kp.copy()
    O.paged_write(kp, k_vid, O.slot_mapping(video_ids, np.arange(end), B), O.F32, O.F32)
    O.paged_write(vp, v_vid, O.slot_mapping(video_ids, np.arange(end), B), O.F32, O.F32)
    O.paged_write(kp, k_act, O.slot_mapping(action_ids, np.arange(a), B), O.F32, O.F32)
    O.paged_write(vp, v_act, O.slot_mapping(action_ids, np.arange(a), B), O.F32, O.F32)
    win = O.with_action_tokens(O.visible_window(video_ids, end, 0, window, B), action_ids, a, B)
    assert win.table == [2, 7, 11] and win.kv_len == window + a
    rows = chunk + a
    segs = O.segments_for_rows([None], [rows], [win.kv_len])
    got = O.paged_attention(q, O.F32, kp, vp, O.F32, np.array([win.table]), [0, rows], [win.kv_len], segs,
                            D ** -0.5, B)
    # the dense reference, built from the source tensors without pools or tables
    k_ref = np.concatenate([k_vid[-window:], k_act]).astype(np.float64)
    v_ref = np.concatenate([v_vid[-window:], v_act]).astype(np.float64)
    limits = np.full(rows, window + a)
    ref = O.attention_bruteforce(q.astype(np.float64), k_ref, v_ref, limits, D ** -0.5)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_action_tokens_after_a_partly_written_block_are_refused():
    """P2 ``test_action_tokens_after_a_partly_written_video_block_are_refused``:
    a 24-token chunk from an empty history ends 8 slots into its second block."""
    win = O.visible_window([4, 6], 24, 0, 48, 16)
    assert win.kv_len == 24
    with pytest.raises(ValueError, match="partly written video block"):
        O.with_action_tokens(win, [9], 3, 16)
    assert O.with_action_tokens(win, [9], 0, 16) is win  # no actions: nothing to refuse


def test_action_tokens_take_whole_scratch_blocks():
    win = O.visible_window([1, 2], 32, 0, 32, 16)
    for a, blocks in ((1, 1), (16, 1), (17, 2), (40, 3)):
        w = O.with_action_tokens(win, [8, 9, 10], a, 16)
        assert w.table == [1, 2] + [8, 9, 10][:blocks] and w.kv_len == 32 + a
        assert w.positions[32:] == [-(1 + i) for i in range(a)]


# --------------------------------------------------------------------------- staging reuse


def _decide(state, session, history, chunk, B, sink, window, max_seq_len, ids, capacity=1 << 20, actions=0, seqs=1):
    win = O.visible_window(ids, history + chunk, sink, window, B)
    return O.staging_decision(state, session, num_seqs=seqs, action_len=actions, capacity_tokens=capacity,
                              history_tokens=history, window=win, max_seq_len=max_seq_len, chunk_tokens=chunk,
                              block_size=B)


@pytest.mark.parametrize("history_chunks", [0, 1, 2, 3])
def test_staged_reuse_refreshes_the_current_blocks_at_their_live_offset(history_chunks):
    """P2 ``test_staged_reuse_refreshes_the_current_blocks_at_their_live_offset``
    with a window of two 16-token blocks and one-block chunks: the first probe
    of an AR block restages everything, the second reuses the history and
    refreshes from the visible history's block count, which is not the end of
    the padded table (capacity: 2 window blocks + 1 action-capacity block)."""
    B = 16
    ids = list(range(100, 100 + history_chunks + 1))
    state, session = O.StagingState(), object()
    max_seq_len = 3 * B
    enabled, reuse, first = _decide(state, session, history_chunks * B, B, B, 0, 2 * B, max_seq_len, ids)
    assert enabled and not reuse
    enabled, reuse, first = _decide(state, session, history_chunks * B, B, B, 0, 2 * B, max_seq_len, ids)
    assert enabled and reuse
    assert first == min(history_chunks, 1)
    assert max_seq_len // B - 1 != first


def test_ragged_chunks_never_reuse_the_staged_history():
    """P2 ``test_history_staging_holds_a_ragged_window_and_restages_it_whole``:
    24-token chunks share a block with the history's tail, so no probe reuses."""
    B, C = 16, 24
    state, session = O.StagingState(), object()
    for chunk in range(6):
        h = chunk * C
        ids = list(range(-(-(h + C) // B)))
        for _probe in range(2):
            enabled, reuse, _ = _decide(state, session, h, C, B, C, 2 * C, 8 * B, ids)
            assert enabled and not reuse


def test_staging_reuse_needs_the_same_session_and_history():
    B = 16
    ids = list(range(10))
    state = O.StagingState()
    s1, s2 = object(), object()
    assert not _decide(state, s1, 64, 32, B, 0, 96, 160, ids)[1]
    assert _decide(state, s1, 64, 32, B, 0, 96, 160, ids)[1]
    assert not _decide(state, s2, 64, 32, B, 0, 96, 160, ids)[1]  # another request
    assert not _decide(state, s2, 96, 32, B, 0, 96, 160, ids)[1]  # the history moved on
    assert not _decide(state, s2, 96, 32, B, 0, 96, 176, ids)[1]  # a different capacity
    assert _decide(state, s2, 96, 32, B, 0, 96, 176, ids)[1]
    moved = list(ids)
    moved[4] = 77  # the same length but another block in the visible history
    assert not _decide(state, s2, 96, 32, B, 0, 96, 176, moved)[1]


def test_staging_is_off_for_actions_and_batches_and_refuses_a_small_buffer():
    B = 16
    state, s = O.StagingState(), object()
    assert _decide(state, s, 32, 16, B, 0, 48, 64, list(range(4)), actions=3) == (False, False, 0)
    assert _decide(state, s, 32, 16, B, 0, 48, 64, list(range(4)), seqs=2) == (False, False, 0)
    assert state.signature is None  # the state is left alone
    with pytest.raises(RuntimeError):
        _decide(state, s, 32, 16, B, 0, 48, 64, list(range(4)), capacity=48)


# --------------------------------------------------------------------------- query shards


def _shard_case(seed=3, S=40, rows=24, Hq=4, Hkv=2, D=8):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((rows, Hq, D))
    k = rng.standard_normal((S, Hkv, D))
    v = rng.standard_normal((S, Hkv, D))
    return q, k, v


@pytest.mark.parametrize("spans", [[], [(20, 30)], [(16, 28), (30, 40)], [(0, 40)], [(25, 60)]])
def test_piecewise_attention_without_ranges_is_the_suffix_rule_by_brute_force(spans):
    q, k, v = _shard_case()
    S, rows = k.shape[0], q.shape[0]
    got = O.piecewise_attention(q, k, v, spans, 0.3)
    # limits from the rule itself: a row at g sees keys < the unclipped end of the
    # span holding it, else keys <= g
    limits = []
    for i in range(rows):
        g = S - rows + i
        holder = [b for a, b in spans if a <= g < b]
        limits.append(holder[0] if holder else g + 1)
    limits = np.minimum(np.asarray(limits), S)
    ref = O.attention_bruteforce(q, k, v, limits, 0.3)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("cuts", [(8,), (5, 17), (1, 2, 23)])
def test_query_shards_reproduce_the_rows_of_the_whole_query(cuts):
    """P3 build_segments keeps a full span's unclipped end as kv_end so that a
    local query shard attends past its own boundary: shards of a query give
    exactly the rows the whole query gives."""
    q, k, v = _shard_case(seed=11)
    S, rows = k.shape[0], q.shape[0]
    spans = [(18, 26), (30, 40)]
    whole = O.piecewise_attention(q, k, v, spans, 0.25)
    edges = [0, *cuts, rows]
    g0 = S - rows
    for a, b in zip(edges, edges[1:]):
        part = O.piecewise_attention(q[a:b], k, v, spans, 0.25, query_ranges=[(0, b - a, g0 + a)])
        np.testing.assert_allclose(part, whole[a:b], rtol=0, atol=1e-12)
    ranges = [(a, b, g0 + a) for a, b in zip(edges, edges[1:])]
    np.testing.assert_allclose(O.piecewise_attention(q, k, v, spans, 0.25, query_ranges=ranges), whole,
                               rtol=0, atol=1e-12)


def test_a_shard_in_the_middle_of_the_keys():
    """A shard whose rows are not at the end of the keys: causal rows see keys up
    to themselves, full rows up to their span's end, beyond the shard."""
    q, k, v = _shard_case(seed=5, S=50, rows=10)
    spans = [(22, 35)]
    got = O.piecewise_attention(q, k, v, spans, 0.4, query_ranges=[(0, 10, 18)])  # rows at 18..27
    limits = np.array([g + 1 if g < 22 else 35 for g in range(18, 28)])
    np.testing.assert_allclose(got, O.attention_bruteforce(q, k, v, limits, 0.4), rtol=0, atol=1e-12)


def test_query_ranges_must_cover_the_local_query_in_order():
    q, k, v = _shard_case()
    with pytest.raises(ValueError, match="contiguously"):
        O.piecewise_attention(q, k, v, [], 0.3, query_ranges=[(0, 10, 16), (12, 24, 28)])
    with pytest.raises(ValueError, match="full local query"):
        O.piecewise_attention(q, k, v, [], 0.3, query_ranges=[(0, 10, 16)])


# --------------------------------------------------------------------------- window residency model


def _kept_positions(end, sink, window):
    return set(range(min(sink, end))) | set(range(max(end - window, 0), end))


@pytest.mark.parametrize("sink_chunks,window_chunks,reset", [(1, 2, False), (0, 2, False), (1, 3, False),
                                                              (2, 2, True), (0, 2, True)])
def test_window_model_reads_every_kept_token_and_nothing_unwritten(sink_chunks, window_chunks, reset):
    """P2 ``test_attention_after_eviction_reads_every_kept_token_and_nothing_unwritten``
    with 24-token chunks against 16-token blocks: every token the window keeps
    (when it is still resident) is read, every token read was written, and
    eviction happens."""
    C, B = 24, 16
    m = O.WindowModel(B, C, sink_chunks, window_chunks, reset, chunks_per_block=2)
    evicted = False
    for _ in range(10):
        win = m.window(C)
        end = m.end + C
        read = [p for p in win.positions]
        assert all(0 <= p < end for p in read) and len(set(read)) == len(read) and read == sorted(read)
        resident = {p for p in range(end) if p // B in m.kept or p >= m.end}
        want = _kept_positions(end, m.S, m.W) & resident
        assert want <= set(read)
        # whole blocks: what is read beyond the kept tokens shares a block with one
        assert {p // B for p in read} <= {p // B for p in want}
        m.commit(C)
        evicted = evicted or len(m.kept) < -(-m.end // B)
    assert evicted


def test_window_model_reset_keeps_only_the_sink_across_a_boundary():
    """P2: the reset case keeps only the sink across a boundary, so the recent
    window reaches back over blocks that are no longer resident."""
    C, B = 32, 16  # chunks are whole blocks: no partly written tail survives the reset
    m = O.WindowModel(B, C, 1, 3, reset_at_boundary=True, chunks_per_block=2)
    m.commit(C)
    m.commit(C)  # completes an AR block
    assert m.kept == {0, 1}  # the sink's blocks
    win = m.window(C)
    assert win.positions == list(range(C)) + list(range(2 * C, 3 * C))


def test_window_model_shipped_geometry():
    """P2 ``test_the_shipped_geometry_reads_exactly_the_window_on_every_tick``:
    1560-token frames, 16-token blocks, a 9-frame sink and window, three
    frames per tick: every kept token is read, and the window stays within
    the width bound (whole blocks add at most B - 1 tokens at each of its two
    boundaries)."""
    C, B = 1560, 16
    m = O.WindowModel(B, C, 9, 9)
    filled = False
    for _ in range(12):
        win = m.window(3 * C)
        end = m.end + 3 * C
        assert _kept_positions(end, m.S, m.W) <= set(win.positions)
        assert win.kv_len <= m.S + m.W + 2 * (B - 1)
        filled = filled or end > m.S + m.W
        m.commit(3 * C)
    assert filled
    # residency is bounded by the window, not by the history
    assert len(m.kept) <= -(-m.S // B) + -(-(m.W + 3 * C) // B) + 1

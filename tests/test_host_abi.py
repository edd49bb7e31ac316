"""The C library without a GPU: it loads, exports every entry point of
include/pkv.h, and its host-side metadata (slot mapping, visible-window table,
segments, validation) agrees with the oracle bit for bit."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
from oracle import harness as H
from workloads import CONFIGS, make_workload, small_variant

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_174_amd as P

    if not os.path.exists(P._lib.LIB_PATH):
        from paged_kv_cache_174_amd.build import build

        build()
    P.lib()
    return P


def _header_functions():
    with open(os.path.join(ROOT, "include", "pkv.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol(pkv):
    declared = _header_functions()
    assert declared, "no declarations parsed"
    handle = ctypes.CDLL(pkv._lib.LIB_PATH)
    for name in declared:
        assert hasattr(handle, name), name
    assert sorted(pkv.EXPORTED) == declared
    assert pkv.pkv_version().startswith("pkv")


def test_slot_mapping_matches_oracle(pkv):
    rng = np.random.default_rng(0)
    ids = rng.permutation(800)[:400]
    for first, n in [(0, 1), (8, 24), (1560, 1560), (4680, 1560), (37, 1000)]:
        got = pkv.pkv_slot_mapping(ids, first, n, 16)
        want = O.slot_mapping(ids, np.arange(first, first + n), 16)
        assert np.array_equal(got, want)
    with pytest.raises(ValueError):
        pkv.pkv_slot_mapping(ids[:2], 0, 40, 16)
    with pytest.raises(ValueError):
        pkv.pkv_slot_mapping([-1, 2], 0, 4, 16)


@pytest.mark.parametrize("chunk,sink_chunks,window_chunks,ticks", [(24, 1, 2, 12), (24, 0, 2, 8), (1560, 1, 3, 9), (1560, 9, 9, 12), (16, 2, 2, 6)])
def test_window_table_matches_oracle(pkv, chunk, sink_chunks, window_chunks, ticks):
    rng = np.random.default_rng(chunk + sink_chunks)
    ids = rng.permutation(ticks * chunk // 16 + 8)
    for tick in range(ticks):
        h = tick * chunk
        table, kv_len = pkv.pkv_window_table(ids, h, chunk, sink_chunks * chunk, window_chunks * chunk, 16)
        want = O.visible_window(ids, h + chunk, sink_chunks * chunk, window_chunks * chunk, 16)
        assert list(table) == want.table and kv_len == want.kv_len


def test_window_table_skips_evicted_blocks_like_the_oracle(pkv):
    ids = np.arange(100, 140)
    ids[10:20] = -1  # evicted gap between sink and window
    table, kv_len = pkv.pkv_window_table(ids, 600, 24, 48, 72, 16)
    want = O.visible_window(ids, 624, 48, 72, 16)
    assert list(table) == want.table and kv_len == want.kv_len


def test_window_table_errors(pkv):
    ids = np.arange(10)
    with pytest.raises(ValueError):
        pkv.pkv_window_table(ids, 0, 24, 0, 16, 16)  # window smaller than the chunk
    with pytest.raises(ValueError):
        pkv.pkv_window_table(ids[:1], 0, 40, 0, 40, 16)  # too few block ids


def test_window_capacity_worked_example(pkv):
    """P1 max_video_blocks' own case: at 1560 tokens per frame a 9-frame sink and
    a 9-frame window are each 8 tokens past a block edge, 28080 tokens
    together: rounding the sum once (1755 blocks) is a block short, rounding
    each range on its own gives 878 + 878.  One action block comes on top even
    without actions (P1 build_block_table)."""
    assert pkv.pkv_window_capacity(9 * 1560, 9 * 1560, 1560, 16, 0) == 878 + 878 + 1
    assert -(-(18 * 1560) // 16) == 1755
    assert pkv.pkv_window_capacity(1560, 4680, 1560, 16, 0) == 98 + 293 + 1  # the frame workload: 392 blocks
    assert pkv.pkv_window_capacity(0, 64, 32, 16, 40) == 0 + 4 + 3  # whole-block chunks never straddle
    with pytest.raises(ValueError):
        pkv.pkv_window_capacity(0, 64, 0, 16)


@pytest.mark.parametrize("chunk,sink_chunks,window_chunks", [(1560, 1, 3), (24, 1, 2), (40, 2, 3), (7, 3, 5), (48, 0, 4), (30, 1, 1)])
def test_window_capacity_bounds_every_tick_and_is_reached(pkv, chunk, sink_chunks, window_chunks):
    """Brute force over AR ticks: the blocks holding a kept position (the sink,
    and the recent window ending at the chunk's end, which sits on a whole
    number of chunks) never outnumber the capacity's video part, and some tick
    needs all of it once the recent range has slid past the sink."""
    B, S, W = 16, sink_chunks * chunk, window_chunks * chunk
    video_cap = pkv.pkv_window_capacity(S, W, chunk, B, 0) - 1
    most = 0
    for tick in range(64):
        end = (tick + 1) * chunk
        kept = set(range(min(S, end))) | set(range(max(0, end - W), end))
        most = max(most, len({p // B for p in kept}))
    assert most == video_cap


def test_fixed_capacity_plan_needs_a_bounded_window(pkv):
    """P1's fixed-shape metadata: width and max_seq_len from the window's
    capacity; a window that keeps everything has no capacity to pad to."""
    geom = CONFIGS["frame_bf16"]
    wl = make_workload(geom, device="cpu")
    plan = pkv.ForwardPlan.build(wl.block_ids, geom.history_lens, geom.query_lens, geom.sink_tokens,
                                 geom.window_tokens, geom.full_spans, geom.causal_default, geom.block_size,
                                 fixed_capacity=True)
    assert plan.block_table_host.shape == (2, 392) and plan.max_seq_len == 392 * 16 and plan.kv_lens == [6240, 6240]
    assert (plan.block_table_host[:, 390:] == 0).all()  # tail padding with block 0, never read
    big = small_variant(geom, name="unbounded", window_tokens=(1 << 30, 1 << 30), sink_tokens=(0, 0))
    wl = make_workload(big, device="cpu")
    with pytest.raises(ValueError, match="bounded window"):
        pkv.ForwardPlan.build(wl.block_ids, big.history_lens, big.query_lens, big.sink_tokens, big.window_tokens,
                              big.full_spans, big.causal_default, big.block_size, fixed_capacity=True)


def _attn_on_fake_pointers(pkv, num_seqs, q_len, hq, hkv, max_seq_len, host=None, workspace_bytes=1 << 40):
    """pkv_paged_attn with placeholder device pointers: the host checks and the
    split planner run, and a call they refuse returns before any launch."""
    lib = pkv.lib()
    pools = pkv._lib._Pools(key=16, value=16, num_blocks=1 << 22, block_size=16, num_kv_heads=hkv, head_dim=128,
                             dtype=pkv.PKV_BF16, k_scale=1.0, v_scale=1.0, k_inv_scale=1.0, v_inv_scale=1.0)
    hl = (ctypes.c_int32 * num_seqs)(*host) if host else None
    p = ctypes.c_void_p(16)
    return lib.pkv_paged_attn(p, pkv.PKV_BF16, num_seqs * q_len, hq, ctypes.byref(pools), p, (max_seq_len + 15) // 16,
                              p, p, num_seqs, q_len, max_seq_len, p, p, None, hl, 0.088, p, p, workspace_bytes, None)


def test_more_key_splits_than_the_kernels_take_are_refused_before_launch(pkv):
    """A key range needing more than 16 splits of one workgroup's table slice
    (4095 blocks) is refused on the host even with a workspace for them."""
    split_keys = 4095 * 16
    assert _attn_on_fake_pointers(pkv, 1, 64, 2, 2, 16 * split_keys + 16) == pkv._lib.PKV_EUNSUPPORTED
    assert "16 key splits" in pkv.pkv_last_error()


@pytest.mark.parametrize("num_seqs,q_len,hq,hkv,max_seq_len,host", [
    (2, 1560, 12, 12, 6272, [6240, 6240]), (2, 1560, 40, 40, 9392, [9360, 9360]), (1, 4680, 40, 8, 6240, None),
    (3, 700, 8, 2, 200000, [150000, 90000, 3000]), (2, 300, 4, 4, 70000, None), (1, 2000, 4, 1, 1000000, None)])
def test_long_split_plans_cover_the_keys(pkv, num_seqs, q_len, hq, hkv, max_seq_len, host):
    """The long bf16 kernel's split plan: cuts on 64-key tiles from 0, split
    lengths that never increase, no split longer than one table slice, and the
    last split running on to max_seq_len.  (Read from the plan string of a call
    whose launch fails: CPU only, it would launch on a GPU.)"""
    import torch

    if torch.cuda.device_count() > 0:
        pytest.skip("the call would launch on placeholder pointers")
    rc = _attn_on_fake_pointers(pkv, num_seqs, q_len, hq, hkv, max_seq_len, host)
    assert rc == pkv._lib.PKV_EHIP  # the checks and the plan passed; only the launch failed
    plan = pkv.pkv_last_attn_plan()
    fields = dict(f.split("=") for f in plan.split()[1:])
    assert plan.startswith("long ")
    splits = int(fields["splits"])
    cuts = [0] + ([int(c) for c in fields["cut"].split(",")] if splits > 1 else []) + [max_seq_len]
    assert len(cuts) == splits + 1 and all(c % 64 == 0 for c in cuts[:-1])
    lens = [b - a for a, b in zip(cuts, cuts[1:])]
    assert all(x > 0 for x in lens) and all(x <= 4095 * 16 for x in lens)
    assert all(a >= b for a, b in zip(lens[:-2], lens[1:-1]))  # the last one also runs on past the plan


def test_segments_match_oracle(pkv):
    rng = np.random.default_rng(11)
    for _ in range(300):
        s = int(rng.integers(1, 80))
        q = int(rng.integers(1, s + 1))
        cuts = sorted(set(rng.integers(0, s + 1, size=int(rng.integers(0, 8))).tolist()))
        spans = [(cuts[i], cuts[i + 1]) for i in range(0, len(cuts) - 1, 2) if cuts[i] < cuts[i + 1]]
        if rng.random() < 0.3 and len(spans) >= 2:  # make two spans touch
            spans[1] = (spans[0][1], spans[1][1])
        got = pkv.pkv_build_segments(spans, s - q, q)
        want = O.build_segments(spans, s - q, q)
        assert [tuple(r) for r in got.tolist()] == [
            (g.q_start, g.q_end, g.kv_end, 1 if g.mode == "full" else 0) for g in want
        ]
    with pytest.raises(ValueError):
        pkv.pkv_build_segments([(5, 3)], 0, 10)
    with pytest.raises(ValueError):
        pkv.pkv_build_segments([(0, 5), (4, 8)], 0, 10)


@pytest.mark.parametrize("name", ["tiny_f32", "frame_bf16", "piecewise_gqa_bf16", "varlen_fp8", "ar_step_40L_bf16"])
def test_forward_plan_matches_oracle_metadata(pkv, name):
    geom = CONFIGS[name]
    wl = make_workload(geom)
    plan = pkv.ForwardPlan.build(
        wl.block_ids, geom.history_lens, geom.query_lens, geom.sink_tokens, geom.window_tokens,
        geom.full_spans, geom.causal_default, geom.block_size,
    )
    meta = H.metadata(wl)
    assert np.array_equal(plan.block_table_host, meta.block_table)
    assert plan.kv_lens == meta.kv_lens
    assert np.array_equal(plan.query_start_host, meta.query_start_loc)
    assert np.array_equal(plan.cur_slots_host, np.concatenate(meta.cur_slots))
    assert np.array_equal(plan.hist_slots_host, np.concatenate(meta.hist_slots))
    flat = [(g.q_start, g.q_end, g.kv_end, 1 if g.mode == "full" else 0) for segs in meta.segments for g in segs]
    assert [tuple(r) for r in plan.segments_host.tolist()] == flat
    plan.validate(geom.pool_blocks())


def test_validate_metadata_rejects_what_the_pages_reject(pkv):
    geom = small_variant(CONFIGS["piecewise_gqa_bf16"], history_lens=(40,), query_lens=(60,),
                         full_spans=(((40, 60), (80, 100)),))
    wl = make_workload(geom)
    plan = pkv.ForwardPlan.build(wl.block_ids, geom.history_lens, geom.query_lens, geom.sink_tokens,
                                 geom.window_tokens, geom.full_spans, geom.causal_default)
    nb = geom.pool_blocks()
    plan.validate(nb)
    args = dict(query_start_loc=plan.query_start_host, seq_lens=np.asarray(plan.kv_lens, np.int32),
                block_table=plan.block_table_host, num_blocks=nb, block_size=16,
                max_query_len=plan.max_query_len, max_seq_len=plan.max_seq_len,
                segments=plan.segments_host, segment_start_loc=plan.segment_start_host)

    def bad(**kw):
        a = dict(args)
        a.update(kw)
        with pytest.raises(ValueError):
            pkv.pkv_validate_metadata_host(**a)

    bad(seq_lens=np.asarray([59], np.int32))  # shorter than the query
    bad(max_seq_len=50)
    bad(max_query_len=10)
    bad(num_blocks=1)
    seg = plan.segments_host.copy()
    seg[1, 2] += 1  # causal kv_end != q_end
    bad(segments=seg)
    seg = plan.segments_host.copy()
    seg[0, 2] = 200  # full kv_end past seq_len
    bad(segments=seg)
    seg = plan.segments_host.copy()
    seg[1, 0] += 1  # gap in the tiling
    bad(segments=seg)


def test_validate_metadata_rejects_decreasing_row_limits(pkv):
    """The kernels bound a row tile's keys by its last row's limit and skip
    the mask below a wave's first row's, so a segment list whose per-row key
    limit L(g) drops from one row to the next must be refused (P3's
    build_segments never makes one: a full segment reaches past its q_end
    only as the last segment)."""
    F, C = 1, 0

    def check(seq_len, q_len, segs, query_pos=None, ok=False):
        nb = (seq_len + 15) // 16
        kw = dict(query_start_loc=np.array([0, q_len], np.int32), seq_lens=np.array([seq_len], np.int32),
                  block_table=np.arange(nb, dtype=np.int32)[None, :], num_blocks=nb, block_size=16,
                  max_query_len=q_len, max_seq_len=seq_len, segments=np.array(segs, np.int32),
                  segment_start_loc=np.array([0, len(segs)], np.int32),
                  query_pos=None if query_pos is None else np.array([query_pos], np.int32))
        if ok:
            pkv.pkv_validate_metadata_host(**kw)
        else:
            with pytest.raises(ValueError, match="decrease"):
                pkv.pkv_validate_metadata_host(**kw)

    # full rows see 600 keys, the causal rows after them 11 .. 600
    check(600, 600, [(0, 10, 600, F), (10, 600, 600, C)])
    # a shard [100, 200) of 300 keys: full rows see 300, the causal rows 151 .. 200
    check(300, 100, [(100, 150, 300, F), (150, 200, 200, C)], query_pos=100)
    # two full segments with falling kv_end
    check(300, 300, [(0, 100, 250, F), (100, 300, 300, C)])
    # allowed: equal limits across the boundary, and a last full segment reaching past the query
    check(300, 300, [(0, 10, 11, F), (10, 300, 300, C)], ok=True)
    check(300, 100, [(100, 150, 150, C), (150, 200, 300, F)], query_pos=100, ok=True)


# --------------------------------------------------------------------------- action tokens and staging reuse


def _action_geom(pool="bf16", actions=(3, 17), name="actions"):
    """Two sequences whose windows end on a block edge, with action tokens."""
    base = CONFIGS["frame_bf16"] if pool == "bf16" else CONFIGS["tiny_f32"]
    n = len(actions)
    return small_variant(
        base, name=name, num_q_heads=4, num_kv_heads=2 if pool == "bf16" else 4,
        history_lens=(64, 96)[:n], query_lens=(32, 48)[:n], sink_tokens=(16, 0)[:n],
        window_tokens=(64, 1 << 30)[:n], full_spans=(None,) * n, action_lens=tuple(actions),
    )


def test_action_table_matches_oracle(pkv):
    rng = np.random.default_rng(5)
    for _ in range(200):
        chunk = int(rng.choice([16, 24, 32, 48]))
        ticks = int(rng.integers(1, 6))
        ids = rng.permutation(64)[: ticks * 4 + 4]
        h = (ticks - 1) * chunk
        a = int(rng.integers(0, 40))
        act_ids = rng.permutation(np.arange(100, 110))
        table, kv_len = pkv.pkv_window_table(ids, h, chunk, chunk, 2 * chunk, 16)
        win = O.visible_window(ids, h + chunk, chunk, 2 * chunk, 16)
        try:
            want = O.with_action_tokens(win, act_ids, a, 16)
        except ValueError:
            with pytest.raises(ValueError, match="partly written video block"):
                pkv.pkv_action_table(table, kv_len, act_ids, a, 16)
            continue
        got_table, got_len = pkv.pkv_action_table(table, kv_len, act_ids, a, 16)
        assert list(got_table) == want.table and got_len == want.kv_len


def test_action_table_errors(pkv):
    with pytest.raises(ValueError):
        pkv.pkv_action_table([1, 2], 32, [7], 20, 16)  # 20 action tokens need 2 scratch blocks
    with pytest.raises(ValueError):
        pkv.pkv_action_table([1, 2], 32, [-3], 2, 16)


@pytest.mark.parametrize("actions", [(3, 17), (16, 0)])
def test_forward_plan_with_actions_matches_oracle_metadata(pkv, actions):
    geom = _action_geom(actions=actions)
    wl = make_workload(geom)
    plan = pkv.ForwardPlan.build(
        wl.block_ids, geom.history_lens, geom.query_lens, geom.sink_tokens, geom.window_tokens,
        geom.full_spans, geom.causal_default, geom.block_size,
        action_lens=geom.action_lens, action_block_ids=wl.action_block_ids,
    )
    meta = H.metadata(wl)
    assert np.array_equal(plan.block_table_host, meta.block_table)
    assert plan.kv_lens == meta.kv_lens
    assert np.array_equal(plan.query_start_host, meta.query_start_loc)
    assert np.array_equal(plan.cur_slots_host, np.concatenate(meta.cur_slots))
    assert np.array_equal(plan.act_slots_host, np.concatenate(meta.act_slots))
    flat = [(g.q_start, g.q_end, g.kv_end, 1 if g.mode == "full" else 0) for segs in meta.segments for g in segs]
    assert [tuple(r) for r in plan.segments_host.tolist()] == flat
    plan.validate(geom.pool_blocks())


def test_forward_plan_refuses_actions_after_a_partly_written_block(pkv):
    with pytest.raises(ValueError, match="partly written video block"):
        pkv.ForwardPlan.build([np.array([4, 6])], [0], [24], [0], [48], [None], action_lens=[3],
                              action_block_ids=[np.array([9])])


def _tick_events(seed):
    """A random run of forwards: AR blocks of 1-3 probes, sessions that change,
    chunk sizes that are or are not whole blocks, windows that slide."""
    rng = np.random.default_rng(seed)
    chunk = int(rng.choice([16, 24, 32]))
    sink = int(rng.choice([0, chunk]))
    window = int(rng.choice([2, 3])) * chunk
    sessions = [object(), object()]
    cap_blocks = -(-sink // 16) + -(-window // 16) + 2
    ids = rng.permutation(200)
    h = 0
    events = []
    for _ in range(10):
        session = sessions[int(rng.integers(0, 2))] if rng.random() < 0.3 else sessions[0]
        for _probe in range(int(rng.integers(1, 4))):
            events.append((session, h, chunk, sink, window, cap_blocks * 16, ids))
        h += chunk
    return events


@pytest.mark.parametrize("seed", range(8))
def test_history_staging_decisions_match_oracle(pkv, seed):
    product = pkv.HistoryStaging(capacity_tokens=1 << 20)
    state = O.StagingState()
    reused = 0
    for session, h, chunk, sink, window, max_seq_len, ids in _tick_events(seed):
        plan = pkv.ForwardPlan.build([ids], [h], [chunk], [sink], [window], [None], max_seq_len=max_seq_len,
                                     table_width=max_seq_len // 16)
        got = product.decide(session, plan)
        win = O.visible_window(ids, h + chunk, sink, window, 16)
        want = O.staging_decision(state, session, num_seqs=1, action_len=0, capacity_tokens=1 << 20,
                                  history_tokens=h, window=win, max_seq_len=max_seq_len, chunk_tokens=chunk,
                                  block_size=16)
        assert (got.enabled, got.reuse, got.first_block) == want
        reused += got.reuse
    assert reused > 0 or _tick_events(seed)[0][2] % 16  # aligned runs must reuse somewhere


def test_staging_decide_c_abi(pkv):
    """pkv_staging_decide on its own: reuse needs the same session id, history,
    extent and chunk length and a chunk of whole blocks; without reuse
    first_block is 0; a refused call leaves the state as it was."""
    from paged_kv_cache_174_amd import _lib as L

    st = L.StagingState(8)
    table = [5, 6, 7, 9]  # three history blocks, then the chunk's block
    assert L.pkv_staging_decide(st, 1, table, 48, 16, 64, 16, 64) == (False, 0)
    assert L.pkv_staging_decide(st, 1, table, 48, 16, 64, 16, 64) == (True, 3)
    assert L.pkv_staging_decide(st, 2, table, 48, 16, 64, 16, 64) == (False, 0)  # another request
    assert L.pkv_staging_decide(st, 2, [5, 6, 8, 9], 48, 16, 64, 16, 64) == (False, 0)  # a history block moved
    with pytest.raises(RuntimeError):
        L.pkv_staging_decide(st, 2, [5, 6, 8, 9], 48, 16, 80, 16, 64)  # extent past the buffers
    assert L.pkv_staging_decide(st, 2, [5, 6, 8, 9], 48, 16, 64, 16, 64) == (True, 3)  # state kept
    # a chunk that shares its first block with the history never reuses
    assert L.pkv_staging_decide(st, 3, [5, 6, 7], 40, 8, 48, 16, 64) == (False, 0)
    assert L.pkv_staging_decide(st, 3, [5, 6, 7], 40, 8, 48, 16, 64) == (False, 0)
    with pytest.raises(ValueError):
        L.pkv_staging_decide(st, 3, [5], 40, 40, 48, 16, 64)  # the table cannot hold the chunk


def test_history_staging_is_off_for_actions_and_batches(pkv):
    st = pkv.HistoryStaging(capacity_tokens=1024)
    geom = _action_geom()
    wl = make_workload(geom)
    plan = pkv.ForwardPlan.build(wl.block_ids, geom.history_lens, geom.query_lens, geom.sink_tokens,
                                 geom.window_tokens, geom.full_spans, action_lens=geom.action_lens,
                                 action_block_ids=wl.action_block_ids)
    d = st.decide(object(), plan)
    assert (d.enabled, d.reuse, d.first_block) == (False, False, 0)
    small = pkv.HistoryStaging(capacity_tokens=16)
    one = pkv.ForwardPlan.build([np.arange(8)], [32], [16], [0], [48], [None])
    with pytest.raises(RuntimeError):
        small.decide(object(), one)


# --------------------------------------------------------------------------- query shards


def test_sharded_plan_matches_the_oracle_segments(pkv):
    geom = small_variant(CONFIGS["piecewise_gqa_bf16"], history_lens=(100, 40), query_lens=(300, 60),
                         sink_tokens=(0, 0), window_tokens=(1 << 30,) * 2,
                         full_spans=(((100, 180), (250, 400)), None))
    wl = make_workload(geom)
    plan = pkv.ForwardPlan.build(wl.block_ids, geom.history_lens, geom.query_lens, geom.sink_tokens,
                                 geom.window_tokens, geom.full_spans)
    ranges = [[(0, 90, 150), (90, 200, 240)], [(0, 0, 5), (0, 30, 70)]]
    sh = plan.shard(ranges)
    sh.validate(geom.pool_blocks())
    assert sh.num_seqs == 3 and list(sh.entry_seq) == [0, 0, 1]
    assert list(sh.query_pos_host) == [150, 240, 70] and sh.query_lens == [90, 110, 30]
    spans = [[(100, 180), (250, 400)], [(40, 100)]]  # sequence 1: the AR default, its whole chunk
    want = []
    for (_, n, g0), b in zip([(0, 90, 150), (0, 110, 240), (0, 30, 70)], [0, 0, 1]):
        want += [(s.q_start, s.q_end, s.kv_end, 1 if s.mode == "full" else 0) for s in O.build_segments(spans[b], g0, n)]
    assert [tuple(r) for r in sh.segments_host.tolist()] == want
    assert np.array_equal(sh.block_table_host[1], plan.block_table_host[0])


def test_shards_are_checked_like_the_pages_check_them(pkv):
    plan = pkv.ForwardPlan.build([np.arange(10)], [64], [32], [0], [1 << 30], [None])
    with pytest.raises(ValueError, match="contiguously"):
        plan.shard([[(0, 10, 64), (12, 32, 76)]])
    with pytest.raises(ValueError, match="outside"):
        plan.shard([[(0, 32, 80)]])
    bad = plan.shard([[(0, 32, 64)]])
    with pytest.raises(ValueError):  # the query rows must lie inside the keys
        pkv.pkv_validate_metadata_host(bad.query_start_host, bad.kv_lens, bad.block_table_host, 10, 16,
                                       bad.max_query_len, bad.max_seq_len, bad.segments_host,
                                       bad.segment_start_host, query_pos=[70])


def test_probe_entry_points_check_their_arguments(pkv):
    """The measured-peak probes refuse null pointers and sizes out of range
    before touching a device (no GPU needed)."""
    lib = pkv.lib()
    flop = ctypes.c_int64(0)
    assert lib.pkv_probe_mfma(0, ctypes.c_void_p(16), 1 << 20, ctypes.byref(flop), None) == pkv._lib.PKV_EINVAL
    assert lib.pkv_probe_mfma(10, None, 1 << 20, ctypes.byref(flop), None) == pkv._lib.PKV_EINVAL
    assert lib.pkv_probe_mfma(10, ctypes.c_void_p(16), 1 << 20, None, None) == pkv._lib.PKV_EINVAL
    assert "pkv_probe_mfma" in pkv.pkv_last_error()
    assert lib.pkv_probe_stream(None, 1 << 20, ctypes.c_void_p(16), None) == pkv._lib.PKV_EINVAL
    assert lib.pkv_probe_stream(ctypes.c_void_p(16), 15, ctypes.c_void_p(16), None) == pkv._lib.PKV_EINVAL
    assert lib.pkv_probe_stream(ctypes.c_void_p(16), 1 << 20, None, None) == pkv._lib.PKV_EINVAL
    assert "pkv_probe_stream" in pkv.pkv_last_error()


def test_last_attn_plan_is_empty_before_any_attention_call(pkv):
    """The plan diagnostic is a thread-local string; on a thread that made no
    attention call it is empty."""
    import threading

    seen = []
    t = threading.Thread(target=lambda: seen.append(pkv.pkv_last_attn_plan()))
    t.start()
    t.join()
    assert seen == [""]

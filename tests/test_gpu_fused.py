"""The fused per-layer call (P1 ``_paged_write_attn_impl``) on the GPU.

pkv_paged_write_attn writes the current video K/V and the action K/V through
their slot mappings, optionally stages the visible window into caller-owned
buffers (full, or from the first current block when the history is reused),
and attends.  Checked against the float64 oracle: pools and staging buffers
bit for bit, outputs within the dtype's bound (1e-4 fp32, 2e-2 bf16, 6e-2 fp8
K/V), and, captured once in a HIP graph, over several AR ticks whose metadata
changes in place.
Pages cited by tag and function: P1 "vllm_omni/experimental/ar_diffusion/kv_cache/paged_attention.py",
P2 "tests/diffusion/ar_diffusion/test_paged_attention.py".
"""

import numpy as np
import pytest
import torch

import oracle as O
from oracle import harness as H
from workloads import CONFIGS, make_workload, small_variant
from workloads.configs import Workload

from . import gpu_harness as G

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    G.ensure_built()


def _err(geom, out, ref):
    got = G.as_f64(out)
    assert np.isfinite(got).all(), "non-finite output (an unwritten slot was read?)"
    err = float(np.max(np.abs(got - ref)))
    assert err <= TOL[geom.pool_dtype], f"{geom.name}: max abs error {err:.3e}"
    return err


FUSED = [
    CONFIGS["tiny_f32"],
    small_variant(CONFIGS["tiny_f32"], name="f32_actions", history_lens=(32,), query_lens=(16,),
                  action_lens=(3,)),
    small_variant(CONFIGS["frame_bf16"], name="bf16_actions", num_q_heads=4, num_kv_heads=2,
                  history_lens=(64, 96), query_lens=(32, 48), sink_tokens=(16, 0), window_tokens=(64, 1 << 30),
                  action_lens=(3, 17)),
    small_variant(CONFIGS["frame_bf16"], name="bf16_ragged_window", num_q_heads=3, num_kv_heads=3,
                  history_lens=(600, 600), query_lens=(300, 300), sink_tokens=(300, 300),
                  window_tokens=(900, 900)),
    small_variant(CONFIGS["piecewise_gqa_bf16"], name="piecewise_small", num_q_heads=10, num_kv_heads=2,
                  history_lens=(100,), query_lens=(300,), full_spans=(((100, 180), (250, 400)),)),
    small_variant(CONFIGS["varlen_fp8"], name="fp8_actions", num_q_heads=8, num_kv_heads=2,
                  history_lens=(112, 1984, 0), query_lens=(16, 64, 32), sink_tokens=(0,) * 3,
                  window_tokens=(1 << 30,) * 3, full_spans=(None,) * 3, causal_default=False,
                  action_lens=(5, 40, 16)),
]


@pytest.mark.parametrize("geom", FUSED, ids=[g.name for g in FUSED])
def test_fused_call_matches_oracle(geom):
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    plan = G.make_plan(wl)
    pools = G.make_pools(geom, li)
    G.say("fused", geom.name)
    if li.k_hist.shape[0]:
        G.P.pkv_paged_write(li.k_hist, li.v_hist, plan.history_slot_mapping, pools)
    out = G.write_attend(plan, pools, li, geom)
    torch.cuda.synchronize()
    _, k_ref, v_ref, ref = H.run_layer(wl, li=li)
    assert G.bits_equal(pools.key, k_ref) and G.bits_equal(pools.value, v_ref)
    _err(geom, out, ref)


CAPACITY = [
    small_variant(CONFIGS["frame_bf16"], name="bf16_actions_windowed", num_q_heads=4, num_kv_heads=2,
                  history_lens=(64, 96), query_lens=(32, 48), sink_tokens=(16, 0), window_tokens=(64, 144),
                  action_lens=(3, 17)),
    FUSED[3],
]


@pytest.mark.parametrize("geom", CAPACITY, ids=[g.name for g in CAPACITY])
def test_fused_call_with_fixed_capacity_metadata(geom):
    """P1 build_block_table's fixed-shape metadata: the table padded with block
    0 to the window's capacity and max_seq_len that capacity, larger than
    every sequence; the kernels read only ceil(seq_len / 16) entries and the
    planner works from the real lengths, so the result is the oracle's."""
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    plan = G.make_plan(wl, fixed_capacity=True)
    width = plan.block_table.shape[1]
    assert plan.max_seq_len == 16 * width > max(plan.kv_lens) and min(len(t) for t in plan.tables) < width
    pools = G.make_pools(geom, li)
    G.say("fused fixed capacity", geom.name)
    if li.k_hist.shape[0]:
        G.P.pkv_paged_write(li.k_hist, li.v_hist, plan.history_slot_mapping, pools)
    out = G.write_attend(plan, pools, li, geom)
    torch.cuda.synchronize()
    _, k_ref, v_ref, ref = H.run_layer(wl, li=li)
    assert G.bits_equal(pools.key, k_ref) and G.bits_equal(pools.value, v_ref)
    _err(geom, out, ref)


def test_fused_call_equals_the_separate_calls():
    geom = FUSED[2]
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    plan = G.make_plan(wl)
    G.say("fused vs separate", geom.name)
    p1, p2 = G.make_pools(geom, li), G.make_pools(geom, li)
    G.P.pkv_paged_write(li.k_hist, li.v_hist, plan.history_slot_mapping, p1)
    G.P.pkv_paged_write(li.k_hist, li.v_hist, plan.history_slot_mapping, p2)
    fused = G.write_attend(plan, p1, li, geom)
    G.write_layer(plan, p2, li)  # history again (same bits), current, actions
    sep = G.attend(plan, p2, li, geom)
    torch.cuda.synchronize()
    assert torch.equal(p1.key.view(torch.int16), p2.key.view(torch.int16))
    assert torch.equal(fused.view(torch.int16), sep.view(torch.int16))


def test_fused_call_checks_everything_before_enqueueing():
    geom = FUSED[2]
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    plan = G.make_plan(wl)
    pools = G.make_pools(geom, li)
    before = pools.key.clone()
    G.say("fused bad args", geom.name)
    with pytest.raises(ValueError):  # staging covers one sequence
        stage = torch.zeros((plan.max_seq_len + 64, geom.num_kv_heads, geom.head_dim), dtype=torch.bfloat16,
                            device="cuda")
        G.write_attend(plan, pools, li, geom, stage_key=stage, stage_value=stage.clone())
    with pytest.raises(ValueError):  # q dtype does not go with the pool
        G.P.pkv_paged_write_attn(li.q.float(), li.k_cur, li.v_cur, plan.slot_mapping, pools, plan, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(before.view(torch.int16), pools.key.view(torch.int16)), "a refused call wrote the pools"


# --------------------------------------------------------------------------- staging


def _staged_geom(pool="bf16", chunk=64):
    base = CONFIGS["frame_bf16"] if pool == "bf16" else CONFIGS["tiny_f32"]
    return small_variant(base, name=f"staged_{pool}", num_q_heads=4, num_kv_heads=2 if pool == "bf16" else 4,
                         history_lens=(3 * chunk,), query_lens=(chunk,), sink_tokens=(chunk,),
                         window_tokens=(3 * chunk,), full_spans=(None,))


def _padded(meta, n_blocks):
    """The oracle's table of sequence 0, padded with block 0 to n_blocks entries
    (P1 build_block_table pads to a fixed width with block 0)."""
    t = np.zeros(n_blocks, dtype=np.int64)
    t[: len(meta.tables[0])] = meta.tables[0]
    return t


SENTINEL = -7.0  # P2 fills the staging buffers with -7 and checks the rows past the window keep it


@pytest.mark.parametrize("pool", ["bf16", "f32"])
def test_staged_fused_call_restages_then_reuses(pool):
    """P2 ``test_staged_reuse_refreshes_the_current_blocks_at_their_live_offset``
    on the GPU: probe 1 of an AR block gathers the whole window, probe 2 (new
    current K/V, same history) only its current blocks; both staging buffers
    equal the oracle's full gather, rows past the window keep the sentinel,
    and attention over them matches the oracle."""
    geom = _staged_geom(pool)
    B = geom.block_size
    wl = make_workload(geom, device="cuda")
    cap_blocks = -(-geom.sink_tokens[0] // B) + -(-geom.window_tokens[0] // B) + 1  # + one action block
    plan = G.make_plan(wl, fixed_capacity=True)  # P1 build_block_table's fixed shape (whole-block chunks)
    assert plan.block_table.shape[1] == cap_blocks and plan.max_seq_len == cap_blocks * B
    n_blocks = plan.max_seq_len // B
    dt = G.TORCH_DT[pool]
    shape = (plan.max_seq_len + 2 * B, geom.num_kv_heads, geom.head_dim)
    sk = torch.full(shape, SENTINEL, dtype=dt, device="cuda")
    sv = torch.full(shape, SENTINEL, dtype=dt, device="cuda")
    staging = G.P.HistoryStaging(capacity_tokens=shape[0])
    session = object()
    li0 = wl.layer(0)
    pools = G.make_pools(geom, li0)
    G.P.pkv_paged_write(li0.k_hist, li0.v_hist, plan.history_slot_mapping, pools)
    meta = H.metadata(wl)
    table = _padded(meta, n_blocks)
    k_ref, v_ref = H.empty_pool(geom), H.empty_pool(geom)
    H.write_history(geom, meta, li0, k_ref, v_ref)
    for probe in range(2):
        li = wl.layer(probe)  # same history, new current K/V and queries
        li.k_hist, li.v_hist = li0.k_hist, li0.v_hist
        d = staging.decide(session, plan)
        assert d.enabled and d.reuse == (probe == 1)
        assert d.first_block == (plan.kv_lens[0] // B - geom.query_lens[0] // B if d.reuse else 0)
        G.say("staged", pool, "probe", probe, "first_block", d.first_block)
        out = G.write_attend(plan, pools, li, geom, stage_key=sk, stage_value=sv,
                             first_block=d.first_block)
        torch.cuda.synchronize()
        H.write_current(geom, meta, li, k_ref, v_ref)
        want_k = np.full((shape[0],) + k_ref.shape[1:], 0, dtype=k_ref.dtype)
        want_v = want_k.copy()
        O.gather(k_ref, table, n_blocks, 0, want_k, B)
        O.gather(v_ref, table, n_blocks, 0, want_v, B)
        rows = plan.max_seq_len
        assert G.bits_equal(sk[:rows], want_k[:rows]) and G.bits_equal(sv[:rows], want_v[:rows])
        assert (sk[rows:].float() == SENTINEL).all() and (sv[rows:].float() == SENTINEL).all()
        ref = H.attention(geom, meta, li, k_ref, v_ref)
        _err(geom, out, ref)
    # A reusing call touches only block rows [first_block, n_blocks).
    first = d.first_block
    sk[: first * B] = 123.0
    li = wl.layer(2)
    li.k_hist, li.v_hist = li0.k_hist, li0.v_hist
    G.say("staged", pool, "reuse leaves the history rows alone")
    G.write_attend(plan, pools, li, geom, stage_key=sk, stage_value=sv, first_block=first)
    torch.cuda.synchronize()
    assert (sk[: first * B].float() == 123.0).all()
    H.write_current(geom, meta, li, k_ref, v_ref)
    want_k = np.zeros((n_blocks * B,) + k_ref.shape[1:], dtype=k_ref.dtype)
    O.gather(k_ref, table, n_blocks, 0, want_k, B)
    assert G.bits_equal(sk[first * B: n_blocks * B], want_k[first * B:])


def test_staged_reuse_refuses_a_ragged_chunk():
    geom = _staged_geom("bf16", chunk=24)
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    plan = G.make_plan(wl, table_width=16, max_seq_len=256)
    pools = G.make_pools(geom, li)
    stage = torch.zeros((256, geom.num_kv_heads, geom.head_dim), dtype=torch.bfloat16, device="cuda")
    G.say("staged ragged refusal")
    with pytest.raises(ValueError, match="block-aligned"):
        G.write_attend(plan, pools, li, geom, stage_key=stage, stage_value=stage.clone(), first_block=2)


# --------------------------------------------------------------------------- HIP graph


def _ticks_geometry(pool, seqs, chunk, sink, window, heads, kv_heads):
    base = CONFIGS["frame_bf16"] if pool == "bf16" else CONFIGS["varlen_fp8"]
    return small_variant(base, name=f"graph_{pool}", pool_dtype=pool, num_q_heads=heads, num_kv_heads=kv_heads,
                         history_lens=(0,) * seqs, query_lens=(chunk,) * seqs, sink_tokens=(sink,) * seqs,
                         window_tokens=(window,) * seqs, full_spans=(None,) * seqs, causal_default=False)


def _draw(shape, seed, dtype):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    return torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(dtype)


@pytest.mark.parametrize("pool", ["bf16", "fp8"])
def test_fused_call_replays_in_a_hip_graph_across_ticks(pool):
    """Capture the fused call once, then replay it for successive AR ticks of
    two sequences: each tick copies its queries, K/V, slot mapping, block
    table and lengths into the captured tensors (fixed table width and
    max_seq_len, P1 build_block_table), the window grows and then slides, and
    the keys are split (the merge is in the graph too).  Every replay equals an
    eager call bit for bit and the oracle within the bound; the pools equal
    the oracle's bit for bit."""
    B, chunk, sink, window = 16, 256, 512, 2048
    geom = _ticks_geometry(pool, 2, chunk, sink, window, 4, 2)
    ticks = [1792, 2048, 2304, 2560, 2816]  # history before each tick (a multiple of the chunk)
    cap_blocks = -(-sink // B) + -(-window // B) + 1
    width, max_seq = cap_blocks, cap_blocks * B
    rng = np.random.default_rng(3)
    per_seq = -(-(ticks[-1] + chunk) // B)
    perm = rng.permutation(2 * per_seq + 8)
    ids = [perm[:per_seq].astype(np.int64), perm[per_seq: 2 * per_seq].astype(np.int64)]
    geom = small_variant(geom, num_blocks=len(perm))
    Hq, Hkv, D = geom.num_q_heads, geom.num_kv_heads, geom.head_dim
    act = torch.bfloat16
    # fp8 scale fixed up front for every tick (identity-like, as the pages' adapter uses)
    k_scale = v_scale = 1.0 / 64 if pool == "fp8" else 1.0
    inv = 64.0 if pool == "fp8" else 1.0

    def tick_inputs(t, h):
        g = small_variant(geom, history_lens=(h, h), num_blocks=geom.num_blocks)
        wl = Workload(geom=g, device="cuda", block_ids=ids, action_block_ids=[np.zeros(0, np.int64)] * 2)
        plan = G.P.ForwardPlan.build(ids, g.history_lens, g.query_lens, g.sink_tokens, g.window_tokens,
                                     g.full_spans, g.causal_default, B, fixed_capacity=True, device="cuda")
        assert plan.block_table.shape[1] == width and plan.max_seq_len == max_seq  # one shape for every tick
        plan.validate(g.pool_blocks())
        q = _draw((2 * chunk, Hq, D), 100 + t, act)
        k = _draw((2 * chunk, Hkv, D), 200 + t, act)
        v = _draw((2 * chunk, Hkv, D), 300 + t, act)
        return g, wl, plan, q, k, v

    # pools hold every earlier tick's chunk: write the history before the first tick
    kp = G.poisoned_pool(geom)
    vp = G.poisoned_pool(geom)
    pools = G.P.Pools(kp, vp, B, k_scale, v_scale, inv, inv)
    k_ref, v_ref = H.empty_pool(geom), H.empty_pool(geom)
    h0 = ticks[0]
    hist_k = _draw((2 * h0, Hkv, D), 7, act)
    hist_v = _draw((2 * h0, Hkv, D), 8, act)
    slots = np.concatenate([O.slot_mapping(ids[b], np.arange(h0), B) for b in range(2)])
    G.P.pkv_paged_write(hist_k, hist_v, torch.from_numpy(slots).cuda(), pools)
    src = O.BF16
    O.paged_write(k_ref, H.storage_bits(hist_k), slots, src, pool, inv)
    O.paged_write(v_ref, H.storage_bits(hist_v), slots, src, pool, inv)

    g0, wl0, plan0, q0, k0, v0 = tick_inputs(0, ticks[0])
    static = dict(q=q0.clone(), k=k0.clone(), v=v0.clone())
    out = torch.empty_like(static["q"])
    ws = G.workspace_for(plan0, geom)
    assert ws is not None, "the keys should be split so that the merge is captured too"
    scale = H.softmax_scale(D)

    def call(o):
        return G.P.pkv_paged_write_attn(static["q"], static["k"], static["v"], plan0.slot_mapping, pools, plan0,
                                        scale, out=o, workspace=ws)

    G.say("graph", pool, "warm-up and capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out)
    torch.cuda.synchronize()

    for t, h in enumerate(ticks):
        g, wl, plan, q, k, v = tick_inputs(t, h)
        # new contents, same tensors
        for name, src_t in (("q", q), ("k", k), ("v", v)):
            static[name].copy_(src_t)
        for field in ("block_table", "query_start_loc", "seq_lens", "segments", "segment_start_loc", "seq_order",
                      "slot_mapping"):
            dst, new = getattr(plan0, field), getattr(plan, field)
            assert dst.shape == new.shape, field
            dst.copy_(new)
        torch.cuda.synchronize()
        G.say("graph", pool, "replay tick", t, "kv_lens", plan.kv_lens)
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        eager = torch.empty_like(out)
        call(eager)  # writes the same K/V to the same slots again, then attends
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), eager.view(torch.int16)), f"tick {t}: replay differs from eager"
        meta = H.metadata(wl)
        cur = np.concatenate(meta.cur_slots)
        O.paged_write(k_ref, H.storage_bits(k), cur, src, pool, inv)
        O.paged_write(v_ref, H.storage_bits(v), cur, src, pool, inv)
        assert G.bits_equal(pools.key, k_ref) and G.bits_equal(pools.value, v_ref), f"tick {t}: pools"
        li = type("L", (), dict(q=q, k_scale=k_scale, v_scale=v_scale))()
        ref = H.attention(g, meta, li, k_ref, v_ref)
        _err(g, got, ref)


def test_staged_calls_replay_in_two_graphs():
    """The staging decision is a host value (P1 _prepare_history_staging), so a
    captured forward has two variants: restage everything, or refresh the
    current blocks.  One AR block's two probes replay one each; both equal the
    oracle."""
    B, chunk = 16, 64
    geom = _staged_geom("bf16", chunk)
    cap_blocks = -(-geom.sink_tokens[0] // B) + -(-geom.window_tokens[0] // B) + 1
    wl = make_workload(geom, device="cuda")
    plan = G.make_plan(wl, fixed_capacity=True)
    assert plan.block_table.shape[1] == cap_blocks and plan.max_seq_len == cap_blocks * B
    li0 = wl.layer(0)
    pools = G.make_pools(geom, li0)
    G.P.pkv_paged_write(li0.k_hist, li0.v_hist, plan.history_slot_mapping, pools)
    shape = (plan.max_seq_len, geom.num_kv_heads, geom.head_dim)
    sk = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    sv = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    static = dict(q=li0.q.clone(), k=li0.k_cur.clone(), v=li0.v_cur.clone())
    out = torch.empty_like(static["q"])
    staging = G.P.HistoryStaging(capacity_tokens=shape[0])
    session = object()
    staging.decide(session, plan)
    d = staging.decide(session, plan)  # the same window again: the history is kept
    assert d.reuse and d.first_block > 0
    first = d.first_block
    scale = H.softmax_scale(geom.head_dim)

    def call(first_block):
        return G.P.pkv_paged_write_attn(static["q"], static["k"], static["v"], plan.slot_mapping, pools, plan,
                                        scale, stage_key=sk, stage_value=sv, first_block=first_block, out=out)

    G.say("staged graphs: capture")
    call(0)
    call(first)
    torch.cuda.synchronize()
    graphs = []
    for fb in (0, first):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            call(fb)
        graphs.append(gr)
    torch.cuda.synchronize()
    meta = H.metadata(wl)
    table = _padded(meta, plan.max_seq_len // B)
    k_ref, v_ref = H.empty_pool(geom), H.empty_pool(geom)
    H.write_history(geom, meta, li0, k_ref, v_ref)
    for probe, gr in enumerate(graphs + graphs):
        li = wl.layer(10 + probe)
        static["q"].copy_(li.q)
        static["k"].copy_(li.k_cur)
        static["v"].copy_(li.v_cur)
        torch.cuda.synchronize()
        G.say("staged graphs: replay", probe)
        gr.replay()
        torch.cuda.synchronize()
        H.write_current(geom, meta, li, k_ref, v_ref)
        want = np.zeros((shape[0],) + k_ref.shape[1:], dtype=k_ref.dtype)
        O.gather(k_ref, table, plan.max_seq_len // B, 0, want, B)
        assert G.bits_equal(sk, want), f"probe {probe}: staged keys"
        _err(geom, out, H.attention(geom, meta, li, k_ref, v_ref))

"""Layout and mask invariants of the GPU path: determinism, paged == contiguous,
physical-block permutation, row independence, exact per-row mask limits, the
fp8 decode of every code, and no over-read past seq_len."""

import numpy as np
import pytest
import torch

import oracle as O
import paged_kv_cache_174_amd as P
from oracle import harness as H
from workloads import CONFIGS, make_workload, small_variant
from workloads.configs import Workload

from . import gpu_harness as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    G.ensure_built()


GEOMS = {
    "bf16": small_variant(CONFIGS["piecewise_gqa_bf16"], name="inv_bf16", num_q_heads=6, num_kv_heads=2,
                          history_lens=(200, 57), query_lens=(300, 70), sink_tokens=(0, 0),
                          window_tokens=(1 << 30,) * 2, full_spans=(((250, 330),), None)),
    "fp8_short": small_variant(CONFIGS["varlen_fp8"], name="inv_fp8_short", num_q_heads=8, num_kv_heads=2,
                               history_lens=(900, 2100, 250), query_lens=(16, 7, 16), sink_tokens=(0,) * 3,
                               window_tokens=(1 << 30,) * 3, full_spans=(None,) * 3),
    "fp8": small_variant(CONFIGS["varlen_fp8"], name="inv_fp8", num_q_heads=4, num_kv_heads=2,
                         history_lens=(500, 31), query_lens=(16, 200), sink_tokens=(0, 0),
                         window_tokens=(1 << 30,) * 2, full_spans=(None, None)),
}


@pytest.mark.parametrize("kind", list(GEOMS))
@pytest.mark.parametrize("workspace", ["auto", None], ids=["split", "nosplit"])
def test_reruns_are_bit_identical(kind, workspace):
    wl = make_workload(GEOMS[kind], device="cuda")
    li = wl.layer(0)
    G.say("determinism", kind, workspace)
    plan, pools, _, out1 = G.run(wl, li=li, workspace=workspace)
    out2 = G.attend(plan, pools, li, wl.geom, workspace)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


def test_one_workspace_serves_calls_of_different_shapes():
    """The split path writes one partial result per split into the workspace
    and a second launch merges them: a workspace full of garbage, then reused
    by a call with another tiling, gives the same bits as a fresh one each
    time."""
    geoms = [
        small_variant(CONFIGS["piecewise_gqa_bf16"], name="ws_a", num_q_heads=2, num_kv_heads=2,
                      history_lens=(2000,), query_lens=(700,), full_spans=((),)),
        small_variant(CONFIGS["piecewise_gqa_bf16"], name="ws_b", num_q_heads=8, num_kv_heads=2,
                      history_lens=(1500, 40), query_lens=(300, 90), full_spans=(None, ((40, 100),)), sink_tokens=(0, 0), window_tokens=(1 << 30,) * 2),
    ]
    runs = []
    for geom in geoms:
        wl = make_workload(geom, device="cuda")
        li = wl.layer(0)
        plan, pools, _, ref = G.run(wl, li=li, workspace="auto")
        runs.append((geom, plan, pools, li, ref))
    size = max(G.workspace_for(plan, geom).numel() for geom, plan, _, _, _ in runs)
    ws = torch.full((size,), 0xFF, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        for geom, plan, pools, li, ref in runs:
            G.say("shared workspace", geom.name, rep)
            out = G.attend(plan, pools, li, geom, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (geom.name, rep)


@pytest.mark.parametrize("kind", ["fp8", "fp8_short", "bf16"])
def test_dispatch_order_does_not_change_the_result(kind):
    """The sequences' dispatch order (natural, longest first, reversed) only
    changes which workgroup runs when: with the same work split (the same
    length hint), the bits are the same."""
    import paged_kv_cache_174_amd as P

    geom = GEOMS[kind]
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    G.say("dispatch order", kind)
    plan, pools, _, ref = G.run(wl, li=li, workspace="auto")
    ws = G.workspace_for(plan, geom)
    args = (li.q, pools, plan.block_table, plan.query_start_loc, plan.seq_lens, plan.segments,
            plan.segment_start_loc, H.softmax_scale(geom.head_dim), plan.max_query_len, plan.max_seq_len)
    rev = torch.arange(plan.num_seqs - 1, -1, -1, dtype=torch.int32, device="cuda")
    for order in (None, plan.seq_order, rev):
        out = P.pkv_paged_attn(*args, workspace=ws, seq_order=order, host_seq_lens=plan.kv_lens)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("kind", list(GEOMS))
def test_main_then_merge_equals_one_call(kind):
    """pkv_paged_attn_main followed by pkv_paged_attn_merge (same arguments)
    gives pkv_paged_attn's bits, split or not."""
    import paged_kv_cache_174_amd as P

    geom = GEOMS[kind]
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    G.say("main+merge", kind)
    plan, pools, _, ref = G.run(wl, li=li, workspace="auto")
    for ws in (G.workspace_for(plan, geom), None):
        args = (li.q, pools, plan.block_table, plan.query_start_loc, plan.seq_lens, plan.segments,
                plan.segment_start_loc, H.softmax_scale(geom.head_dim), plan.max_query_len, plan.max_seq_len)
        out = torch.empty_like(li.q)
        kw = dict(workspace=ws, seq_order=plan.seq_order, host_seq_lens=plan.kv_lens)  # the harness's plan
        P.pkv_paged_attn_main(*args, out=out, **kw)
        P.pkv_paged_attn_merge(*args, out=out, **kw)
        one = P.pkv_paged_attn(*args, **kw)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), one.view(torch.int16))
        if ws is not None:
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("kind", list(GEOMS))
def test_paged_equals_contiguous_staging(kind):
    """Gather each sequence's visible blocks into a staging buffer and attend
    over it with an identity block table: bit-identical to the paged read."""
    geom = GEOMS[kind]
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    G.say("paged==contiguous", kind)
    plan, pools, _, out = G.run(wl, li=li, workspace=None)
    width = plan.block_table_host.shape[1]
    n_total = width * geom.num_seqs
    shape = (n_total * geom.block_size, geom.num_kv_heads, geom.head_dim)
    sk = torch.zeros(shape, dtype=pools.key.dtype, device="cuda")
    sv = torch.zeros_like(sk)
    for b in range(geom.num_seqs):
        n = len(plan.tables[b])
        ids = torch.from_numpy(plan.tables[b].astype(np.int32)).cuda()
        rows = slice(b * width * geom.block_size, (b * width + n) * geom.block_size)
        G.P.pkv_gather(pools, ids, n, 0, sk[rows], sv[rows])
    staged = G.P.Pools(sk, sv, geom.block_size, pools.k_scale, pools.v_scale, pools.k_inv_scale, pools.v_inv_scale)
    ident = torch.arange(n_total, dtype=torch.int32, device="cuda").reshape(geom.num_seqs, width).contiguous()
    out2 = G.P.pkv_paged_attn(li.q, staged, ident, plan.query_start_loc, plan.seq_lens, plan.segments,
                              plan.segment_start_loc, H.softmax_scale(geom.head_dim), plan.max_query_len,
                              plan.max_seq_len)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


def test_physical_block_permutation_is_invisible():
    geom = GEOMS["bf16"]
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    G.say("permutation")
    _, _, _, out1 = G.run(wl, li=li)
    rng = np.random.default_rng(99)
    perm = rng.permutation(geom.pool_blocks())
    wl2 = Workload(geom=geom, device="cuda", block_ids=[perm[ids] for ids in wl.block_ids])
    _, _, _, out2 = G.run(wl2, li=li)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


def test_rows_of_other_sequences_do_not_leak():
    geom = GEOMS["bf16"]
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    G.say("row independence")
    _, _, _, out1 = G.run(wl, li=li)
    h0 = geom.history_lens[0]
    li.k_hist[h0:] = li.k_hist[h0:] * -1.5 + 0.25  # sequence 1's history only
    li.v_cur[geom.query_lens[0]:] = 3.0
    _, _, _, out2 = G.run(wl, li=li)
    q0 = geom.query_lens[0]
    assert torch.equal(out1[:q0].view(torch.int16), out2[:q0].view(torch.int16))
    assert not torch.equal(out1[q0:].view(torch.int16), out2[q0:].view(torch.int16))


@pytest.mark.parametrize("workspace", ["auto", None], ids=["split", "nosplit"])
def test_zero_queries_reveal_each_rows_key_limit_exactly(workspace):
    """Q = 0 makes every visible logit 0, so a row's output is the mean of the
    values it may see.  With V[j] = j (exact in bf16) that mean is (L - 1) / 2,
    exactly: the test reads every row's key limit L(g) off the output."""
    # seq_len <= 256 keeps every (L - 1) / 2 exactly representable in bf16
    geom = small_variant(CONFIGS["piecewise_gqa_bf16"], name="mask_reveal", num_q_heads=4, num_kv_heads=2,
                         history_lens=(100, 0), query_lens=(150, 77), sink_tokens=(0, 0),
                         window_tokens=(1 << 30,) * 2,
                         full_spans=(((110, 130), (180, 200), (230, 250)), ()))
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    li.q.zero_()
    # position-valued V: history positions 0..h-1, current h..h+q-1 (per sequence)
    hoff = np.concatenate([[0], np.cumsum(geom.history_lens)])
    qoff = np.concatenate([[0], np.cumsum(geom.query_lens)])
    for b in range(geom.num_seqs):
        h, q = geom.history_lens[b], geom.query_lens[b]
        pos_h = torch.arange(h, device="cuda", dtype=torch.float32)[:, None, None]
        pos_q = torch.arange(h, h + q, device="cuda", dtype=torch.float32)[:, None, None]
        li.v_hist[hoff[b]:hoff[b + 1]] = pos_h.to(torch.bfloat16)
        li.v_cur[qoff[b]:qoff[b + 1]] = pos_q.to(torch.bfloat16)
    G.say("mask reveal", workspace)
    plan, _, _, out = G.run(wl, li=li, workspace=workspace)
    segs = O.segments_for_rows(geom.full_spans, geom.query_lens, plan.kv_lens, geom.causal_default)
    for b in range(geom.num_seqs):
        lim = O.row_limits(segs[b], plan.kv_lens[b], geom.query_lens[b])
        want = (lim - 1) / 2.0
        got = G.as_f64(out[qoff[b]:qoff[b + 1]])
        assert np.array_equal(got, np.broadcast_to(want[:, None, None], got.shape))


def test_every_fp8_code_decodes_exactly():
    """One visible key: the softmax weight is exactly 1, so the output is the
    decoded value of each V code times v_scale (1 here), exactly."""
    geom = small_variant(CONFIGS["varlen_fp8"], name="fp8_codes", num_q_heads=2, num_kv_heads=2,
                         history_lens=(0,), query_lens=(1,), sink_tokens=(0,), window_tokens=(1 << 30,),
                         full_spans=(None,))
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    plan = G.make_plan(wl)
    pools = G.P.Pools(G.poisoned_pool(geom), G.poisoned_pool(geom), 16, 1.0, 1.0, 1.0, 1.0)
    slot = int(plan.cur_slots_host[0])
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).reshape(2, 128).cuda()
    pools.value[slot] = codes
    pools.key[slot] = 0x38  # 1.0
    G.say("fp8 codes")
    out = G.attend(plan, pools, li, geom, workspace=None)
    torch.cuda.synchronize()
    got = G.as_f64(out[0]).reshape(-1)
    want = O.e4m3_decode(np.arange(256, dtype=np.uint8))
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all(), np.nonzero(~same)


def test_nothing_past_seq_len_is_read():
    """Overwrite the unwritten tail of each sequence's last, partly written
    block with huge finite values: if any were read the output would move."""
    geom = small_variant(CONFIGS["frame_bf16"], name="tail", num_q_heads=2, num_kv_heads=2,
                         history_lens=(40, 9), query_lens=(20, 3), sink_tokens=(0, 0),
                         window_tokens=(1 << 30,) * 2, full_spans=(None, None))
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    G.say("tail over-read")
    plan, pools, _, out1 = G.run(wl, li=li)
    for b in range(geom.num_seqs):
        s = plan.kv_lens[b]
        assert s % 16, "the case needs a partly written last block"
        last = int(plan.tables[b][-1])
        pools.key[last * 16 + s % 16:(last + 1) * 16] = 3.0e38
        pools.value[last * 16 + s % 16:(last + 1) * 16] = 3.0e38
    out2 = G.attend(plan, pools, li, geom)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


def test_length_hint_changes_only_the_work_split():
    """The host length hint re-plans the short-query work split; with it,
    without it, and with a stale one the output matches the oracle and the
    three agree within rounding."""
    geom = small_variant(CONFIGS["varlen_fp8"], name="hint_fp8", num_q_heads=8, num_kv_heads=2,
                         history_lens=(6000, 700, 90, 3100), query_lens=(16, 16, 3, 16), sink_tokens=(0,) * 4,
                         window_tokens=(1 << 30,) * 4, full_spans=(None,) * 4)
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    plan = G.make_plan(wl)
    pools = G.make_pools(geom, li)
    G.write_layer(plan, pools, li)
    ws = G.workspace_for(plan, geom)
    args = (li.q, pools, plan.block_table, plan.query_start_loc, plan.seq_lens, plan.segments,
            plan.segment_start_loc, H.softmax_scale(geom.head_dim), plan.max_query_len, plan.max_seq_len)
    G.say("length hint", geom.name)
    outs = [G.P.pkv_paged_attn(*args, workspace=ws, seq_order=plan.seq_order, host_seq_lens=hint)
            for hint in (plan.kv_lens, None, [plan.max_seq_len] * plan.num_seqs, [1] * plan.num_seqs)]
    torch.cuda.synchronize()
    _, _, _, ref = H.run_layer(wl, li=li)
    for o in outs:
        got = G.as_f64(o)
        assert np.isfinite(got).all() and np.max(np.abs(got - ref)) <= 6e-2
        assert np.max(np.abs(got - G.as_f64(outs[0]))) <= 2e-2


def test_peak_probes_report_plausible_rates():
    """The diagnostic probes bench.py states its measured-peak fractions against:
    the bf16 matrix-core rate lies between a tenth of and the vendor's 2.5
    PFLOP/s, the HBM read rate between a tenth of and the vendor's 8 TB/s."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(512 * cus, dtype=torch.float32, device="cuda")
    flop = P.pkv_probe_mfma(2000, sink)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    flop = P.pkv_probe_mfma(20000, sink)
    b.record()
    b.synchronize()
    tflops = flop / (a.elapsed_time(b) * 1e-3) / 1e12
    assert 250 < tflops <= 2500 * 1.02, tflops
    assert torch.isfinite(sink).all()
    buf = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")  # four times the last-level cache
    sink8 = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    P.pkv_probe_stream(buf, sink8)
    torch.cuda.synchronize()
    a.record()
    P.pkv_probe_stream(buf, sink8)
    b.record()
    b.synchronize()
    gbps = buf.numel() / (a.elapsed_time(b) * 1e-3) / 1e9
    assert 800 < gbps <= 8000 * 1.05, gbps

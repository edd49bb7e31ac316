"""Edge sizes on the GPU: an empty write, key ranges longer than one split can
stage (so the key range must be split however few rows there are), and a key
range past the supported number of splits (refused before any launch).

Attention is checked against the float64 oracle on sampled rows with the
tolerances of the other attention tests (max |O_gpu - O_oracle| <= 2e-2 for
bf16 pools, 6e-2 for fp8)."""

import numpy as np
import pytest
import torch

from oracle import harness as H
from workloads import CONFIGS, make_workload, small_variant

from . import gpu_harness as G

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "fp8": 6e-2}
# keys one workgroup's block-table slice covers (4095 blocks of 16)
SPLIT_KEYS = 4095 * 16


@pytest.fixture(scope="module", autouse=True)
def _lib():
    G.ensure_built()


def test_write_of_no_tokens_changes_nothing():
    geom = CONFIGS["tiny_f32"]
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    pools = G.make_pools(geom, li)
    before_k, before_v = pools.key.clone(), pools.value.clone()
    empty = li.k_cur[:0].contiguous()
    G.say("write of 0 tokens")
    G.P.pkv_paged_write(empty, empty, torch.zeros(0, dtype=torch.int64, device="cuda"), pools)
    torch.cuda.synchronize()
    assert torch.equal(pools.key.view(torch.uint8), before_k.view(torch.uint8))
    assert torch.equal(pools.value.view(torch.uint8), before_v.view(torch.uint8))


LONG = [
    # long path (rows per KV head > 64): causal rows over a history longer than a split
    small_variant(CONFIGS["piecewise_gqa_bf16"], name="past_split_keys_bf16", num_q_heads=4, num_kv_heads=2,
                  history_lens=(SPLIT_KEYS + 3000,), query_lens=(200,), full_spans=((),)),
    # short path (16 tokens x 4 heads per KV head), two sequences either side of the capacity
    small_variant(CONFIGS["varlen_fp8"], name="past_split_keys_fp8_short", num_q_heads=8, num_kv_heads=2,
                  history_lens=(SPLIT_KEYS + 1, SPLIT_KEYS - 17), query_lens=(16, 16), sink_tokens=(0, 0),
                  window_tokens=(1 << 30,) * 2, full_spans=(None, None)),
]


@pytest.mark.parametrize("geom", LONG, ids=[g.name for g in LONG])
def test_key_ranges_longer_than_one_split(geom):
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    G.say("attn past split capacity", geom.name)
    plan, _, _, out = G.run(wl, li=li)
    assert max(plan.kv_lens) > SPLIT_KEYS
    qsl = np.concatenate([[0], np.cumsum(geom.query_lens)])
    rng = np.random.default_rng(7)
    rows = []
    for b in range(geom.num_seqs):
        lo, hi = int(qsl[b]), int(qsl[b + 1])
        rows.extend(sorted({lo, hi - 1} | set(rng.integers(lo, hi, size=6).tolist())))
    _, _, _, ref = H.run_layer(wl, li=li, rows=rows)
    got = G.as_f64(out)[np.asarray(rows)]
    assert np.isfinite(got).all()
    err = float(np.max(np.abs(got - ref)))
    assert err <= TOL[geom.pool_dtype], f"{geom.name}: max abs error {err:.3e}"


def test_more_key_splits_than_supported_are_refused():
    """16 splits of at most SPLIT_KEYS keys bound a sequence; one key more is
    an error from the host, before anything is launched."""
    geom = small_variant(CONFIGS["frame_bf16"], name="refused", num_q_heads=2, num_kv_heads=2,
                         history_lens=(64,), query_lens=(64,), sink_tokens=(0,), window_tokens=(1 << 30,),
                         full_spans=(None,))
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    plan = G.make_plan(wl)
    pools = G.make_pools(geom, li)
    max_seq_len = 16 * SPLIT_KEYS + 16
    table = torch.zeros((1, max_seq_len // 16), dtype=torch.int32, device="cuda")
    table[0, : plan.block_table.shape[1]] = plan.block_table[0]
    with pytest.raises(G.P.PkvError):
        G.P.pkv_paged_attn(li.q, pools, table, plan.query_start_loc, plan.seq_lens, plan.segments,
                           plan.segment_start_loc, 0.1, plan.max_query_len, max_seq_len)
    # with a workspace for any number of splits it is still refused (unsupported), not run
    ws = torch.empty(32 * sum(plan.query_lens) * geom.num_q_heads * 264, dtype=torch.uint8, device="cuda")
    with pytest.raises(G.P.PkvError) as err:
        G.P.pkv_paged_attn(li.q, pools, table, plan.query_start_loc, plan.seq_lens, plan.segments,
                           plan.segment_start_loc, 0.1, plan.max_query_len, max_seq_len, workspace=ws)
    assert err.value.status == G.P._lib.PKV_EUNSUPPORTED


def test_gqa_rows_straddling_waves_with_key_splits():
    """Five query heads per KV head (a token's rows straddle the 32-row wave
    blocks), a ragged last row tile (1000 rows = 3 x 256 + 232), a full span
    inside a causal chunk, and a history long enough that the planner splits
    the keys: the output rows leave through each wave's LDS staging and the
    split partials through the merge."""
    geom = small_variant(CONFIGS["piecewise_gqa_bf16"], name="gqa5_splits_bf16", num_q_heads=10, num_kv_heads=2,
                         history_lens=(20000,), query_lens=(200,), full_spans=(((20050, 20120),),))
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    G.say("attn gqa5 with splits", geom.name)
    plan, _, _, out = G.run(wl, li=li)
    rng = np.random.default_rng(11)
    rows = sorted({0, 31, 32, 63, 199} | set(rng.integers(0, 200, size=10).tolist()))
    _, _, _, ref = H.run_layer(wl, li=li, rows=rows)
    got = G.as_f64(out)[np.asarray(rows)]
    assert np.isfinite(got).all()
    err = float(np.max(np.abs(got - ref)))
    assert err <= TOL["bf16"], f"{geom.name}: max abs error {err:.3e}"

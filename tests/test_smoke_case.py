"""The case `__graft_entry__.smoke()` runs on the GPU, checked on the host: its
geometry must be accepted by the window planner (the recent window holds the
chunk) and must exercise what it is meant to (a sliding window with a sink, a
full span inside a causal chunk, two sequences)."""

import __graft_entry__ as E
import paged_kv_cache_174_amd as P
from workloads import make_workload


def test_smoke_geometry_plans_on_the_host():
    geom = E.smoke_geometry()
    wl = make_workload(geom, device="cpu")
    plan = P.ForwardPlan.build(
        wl.block_ids, geom.history_lens, geom.query_lens, geom.sink_tokens, geom.window_tokens,
        geom.full_spans, geom.causal_default, geom.block_size, device="cpu",
    )
    plan.validate(geom.pool_blocks())
    assert plan.num_seqs == 2
    # the first sequence's history and chunk overflow sink + window: the window slides
    total0 = geom.history_lens[0] + geom.query_lens[0]
    assert plan.kv_lens[0] == geom.sink_tokens[0] + geom.window_tokens[0] < total0
    # its chunk holds causal and full segments; the second sequence is one full segment
    seg = [int(x) for x in plan.segments.reshape(-1).tolist()]
    modes0 = {seg[4 * k + 3] for k in range(int(plan.segment_start_loc[0]), int(plan.segment_start_loc[1]))}
    assert modes0 == {0, 1}

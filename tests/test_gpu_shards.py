"""Query shards on the GPU (P3 ``piecewise_attn`` with ``query_ranges``).

A sharded plan gives each range of a sequence's local query its own attention
entry, with its rows at the range's key positions; full segments keep their
span's end, so a shard's rows attend past the shard.  Checked against the
oracle's restatement of P3 (max |O_gpu - O_oracle| <= 2e-2 for bf16 pools,
6e-2 for fp8, 1e-4 for fp32), and against the unsharded call on the same rows.
Pages cited by tag and function: P3 "vllm_omni/diffusion/attention/backends/utils/piecewise_attn.py".
"""

import numpy as np
import pytest
import torch

import oracle as O
from oracle import harness as H
from workloads import CONFIGS, make_workload, small_variant

from . import gpu_harness as G

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    G.ensure_built()


CASES = [
    (small_variant(CONFIGS["piecewise_gqa_bf16"], name="shards_piecewise", num_q_heads=10, num_kv_heads=2,
                   history_lens=(100,), query_lens=(700,), full_spans=(((100, 300), (450, 800)),)),
     [[(0, 150, 120), (150, 400, 270), (400, 700, 420)]]),
    (small_variant(CONFIGS["frame_bf16"], name="shards_frame", num_q_heads=4, num_kv_heads=4,
                   history_lens=(600, 320), query_lens=(300, 96), sink_tokens=(100, 0),
                   window_tokens=(600, 1 << 30)),
     [[(0, 64, None), (64, 300, None)], [(0, 96, None)]]),
    (small_variant(CONFIGS["varlen_fp8"], name="shards_causal_fp8", num_q_heads=8, num_kv_heads=2,
                   history_lens=(2000, 30), query_lens=(48, 40), sink_tokens=(0, 0),
                   window_tokens=(1 << 30,) * 2, full_spans=(None, None)),
     [[(0, 16, None), (16, 48, None)], [(0, 40, None)]]),
    (small_variant(CONFIGS["tiny_f32"], name="shards_f32", history_lens=(40,), query_lens=(24,),
                   full_spans=(((44, 60),),)),
     [[(0, 5, 40), (5, 24, 45)]]),
]


def _resolve(plan, ranges):
    """Global starts left as None sit at the matching rows of the suffix query."""
    out = []
    for b, rs in enumerate(ranges):
        g0 = plan.kv_lens[b] - plan.query_lens[b]
        out.append([(a, e, g0 + a if g is None else g) for a, e, g in rs])
    return out


@pytest.mark.parametrize("geom,ranges", CASES, ids=[c[0].name for c in CASES])
def test_sharded_attention_matches_the_oracle(geom, ranges):
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    plan = G.make_plan(wl)
    pools = G.make_pools(geom, li)
    G.write_layer(plan, pools, li)
    ranges = _resolve(plan, ranges)
    sh = plan.shard(ranges, device="cuda")
    sh.validate(geom.pool_blocks())
    # the local query: each range takes the chunk rows at its key positions
    qsl = plan.query_start_host
    rows = []
    for b, rs in enumerate(ranges):
        g0 = plan.kv_lens[b] - plan.query_lens[b]
        for a, e, g in rs:
            rows.extend(range(qsl[b] + g - g0, qsl[b] + g - g0 + (e - a)))
    q_local = li.q[torch.tensor(rows, device="cuda")].contiguous()
    scale = H.softmax_scale(geom.head_dim)
    G.say("shards", geom.name, ranges)
    ws = G.workspace_for(sh, geom)
    got = G.P.pkv_paged_write_attn(q_local, None, None, None, pools, sh, scale, workspace=ws)
    whole = G.attend(plan, pools, li, geom)
    torch.cuda.synchronize()
    meta, k_ref, v_ref, _ = H.run_layer(wl, li=li)
    qbits = H.storage_bits(q_local)
    qf = O.decode_storage(qbits, geom.q_dtype)
    ref = np.zeros(qf.shape)
    offs = 0
    for b, rs in enumerate(ranges):
        n = rs[-1][1]
        s = meta.kv_lens[b]
        k = O.kernel_view(k_ref, meta.block_table[b], s, geom.block_size, geom.pool_dtype, li.k_scale)
        v = O.kernel_view(v_ref, meta.block_table[b], s, geom.block_size, geom.pool_dtype, li.v_scale)
        spans = geom.full_spans[b]
        if spans is None:
            q_b = geom.query_lens[b]
            spans = [] if geom.causal_default else [(s - q_b, s)]
        ref[offs: offs + n] = O.piecewise_attention(qf[offs: offs + n], k, v, spans, scale, query_ranges=rs)
        offs += n
    out = G.as_f64(got)
    assert np.isfinite(out).all()
    err = float(np.max(np.abs(out - ref)))
    assert err <= TOL[geom.pool_dtype], f"{geom.name}: max abs error {err:.3e}"
    # the same rows of the unsharded call (its query is the whole chunk)
    w = G.as_f64(whole)[np.asarray(rows)]
    assert float(np.max(np.abs(out - w))) <= 2 * TOL[geom.pool_dtype]

"""Runs a generated workload through the HIP library (tests only).

Every kernel launch goes through the C ABI via the package's ctypes binding;
the metadata is validated on the host first, so no launch ever sees
inconsistent shapes or out-of-range table entries.
"""

from __future__ import annotations

import os
import sys

import numpy as np
import torch

import paged_kv_cache_174_amd as P
from oracle.harness import softmax_scale

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}
POISON_BITS = {"f32": 0x7FC00000, "bf16": 0x7FC0, "fp8": 0x7F}


def ensure_built():
    if not os.path.exists(P._lib.LIB_PATH):
        from paged_kv_cache_174_amd.build import build

        build()
    P.lib()


def say(*msg):
    """Names the case before each GPU step (flushed, so it survives a crash)."""
    print("[gpu]", *msg, file=sys.stderr, flush=True)


def poisoned_pool(geom, device="cuda"):
    rows = geom.pool_blocks() * geom.block_size
    shape = (rows, geom.num_kv_heads, geom.head_dim)
    if geom.pool_dtype == "f32":
        return torch.full(shape, float("nan"), dtype=torch.float32, device=device)
    if geom.pool_dtype == "bf16":
        return torch.full(shape, float("nan"), dtype=torch.bfloat16, device=device)
    return torch.full(shape, POISON_BITS["fp8"], dtype=torch.uint8, device=device)


def make_plan(wl, device="cuda", **kw):
    g = wl.geom
    if g.action_lens:
        kw.setdefault("action_lens", g.action_lens)
        kw.setdefault("action_block_ids", wl.action_block_ids)
    plan = P.ForwardPlan.build(
        wl.block_ids, g.history_lens, g.query_lens, g.sink_tokens, g.window_tokens, g.full_spans,
        g.causal_default, g.block_size, device=device, **kw,
    )
    plan.validate(g.pool_blocks())
    return plan


def make_pools(geom, li, device="cuda"):
    kp, vp = poisoned_pool(geom, device), poisoned_pool(geom, device)
    return P.Pools(kp, vp, geom.block_size, li.k_scale, li.v_scale, li.k_inv_scale, li.v_inv_scale)


def write_layer(plan, pools, li):
    if li.k_hist.shape[0]:
        P.pkv_paged_write(li.k_hist, li.v_hist, plan.history_slot_mapping, pools)
    P.pkv_paged_write(li.k_cur, li.v_cur, plan.slot_mapping, pools)
    if li.k_act is not None:
        P.pkv_paged_write(li.k_act, li.v_act, plan.action_slot_mapping, pools)


def write_attend(plan, pools, li, geom, workspace="auto", out=None, **staging):
    """The fused per-layer call: current (and action) writes, then attention."""
    ws = workspace_for(plan, geom) if workspace == "auto" else workspace
    acts = {}
    if li.k_act is not None:
        acts = dict(action_key=li.k_act, action_value=li.v_act, action_slot_mapping=plan.action_slot_mapping)
    return P.pkv_paged_write_attn(
        li.q, li.k_cur, li.v_cur, plan.slot_mapping, pools, plan, softmax_scale(geom.head_dim),
        out=out, workspace=ws, **acts, **staging,
    )


def workspace_for(plan, geom, device="cuda"):
    n = P.pkv_paged_attn_workspace_size(
        sum(plan.query_lens), geom.num_q_heads, geom.num_kv_heads, geom.head_dim, plan.num_seqs,
        plan.max_query_len, plan.max_seq_len,
    )
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device) if n else None


def attend(plan, pools, li, geom, workspace="auto", out=None):
    ws = workspace_for(plan, geom) if workspace == "auto" else workspace
    return P.pkv_paged_attn(
        li.q, pools, plan.block_table, plan.query_start_loc, plan.seq_lens, plan.segments,
        plan.segment_start_loc, softmax_scale(geom.head_dim), plan.max_query_len, plan.max_seq_len,
        out=out, workspace=ws, seq_order=plan.seq_order, host_seq_lens=plan.kv_lens,
    )


def run(wl, layer=0, li=None, workspace="auto"):
    """History write, current write, attention.  Returns (plan, pools, li, out)."""
    geom = wl.geom
    li = wl.layer(layer) if li is None else li
    plan = make_plan(wl)
    pools = make_pools(geom, li)
    write_layer(plan, pools, li)
    out = attend(plan, pools, li, geom, workspace)
    torch.cuda.synchronize()
    return plan, pools, li, out


def as_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().double().cpu().numpy()


def bits_equal(gpu_tensor: torch.Tensor, oracle_bits: np.ndarray) -> bool:
    from oracle.harness import storage_bits

    g = storage_bits(gpu_tensor)
    if g.dtype == np.float32:
        return np.array_equal(g.view(np.uint32), oracle_bits.astype(np.float32).view(np.uint32))
    return np.array_equal(g, oracle_bits)

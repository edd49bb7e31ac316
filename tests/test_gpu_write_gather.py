"""Paged write and history-staging gather on the GPU: bit-exact against the oracle."""

import numpy as np
import pytest
import torch

import oracle as O
from oracle import harness as H
from workloads import CONFIGS, make_workload, small_variant

from . import gpu_harness as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    G.ensure_built()


SMALL = {
    "tiny_f32": CONFIGS["tiny_f32"],
    "frame_small_bf16": small_variant(
        CONFIGS["frame_bf16"], name="frame_small_bf16", num_q_heads=3, num_kv_heads=3,
        history_lens=(600, 600), query_lens=(300, 300), sink_tokens=(300, 300), window_tokens=(900, 900),
    ),
    "varlen_small_fp8": small_variant(
        CONFIGS["varlen_fp8"], name="varlen_small_fp8", num_q_heads=8, num_kv_heads=2,
        history_lens=(100, 40, 777, 0, 5), query_lens=(16, 100, 16, 50, 1), sink_tokens=(0,) * 5,
        window_tokens=(1 << 30,) * 5, full_spans=(None,) * 5,
    ),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_write_is_bit_exact(name):
    geom = SMALL[name]
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    G.say("write", name)
    plan = G.make_plan(wl)
    pools = G.make_pools(geom, li)
    G.write_layer(plan, pools, li)
    torch.cuda.synchronize()
    meta, kp, vp, _ = H.run_layer(wl, li=li, rows=[0], heads=[0])
    assert G.bits_equal(pools.key, kp)
    assert G.bits_equal(pools.value, vp)


@pytest.mark.parametrize("inv_scale", [1.0, 0.37, 93.5])
def test_fp8_quantiser_is_bit_exact_on_every_bf16_pattern(inv_scale):
    """All 65536 bf16 bit patterns through the pool cast, against the oracle's
    rounding from the e4m3 definition."""
    Hkv, D = 2, 128
    T = (1 << 16) // (Hkv * D)
    bits = torch.arange(1 << 16, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    src = bits.reshape(T, Hkv, D).cuda()
    pool = torch.full((T * 2, Hkv, D), 0x7F, dtype=torch.uint8, device="cuda")
    pool_v = pool.clone()
    pools = G.P.Pools(pool, pool_v, 16, 1.0, 1.0, inv_scale, inv_scale)
    slots = torch.arange(T, dtype=torch.int64, device="cuda") * 2 + 1
    G.say("fp8 quantiser", inv_scale)
    G.P.pkv_paged_write(src, src, slots, pools)
    torch.cuda.synchronize()
    want = O.encode_for_pool(bits.view(torch.int16).numpy().view(np.uint16), O.BF16, O.FP8, inv_scale)
    got = pool.cpu().numpy()
    assert np.array_equal(got[1::2].reshape(-1), want)
    assert np.all(got[0::2] == 0x7F)  # untouched slots
    assert np.array_equal(pool_v.cpu().numpy(), got)


@pytest.mark.parametrize("name", ["frame_bf16", "tiny_f32", "varlen_small_fp8"])
@pytest.mark.parametrize("first_block", [0, 5])
def test_gather_is_bit_exact_and_leaves_other_rows(name, first_block):
    geom = CONFIGS.get(name) or SMALL[name]
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    G.say("gather", name, first_block)
    plan = G.make_plan(wl)
    pools = G.make_pools(geom, li)
    G.write_layer(plan, pools, li)
    b = int(np.argmax(plan.kv_lens))
    ids = torch.from_numpy(plan.tables[b].astype(np.int32)).cuda()
    n = len(plan.tables[b])
    first_block = min(first_block, n - 1)
    cap = (n + 3) * geom.block_size
    sentinel = {"f32": -7.0, "bf16": -7.0}
    shape = (cap, geom.num_kv_heads, geom.head_dim)
    if geom.pool_dtype == "fp8":
        sk = torch.full(shape, 0xC7, dtype=torch.uint8, device="cuda")
    else:
        sk = torch.full(shape, sentinel[geom.pool_dtype], dtype=G.TORCH_DT[geom.pool_dtype], device="cuda")
    sv = sk.clone()
    sentinel_copy = sk.clone()
    G.P.pkv_gather(pools, ids, n, first_block, sk, sv)
    torch.cuda.synchronize()
    from oracle.harness import storage_bits

    kp, vp = storage_bits(pools.key), storage_bits(pools.value)
    init = storage_bits(sentinel_copy)  # the staging contents before the gather
    want_k, want_v = init.copy(), init.copy()
    O.gather(kp, plan.tables[b], n, first_block, want_k, geom.block_size)
    O.gather(vp, plan.tables[b], n, first_block, want_v, geom.block_size)
    got_k, got_v = storage_bits(sk), storage_bits(sv)
    view = (lambda a: a.view(np.uint32)) if geom.pool_dtype == "f32" else (lambda a: a)
    assert np.array_equal(view(got_k), view(want_k))
    assert np.array_equal(view(got_v), view(want_v))
    B = geom.block_size
    assert np.array_equal(view(got_k[: first_block * B]), view(init[: first_block * B]))
    assert np.array_equal(view(got_k[n * B :]), view(init[n * B :]))


def test_gather_rejects_bad_ranges():
    geom = SMALL["frame_small_bf16"]
    wl = make_workload(geom, device="cuda")
    li = wl.layer(0)
    pools = G.make_pools(geom, li)
    ids = torch.zeros(4, dtype=torch.int32, device="cuda")
    st = torch.zeros((64, geom.num_kv_heads, geom.head_dim), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        G.P.pkv_gather(pools, ids, 4, 5, st, st)
    with pytest.raises(ValueError):
        G.P.pkv_gather(pools, ids, 4, -1, st, st)

"""Attention after eviction, on the GPU, through the host window manager's
tables (P2 ``test_attention_after_eviction_reads_every_kept_token_and_nothing_unwritten``).

24-token chunks against 16-token blocks, pools poisoned with NaN, every slot
of a chunk's blocks poisoned again before the chunk is written, so reading an
unwritten slot turns the output NaN.  Each chunk runs an uncommitted and a
committing forward; the output must match dense float64 attention over the
tokens the oracle's residency model says the window reads (max abs error
1e-4 for fp32 pools, 2e-2 for bf16).
Pages cited by tag and function: P2 "tests/diffusion/ar_diffusion/test_paged_attention.py".
"""

import numpy as np
import pytest
import torch

import oracle as O

from . import gpu_harness as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    G.ensure_built()


@pytest.mark.parametrize("pool", ["f32", "bf16"])
@pytest.mark.parametrize("sink_chunks,window_chunks,reset", [(1, 2, False), (0, 2, False), (1, 3, False),
                                                              (2, 2, True), (0, 2, True)])
def test_attention_after_eviction(pool, sink_chunks, window_chunks, reset):
    P = G.P
    C, B, H, D = 24, 16, 4, 128 if pool == "bf16" else 64
    cfg = P.WindowConfig(num_blocks=256, chunk_size=C, window_chunks=window_chunks, sink_chunks=sink_chunks,
                         chunks_per_block=2, reset_at_boundary=reset, scratch_blocks=4)
    wm = P.WindowManager(cfg)
    model = O.WindowModel(B, C, sink_chunks, window_chunks, reset, 2)
    rid = wm.begin_request()
    dt = G.TORCH_DT[pool]
    kp = torch.full((cfg.num_blocks * B, H, D), float("nan"), dtype=dt, device="cuda")
    vp = torch.full_like(kp, float("nan"))
    pools = P.Pools(kp, vp, B)
    width = cfg.max_video_blocks + 1
    gen = torch.Generator(device="cuda")
    gen.manual_seed(17)
    written = {}
    scale = float(np.float32(D ** -0.5))
    tol = 1e-4 if pool == "f32" else 2e-2
    for chunk in range(8):
        for commit in (False, True):
            slots, _ = wm.prepare(rid, C, commit)
            E = wm.info(rid)["absolute_num_computed_tokens"]
            # poison the chunk's blocks from its first slot on, then write it
            first = int(slots[0])
            for blk in sorted({int(s) // B for s in slots}):
                lo = first if blk == first // B else blk * B
                kp[lo:(blk + 1) * B] = float("nan")
                vp[lo:(blk + 1) * B] = float("nan")
            k = torch.randn((C, H, D), generator=gen, device="cuda").to(dt)
            v = torch.randn((C, H, D), generator=gen, device="cuda").to(dt)
            P.pkv_paged_write(k, v, torch.from_numpy(slots).cuda(), pools)
            kf, vf = k.double().cpu().numpy(), v.double().cpu().numpy()
            cur = {E + t: (kf[t], vf[t]) for t in range(C)}
            table, kv_len, _ = wm.window_table(rid)
            want = model.window(C)
            assert kv_len == want.kv_len
            bt = np.zeros((1, width), dtype=np.int32)
            bt[0, : len(table)] = table
            seg = P.pkv_build_segments([(kv_len - C, kv_len)], kv_len - C, C)
            P.pkv_validate_metadata_host([0, C], [kv_len], bt, cfg.num_blocks, B, C, width * B, seg, [0, 1])
            q = torch.randn((C, H, D), generator=gen, device="cuda").to(dt)
            G.say("window", pool, sink_chunks, window_chunks, reset, "chunk", chunk, "commit", commit)
            out = P.pkv_paged_attn(
                q, pools, torch.from_numpy(bt).cuda(), torch.tensor([0, C], dtype=torch.int32, device="cuda"),
                torch.tensor([kv_len], dtype=torch.int32, device="cuda"),
                torch.from_numpy(seg.reshape(-1)).cuda(), torch.tensor([0, 1], dtype=torch.int32, device="cuda"),
                scale, C, width * B,
            )
            torch.cuda.synchronize()
            src = dict(written)
            src.update(cur)
            kk = np.stack([src[p][0] for p in want.positions])
            vv = np.stack([src[p][1] for p in want.positions])
            ref = O.dense_attention(q.double().cpu().numpy(), kk, vv, np.full(C, kv_len), scale)
            got = out.double().cpu().numpy()
            assert np.isfinite(got).all(), "an unwritten slot was read"
            err = float(np.max(np.abs(got - ref)))
            assert err <= tol, f"chunk {chunk} commit {commit}: max abs error {err:.3e}"
            wm.commit(rid)
        written.update(cur)
        model.commit(C)
    assert wm.info(rid)["compacted_tokens"] > 0

"""Throughput of the paged-attention hot path on one MI355X.

A step is one pass of the path over one batch, issued as one fused call per
layer (pkv_paged_write_attn): the current chunk's K/V is scattered into the
pools through the slot mapping, then the chunk's queries attend over the
visible history through the block table (the attention kernel, then the merge
of key splits).  The 40-layer workload runs that call once per layer, each
layer with its own pools and inputs, all sharing one metadata plan; workloads
with a sliding window get the pages' fixed-capacity metadata (table width and
max_seq_len at the window's capacity).  Inputs, pools and metadata are
resident in HBM before timing starts; the history is written (untimed) during
setup.

Prints one JSON line.  `value` is algorithmic attention TFLOP/s over whole
steps (4 * D * Hq * visible query-key pairs per call).  `roofline` is for the
attention kernel (attn_long_kernel for bf16 chunks), timed with HIP events on
the stream the library launches on; its `traffic` comes from the committed
rocprofv3 FETCH_SIZE / WRITE_SIZE summary for this workload when that summary
was taken on the current kernel sources (null otherwise).  `kv_bound` times
the short-query kernel and its split merge on the KV-bound half of the varlen
fp8 batch (query length 16) against HBM bandwidth.  `parts` reports the write,
the merge and the history-staging gather on their own (the per-launch pass
issues the three calls separately, with events between them), the step as
three separate calls per layer, the step captured once in a HIP graph and
replayed, the write and the gather at 1 GiB (HBM figures), and whole steps of
the other workloads (`configs`: the piecewise GQA chunk, the 40-layer step,
and the whole varlen fp8 batch against max(FLOPs / MFMA peak, bytes / HBM
bandwidth)).

    python bench.py [--steps K] [--warmup W] [--workload frame_bf16]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged-attn TFLOP/s + KV GB/s (% roofline), 1560-tok chunk over windowed history"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E
ELT = {"f32": 4, "bf16": 2, "fp8": 1}


# Sources whose change invalidates a stored traffic measurement of the attention kernel.
KERNEL_SOURCES = ("attn_long.hip", "attn_mfma.hip", "mfma_util.hpp", "attn_common.hpp", "pkv_internal.hpp",
                  "pkv_api.cpp")
# The non-headline workloads reported under parts.configs (each timed as whole steps).
OTHER_CONFIGS = ("piecewise_gqa_bf16", "ar_step_40L_bf16", "varlen_fp8")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="frame_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kv-bound", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--no-configs", action="store_true", help="skip the other workloads under parts.configs")
    ap.add_argument("--no-hbm-copies", action="store_true", help="skip the 1 GiB write and gather figures")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (the gather kernel) a few times, so that a "
                         "counter run can scale FETCH_SIZE / WRITE_SIZE by a known byte count")
    return ap.parse_args()


def kernel_source_hash() -> str:
    """SHA-256 of the kernel sources with comments and blank space removed, so
    that an edit of a comment does not invalidate a measurement."""
    import re

    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_174_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def stored_traffic(workload: str, kernel: str = "attn_long"):
    """HBM bytes per attention launch from the committed counter summary, or
    None when there is none or it was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != kernel_source_hash():
        return None
    try:
        return int(kv["fetch_bytes_per_launch"]) + int(kv["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class ClockSampler:
    """Samples the shader clock the GPU's power management reports (the
    starred level of ``pp_dpm_sclk``, an SMU average) from a host thread while
    a block of work runs.  The matrix-core peak assumes 2.4 GHz; the sampled
    clock says what the chip could deliver during the measurement."""

    def __init__(self, period_s=0.01):
        import glob
        import threading

        paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = paths[0] if paths else None
        self.period = period_s
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        try:
            with open(self.path) as f:
                for ln in f:
                    if ln.rstrip().endswith("*"):
                        return float(ln.split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz"))
        except (OSError, ValueError, IndexError):
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        if self.path:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread.is_alive():
            self._thread.join()

    def summary(self):
        if not self.samples:
            return None
        x = np.asarray(self.samples[len(self.samples) // 4:] or self.samples)
        return {"median_mhz": round(float(np.median(x)), 1), "min_mhz": round(float(x.min()), 1),
                "samples": len(x), "source": "pp_dpm_sclk, current level, during the settling steps"}


def _softmax_scale(d):
    return float(np.float32(d ** -0.5))


def setup(geom, device="cuda"):
    import paged_kv_cache_174_amd as P
    from workloads import make_workload

    wl = make_workload(geom, device=device)
    # AR workloads with a sliding window get P1 build_block_table's fixed-shape
    # metadata (table width and max_seq_len at the window's capacity); the
    # real lengths go to the library as its planning hint.
    windowed = max(geom.window_tokens) < (1 << 29)
    plan = P.ForwardPlan.build(
        wl.block_ids, geom.history_lens, geom.query_lens, geom.sink_tokens, geom.window_tokens,
        geom.full_spans, geom.causal_default, geom.block_size, device=device, fixed_capacity=windowed,
    )
    plan.validate(geom.pool_blocks())
    rows = geom.pool_blocks() * geom.block_size
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[geom.pool_dtype]
    layers = []
    for layer in range(geom.num_layers):
        li = wl.layer(layer)
        kp = torch.zeros((rows, geom.num_kv_heads, geom.head_dim), dtype=dt, device=device)
        vp = torch.zeros_like(kp)
        pools = P.Pools(kp, vp, geom.block_size, li.k_scale, li.v_scale, li.k_inv_scale, li.v_inv_scale)
        if li.k_hist.shape[0]:
            P.pkv_paged_write(li.k_hist, li.v_hist, plan.history_slot_mapping, pools)
        li.k_hist = li.v_hist = None  # history now lives in the pools only
        layers.append((li, pools, torch.empty_like(li.q)))
    ws_bytes = P.pkv_paged_attn_workspace_size(
        sum(geom.query_lens), geom.num_q_heads, geom.num_kv_heads, geom.head_dim, geom.num_seqs,
        plan.max_query_len, plan.max_seq_len,
    )
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=device) if ws_bytes else None
    torch.cuda.synchronize()
    return wl, plan, layers, ws


def attn_bytes(geom, plan):
    """Algorithmic bytes of one attention call: each visible K and V element once
    per (sequence, KV head) at storage width, Q once, O once, the table entries read."""
    kv = sum(plan.kv_lens) * geom.num_kv_heads * geom.head_dim * ELT[geom.pool_dtype] * 2
    qo = sum(geom.query_lens) * geom.num_q_heads * geom.head_dim * ELT[geom.q_dtype] * 2
    table = sum(-(-s // geom.block_size) for s in plan.kv_lens) * 4
    return kv + qo + table


def back_to_back_ms(stream, fn, reps, per_rep):
    """Average duration of one launch: `reps` calls of `fn` (each `per_rep`
    launches of the kernel measured, one after another on `stream`) between
    two events.  Unlike an event pair around every launch, this leaves out the
    events' own packets and the dispatch latency they expose (about 5 us per
    launch here), and keeps the gaps between back-to-back launches."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (reps * per_rep)


def write_bytes(geom):
    t = sum(geom.query_lens) * geom.num_kv_heads * geom.head_dim
    return 2 * t * (ELT[geom.q_dtype] + ELT[geom.pool_dtype]) + 8 * sum(geom.query_lens)


def run_bench(args, geom):
    import paged_kv_cache_174_amd as P

    wl, plan, layers, ws = setup(geom)
    scale = _softmax_scale(geom.head_dim)
    stream = torch.cuda.current_stream()

    def attn_args(li, pools):
        return (li.q, pools, plan.block_table, plan.query_start_loc, plan.seq_lens, plan.segments,
                plan.segment_start_loc, scale, plan.max_query_len, plan.max_seq_len)

    def step():
        """One pass of the path: the fused per-layer call (current K/V slot
        writes, attention, split merge) for every layer."""
        for li, pools, out in layers:
            P.pkv_paged_write_attn(li.q, li.k_cur, li.v_cur, plan.slot_mapping, pools, plan, scale, out=out,
                                   workspace=ws)

    def separate_step(ev=None):
        """The same work as three calls per layer (write, attention kernel,
        merge), with events between the launches when `ev` is given."""
        for i, (li, pools, out) in enumerate(layers):
            if ev is not None:
                ev[4 * i].record(stream)
            P.pkv_paged_write(li.k_cur, li.v_cur, plan.slot_mapping, pools)
            if ev is not None:
                ev[4 * i + 1].record(stream)
            P.pkv_paged_attn_main(*attn_args(li, pools), out=out, workspace=ws, seq_order=plan.seq_order,
                                  host_seq_lens=plan.kv_lens)
            if ev is not None:
                ev[4 * i + 2].record(stream)
            P.pkv_paged_attn_merge(*attn_args(li, pools), out=out, workspace=ws, seq_order=plan.seq_order,
                                   host_seq_lens=plan.kv_lens)
            if ev is not None:
                ev[4 * i + 3].record(stream)

    def timed(fn):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(args.steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    # Bring the GPU to its sustained state under this load before anything is
    # measured: back-to-back steps for about a second.  (Kernels run faster
    # for the first milliseconds of continuous load, before the power
    # management settles the clocks, so short measurements started from idle
    # overstate sustained throughput.)
    settle0 = time.perf_counter()
    with ClockSampler() as clock:
        while time.perf_counter() - settle0 < 1.0:
            for _ in range(16):
                step()
            torch.cuda.synchronize()

    # Passes for `parts` and the roofline: the separate calls, per launch with
    # events between them and as whole steps.
    nl = len(layers)
    for _ in range(2):
        separate_step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4 * nl)] for _ in range(args.steps)]
    for k in range(args.steps):
        separate_step(evs[k])
    torch.cuda.synchronize()

    def mean_gap(a, b):
        return float(np.mean([e[4 * i + a].elapsed_time(e[4 * i + b]) for e in evs for i in range(nl)]))

    write_ms, main_bracketed_ms, merge_ms = mean_gap(0, 1), mean_gap(1, 2), mean_gap(2, 3)
    plan_desc = P.pkv_last_attn_plan()

    def mains():
        for li, pools, out in layers:
            P.pkv_paged_attn_main(*attn_args(li, pools), out=out, workspace=ws, seq_order=plan.seq_order,
                                  host_seq_lens=plan.kv_lens)

    # the attention kernel's average launch, back to back over the layers
    main_ms = back_to_back_ms(stream, mains, args.steps, nl)
    separate_ms = timed(separate_step)

    # whole-step timing (the number `value` is computed from): W warm-up
    # steps, then exactly K timed steps
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    step_ms = timed(step)
    wall = time.perf_counter() - wall0

    # the history-staging gather over the whole visible window, and the
    # contiguous path that attends over the staged buffer (identity table)
    li, pools, out = layers[0]
    width = plan.block_table_host.shape[1]
    n_total = width * plan.num_seqs
    sk = torch.empty((n_total * geom.block_size, geom.num_kv_heads, geom.head_dim), dtype=pools.key.dtype,
                     device="cuda")
    sv = torch.empty_like(sk)
    ids = [torch.from_numpy(t.astype(np.int32)).cuda() for t in plan.tables]
    staged = P.Pools(sk, sv, geom.block_size, pools.k_scale, pools.v_scale, pools.k_inv_scale, pools.v_inv_scale)
    ident = torch.arange(n_total, dtype=torch.int32, device="cuda").reshape(plan.num_seqs, width).contiguous()
    rows_per_seq = width * geom.block_size

    def gather_all():
        for b in range(plan.num_seqs):
            r = slice(b * rows_per_seq, (b + 1) * rows_per_seq)
            P.pkv_gather(pools, ids[b], len(plan.tables[b]), 0, sk[r], sv[r])

    def staged_attn():
        P.pkv_paged_attn(li.q, staged, ident, plan.query_start_loc, plan.seq_lens, plan.segments,
                         plan.segment_start_loc, scale, plan.max_query_len, plan.max_seq_len, out=out,
                         workspace=ws, seq_order=plan.seq_order, host_seq_lens=plan.kv_lens)

    if args.copy_calibration:
        copy_calibration(pools)

    for _ in range(2):
        gather_all()
        staged_attn()
    ge = [torch.cuda.Event(enable_timing=True) for _ in range(3 * args.steps)]
    for k in range(args.steps):
        ge[3 * k].record(stream)
        gather_all()
        ge[3 * k + 1].record(stream)
        staged_attn()
        ge[3 * k + 2].record(stream)
    torch.cuda.synchronize()
    gather_ms = np.mean([ge[3 * k].elapsed_time(ge[3 * k + 1]) for k in range(args.steps)])
    staged_ms = np.mean([ge[3 * k + 1].elapsed_time(ge[3 * k + 2]) for k in range(args.steps)])

    # The step captured once in a HIP graph and replayed, last: on this
    # software stack eager launches that follow a graph replay in the same
    # process run measurably slower, so nothing else is timed after it.
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    graph.replay()
    graph_ms = timed(graph.replay)
    del graph

    flops = plan.attn_flops(geom.num_q_heads, geom.head_dim)
    abytes = attn_bytes(geom, plan)
    gbytes = 2 * 2 * sum(len(t) for t in plan.tables) * geom.block_size * geom.num_kv_heads * geom.head_dim * ELT[geom.pool_dtype]
    wbytes = write_bytes(geom)
    return {
        "step_ms": step_ms,
        "wall_s": wall,
        "value": flops * nl / (step_ms * 1e-3) / 1e12,
        "flops": flops,
        "main_ms": main_ms,
        "main_bracketed_ms": main_bracketed_ms,
        "merge_ms": merge_ms,
        "achieved_tflops": flops / (main_ms * 1e-3) / 1e12,
        "attn_bytes": abytes,
        "kv_gbps": abytes / (main_ms * 1e-3) / 1e9,
        "write_ms": write_ms,
        "write_gbps": wbytes / (write_ms * 1e-3) / 1e9,
        "gather_ms": gather_ms,
        "gather_gbps": gbytes / (gather_ms * 1e-3) / 1e9,
        "staged_attn_ms": staged_ms,
        "separate_ms": separate_ms,
        "graph_ms": graph_ms,
        "plan": plan,
        "plan_desc": plan_desc,
        "layers": nl,
        "clock": clock.summary(),
    }


def run_config(geom, steps, warmup):
    """Whole steps of another workload (the fused call per layer), and a
    per-launch pass of its attention kernel and merge with events between.
    For a workload that is not MFMA-bound throughout (the varlen fp8 batch
    mixes 16-row decode-like sequences with 1560-row chunks) the step is also
    compared with max(F / P, B / BW): its algorithmic FLOPs at the bf16 MFMA
    peak or its algorithmic bytes at HBM bandwidth, whichever takes longer."""
    import paged_kv_cache_174_amd as P

    wl, plan, layers, ws = setup(geom)
    scale = _softmax_scale(geom.head_dim)
    stream = torch.cuda.current_stream()

    def attn_args(li, pools):
        return (li.q, pools, plan.block_table, plan.query_start_loc, plan.seq_lens, plan.segments,
                plan.segment_start_loc, scale, plan.max_query_len, plan.max_seq_len)

    def step():
        for li, pools, out in layers:
            P.pkv_paged_write_attn(li.q, li.k_cur, li.v_cur, plan.slot_mapping, pools, plan, scale, out=out,
                                   workspace=ws)

    settle0 = time.perf_counter()
    while time.perf_counter() - settle0 < 0.5:
        step()
        torch.cuda.synchronize()
    nl = len(layers)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * nl * steps)]
    k = 0
    for _ in range(steps):
        for li, pools, out in layers:
            ev[k].record(stream)
            P.pkv_paged_attn_main(*attn_args(li, pools), out=out, workspace=ws, seq_order=plan.seq_order,
                                  host_seq_lens=plan.kv_lens)
            ev[k + 1].record(stream)
            P.pkv_paged_attn_merge(*attn_args(li, pools), out=out, workspace=ws, seq_order=plan.seq_order,
                                   host_seq_lens=plan.kv_lens)
            ev[k + 2].record(stream)
            k += 3
    torch.cuda.synchronize()
    main_bracketed_ms = float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(0, k, 3)]))
    merge_ms = float(np.mean([ev[i + 1].elapsed_time(ev[i + 2]) for i in range(0, k, 3)]))

    def mains(merge):
        for li, pools, out in layers:
            P.pkv_paged_attn_main(*attn_args(li, pools), out=out, workspace=ws, seq_order=plan.seq_order,
                                  host_seq_lens=plan.kv_lens)
            if merge:
                P.pkv_paged_attn_merge(*attn_args(li, pools), out=out, workspace=ws, seq_order=plan.seq_order,
                                       host_seq_lens=plan.kv_lens)

    # average launches, back to back over the layers: the kernel alone, and
    # the kernel with its merge
    main_ms = back_to_back_ms(stream, lambda: mains(False), steps, nl)
    call_ms = back_to_back_ms(stream, lambda: mains(True), steps, nl)
    for _ in range(warmup):
        step()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(steps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    step_ms = a.elapsed_time(b) / steps
    flops = plan.attn_flops(geom.num_q_heads, geom.head_dim)
    abytes = attn_bytes(geom, plan)
    bound_ms = max(flops / (PEAK_BF16_TFLOPS * 1e12), abytes / (PEAK_HBM_GBPS * 1e9)) * 1e3
    res = {
        "layers": nl,
        "step_ms": round(step_ms, 4),
        "tflops": round(flops * nl / (step_ms * 1e-3) / 1e12, 2),
        "attn_call_ms": round(call_ms, 5),
        "attn_main_ms": round(main_ms, 5),
        "attn_main_ms_bracketed": round(main_bracketed_ms, 5),
        "attn_merge_ms_bracketed": round(merge_ms, 5),
        "attn_tflops": round(flops / (call_ms * 1e-3) / 1e12, 2),
        "attn_frac_of_bf16_peak": round(flops / (call_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "main_tflops": round(flops / (main_ms * 1e-3) / 1e12, 2),
        "main_frac_of_bf16_peak": round(flops / (main_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "flop_per_call": flops,
        "bytes_per_call": abytes,
        "bound_ms": round(bound_ms, 5),
        "bound": "mfma" if flops / (PEAK_BF16_TFLOPS * 1e12) >= abytes / (PEAK_HBM_GBPS * 1e9) else "hbm",
        "frac_of_bound": round(bound_ms / call_ms, 4),
    }
    del layers, ws, wl
    torch.cuda.empty_cache()
    return res


def hbm_copies(geom, total_bytes=1 << 30, reps=5):
    """The write and the gather on their own at HBM scale: one write call
    scattering `total_bytes` of K+V rows (bf16 into the workload's pool dtype)
    into a pool twice that size through a shuffled block-granular slot
    mapping, and one gather of `total_bytes` of K+V blocks by shuffled block
    ids into a staging buffer.  Both sides are far larger than the caches,
    so the rates are HBM figures."""
    import paged_kv_cache_174_amd as P

    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[geom.pool_dtype]
    B, H, D = geom.block_size, geom.num_kv_heads, geom.head_dim
    src_elt = 4 if geom.pool_dtype == "f32" else 2
    tokens = total_bytes // 2 // (H * D * src_elt) // B * B
    blocks = tokens // B
    pool_blocks = 2 * blocks
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    kp = torch.zeros((pool_blocks * B, H, D), dtype=dt, device="cuda")
    vp = torch.zeros_like(kp)
    pools = P.Pools(kp, vp, B, 1.0, 1.0, 1.0, 1.0)
    sdt = torch.float32 if geom.pool_dtype == "f32" else torch.bfloat16
    k = torch.randn((tokens, H, D), generator=g, device="cuda").to(sdt)
    v = torch.randn((tokens, H, D), generator=g, device="cuda").to(sdt)
    perm = torch.randperm(pool_blocks, generator=g, device="cuda")[:blocks]
    slots = (perm[:, None] * B + torch.arange(B, device="cuda")[None, :]).reshape(-1).to(torch.int64)
    ids = torch.randperm(pool_blocks, generator=g, device="cuda")[:blocks].to(torch.int32)
    sk = torch.empty((tokens, H, D), dtype=dt, device="cuda")
    sv = torch.empty_like(sk)
    torch.cuda.synchronize()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    w_ms = timed(lambda: P.pkv_paged_write(k, v, slots, pools))
    g_ms = timed(lambda: P.pkv_gather(pools, ids, blocks, 0, sk, sv))
    pool_elt = kp.element_size()
    w_bytes = 2 * tokens * H * D * (src_elt + pool_elt) + 8 * tokens
    g_bytes = 2 * 2 * tokens * H * D * pool_elt + 4 * blocks
    res = {
        "paged_write_1gib": {"ms": round(w_ms, 4), "bytes": int(w_bytes), "gbps": round(w_bytes / (w_ms * 1e-3) / 1e9, 1),
                             "frac_of_hbm": round(w_bytes / (w_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)},
        "gather_1gib": {"ms": round(g_ms, 4), "bytes": int(g_bytes), "gbps": round(g_bytes / (g_ms * 1e-3) / 1e9, 1),
                        "frac_of_hbm": round(g_bytes / (g_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)},
    }
    del kp, vp, k, v, sk, sv, pools
    torch.cuda.empty_cache()
    return res


def copy_calibration(pools, total_bytes=1 << 30, reps=3):
    """A plain device copy of known size for scaling memory counters: the
    gather kernel copying whole blocks of K and V (reads and writes
    `total_bytes` each).  Not part of any reported number."""
    import paged_kv_cache_174_amd as P

    elt = pools.key.element_size()
    row = pools.num_kv_heads * pools.head_dim * elt
    n_blocks = total_bytes // 2 // (16 * row)
    src = torch.empty((n_blocks * 16, pools.num_kv_heads, pools.head_dim), dtype=pools.key.dtype, device="cuda")
    src.view(torch.uint8).fill_(1)
    dk, dv = torch.empty_like(src), torch.empty_like(src)
    cal = P.Pools(src, src, 16, pools.k_scale, pools.v_scale, pools.k_inv_scale, pools.v_inv_scale)
    ids = torch.arange(n_blocks, dtype=torch.int32, device="cuda")
    for _ in range(reps):
        P.pkv_gather(cal, ids, n_blocks, 0, dk, dv)
    torch.cuda.synchronize()
    print(f"[copy-calibration] gather_kernel reads {2 * n_blocks * 16 * row} B and writes "
          f"{2 * n_blocks * 16 * row} B per launch", file=sys.stderr, flush=True)


def run_kv_bound(args):
    """The attention kernel on the KV-bound half of the varlen fp8 batch
    (query length 16), rotating through independent pools so each launch
    reads its K/V from HBM, against HBM bandwidth."""
    import paged_kv_cache_174_amd as P
    from workloads import CONFIGS

    geom = CONFIGS["varlen_fp8_q16"]
    wl, plan, layers, ws = setup(geom)
    scale = _softmax_scale(geom.head_dim)
    stream = torch.cuda.current_stream()

    def launch(li, pools, out):
        args_ = (li.q, pools, plan.block_table, plan.query_start_loc, plan.seq_lens, plan.segments,
                 plan.segment_start_loc, scale, plan.max_query_len, plan.max_seq_len)
        P.pkv_paged_attn_main(*args_, out=out, workspace=ws, seq_order=plan.seq_order,
                              host_seq_lens=plan.kv_lens)

    # sustained state first (back-to-back launches for about half a second)
    settle0 = time.perf_counter()
    while time.perf_counter() - settle0 < 0.5:
        for layer in layers:
            launch(*layer)
        torch.cuda.synchronize()
    for _ in range(max(args.warmup, 1)):
        for layer in layers:
            launch(*layer)
    torch.cuda.synchronize()
    n = max(args.steps, 5)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * n * len(layers))]
    k = 0
    for _ in range(n):
        for layer in layers:
            ev[k].record(stream)
            launch(*layer)
            ev[k + 1].record(stream)
            P.pkv_paged_attn_merge(layer[0].q, layer[1], plan.block_table, plan.query_start_loc, plan.seq_lens,
                                   plan.segments, plan.segment_start_loc, scale, plan.max_query_len,
                                   plan.max_seq_len, out=layer[2], workspace=ws, seq_order=plan.seq_order,
                                   host_seq_lens=plan.kv_lens)
            ev[k + 2].record(stream)
            k += 3
    torch.cuda.synchronize()
    plan_desc = P.pkv_last_attn_plan()
    ms_bracketed = float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(0, len(ev), 3)]))
    call_ms_bracketed = float(np.mean([ev[i].elapsed_time(ev[i + 2]) for i in range(0, len(ev), 3)]))

    def calls(merge):
        for layer in layers:
            launch(*layer)
            if merge:
                P.pkv_paged_attn_merge(layer[0].q, layer[1], plan.block_table, plan.query_start_loc,
                                       plan.seq_lens, plan.segments, plan.segment_start_loc, scale,
                                       plan.max_query_len, plan.max_seq_len, out=layer[2], workspace=ws,
                                       seq_order=plan.seq_order, host_seq_lens=plan.kv_lens)

    # average launches, back to back over the rotating pools: the kernel
    # alone, and the kernel with its merge (the figure `achieved` is from)
    ms = back_to_back_ms(stream, lambda: calls(False), n, len(layers))
    call_ms = back_to_back_ms(stream, lambda: calls(True), n, len(layers))
    abytes = attn_bytes(geom, plan)
    flops = plan.attn_flops(geom.num_q_heads, geom.head_dim)
    gbps = abytes / (call_ms * 1e-3) / 1e9
    main_gbps = abytes / (ms * 1e-3) / 1e9
    return {
        "workload": geom.name,
        "kernel": "attn_mfma_kernel<fp8, short rows> + attn_combine_kernel",
        "plan": plan_desc,
        "bound": "hbm",
        "achieved": round(gbps, 1),
        "peak": PEAK_HBM_GBPS,
        "unit": "GB/s",
        "frac": round(gbps / PEAK_HBM_GBPS, 4),
        "bytes_per_call": abytes,
        "avg_call_ms": round(call_ms, 5),
        "avg_call_ms_bracketed": round(call_ms_bracketed, 5),
        "main_only": {"avg_launch_ms": round(ms, 5), "gbps": round(main_gbps, 1),
                      "frac": round(main_gbps / PEAK_HBM_GBPS, 4),
                      "avg_launch_ms_bracketed": round(ms_bracketed, 5)},
        "tflops": round(flops / (call_ms * 1e-3) / 1e12, 2),
        "rotating_pools": len(layers),
        "seq_lens": [int(x) for x in plan.kv_lens],
        "traffic_main": stored_traffic(geom.name, "attn_mfma"),
    }


def measured_peaks(reps=5):
    """The chip's sustained bf16 matrix-core rate and HBM read rate, from the
    library's two probe kernels (independent MFMA chains on every SIMD; one
    grid-stride read of 2 GiB), each the median of `reps` launches timed with
    events after two untimed ones."""
    import paged_kv_cache_174_amd as P

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()

    def median_ms(fn):
        for _ in range(2):
            fn()
        ts = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    sink = torch.empty(512 * cus, dtype=torch.float32, device="cuda")
    flop = [0]

    def mfma():
        flop[0] = P.pkv_probe_mfma(40000, sink)

    mfma_ms = median_ms(mfma)
    buf = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    sink8 = torch.empty(4096, dtype=torch.uint8, device="cuda")
    read_ms = median_ms(lambda: P.pkv_probe_stream(buf, sink8))
    del buf
    torch.cuda.empty_cache()
    return {
        "mfma_bf16_tflops": round(flop[0] / (mfma_ms * 1e-3) / 1e12, 1),
        "hbm_read_gbps": round((2 << 30) / (read_ms * 1e-3) / 1e9, 1),
        "method": "pkv_probe_mfma (4 independent 32x32x16 bf16 chains per wave, 2 waves per SIMD) and "
                  "pkv_probe_stream (one read of 2 GiB, a contiguous chunk per workgroup), median of 5 event-timed launches",
    }


def cpu_baseline(geom, budget_s, min_s=10.0):
    """The float64 oracle on the host cores, on a bounded sample of the same
    workload: layer 0's oracle metadata, its pool writes and its attention,
    one (sequence, query head) at a time, until the budget is spent (small
    workloads are repeated until at least `min_s` of work has been timed)."""
    from oracle import harness as H
    from workloads import make_workload

    wl = make_workload(geom, device="cpu")
    li = wl.layer(0)
    t0 = time.perf_counter()
    meta = H.metadata(wl)
    kp, vp = H.empty_pool(geom), H.empty_pool(geom)
    seqs = list(range(geom.num_seqs))
    H.write_history(geom, meta, li, kp, vp)
    H.write_current(geom, meta, li, kp, vp)
    setup_s = time.perf_counter() - t0
    qsl = meta.query_start_loc
    pairs = [(b, h) for b in seqs for h in range(geom.num_q_heads)]
    per_pair = [4.0 * geom.head_dim * float(H.O.row_limits(meta.segments[b], meta.kv_lens[b],
                                                           geom.query_lens[b]).sum()) for b in seqs]
    done, flops, t_attn, passes = 0, 0.0, 0.0, 0
    while True:
        b, h = pairs[done % len(pairs)]
        t1 = time.perf_counter()
        H.attention(geom, meta, li, kp, vp, heads=[h], rows=list(range(int(qsl[b]), int(qsl[b + 1]))))
        t_attn += time.perf_counter() - t1
        flops += per_pair[b]
        done += 1
        passes = done // len(pairs)
        total = setup_s + t_attn
        if total >= budget_s or (done % len(pairs) == 0 and total >= min_s):
            break
    threads = os.cpu_count()
    blas = None
    try:
        from threadpoolctl import threadpool_info

        info = threadpool_info()
        threads = max(int(i.get("num_threads", 0)) for i in info) or threads
        libs = [f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer', '')})" for i in info
                if i.get("user_api") == "blas"]
        blas = ", ".join(libs) or None
    except Exception:
        pass
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": flops / total / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "cpu_model": cpu_model,
        "blas": blas,
        "sample": f"layer 0: oracle metadata and pool writes for all {geom.num_seqs} sequences, then attention "
                  f"for {done} (sequence, query head) pairs ({passes} full passes) in float64 numpy; "
                  f"{total:.1f} s wall",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; run with --gpus 1"}))
        sys.exit(2)
    from workloads import CONFIGS

    geom = CONFIGS[args.workload]
    import paged_kv_cache_174_amd as P

    P.lib()  # fail loudly if the HIP library is missing
    # The KV-bound leg runs first: the main leg ends with a HIP graph replay,
    # after which eager launches in the same process run slower.
    kvb = None if args.no_kv_bound else run_kv_bound(args)
    r = run_bench(args, geom)
    plan = r.pop("plan")
    configs = {}
    if not args.no_configs:
        for name in OTHER_CONFIGS:
            if name != geom.name:
                print(f"[bench] config {name}", file=sys.stderr, flush=True)
                configs[name] = run_config(CONFIGS[name], max(3, args.steps // 2), max(1, args.warmup // 2))
    copies = None if args.no_hbm_copies else hbm_copies(geom)
    peaks = measured_peaks()
    if kvb is not None:
        kvb["frac_of_measured_peak"] = round(kvb["achieved"] / peaks["hbm_read_gbps"], 4)
    cpu = None if args.no_cpu_baseline else cpu_baseline(geom, args.cpu_budget_s)
    traffic = stored_traffic(geom.name)
    line = {
        "metric": METRIC,
        "value": round(r["value"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["step_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if geom.pool_dtype == "bf16" else f"bf16 q / {geom.pool_dtype} kv",
        "data": "synthetic",
        "config": {
            "workload": geom.name,
            "num_seqs": geom.num_seqs,
            "query_lens": sorted(set(geom.query_lens)),
            "seq_lens": sorted(set(plan.kv_lens))[:4],
            "num_q_heads": geom.num_q_heads,
            "num_kv_heads": geom.num_kv_heads,
            "head_dim": geom.head_dim,
            "block_size": geom.block_size,
            "layers": r["layers"],
            "pool_dtype": geom.pool_dtype,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(r["achieved_tflops"], 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(r["achieved_tflops"] / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "kernel": "attn_long_kernel (bf16)",
            "plan": r["plan_desc"],
            "flop_per_launch": r["flops"],
            "avg_launch_ms": round(r["main_ms"], 5),
            "avg_launch_ms_bracketed": round(r["main_bracketed_ms"], 5),
            "shader_clock": r["clock"],
            "frac_of_peak_at_clock": (round(r["achieved_tflops"] / (PEAK_BF16_TFLOPS * r["clock"]["median_mhz"] / 2400.0), 4)
                                      if r["clock"] else None),
            "frac_of_measured_peak": round(r["achieved_tflops"] / peaks["mfma_bf16_tflops"], 4),
        },
        "kv": {
            "achieved_gbps": round(r["kv_gbps"], 1),
            "peak_gbps": PEAK_HBM_GBPS,
            "frac": round(r["kv_gbps"] / PEAK_HBM_GBPS, 4),
            "bytes_per_launch": r["attn_bytes"],
        },
        "kv_bound": kvb,
        "measured_peaks": peaks,
        "parts": {
            "paged_write": {"ms": round(r["write_ms"], 5), "gbps": round(r["write_gbps"], 1)},
            "split_merge_ms": round(r["merge_ms"], 5),
            "paged_attn_call_ms": round(r["main_bracketed_ms"] + r["merge_ms"], 5),
            "gather_whole_window": {"ms": round(r["gather_ms"], 5), "gbps": round(r["gather_gbps"], 1)},
            "attn_over_staged_buffer_ms": round(r["staged_attn_ms"], 5),
            "separate_calls_step_ms": round(r["separate_ms"], 5),
            "graph_replay_step_ms": round(r["graph_ms"], 5),
            "hbm_copies": copies,
            "configs": configs,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

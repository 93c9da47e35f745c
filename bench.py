"""Benchmark of the block-causal attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload magi4.5b]

One step = the whole hot path over one batch of synthetic input already
resident in HBM: mask -> AttnSlices (host), atomic-free schedule (host) and
its upload, the QK-Norm + 3D-RoPE prologue kernel on Q and K, and the
Flex-Flash-Attention forward kernel.  The metric counts masked FLOPs,
4 * head_dim * query_heads * (visible query-key pairs), per second.

Prints ONE JSON line.  ``roofline`` describes the attention kernel (the
dominant one) from HIP events recorded around each of its launches on the
stream it runs on; ``cpu_baseline`` times the float64 oracle on a bounded
sample of the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-causal attn fwd TFLOPS (masked FLOPs) and % of MI355X bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published


def visible_pairs(wl) -> int:
    """Visible (query, key) pairs per head, from the chunk arithmetic."""
    total = 0
    for s in wl.seqs:
        first = s.num_kv_chunks - s.num_q_chunks
        for j in range(s.num_q_chunks):
            c = first + j
            r = s.kv_range[j]
            lo = 0 if r < 0 else max(0, c - r)
            total += s.chunk_len * s.chunk_len * (c + 1 - lo)
    return total


def masked_flops(wl) -> float:
    return 4.0 * wl.head_dim * wl.hq * visible_pairs(wl)


CLOCK_GHZ = 2.4   # the clock the published peaks assume (256 CUs, 1024 SIMDs)


MFMA_EXP_OVERLAP = 0.41  # measured: MFMA and exp streams overlap by 41 % of the shorter one


def ceilings(d: int) -> dict:
    """The ceilings of the bf16 forward at head_dim d, in masked TFLOP/s at
    the 2.4 GHz of the published peak.

    Per 32-key x 32-row score block of one wave (4 d 1024 useful FLOPs):
    * VALU: 16 v_exp_f32 at half rate (8 issue cycles each; 31 of 64 lanes
      per clock per CU measured) + 8 v_cvt_pk_bf16_f32 (4 cycles each) =
      160 issue cycles of one SIMD, the softmax work that cannot leave it;
    * MFMA: the padded products, ceil(d/16) Q.K steps and 2 x ceil((d+1)/32)
      P.V steps of v_mfma_f32_32x32x16_bf16 (32768 FLOPs, 32 cycles each),
      of which d / 8 carry the counted work (d = 24: 3 of 4; d = 48: 6 of 7);
    * co-issue: both on one SIMD, whose MFMA and exp streams overlap by only
      MFMA_EXP_OVERLAP of the shorter one (the magi_rates probe with half
      the waves of every SIMD on each): MFMA + VALU - 0.41 min(MFMA, VALU)
      cycles per block (d = 24: 235.5, d = 48: 318.4).
    """
    valu_cyc = 16 * 8 + 8 * 4
    issued = -(-d // 16) + 2 * -(-(d + 1) // 32)
    mfma_cyc = 32 * issued
    both_cyc = mfma_cyc + valu_cyc - MFMA_EXP_OVERLAP * min(mfma_cyc, valu_cyc)
    valu = 1024 * CLOCK_GHZ * 1e9 * 4.0 * d * 1024 / valu_cyc / 1e12
    mfma = PEAK_BF16_TFLOPS * (d / 8.0) / issued
    return {"valu_tflops": round(valu, 1), "mfma_padded_tflops": round(mfma, 1),
            "coissue_tflops": round(mfma * mfma_cyc / both_cyc, 1)}


def with_ceilings(rec: dict, tflops: float, d: int) -> dict:
    """add the fractions of the VALU, padded-MFMA and co-issue ceilings
    beside the fraction of the bf16 peak"""
    c = ceilings(d)
    rec["frac_of_valu_ceiling"] = round(tflops / c["valu_tflops"], 4)
    rec["frac_of_mfma_padded_ceiling"] = round(tflops / c["mfma_padded_tflops"], 4)
    rec["frac_of_coissue_ceiling"] = round(tflops / c["coissue_tflops"], 4)
    return rec


MIN_WARM_S = 0.5
SYNC_EVERY = 32  # warm-up steps between synchronisations (bounds the host's run-ahead)


class steady_timing:
    """No garbage-collection pass inside the warm-up or the timed region (as
    timeit does; a full pass over large heaps stalls the host for ms)."""

    def __enter__(self):
        gc.collect()
        gc.disable()

    def __exit__(self, *exc):
        gc.enable()


def warm_up(step, warmup):
    """At least ``warmup`` untimed steps and MIN_WARM_S seconds of them,
    synchronising every SYNC_EVERY steps, then a synchronisation.

    The shader clock of an idle GPU takes a few hundred ms of load to settle.
    The periodic synchronisation keeps the host at most SYNC_EVERY steps
    ahead: after an unbounded burst of thousands of queued launches the HIP
    runtime spends many later calls retiring it, the host then falls behind
    the GPU at the start of the timed region, and the kernels that follow
    idle gaps run up to 20 % slower (measured on the 4.5B-shaped layer:
    0.330 ms per attention launch with this warm-up against 0.355-0.40 ms
    after an unbounded one)."""
    import torch
    t_w, i = time.perf_counter(), 0
    while i < warmup or time.perf_counter() - t_w < MIN_WARM_S:
        step(False)
        i += 1
        if i % SYNC_EVERY == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def window_pairs(wl, window) -> int:
    """visible pairs per head when every packed video is one causal
    sliding-window sequence: row i of a sequence sees min(window, i + 1) keys"""
    tot = 0
    for s in wl.seqs:
        n = s.num_q_chunks * s.chunk_len
        m = min(window, n)
        tot += m * (m + 1) // 2 + (n - m) * window
    return tot


LAST_LAUNCHES_MS = []  # per-launch attention times of the last run_gpu call


def event_pool(steps, stream):
    """Timing event pairs for ``steps`` attention launches, to be recorded by
    the kernel's own dispatch (ops.ffa_fwd(..., events=pair), i.e.
    magi_ffa_fwd_timed), so that no marker packets of their own sit between
    the kernels; each is recorded once here, so that the HIP event exists
    before it is handed to the library."""
    import torch
    pool = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for pair in pool:
        for e in pair:
            e.record(stream)
    return pool


def run_gpu(wl, steps, warmup, seed=0, window=None):
    """One step = plan build and upload, prologue, forward.  With ``window``
    the mask is causal sliding-window attention of that many tokens over
    each packed video instead of the block-causal one."""
    import torch
    import workloads as W
    from block_causal_attention_amd import ops

    dev = "cuda"
    inp = W.make_inputs(wl, seed)
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    gq, gk, pq, pk = (t.to(dev) for t in (inp.gain_q, inp.gain_k, inp.pos_q, inp.pos_k))
    base = torch.tensor(wl.rope_base, dtype=torch.float32, device=dev)
    tdt = q.dtype
    # K and V reach the attention group-major (written so by the prologue)
    qh = torch.empty_like(q)
    kh = ops.kv_group_major(wl.nk, wl.hkv, wl.head_dim, tdt, dev)
    vh = ops.kv_group_major(wl.nk, wl.hkv, wl.head_dim, tdt, dev)
    knm = torch.empty(wl.hkv, dtype=torch.float32, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    ev = []

    spec = None if window is None else [(s.num_q_chunks * s.chunk_len, window, s.q_offset, s.k_offset)
                                         for s in wl.seqs]
    pool = event_pool(steps, stream)

    # A streaming step's cached keys and values were processed by earlier
    # steps: they are written once here, and a step's prologue covers the
    # in-flight rows only.
    kf = wl.k_fresh_start
    if kf:
        ops.qknorm_rope(q[:1], k[:kf], gq, gk, pq[:1], pk[:kf], base, wl.eps, q_out=qh[:1], k_out=kh[:kf],
                        k_scale=wl.softmax_scale * ops.LOG2E, v=v[:kf], v_out=vh[:kf])

    def step(record):
        if spec is None:
            plan = ops.plan_for_videos(wl.seqs, wl.nq, wl.nk, wl.hq, wl.hkv, wl.head_dim, tdt, dev)
        else:
            plan = ops.make_plan(ops.build_window_slices(spec), wl.nq, wl.nk, wl.hq, wl.hkv, wl.head_dim, tdt, dev)
        # the softmax scale (times log2 e) is folded into K by the prologue
        ops.qknorm_rope(q, k[kf:], gq, gk, pq, pk[kf:], base, wl.eps, q_out=qh, k_out=kh[kf:],
                        k_scale=wl.softmax_scale * ops.LOG2E, k_norm_max=knm, v=v[kf:], v_out=vh[kf:])
        # the events bracket the attention kernel alone; the wait for the
        # plan upload (a side stream) comes before it, inside the step time
        evs = pool[len(ev)] if record else None
        ops.ffa_fwd(qh, kh, vh, plan, out=out, lse=lse, softmax_scale=ops.LN2, k_norm_max=knm, events=evs)
        if record:
            ev.append(evs)
        return plan

    with steady_timing():
        warm_up(step, warmup)
        t0 = time.perf_counter()
        for _ in range(steps):
            plan = step(True)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    kernel_ms = [a.elapsed_time(b) for a, b in ev]
    LAST_LAUNCHES_MS[:] = kernel_ms
    return (t1 - t0) * 1e3 / steps, float(np.mean(kernel_ms)), plan.num_work


def run_backward(wl, steps, warmup, seed=0):
    """Backward of the attention (magi_ffa_bwd) after one forward on the
    prologue's outputs; returns the average launch time in ms from HIP events
    on the launching stream."""
    import torch
    import workloads as W
    from block_causal_attention_amd import ops

    dev = "cuda"
    inp = W.make_inputs(wl, seed)
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    gq, gk, pq, pk = (t.to(dev) for t in (inp.gain_q, inp.gain_k, inp.pos_q, inp.pos_k))
    base = torch.tensor(wl.rope_base, dtype=torch.float32, device=dev)
    knm = torch.empty(wl.hkv, dtype=torch.float32, device=dev)
    qh, kh, vh = ops.qknorm_rope(q, k, gq, gk, pq, pk, base, wl.eps, k_scale=wl.softmax_scale * ops.LOG2E,
                                 k_norm_max=knm, k_out=ops.kv_group_major(wl.nk, wl.hkv, wl.head_dim, q.dtype, dev),
                                 v=v)
    plan = ops.plan_for_videos(wl.seqs, wl.nq, wl.nk, wl.hq, wl.hkv, wl.head_dim, q.dtype, dev, backward=True)
    out, lse = ops.ffa_fwd(qh, kh, vh, plan, softmax_scale=ops.LN2, k_norm_max=knm)
    g = torch.Generator(device="cpu").manual_seed(seed + 1)
    dout = torch.randn(out.shape, generator=g).to(out.dtype).to(dev)
    dq, dk, dv = torch.empty_like(qh), torch.empty_like(kh), torch.empty_like(vh)
    stream = torch.cuda.current_stream()
    ev = []

    def step(rec):
        if rec:
            plan.wait(stream)  # the upload wait stays outside the kernels' events
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
        ops.ffa_bwd(qh, kh, vh, out, dout, lse, plan, softmax_scale=ops.LN2, dq=dq, dk=dk, dv=dv)
        if rec:
            b.record(stream)
            ev.append((a, b))

    with steady_timing():
        warm_up(step, warmup)
        for _ in range(steps):
            step(True)
        torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev]))


TEXT_TOKENS = 800  # condition tokens per sample for the cross-attention record


def run_cross(wl, steps, warmup, seed=0):
    """Cross-attention of the parallel block: the workload's video tokens over
    TEXT_TOKENS condition tokens (one sample), QK-Norm on both sides without
    rotation, then FFA over the cross slice.  Returns (ms per step, kernel ms)."""
    import torch
    from block_causal_attention_amd import ops

    dev = "cuda"
    g = torch.Generator(device="cpu").manual_seed(seed + 7)
    mk = lambda *shape: torch.randn(shape, generator=g).to(torch.bfloat16).to(dev)
    q, k, v = mk(wl.nq, wl.hq, wl.head_dim), mk(TEXT_TOKENS, wl.hkv, wl.head_dim), mk(TEXT_TOKENS, wl.hkv, wl.head_dim)
    gq = (0.8 + 0.4 * torch.rand(wl.head_dim, generator=g)).to(dev)
    gk = (0.8 + 0.4 * torch.rand(wl.head_dim, generator=g)).to(dev)
    zq = torch.zeros((wl.nq, 3), dtype=torch.int32, device=dev)
    zk = torch.zeros((TEXT_TOKENS, 3), dtype=torch.int32, device=dev)
    base = torch.tensor(wl.rope_base, dtype=torch.float32, device=dev)
    qh = torch.empty_like(q)
    kh = ops.kv_group_major(TEXT_TOKENS, wl.hkv, wl.head_dim, q.dtype, dev)
    vh = ops.kv_group_major(TEXT_TOKENS, wl.hkv, wl.head_dim, q.dtype, dev)
    knm = torch.empty(wl.hkv, dtype=torch.float32, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    ev = []
    pool = event_pool(steps, stream)

    def step(record):
        sl = ops.build_cross_slices([(0, wl.nq, 0, TEXT_TOKENS)])
        plan = ops.make_plan(sl, wl.nq, TEXT_TOKENS, wl.hq, wl.hkv, wl.head_dim, q.dtype, dev)
        ops.qknorm_rope(q, k, gq, gk, zq, zk, base, wl.eps, q_out=qh, k_out=kh,
                        k_scale=wl.softmax_scale * ops.LOG2E, k_norm_max=knm, v=v, v_out=vh)
        # the events bracket the attention kernel alone (the wait for the
        # plan upload comes before it, inside the step time)
        evs = pool[len(ev)] if record else None
        ops.ffa_fwd(qh, kh, vh, plan, out=out, lse=lse, softmax_scale=ops.LN2, k_norm_max=knm, events=evs)
        if record:
            ev.append(evs)

    with steady_timing():
        warm_up(step, warmup)
        t0 = time.perf_counter()
        for _ in range(steps):
            step(True)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    return (t1 - t0) * 1e3 / steps, float(np.mean([a.elapsed_time(b) for a, b in ev]))


def run_prologue(wl, steps=200, warmup=50, seed=0):
    """The prologue alone (QK-Norm + 3D RoPE of Q and K, V moved group-major,
    as in the step), timed with HIP events on its stream: (mean ms, median
    ms, algorithmic HBM bytes = every Q/K/V element read and written once
    plus the positions)."""
    import torch
    import workloads as W
    from block_causal_attention_amd import ops

    dev = "cuda"
    inp = W.make_inputs(wl, seed)
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    gq, gk, pq, pk = (t.to(dev) for t in (inp.gain_q, inp.gain_k, inp.pos_q, inp.pos_k))
    base = torch.tensor(wl.rope_base, dtype=torch.float32, device=dev)
    qh = torch.empty_like(q)
    kh = ops.kv_group_major(wl.nk, wl.hkv, wl.head_dim, q.dtype, dev)
    vh = ops.kv_group_major(wl.nk, wl.hkv, wl.head_dim, q.dtype, dev)
    knm = torch.empty(wl.hkv, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def f():
        ops.qknorm_rope(q, k, gq, gk, pq, pk, base, wl.eps, q_out=qh, k_out=kh,
                        k_scale=wl.softmax_scale * ops.LOG2E, k_norm_max=knm, v=v, v_out=vh)

    ev = []
    with steady_timing():
        warm_up(lambda rec: f(), warmup)
        for _ in range(steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            f()
            b.record(stream)
            ev.append((a, b))
        torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    el = q.element_size()
    nbytes = 2 * el * (q.numel() + 2 * k.numel()) + 2 * 4 * 3 * (wl.nq + wl.nk)
    return float(np.mean(ms)), ms[len(ms) // 2], nbytes


def run_copy(nbytes, steps=200, warmup=50):
    """A plain device-to-device copy (torch copy_) that reads and writes
    nbytes / 2 bytes each, timed like run_prologue: what a streaming kernel
    with the prologue's traffic reaches on this GPU (mean ms)."""
    import torch
    src = torch.ones(nbytes // 2, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    ev = []
    with steady_timing():
        warm_up(lambda rec: dst.copy_(src), warmup)
        for _ in range(steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            dst.copy_(src)
            b.record(stream)
            ev.append((a, b))
        torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev]))


def run_first_chunk(steps=300, warmup=100, d=24):
    """A streaming generation's first chunk (2 latent frames x 12 x 16 = 384
    tokens, 128/8 heads): prologue + attention, launch-bound.  Wall time per
    step eagerly with the plan built every step, eagerly with the plan kept
    (it is the same for every denoising step of the chunk), and as one HIP
    graph replay of the prologue and the attention."""
    import torch
    import workloads as W
    from block_causal_attention_amd import ops

    dev = "cuda"
    wl = W.custom_block_causal(1, 2, 12, 16, 128, 8, d)
    inp = W.make_inputs(wl, 0)
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    gq, gk, pq, pk = (t.to(dev) for t in (inp.gain_q, inp.gain_k, inp.pos_q, inp.pos_k))
    base = torch.tensor(wl.rope_base, dtype=torch.float32, device=dev)
    qh = torch.empty_like(q)
    kh = ops.kv_group_major(wl.nk, wl.hkv, d, q.dtype, dev)
    vh = ops.kv_group_major(wl.nk, wl.hkv, d, q.dtype, dev)
    knm = torch.empty(wl.hkv, dtype=torch.float32, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty(wl.nq, wl.hq, dtype=torch.float32, device=dev)
    kept = ops.plan_for_videos(wl.seqs, wl.nq, wl.nk, wl.hq, wl.hkv, d, q.dtype, dev).settle()

    def body(plan):
        ops.qknorm_rope(q, k, gq, gk, pq, pk, base, wl.eps, q_out=qh, k_out=kh, k_scale=wl.softmax_scale * ops.LOG2E,
                        k_norm_max=knm, v=v, v_out=vh)
        ops.ffa_fwd(qh, kh, vh, plan, out=out, lse=lse, softmax_scale=ops.LN2, k_norm_max=knm)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    eager_plan = timed(lambda: body(ops.plan_for_videos(wl.seqs, wl.nq, wl.nk, wl.hq, wl.hkv, d, q.dtype, dev)))
    eager_kept = timed(lambda: body(kept))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        body(kept)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body(kept)
    graph = timed(g.replay)
    return {"tokens": wl.nq, "heads": f"{wl.hq}/{wl.hkv}", "head_dim": d,
            "eager_ms_per_step_plan_built": round(eager_plan, 4), "eager_ms_per_step_plan_kept": round(eager_kept, 4),
            "graph_ms_per_step": round(graph, 4)}


def run_ring(steps, warmup, seed=0):
    """One streaming step over a ring-buffer KV cache at the streaming
    workload's shape (chunks of 3600 tokens = 6 x 24x25, 128/8 heads, d=48):
    24 chunk slots holding global chunks 100..123, the newest 4 in flight
    (so the ring wraps).  A step = slices of the ring + schedule + upload,
    the prologue on the in-flight queries and on the in-flight keys written
    straight into their ring slots, and FFA over the wrapped slices.
    Returns (ms per step, kernel ms, masked FLOPs)."""
    import torch
    from block_causal_attention_amd import ops

    C, S, first, count, n, hq, hkv, d = 3600, 24, 100, 24, 4, 128, 8, 48
    dev = "cuda"
    g = torch.Generator(device="cpu").manual_seed(seed + 11)
    mk = lambda *shape: torch.randn(shape, generator=g).to(torch.bfloat16).to(dev)
    q, knew, vnew = mk(n * C, hq, d), mk(n * C, hkv, d), mk(n * C, hkv, d)
    gq = (0.8 + 0.4 * torch.rand(d, generator=g)).to(dev)
    gk = (0.8 + 0.4 * torch.rand(d, generator=g)).to(dev)
    pos = torch.randint(0, 24, (n * C, 3), generator=g, dtype=torch.int32).to(dev)
    base = torch.tensor((1e4, 1e4, 1e4), dtype=torch.float32, device=dev)
    qh = torch.empty_like(q)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[0], hq, dtype=torch.float32, device=dev)
    knm = torch.empty(hkv, dtype=torch.float32, device=dev)
    scale = d ** -0.5
    # cached chunks, processed by earlier steps: normalised, rotated and
    # scaled by the prologue into their slots, group-major
    ring_k, ring_v = ops.kv_group_major(S * C, hkv, d, torch.bfloat16, dev), \
        ops.kv_group_major(S * C, hkv, d, torch.bfloat16, dev)
    pos_c = torch.randint(0, 24, (S * C, 3), generator=g, dtype=torch.int32).to(dev)
    ops.qknorm_rope(q[:1], mk(S * C, hkv, d), gq, gk, pos[:1], pos_c, base, 1e-6, q_out=qh[:1], k_out=ring_k,
                    k_scale=scale * ops.LOG2E, v=mk(S * C, hkv, d), v_out=ring_v)
    stream = torch.cuda.current_stream()
    runs = ops.ring_slot_runs(S, first + count - n, n)
    ev = []
    pool = event_pool(steps, stream)
    visible = 0

    def step(record):
        nonlocal visible
        sl = ops.build_ring_slices(C, S, first, count, n)
        visible = int(((sl[:, 1] - sl[:, 0]).astype(np.int64) * (sl[:, 3] - sl[:, 2])).sum())
        plan = ops.make_plan(sl, n * C, S * C, hq, hkv, d, q.dtype, dev)
        done = 0
        for s0, m in runs:   # in-flight keys and values into their slots (the ring wraps at most once)
            ops.qknorm_rope(q[:1] if done else q, knew[done * C:(done + m) * C], gq, gk,
                            pos[:1] if done else pos, pos[done * C:(done + m) * C], base, 1e-6,
                            q_out=qh[:1] if done else qh, k_out=ring_k[s0 * C:(s0 + m) * C],
                            k_scale=scale * ops.LOG2E, k_norm_max=knm, v=vnew[done * C:(done + m) * C],
                            v_out=ring_v[s0 * C:(s0 + m) * C])
            done += m
        # the bound on key norms follows from the QK-Norm gains, so it holds
        # for the cached keys as well as for this step's; the events bracket
        # the kernel alone (the upload wait comes before it)
        evs = pool[len(ev)] if record else None
        ops.ffa_fwd(qh, ring_k, ring_v, plan, out=out, lse=lse, softmax_scale=ops.LN2, k_norm_max=knm,
                    events=evs)
        if record:
            ev.append(evs)

    with steady_timing():
        warm_up(step, warmup)
        t0 = time.perf_counter()
        for _ in range(steps):
            step(True)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    return (t1 - t0) * 1e3 / steps, float(np.mean([a.elapsed_time(b) for a, b in ev])), 4.0 * d * hq * visible


def kernel_sources_sha256() -> str:
    """sha256 over the sources the forward kernel is compiled from"""
    import hashlib
    h = hashlib.sha256()
    for f in ("ffa_fwd.hip", "ffa_common.h", "kernels.h"):
        h.update(open(os.path.join(ROOT, "block_causal_attention_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def committed_traffic(wl_name: str):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary (profiles/traffic_<workload>.json), or None when the kernel
    source changed since those counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{wl_name}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_sources_sha256") != kernel_sources_sha256():
        return None
    return float(rec["traffic_bytes_per_launch"])


def cpu_baseline(wl, target_s=30.0, seed=0):
    """Time the float64 oracle on a seeded row sample (all heads) of the workload."""
    import oracle
    import workloads as W
    from threadpoolctl import threadpool_info, threadpool_limits

    inp = W.make_inputs(wl, seed)
    f64 = lambda t: t.float().numpy().astype(np.float64)
    K, V, gk = f64(inp.k), f64(inp.v), f64(inp.gain_k)
    gq = f64(inp.gain_q)

    def run(rows):
        mask = oracle.video_mask(wl.seqs, wl.nq, wl.nk, rows)
        t = time.perf_counter()
        oracle.forward(f64(inp.q[rows]), K, V, gq, gk, inp.pos_q[rows].numpy(), inp.pos_k.numpy(),
                       wl.rope_base, wl.eps, mask, wl.softmax_scale)
        return time.perf_counter() - t, int(mask.sum())

    # the oracle's BLAS runs on every core this process may use
    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores, user_api="blas"):
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] + [1])
        rng = np.random.Generator(np.random.PCG64(seed))
        probe = np.sort(rng.choice(wl.nq, 16, replace=False))
        dt, _ = run(probe)
        n = int(np.clip(16 * target_s / max(dt, 1e-3), 16, wl.nq))
        rows = np.sort(rng.choice(wl.nq, n, replace=False))
        dt, pairs = run(rows)
    flops = 4.0 * wl.head_dim * wl.hq * pairs
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(min(threads, cores)), "kind": "oracle",
            "sample": f"{n} random query rows x {wl.hq} heads of {wl.name} (float64 numpy, "
                      f"{dt:.1f} s, incl. QK-Norm+RoPE of all {wl.nk} keys)"}


def summarize_trace(path, steps):
    """The headline run's launches in a rocprofv3 kernel trace (CSV) of this
    script's default command: the attention and prologue dispatches of the
    4.5B-shaped layer's main run (the ones before the first 24B-shaped
    attention launch, at the layer's full grid), the last ``steps`` of which
    are the timed ones.  Prints a markdown table (durations in microseconds)."""
    import csv
    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Start_Timestamp"]))
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    end = min([int(r["Start_Timestamp"]) for r in rows if "ffa_fwd_bf16<48" in r["Kernel_Name"]] +
              [int(rows[-1]["End_Timestamp"]) + 1])
    grid = max(int(r["Grid_Size_X"]) for r in rows
               if "ffa_fwd_bf16<24" in r["Kernel_Name"] and int(r["Start_Timestamp"]) < end)
    att = [r for r in rows if "ffa_fwd_bf16<24" in r["Kernel_Name"] and int(r["Grid_Size_X"]) == grid
           and int(r["Start_Timestamp"]) < end]
    t0 = int(att[-steps]["Start_Timestamp"])
    prev_end = int(att[-steps - 1]["End_Timestamp"]) if len(att) > steps else t0
    pro = [r for r in rows if "qknorm_rope_kernelILi24" in r["Kernel_Name"] and prev_end <= int(r["Start_Timestamp"]) < end]
    print("| launches | count | avg us | median us | min us | max us |")
    print("|---|---|---|---|---|---|")
    for name, sel in (("attention, timed steps", att[-steps:]), ("attention, warm-up steps", att[:-steps]),
                      ("prologue, timed steps", pro)):
        d = np.array([dur(r) for r in sel]) if sel else np.zeros(1)
        print(f"| {name} | {len(sel)} | {d.mean():.1f} | {np.median(d):.1f} | {d.min():.1f} | {d.max():.1f} |")
    gaps = [(int(att[i]["Start_Timestamp"]) - int(att[i - 1]["End_Timestamp"])) / 1e3
            for i in range(len(att) - steps + 1, len(att))]
    print(f"\nkernel: `{att[-1]['Kernel_Name'][:80]}`; grid {grid}; idle before the first timed launch "
          f"{(t0 - prev_end) / 1e3:.1f} us; mean gap between timed attention launches {np.mean(gaps):.1f} us "
          "(the prologue and the event packets)")


def counter_means(path, name_part):
    """Mean per dispatch of each counter in a rocprofv3 --pmc CSV, over the
    dispatches whose kernel name contains ``name_part`` (rows of one
    dispatch and counter are summed first)."""
    import csv
    per = {}
    for r in csv.DictReader(open(path)):
        if name_part not in r["Kernel_Name"]:
            continue
        key = (r["Dispatch_Id"], r["Counter_Name"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (_, cname), v in per.items():
        out.setdefault(cname, []).append(v)
    return {k: float(np.mean(v)) for k, v in out.items()}


def traffic_record(wl_name, kernel, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_bytes):
    """HBM bytes per launch of ``kernel`` from FETCH_SIZE and WRITE_SIZE (KiB
    per dispatch), each scaled by what the same counter reads for a plain
    device copy of ``copy_bytes`` bytes; the record committed_traffic()
    reads back (tied to the kernel sources' sha256)."""
    f = counter_means(fetch_csv, kernel)["FETCH_SIZE"]
    w = counter_means(write_csv, kernel)["WRITE_SIZE"]
    cf = counter_means(copy_fetch_csv, "copyBuffer")["FETCH_SIZE"]
    cw = counter_means(copy_write_csv, "copyBuffer")["WRITE_SIZE"]
    ff, wf = copy_bytes / 1024.0 / cf, copy_bytes / 1024.0 / cw
    return {"workload": wl_name, "kernel": kernel, "fetch_kib": f, "write_kib": w, "fetch_factor": ff,
            "write_factor": wf, "traffic_bytes_per_launch": 1024.0 * (f * ff + w * wf),
            "kernel_sources_sha256": kernel_sources_sha256()}


def counter_table(kernel, d, csvs, blocks):
    """Derived figures of a kernel (the forward by default) from rocprofv3
    --pmc CSVs (the passes in profiles/counters_ffa_fwd.md and
    profiles/counters_ffa_bwd.md): MFMA busy share, co-issue,
    LDS bank-conflict share, resident waves, instructions per 32 x 32 score
    block.  Returns a dict of counter means per dispatch and the derived
    values."""
    c = {}
    for path in csvs:
        c.update(counter_means(path, kernel))
    out = dict(c)
    cyc = c.get("GRBM_GUI_ACTIVE", 0.0) / 8.0        # summed over the 8 XCDs
    simds = 1024
    if cyc:
        out["kernel_cycles"] = cyc
        out["mfma_busy"] = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (simds * cyc)
        out["waves_per_simd"] = 4.0 * c.get("SQ_WAVE_CYCLES", 0.0) / (simds * cyc)
    if c.get("SQ_VALU_MFMA_BUSY_CYCLES"):
        out["mfma_coexec"] = c.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0.0) / c["SQ_VALU_MFMA_BUSY_CYCLES"]
    if c.get("SQ_ACTIVE_INST_LDS"):
        out["lds_conflict_share"] = c.get("SQ_LDS_BANK_CONFLICT", 0.0) / c["SQ_ACTIVE_INST_LDS"]
    # per 32-key x 32-row score block of one wave (blocks = masked FLOPs / (4 d 1024))
    for name in ("SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_VALU_CVT", "SQ_INSTS_LDS",
                 "SQ_INSTS_SALU"):
        if name in c:
            out[name + "_per_block"] = c[name] / blocks
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="magi4.5b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--first-chunk", action="store_true",
                    help="only run the streaming first-chunk record (eager and HIP graph) and print it")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device-to-device copy of this many bytes (a known-size "
                         "reference for calibrating the FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--summarize-trace", metavar="CSV",
                    help="print the headline run's timed launches from a rocprofv3 kernel trace of this script "
                         "(no GPU needed) and exit")
    ap.add_argument("--traffic-record", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="print the HBM-traffic record of the workload's attention kernel from four rocprofv3 "
                         "--pmc CSVs (FETCH_SIZE, WRITE_SIZE of this script; the same of --copy-bytes 1 GiB) "
                         "and exit (no GPU needed)")
    ap.add_argument("--counter-table", nargs="+", metavar="PMC_CSV",
                    help="print the forward kernel's derived counter figures (workload's head_dim) from "
                         "rocprofv3 --pmc CSVs of this script and exit (no GPU needed)")
    ap.add_argument("--counter-kernel", metavar="NAME",
                    help="kernel-name prefix for --counter-table instead of the forward's (e.g. bwd_dkdv_bf16<48); "
                         "per-block figures still count the layer's 32 x 32 score blocks")
    args = ap.parse_args()
    if args.counter_table:
        d = 24 if args.workload == "magi4.5b" else 48
        import workloads as W
        blocks = masked_flops(W.make_workload(args.workload)) / (4.0 * d * 1024)
        kernel = args.counter_kernel or f"ffa_fwd_bf16<{d}"
        print(json.dumps(counter_table(kernel, d, args.counter_table, blocks), indent=1))
        return
    if args.traffic_record:
        d = 24 if args.workload == "magi4.5b" else 48
        print(json.dumps(traffic_record(args.workload, f"ffa_fwd_bf16<{d}", *args.traffic_record, 1 << 30),
                         indent=1))
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.steps)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the attention path has no "
              "multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    first_chunk = None
    if not args.no_secondary and not args.first_chunk and not args.copy_bytes:
        # The launch-bound first-chunk record runs in a fresh child process,
        # started before this process touches the GPU: in a process that has
        # already run the large layers, graph replays measured about twice
        # as slow (≈ 0.035-0.041 vs 0.020 ms) while eager steps did not move.
        import subprocess
        res = subprocess.run([sys.executable, os.path.abspath(__file__), "--first-chunk"], capture_output=True,
                             text=True, timeout=600)
        lines = [ln for ln in res.stdout.splitlines() if ln.startswith("{")]
        first_chunk = json.loads(lines[-1]) if res.returncode == 0 and lines else \
            {"error": f"child exited with {res.returncode}"}

    import torch
    import workloads as W
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.first_chunk:
        print(json.dumps(run_first_chunk()), flush=True)
        return
    if args.copy_bytes:
        src = torch.ones(args.copy_bytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel() * 4, "launches": 5}), flush=True)
        return

    wl = W.make_workload(args.workload)
    flops = masked_flops(wl)
    ms_step, ms_kernel, nwork = run_gpu(wl, args.steps, args.warmup)
    launches = sorted(LAST_LAUNCHES_MS)
    achieved = flops / (ms_kernel * 1e-3) / 1e12
    rec = {
        "metric": METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "fp32",
        "data": "synthetic (seeded N(0,1) Q/K/V, U(0.8,1.2) QK-Norm gains; no weights)",
        "config": {"workload": wl.name, "description": wl.description, "tokens": wl.nq,
                   "query_heads": wl.hq, "kv_groups": wl.hkv, "head_dim": wl.head_dim,
                   "masked_flops_per_step": flops, "work_items": nwork, "parallelism": "single GPU",
                   "kv_layout": "group-major [hkv][nk][d], written by the prologue"},
        # whole step (plan, upload, prologue, attention) against the bf16 peak;
        # the attention kernel alone is in roofline.frac
        "step_pct_of_bf16_peak": round(100.0 * flops / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "roofline": with_ceilings(
            {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
             "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
             "traffic": committed_traffic(wl.name),
             "kernel": "ffa_fwd_bf16", "avg_launch_ms": round(ms_kernel, 5),
             "median_launch_ms": round(launches[len(launches) // 2], 5),
             "min_launch_ms": round(launches[0], 5), "ceilings": ceilings(wl.head_dim)},
            achieved, wl.head_dim),
    }
    if first_chunk is not None:
        rec["first_chunk"] = first_chunk
    if not args.no_secondary and wl.name == "magi4.5b":
        wl2 = W.make_workload("magi24b")
        f2 = masked_flops(wl2)
        s2, k2, _ = run_gpu(wl2, max(3, args.steps // 2), 2)
        kt2 = f2 / (k2 * 1e-3) / 1e12
        rec["secondary"] = with_ceilings(
            {"workload": wl2.name, "ms_per_step": round(s2, 4), "value": round(f2 / (s2 * 1e-3) / 1e12, 2),
             "avg_launch_ms": round(k2, 4), "kernel_tflops": round(kt2, 2),
             "pct_of_bf16_peak": round(100.0 * kt2 / PEAK_BF16_TFLOPS, 2)}, kt2, wl2.head_dim)
        # the streaming step (linear layout: 20 cached + 4 in-flight chunks)
        # and the packed varlen layer with KV-range-limited chunks (seed 0)
        more = {}
        for name in ("stream", "varlen"):
            w = W.make_workload(name)
            fm = masked_flops(w)
            sm, km, nw = run_gpu(w, 3, 1)
            kt = fm / (km * 1e-3) / 1e12
            more[name] = with_ceilings(
                {"description": w.description, "masked_flops": fm, "work_items": nw, "ms_per_step": round(sm, 4),
                 "value": round(fm / (sm * 1e-3) / 1e12, 2), "avg_launch_ms": round(km, 4),
                 "kernel_tflops": round(kt, 2), "pct_of_bf16_peak": round(100.0 * kt / PEAK_BF16_TFLOPS, 2)},
                kt, w.head_dim)
        rec["stream"] = more["stream"]
        rec["varlen"] = more["varlen"]
    if not args.no_secondary:
        # backward: 5 products of 2 d flops per visible pair and head
        # (S recomputed, dP, dV, dK, dQ) = 2.5 x the forward's masked FLOPs
        bwd = {}
        for name in ("magi4.5b", "magi24b"):
            w = W.make_workload(name)
            kb = run_backward(w, 5 if name == "magi24b" else 10, 2)
            fb = 2.5 * masked_flops(w)
            bwd[name] = {"avg_launch_ms": round(kb, 4), "tflops": round(fb / (kb * 1e-3) / 1e12, 2),
                         "pct_of_bf16_peak": round(100.0 * fb / (kb * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)}
        rec["backward"] = bwd
        cross = {}
        for name in ("magi4.5b", "magi24b"):
            w = W.make_workload(name)
            ms_s, ms_k = run_cross(w, 10, 3)
            fc = 4.0 * w.head_dim * w.hq * w.nq * TEXT_TOKENS
            cross[name] = {"text_tokens": TEXT_TOKENS, "ms_per_step": round(ms_s, 4), "avg_launch_ms": round(ms_k, 4),
                           "kernel_tflops": round(fc / (ms_k * 1e-3) / 1e12, 2)}
        rec["cross_attention"] = cross
        win = {}
        for name, w_tok in (("magi4.5b", 1440), ("magi24b", 3600)):
            w = W.make_workload(name)
            ms_s, ms_k, _ = run_gpu(w, 10, 3, window=w_tok)
            fw = 4.0 * w.head_dim * w.hq * window_pairs(w, w_tok)
            kt = fw / (ms_k * 1e-3) / 1e12
            win[name] = with_ceilings({"window_tokens": w_tok, "ms_per_step": round(ms_s, 4),
                                       "avg_launch_ms": round(ms_k, 4), "kernel_tflops": round(kt, 2),
                                       "pct_of_bf16_peak": round(100.0 * kt / PEAK_BF16_TFLOPS, 2)}, kt, w.head_dim)
        rec["sliding_window"] = win
        pro = {}
        for name in ("magi4.5b", "magi24b"):
            w = W.make_workload(name)
            mean_ms, med_ms, nbytes = run_prologue(w)
            copy_ms = run_copy(nbytes)
            pro[name] = {"avg_launch_ms": round(mean_ms, 5), "median_launch_ms": round(med_ms, 5),
                         "algorithmic_bytes": nbytes, "GB/s": round(nbytes / (mean_ms * 1e-3) / 1e9, 1),
                         "frac_of_hbm_peak": round(nbytes / (mean_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                         "same_size_copy_GB/s": round(nbytes / (copy_ms * 1e-3) / 1e9, 1),
                         "frac_of_same_size_copy": round(copy_ms / mean_ms, 4)}
        rec["prologue"] = pro
        ms_s, ms_k, fr = run_ring(5, 2)
        rec["streaming_ring"] = {"shape": "4 in-flight x 3600 queries over a 24-slot ring (86400 keys), 128/8, d=48",
                                 "ms_per_step": round(ms_s, 4), "avg_launch_ms": round(ms_k, 4),
                                 "kernel_tflops": round(fr / (ms_k * 1e-3) / 1e12, 2)}
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

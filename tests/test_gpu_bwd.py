"""GPU parity of the attention backward (magi_ffa_bwd through the C ABI)
against the float64 oracle's gradients.

The oracle gets exactly the tensors the GPU used (the bf16-rounded q, k, v,
dO), so the differences come from the kernel's own arithmetic: bf16 rounding
of P and dS before their products, of O (delta = rowsum(dO * O) uses the
stored bf16 O), and of the stored gradients, each ~2^-9 relative, with fp32
accumulation.  Bar (bf16): relative L2 <= 1e-2 and max-abs <= 2e-2 x the
largest reference magnitude, per gradient.  fp32: relative L2 <= 1e-5.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from block_causal_attention_amd import _lib, ops

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = {"bf16": dict(rel_l2=1e-2, max_rel=2e-2), "fp32": dict(rel_l2=1e-5, max_rel=1e-5)}


def note(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def np64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def rand(shape, seed, scale=1.0):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape).astype(np.float32) * scale


def compare(got, want, kind, what):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    diff = got - want
    ref = float(np.abs(want).max()) if want.size else 0.0
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    den = float(np.linalg.norm(want))
    rel = float(np.linalg.norm(diff)) / den if den > 0 else float(np.linalg.norm(diff))
    note(f"{what}: max-abs {max_abs:.3e} (ref max {ref:.3e}) rel-L2 {rel:.3e}")
    tol = TOL[kind]
    assert rel <= tol["rel_l2"], f"{what} rel-L2 {rel:.3e} > {tol['rel_l2']}"
    assert max_abs <= tol["max_rel"] * max(ref, 1e-30), f"{what} max-abs {max_abs:.3e} > {tol['max_rel']} x {ref:.3e}"


def bwd_case(q, k, v, dO, slices, kind, scale=None):
    """forward + backward on the GPU; the oracle backward on the same rounded
    inputs.  Returns the GPU (dq, dk, dv) tensors."""
    nq, hq, dd = q.shape
    nk, hkv = k.shape[0], k.shape[1]
    tdt = torch.bfloat16 if kind == "bf16" else torch.float32
    qd, kd, vd, dod = (torch.from_numpy(x).to(tdt).to(DEV) for x in (q, k, v, dO))
    sl = np.asarray(slices, np.int32).reshape(-1, 5)
    plan = ops.make_plan(sl, nq, nk, hq, hkv, dd, tdt, backward=True)
    O, L = ops.ffa_fwd(qd, kd, vd, plan, softmax_scale=scale)
    dq = torch.full_like(qd, float("nan"))
    dk = torch.full_like(kd, float("nan"))
    dv = torch.full_like(vd, float("nan"))
    ops.ffa_bwd(qd, kd, vd, O, dod, L, plan, softmax_scale=scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert not torch.isnan(t).any(), f"{name} has unwritten or NaN entries"
    mask = oracle.slices_mask([tuple(int(x) for x in s) for s in sl], nq, nk) if len(sl) else np.zeros((nq, nk), bool)
    gq, gk, gv = oracle.attention_backward(np64(qd), np64(kd), np64(vd), np64(dod), mask,
                                           scale if scale else dd ** -0.5)
    compare(np64(dq), gq, kind, "dQ")
    compare(np64(dk), gk, kind, "dK")
    compare(np64(dv), gv, kind, "dV")
    return dq, dk, dv, mask


@pytest.mark.parametrize("d", [24, 48])
@pytest.mark.parametrize("G", [16, 4, 1, 3])
def test_bwd_block_causal_ragged(d, G):
    # 3 chunks of 37 tokens: no tile boundary lines up with a chunk
    note(f"bwd block-causal ragged d={d} G={G}")
    hkv = 2
    sl = ops.build_slices([W.SeqDesc(37, 3, 3, 0, 0, (-1, -1, -1), 1, 1, 37)])
    bwd_case(rand((111, G * hkv, d), 1), rand((111, hkv, d), 2), rand((111, hkv, d), 3),
             rand((111, G * hkv, d), 4), sl, "bf16")


@pytest.mark.parametrize("d", [24, 48])
def test_bwd_causal_and_irregular_slices(d):
    note(f"bwd irregular slices d={d}")
    nq, nk = 150, 330
    slices = [
        (0, 70, 0, 70, _lib.MASK_CAUSAL),          # square causal
        (70, 100, 0, 40, _lib.MASK_FULL),          # two k ranges for one q band
        (70, 100, 60, 130, _lib.MASK_CAUSAL),      # wide causal, bottom-right aligned
        (100, 140, 130, 150, _lib.MASK_CAUSAL),    # tall causal: early rows see nothing
        (100, 140, 150, 300, _lib.MASK_FULL),      # a key tile wider than one work item
        # rows 140..149 and keys 300..329 are covered by no slice
    ]
    dq, dk, dv, _ = bwd_case(rand((nq, 16, d), 5), rand((nk, 1, d), 6), rand((nk, 1, d), 7),
                             rand((nq, 16, d), 8), np.array(slices), "bf16")
    assert torch.all(dq[140:] == 0) and torch.all(dk[300:] == 0) and torch.all(dv[300:] == 0)


@pytest.mark.parametrize("d", [24, 48])
def test_bwd_prescaled_keys(d):
    # the forward run the benchmark uses (K times scale*log2 e, softmax scale
    # ln 2) differentiates with respect to the prescaled keys; the oracle on
    # the same prescaled keys with scale ln 2 is the same function
    note(f"bwd prescaled K d={d}")
    c = d ** -0.5 * ops.LOG2E
    k = torch.from_numpy(rand((300, 2, d), 21) * c).to(torch.bfloat16).float().numpy()
    sl = ops.build_slices([W.SeqDesc(100, 3, 3, 0, 0, (-1, -1, 1), 1, 1, 100)])
    bwd_case(rand((300, 32, d), 20), k, rand((300, 2, d), 22), rand((300, 32, d), 23), sl, "bf16",
             scale=ops.LN2)


def test_bwd_fp32_tiny():
    note("bwd fp32 tiny")
    wl = W.make_workload("tiny")
    inp = W.make_inputs(wl, 0)
    sl = ops.build_slices(wl.seqs)
    bwd_case(inp.q.numpy(), inp.k.numpy(), inp.v.numpy(), rand(tuple(inp.q.shape), 9), sl, "fp32")


def oracle_prologue(wl, inp, rows=None):
    """q_hat (of ``rows``, all rows if None) and the prescaled k_hat from the
    oracle's QK-Norm + 3D RoPE of the raw inputs, float64 (never the GPU's)"""
    inv = oracle.rope_inv_freq(wl.rope_base, wl.head_dim)
    q = inp.q if rows is None else inp.q[rows]
    pq = inp.pos_q if rows is None else inp.pos_q[rows]
    qn = oracle.rope_3d(oracle.qk_norm(np64(q), np64(inp.gain_q), wl.eps), pq.numpy(), inv)
    kn = oracle.rope_3d(oracle.qk_norm(np64(inp.k), np64(inp.gain_k), wl.eps), inp.pos_k.numpy(), inv)
    return qn, kn * (wl.softmax_scale * ops.LOG2E)


def gpu_fwd_bwd(wl, inp, dO):
    """the path as the benchmark runs it: prologue (scale folded into K, K
    and V written group-major, key-norm bound), forward, then the backward
    over the same plan; returns (dq, dk, dv, plan)"""
    g = lambda t: t.to(DEV)
    knm = torch.empty(wl.hkv, dtype=torch.float32, device=DEV)
    qh, kh, vh = ops.qknorm_rope(g(inp.q), g(inp.k), g(inp.gain_q), g(inp.gain_k), g(inp.pos_q), g(inp.pos_k),
                                 torch.tensor(wl.rope_base, dtype=torch.float32, device=DEV), wl.eps,
                                 k_out=ops.kv_group_major(wl.nk, wl.hkv, wl.head_dim, torch.bfloat16),
                                 k_scale=wl.softmax_scale * ops.LOG2E, k_norm_max=knm, v=g(inp.v))
    plan = ops.plan_for_videos(wl.seqs, wl.nq, wl.nk, wl.hq, wl.hkv, wl.head_dim, torch.bfloat16, backward=True)
    O, L = ops.ffa_fwd(qh, kh, vh, plan, softmax_scale=ops.LN2, k_norm_max=knm)
    dq, dk, dv = ops.ffa_bwd(qh, kh, vh, O, g(dO), L, plan, softmax_scale=ops.LN2)
    torch.cuda.synchronize()
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert not torch.isnan(t).any(), f"{name} has NaN entries"
    return dq, dk, dv, plan


def test_bwd_video_after_prologue():
    # the path as the model runs it: QK-Norm + RoPE prologue, scale folded
    # into K, forward, then the backward of the attention on 4 chunks x 240
    # tokens, 32 query heads over 2 groups; the oracle takes q_hat and k_hat
    # from its own prologue of the raw inputs, so the difference also holds
    # the bf16 storage of q_hat and k_hat (about 2^-9 relative)
    note("bwd video after prologue")
    seqs = [W.SeqDesc(240, 4, 4, 0, 0, (-1, -1, -1, -1), 1, 15, 16)]
    wl = W.Workload("bwdvideo", seqs, 960, 960, 32, 2, 24, "bf16", (0.8, 1.2))
    inp = W.make_inputs(wl, 3)
    dO = torch.from_numpy(rand((960, 32, 24), 10)).to(torch.bfloat16)
    dq, dk, dv, _ = gpu_fwd_bwd(wl, inp, dO)
    mask = oracle.video_mask(wl.seqs, wl.nq, wl.nk)
    qn, kn = oracle_prologue(wl, inp)
    gq, gk, gv = oracle.attention_backward(qn, kn, np64(inp.v), np64(dO), mask, ops.LN2)
    compare(np64(dq), gq, "bf16", "dQ")
    compare(np64(dk), gk, "bf16", "dK")
    compare(np64(dv), gv, "bf16", "dV")


def test_bwd_full_size_magi45b():
    # the 4.5B-shaped layer at full size in the benchmark's configuration
    # (split key tiles and the partial-slot reduce included): every dQ row of
    # one KV group's 16 heads and every key's dK, dV of that group against
    # the oracle (rows in blocks; dK, dV summed over them), plus sampled dQ
    # rows over all 128 heads
    wl = W.make_workload("magi4.5b")
    note("bwd full size magi4.5b: inputs")
    inp = W.make_inputs(wl, 0)
    dO = torch.from_numpy(rand((wl.nq, wl.hq, wl.head_dim), 31)).to(torch.bfloat16)
    note("bwd full size magi4.5b: GPU forward + backward")
    dq, dk, dv, plan = gpu_fwd_bwd(wl, inp, dO)
    assert plan.num_slots > 0 and plan.host["kreduce"].shape[0] > 0, "the split dK/dV path must run"
    note(f"bwd full size magi4.5b: oracle ({plan.num_slots} partial slots on the GPU)")
    qn, kn = oracle_prologue(wl, inp)
    v64, do64 = np64(inp.v), np64(dO)
    mask = oracle.video_mask(wl.seqs, wl.nq, wl.nk)
    g, G = 5, wl.hq // wl.hkv
    hs = slice(g * G, (g + 1) * G)
    gq = np.zeros((wl.nq, G, wl.head_dim))
    gk = np.zeros((wl.nk, 1, wl.head_dim))
    gv = np.zeros((wl.nk, 1, wl.head_dim))
    for r0 in range(0, wl.nq, 720):
        rs = slice(r0, r0 + 720)
        a, b, c = oracle.attention_backward(qn[rs, hs], kn[:, g:g + 1], v64[:, g:g + 1], do64[rs, hs], mask[rs],
                                            ops.LN2)
        gq[rs], gk, gv = a, gk + b, gv + c
    compare(np64(dq[:, hs]), gq, "bf16", f"dQ group {g}")
    compare(np64(dk[:, g]), gk[:, 0], "bf16", f"dK group {g}")
    compare(np64(dv[:, g]), gv[:, 0], "bf16", f"dV group {g}")
    rows = W.sample_rows(wl, 48, 1)
    a, _, _ = oracle.attention_backward(qn[rows], kn, v64, do64[rows], mask[rows], ops.LN2)
    compare(np64(dq[rows]), a, "bf16", "dQ sampled rows, all heads")


def test_bwd_full_size_magi24b():
    # the 24B-shaped layer at full size: sampled dQ rows over all heads
    # against the oracle, and two sums that hold at any size for every KV
    # group (every row sees a key): sum_k dV[k] = sum over the group's rows
    # and heads of dO, and sum_k dK[k] = 0 (sum_k dS = dO.O - delta = 0 per row)
    wl = W.make_workload("magi24b")
    note("bwd full size magi24b: inputs")
    inp = W.make_inputs(wl, 0)
    dO = torch.from_numpy(rand((wl.nq, wl.hq, wl.head_dim), 41)).to(torch.bfloat16)
    note("bwd full size magi24b: GPU forward + backward")
    dq, dk, dv, plan = gpu_fwd_bwd(wl, inp, dO)
    assert plan.num_slots > 0
    rows = W.sample_rows(wl, 24, 2)
    note(f"bwd full size magi24b: oracle on {len(rows)} rows")
    qn, kn = oracle_prologue(wl, inp, rows)
    mask = oracle.video_mask(wl.seqs, wl.nq, wl.nk, rows)
    a, _, _ = oracle.attention_backward(qn, kn, np64(inp.v), np64(dO[rows]), mask, ops.LN2)
    compare(np64(dq[rows]), a, "bf16", "dQ sampled rows, all heads")
    G = wl.hq // wl.hkv
    do_sum = dO.double().view(wl.nq, wl.hkv, G, wl.head_dim).sum(dim=(0, 2)).numpy()
    dv_sum = dv.double().sum(dim=0).cpu().numpy()
    dk_sum = dk.double().sum(dim=0).cpu().numpy()
    scale_v = np.linalg.norm(do_sum)
    err_v = np.linalg.norm(dv_sum - do_sum) / scale_v
    # against the sum of |dK| entries: cancellation leaves rounding of that order
    err_k = np.abs(dk_sum).max() / dk.double().abs().sum(dim=0).max().item()
    note(f"sum dV vs sum dO rel {err_v:.3e}; |sum dK| / sum |dK| {err_k:.3e}")
    assert err_v <= 1e-2 and err_k <= 1e-2


def test_bwd_full_size_varlen():
    # the packed varlen layer at full size (6 videos of 5-15 chunks x 2400
    # tokens, 10 chunks at KV range 3, 129,600 tokens, split key tiles):
    # sampled dQ rows of every video over all heads against the oracle, which
    # is given only the row's own video (its mask is empty elsewhere), and
    # per video and KV group the sums that hold at any size when every row
    # sees a key: sum_k dV[k] over the video's keys = sum of the group's dO
    # over the video's rows, sum_k dK[k] = 0
    wl = W.make_workload("varlen")
    note("bwd full size varlen: inputs")
    inp = W.make_inputs(wl, 0)
    dO = torch.from_numpy(rand((wl.nq, wl.hq, wl.head_dim), 51)).to(torch.bfloat16)
    note("bwd full size varlen: GPU forward + backward")
    dq, dk, dv, plan = gpu_fwd_bwd(wl, inp, dO)
    assert plan.num_slots > 0
    G = wl.hq // wl.hkv
    rng = np.random.Generator(np.random.PCG64(52))
    v64 = np64(inp.v)
    for vi, s in enumerate(wl.seqs):
        q0, q1 = s.q_offset, s.q_offset + s.num_q_chunks * s.chunk_len
        k0, k1 = s.k_offset, s.k_offset + s.num_kv_chunks * s.chunk_len
        rows = np.unique(np.concatenate([[q0, q1 - 1], rng.integers(q0, q1, size=3)])).astype(np.int64)
        note(f"bwd full size varlen: video {vi} ({s.num_q_chunks} chunks), rows {rows.tolist()}")
        qn, kn = oracle_prologue(wl, inp, rows)
        mask = oracle.video_mask(wl.seqs, wl.nq, wl.nk, rows)[:, k0:k1]
        assert mask.any(axis=1).all()
        a, _, _ = oracle.attention_backward(qn, kn[k0:k1], v64[k0:k1], np64(dO[rows]), mask, ops.LN2)
        compare(np64(dq[rows]), a, "bf16", f"dQ video {vi}, sampled rows, all heads")
        do_sum = dO[q0:q1].double().view(q1 - q0, wl.hkv, G, wl.head_dim).sum(dim=(0, 2)).numpy()
        dv_sum = dv[k0:k1].double().sum(dim=0).cpu().numpy()
        dk_sum = dk[k0:k1].double().sum(dim=0).cpu().numpy()
        err_v = np.linalg.norm(dv_sum - do_sum) / np.linalg.norm(do_sum)
        err_k = np.abs(dk_sum).max() / dk[k0:k1].double().abs().sum(dim=0).max().item()
        note(f"video {vi}: sum dV vs sum dO rel {err_v:.3e}; |sum dK| / sum |dK| {err_k:.3e}")
        assert err_v <= 1e-2 and err_k <= 1e-2


def test_bwd_bitwise_deterministic():
    note("bwd determinism")
    d, G, hkv = 24, 16, 2
    sl = ops.build_slices([W.SeqDesc(70, 3, 3, 0, 0, (-1, -1, -1), 1, 1, 70)])
    q, k, v, dO = (torch.from_numpy(x).to(torch.bfloat16).to(DEV) for x in
                   (rand((210, G * hkv, d), 11), rand((210, hkv, d), 12), rand((210, hkv, d), 13),
                    rand((210, G * hkv, d), 14)))
    plan = ops.make_plan(sl, 210, 210, G * hkv, hkv, d, torch.bfloat16, backward=True)
    O, L = ops.ffa_fwd(q, k, v, plan)
    a = ops.ffa_bwd(q, k, v, O, dO, L, plan)
    b = ops.ffa_bwd(q, k, v, O, dO, L, plan)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("d", [24, 48])
def test_bwd_group_major_kv_identical(d):
    # K, V (and so dK, dV) stored group-major: only addressing changes, so the
    # gradients equal the token-major run's bit for bit
    note(f"bwd group-major K/V d={d}")
    G, hkv = 16, 2
    sl = ops.build_slices([W.SeqDesc(70, 3, 3, 0, 0, (-1, -1, -1), 1, 1, 70)])
    q, k, v, dO = (torch.from_numpy(x).to(torch.bfloat16).to(DEV) for x in
                   (rand((210, G * hkv, d), 51), rand((210, hkv, d), 52), rand((210, hkv, d), 53),
                    rand((210, G * hkv, d), 54)))
    plan = ops.make_plan(sl, 210, 210, G * hkv, hkv, d, torch.bfloat16, backward=True)
    O, L = ops.ffa_fwd(q, k, v, plan)
    a = ops.ffa_bwd(q, k, v, O, dO, L, plan)
    kg = ops.kv_group_major(210, hkv, d, torch.bfloat16)
    vg = ops.kv_group_major(210, hkv, d, torch.bfloat16)
    kg.copy_(k)
    vg.copy_(v)
    b = ops.ffa_bwd(q, kg, vg, O, dO, L, plan)
    torch.cuda.synchronize()
    assert b[1].stride() == kg.stride() and b[2].stride() == vg.stride()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("d", [24, 48])
@pytest.mark.parametrize("G", [16, 3])
def test_bwd_strided_rows_identical(d, G):
    # Q, O, dO and dQ as views into wider rows (token stride above heads x d,
    # as for a fused projection): only addressing changes, so outputs and
    # gradients equal the contiguous run's bit for bit.  G = 3 leaves the
    # last row of every 64-row Q/dO tile of the dK/dV pass empty.
    note(f"bwd row-strided Q/O/dO d={d} G={G}")
    hkv, n, pad = 2, 210, 3
    hq = G * hkv
    sl = ops.build_slices([W.SeqDesc(70, 3, 3, 0, 0, (-1, -1, -1), 1, 1, 70)])
    q, k, v, dO = (torch.from_numpy(x).to(torch.bfloat16).to(DEV) for x in
                   (rand((n, hq, d), 61), rand((n, hkv, d), 62), rand((n, hkv, d), 63), rand((n, hq, d), 64)))
    plan = ops.make_plan(sl, n, n, hq, hkv, d, torch.bfloat16, backward=True)
    O, L = ops.ffa_fwd(q, k, v, plan)
    a = ops.ffa_bwd(q, k, v, O, dO, L, plan)

    def wide(x=None):
        w = torch.full((n, hq + pad, d), float("nan"), dtype=torch.bfloat16, device=DEV)
        if x is not None:
            w[:, :hq] = x
        return w[:, :hq]

    qs, dOs, Os, dqs = wide(q), wide(dO), wide(), wide()
    assert qs.stride(0) == (hq + pad) * d and not qs.is_contiguous()
    Ls = torch.empty_like(L)
    ops.ffa_fwd(qs, k, v, plan, out=Os, lse=Ls)
    b = ops.ffa_bwd(qs, k, v, Os, dOs, Ls, plan, dq=dqs)
    torch.cuda.synchronize()
    assert torch.equal(O, Os) and torch.equal(L, Ls)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("case", range(6))
def test_bwd_fuzz_raw_slices(case):
    # seeded random shapes, group sizes and slice lists against the oracle's gradients
    from test_gpu_parity import random_slices
    rng = np.random.Generator(np.random.PCG64(5000 + case))
    d, hkv = int(rng.choice([24, 48])), int(rng.choice([1, 2]))
    G = int(rng.choice([1, 3, 8, 16, 64]))
    nq, nk = int(rng.integers(1, 200)), int(rng.integers(1, 260))
    sl = random_slices(rng, nq, nk)
    note(f"bwd fuzz case {case}: d={d} G={G} hkv={hkv} nq={nq} nk={nk} slices={len(sl)}")
    bwd_case(rand((nq, G * hkv, d), 6000 + case), rand((nk, hkv, d), 7000 + case), rand((nk, hkv, d), 8000 + case),
             rand((nq, G * hkv, d), 9000 + case), sl, "bf16")



@pytest.mark.parametrize("case", range(6))
def test_bwd_fuzz_all_slice_types(case):
    # random slices of all four types, lower key bounds included
    from test_gpu_parity import random_slices
    rng = np.random.Generator(np.random.PCG64(5100 + case))
    d, hkv = int(rng.choice([24, 48])), int(rng.choice([1, 2]))
    G = int(rng.choice([1, 3, 8, 16]))
    nq, nk = int(rng.integers(1, 200)), int(rng.integers(1, 260))
    sl = random_slices(rng, nq, nk, all_types=True)
    note(f"bwd all-types fuzz case {case}: d={d} G={G} hkv={hkv} nq={nq} nk={nk} slices={len(sl)}")
    args = (rand((nq, G * hkv, d), 6100 + case), rand((nk, hkv, d), 7100 + case), rand((nk, hkv, d), 8100 + case),
            rand((nq, G * hkv, d), 9100 + case), sl)
    bwd_case(*args, "bf16")
    bwd_case(*args, "fp32")


@pytest.mark.parametrize("d", [24, 48])
@pytest.mark.parametrize("window", [5, 160])
def test_bwd_sliding_window(d, window):
    # gradients of causal sliding-window attention over two packed
    # sequences, long enough that key tiles are split into parts
    note(f"bwd sliding window d={d} w={window}")
    spec = [(600, window, 0, 0), (300, window, 600, 600)]
    sl = ops.build_window_slices(spec)
    n = 900
    bwd_case(rand((n, 32, d), 71), rand((n, 2, d), 72), rand((n, 2, d), 73), rand((n, 32, d), 74), sl, "bf16")

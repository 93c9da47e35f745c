"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Tolerances (bf16 storage): max-abs <= 2e-2 and relative L2 <= 5e-3 on O;
fp32: max-abs <= 1e-5.  LSE is checked with max-abs 1e-2 (bf16) / 1e-5
(fp32).  Full-size workloads run the kernel at full size, in the launch
configuration the benchmark times, and compare a seeded sample of rows (all
heads) that the oracle computes one by one; small cases compare every row.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from block_causal_attention_amd import _lib, ops

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = {"bf16": dict(max_abs=2e-2, rel_l2=5e-3, lse=1e-2), "fp32": dict(max_abs=1e-5, rel_l2=1e-5, lse=1e-5)}


def note(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def compare(got, want, kind, what="O"):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    tol = TOL[kind]
    if what == "LSE":
        fin = np.isfinite(want)
        assert np.array_equal(fin, np.isfinite(got)), "LSE -inf pattern differs"
        if fin.any():
            err = np.abs(got[fin] - want[fin]).max()
            assert err <= tol["lse"], f"LSE max-abs {err:.3e}"
        return
    diff = got - want
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    den = float(np.linalg.norm(want))
    rel = float(np.linalg.norm(diff)) / den if den > 0 else float(np.linalg.norm(diff))
    note(f"{what}: max-abs {max_abs:.3e} rel-L2 {rel:.3e}")
    assert max_abs <= tol["max_abs"], f"{what} max-abs {max_abs:.3e} > {tol['max_abs']}"
    assert rel <= tol["rel_l2"], f"{what} rel-L2 {rel:.3e} > {tol['rel_l2']}"


def dev_inputs(wl, inp):
    g = lambda t: t.to(DEV)
    return dict(q=g(inp.q), k=g(inp.k), v=g(inp.v), gq=g(inp.gain_q), gk=g(inp.gain_k), pq=g(inp.pos_q),
                pk=g(inp.pos_k), base=torch.tensor(wl.rope_base, dtype=torch.float32, device=DEV))


def gpu_forward(wl, d, group_major=True):
    """prologue (Q and K, softmax scale folded into K; K and V written
    group-major) then FFA over the builder's slices, exactly as the benchmark
    runs it (group_major=False keeps K and V token-major)."""
    knm = torch.empty(wl.hkv, dtype=torch.float32, device=DEV)
    if group_major:
        kg = ops.kv_group_major(wl.nk, wl.hkv, wl.head_dim, d["k"].dtype)
        qh, kh, vh = ops.qknorm_rope(d["q"], d["k"], d["gq"], d["gk"], d["pq"], d["pk"], d["base"], wl.eps,
                                     k_out=kg, k_scale=wl.softmax_scale * ops.LOG2E, k_norm_max=knm, v=d["v"])
    else:
        qh, kh = ops.qknorm_rope(d["q"], d["k"], d["gq"], d["gk"], d["pq"], d["pk"], d["base"], wl.eps,
                                 k_scale=wl.softmax_scale * ops.LOG2E, k_norm_max=knm)
        vh = d["v"]
    plan = ops.plan_for_videos(wl.seqs, wl.nq, wl.nk, wl.hq, wl.hkv, wl.head_dim, d["q"].dtype)
    O, L = ops.ffa_fwd(qh, kh, vh, plan, softmax_scale=ops.LN2, k_norm_max=knm)
    torch.cuda.synchronize()
    return qh, kh, O, L


def np64(t):
    return t.detach().to("cpu", torch.float64).numpy()


# --------------------------------------------------------------------------- prologue

@pytest.mark.parametrize("name", ["tiny", "magi4.5b", "magi24b"])
def test_prologue_matches_oracle(name):
    note(f"prologue {name}")
    wl = W.make_workload(name)
    inp = W.make_inputs(wl, 0)
    d = dev_inputs(wl, inp)
    qh, kh = ops.qknorm_rope(d["q"], d["k"], d["gq"], d["gk"], d["pq"], d["pk"], d["base"], wl.eps)
    torch.cuda.synchronize()
    inv = oracle.rope_inv_freq(wl.rope_base, wl.head_dim)
    rows = np.arange(wl.nq) if wl.nq <= 6000 else W.sample_rows(wl, 2000)
    want_q = oracle.rope_3d(oracle.qk_norm(np64(inp.q[rows]), np64(inp.gain_q), wl.eps), inp.pos_q[rows].numpy(), inv)
    want_k = oracle.rope_3d(oracle.qk_norm(np64(inp.k), np64(inp.gain_k), wl.eps), inp.pos_k.numpy(), inv)
    compare(np64(qh)[rows], want_q, wl.dtype, "q_hat")
    compare(np64(kh), want_k, wl.dtype, "k_hat")


def test_prologue_output_scale():
    note("prologue with q/k output scales")
    wl = W.custom_block_causal(2, 2, 4, 5, 16, 2, 24)
    inp = W.make_inputs(wl, 4)
    d = dev_inputs(wl, inp)
    qh, kh = ops.qknorm_rope(d["q"], d["k"], d["gq"], d["gk"], d["pq"], d["pk"], d["base"], wl.eps,
                             q_scale=0.5, k_scale=0.2946)
    torch.cuda.synchronize()
    inv = oracle.rope_inv_freq(wl.rope_base, 24)
    wq = oracle.rope_3d(oracle.qk_norm(np64(inp.q), np64(inp.gain_q), wl.eps), inp.pos_q.numpy(), inv) * 0.5
    wk = oracle.rope_3d(oracle.qk_norm(np64(inp.k), np64(inp.gain_k), wl.eps), inp.pos_k.numpy(), inv) * 0.2946
    compare(np64(qh), wq, "bf16", "q_hat")
    compare(np64(kh), wk, "bf16", "k_hat")


def test_prologue_key_norm_bound():
    note("prologue key-norm bound")
    wl = W.custom_block_causal(2, 2, 4, 5, 16, 4, 48)
    inp = W.make_inputs(wl, 6)
    d = dev_inputs(wl, inp)
    rng = np.random.Generator(np.random.PCG64(6))
    # per-head gains (the gain stride is shared by Q and K)
    gq = torch.from_numpy(rng.uniform(0.5, 1.5, (16, 48)).astype(np.float32)).to(DEV)
    gk = torch.from_numpy(rng.uniform(0.5, 1.5, (4, 48)).astype(np.float32)).to(DEV)
    knm = torch.full((4,), float("nan"), dtype=torch.float32, device=DEV)
    _, kh = ops.qknorm_rope(d["q"], d["k"], gq, gk, d["pq"], d["pk"], d["base"], wl.eps,
                            k_scale=0.3, k_norm_max=knm)
    torch.cuda.synchronize()
    norms = kh.float().norm(dim=-1).amax(dim=0).cpu().numpy()
    bound = knm.cpu().numpy()
    want = 48 ** 0.5 * gk.abs().amax(dim=1).cpu().numpy() * 0.3 * (1 + 2 ** -7)
    np.testing.assert_allclose(bound, want, rtol=1e-6)
    assert (norms <= bound).all() and (norms > 0.5 * bound).all()


def test_prologue_per_head_gain_in_place_and_strided():
    note("prologue per-head gains, in place, strided view")
    wl = W.custom_block_causal(2, 2, 3, 4, 16, 2, 48)
    inp = W.make_inputs(wl, 7)
    rng = np.random.Generator(np.random.PCG64(7))
    gq = rng.uniform(0.5, 1.5, (16, 48)).astype(np.float32)
    base = torch.tensor([1e4, 3e3, 5e2], dtype=torch.float32, device=DEV)
    # Q lives inside a wider row (a fused projection layout): row stride 20 heads
    buf = torch.zeros(wl.nq, 20, 48, dtype=torch.bfloat16, device=DEV)
    buf[:, 2:18] = inp.q.to(DEV)
    qv = buf[:, 2:18]
    ops.qknorm_rope(qv, None, torch.from_numpy(gq).to(DEV), None, inp.pos_q.to(DEV), None, base, 1e-6, q_out=qv)
    torch.cuda.synchronize()
    want = oracle.rope_3d(oracle.qk_norm(np64(inp.q), gq, 1e-6), inp.pos_q.numpy(),
                          oracle.rope_inv_freq((1e4, 3e3, 5e2), 48))
    compare(np64(qv), want, "bf16", "q_hat")
    assert torch.count_nonzero(buf[:, :2]) == 0 and torch.count_nonzero(buf[:, 18:]) == 0


@pytest.mark.parametrize("d", [24, 48])
def test_prologue_more_heads_than_threads(d):
    # 320 query heads and 40 key heads: a Q token has more heads than a
    # 256-thread block has threads, so threads take a second vector of the
    # token (at d = 48 after the first was loaded before the rotation table)
    note(f"prologue with 320 heads, d={d}")
    n, hq, hk = 37, 320, 40
    rng = np.random.Generator(np.random.PCG64(60 + d))
    q = rng.standard_normal((n, hq, d)).astype(np.float32)
    k = rng.standard_normal((n, hk, d)).astype(np.float32)
    gq = rng.uniform(0.8, 1.2, d).astype(np.float32)
    gk = rng.uniform(0.8, 1.2, d).astype(np.float32)
    pos = rng.integers(0, 50, (n, 3)).astype(np.int32)
    base = (1e4, 2e3, 7e2)
    dv = lambda x: torch.from_numpy(x).to(DEV)
    qd, kd = dv(q).to(torch.bfloat16), dv(k).to(torch.bfloat16)
    qh, kh = ops.qknorm_rope(qd, kd, dv(gq), dv(gk), dv(pos), dv(pos),
                             torch.tensor(base, dtype=torch.float32, device=DEV), 1e-6)
    torch.cuda.synchronize()
    inv = oracle.rope_inv_freq(base, d)
    compare(np64(qh), oracle.rope_3d(oracle.qk_norm(np64(qd), gq, 1e-6), pos, inv), "bf16", "q_hat")
    compare(np64(kh), oracle.rope_3d(oracle.qk_norm(np64(kd), gk, 1e-6), pos, inv), "bf16", "k_hat")


# --------------------------------------------------------------------------- attention alone

def ffa_case(q, k, v, slices, kind, scale=None, check_lse=True, knm=None):
    nq, hq, dd = q.shape
    nk, hkv = k.shape[0], k.shape[1]
    tdt = torch.bfloat16 if kind == "bf16" else torch.float32
    qd, kd, vd = (torch.from_numpy(x).to(tdt).to(DEV) for x in (q, k, v))
    plan = ops.make_plan(np.asarray(slices, np.int32).reshape(-1, 5), nq, nk, hq, hkv, dd, tdt)
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((nq, hq), float("nan"), dtype=torch.float32, device=DEV)
    kn = None if knm is None else torch.tensor(knm, dtype=torch.float32, device=DEV)
    O, L = ops.ffa_fwd(qd, kd, vd, plan, softmax_scale=scale, out=out, lse=lse, k_norm_max=kn)
    torch.cuda.synchronize()
    mask = oracle.slices_mask([tuple(int(x) for x in s) for s in slices], nq, nk) if len(slices) else \
        np.zeros((nq, nk), bool)
    qr, kr, vr = (np64(t) for t in (qd, kd, vd))
    Ow, Lw = oracle.attention(qr, kr, vr, mask, scale if scale else dd ** -0.5)
    assert not torch.isnan(O).any(), "output rows left unwritten"
    compare(np64(O), Ow, kind)
    if check_lse:
        compare(np64(L), Lw, kind, "LSE")
    return O, L


def rand(shape, seed, scale=1.0):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape).astype(np.float32) * scale


@pytest.mark.parametrize("d", [24, 48])
@pytest.mark.parametrize("G", [16, 4, 1, 3])
def test_ffa_block_causal_ragged(d, G):
    # 3 chunks of 37 tokens: no tile or 64-key boundary lines up
    note(f"ffa block-causal ragged d={d} G={G}")
    hkv = 2
    seqs = [W.SeqDesc(37, 3, 3, 0, 0, (-1, -1, -1), 1, 1, 37)]
    sl = ops.build_slices(seqs)
    q, k, v = rand((111, G * hkv, d), 1), rand((111, hkv, d), 2), rand((111, hkv, d), 3)
    ffa_case(q, k, v, sl, "bf16")


@pytest.mark.parametrize("d", [24, 48])
def test_ffa_causal_and_irregular_slices(d):
    note(f"ffa irregular slices d={d}")
    nq, nk = 150, 210
    slices = [
        (0, 70, 0, 70, _lib.MASK_CAUSAL),          # square causal
        (70, 100, 0, 40, _lib.MASK_FULL),          # two k ranges for one q band
        (70, 100, 60, 130, _lib.MASK_CAUSAL),      # wide causal, bottom-right aligned
        (100, 140, 130, 150, _lib.MASK_CAUSAL),    # tall causal: early rows see nothing
        # rows 140..149 are covered by no slice: O = 0, LSE = -inf
    ]
    q, k, v = rand((nq, 16, d), 4), rand((nk, 1, d), 5), rand((nk, 1, d), 6)
    O, L = ffa_case(q, k, v, np.array(slices), "bf16")
    assert torch.all(O[140:] == 0) and torch.all(torch.isneginf(L[140:]))


@pytest.mark.parametrize("d", [24, 48])
def test_ffa_prescaled_keys(d):
    # K stored pre-multiplied by scale*log2(e) and softmax_scale = ln 2: the
    # kernel takes its no-multiply path; the oracle sees the same rounded K
    note(f"ffa prescaled K d={d}")
    c = d ** -0.5 * ops.LOG2E
    k = torch.from_numpy(rand((300, 2, d), 21) * c).to(torch.bfloat16).float().numpy()
    seqs = [W.SeqDesc(100, 3, 3, 0, 0, (-1, -1, 1), 1, 1, 100)]
    ffa_case(rand((300, 32, d), 20), k, rand((300, 2, d), 22), ops.build_slices(seqs), "bf16", scale=ops.LN2)


@pytest.mark.parametrize("d", [24, 48])
@pytest.mark.parametrize("loose", [False, True])
def test_ffa_key_norm_bound(d, loose):
    # the bounded reference (no running max) must give the online-max result;
    # a bound too loose to use (> 60 in log2 units) falls back to the running max
    note(f"ffa key-norm bound d={d} loose={loose}")
    hkv = 2
    q, k, v = rand((150, 32, d), 30 + d), rand((150, hkv, d), 31), rand((150, hkv, d), 32)
    kb = torch.from_numpy(k).to(torch.bfloat16).float().norm(dim=-1).amax(dim=0).numpy() * 1.001
    if loose:
        kb = kb * 40.0
    seqs = [W.SeqDesc(50, 3, 3, 0, 0, (-1, -1, 1), 1, 1, 50)]
    ffa_case(q, k, v, ops.build_slices(seqs), "bf16", knm=kb)
    ffa_case(q, k, v, np.array([(0, 150, 0, 150, 1)]), "bf16", knm=kb)


def test_ffa_fp32_tiny_full():
    note("ffa fp32 tiny")
    wl = W.make_workload("tiny")
    inp = W.make_inputs(wl, 0)
    ffa_case(inp.q.numpy(), inp.k.numpy(), inp.v.numpy(), ops.build_slices(wl.seqs), "fp32")


def test_ffa_fp32_irregular():
    note("ffa fp32 irregular")
    slices = np.array([(0, 40, 0, 40, 1), (40, 70, 10, 30, 0), (40, 70, 35, 80, 1)])
    ffa_case(rand((80, 8, 48), 8), rand((80, 2, 48), 9), rand((80, 2, 48), 10), slices, "fp32", scale=0.3)


def test_ffa_no_keys_and_scale():
    note("ffa nk=0 and explicit scale")
    q = torch.randn(20, 16, 24, device=DEV).to(torch.bfloat16)
    k = torch.zeros(0, 1, 24, device=DEV, dtype=torch.bfloat16)
    plan = ops.make_plan(np.zeros((0, 5), np.int32), 20, 0, 16, 1, 24, torch.bfloat16)
    O, L = ops.ffa_fwd(q, k, k, plan)
    torch.cuda.synchronize()
    assert torch.all(O == 0) and torch.all(torch.isneginf(L))
    sl = np.array([(0, 30, 0, 50, 0)])
    ffa_case(rand((30, 16, 24), 11, 3.0), rand((50, 1, 24), 12, 3.0), rand((50, 1, 24), 13), sl, "bf16", scale=0.05)


def test_empty_query_and_key_sets():
    # no query tokens at all (nothing to launch), and window / band slices
    # whose rows see no key (an empty band, a window slice over no keys)
    note("empty query set, empty bands")
    q0 = torch.zeros(0, 16, 24, device=DEV, dtype=torch.bfloat16)
    k = torch.randn(7, 1, 24, device=DEV).to(torch.bfloat16)
    plan = ops.make_plan(np.zeros((0, 5), np.int32), 0, 7, 16, 1, 24, torch.bfloat16)
    O, L = ops.ffa_fwd(q0, k, k, plan)
    qh, kh = ops.qknorm_rope(q0, k[:0], torch.ones(24, device=DEV), torch.ones(24, device=DEV),
                             torch.zeros(0, 3, dtype=torch.int32, device=DEV),
                             torch.zeros(0, 3, dtype=torch.int32, device=DEV),
                             torch.full((3,), 1e4, device=DEV), 1e-6)
    torch.cuda.synchronize()
    assert O.shape == (0, 16, 24) and L.shape == (0, 16) and qh.shape == (0, 16, 24) and kh.shape == (0, 1, 24)
    # a band narrower than its query range shows no row a key (width
    # 5 - 9 + 1 < 1), next to a band that does; rows of the empty band get
    # O = 0 and LSE = -inf
    sl = np.array([(0, 9, 0, 5, 3), (9, 20, 5, 20, 3)])
    ffa_case(rand((20, 16, 24), 21), rand((20, 1, 24), 22), rand((20, 1, 24), 23), sl, "bf16")
    ffa_case(rand((20, 16, 48), 24), rand((20, 1, 48), 25), rand((20, 1, 48), 26), sl, "fp32")


def random_slices(rng, nq, nk, all_types=False):
    """Disjoint AttnSlices: query bands, each with a few disjoint key ranges,
    FULL or CAUSAL (bottom-right aligned; with all_types also INVCAUSAL and
    BICAUSAL), some bands and gaps left empty."""
    slices = []
    q = 0
    while q < nq:
        qe = min(nq, q + int(rng.integers(1, 60)))
        if rng.random() < 0.85:
            k = int(rng.integers(0, 8))
            while k < nk:
                ke = min(nk, k + int(rng.integers(1, 90)))
                t = int(rng.integers(0, 4)) if all_types else int(rng.random() < 0.4)
                slices.append((q, qe, k, ke, t))
                k = ke + int(rng.integers(0, 20))
        q = qe + int(rng.integers(0, 5))
    return np.array(slices, np.int32).reshape(-1, 5)


@pytest.mark.parametrize("case", range(10))
def test_ffa_fuzz_raw_slices(case):
    # seeded random shapes, group sizes and slice lists against the oracle
    rng = np.random.Generator(np.random.PCG64(1000 + case))
    d, hkv = int(rng.choice([24, 48])), int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2, 3, 5, 8, 16, 32]))
    nq, nk = int(rng.integers(1, 260)), int(rng.integers(1, 330))
    sl = random_slices(rng, nq, nk)
    note(f"ffa fuzz case {case}: d={d} G={G} hkv={hkv} nq={nq} nk={nk} slices={len(sl)}")
    ffa_case(rand((nq, G * hkv, d), 2000 + case), rand((nk, hkv, d), 3000 + case), rand((nk, hkv, d), 4000 + case),
             sl, "bf16")


@pytest.mark.parametrize("case", range(8))
def test_ffa_fuzz_all_slice_types(case):
    # random slices of all four types (lower key bounds included), bf16 with
    # and without the key-norm bound, and the fp32 kernel
    rng = np.random.Generator(np.random.PCG64(1100 + case))
    d, hkv = int(rng.choice([24, 48])), int(rng.choice([1, 2]))
    G = int(rng.choice([1, 3, 8, 16]))
    nq, nk = int(rng.integers(1, 260)), int(rng.integers(1, 330))
    sl = random_slices(rng, nq, nk, all_types=True)
    note(f"ffa all-types fuzz case {case}: d={d} G={G} hkv={hkv} nq={nq} nk={nk} slices={len(sl)}")
    q, k, v = rand((nq, G * hkv, d), 2100 + case), rand((nk, hkv, d), 3100 + case), rand((nk, hkv, d), 4100 + case)
    ffa_case(q, k, v, sl, "bf16")
    kb = np.linalg.norm(k.astype(np.float64), axis=-1).max(axis=0) * 1.01
    ffa_case(q, k, v, sl, "bf16", knm=kb)
    ffa_case(q, k, v, sl, "fp32")


def window_forward(wl, inp, spec, d):
    """prologue + FFA over sliding-window slices, in the benchmark's
    configuration (scale folded into K, K/V group-major, key-norm bound)"""
    knm = torch.empty(wl.hkv, dtype=torch.float32, device=DEV)
    kg = ops.kv_group_major(wl.nk, wl.hkv, wl.head_dim, d["k"].dtype)
    qh, kh, vh = ops.qknorm_rope(d["q"], d["k"], d["gq"], d["gk"], d["pq"], d["pk"], d["base"], wl.eps,
                                 k_out=kg, k_scale=wl.softmax_scale * ops.LOG2E, k_norm_max=knm, v=d["v"])
    plan = ops.make_plan(ops.build_window_slices(spec), wl.nq, wl.nk, wl.hq, wl.hkv, wl.head_dim, d["q"].dtype)
    O, L = ops.ffa_fwd(qh, kh, vh, plan, softmax_scale=ops.LN2, k_norm_max=knm)
    torch.cuda.synchronize()
    return O, L


@pytest.mark.parametrize("d", [24, 48])
@pytest.mark.parametrize("window", [1, 37, 300, 720])
def test_sliding_window_end_to_end(d, window):
    # causal sliding-window attention over the tokens of a packed video
    # (3 chunks x 240 tokens) and a second, shorter sequence, QK-Norm and 3D
    # RoPE applied by the prologue, against the oracle's window mask
    note(f"sliding window d={d} w={window}")
    wl = W.custom_packed([(3, 2, 10, 12, None), (1, 2, 7, 9, None)], 32, 2, d)
    inp = W.make_inputs(wl, 0)
    dd = dev_inputs(wl, inp)
    spec = [(720, window, 0, 0), (wl.nq - 720, window, 720, 720)]
    O, L = window_forward(wl, inp, spec, dd)
    mask = oracle.window_mask(spec, wl.nq, wl.nk)
    Ow, Lw = oracle.forward(np64(inp.q), np64(inp.k), np64(inp.v), np64(inp.gain_q), np64(inp.gain_k),
                            inp.pos_q.numpy(), inp.pos_k.numpy(), wl.rope_base, wl.eps, mask, wl.softmax_scale)
    compare(np64(O), Ow, "bf16")
    # LSE: with a handful of visible keys the rounding is not averaged out.
    # q_hat and scale * log2(e) * k_hat are stored in bf16 (unit roundoff
    # u = 2^-8), so a logit moves by up to 2u * scale * |q_hat| * |k_hat|;
    # the denominator sums P after its own bf16 rounding, which moves
    # ln(sum P) by up to u.  Per row the bound is that sum, at least the
    # usual 1e-2.
    inv = oracle.rope_inv_freq(wl.rope_base, wl.head_dim)
    qn = np.linalg.norm(oracle.rope_3d(oracle.qk_norm(np64(inp.q), np64(inp.gain_q), wl.eps),
                                       inp.pos_q.numpy(), inv), axis=-1)
    kn = np.linalg.norm(oracle.rope_3d(oracle.qk_norm(np64(inp.k), np64(inp.gain_k), wl.eps),
                                       inp.pos_k.numpy(), inv), axis=-1).max(axis=0)
    u = 2.0 ** -8
    bound = np.maximum(1e-2, 2 * u * wl.softmax_scale * qn * np.repeat(kn, wl.hq // wl.hkv)[None, :] * 1.05 + u)
    Lg = np64(L)
    assert np.array_equal(np.isfinite(Lg), np.isfinite(Lw))
    err = np.abs(Lg - Lw)
    note(f"LSE: max-abs {err.max():.3e}, worst err/bound {(err / bound).max():.3f}")
    assert (err <= bound).all()


def test_sliding_window_large_sampled():
    # the 24B-shaped layer (8 chunks x 3600 tokens, 128/8 heads, d = 48) under
    # a 3600-token window: sampled rows against the oracle
    note("sliding window magi24b w=3600 sampled")
    wl = W.make_workload("magi24b")
    inp = W.make_inputs(wl, 0)
    dd = dev_inputs(wl, inp)
    spec = [(wl.nq, 3600, 0, 0)]
    O, L = window_forward(wl, inp, spec, dd)
    rows = W.sample_rows(wl, 192)
    mask = oracle.window_mask(spec, wl.nq, wl.nk, rows)
    keys = np.flatnonzero(mask.any(axis=0))
    Ow, Lw = oracle.forward(np64(inp.q[rows]), np64(inp.k[keys]), np64(inp.v[keys]), np64(inp.gain_q),
                            np64(inp.gain_k), inp.pos_q[rows].numpy(), inp.pos_k[keys].numpy(), wl.rope_base,
                            wl.eps, mask[:, keys], wl.softmax_scale)
    compare(np64(O)[rows], Ow, "bf16")
    compare(np64(L)[rows], Lw, "bf16", "LSE")


@pytest.mark.parametrize("d", [24, 48])
def test_ffa_largest_group(d):
    # 256 query heads over one KV group: one token per work item
    note(f"ffa G=256 d={d}")
    sl = ops.build_slices([W.SeqDesc(9, 3, 3, 0, 0, (-1, -1, -1), 1, 1, 9)])
    ffa_case(rand((27, 256, d), 60), rand((27, 1, d), 61), rand((27, 1, d), 62), sl, "bf16")


def to_group_major(t):
    """a copy of a token-major [n, heads, d] tensor stored group-major"""
    g = ops.kv_group_major(t.shape[0], t.shape[1], t.shape[2], t.dtype, t.device)
    g.copy_(t)
    return g


@pytest.mark.parametrize("d", [24, 48])
@pytest.mark.parametrize("bound", [False, True])
def test_kv_layouts_give_identical_results(d, bound):
    # only the addressing of K/V tiles differs between the layouts, so the
    # results must agree bit for bit (and the token-major run matches the
    # oracle in the tests above)
    note(f"ffa K/V group-major vs token-major d={d} bound={bound}")
    hkv, G = 2, 16
    seqs = [W.SeqDesc(70, 3, 3, 0, 0, (-1, -1, 1), 1, 1, 70)]
    sl = ops.build_slices(seqs)
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).to(DEV) for x in
               (rand((210, G * hkv, d), 40), rand((210, hkv, d), 41), rand((210, hkv, d), 42)))
    knm = k.float().norm(dim=-1).amax(dim=0) * 1.01 if bound else None
    plan = ops.make_plan(sl, 210, 210, G * hkv, hkv, d, torch.bfloat16)
    O1, L1 = ops.ffa_fwd(q, k, v, plan, k_norm_max=knm)
    kg, vg = to_group_major(k), to_group_major(v)
    assert kg.stride() == (d, 210 * d, 1)
    O2, L2 = ops.ffa_fwd(q, kg, vg, plan, k_norm_max=knm)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(L1, L2)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_timed_forward_identical_and_events_bracket_kernel(dtype):
    # magi_ffa_fwd_timed launches the same kernel, so the outputs agree bit
    # for bit; the events its dispatch records give a positive duration no
    # longer than the host's wall time around the call
    import time
    note(f"ffa timed entry point {dtype}")
    d, hkv, G = 24, 2, 16
    seqs = [W.SeqDesc(70, 3, 3, 0, 0, (-1, -1, 1), 1, 1, 70)]
    plan = ops.make_plan(ops.build_slices(seqs), 210, 210, G * hkv, hkv, d, dtype)
    q, k, v = (torch.from_numpy(x).to(dtype).to(DEV) for x in
               (rand((210, G * hkv, d), 50), rand((210, hkv, d), 51), rand((210, hkv, d), 52)))
    O1, L1 = ops.ffa_fwd(q, k, v, plan)
    evs = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    O2, L2 = ops.ffa_fwd(q, k, v, plan, events=evs)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
    ms = evs[0].elapsed_time(evs[1])
    assert 0.0 < ms <= wall_ms
    with pytest.raises(ValueError):
        ops.ffa_fwd(q, k, v, plan, events=(torch.cuda.Event(enable_timing=True),) * 2)  # never recorded


def test_kv_layouts_fp32_identical():
    note("ffa fp32 K/V group-major vs token-major")
    wl = W.make_workload("tiny")
    inp = W.make_inputs(wl, 0)
    q, k, v = (t.to(DEV) for t in (inp.q, inp.k, inp.v))
    plan = ops.make_plan(ops.build_slices(wl.seqs), wl.nq, wl.nk, wl.hq, wl.hkv, wl.head_dim, torch.float32)
    O1, L1 = ops.ffa_fwd(q, k, v, plan)
    O2, L2 = ops.ffa_fwd(q, to_group_major(k), to_group_major(v), plan)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(L1, L2)


@pytest.mark.parametrize("name", ["tiny", "magi4.5b"])
def test_prologue_group_major_output_and_v_copy(name):
    # group-major K output holds the same values as the token-major one; V is
    # moved unchanged; the key-norm bound does not depend on the layout
    note(f"prologue group-major K and V copy {name}")
    wl = W.make_workload(name)
    d = dev_inputs(wl, W.make_inputs(wl, 0))
    args = (d["q"], d["k"], d["gq"], d["gk"], d["pq"], d["pk"], d["base"], wl.eps)
    n1 = torch.empty(wl.hkv, dtype=torch.float32, device=DEV)
    n2 = torch.empty(wl.hkv, dtype=torch.float32, device=DEV)
    q1, k1 = ops.qknorm_rope(*args, k_scale=0.5, k_norm_max=n1)
    kg = ops.kv_group_major(wl.nk, wl.hkv, wl.head_dim, d["k"].dtype)
    q2, k2, v2 = ops.qknorm_rope(*args, k_out=kg, k_scale=0.5, k_norm_max=n2, v=d["v"])
    torch.cuda.synchronize()
    assert k2.data_ptr() == kg.data_ptr() and v2.stride() == kg.stride()
    assert torch.equal(q1, q2) and torch.equal(k1, k2) and torch.equal(v2, d["v"]) and torch.equal(n1, n2)


def gpu_forward_fused(wl, d, q_hat=None):
    """the benchmark's fused configuration: the prologue on K (V moved
    group-major), QK-Norm + RoPE of Q inside the attention kernel"""
    knm = torch.empty(wl.hkv, dtype=torch.float32, device=DEV)
    kg = ops.kv_group_major(wl.nk, wl.hkv, wl.head_dim, d["k"].dtype)
    _, kh, vh = ops.qknorm_rope(None, d["k"], None, d["gk"], None, d["pk"], d["base"], wl.eps, k_out=kg,
                                k_scale=wl.softmax_scale * ops.LOG2E, k_norm_max=knm, v=d["v"])
    plan = ops.plan_for_videos(wl.seqs, wl.nq, wl.nk, wl.hq, wl.hkv, wl.head_dim, d["q"].dtype)
    qn = ops.QNorm(d["gq"], d["pq"], d["base"], wl.eps, 1.0, q_hat)
    O, L = ops.ffa_fwd(d["q"], kh, vh, plan, softmax_scale=ops.LN2, k_norm_max=knm, qnorm=qn)
    torch.cuda.synchronize()
    return O, L


@pytest.mark.parametrize("name,nrows", [("magi4.5b", 384), ("magi24b", 160), ("varlen", 64)])
def test_fused_q_prologue_end_to_end(name, nrows):
    # fused path against the oracle on sampled rows, and against the
    # two-kernel path (prologue on Q, then attention) on every row
    wl = W.make_workload(name, 0)
    inp = W.make_inputs(wl, 0)
    d = dev_inputs(wl, inp)
    note(f"fused Q prologue {name}")
    qh_ref = torch.empty_like(d["q"])
    O, L = gpu_forward_fused(wl, d, q_hat=qh_ref)
    rows = W.sample_rows(wl, nrows, 0)
    mask = oracle.video_mask(wl.seqs, wl.nq, wl.nk, rows)
    Ow, Lw = oracle.forward(np64(inp.q[rows]), np64(inp.k), np64(inp.v), np64(inp.gain_q), np64(inp.gain_k),
                            inp.pos_q[rows].numpy(), inp.pos_k.numpy(), wl.rope_base, wl.eps, mask,
                            wl.softmax_scale)
    compare(np64(O[rows]), Ow, wl.dtype)
    compare(np64(L[rows]), Lw, wl.dtype, "LSE")
    qh, _, O2, L2 = gpu_forward(wl, d)
    # q_hat is the prologue's Q up to the last bf16 bit (the hardware sine and
    # cosine differ from sincosf by ~1e-6)
    dq = (qh_ref.float() - qh.float()).abs()
    assert float(dq.max()) <= 2 ** -7 * float(qh.float().abs().max())
    assert float((dq > 0).float().mean()) < 0.05
    compare(np64(O), np64(O2), wl.dtype, "O fused vs two kernels")


def test_fused_q_prologue_small_cases():
    # G = 4 and 1 (several tokens per item), d = 48, per-head gains, a q_scale,
    # no key-norm bound (online max path), against the oracle on every row
    for (C_, G, hkv, dd) in ((3, 4, 2, 48), (2, 1, 3, 24)):
        wl = W.custom_block_causal(C_, 2, 3, 4, G * hkv, hkv, dd)
        inp = W.make_inputs(wl, 11)
        d = dev_inputs(wl, inp)
        rng = np.random.Generator(np.random.PCG64(11))
        gq = torch.from_numpy(rng.uniform(0.5, 1.5, (G * hkv, dd)).astype(np.float32)).to(DEV)
        plan = ops.plan_for_videos(wl.seqs, wl.nq, wl.nk, wl.hq, wl.hkv, dd, torch.bfloat16)
        _, kh = ops.qknorm_rope(None, d["k"], None, d["gk"], None, d["pk"], d["base"], wl.eps)
        O, L = ops.ffa_fwd(d["q"], kh, d["v"], plan, qnorm=ops.QNorm(gq, d["pq"], d["base"], wl.eps, 0.7))
        torch.cuda.synchronize()
        mask = oracle.video_mask(wl.seqs, wl.nq, wl.nk)
        qhat = oracle.rope_3d(oracle.qk_norm(np64(inp.q), gq.cpu().numpy().astype(np.float64), wl.eps) * 0.7,
                              inp.pos_q.numpy(), oracle.rope_inv_freq(wl.rope_base, dd))
        khat = oracle.rope_3d(oracle.qk_norm(np64(inp.k), np64(inp.gain_k), wl.eps), inp.pos_k.numpy(),
                              oracle.rope_inv_freq(wl.rope_base, dd))
        Ow, Lw = oracle.attention(qhat, khat, np64(inp.v), mask, dd ** -0.5)
        note(f"fused small case G={G} hkv={hkv} d={dd}")
        compare(np64(O), Ow, "bf16")
        compare(np64(L), Lw, "bf16", "LSE")


def test_end_to_end_magi45b_token_major():
    # the full 4.5B layer with K and V left token-major
    wl = W.make_workload("magi4.5b", 0)
    inp = W.make_inputs(wl, 0)
    d = dev_inputs(wl, inp)
    note("end-to-end magi4.5b token-major K/V")
    _, _, O1, L1 = gpu_forward(wl, d, group_major=False)
    _, _, O2, L2 = gpu_forward(wl, d, group_major=True)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)


# --------------------------------------------------------------------------- full workloads

def sampled_forward_parity(name, nrows, seed=0):
    wl = W.make_workload(name, seed)
    note(f"end-to-end {name} seed={seed}: drawing inputs")
    inp = W.make_inputs(wl, seed)
    d = dev_inputs(wl, inp)
    note(f"end-to-end {name}: GPU run")
    qh, kh, O, L = gpu_forward(wl, d)
    rows = W.sample_rows(wl, nrows, seed)
    note(f"end-to-end {name}: oracle on {len(rows)} rows")
    mask = oracle.video_mask(wl.seqs, wl.nq, wl.nk, rows)
    Ow, Lw = oracle.forward(np64(inp.q[rows]), np64(inp.k), np64(inp.v), np64(inp.gain_q), np64(inp.gain_k),
                            inp.pos_q[rows].numpy(), inp.pos_k.numpy(), wl.rope_base, wl.eps, mask,
                            wl.softmax_scale)
    compare(np64(O[rows]), Ow, wl.dtype)
    compare(np64(L[rows]), Lw, wl.dtype, "LSE")
    assert not torch.isnan(O).any()


def test_end_to_end_tiny_all_rows():
    wl = W.make_workload("tiny")
    inp = W.make_inputs(wl, 0)
    d = dev_inputs(wl, inp)
    qh, kh, O, L = gpu_forward(wl, d)
    mask = oracle.video_mask(wl.seqs, wl.nq, wl.nk)
    Ow, Lw = oracle.forward(np64(inp.q), np64(inp.k), np64(inp.v), np64(inp.gain_q), np64(inp.gain_k),
                            inp.pos_q.numpy(), inp.pos_k.numpy(), wl.rope_base, wl.eps, mask, wl.softmax_scale)
    compare(np64(O), Ow, "fp32")
    compare(np64(L), Lw, "fp32", "LSE")


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_end_to_end_magi45b(seed):
    sampled_forward_parity("magi4.5b", 384, seed)


@pytest.mark.parametrize("seed", [0, 2])
def test_end_to_end_magi24b(seed):
    sampled_forward_parity("magi24b", 160, seed)


def test_end_to_end_stream():
    # 256 uniform rows over the four in-flight chunks (seed 0: 61 / 64 / 86 / 57)
    # plus the first, second and last row of each: every row sees the whole
    # 72,000-token cache and the in-flight chunks up to its own
    sampled_forward_parity("stream", 256)


def test_streaming_ring_cache_full_size():
    # the streaming layer (4 in-flight chunks of 3600 tokens over 24 chunks of
    # keys, 128/8 heads, d = 48) with its keys and values in a 24-slot ring
    # holding global chunks 100..123, so the ring wraps inside the in-flight
    # chunks: every chunk written into its slot by the prologue, the key-norm
    # bound passed, FULL slices over the ring; sampled rows against the oracle
    # of the same chunks in linear order
    wl = W.make_workload("stream")
    C, S, first, n = 3600, 24, 100, 4
    note("streaming ring cache full size: inputs")
    inp = W.make_inputs(wl, 0)
    d = dev_inputs(wl, inp)
    ring_k = ops.kv_group_major(S * C, wl.hkv, wl.head_dim, torch.bfloat16)
    ring_v = ops.kv_group_major(S * C, wl.hkv, wl.head_dim, torch.bfloat16)
    knm = torch.empty(wl.hkv, dtype=torch.float32, device=DEV)
    kscale = wl.softmax_scale * ops.LOG2E
    j = 0
    for s0, m in ops.ring_slot_runs(S, first, S):   # linear chunk j holds global chunk first + j
        ops.qknorm_rope(d["q"][:1], d["k"][j * C:(j + m) * C], d["gq"], d["gk"], d["pq"][:1],
                        d["pk"][j * C:(j + m) * C], d["base"], wl.eps, q_out=torch.empty_like(d["q"][:1]),
                        k_out=ring_k[s0 * C:(s0 + m) * C], k_scale=kscale, k_norm_max=knm,
                        v=d["v"][j * C:(j + m) * C], v_out=ring_v[s0 * C:(s0 + m) * C])
        j += m
    qh, _ = ops.qknorm_rope(d["q"], None, d["gq"], None, d["pq"], None, d["base"], wl.eps)
    sl = ops.build_ring_slices(C, S, first, S, n)
    plan = ops.make_plan(sl, n * C, S * C, wl.hq, wl.hkv, wl.head_dim, torch.bfloat16)
    note("streaming ring cache full size: GPU run")
    O, L = ops.ffa_fwd(qh, ring_k, ring_v, plan, softmax_scale=ops.LN2, k_norm_max=knm)
    torch.cuda.synchronize()
    rows = W.sample_rows(wl, 96, 3)
    note(f"streaming ring cache full size: oracle on {len(rows)} rows")
    mask = oracle.video_mask(wl.seqs, wl.nq, wl.nk, rows)
    Ow, Lw = oracle.forward(np64(inp.q[rows]), np64(inp.k), np64(inp.v), np64(inp.gain_q), np64(inp.gain_k),
                            inp.pos_q[rows].numpy(), inp.pos_k.numpy(), wl.rope_base, wl.eps, mask, wl.softmax_scale)
    compare(np64(O[rows]), Ow, "bf16")
    compare(np64(L[rows]), Lw, "bf16", "LSE")
    assert not torch.isnan(O).any()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_end_to_end_varlen(seed):
    # the seed also draws the videos' chunk counts and range-limited chunks
    sampled_forward_parity("varlen", 64, seed)


# --------------------------------------------------------------------------- invariants

def test_bitwise_determinism_and_causality():
    note("bitwise determinism and causality on magi4.5b")
    wl = W.make_workload("magi4.5b")
    inp = W.make_inputs(wl, 3)
    d = dev_inputs(wl, inp)
    plan = ops.plan_for_videos(wl.seqs, wl.nq, wl.nk, wl.hq, wl.hkv, wl.head_dim, torch.bfloat16)
    O1, L1 = ops.ffa_fwd(d["q"], d["k"], d["v"], plan)
    O2, L2 = ops.ffa_fwd(d["q"], d["k"], d["v"], plan)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
    # perturb the last two chunks' K and V: the first two chunks' rows are bitwise unchanged
    k2, v2 = d["k"].clone(), d["v"].clone()
    k2[2 * 1440:] = torch.randn_like(k2[2 * 1440:])
    v2[2 * 1440:] = 7.0
    O3, L3 = ops.ffa_fwd(d["q"], k2, v2, plan)
    torch.cuda.synchronize()
    assert torch.equal(O3[:2 * 1440], O1[:2 * 1440]) and torch.equal(L3[:2 * 1440], L1[:2 * 1440])
    assert not torch.equal(O3[2 * 1440:], O1[2 * 1440:])


def test_streaming_rows_equal_full_run():
    note("streaming == rows of the full run")
    full = W.custom_block_causal(6, 2, 10, 12, 16, 1, 48)
    strm = W.custom_block_causal(6, 2, 10, 12, 16, 1, 48, num_q_chunks=2)
    inp = W.make_inputs(full, 5)
    q, k, v = (t.to(DEV) for t in (inp.q, inp.k, inp.v))
    pf = ops.plan_for_videos(full.seqs, full.nq, full.nk, 16, 1, 48, torch.bfloat16)
    ps = ops.plan_for_videos(strm.seqs, strm.nq, strm.nk, 16, 1, 48, torch.bfloat16)
    Of, Lf = ops.ffa_fwd(q, k, v, pf)
    Os, Ls = ops.ffa_fwd(q[4 * 240:].contiguous(), k, v, ps)
    torch.cuda.synchronize()
    assert torch.equal(Os, Of[4 * 240:]) and torch.equal(Ls, Lf[4 * 240:])


def test_packing_equals_separate_videos_gpu():
    note("packing == separate videos")
    pk = W.custom_packed([(3, 1, 8, 10, None), (2, 1, 8, 10, [-1, 1]), (4, 1, 8, 10, [-1, -1, 1, 1])], 16, 2, 24)
    inp = W.make_inputs(pk, 9)
    q, k, v = (t.to(DEV) for t in (inp.q, inp.k, inp.v))
    O, L = ops.ffa_fwd(q, k, v, ops.plan_for_videos(pk.seqs, pk.nq, pk.nk, 16, 2, 24, torch.bfloat16))
    torch.cuda.synchronize()
    for s in pk.seqs:
        a, b = s.q_offset, s.q_offset + s.nq
        one = W.SeqDesc(s.chunk_len, s.num_kv_chunks, s.num_q_chunks, 0, 0, s.kv_range, 1, 8, 10)
        Os, Ls = ops.ffa_fwd(q[a:b].contiguous(), k[a:b].contiguous(), v[a:b].contiguous(),
                             ops.plan_for_videos([one], s.nq, s.nk, 16, 2, 24, torch.bfloat16))
        torch.cuda.synchronize()
        assert torch.equal(Os, O[a:b]) and torch.equal(Ls, L[a:b])


def test_window_packing_equals_separate_sequences_gpu():
    # causal sliding windows over packed sequences: each sequence's rows are
    # bit for bit those of the sequence run alone
    note("window packing == separate sequences")
    spec = [(300, 64, 0, 0), (130, 200, 300, 300), (250, 1, 430, 430)]
    n = 680
    q, k, v = (torch.from_numpy(rand((n, h, 48), 80 + i)).to(torch.bfloat16).to(DEV)
               for i, h in enumerate((16, 2, 2)))
    O, L = ops.ffa_fwd(q, k, v, ops.make_plan(ops.build_window_slices(spec), n, n, 16, 2, 48, torch.bfloat16))
    torch.cuda.synchronize()
    for ln, w, a, _ in spec:
        Os, Ls = ops.ffa_fwd(q[a:a + ln].contiguous(), k[a:a + ln].contiguous(), v[a:a + ln].contiguous(),
                             ops.make_plan(ops.build_window_slices([(ln, w, 0, 0)]), ln, ln, 16, 2, 48, torch.bfloat16))
        torch.cuda.synchronize()
        assert torch.equal(Os, O[a:a + ln]) and torch.equal(Ls, L[a:a + ln])


# --------------------------------------------------------------------------- cross-attention

@pytest.mark.parametrize("name", ["magi4.5b", "magi24b"])
def test_cross_attention_full_size(name):
    # the layer's video tokens over 800 condition tokens, run as the
    # benchmark runs it (QK-Norm on both sides without rotation, the softmax
    # scale folded into K, K and V group-major, the key-norm bound): sampled
    # rows over all heads against the oracle
    wl = W.make_workload(name)
    T = 800
    note(f"cross-attention full size {name}")
    q, k, v = rand((wl.nq, wl.hq, wl.head_dim), 70), rand((T, wl.hkv, wl.head_dim), 71), rand((T, wl.hkv, wl.head_dim), 72)
    gq = np.random.Generator(np.random.PCG64(73)).uniform(0.8, 1.2, wl.head_dim).astype(np.float32)
    gk = np.random.Generator(np.random.PCG64(74)).uniform(0.8, 1.2, wl.head_dim).astype(np.float32)
    qd, kd, vd = (torch.from_numpy(x).to(torch.bfloat16).to(DEV) for x in (q, k, v))
    zq = torch.zeros((wl.nq, 3), dtype=torch.int32, device=DEV)
    zk = torch.zeros((T, 3), dtype=torch.int32, device=DEV)
    base = torch.tensor(wl.rope_base, dtype=torch.float32, device=DEV)
    knm = torch.empty(wl.hkv, dtype=torch.float32, device=DEV)
    qh, kh, vh = ops.qknorm_rope(qd, kd, torch.from_numpy(gq).to(DEV), torch.from_numpy(gk).to(DEV), zq, zk, base,
                                 wl.eps, k_out=ops.kv_group_major(T, wl.hkv, wl.head_dim, torch.bfloat16),
                                 k_scale=wl.softmax_scale * ops.LOG2E, k_norm_max=knm, v=vd)
    plan = ops.make_plan(ops.build_cross_slices([(0, wl.nq, 0, T)]), wl.nq, T, wl.hq, wl.hkv, wl.head_dim,
                         torch.bfloat16)
    O, L = ops.ffa_fwd(qh, kh, vh, plan, softmax_scale=ops.LN2, k_norm_max=knm)
    torch.cuda.synchronize()
    rows = W.sample_rows(wl, 64, 5)
    Ow, Lw = oracle.forward(np64(qd[rows]), np64(kd), np64(vd), gq.astype(np.float64), gk.astype(np.float64),
                            np.zeros((len(rows), 3), np.int32), np.zeros((T, 3), np.int32), wl.rope_base, wl.eps,
                            np.ones((len(rows), T), bool), wl.softmax_scale)
    compare(np64(O[rows]), Ow, "bf16")
    compare(np64(L[rows]), Lw, "bf16", "LSE")


@pytest.mark.parametrize("group_major", [False, True])
def test_cross_attention_packed_samples(group_major):
    # the parallel block's cross-attention: each sample's video tokens see its
    # own condition tokens (FULL slices from magi_slices_cross); QK-Norm on
    # both sides and no rotation (zero positions), GQA 32/2, d = 24; K and V
    # token-major or group-major (as the benchmark runs it)
    note(f"cross-attention packed samples group_major={group_major}")
    d, hq, hkv = 24, 32, 2
    samples = [(0, 300, 0, 77), (300, 240, 77, 50)]
    nq, nk = 540, 127
    q, k, v = rand((nq, hq, d), 40), rand((nk, hkv, d), 41), rand((nk, hkv, d), 42)
    gq = np.random.Generator(np.random.PCG64(43)).uniform(0.8, 1.2, d).astype(np.float32)
    gk = np.random.Generator(np.random.PCG64(44)).uniform(0.8, 1.2, d).astype(np.float32)
    qd, kd, vd = (torch.from_numpy(x).to(torch.bfloat16).to(DEV) for x in (q, k, v))
    zq = torch.zeros((nq, 3), dtype=torch.int32, device=DEV)
    zk = torch.zeros((nk, 3), dtype=torch.int32, device=DEV)
    base = torch.tensor((1e4, 1e4, 1e4), dtype=torch.float32, device=DEV)
    if group_major:
        qh, kh, vh = ops.qknorm_rope(qd, kd, torch.from_numpy(gq).to(DEV), torch.from_numpy(gk).to(DEV), zq, zk, base,
                                     1e-6, k_out=ops.kv_group_major(nk, hkv, d, torch.bfloat16), v=vd)
    else:
        qh, kh = ops.qknorm_rope(qd, kd, torch.from_numpy(gq).to(DEV), torch.from_numpy(gk).to(DEV), zq, zk, base,
                                 1e-6)
        vh = vd
    sl = ops.build_cross_slices(samples)
    plan = ops.make_plan(sl, nq, nk, hq, hkv, d, torch.bfloat16)
    O, L = ops.ffa_fwd(qh, kh, vh, plan)
    torch.cuda.synchronize()
    mask = oracle.slices_mask([tuple(int(x) for x in s) for s in sl], nq, nk)
    Ow, Lw = oracle.forward(np64(qd), np64(kd), np64(vd), gq, gk, np.zeros((nq, 3)), np.zeros((nk, 3)),
                            (1e4, 1e4, 1e4), 1e-6, mask, d ** -0.5)
    compare(np64(O), Ow, "bf16")
    compare(np64(L), Lw, "bf16", "LSE")


# --------------------------------------------------------------------------- streaming ring KV cache

@pytest.mark.parametrize("group_major", [False, True])
def test_streaming_step_over_ring_cache(group_major):
    # ring of 6 chunk slots holding global chunks 4..9, chunks 7..9 in flight
    # (slots 1..3 after wrapping) with per-chunk KV ranges 2, unlimited, 1.
    # The prologue writes every chunk's keys straight into its slot (cached
    # chunks in "earlier steps"); the oracle runs the same chunks laid out
    # linearly, so the ring order of the keys must not matter
    note(f"streaming step over a ring KV cache group_major={group_major}")
    C, S, first, count, n = 48, 6, 4, 6, 3
    d, hq, hkv = 24, 32, 2
    kvr = [2, -1, 1]
    nchunks = first + count
    frames, gh, gw = 3, 4, 4
    kraw, vraw = rand((nchunks * C, hkv, d), 50), rand((nchunks * C, hkv, d), 51)
    qraw = rand((n * C, hq, d), 52)
    gq = np.random.Generator(np.random.PCG64(53)).uniform(0.8, 1.2, d).astype(np.float32)
    gk = np.random.Generator(np.random.PCG64(54)).uniform(0.8, 1.2, d).astype(np.float32)

    def pos_of(c):   # (t, h, w) of chunk c's tokens: t continues across chunks
        f, y, x = np.meshgrid(np.arange(frames), np.arange(gh), np.arange(gw), indexing="ij")
        return np.stack([c * frames + f.ravel(), y.ravel(), x.ravel()], 1).astype(np.int32)

    dv_ = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    base = torch.tensor((1e4, 1e4, 1e4), dtype=torch.float32, device=DEV)
    gqd, gkd = dv_(gq), dv_(gk)
    scale = d ** -0.5
    # group-major: the ring stored [hkv][slots x C][d] and the attention
    # given the prologue's key-norm bound, as the benchmark runs it
    knm = torch.empty(hkv, dtype=torch.float32, device=DEV) if group_major else None
    if group_major:
        ring_k = ops.kv_group_major(S * C, hkv, d, torch.bfloat16).zero_()
        ring_v = ops.kv_group_major(S * C, hkv, d, torch.bfloat16).zero_()
    else:
        ring_k = torch.zeros((S * C, hkv, d), dtype=torch.bfloat16, device=DEV)
        ring_v = torch.zeros_like(ring_k)
    for c in range(first, nchunks):
        s = c % S
        kc = dv_(kraw[c * C:(c + 1) * C]).to(torch.bfloat16)
        # the prologue call needs a query tensor; one dummy row rides along
        ops.qknorm_rope(dv_(qraw[:1]).to(torch.bfloat16), kc, gqd, gkd, dv_(np.zeros((1, 3), np.int32)),
                        dv_(pos_of(c)), base, 1e-6, k_out=ring_k[s * C:(s + 1) * C], k_scale=scale * ops.LOG2E,
                        k_norm_max=knm)
        ring_v[s * C:(s + 1) * C] = dv_(vraw[c * C:(c + 1) * C]).to(torch.bfloat16)
    qpos = np.concatenate([pos_of(c) for c in range(nchunks - n, nchunks)])
    qd = dv_(qraw).to(torch.bfloat16)
    qh, _ = ops.qknorm_rope(qd, None, gqd, None, dv_(qpos), None, base, 1e-6)
    sl = ops.build_ring_slices(C, S, first, count, n, kvr)
    plan = ops.make_plan(sl, n * C, S * C, hq, hkv, d, torch.bfloat16)
    O, L = ops.ffa_fwd(qh, ring_k, ring_v, plan, softmax_scale=ops.LN2, k_norm_max=knm)
    torch.cuda.synchronize()
    # oracle: chunks first..nchunks-1 in linear order, the same windows
    klin = np64(dv_(kraw[first * C:]).to(torch.bfloat16))
    vlin = np64(dv_(vraw[first * C:]).to(torch.bfloat16))
    kpos = np.concatenate([pos_of(c) for c in range(first, nchunks)])
    mask = np.zeros((n * C, count * C), bool)
    for j in range(n):
        c = nchunks - n + j
        lo = first if kvr[j] < 0 else max(first, c - kvr[j])
        mask[j * C:(j + 1) * C, (lo - first) * C:(c + 1 - first) * C] = True
    Ow, Lw = oracle.forward(np64(qd), klin, vlin, gq, gk, qpos, kpos, (1e4, 1e4, 1e4), 1e-6, mask, scale)
    compare(np64(O), Ow, "bf16")
    compare(np64(L), Lw, "bf16", "LSE")

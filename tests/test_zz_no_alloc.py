"""magi_ffa_bwd_noalloc (the backward with its workspace in the library's
static device scratch) against magi_ffa_bwd (caller-passed workspace), both
through the C ABI: two calls in a row on one GPU, the second with a smaller
input, each bitwise equal to the allocating entry point's gradients (the two
share their kernels, which are deterministic) and within the oracle bar."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from block_causal_attention_amd import _lib, ops

pytestmark = pytest.mark.gpu
DEV = "cuda"


def note(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape).astype(np.float32)


def one_call(chunk, nchunks, hq, hkv, d, seed):
    n = chunk * nchunks
    sl = ops.build_slices([W.SeqDesc(chunk, nchunks, nchunks, 0, 0, (-1,) * nchunks, 1, 1, chunk)])
    q, k, v, do = (torch.from_numpy(rand(s, seed + i)).to(torch.bfloat16).to(DEV)
                   for i, s in enumerate(((n, hq, d), (n, hkv, d), (n, hkv, d), (n, hq, d))))
    plan = ops.make_plan(sl, n, n, hq, hkv, d, torch.bfloat16, backward=True)
    assert plan.num_slots > 0, "the case must exercise the split (partial-sum) path"
    out, lse = ops.ffa_fwd(q, k, v, plan)
    ref = ops.ffa_bwd(q, k, v, out, do, lse, plan)
    got = [torch.full_like(t, float("nan")) for t in (q, k, v)]
    ops.ffa_bwd_noalloc(q, k, v, out, do, lse, plan, *got)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert not torch.isnan(a).any(), f"{name}: unwritten entries"
        assert torch.equal(a, b), f"{name}: no-alloc result differs from magi_ffa_bwd"
    # and the oracle bar of the backward tests (bf16: rel-L2 <= 1e-2)
    f64 = lambda t: t.to("cpu", torch.float64).numpy()
    mask = oracle.slices_mask([tuple(int(x) for x in s) for s in sl], n, n)
    want = oracle.attention_backward(f64(q), f64(k), f64(v), f64(do), mask, d ** -0.5)
    for name, a, w in zip(("dq", "dk", "dv"), got, want):
        rel = float(np.linalg.norm(f64(a) - w) / np.linalg.norm(w))
        note(f"{name} rel-L2 {rel:.3e}")
        assert rel <= 1e-2, f"{name} rel-L2 {rel:.3e}"
    return plan.num_slots


@pytest.mark.parametrize("d", [24, 48])
def test_noalloc_backward_two_calls(d):
    note(f"noalloc bwd d={d}: 4 chunks x 240, then 3 chunks x 100")
    s1 = one_call(240, 4, 32, 2, d, 10)
    s2 = one_call(100, 3, 32, 2, d, 20)
    assert s2 < s1


def test_noalloc_rejects_oversize_before_any_launch():
    # 600-token chunks x 4 at 128/8 heads, d = 48: 1920 partial slots need
    # more than the 64 MiB scratch; the call fails on the host
    note("noalloc oversize rejection")
    n, hq, hkv, d = 2400, 128, 8, 48
    sl = ops.build_slices([W.SeqDesc(600, 4, 4, 0, 0, (-1,) * 4, 1, 1, 600)])
    q = torch.zeros((n, hq, d), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((n, hkv, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros((n, hq), dtype=torch.float32, device=DEV)
    plan = ops.make_plan(sl, n, n, hq, hkv, d, torch.bfloat16, backward=True)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(k)
    with pytest.raises(_lib.MagiError) as e:
        ops.ffa_bwd_noalloc(q, k, k, q, q, lse, plan, dq, dk, dv)
    assert e.value.status == _lib.MAGI_ERR_UNSUPPORTED
    torch.cuda.synchronize()

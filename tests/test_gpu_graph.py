"""HIP graph capture of the hot path (prologue + attention) for a small,
launch-bound step: a streaming generation's first chunk, whose plan is the
same for every denoising step.  The pages capture this case in a GPU graph
(study notes, "推理 Infra", first-chunk bullet).  Every replay is checked
bit for bit against the eager result, with the program's own eager work and
synchronisations between replays."""
import numpy as np
import pytest
import torch

import workloads as W
from block_causal_attention_amd import ops

pytestmark = pytest.mark.gpu
DEV = "cuda"


def note(msg):
    print(f"[gpu-case] {msg}", flush=True)


def first_chunk_step(d):
    """static buffers and the step body (prologue, then attention over one
    chunk of 2 latent frames x 12 x 16 = 384 tokens, 32 heads over 2 groups)"""
    wl = W.custom_block_causal(1, 2, 12, 16, 32, 2, d)
    inp = W.make_inputs(wl, 0)
    st = dict(q=inp.q.to(DEV), k=inp.k.to(DEV), v=inp.v.to(DEV), gq=inp.gain_q.to(DEV), gk=inp.gain_k.to(DEV),
              pq=inp.pos_q.to(DEV), pk=inp.pos_k.to(DEV),
              base=torch.tensor(wl.rope_base, dtype=torch.float32, device=DEV))
    st["qh"] = torch.empty_like(st["q"])
    st["kh"] = ops.kv_group_major(wl.nk, wl.hkv, d, st["k"].dtype, DEV)
    st["vh"] = ops.kv_group_major(wl.nk, wl.hkv, d, st["k"].dtype, DEV)
    st["knm"] = torch.empty(wl.hkv, dtype=torch.float32, device=DEV)
    st["out"] = torch.empty_like(st["q"])
    st["lse"] = torch.empty(wl.nq, wl.hq, dtype=torch.float32, device=DEV)
    plan = ops.plan_for_videos(wl.seqs, wl.nq, wl.nk, wl.hq, wl.hkv, d, st["q"].dtype, DEV).settle()

    def body():
        ops.qknorm_rope(st["q"], st["k"], st["gq"], st["gk"], st["pq"], st["pk"], st["base"], wl.eps,
                        q_out=st["qh"], k_out=st["kh"], k_scale=wl.softmax_scale * ops.LOG2E,
                        k_norm_max=st["knm"], v=st["v"], v_out=st["vh"])
        ops.ffa_fwd(st["qh"], st["kh"], st["vh"], plan, out=st["out"], lse=st["lse"], softmax_scale=ops.LN2,
                    k_norm_max=st["knm"])
    return wl, st, body


def capture(body):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        body()   # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("d", [24, 48])
def test_graph_replays_match_eager(d):
    note(f"graph first chunk d={d}")
    wl, st, body = first_chunk_step(d)
    body()
    torch.cuda.synchronize()
    want_o, want_l = st["out"].clone(), st["lse"].clone()
    g = capture(body)
    for r in range(4):
        # the program's own eager work between replays: clobber the outputs
        # and run an unrelated reduction, synchronised
        st["out"].fill_(float("nan"))
        st["lse"].zero_()
        junk = torch.randn(256, 256, device=DEV).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        note(f"replay {r}: junk {float(junk):.3f}")
        assert torch.equal(st["out"], want_o), f"replay {r}: output differs from eager"
        assert torch.equal(st["lse"], want_l), f"replay {r}: LSE differs from eager"
    # new input contents in the same buffers: a replay equals an eager run on them
    gen = torch.Generator(device="cpu").manual_seed(5)
    st["q"].copy_(torch.randn(st["q"].shape, generator=gen).to(st["q"].dtype))
    g.replay()
    torch.cuda.synchronize()
    got_o, got_l = st["out"].clone(), st["lse"].clone()
    body()
    torch.cuda.synchronize()
    assert torch.equal(got_o, st["out"]) and torch.equal(got_l, st["lse"])
    assert not torch.equal(got_o, want_o)

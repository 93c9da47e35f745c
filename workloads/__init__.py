"""Seeded synthetic workloads for block-causal GQA attention.

This module only *describes and draws* inputs: the sequence layout of each
workload (chunk lengths, how many chunks carry queries, the KV-range limit of
each chunk, the latent video grid each chunk covers), the random Q/K/V
tensors, the QK-Norm gains and the (t, h, w) token coordinates.  It holds none
of the method's arithmetic (no normalisation, rotation, masking or softmax).
Both the CPU oracle under ``oracle/`` and the HIP path draw their inputs from
here, so they see bit-identical values.

Shapes follow the MAGI-1 pages:
  * a chunk is 24 raw frames = 6 latent frames after the VAE's 4x temporal
    compression (MAGI-1 study notes, zhao9797.github.io, section
    "整体 pipeline（分块自回归去噪）" and the Transformer-VAE paragraph);
  * 128 query heads over 8 KV groups, model dims 3072 (4.5B) and 6144 (24B),
    hence head_dim 24 and 48 (same notes, "模型规格（Table 2）");
  * up to 4 chunks in flight (same notes, "一句话定位");
  * videos of mixed length are packed into one sequence and must not see each
    other (interview with Zhang Zheng, zhengguannews.cn, answer on FFA);
  * a chunk's KV range limits how many earlier chunks it attends to (study
    notes, "推理技巧", KV Cache bullet).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "SeqDesc", "Workload", "WORKLOAD_NAMES", "make_workload", "make_inputs",
    "Inputs", "token_coords", "varlen_chunk_plan",
]


@dataclass(frozen=True)
class SeqDesc:
    """One packed video: ``num_kv_chunks`` equal chunks of ``chunk_len`` tokens.

    The last ``num_q_chunks`` chunks carry queries (all of them unless the
    workload is a streaming step).  ``kv_range[i]`` belongs to query chunk i:
    -1 = unlimited, r >= 0 = the chunk sees itself and its r predecessors.
    ``frames``, ``grid_h``, ``grid_w`` give the latent video grid of one chunk
    (chunk_len == frames * grid_h * grid_w); tokens inside a chunk are ordered
    frame-major, then row, then column.
    """
    chunk_len: int
    num_kv_chunks: int
    num_q_chunks: int
    q_offset: int
    k_offset: int
    kv_range: tuple
    frames: int
    grid_h: int
    grid_w: int

    @property
    def first_q_chunk(self) -> int:
        return self.num_kv_chunks - self.num_q_chunks

    @property
    def nq(self) -> int:
        return self.num_q_chunks * self.chunk_len

    @property
    def nk(self) -> int:
        return self.num_kv_chunks * self.chunk_len


@dataclass(frozen=True)
class Workload:
    name: str
    seqs: tuple
    nq: int
    nk: int
    hq: int
    hkv: int
    head_dim: int
    dtype: str                      # "fp32" or "bf16": storage type of Q, K, V, O
    gain_range: Optional[tuple]     # None -> gains are exactly 1
    rope_base: tuple = (10000.0, 10000.0, 10000.0)
    eps: float = 1e-6
    # first key row that the prologue rotates in a streaming step; rows before
    # it belong to the KV cache and were processed by an earlier step
    k_fresh_start: int = 0
    description: str = ""

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def softmax_scale(self) -> float:
        return float(self.head_dim) ** -0.5


WORKLOAD_NAMES = ("tiny", "magi4.5b", "magi24b", "stream", "varlen")


def varlen_chunk_plan(seed: int, num_seqs: int = 6, total_chunks: int = 54,
                      lo: int = 2, hi: int = 16, limit_prob: float = 0.25,
                      limit_from: int = 4):
    """Chunk counts and KV-range-limited flags of the packed varlen workload.

    Counts are drawn uniformly in [lo, hi] per sequence, redrawn until they sum
    to ``total_chunks``; then, in sequence order and chunk order, a chunk with
    index >= ``limit_from`` is limited with probability ``limit_prob``.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    while True:
        counts = rng.integers(lo, hi + 1, size=num_seqs)
        if int(counts.sum()) == total_chunks:
            break
    limited = []
    for n in counts:
        flags = []
        for i in range(int(n)):
            flags.append(bool(i >= limit_from and rng.random() < limit_prob))
        limited.append(flags)
    return [int(c) for c in counts], limited


def _block_causal(name, chunks, frames, gh, gw, hq, hkv, d, dtype, gain_range,
                  description):
    C = frames * gh * gw
    s = SeqDesc(C, chunks, chunks, 0, 0, tuple([-1] * chunks), frames, gh, gw)
    return Workload(name, (s,), C * chunks, C * chunks, hq, hkv, d, dtype,
                    gain_range, description=description)


def make_workload(name: str, seed: int = 0) -> Workload:
    """The five workloads: a tiny fp32 case and four MAGI-1-shaped bf16 layers."""
    if name == "tiny":
        return _block_causal(
            "tiny", 3, 3, 4, 4, 8, 2, 24, "fp32", None,
            "3 chunks x 48 tokens (3 latent frames x 4x4), 8/2 heads, d=24, fp32")
    if name == "magi4.5b":
        return _block_causal(
            "magi4.5b", 4, 6, 15, 16, 128, 8, 24, "bf16", (0.8, 1.2),
            "4 chunks x 1440 tokens (6 x 15x16), 128/8 heads, d=24, bf16")
    if name == "magi24b":
        return _block_causal(
            "magi24b", 8, 6, 24, 25, 128, 8, 48, "bf16", (0.8, 1.2),
            "8 chunks x 3600 tokens (6 x 24x25), 128/8 heads, d=48, bf16")
    if name == "stream":
        C = 6 * 24 * 25
        s = SeqDesc(C, 24, 4, 0, 0, tuple([-1] * 4), 6, 24, 25)
        return Workload("stream", (s,), 4 * C, 24 * C, 128, 8, 48, "bf16",
                        (0.8, 1.2), k_fresh_start=20 * C,
                        description="4 in-flight chunks x 3600 queries over 20 cached + 4 "
                                    "in-flight chunks (86400 keys), 128/8 heads, d=48, bf16")
    if name == "varlen":
        counts, limited = varlen_chunk_plan(seed)
        C = 6 * 20 * 20
        seqs, off = [], 0
        for n, flags in zip(counts, limited):
            kvr = tuple(3 if f else -1 for f in flags)
            seqs.append(SeqDesc(C, n, n, off, off, kvr, 6, 20, 20))
            off += n * C
        return Workload("varlen", tuple(seqs), off, off, 128, 8, 48, "bf16",
                        (0.8, 1.2),
                        description=f"{len(counts)} packed videos with {counts} chunks of 2400 "
                                    f"tokens (6 x 20x20), {sum(map(sum, limited))} chunks at "
                                    "KV range 3, 128/8 heads, d=48, bf16")
    raise ValueError(f"unknown workload {name!r}; choose from {WORKLOAD_NAMES}")


def custom_block_causal(chunks: int, frames: int, gh: int, gw: int, hq: int,
                        hkv: int, d: int, dtype: str = "bf16",
                        gain_range=(0.8, 1.2), kv_range: Optional[Sequence[int]] = None,
                        num_q_chunks: Optional[int] = None,
                        name: str = "custom") -> Workload:
    """A single-video workload of arbitrary size (used for edge-case tests)."""
    C = frames * gh * gw
    nqc = chunks if num_q_chunks is None else num_q_chunks
    kvr = tuple(kv_range) if kv_range is not None else tuple([-1] * nqc)
    assert len(kvr) == nqc
    s = SeqDesc(C, chunks, nqc, 0, 0, kvr, frames, gh, gw)
    return Workload(name, (s,), nqc * C, chunks * C, hq, hkv, d, dtype,
                    gain_range, k_fresh_start=(chunks - nqc) * C)


def custom_packed(seqs_spec, hq: int, hkv: int, d: int, dtype: str = "bf16",
                  gain_range=(0.8, 1.2), name: str = "packed") -> Workload:
    """Packed videos: ``seqs_spec`` is a list of (chunks, frames, gh, gw, kv_range list)."""
    seqs, off = [], 0
    for chunks, frames, gh, gw, kvr in seqs_spec:
        C = frames * gh * gw
        kvr = tuple(kvr) if kvr is not None else tuple([-1] * chunks)
        seqs.append(SeqDesc(C, chunks, chunks, off, off, kvr, frames, gh, gw))
        off += chunks * C
    return Workload(name, tuple(seqs), off, off, hq, hkv, d, dtype, gain_range)


def token_coords(wl: Workload):
    """(t, h, w) latent coordinates of every query and key token, int32 [n, 3].

    t counts latent frames from the start of the token's own video (so it
    restarts at 0 for each packed video, and in a streaming step the in-flight
    chunks continue after the cached ones); h, w are the grid row and column.
    """
    pos_q = np.zeros((wl.nq, 3), np.int32)
    pos_k = np.zeros((wl.nk, 3), np.int32)
    for s in wl.seqs:
        C = s.chunk_len
        idx = np.arange(C)
        f = idx // (s.grid_h * s.grid_w)
        h = (idx // s.grid_w) % s.grid_h
        w = idx % s.grid_w
        for c in range(s.num_kv_chunks):
            rows = slice(s.k_offset + c * C, s.k_offset + (c + 1) * C)
            pos_k[rows, 0] = c * s.frames + f
            pos_k[rows, 1] = h
            pos_k[rows, 2] = w
        for j in range(s.num_q_chunks):
            c = s.first_q_chunk + j
            rows = slice(s.q_offset + j * C, s.q_offset + (j + 1) * C)
            pos_q[rows, 0] = c * s.frames + f
            pos_q[rows, 1] = h
            pos_q[rows, 2] = w
    return pos_q, pos_k


_BLOCK = 512  # tokens per independently seeded block of a random tensor


def _draw_normal(seed: int, tag: int, n: int, width: int, rows=None) -> np.ndarray:
    """N(0,1) float32 [n, width], drawn in 512-token blocks each with its own
    SeedSequence((seed, tag, block)), so any subset of rows can be reproduced
    without drawing the rest."""
    nblocks = (n + _BLOCK - 1) // _BLOCK
    blocks = range(nblocks) if rows is None else sorted({int(r) // _BLOCK for r in rows})
    out = np.empty((n if rows is None else len(blocks) * _BLOCK, width), np.float32)
    dst = {}
    for i, b in enumerate(blocks):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence((seed, tag, b))))
        lo, hi = b * _BLOCK, min(n, (b + 1) * _BLOCK)
        blk = rng.standard_normal((hi - lo, width), dtype=np.float32)
        if rows is None:
            out[lo:hi] = blk
        else:
            out[i * _BLOCK: i * _BLOCK + hi - lo] = blk
            dst[b] = i * _BLOCK
    if rows is None:
        return out
    rows = np.asarray(rows)
    return out[[dst[int(r) // _BLOCK] + int(r) % _BLOCK for r in rows]]


@dataclass
class Inputs:
    """Host copies of one workload's inputs (torch CPU tensors).

    q [nq, hq, d], k/v [nk, hkv, d] in the workload's storage dtype (bf16
    values are the round-to-nearest-even images of the float32 draws);
    gain_q/gain_k float32 [d]; pos_q/pos_k int32 [n, 3].
    """
    q: "torch.Tensor"
    k: "torch.Tensor"
    v: "torch.Tensor"
    gain_q: "torch.Tensor"
    gain_k: "torch.Tensor"
    pos_q: "torch.Tensor"
    pos_k: "torch.Tensor"
    extra: dict = field(default_factory=dict)


def _store(x: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(x)
    return t.to(torch.bfloat16) if dtype == "bf16" else t.contiguous()


def make_inputs(wl: Workload, seed: int = 0, q_rows=None) -> Inputs:
    """Draw the workload's tensors.  Tags: 1=Q, 2=K, 3=V, 4=gains.

    ``q_rows`` (optional) draws only those query rows (for sampled oracle
    checks at full size); K and V are always drawn whole.
    """
    import torch
    d = wl.head_dim
    q = _draw_normal(seed, 1, wl.nq, wl.hq * d, q_rows).reshape(-1, wl.hq, d)
    k = _draw_normal(seed, 2, wl.nk, wl.hkv * d).reshape(wl.nk, wl.hkv, d)
    v = _draw_normal(seed, 3, wl.nk, wl.hkv * d).reshape(wl.nk, wl.hkv, d)
    if wl.gain_range is None:
        gq = np.ones(d, np.float32)
        gk = np.ones(d, np.float32)
    else:
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence((seed, 4))))
        lo, hi = wl.gain_range
        gq = rng.uniform(lo, hi, d).astype(np.float32)
        gk = rng.uniform(lo, hi, d).astype(np.float32)
    pos_q, pos_k = token_coords(wl)
    if q_rows is not None:
        pos_q = pos_q[np.asarray(q_rows)]
    return Inputs(_store(q, wl.dtype), _store(k, wl.dtype), _store(v, wl.dtype),
                  torch.from_numpy(gq), torch.from_numpy(gk),
                  torch.from_numpy(np.ascontiguousarray(pos_q)),
                  torch.from_numpy(np.ascontiguousarray(pos_k)))


def sample_rows(wl: Workload, n: int, seed: int = 0) -> np.ndarray:
    """Seeded query rows for sampled checks: the first and last row of every
    query chunk plus ``n`` uniform draws, sorted and unique."""
    rows = set()
    for s in wl.seqs:
        for j in range(s.num_q_chunks):
            a = s.q_offset + j * s.chunk_len
            rows.update((a, a + 1, a + s.chunk_len - 1))
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence((seed, 99))))
    rows.update(int(x) for x in rng.integers(0, wl.nq, size=n))
    return np.array(sorted(rows), dtype=np.int64)

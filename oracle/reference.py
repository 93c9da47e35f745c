"""Float64 reference implementation (test infrastructure only; see package doc).

Sources, cited by page and section (the pages are the MAGI-1 material):
  [interview]  "对话Sand.ai首席科学家张拯：用自回归开启视频生成下半场"
               (wap.zhengguannews.cn), Q&A on MagiAttention / FFA
  [notes]      MAGI-1 study notes (zhao9797.github.io/ai-research/omni/2025/magi-1)
  [qbitai]     "清华特奖得主团队视频生成AI一夜刷屏！…" (dakule.com, 量子位)
"""
from __future__ import annotations

import numpy as np

MASK_FULL = 0
MASK_CAUSAL = 1
MASK_INVCAUSAL = 2
MASK_BICAUSAL = 3


def qk_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """QK-Norm: each (token, head) vector divided by its root-mean-square over
    the head dimension (plus ``eps`` under the root), then scaled elementwise
    by ``gain``.

    The pages say Q and K are normalised for training stability ([notes]
    "自回归去噪 DiT", QK-Norm + GQA bullet; [qbitai] "QK-Norm和GQA") but give no
    formula; RMS normalisation with a learned gain over head_dim is the reading
    taken here.  x: [n, h, d]; gain: [d] or [h, d].
    """
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gain, np.float64)


def rope_inv_freq(bases, head_dim: int) -> np.ndarray:
    """Rotation frequencies of the 3D RoPE, float64 [head_dim // 2].

    The head dimension is split into three equal sections for the t, h and w
    axes; section a holds head_dim/3 channels = head_dim/6 rotated pairs, and
    pair j of section a turns at base_a ** (-2j / (head_dim/3)).  The base of
    each axis is the learnable parameter ([notes] "自回归去噪 DiT",
    Block-Causal Attention bullet; [qbitai] "Block-Causal Attention").
    """
    if head_dim % 6:
        raise ValueError("3D RoPE needs head_dim divisible by 6")
    sec = head_dim // 3
    out = np.empty(head_dim // 2, np.float64)
    for a in range(3):
        for j in range(sec // 2):
            out[a * (sec // 2) + j] = float(bases[a]) ** (-2.0 * j / sec)
    return out


def rope_3d(x: np.ndarray, pos: np.ndarray, inv_freq: np.ndarray) -> np.ndarray:
    """Rotate each adjacent channel pair (2i, 2i+1) of section a by the angle
    pos[:, a] * inv_freq[pair] (counter-clockwise: (x, y) -> (x cos - y sin,
    x sin + y cos)).  x: [n, h, d]; pos: int [n, 3] (t, h, w).
    """
    x = np.asarray(x, np.float64)
    n, _, d = x.shape
    sec = d // 3
    y = np.empty_like(x)
    for a in range(3):
        for j in range(sec // 2):
            p = a * (sec // 2) + j
            theta = np.asarray(pos[:, a], np.float64) * inv_freq[p]
            c = np.cos(theta)[:, None]
            s = np.sin(theta)[:, None]
            i0 = a * sec + 2 * j
            x0 = x[:, :, i0]
            x1 = x[:, :, i0 + 1]
            y[:, :, i0] = x0 * c - x1 * s
            y[:, :, i0 + 1] = x0 * s + x1 * c
    return y


def _token_labels(seqs, n: int, side: str):
    """Video id and chunk index of every query (side='q') or key row; rows
    that belong to no video get video id -1."""
    vid = np.full(n, -1, np.int64)
    chunk = np.zeros(n, np.int64)
    rng_lim = np.full(n, -1, np.int64)
    for i, s in enumerate(seqs):
        C = s.chunk_len
        if side == "q":
            first = s.num_kv_chunks - s.num_q_chunks
            for j in range(s.num_q_chunks):
                a = s.q_offset + j * C
                vid[a:a + C] = i
                chunk[a:a + C] = first + j
                rng_lim[a:a + C] = s.kv_range[j]
        else:
            for c in range(s.num_kv_chunks):
                a = s.k_offset + c * C
                vid[a:a + C] = i
                chunk[a:a + C] = c
    return vid, chunk, rng_lim


def video_mask(seqs, nq: int, nk: int, q_rows=None) -> np.ndarray:
    """Dense boolean mask rows [len(q_rows), nk] of packed block-causal video
    attention.

    Query token i may see key token j iff both lie in the same packed video
    ([interview] packed videos must not see each other), j's chunk is not
    later than i's chunk (full attention inside a chunk, causal across
    chunks: [notes] "整体 pipeline"; [qbitai] "Block-Causal Attention"), and,
    when i's chunk has a KV range r >= 0, j's chunk is at most r chunks
    earlier ([notes] "推理技巧", KV Cache bullet).  In a streaming step the
    queries are the last ``num_q_chunks`` chunks of the video.
    """
    q_rows = np.arange(nq) if q_rows is None else np.asarray(q_rows)
    vq, cq, rq = _token_labels(seqs, nq, "q")
    vk, ck, _ = _token_labels(seqs, nk, "k")
    vq, cq, rq = vq[q_rows, None], cq[q_rows, None], rq[q_rows, None]
    m = (vq == vk[None, :]) & (vq >= 0) & (ck[None, :] <= cq)
    m &= (rq < 0) | (ck[None, :] >= cq - rq)
    return m


def slices_mask(slices, nq: int, nk: int, q_rows=None) -> np.ndarray:
    """Dense boolean mask rows denoted by AttnSlices (q_start, q_end, k_start,
    k_end, type), half-open ranges.

    An irregular mask is the union of slices, each a full or causal
    rectangle over a q range and a k range ([notes] "训练 Infra", FFA bullet;
    [qbitai] "Flex-Flash-Attention"; [interview] q_range / k_range).  A causal
    slice is aligned at its bottom-right corner: row r of [qs, qe) sees keys
    k in [ks, ke) with k - ke <= r - qe, which for a square slice is the
    ordinary lower triangle.  A pair listed by two slices is an error.

    Sliding-window attention, which the interview names as the next mask
    form for FFA, needs a lower key bound that moves with the row; two more
    types give it (the reading taken here): an inverse causal slice is
    aligned at its top-left corner, row r seeing k with k - ks >= r - qs
    (for a square slice the upper triangle with the diagonal), and a
    bicausal slice applies both bounds (a band).
    """
    q_rows = np.arange(nq) if q_rows is None else np.asarray(q_rows)
    m = np.zeros((len(q_rows), nk), bool)
    kk = np.arange(nk)[None, :]
    r = q_rows[:, None]
    for qs, qe, ks, ke, t in slices:
        if not (0 <= qs <= qe <= nq and 0 <= ks <= ke <= nk):
            raise ValueError(f"slice out of range: {(qs, qe, ks, ke)}")
        cell = (r >= qs) & (r < qe) & (kk >= ks) & (kk < ke)
        if t not in (MASK_FULL, MASK_CAUSAL, MASK_INVCAUSAL, MASK_BICAUSAL):
            raise ValueError(f"unknown mask type {t}")
        if t in (MASK_CAUSAL, MASK_BICAUSAL):
            cell &= (kk - ke) <= (r - qe)
        if t in (MASK_INVCAUSAL, MASK_BICAUSAL):
            cell &= (kk - ks) >= (r - qs)
        if np.any(m & cell):
            raise ValueError("slices overlap")
        m |= cell
    return m


def window_mask(seqs, nq: int, nk: int, q_rows=None) -> np.ndarray:
    """Dense boolean mask rows [len(q_rows), nk] of packed causal
    sliding-window attention.

    ``seqs`` holds (length, window, q_offset, k_offset) per sequence: query
    token i of a sequence sees key token j of the same sequence iff
    i - window < j <= i (positions counted from the sequence start).  The
    interview names sliding-window attention as the mask form FFA is to
    support next ([interview], answer on FFA's mask types) without defining
    it; this is the usual causal reading, the window counted in tokens and
    including the token itself.  Packed sequences never see each other
    ([interview] packed videos must not see each other).
    """
    q_rows = np.arange(nq) if q_rows is None else np.asarray(q_rows)
    m = np.zeros((len(q_rows), nk), bool)
    kk = np.arange(nk)[None, :]
    r = q_rows[:, None]
    for length, window, qo, ko in seqs:
        pos_q = r - qo
        pos_k = kk - ko
        inside = (pos_q >= 0) & (pos_q < length) & (pos_k >= 0) & (pos_k < length)
        m |= inside & (pos_k <= pos_q) & (pos_k > pos_q - window)
    return m


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
              scale: float):
    """Masked softmax attention with grouped K/V heads, float64.

    q: [r, hq, d] query rows; k, v: [nk, hkv, d]; mask: bool [r, nk].  Query
    head h reads K/V head h // (hq // hkv) (128 query heads over 8 groups:
    [notes] "模型规格（Table 2）"; [qbitai] "QK-Norm和GQA").  Logits are
    scale * q.k; masked logits are -inf; O = softmax(logits) @ V and
    LSE = log-sum-exp of the visible logits.  A row that sees no key gets
    O = 0 and LSE = -inf.  Returns (O [r, hq, d], LSE [r, hq]).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    r, hq, d = q.shape
    hkv = k.shape[1]
    G = hq // hkv
    O = np.zeros((r, hq, d), np.float64)
    LSE = np.full((r, hq), -np.inf, np.float64)
    live = mask.any(axis=1)
    for h in range(hq):
        g = h // G
        s = (q[:, h, :] @ k[:, g, :].T) * scale          # [r, nk]
        s = np.where(mask, s, -np.inf)
        mx = np.max(s, axis=1)
        mx = np.where(live, mx, 0.0)
        p = np.exp(s - mx[:, None])                        # exp(-inf) = 0
        l = p.sum(axis=1)
        o = p @ v[:, g, :]
        O[live, h, :] = o[live] / l[live, None]
        LSE[live, h] = mx[live] + np.log(l[live])
    return O, LSE


def attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray,
                       mask: np.ndarray, scale: float):
    """Gradients of ``attention`` with respect to q, k and v, float64.

    The attention is trained with the same kernel family ([notes] "训练 Infra":
    Flex-Flash-Attention serves training; [interview] Q&A on MagiAttention),
    so its backward is part of the method; the pages give no formula, and
    this is the chain rule of the definition above written out per head h
    with group g = h // (hq // hkv):
        P  = softmax over visible keys of scale * q k^T     (rows x keys)
        dV_g += P^T dO_h
        dP = dO_h V_g^T
        dS = P * (dP - rowsum(dO_h * O_h))                  (zero off the mask)
        dQ_h  = scale * dS K_g
        dK_g += scale * dS^T Q_h
    A row that sees no key contributes nothing.  q, dout: [r, hq, d];
    k, v: [nk, hkv, d]; mask: bool [r, nk].  Returns (dQ, dK, dV).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    dout = np.asarray(dout, np.float64)
    r, hq, d = q.shape
    hkv = k.shape[1]
    G = hq // hkv
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    live = mask.any(axis=1)
    for h in range(hq):
        g = h // G
        s = (q[:, h, :] @ k[:, g, :].T) * scale
        s = np.where(mask, s, -np.inf)
        mx = np.where(live, np.max(s, axis=1), 0.0)
        p = np.exp(s - mx[:, None])
        l = np.where(live, p.sum(axis=1), 1.0)
        p = p / l[:, None]                                   # rows with no key stay 0
        o = p @ v[:, g, :]
        dV[:, g, :] += p.T @ dout[:, h, :]
        dp = dout[:, h, :] @ v[:, g, :].T
        delta = np.sum(dout[:, h, :] * o, axis=1)
        ds = p * (dp - delta[:, None])
        dQ[:, h, :] = scale * (ds @ k[:, g, :])
        dK[:, g, :] += scale * (ds.T @ q[:, h, :])
    return dQ, dK, dV


def forward(q, k, v, gain_q, gain_k, pos_q, pos_k, bases, eps, mask, scale,
            q_rows=None):
    """QK-Norm, then 3D RoPE on Q and K, then masked GQA attention.

    Order: normalise, then rotate (the pages list QK-Norm and the learnable
    3D RoPE as the attention's input transforms without fixing the order;
    normalising first keeps the rotation norm-preserving on unit-RMS
    vectors).  ``q`` and ``pos_q`` hold only the rows in ``q_rows`` when it is
    given (rows are independent); ``mask`` holds the matching rows.
    """
    d = q.shape[-1]
    inv = rope_inv_freq(bases, d)
    qh = rope_3d(qk_norm(q, gain_q, eps), pos_q, inv)
    kh = rope_3d(qk_norm(k, gain_k, eps), pos_k, inv)
    return attention(qh, kh, v, mask, scale)

"""Pins for the float64 oracle: library routines, closed forms, brute force and
invariants that fix what the oracle computes independently of its own code.

Each test names the plausible mistake it would catch.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import (MASK_BICAUSAL, MASK_CAUSAL, MASK_FULL, MASK_INVCAUSAL, attention, qk_norm, rope_3d,
                    rope_inv_freq, slices_mask, video_mask, window_mask)
from workloads import SeqDesc

RNG = np.random.Generator(np.random.PCG64(1234))


def _seq(C, nkv, nq=None, qo=0, ko=0, kvr=None, frames=1, gh=1, gw=None):
    nq = nkv if nq is None else nq
    kvr = tuple([-1] * nq) if kvr is None else tuple(kvr)
    return SeqDesc(C, nkv, nq, qo, ko, kvr, frames, gh, C // (frames * gh) if gw is None else gw)


# --------------------------------------------------------------------------- QK-Norm

def test_qknorm_matches_torch_rms_norm():
    # catches: mean vs sum, missing eps, eps outside the root, gain misapplied
    x = RNG.standard_normal((7, 5, 24)) * 3
    g = RNG.uniform(0.5, 1.5, 24)
    for eps in (1e-6, 0.3):
        ref = F.rms_norm(torch.from_numpy(x), (24,), torch.from_numpy(g), eps).numpy()
        np.testing.assert_allclose(qk_norm(x, g, eps), ref, rtol=1e-13, atol=1e-13)


def test_qknorm_unit_rms_and_scale_invariance():
    x = RNG.standard_normal((9, 3, 48))
    y = qk_norm(x, np.ones(48), 0.0)
    np.testing.assert_allclose(np.sqrt((y * y).mean(-1)), 1.0, rtol=1e-13)
    np.testing.assert_allclose(qk_norm(7.5 * x, np.ones(48), 0.0), y, rtol=1e-12, atol=1e-13)


def test_qknorm_per_head_gain():
    x = RNG.standard_normal((4, 3, 24))
    g = RNG.uniform(0.5, 1.5, (3, 24))
    y = qk_norm(x, g, 1e-6)
    for h in range(3):
        np.testing.assert_allclose(y[:, h], qk_norm(x[:, h:h + 1], g[h], 1e-6)[:, 0], rtol=1e-14)


# --------------------------------------------------------------------------- RoPE

def test_inv_freq_closed_form():
    # base 10000, section width 8 (d=24): 10000^(-2j/8) = 10^-j
    np.testing.assert_allclose(rope_inv_freq((1e4, 1e4, 1e4), 24),
                               np.tile([1.0, 0.1, 0.01, 0.001], 3), rtol=1e-14)
    # section width 16 (d=48): 10000^(-2j/16) = 10^(-j/2)
    np.testing.assert_allclose(rope_inv_freq((1e4, 1e4, 1e4), 48),
                               np.tile(10.0 ** (-np.arange(8) / 2), 3), rtol=1e-14)
    # each axis uses its own base (section order t, h, w)
    np.testing.assert_allclose(rope_inv_freq((1e4, 1e2, 1e8), 24),
                               np.concatenate([10.0 ** -np.arange(4), 10.0 ** (-np.arange(4) / 2),
                                               10.0 ** (-2 * np.arange(4))]), rtol=1e-14)
    with pytest.raises(ValueError):
        rope_inv_freq((1e4,) * 3, 32)


def test_rope_matches_complex_rotation():
    # catches: rotation sign, half-split instead of adjacent pairing, wrong section
    d = 24
    x = RNG.standard_normal((11, 4, d))
    pos = RNG.integers(0, 50, (11, 3))
    freqs = np.tile([1.0, 0.1, 0.01, 0.001], 3)
    y = rope_3d(x, pos, freqs)
    z = x[..., 0::2] + 1j * x[..., 1::2]                  # [n, h, 12] complex pairs
    axis = np.repeat(np.arange(3), 4)                      # pair -> axis
    theta = pos[:, axis] * freqs[None, :]                  # [n, 12]
    zr = z * np.exp(1j * theta)[:, None, :]
    np.testing.assert_allclose(y[..., 0::2], zr.real, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y[..., 1::2], zr.imag, rtol=1e-12, atol=1e-12)


def test_rope_one_axis_reduces_to_1d_rope():
    # with h = w = 0 only the t-section turns; it equals 1D RoPE on 8 channels
    d = 24
    x = RNG.standard_normal((6, 2, d))
    pos = np.zeros((6, 3), np.int64)
    pos[:, 0] = np.arange(6) * 5
    y = rope_3d(x, pos, rope_inv_freq((1e4,) * 3, d))
    np.testing.assert_array_equal(y[..., 8:], x[..., 8:])
    for i in range(6):
        for p in range(4):
            th = pos[i, 0] * 10.0 ** -p
            c, s = math.cos(th), math.sin(th)
            a, b = x[i, :, 2 * p], x[i, :, 2 * p + 1]
            np.testing.assert_allclose(y[i, :, 2 * p], a * c - b * s, atol=1e-13)
            np.testing.assert_allclose(y[i, :, 2 * p + 1], a * s + b * c, atol=1e-13)


def test_rope_identity_at_origin_and_norm_preserving():
    x = RNG.standard_normal((5, 3, 48))
    inv = rope_inv_freq((1e4,) * 3, 48)
    np.testing.assert_array_equal(rope_3d(x, np.zeros((5, 3), np.int64), inv), x)
    y = rope_3d(x, RNG.integers(0, 200, (5, 3)), inv)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)


def test_rope_relative_position_property():
    # logits depend only on the coordinate difference
    inv = rope_inv_freq((1e4, 5e3, 2e4), 48)
    q = RNG.standard_normal((8, 1, 48))
    k = RNG.standard_normal((8, 1, 48))
    pq = RNG.integers(0, 30, (8, 3))
    pk = RNG.integers(0, 30, (8, 3))
    shift = np.array([[7, -3, 11]])
    l0 = np.einsum("qd,kd->qk", rope_3d(q, pq, inv)[:, 0], rope_3d(k, pk, inv)[:, 0])
    l1 = np.einsum("qd,kd->qk", rope_3d(q, pq + shift, inv)[:, 0], rope_3d(k, pk + shift, inv)[:, 0])
    np.testing.assert_allclose(l1, l0, rtol=1e-11, atol=1e-11)


# --------------------------------------------------------------------------- masks

def _range_mask(seqs, nq, nk):
    """Same mask written as per-chunk key ranges with Python loops."""
    m = np.zeros((nq, nk), bool)
    for s in seqs:
        C = s.chunk_len
        first = s.num_kv_chunks - s.num_q_chunks
        for j in range(s.num_q_chunks):
            c = first + j
            r = s.kv_range[j]
            lo = 0 if r < 0 else max(0, c - r)
            for qi in range(s.q_offset + j * C, s.q_offset + (j + 1) * C):
                for kj in range(s.k_offset + lo * C, s.k_offset + (c + 1) * C):
                    m[qi, kj] = True
    return m


def test_video_mask_one_chunk_is_full():
    s = _seq(10, 1)
    assert video_mask([s], 10, 10).all()


def test_video_mask_unit_chunks_is_causal():
    s = _seq(1, 9)
    np.testing.assert_array_equal(video_mask([s], 9, 9), np.tril(np.ones((9, 9), bool)))


def test_video_mask_block_causal_pattern():
    # 3 chunks of 2: block lower-triangular
    m = video_mask([_seq(2, 3)], 6, 6)
    want = np.kron(np.tril(np.ones((3, 3), bool)), np.ones((2, 2), bool))
    np.testing.assert_array_equal(m, want)


@pytest.mark.parametrize("trial", range(12))
def test_video_mask_matches_range_loops(trial):
    rng = np.random.Generator(np.random.PCG64(trial))
    seqs, qo, ko = [], 0, 0
    for _ in range(int(rng.integers(1, 4))):
        C = int(rng.integers(1, 5))
        nkv = int(rng.integers(1, 6))
        nq = int(rng.integers(1, nkv + 1))
        kvr = [int(x) for x in rng.integers(-1, 3, nq)]
        seqs.append(_seq(C, nkv, nq, qo, ko, kvr))
        qo += nq * C
        ko += nkv * C
    np.testing.assert_array_equal(video_mask(seqs, qo, ko), _range_mask(seqs, qo, ko))
    rows = rng.integers(0, qo, 5)
    np.testing.assert_array_equal(video_mask(seqs, qo, ko, rows), _range_mask(seqs, qo, ko)[rows])


def test_slices_mask_causal_alignment():
    # square causal slice = lower triangle
    np.testing.assert_array_equal(slices_mask([(0, 7, 0, 7, MASK_CAUSAL)], 7, 7),
                                  np.tril(np.ones((7, 7), bool)))
    # q=[3,7), k=[0,7) causal = rows 3..6 of the 7x7 lower triangle (bottom-right)
    m = slices_mask([(3, 7, 0, 7, MASK_CAUSAL)], 7, 7)
    np.testing.assert_array_equal(m[3:], np.tril(np.ones((7, 7), bool))[3:])
    assert not m[:3].any()
    # wide slice: 2 rows over 5 keys -> row 0 sees 4 keys, row 1 sees 5
    m = slices_mask([(0, 2, 0, 5, MASK_CAUSAL)], 2, 5)
    np.testing.assert_array_equal(m.sum(1), [4, 5])
    # tall slice: 5 rows over 2 keys -> first 3 rows see nothing
    m = slices_mask([(0, 5, 0, 2, MASK_CAUSAL)], 5, 2)
    np.testing.assert_array_equal(m.sum(1), [0, 0, 0, 1, 2])


def test_slices_mask_union_and_overlap():
    m = slices_mask([(0, 2, 0, 2, MASK_FULL), (2, 4, 0, 4, MASK_FULL)], 4, 4)
    np.testing.assert_array_equal(m, video_mask([_seq(2, 2)], 4, 4))
    with pytest.raises(ValueError):
        slices_mask([(0, 3, 0, 3, MASK_FULL), (2, 4, 2, 4, MASK_FULL)], 4, 4)
    with pytest.raises(ValueError):
        slices_mask([(0, 5, 0, 3, MASK_FULL)], 4, 4)


# --------------------------------------------------------------------------- attention

def _sdpa(q, k, v, mask=None, causal=False, scale=None):
    G = q.shape[1] // k.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k).repeat_interleave(G, dim=1).permute(1, 0, 2)
    vt = torch.from_numpy(v).repeat_interleave(G, dim=1).permute(1, 0, 2)
    am = None if mask is None else torch.from_numpy(mask)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=am, is_causal=causal, scale=scale)
    return o.permute(1, 0, 2).numpy()


def test_attention_full_matches_sdpa_with_gqa():
    # catches: GQA head mapping (h // G), scale, transposed operands
    q = RNG.standard_normal((13, 8, 24))
    k = RNG.standard_normal((17, 2, 24))
    v = RNG.standard_normal((17, 2, 24))
    O, _ = attention(q, k, v, np.ones((13, 17), bool), 24 ** -0.5)
    np.testing.assert_allclose(O, _sdpa(q, k, v), rtol=1e-12, atol=1e-12)


def test_attention_causal_matches_sdpa():
    q = RNG.standard_normal((20, 4, 48))
    k = RNG.standard_normal((20, 1, 48))
    v = RNG.standard_normal((20, 1, 48))
    mask = video_mask([_seq(1, 20)], 20, 20)
    O, _ = attention(q, k, v, mask, 48 ** -0.5)
    np.testing.assert_allclose(O, _sdpa(q, k, v, causal=True), rtol=1e-12, atol=1e-12)


def test_attention_block_causal_matches_sdpa_masked():
    q = RNG.standard_normal((12, 4, 24))
    k = RNG.standard_normal((12, 2, 24))
    v = RNG.standard_normal((12, 2, 24))
    mask = video_mask([_seq(4, 3)], 12, 12)
    O, _ = attention(q, k, v, mask, 0.3)
    np.testing.assert_allclose(O, _sdpa(q, k, v, mask=mask, scale=0.3), rtol=1e-12, atol=1e-12)


def test_attention_brute_force_scalar_loops():
    # a scalar re-derivation with math.exp on random masks, incl. empty rows
    q = RNG.standard_normal((6, 4, 6))
    k = RNG.standard_normal((7, 2, 6))
    v = RNG.standard_normal((7, 2, 6))
    mask = RNG.random((6, 7)) < 0.5
    mask[2] = False
    O, L = attention(q, k, v, mask, 0.7)
    for i in range(6):
        for h in range(4):
            g = h // 2
            logits = [(j, 0.7 * sum(q[i, h, c] * k[j, g, c] for c in range(6))) for j in range(7) if mask[i, j]]
            if not logits:
                assert np.all(O[i, h] == 0) and L[i, h] == -np.inf
                continue
            mx = max(s for _, s in logits)
            w = [(j, math.exp(s - mx)) for j, s in logits]
            tot = sum(x for _, x in w)
            for c in range(6):
                assert abs(O[i, h, c] - sum(x * v[j, g, c] for j, x in w) / tot) < 1e-12
            assert abs(L[i, h] - (mx + math.log(tot))) < 1e-12


def test_attention_equal_keys_closed_form():
    # all keys equal -> uniform weights: O = mean of visible V, LSE = s + ln(n)
    q = RNG.standard_normal((5, 2, 24))
    k = np.tile(RNG.standard_normal((1, 1, 24)), (9, 1, 1))
    v = RNG.standard_normal((9, 1, 24))
    mask = video_mask([_seq(3, 3)], 9, 9)[[0, 3, 4, 6, 8]]
    O, L = attention(q, k, v, mask, 0.2)
    for i in range(5):
        n = mask[i].sum()
        for h in range(2):
            np.testing.assert_allclose(O[i, h], v[mask[i], 0].mean(0), rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(L[i, h], 0.2 * q[i, h] @ k[0, 0] + math.log(n), rtol=1e-13)


def test_attention_shift_invariance():
    # adding a vector c to every key shifts each row's logits by q.c: O unchanged
    q = RNG.standard_normal((8, 2, 24))
    k = RNG.standard_normal((8, 1, 24))
    v = RNG.standard_normal((8, 1, 24))
    mask = video_mask([_seq(2, 4)], 8, 8)
    O0, L0 = attention(q, k, v, mask, 0.25)
    c = RNG.standard_normal(24)
    O1, L1 = attention(q, k + c, v, mask, 0.25)
    np.testing.assert_allclose(O1, O0, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(L1 - L0, 0.25 * (q @ c), rtol=1e-11, atol=1e-11)


def test_block_causal_later_chunks_do_not_leak():
    q = RNG.standard_normal((12, 4, 24))
    k = RNG.standard_normal((12, 2, 24))
    v = RNG.standard_normal((12, 2, 24))
    mask = video_mask([_seq(4, 3)], 12, 12)
    O0, L0 = attention(q, k, v, mask, 0.2)
    k2, v2 = k.copy(), v.copy()
    k2[8:] += 5.0
    v2[8:] -= 3.0
    O1, L1 = attention(q, k2, v2, mask, 0.2)
    np.testing.assert_array_equal(O1[:8], O0[:8])
    np.testing.assert_array_equal(L1[:8], L0[:8])
    assert not np.allclose(O1[8:], O0[8:])


def test_packing_equals_separate_videos():
    a, b = _seq(3, 2, qo=0, ko=0), _seq(2, 3, qo=6, ko=6)
    q = RNG.standard_normal((12, 4, 24))
    k = RNG.standard_normal((12, 2, 24))
    v = RNG.standard_normal((12, 2, 24))
    Op, Lp = attention(q, k, v, video_mask([a, b], 12, 12), 0.2)
    Oa, La = attention(q[:6], k[:6], v[:6], video_mask([_seq(3, 2)], 6, 6), 0.2)
    Ob, Lb = attention(q[6:], k[6:], v[6:], video_mask([_seq(2, 3)], 6, 6), 0.2)
    np.testing.assert_allclose(Op, np.concatenate([Oa, Ob]), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(Lp, np.concatenate([La, Lb]), rtol=1e-13)


def test_streaming_equals_rows_of_full_run():
    # queries of the last 2 of 5 chunks over all 5 chunks' keys
    q = RNG.standard_normal((15, 2, 24))
    k = RNG.standard_normal((15, 1, 24))
    v = RNG.standard_normal((15, 1, 24))
    full = attention(q, k, v, video_mask([_seq(3, 5)], 15, 15), 0.2)
    stream = attention(q[9:], k, v, video_mask([_seq(3, 5, nq=2)], 6, 15), 0.2)
    np.testing.assert_array_equal(stream[0], full[0][9:])
    np.testing.assert_array_equal(stream[1], full[1][9:])


def test_kv_range_equals_truncated_video():
    # chunk 4 of 5 with KV range 1 equals attention over chunks 3..4 alone
    q = RNG.standard_normal((15, 2, 24))
    k = RNG.standard_normal((15, 1, 24))
    v = RNG.standard_normal((15, 1, 24))
    mask = video_mask([_seq(3, 5, kvr=[-1, -1, -1, -1, 1])], 15, 15)
    O, L = attention(q, k, v, mask, 0.2)
    Ot, Lt = attention(q[12:], k[9:], v[9:], video_mask([_seq(3, 2)], 6, 6)[3:], 0.2)
    np.testing.assert_allclose(O[12:], Ot, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(L[12:], Lt, rtol=1e-13)


# --------------------------------------------------------------------------- end to end

def test_forward_matches_torch_composition():
    # torch fp64: rms_norm -> complex rotation -> masked SDPA
    n, hq, hkv, d = 18, 4, 2, 24
    q = RNG.standard_normal((n, hq, d))
    k = RNG.standard_normal((n, hkv, d))
    v = RNG.standard_normal((n, hkv, d))
    gq, gk = RNG.uniform(0.8, 1.2, d), RNG.uniform(0.8, 1.2, d)
    pos = RNG.integers(0, 9, (n, 3))
    mask = video_mask([_seq(6, 3)], n, n)
    O, _ = oracle.forward(q, k, v, gq, gk, pos, pos, (1e4, 1e4, 1e4), 1e-6, mask, d ** -0.5)

    def t_norm_rope(x, g):
        y = F.rms_norm(torch.from_numpy(x), (d,), torch.from_numpy(g), 1e-6)
        z = torch.view_as_complex(y.reshape(n, -1, d // 2, 2).contiguous())
        fr = torch.tensor(np.tile([1.0, 0.1, 0.01, 0.001], 3))
        ax = torch.tensor(np.repeat(np.arange(3), 4))
        th = torch.from_numpy(pos)[:, ax].double() * fr
        z = z * torch.polar(torch.ones_like(th), th)[:, None, :]
        return torch.view_as_real(z).reshape(n, -1, d).numpy()

    ref = _sdpa(t_norm_rope(q, gq), t_norm_rope(k, gk), v, mask=mask)
    np.testing.assert_allclose(O, ref, rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------------- attention backward

def _random_mask(r, nk, empty_rows=()):
    m = RNG.random((r, nk)) < 0.6
    m[np.arange(r), RNG.integers(0, nk, r)] = True
    for i in empty_rows:
        m[i] = False
    return m


def test_attention_backward_matches_finite_differences():
    # brute force: central differences of sum(O * dO) through the forward;
    # catches a wrong sign in dS, a missing delta term, a transposed dS or a
    # dropped scale in dQ / dK, and GQA accumulation errors in dK / dV
    r, nk, hq, hkv, d = 5, 6, 4, 2, 3
    q = RNG.standard_normal((r, hq, d))
    k = RNG.standard_normal((nk, hkv, d))
    v = RNG.standard_normal((nk, hkv, d))
    dO = RNG.standard_normal((r, hq, d))
    mask = _random_mask(r, nk, empty_rows=(2,))
    scale = 0.7
    dQ, dK, dV = oracle.attention_backward(q, k, v, dO, mask, scale)

    def f(qq, kk, vv):
        return float(np.sum(attention(qq, kk, vv, mask, scale)[0] * dO))

    eps = 1e-6
    for name, x, g in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v, name: xp}
            args_m = {"q": q, "k": k, "v": v, name: xm}
            num[idx] = (f(args_p["q"], args_p["k"], args_p["v"]) - f(args_m["q"], args_m["k"], args_m["v"])) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8, err_msg=name)
    assert not dQ[2].any()   # the row that sees no key gets no gradient


def test_attention_backward_matches_torch_autograd_sdpa():
    # library routine: autograd through torch's SDPA (float64, GQA by
    # repeating K/V) on a block-causal mask
    n, hq, hkv, d = 12, 8, 2, 24
    G = hq // hkv
    q = RNG.standard_normal((n, hq, d))
    k = RNG.standard_normal((n, hkv, d))
    v = RNG.standard_normal((n, hkv, d))
    dO = RNG.standard_normal((n, hq, d))
    mask = video_mask([_seq(4, 3)], n, n)
    scale = d ** -0.5
    dQ, dK, dV = oracle.attention_backward(q, k, v, dO, mask, scale)
    qt = torch.from_numpy(q).requires_grad_()
    kt = torch.from_numpy(k).requires_grad_()
    vt = torch.from_numpy(v).requires_grad_()
    o = F.scaled_dot_product_attention(qt.permute(1, 0, 2), kt.repeat_interleave(G, dim=1).permute(1, 0, 2),
                                       vt.repeat_interleave(G, dim=1).permute(1, 0, 2),
                                       attn_mask=torch.from_numpy(mask), scale=scale)
    o.permute(1, 0, 2).backward(torch.from_numpy(dO))
    np.testing.assert_allclose(dQ, qt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dK, kt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dV, vt.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_attention_backward_sum_invariants():
    # each live row's probabilities sum to 1 and its dS sums to 0, so per
    # group sum_k dV[k] = sum of the live rows' dO over the group's heads and
    # sum_k dK[k] = 0; catches a dropped delta term or an unnormalised P
    r, nk, hq, hkv, d = 9, 11, 6, 3, 5
    q = RNG.standard_normal((r, hq, d))
    k = RNG.standard_normal((nk, hkv, d))
    v = RNG.standard_normal((nk, hkv, d))
    dO = RNG.standard_normal((r, hq, d))
    mask = _random_mask(r, nk, empty_rows=(4,))
    _, dK, dV = oracle.attention_backward(q, k, v, dO, mask, 0.4)
    live = mask.any(axis=1)
    G = hq // hkv
    for g in range(hkv):
        np.testing.assert_allclose(dV[:, g].sum(0), dO[live][:, g * G:(g + 1) * G].sum((0, 1)), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dK[:, g].sum(0), 0.0, atol=1e-12)


# --------------------------------------------------------------------------- hand-written fixtures

def _golden(name):
    rows = [ln.strip() for ln in open(os.path.join(os.path.dirname(__file__), "golden", name))
            if ln.strip() and not ln.startswith("#")]
    return np.array([[c == "1" for c in r] for r in rows], bool)


def test_golden_block_causal_mask():
    # [notes] "自回归去噪 DiT": full inside a chunk, causal across chunks
    seqs = [SeqDesc(2, 3, 3, 0, 0, (-1, -1, -1), 1, 1, 2)]
    np.testing.assert_array_equal(oracle.video_mask(seqs, 6, 6), _golden("block_causal_3x2.txt"))


def test_golden_kv_range_mask():
    # [notes] "推理技巧", KV Cache: a chunk with range r sees itself and r earlier chunks
    seqs = [SeqDesc(2, 4, 4, 0, 0, (-1, -1, 1, 1), 1, 1, 2)]
    np.testing.assert_array_equal(oracle.video_mask(seqs, 8, 8), _golden("kv_range_4x2_r1.txt"))


def test_golden_packed_videos_mask():
    # [interview]: packed videos never see each other
    seqs = [SeqDesc(2, 2, 2, 0, 0, (-1, -1), 1, 1, 2), SeqDesc(1, 2, 2, 4, 4, (-1, -1), 1, 1, 1)]
    np.testing.assert_array_equal(oracle.video_mask(seqs, 6, 6), _golden("packed_two_videos.txt"))


def test_golden_slice_types():
    # the four slice types over one 4 x 6 rectangle, written out by hand
    g = _golden("slice_types_4x6.txt")
    for i, t in enumerate((MASK_FULL, MASK_CAUSAL, MASK_INVCAUSAL, MASK_BICAUSAL)):
        np.testing.assert_array_equal(slices_mask([(0, 4, 0, 6, t)], 4, 6), g[4 * i:4 * i + 4])


def test_golden_sliding_window_mask():
    g = _golden("sliding_window_two_seqs.txt")
    np.testing.assert_array_equal(window_mask([(6, 3, 0, 0), (4, 3, 6, 6)], 10, 10), g)


def test_inverse_causal_is_causal_turned_half_round():
    # turning both axes around maps a top-left aligned triangle onto a
    # bottom-right aligned one, for any rectangle shape
    rng = np.random.default_rng(5)
    nq, nk = 9, 11
    for _ in range(40):
        qs, qe = sorted(rng.integers(0, nq + 1, 2))
        ks, ke = sorted(rng.integers(0, nk + 1, 2))
        inv = slices_mask([(qs, qe, ks, ke, MASK_INVCAUSAL)], nq, nk)
        cau = slices_mask([(nq - qe, nq - qs, nk - ke, nk - ks, MASK_CAUSAL)], nq, nk)
        np.testing.assert_array_equal(inv, cau[::-1, ::-1])
        both = slices_mask([(qs, qe, ks, ke, MASK_BICAUSAL)], nq, nk)
        np.testing.assert_array_equal(both, inv & slices_mask([(qs, qe, ks, ke, MASK_CAUSAL)], nq, nk))


def test_square_slice_types_are_textbook_triangles():
    n = 7
    one = np.ones((n, n), bool)
    np.testing.assert_array_equal(slices_mask([(0, n, 0, n, MASK_INVCAUSAL)], n, n), np.triu(one))
    np.testing.assert_array_equal(slices_mask([(0, n, 0, n, MASK_BICAUSAL)], n, n), np.eye(n, dtype=bool))


def test_window_mask_special_cases_and_counts():
    n = 13
    # a window as long as the sequence is plain causal attention, a window
    # of one token sees only itself
    np.testing.assert_array_equal(window_mask([(n, n, 0, 0)], n, n), np.tril(np.ones((n, n), bool)))
    np.testing.assert_array_equal(window_mask([(n, 40, 0, 0)], n, n), np.tril(np.ones((n, n), bool)))
    np.testing.assert_array_equal(window_mask([(n, 1, 0, 0)], n, n), np.eye(n, dtype=bool))
    # brute force: row i of a sequence sees exactly min(w, i + 1) keys, the
    # newest being itself
    for w in (2, 3, 5):
        m = window_mask([(n, w, 2, 1)], n + 2, n + 1)
        for i in range(n):
            row = m[2 + i]
            assert row.sum() == min(w, i + 1)
            assert row[1 + i] and not row[2 + i:].any()


def test_window_mask_equals_attention_over_the_window_alone():
    # the output of a row under the window equals plain softmax attention
    # over exactly the keys of its window
    rng = np.random.default_rng(8)
    n, w, d = 10, 4, 6
    q, k, v = (rng.standard_normal((n, 1, d)) for _ in range(3))
    O, L = attention(q, k, v, window_mask([(n, w, 0, 0)], n, n), 0.5)
    for i in range(n):
        lo = max(0, i - w + 1)
        s = 0.5 * k[lo:i + 1, 0] @ q[i, 0]
        p = np.exp(s - s.max())
        np.testing.assert_allclose(O[i, 0], p @ v[lo:i + 1, 0] / p.sum(), rtol=1e-12, atol=1e-12)


def test_window_mask_packing_is_block_diagonal():
    # packed sequences never see each other: the packed mask is the
    # block-diagonal assembly of the masks of the sequences alone
    spec = [(7, 3, 0, 0), (5, 9, 7, 7), (6, 1, 12, 12)]
    m = window_mask(spec, 18, 18)
    want = np.zeros((18, 18), bool)
    for ln, w, a, _ in spec:
        want[a:a + ln, a:a + ln] = window_mask([(ln, w, 0, 0)], ln, ln)
    np.testing.assert_array_equal(m, want)

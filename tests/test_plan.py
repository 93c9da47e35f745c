"""Host-side checks of libmagi_bca: exported symbols, the mask -> AttnSlice
builder and the atomic-free scheduler (no GPU needed), and the C ABI's
argument validation, which runs before any HIP call."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle
import workloads as W
from block_causal_attention_amd import _lib, ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "magi_bca.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const char\*|int32_t)\s+(magi_\w+)\s*\(", src, re.M)))


def test_library_exports_every_header_symbol():
    L = _lib.lib()
    names = header_functions()
    assert len(names) == 16, names
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
    assert b"gfx950" in L.magi_version()


# --------------------------------------------------------------------------- builder

def expand(slices, nq, nk):
    return oracle.slices_mask([tuple(int(x) for x in s) for s in slices], nq, nk)


@pytest.mark.parametrize("name", ["tiny", "magi4.5b", "magi24b", "varlen"])
def test_builder_round_trip_matches_oracle_mask(name):
    wl = W.make_workload(name)
    sl = ops.build_slices(wl.seqs)
    nchunks = sum(s.num_q_chunks for s in wl.seqs)
    assert len(sl) == nchunks
    # compare on a row sample for the big ones (mask rows are exact booleans)
    rows = np.arange(wl.nq) if wl.nq <= 6000 else W.sample_rows(wl, 300)
    want = oracle.video_mask(wl.seqs, wl.nq, wl.nk, rows)
    got = oracle.slices_mask([tuple(int(x) for x in s) for s in sl], wl.nq, wl.nk, rows)
    np.testing.assert_array_equal(got, want)


def test_builder_streaming_slices():
    wl = W.make_workload("stream")
    sl = ops.build_slices(wl.seqs)
    C_ = 3600
    np.testing.assert_array_equal(sl, [[j * C_, (j + 1) * C_, 0, (21 + j) * C_, 0] for j in range(4)])


@pytest.mark.parametrize("trial", range(20))
def test_builder_fuzz(trial):
    rng = np.random.Generator(np.random.PCG64(100 + trial))
    spec, qo, ko = [], 0, 0
    for _ in range(int(rng.integers(1, 5))):
        Cl = int(rng.integers(1, 6))
        nkv = int(rng.integers(1, 7))
        nqc = int(rng.integers(1, nkv + 1))
        kvr = [int(x) for x in rng.integers(-1, 4, nqc)] if rng.random() < 0.6 else [-1] * nqc
        qo += int(rng.integers(0, 3))  # gaps are allowed (rows/keys of no video)
        ko += int(rng.integers(0, 3))
        spec.append(W.SeqDesc(Cl, nkv, nqc, qo, ko, tuple(kvr), 1, 1, Cl))
        qo += nqc * Cl
        ko += nkv * Cl
    sl = ops.build_slices(spec)
    np.testing.assert_array_equal(expand(sl, qo, ko), oracle.video_mask(spec, qo, ko))


def test_builder_unit_chunks_become_one_causal_slice():
    s = W.SeqDesc(1, 10, 10, 0, 0, tuple([-1] * 10), 1, 1, 1)
    sl = ops.build_slices([s])
    np.testing.assert_array_equal(sl, [[0, 10, 0, 10, _lib.MASK_CAUSAL]])
    st = W.SeqDesc(1, 10, 4, 0, 0, tuple([-1] * 4), 1, 1, 1)
    sl = ops.build_slices([st])
    np.testing.assert_array_equal(sl, [[0, 4, 0, 10, _lib.MASK_CAUSAL]])
    np.testing.assert_array_equal(expand(sl, 4, 10), oracle.video_mask([st], 4, 10))


def test_builder_rejects_bad_descriptors():
    good = W.SeqDesc(4, 3, 3, 0, 0, (-1, -1, -1), 1, 2, 2)
    for bad, code in [
        (W.SeqDesc(0, 3, 3, 0, 0, None, 1, 1, 1), _lib.MAGI_ERR_INVALID_ARG),
        (W.SeqDesc(4, 3, 4, 0, 0, None, 1, 1, 1), _lib.MAGI_ERR_INVALID_ARG),
        (W.SeqDesc(4, 0, 0, 0, 0, None, 1, 1, 1), _lib.MAGI_ERR_INVALID_ARG),
        (W.SeqDesc(4, 3, 3, -1, 0, None, 1, 1, 1), _lib.MAGI_ERR_INVALID_ARG),
        (W.SeqDesc(4, 3, 3, 0, 0, (-1, -2, -1), 1, 1, 1), _lib.MAGI_ERR_INVALID_ARG),
        (W.SeqDesc(2 ** 30, 3, 3, 0, 0, None, 1, 1, 1), _lib.MAGI_ERR_INVALID_ARG),
    ]:
        with pytest.raises(_lib.MagiError) as e:
            ops.build_slices([bad])
        assert e.value.status == code
    # two videos sharing query rows
    with pytest.raises(_lib.MagiError) as e:
        ops.build_slices([good, W.SeqDesc(4, 3, 3, 8, 12, None, 1, 2, 2)])
    assert e.value.status == _lib.MAGI_ERR_OVERLAP
    # NULL count pointer / NULL seqs
    L = _lib.lib()
    assert L.magi_slices_build(None, 1, None, 0, None) == _lib.MAGI_ERR_INVALID_ARG
    n = C.c_int32()
    assert L.magi_slices_build(None, 1, None, 0, C.byref(n)) == _lib.MAGI_ERR_INVALID_ARG
    assert L.magi_slices_build(None, 0, None, 0, C.byref(n)) == 0 and n.value == 0
    # two-call protocol: too small a buffer reports the size
    descs = (_lib.SeqDesc * 1)(_lib.SeqDesc(4, 3, 3, 0, 0, None))
    buf = (_lib.AttnSlice * 2)()
    assert L.magi_slices_build(descs, 1, buf, 2, C.byref(n)) == _lib.MAGI_ERR_BUFFER_TOO_SMALL
    assert n.value == 3
    assert b"slice_cap" in L.magi_last_error()


# --------------------------------------------------------------------------- scheduler

def check_schedule(slices, nq, nk, hq, hkv, d, dtype=_lib.DTYPE_BF16, tile_q=0):
    work, ts = ops.schedule(slices, nq, nk, hq, hkv, d, dtype, tile_q)
    tq = tile_q or ops.default_tile_q(hq, hkv, d, dtype)
    owner = np.full((nq, hkv), -1)
    sl = [tuple(int(x) for x in s) for s in slices]
    full = oracle.slices_mask(sl, nq, nk) if nq * nk <= 4e7 else None
    for i, (q0, ql, sb, se, g, cost) in enumerate(work):
        assert 1 <= ql <= tq and 0 <= g < hkv and 0 <= sb <= se <= len(ts)
        assert (owner[q0:q0 + ql, g] == -1).all(), "row owned twice"
        owner[q0:q0 + ql, g] = i
        mine = [sl[j] for j in ts[sb:se]]
        for (qs, qe, *_r) in mine:
            assert qs <= q0 and q0 + ql <= qe, "tile straddles a slice boundary"
        if full is not None:
            sub = oracle.slices_mask(mine, nq, nk, np.arange(q0, q0 + ql)) if mine else np.zeros((ql, nk), bool)
            np.testing.assert_array_equal(sub, full[q0:q0 + ql])
            assert cost == min(int(sub.sum()), 2 ** 31 - 1)
    assert (owner >= 0).all(), "a (row, group) has no owner"
    costs = work[::hkv, 5]
    assert (np.diff(costs) <= 0).all(), "not heaviest-first"
    for r in range(len(work) // hkv):
        np.testing.assert_array_equal(work[r * hkv:(r + 1) * hkv, 4], np.arange(hkv))
    w2, ts2 = ops.schedule(slices, nq, nk, hq, hkv, d, dtype, tile_q)
    np.testing.assert_array_equal(w2, work)
    np.testing.assert_array_equal(ts2, ts)
    return work, ts


@pytest.mark.parametrize("name", ["tiny", "magi4.5b", "varlen"])
def test_schedule_workloads(name):
    wl = W.make_workload(name)
    sl = ops.build_slices(wl.seqs)
    work, ts = check_schedule(sl, wl.nq, wl.nk, wl.hq, wl.hkv, wl.head_dim,
                              _lib.DTYPE_FP32 if wl.dtype == "fp32" else _lib.DTYPE_BF16)
    area = int(oracle.video_mask(wl.seqs, wl.nq, wl.nk).sum()) if wl.nq < 10000 else None
    if area is not None:
        assert work[:, 5].astype(np.int64).sum() == area * wl.hkv


def test_schedule_area_24b_closed_form():
    wl = W.make_workload("magi24b")
    work, _ = ops.schedule(ops.build_slices(wl.seqs), wl.nq, wl.nk, 128, 8, 48, _lib.DTYPE_BF16)
    assert work[:, 5].astype(np.int64).sum() == 3600 * 3600 * 36 * 8
    assert len(work) == (28800 // 16) * 8


@pytest.mark.parametrize("trial", range(25))
def test_schedule_fuzz_raw_slices(trial):
    rng = np.random.Generator(np.random.PCG64(500 + trial))
    nq, nk = int(rng.integers(1, 120)), int(rng.integers(1, 120))
    hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 3, 4, 16]))
    # non-overlapping random slices: carve the k axis per q band
    slices = []
    q = 0
    while q < nq:
        qe = min(nq, q + int(rng.integers(1, 30)))
        if rng.random() < 0.8:
            k = int(rng.integers(0, 5))
            while k < nk:
                ke = min(nk, k + int(rng.integers(1, 40)))
                slices.append((q, qe, k, ke, int(rng.choice(4, p=[0.5, 0.2, 0.15, 0.15]))))
                k = ke + int(rng.integers(0, 10))
        q = qe + int(rng.integers(0, 4))
    arr = np.array(slices, np.int32).reshape(-1, 5)
    tq = int(rng.choice([0, 1, 5]))
    check_schedule(arr, nq, nk, G * hkv, hkv, 24, _lib.DTYPE_BF16, tile_q=min(tq, 256 // G))


def check_schedule_kv(slices, nq, nk, hq, hkv, d, dtype=_lib.DTYPE_BF16, tile_k=0):
    """Key-major schedule: every (key, group) owned once -- by a direct item
    or by a reduce entry whose parts are items --, each owner's slices
    reproduce the mask's columns over its keys, costs are the visible pairs,
    heaviest first (equal costs token window by window, keys ascending within
    a window) with the groups interleaved, deterministic."""
    work, ts, ext, red, nslots = ops.schedule_kv(slices, nq, nk, hq, hkv, d, dtype, tile_k)
    slot, wlo, whi = ext[:, 0], ext[:, 1], ext[:, 2]
    tk = tile_k or 128
    owner = np.full((nk, hkv), -1)
    sl = [tuple(int(x) for x in s) for s in slices]
    full = oracle.slices_mask(sl, nq, nk) if nq * nk <= 4e7 else None

    smask = {}

    def slice_mask(j):
        if j not in smask:
            smask[j] = oracle.slices_mask([sl[j]], nq, nk)
        return smask[j]

    def part_mask(i, k0, kl):
        """rows x tile keys an item covers: its slices, clipped to its token window"""
        m = np.zeros((nq, kl), bool)
        for j in ts[work[i, 2]:work[i, 3]]:
            m |= slice_mask(int(j))[:, k0:k0 + kl]
        m[:wlo[i]] = False
        m[whi[i]:] = False
        return m

    def check_cols(k0, kl, items):
        idx = [j for i in items for j in ts[work[i, 2]:work[i, 3]]]
        mine = [sl[j] for j in idx]
        for i in items:
            s_ = [sl[j] for j in ts[work[i, 2]:work[i, 3]]]
            assert [m[0] for m in s_] == sorted(m[0] for m in s_), "slices not in query order"
        if full is not None:
            cover = np.zeros((nq, kl), np.int32)
            for i in items:
                pm = part_mask(i, k0, kl)
                assert int(work[i, 5]) == int(pm.sum()), "item cost is not its visible pairs"
                cover += pm
            assert cover.max(initial=0) <= 1, "a (row, key) pair covered twice"
            np.testing.assert_array_equal(cover.astype(bool), full[:, k0:k0 + kl])
            for j in set(int(x) for x in idx):   # every listed slice shows some row a key of the tile
                assert slice_mask(j)[:, k0:k0 + kl].any()

    by_slot = {}
    for i, (k0, kl, sb, se, g, cost) in enumerate(work):
        assert 1 <= kl <= tk and 0 <= g < hkv and 0 <= sb <= se <= len(ts)
        assert 0 <= wlo[i] <= whi[i] <= nq
        if slot[i] < 0:
            assert (owner[k0:k0 + kl, g] == -1).all(), "key owned twice"
            owner[k0:k0 + kl, g] = i
            check_cols(k0, kl, [i])
        else:
            assert 0 <= slot[i] < nslots and slot[i] not in by_slot and se > sb
            by_slot[int(slot[i])] = i
    assert sorted(by_slot) == list(range(nslots)), "slots not used exactly once"
    for r, (k0, kl, g, s0, cnt) in enumerate(red):
        assert cnt >= 2 and 0 <= g < hkv
        items = [by_slot[s] for s in range(s0, s0 + cnt)]
        for i in items:
            assert tuple(work[i, [0, 1, 4]]) == (k0, kl, g)
        # parts follow the tile list in order: a run of slices, or windows of one slice
        step = max(1, 64 // (hq // hkv))   # tokens per row tile of the dK/dV pass
        for a_, b_ in zip(items, items[1:]):
            assert work[a_, 3] == work[b_, 2] or (work[a_, 2] == work[b_, 2] and work[a_, 3] == work[b_, 3]
                                                  and whi[a_] <= wlo[b_])
            if work[a_, 2] == work[b_, 2] and work[a_, 3] == work[b_, 3]:
                # a window that another window of the slice follows holds whole row tiles
                assert (whi[a_] - wlo[a_]) % step == 0
        assert (owner[k0:k0 + kl, g] == -1).all(), "key owned twice"
        owner[k0:k0 + kl, g] = len(work) + r
        check_cols(k0, kl, items)
    assert sum(int(c) for c in red[:, 4]) == nslots if len(red) else nslots == 0
    assert (owner >= 0).all(), "a (key, group) has no owner"
    assert (np.diff(work[::hkv, 5]) <= 0).all(), "not heaviest-first"
    u, ulo = work[::hkv], wlo[::hkv]
    for x in range(len(u) - 1):
        if u[x, 5] == u[x + 1, 5]:
            assert (ulo[x], u[x, 0]) <= (ulo[x + 1], u[x + 1, 0]), "equal-cost units not window by window"
    for r in range(len(work) // hkv):
        np.testing.assert_array_equal(work[r * hkv:(r + 1) * hkv, 4], np.arange(hkv))
    again = ops.schedule_kv(slices, nq, nk, hq, hkv, d, dtype, tile_k)
    for x, y in zip(again[:4], (work, ts, ext, red)):
        np.testing.assert_array_equal(x, y)
    assert again[4] == nslots
    return work, ts, slot, red


@pytest.mark.parametrize("name", ["tiny", "magi4.5b", "varlen", "stream"])
def test_schedule_kv_workloads(name):
    wl = W.make_workload(name)
    sl = ops.build_slices(wl.seqs)
    work, _, slot, red = check_schedule_kv(sl, wl.nq, wl.nk, wl.hq, wl.hkv, wl.head_dim,
                                           _lib.DTYPE_FP32 if wl.dtype == "fp32" else _lib.DTYPE_BF16)
    if wl.nq < 10000:
        assert work[:, 5].astype(np.int64).sum() == int(oracle.video_mask(wl.seqs, wl.nq, wl.nk).sum()) * wl.hkv
    if name == "magi4.5b":
        # block-causal, 4 chunks: a key tile of chunk c is seen by 4 - c chunks;
        # each chunk's rows are cut into token windows, so items cost at most a
        # quarter of 128 x 1440 pairs and there are a few thousand of them
        assert work[:, 5].max() <= 128 * 1440 // 3 and len(red) > 0 and len(work) >= 3000
        assert ((slot >= 0).sum()) == red[:, 4].sum()


@pytest.mark.parametrize("trial", range(25))
def test_schedule_kv_fuzz_raw_slices(trial):
    rng = np.random.Generator(np.random.PCG64(900 + trial))
    nq, nk = int(rng.integers(1, 120)), int(rng.integers(1, 120))
    hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 3, 4, 16]))
    slices = []
    q = 0
    while q < nq:
        qe = min(nq, q + int(rng.integers(1, 30)))
        if rng.random() < 0.8:
            k = int(rng.integers(0, 5))
            while k < nk:
                ke = min(nk, k + int(rng.integers(1, 40)))
                slices.append((q, qe, k, ke, int(rng.choice(4, p=[0.5, 0.2, 0.15, 0.15]))))
                k = ke + int(rng.integers(0, 10))
        q = qe + int(rng.integers(0, 4))
    arr = np.array(slices, np.int32).reshape(-1, 5)
    check_schedule_kv(arr, nq, nk, G * hkv, hkv, 24, _lib.DTYPE_BF16, tile_k=int(rng.choice([0, 1, 7, 64])))


def test_schedule_kv_errors():
    with pytest.raises(_lib.MagiError) as e:   # validated like magi_schedule
        ops.schedule_kv(np.array([(0, 8, 0, 8, 1), (0, 8, 6, 12, 0)]), 8, 12, 16, 1, 24, 0)
    assert e.value.status == _lib.MAGI_ERR_OVERLAP
    with pytest.raises(_lib.MagiError) as e:
        ops.schedule_kv(np.array([(0, 4, 0, 4, 0)]), 4, 4, 16, 1, 24, 0, tile_k=200)
    assert e.value.status == _lib.MAGI_ERR_INVALID_ARG


def test_schedule_causal_overlap_detection():
    # two causal slices that only meet on the last rows of their band
    a = (0, 8, 0, 8, _lib.MASK_CAUSAL)
    b = (0, 8, 6, 12, _lib.MASK_FULL)
    with pytest.raises(_lib.MagiError) as e:
        ops.schedule(np.array([a, b]), 8, 12, 16, 1, 24, 0)
    assert e.value.status == _lib.MAGI_ERR_OVERLAP
    # touching but disjoint: causal row r sees k <= r, full starts at 8
    ok = ops.schedule(np.array([a, (0, 8, 8, 12, 0)]), 8, 12, 16, 1, 24, 0)
    assert len(ok[0]) == 1
    # a tall causal slice whose early rows see nothing is not an overlap
    ops.schedule(np.array([(0, 8, 0, 2, 1), (0, 8, 2, 4, 0)]), 8, 4, 16, 1, 24, 0)


def test_schedule_lower_bound_overlap_detection():
    n = 8
    cau = (0, n, 0, n, _lib.MASK_CAUSAL)
    # the two triangles of one square share its diagonal
    with pytest.raises(_lib.MagiError) as e:
        ops.schedule(np.array([cau, (0, n, 0, n, _lib.MASK_INVCAUSAL)]), n, n + 1, 16, 1, 24, 0)
    assert e.value.status == _lib.MAGI_ERR_OVERLAP
    # shifted one key to the right they tile the rectangle [0, n) x [0, n + 1)
    sl = np.array([cau, (0, n, 1, n + 1, _lib.MASK_INVCAUSAL)])
    work, _ = check_schedule(sl, n, n + 1, 16, 1, 24)
    np.testing.assert_array_equal(expand(sl, n, n + 1), np.ones((n, n + 1), bool))
    # a band and a full rectangle that meet only where the band ends
    band = (0, n, 0, n + 2, _lib.MASK_BICAUSAL)   # row r sees [r, r + 3)
    ops.schedule(np.array([band, (0, n, n + 2, n + 5, 0)]), n, n + 5, 16, 1, 24, 0)
    with pytest.raises(_lib.MagiError) as e:
        ops.schedule(np.array([band, (0, n, n + 1, n + 5, 0)]), n, n + 5, 16, 1, 24, 0)
    assert e.value.status == _lib.MAGI_ERR_OVERLAP
    # k_start + (q_end - q_start) must stay inside int32 for a lower bound
    with pytest.raises(_lib.MagiError) as e:
        ops.schedule(np.array([(0, 4, 2 ** 31 - 3, 2 ** 31 - 1, _lib.MASK_INVCAUSAL)]), 4, 2 ** 31 - 1, 16, 1,
                     24, 0)
    assert e.value.status == _lib.MAGI_ERR_INVALID_ARG


@pytest.mark.parametrize("trial", range(12))
def test_schedule_overlap_decision_matches_brute_force(trial):
    # random slices of every type in a small space, overlapping or not: the
    # scheduler reports an overlap exactly when the dense masks share a pair
    rng = np.random.Generator(np.random.PCG64(1300 + trial))
    nq, nk = 12, 14
    for _ in range(60):
        sl = []
        for _ in range(int(rng.integers(2, 4))):
            qs, qe = sorted(int(x) for x in rng.integers(0, nq + 1, 2))
            ks, ke = sorted(int(x) for x in rng.integers(0, nk + 1, 2))
            sl.append((qs, qe, ks, ke, int(rng.integers(0, 4))))
        try:
            oracle.slices_mask(sl, nq, nk)
            want = 0
        except ValueError:
            want = _lib.MAGI_ERR_OVERLAP
        try:
            ops.schedule(np.array(sl, np.int32), nq, nk, 16, 1, 24, 0)
            got = 0
        except _lib.MagiError as e:
            got = e.status
        assert got == want, sl


def test_schedule_rejects_bad_arguments():
    L = _lib.lib()
    nw, nt = C.c_int32(), C.c_int32()
    good = np.array([[0, 4, 0, 4, 0]], np.int32)

    def call(sl, nq=4, nk=4, hq=16, hkv=1, d=24, dt=0, tq=0):
        s = np.ascontiguousarray(np.asarray(sl, np.int32).reshape(-1, 5))
        return L.magi_schedule(s.ctypes.data_as(C.POINTER(_lib.AttnSlice)), len(s), nq, nk, hq, hkv, d, dt, tq,
                               None, 0, C.byref(nw), None, 0, C.byref(nt))
    assert call(good) == 0 and nw.value == 1 and nt.value == 1
    assert call([[0, 5, 0, 4, 0]]) == _lib.MAGI_ERR_INVALID_ARG      # q beyond nq
    assert call([[2, 1, 0, 4, 0]]) == _lib.MAGI_ERR_INVALID_ARG      # q_start > q_end
    assert call([[0, 4, -1, 4, 0]]) == _lib.MAGI_ERR_INVALID_ARG     # negative k
    assert call([[0, 4, 0, 4, 7]]) == _lib.MAGI_ERR_INVALID_ARG      # bad mask type
    assert call(good, hq=12, hkv=8) == _lib.MAGI_ERR_INVALID_ARG     # hq % hkv
    assert call(good, d=64) == _lib.MAGI_ERR_UNSUPPORTED             # head_dim
    assert call(good, hq=512, hkv=1) == _lib.MAGI_ERR_UNSUPPORTED    # group > 256
    assert call(good, dt=5) == _lib.MAGI_ERR_INVALID_ARG             # dtype
    assert call(good, tq=17) == _lib.MAGI_ERR_INVALID_ARG            # tile_q above kernel capacity
    assert call(good, nq=-1) == _lib.MAGI_ERR_INVALID_ARG
    assert call([[0, 4, 0, 3, 0], [0, 4, 2, 4, 0]]) == _lib.MAGI_ERR_OVERLAP
    assert L.magi_schedule(None, 1, 4, 4, 16, 1, 24, 0, 0, None, 0, C.byref(nw), None, 0, C.byref(nt)) \
        == _lib.MAGI_ERR_INVALID_ARG
    w = (_lib.WorkItem * 1)()
    t = (C.c_int32 * 1)()
    s = np.ascontiguousarray(np.array([[0, 4, 0, 4, 0]] * 1, np.int32))
    assert L.magi_schedule(s.ctypes.data_as(C.POINTER(_lib.AttnSlice)), 1, 40, 4, 16, 8, 24, 0, 0, w, 1,
                           C.byref(nw), t, 1, C.byref(nt)) == _lib.MAGI_ERR_BUFFER_TOO_SMALL
    assert nw.value > 1


def test_schedule_uncovered_rows_get_owners():
    work, ts = ops.schedule(np.array([[3, 5, 0, 2, 0]]), 9, 2, 4, 2, 24, 0)
    cover = sorted((int(w[0]), int(w[1])) for w in work[::2])
    assert cover == [(0, 3), (3, 2), (5, 4)]
    assert all(w[2] == w[3] for w in work if w[0] != 3)


def test_default_tile_q():
    assert ops.default_tile_q(128, 8, 24, 0) == 16
    assert ops.default_tile_q(8, 2, 24, 1) == 64
    assert ops.default_tile_q(48, 16, 48, 0) == 85


# --------------------------------------------------------------------------- device entry validation

def test_device_entry_points_validate_before_any_hip_call():
    L = _lib.lib()
    p = C.c_void_p(4096)  # never dereferenced: every call below fails validation
    f = C.c_void_p(4096)
    # magi_qknorm_rope
    def qk(**kw):
        a = dict(qi=p, qo=p, nq=10, hq=8, qs=192, ki=None, ko=None, nk=0, hkv=1, ks=0, kos=0, kohs=24, vi=None,
                 vo=None, d=24, dt=0, gq=f, gk=None, ghs=0, eps=1e-6, pq=p, pk=None, base=f, qsc=1.0, ksc=1.0,
                 knm=None)
        a.update(kw)
        return L.magi_qknorm_rope(a["qi"], a["qo"], a["nq"], a["hq"], a["qs"], a["ki"], a["ko"], a["nk"], a["hkv"],
                                  a["ks"], a["kos"], a["kohs"], a["vi"], a["vo"], a["d"], a["dt"], a["gq"], a["gk"],
                                  a["ghs"], a["eps"], a["pq"], a["pk"], a["base"], a["qsc"], a["ksc"], a["knm"], None)
    assert qk(d=32) == _lib.MAGI_ERR_UNSUPPORTED
    assert qk(qs=100) == _lib.MAGI_ERR_INVALID_ARG                    # stride < heads*d
    assert qk(qi=C.c_void_p(4098)) == _lib.MAGI_ERR_INVALID_ARG       # misaligned
    assert qk(eps=-1.0) == _lib.MAGI_ERR_INVALID_ARG
    assert qk(ghs=7) == _lib.MAGI_ERR_INVALID_ARG                     # gain stride
    kside = dict(ki=p, ko=C.c_void_p(8192), nk=5, hkv=2, ks=48, kos=48, kohs=24, gk=f, pk=p)
    assert qk(**dict(kside, gk=None)) == _lib.MAGI_ERR_INVALID_ARG    # gain_k NULL
    assert qk(base=None) == _lib.MAGI_ERR_INVALID_ARG                 # rope_base NULL
    assert qk(qi=None) == _lib.MAGI_ERR_INVALID_ARG                   # q NULL
    assert qk(qsc=0.0) == _lib.MAGI_ERR_INVALID_ARG                   # zero scale
    assert qk(knm=f) == _lib.MAGI_ERR_INVALID_ARG                     # k_norm_max without K
    assert qk(ksc=float("inf")) == _lib.MAGI_ERR_INVALID_ARG          # inf scale
    # K output layouts: overlapping vectors, misaligned strides, in-place with a new layout
    assert qk(**dict(kside, kos=24, kohs=24)) == _lib.MAGI_ERR_INVALID_ARG
    assert qk(**dict(kside, kos=24, kohs=100)) == _lib.MAGI_ERR_INVALID_ARG   # group-major needs >= 5*24
    assert qk(**dict(kside, kos=24, kohs=124)) == _lib.MAGI_ERR_INVALID_ARG   # not a 16-byte multiple
    assert qk(**dict(kside, ko=p, kos=24, kohs=120)) == _lib.MAGI_ERR_INVALID_ARG
    # V goes with K, needs both pointers and must not be updated in place
    assert qk(vi=p, vo=f) == _lib.MAGI_ERR_INVALID_ARG
    assert qk(**dict(kside, vi=p)) == _lib.MAGI_ERR_INVALID_ARG
    assert qk(**dict(kside, vi=C.c_void_p(12288), vo=C.c_void_p(12288))) == _lib.MAGI_ERR_INVALID_ARG
    # magi_ffa_fwd
    def ffa(**kw):
        a = dict(q=p, k=p, v=p, out=p, lse=None, nq=16, nk=16, hq=16, hkv=1, d=24, dt=0, qs=384, kvs=24, kvhs=24,
                 os_=384, scale=0.0, knm=None, sl=p, ns=1, w=p, nw=1, ts=p, nts=1)
        a.update(kw)
        return L.magi_ffa_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["nq"], a["nk"], a["hq"], a["hkv"],
                              a["d"], a["dt"], a["qs"], a["kvs"], a["kvhs"], a["os_"], a["scale"], a["knm"], a["sl"],
                              a["ns"], a["w"], a["nw"], a["ts"], a["nts"], None)
    assert ffa(d=64) == _lib.MAGI_ERR_UNSUPPORTED
    assert ffa(dt=3) == _lib.MAGI_ERR_INVALID_ARG
    assert ffa(hq=12, hkv=8) == _lib.MAGI_ERR_INVALID_ARG
    assert ffa(hq=512, hkv=1, qs=512 * 24, os_=512 * 24) == _lib.MAGI_ERR_UNSUPPORTED
    assert ffa(q=None) == _lib.MAGI_ERR_INVALID_ARG
    assert ffa(kvs=20) == _lib.MAGI_ERR_INVALID_ARG
    assert ffa(kvs=28) == _lib.MAGI_ERR_INVALID_ARG      # not a 16-byte multiple
    assert ffa(kvs=1 << 23) == _lib.MAGI_ERR_UNSUPPORTED  # a K/V tile would pass 2^31 bytes
    # K/V layouts: token-major needs kvs >= hkv * kvhs, group-major kvhs >= nk * kvs
    assert ffa(hq=32, hkv=2, qs=768, os_=768, kvs=24, kvhs=24) == _lib.MAGI_ERR_INVALID_ARG
    assert ffa(hq=32, hkv=2, qs=768, os_=768, kvs=24, kvhs=16 * 24 - 8) == _lib.MAGI_ERR_INVALID_ARG
    assert ffa(hq=32, hkv=2, qs=768, os_=768, kvs=48, kvhs=20) == _lib.MAGI_ERR_INVALID_ARG
    assert ffa(hq=32, hkv=2, qs=768, os_=768, kvs=24, kvhs=16 * 24 + 4) == _lib.MAGI_ERR_INVALID_ARG  # 16-byte
    assert ffa(out=C.c_void_p(4100)) == _lib.MAGI_ERR_INVALID_ARG
    assert ffa(lse=C.c_void_p(4098)) == _lib.MAGI_ERR_INVALID_ARG
    assert ffa(scale=float("nan")) == _lib.MAGI_ERR_INVALID_ARG
    assert ffa(knm=C.c_void_p(4098)) == _lib.MAGI_ERR_INVALID_ARG
    assert ffa(w=None) == _lib.MAGI_ERR_INVALID_ARG
    assert ffa(nw=-1) == _lib.MAGI_ERR_INVALID_ARG
    assert ffa(nq=-2) == _lib.MAGI_ERR_INVALID_ARG
    assert ffa(nq=0, q=None, out=None) == _lib.MAGI_ERR_INVALID_ARG  # work for no rows
    assert b"work" in L.magi_last_error()


def test_fused_forward_entry_validates_q_prologue():
    L = _lib.lib()
    p = C.c_void_p(4096)  # never dereferenced: every call below fails validation

    def fq(**kw):
        a = dict(dt=0, gq=p, ghs=0, eps=1e-6, pq=p, base=p, qsc=1.0, qhat=None, qhs=0)
        a.update(kw)
        return L.magi_ffa_fwd_qknorm(p, p, p, p, None, 16, 16, 16, 1, 24, a["dt"], 384, 24, 24, 384, 0.0, None, p, 1,
                                     p, 1, p, 1, a["gq"], a["ghs"], a["eps"], a["pq"], a["base"], a["qsc"], a["qhat"],
                                     a["qhs"], None)
    assert fq(dt=1) == _lib.MAGI_ERR_UNSUPPORTED          # bf16 only
    assert fq(gq=None) == _lib.MAGI_ERR_INVALID_ARG
    assert fq(pq=None) == _lib.MAGI_ERR_INVALID_ARG
    assert fq(base=None) == _lib.MAGI_ERR_INVALID_ARG
    assert fq(ghs=5) == _lib.MAGI_ERR_INVALID_ARG
    assert fq(eps=-1.0) == _lib.MAGI_ERR_INVALID_ARG
    assert fq(qsc=0.0) == _lib.MAGI_ERR_INVALID_ARG
    assert fq(qhat=p, qhs=100) == _lib.MAGI_ERR_INVALID_ARG   # q_hat row stride < heads * d


def test_timed_forward_entry_validates_like_the_forward():
    """magi_ffa_fwd_timed checks its arguments exactly as magi_ffa_fwd, before
    any HIP call (the events are never touched when validation fails)."""
    L = _lib.lib()
    p = C.c_void_p(4096)  # never dereferenced: every call below fails validation

    def ft(**kw):
        a = dict(q=p, nq=16, kvs=24, scale=0.0, w=p, ev=p)
        a.update(kw)
        return L.magi_ffa_fwd_timed(a["q"], p, p, p, None, a["nq"], 16, 16, 1, 24, 0, 384, a["kvs"], 24, 384,
                                    a["scale"], None, p, 1, a["w"], 1, p, 1, None, a["ev"], a["ev"])
    assert ft(q=None) == _lib.MAGI_ERR_INVALID_ARG
    assert ft(kvs=20) == _lib.MAGI_ERR_INVALID_ARG
    assert ft(scale=float("nan")) == _lib.MAGI_ERR_INVALID_ARG
    assert ft(w=None) == _lib.MAGI_ERR_INVALID_ARG
    assert ft(nq=-2, ev=None) == _lib.MAGI_ERR_INVALID_ARG


def test_backward_entry_validates_split_workspace():
    L = _lib.lib()
    p = C.c_void_p(4096)  # never dereferenced: every call below fails validation

    def bwd(**kw):
        a = dict(nq=16, nk=16, hq=16, hkv=1, d=24, dt=0, qs=384, kvs=24, kvhs=24, os_=384, slot=p, red=p, nred=1,
                 nslots=2, part=p, nfl=2 * 2 * 128 * 24, lse=p, delta=p)
        a.update(kw)
        return L.magi_ffa_bwd(p, p, p, p, p, a["lse"], p, p, p, a["delta"], a["nq"], a["nk"], a["hq"], a["hkv"],
                              a["d"], a["dt"], a["qs"], a["kvs"], a["kvhs"], a["os_"], 0.0, p, 1, p, 1, p, 1, p, 1,
                              p, 1, a["slot"], a["red"], a["nred"], a["nslots"], a["part"], a["nfl"], None)
    assert bwd(part=None) == _lib.MAGI_ERR_INVALID_ARG            # split schedule without workspace
    assert bwd(slot=None) == _lib.MAGI_ERR_INVALID_ARG
    assert bwd(nfl=2 * 2 * 128 * 24 - 1) == _lib.MAGI_ERR_INVALID_ARG   # workspace too small
    assert bwd(part=C.c_void_p(4100)) == _lib.MAGI_ERR_INVALID_ARG      # misaligned
    assert bwd(nred=-1) == _lib.MAGI_ERR_INVALID_ARG
    assert bwd(delta=None) == _lib.MAGI_ERR_INVALID_ARG
    assert bwd(kvhs=20) == _lib.MAGI_ERR_INVALID_ARG                    # K/V layout overlaps
    assert b"K/V" in L.magi_last_error() or b"overlap" in L.magi_last_error()
    # a Q/dO tile of the dK/dV pass would pass 32-bit byte offsets
    assert bwd(qs=1 << 23) == _lib.MAGI_ERR_UNSUPPORTED
    assert bwd(os_=1 << 23) == _lib.MAGI_ERR_UNSUPPORTED
    assert b"2^23" in L.magi_last_error()


def test_noalloc_backward_entry_validates_and_bounds_its_scratch():
    # the same checks as magi_ffa_bwd, then the static-scratch bound; every
    # call below fails on the host, before any HIP call
    L = _lib.lib()
    p = C.c_void_p(4096)  # never dereferenced

    def bwd(**kw):
        a = dict(nq=16, nk=16, hq=16, hkv=1, d=24, qs=384, kvs=24, kvhs=24, os_=384, slot=p, red=p, nred=1,
                 nslots=2, lse=p)
        a.update(kw)
        return L.magi_ffa_bwd_noalloc(p, p, p, p, p, a["lse"], p, p, p, a["nq"], a["nk"], a["hq"], a["hkv"],
                                      a["d"], 0, a["qs"], a["kvs"], a["kvhs"], a["os_"], 0.0, p, 1, p, 1, p, 1, p,
                                      1, p, 1, a["slot"], a["red"], a["nred"], a["nslots"], None)
    assert bwd(slot=None) == _lib.MAGI_ERR_INVALID_ARG
    assert bwd(lse=None) == _lib.MAGI_ERR_INVALID_ARG
    assert bwd(kvhs=20) == _lib.MAGI_ERR_INVALID_ARG
    assert bwd(d=32) == _lib.MAGI_ERR_UNSUPPORTED
    # 64 MiB = 16 Mi floats: 2731 slots x 2 x 128 x 24 floats leave no room for delta
    assert bwd(nslots=2731) == _lib.MAGI_ERR_UNSUPPORTED
    assert b"scratch" in L.magi_last_error()
    # delta alone: nq x hq floats past the bound (rows of 48 heads x 24)
    big = (16 << 20) // 48 + 1
    assert bwd(nq=big, hq=48, qs=48 * 24, os_=48 * 24, nk=16, nslots=0, nred=0, slot=None, red=None) == \
        _lib.MAGI_ERR_UNSUPPORTED


def test_cross_slices():
    # one FULL slice per sample with both lengths > 0, matching the dense
    # "video rows of a sample see that sample's condition rows" mask
    samples = [(0, 50, 0, 7), (50, 30, 7, 0), (80, 40, 7, 13), (120, 0, 20, 5), (120, 10, 0, 7)]
    sl = ops.build_cross_slices(samples)
    assert len(sl) == 3
    m = oracle.slices_mask([tuple(int(x) for x in s) for s in sl], 130, 20)
    want = np.zeros((130, 20), bool)
    for qo, ql, ko, kl in samples:
        want[qo:qo + ql, ko:ko + kl] = True
    np.testing.assert_array_equal(m, want)
    check_schedule(sl, 130, 20, 16, 1, 24)
    with pytest.raises(_lib.MagiError) as e:
        ops.build_cross_slices([(0, 10, 0, 5), (5, 10, 5, 5)])
    assert e.value.status == _lib.MAGI_ERR_OVERLAP
    with pytest.raises(_lib.MagiError) as e:
        ops.build_cross_slices([(0, -1, 0, 5)])
    assert e.value.status == _lib.MAGI_ERR_INVALID_ARG


def test_ring_slices_match_chunk_windows():
    # brute force: in-flight chunk c sees exactly the slots of chunks
    # max(first, c - r) .. c of the ring, whatever the wrap
    rng = np.random.Generator(np.random.PCG64(77))
    for _ in range(200):
        C, S = int(rng.integers(1, 5)), int(rng.integers(1, 9))
        cnt = int(rng.integers(1, S + 1))
        n = int(rng.integers(1, cnt + 1))
        first = int(rng.integers(0, 20))
        kvr = [int(x) for x in rng.integers(-1, 6, n)]
        sl = ops.build_ring_slices(C, S, first, cnt, n, kvr, q_offset=3, k_offset=5)
        nq, nk = 3 + n * C, 5 + S * C
        m = oracle.slices_mask([tuple(int(x) for x in s) for s in sl], nq, nk)
        want = np.zeros((nq, nk), bool)
        for j in range(n):
            c = first + cnt - n + j
            lo = first if kvr[j] < 0 else max(first, c - kvr[j])
            for cc in range(lo, c + 1):
                s = cc % S
                want[3 + j * C:3 + (j + 1) * C, 5 + s * C:5 + (s + 1) * C] = True
        np.testing.assert_array_equal(m, want)
    with pytest.raises(_lib.MagiError):
        ops.build_ring_slices(4, 3, 0, 4, 1)          # more chunks than slots
    with pytest.raises(_lib.MagiError):
        ops.build_ring_slices(4, 3, 0, 3, 4)          # more in flight than present
    assert ops.ring_slot_runs(6, 4, 6) == [(4, 2), (0, 4)]


# --------------------------------------------------------------------------- sliding window

@pytest.mark.parametrize("trial", range(15))
def test_window_builder_round_trip(trial):
    rng = np.random.Generator(np.random.PCG64(1500 + trial))
    spec, qo, ko = [], 0, 0
    for _ in range(int(rng.integers(1, 5))):
        ln = int(rng.integers(0, 30))
        w = int(rng.integers(1, 35))
        qo += int(rng.integers(0, 3))
        ko += int(rng.integers(0, 3))
        spec.append((ln, w, qo, ko))
        qo += ln
        ko += ln
    sl = ops.build_window_slices(spec)
    assert set(sl[:, 4]) <= {_lib.MASK_CAUSAL, _lib.MASK_BICAUSAL}
    np.testing.assert_array_equal(expand(sl, qo, ko), oracle.window_mask(spec, qo, ko))
    check_schedule(sl, qo, ko, 16, 2, 24)
    check_schedule_kv(sl, qo, ko, 16, 2, 24, tile_k=int(rng.choice([0, 7])))


def test_window_builder_slices_and_errors():
    np.testing.assert_array_equal(ops.build_window_slices([(10, 4, 0, 0)]),
                                  [[0, 3, 0, 3, _lib.MASK_CAUSAL], [3, 10, 0, 10, _lib.MASK_BICAUSAL]])
    np.testing.assert_array_equal(ops.build_window_slices([(10, 1, 5, 2)]), [[5, 15, 2, 12, _lib.MASK_BICAUSAL]])
    np.testing.assert_array_equal(ops.build_window_slices([(10, 10, 0, 0), (0, 3, 10, 10)]),
                                  [[0, 10, 0, 10, _lib.MASK_CAUSAL]])
    for bad, code in [([(10, 0, 0, 0)], _lib.MAGI_ERR_INVALID_ARG), ([(-1, 2, 0, 0)], _lib.MAGI_ERR_INVALID_ARG),
                      ([(10, 2, -1, 0)], _lib.MAGI_ERR_INVALID_ARG),
                      ([(10, 2, 2 ** 31 - 5, 0)], _lib.MAGI_ERR_INVALID_ARG),
                      ([(10, 2, 0, 0), (10, 2, 5, 20)], _lib.MAGI_ERR_OVERLAP),
                      ([(10, 2, 0, 0), (10, 2, 20, 9)], _lib.MAGI_ERR_OVERLAP)]:
        with pytest.raises(_lib.MagiError) as e:
            ops.build_window_slices(bad)
        assert e.value.status == code
    L = _lib.lib()
    n = C.c_int32()
    assert L.magi_slices_window(None, 1, None, 0, C.byref(n)) == _lib.MAGI_ERR_INVALID_ARG
    assert L.magi_slices_window(None, 0, None, 0, None) == _lib.MAGI_ERR_INVALID_ARG
    descs = (_lib.WindowDesc * 1)(_lib.WindowDesc(10, 4, 0, 0))
    buf = (_lib.AttnSlice * 1)()
    assert L.magi_slices_window(descs, 1, buf, 1, C.byref(n)) == _lib.MAGI_ERR_BUFFER_TOO_SMALL and n.value == 2
    assert L.magi_slices_window(descs, 1, None, 0, C.byref(n)) == 0 and n.value == 2


def test_window_schedule_costs_large():
    # one 28,800-token sequence with a 3,600-token window: the area is
    # closed form, sum over rows of min(w, i + 1)
    n, w = 28800, 3600
    sl = ops.build_window_slices([(n, w, 0, 0)])
    work, _ = ops.schedule(sl, n, n, 128, 8, 48, _lib.DTYPE_BF16)
    area = w * (w + 1) // 2 + (n - w) * w
    assert work[:, 5].astype(np.int64).sum() == area * 8
    work, _, ext, red, nslots = ops.schedule_kv(sl, n, n, 128, 8, 48, _lib.DTYPE_BF16)
    assert work[:, 5].astype(np.int64).sum() == area * 8


def test_product_path_has_no_fallback(tmp_path):
    # without the built library every entry point raises; nothing computes
    # the attention elsewhere (the package never imports the oracle)
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from block_causal_attention_amd import _lib, ops\n"
            "_lib.LIB_PATH = %r\n"
            "try:\n"
            "    ops.build_slices([])\n"
            "except ImportError as e:\n"
            "    print('raised', e)\n") % (ROOT, str(tmp_path / "missing.so"))
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and "raised" in out.stdout and "missing.so is missing" in out.stdout, out
    pkg = os.path.join(ROOT, "block_causal_attention_amd")
    for f in os.listdir(pkg):
        if f.endswith(".py"):
            src = open(os.path.join(pkg, f)).read()
            assert not re.search(r"^\s*(import|from)\s+oracle", src, re.M), f

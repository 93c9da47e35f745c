"""Thin torch binding over libmagi_bca's C ABI: argument marshalling only.

Every step of the attention path runs in the library (host builder and
scheduler in C++, prologue and attention in HIP kernels).  PyTorch supplies
device memory and the current stream.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np
import torch

from . import _lib
from ._lib import AttnSlice, CrossDesc, KvReduce, RingDesc, SeqDesc, WindowDesc, WorkItem, check, lib

LN2 = 0.6931471805599453
LOG2E = 1.4426950408889634

__all__ = ["build_slices", "schedule", "Plan", "make_plan", "plan_for_videos", "qknorm_rope",
           "ffa_fwd", "ffa_bwd", "QNorm", "kv_group_major", "default_tile_q", "dtype_code"]


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return _lib.DTYPE_BF16
    if dt == torch.float32:
        return _lib.DTYPE_FP32
    raise TypeError(f"unsupported dtype {dt} (bfloat16 or float32)")


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def build_slices(seqs: Sequence) -> np.ndarray:
    """magi_slices_build: packed-video descriptors -> int32 [n, 5] slices
    (q_start, q_end, k_start, k_end, mask_type).  ``seqs`` items need the
    fields chunk_len, num_kv_chunks, num_q_chunks, q_offset, k_offset and
    kv_range (sequence of ints, or None)."""
    n = len(seqs)
    descs = (SeqDesc * max(n, 1))()
    keep = []
    for i, s in enumerate(seqs):
        kvr = getattr(s, "kv_range", None)
        arr = None
        if kvr is not None:
            arr = (C.c_int32 * max(len(kvr), 1))(*kvr)
            keep.append(arr)
        descs[i] = SeqDesc(s.chunk_len, s.num_kv_chunks, s.num_q_chunks, s.q_offset, s.k_offset,
                           C.cast(arr, C.POINTER(C.c_int32)) if arr is not None else None)
    # one call with a generous capacity; the size query only on overflow
    cnt = C.c_int32(0)
    cap = 2 * sum(int(s.num_q_chunks) for s in seqs) + 4
    while True:
        out = np.empty((cap, 5), np.int32)
        st = lib().magi_slices_build(descs, n, out.ctypes.data_as(C.POINTER(AttnSlice)), cap, C.byref(cnt))
        if st != _lib.MAGI_ERR_BUFFER_TOO_SMALL:
            check(st)
            return out[:cnt.value]
        cap = cnt.value


def build_cross_slices(samples: Sequence) -> np.ndarray:
    """magi_slices_cross: samples (q_offset, q_len, k_offset, k_len) of a packed
    cross-attention (video tokens over their own condition tokens) -> int32
    [n, 5] FULL slices."""
    n = len(samples)
    descs = (CrossDesc * max(n, 1))()
    for i, (qo, ql, ko, kl) in enumerate(samples):
        descs[i] = CrossDesc(int(qo), int(ql), int(ko), int(kl))
    cnt = C.c_int32(0)
    out = np.empty((max(n, 1), 5), np.int32)
    check(lib().magi_slices_cross(descs, n, out.ctypes.data_as(C.POINTER(AttnSlice)), out.shape[0], C.byref(cnt)))
    return out[:cnt.value]


def build_window_slices(seqs: Sequence) -> np.ndarray:
    """magi_slices_window: packed causal sliding-window sequences (len,
    window, q_offset, k_offset) -> int32 [n, 5] slices (CAUSAL for the rows
    whose window reaches the sequence start, BICAUSAL bands for the rest)."""
    n = len(seqs)
    descs = (WindowDesc * max(n, 1))()
    for i, (ln, w, qo, ko) in enumerate(seqs):
        descs[i] = WindowDesc(int(ln), int(w), int(qo), int(ko))
    cnt = C.c_int32(0)
    out = np.empty((2 * max(n, 1), 5), np.int32)
    check(lib().magi_slices_window(descs, n, out.ctypes.data_as(C.POINTER(AttnSlice)), out.shape[0], C.byref(cnt)))
    return out[:cnt.value]


def build_ring_slices(chunk_len: int, ring_slots: int, first_chunk: int, num_chunks: int, num_inflight: int,
                      kv_range=None, q_offset: int = 0, k_offset: int = 0) -> np.ndarray:
    """magi_slices_ring: a streaming step over a ring-buffer KV cache -> int32
    [n, 5] FULL slices (global chunk c in slot c mod ring_slots)."""
    arr = None
    if kv_range is not None:
        arr = (C.c_int32 * max(len(kv_range), 1))(*[int(x) for x in kv_range])
    desc = RingDesc(chunk_len, ring_slots, first_chunk, num_chunks, num_inflight, q_offset, k_offset,
                    C.cast(arr, C.POINTER(C.c_int32)) if arr is not None else None)
    cnt = C.c_int32(0)
    out = np.empty((2 * max(num_inflight, 1), 5), np.int32)
    check(lib().magi_slices_ring(C.byref(desc), out.ctypes.data_as(C.POINTER(AttnSlice)), out.shape[0],
                                 C.byref(cnt)))
    return out[:cnt.value]


def ring_slot_runs(ring_slots: int, first: int, count: int):
    """Contiguous slot runs [(slot0, n_chunks), ...] holding global chunks
    first .. first + count - 1 (at most two: the ring wraps once)."""
    runs = []
    c = first
    end = first + count
    while c < end:
        s0 = c % ring_slots
        n = min(end - c, ring_slots - s0)
        runs.append((s0, n))
        c += n
    return runs


def default_tile_q(hq: int, hkv: int, head_dim: int, dtype: int) -> int:
    return check(lib().magi_default_tile_q(hq, hkv, head_dim, dtype))


def _schedule(fn, dflt_fn, slices, nq, nk, hq, hkv, head_dim, dtype, tile):
    s = np.ascontiguousarray(np.asarray(slices, np.int32).reshape(-1, 5))
    sp = s.ctypes.data_as(C.POINTER(AttnSlice)) if len(s) else None
    nw, nt = C.c_int32(0), C.c_int32(0)
    # one call with capacities that fit the usual schedule; the exact sizes
    # come back with MAGI_ERR_BUFFER_TOO_SMALL otherwise
    t = tile if tile > 0 else max(check(dflt_fn(hq, hkv, head_dim, dtype)), 1)
    tiles = -(-max(nq, nk) // t) + 2 * len(s) + 1
    wcap, tcap = max(tiles * hkv, 1), max(tiles * min(max(len(s), 1), 8), 1)
    while True:
        work = np.empty((wcap, 6), np.int32)
        ts = np.empty(tcap, np.int32)
        st = fn(sp, len(s), nq, nk, hq, hkv, head_dim, dtype, tile,
                work.ctypes.data_as(C.POINTER(WorkItem)), wcap, C.byref(nw),
                ts.ctypes.data_as(C.POINTER(C.c_int32)), tcap, C.byref(nt))
        if st != _lib.MAGI_ERR_BUFFER_TOO_SMALL:
            check(st)
            return work[:nw.value], ts[:nt.value]
        wcap, tcap = max(nw.value, 1), max(nt.value, 1)


def schedule(slices: np.ndarray, nq: int, nk: int, hq: int, hkv: int, head_dim: int, dtype: int,
             tile_q: int = 0):
    """magi_schedule: slices -> query-major (work int32 [m, 6], tile_slices int32 [t])."""
    L = lib()
    return _schedule(L.magi_schedule, L.magi_default_tile_q, slices, nq, nk, hq, hkv, head_dim, dtype, tile_q)


def schedule_kv(slices: np.ndarray, nq: int, nk: int, hq: int, hkv: int, head_dim: int, dtype: int,
                tile_k: int = 0):
    """magi_schedule_kv: slices -> key-major lists for the backward's dK/dV
    pass: (work int32 [m, 6], tile_slices int32 [t], item_ext int32 [m, 3],
    reduce int32 [r, 5], num_slots).  q_start/q_len of an item are its keys;
    item_ext holds {partial slot of a part of a split key tile or -1, first
    query token, one past the last query token} of each item."""
    L = lib()
    s = np.ascontiguousarray(np.asarray(slices, np.int32).reshape(-1, 5))
    sp = s.ctypes.data_as(C.POINTER(AttnSlice)) if len(s) else None
    nw, nt, nr, ns = C.c_int32(0), C.c_int32(0), C.c_int32(0), C.c_int32(0)
    check(L.magi_schedule_kv(sp, len(s), nq, nk, hq, hkv, head_dim, dtype, tile_k, None, 0, C.byref(nw),
                             None, 0, C.byref(nt), None, None, 0, C.byref(nr), C.byref(ns)))
    work = np.empty((max(nw.value, 1), 6), np.int32)
    ts = np.empty(max(nt.value, 1), np.int32)
    ext = np.empty((max(nw.value, 1), 3), np.int32)
    red = np.empty((max(nr.value, 1), 5), np.int32)
    check(L.magi_schedule_kv(sp, len(s), nq, nk, hq, hkv, head_dim, dtype, tile_k,
                             work.ctypes.data_as(C.POINTER(WorkItem)), work.shape[0], C.byref(nw),
                             ts.ctypes.data_as(C.POINTER(C.c_int32)), ts.shape[0], C.byref(nt),
                             ext.ctypes.data_as(C.POINTER(C.c_int32)),
                             red.ctypes.data_as(C.POINTER(KvReduce)), red.shape[0], C.byref(nr), C.byref(ns)))
    return work[:nw.value], ts[:nt.value], ext[:nw.value], red[:nr.value], ns.value


@dataclass
class Plan:
    """Device copies of a schedule, ready for ffa_fwd (flat int32 views of one
    device buffer; ``host`` keeps the shaped host arrays)."""
    nq: int
    nk: int
    hq: int
    hkv: int
    head_dim: int
    dtype: int
    slices: torch.Tensor
    work: torch.Tensor
    tile_slices: torch.Tensor
    host: dict = field(default_factory=dict)
    ready: Optional[torch.cuda.Event] = None  # recorded after the upload; ffa_fwd waits on it
    kwork: Optional[torch.Tensor] = None        # key-major lists (backward plans only)
    k_tile_slices: Optional[torch.Tensor] = None
    kitem_ext: Optional[torch.Tensor] = None    # {partial slot or -1, token window} per key-major item
    kreduce: Optional[torch.Tensor] = None      # int32 [r, 5] sums of split key tiles
    num_slots: int = 0
    waited: list = field(default_factory=list)  # streams already ordered after ``ready``

    @property
    def num_work(self) -> int:
        return int(self.host["work"].shape[0])

    def wait(self, stream) -> None:
        """Order ``stream`` after the plan's upload, once per stream (later
        work on a stream that has waited is ordered after the upload too)."""
        if self.ready is not None and not any(s == stream for s in self.waited):
            stream.wait_event(self.ready)
            self.waited.append(stream)

    def settle(self) -> "Plan":
        """Wait on the host for the plan's upload and drop its event, so that
        the plan can be used inside HIP graph capture (a captured stream
        cannot wait on an event recorded outside the capture).  A settled
        plan's device lists stay fixed, so a captured graph may replay it any
        number of times.  Returns the plan."""
        if self.ready is not None:
            self.ready.synchronize()
            self.ready = None
        return self


def make_plan(slices: np.ndarray, nq: int, nk: int, hq: int, hkv: int, head_dim: int, dtype,
              device="cuda", tile_q: int = 0, backward: bool = False) -> Plan:
    """schedule (+ schedule_kv when ``backward``) + one upload: the int32
    lists travel in a single pinned host-to-device copy and the plan holds
    views of it."""
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    slices = np.asarray(slices, np.int32).reshape(-1, 5)
    work, ts = schedule(slices, nq, nk, hq, hkv, head_dim, code, tile_q)
    parts = [slices.reshape(-1), work.reshape(-1), ts.reshape(-1)]
    if backward:
        kwork, kts, kext, kred, nslots = schedule_kv(slices, nq, nk, hq, hkv, head_dim, code)
        parts += [kwork.reshape(-1), kts.reshape(-1), kext.reshape(-1), kred.reshape(-1)]
    sizes = [max(p.size, 1) for p in parts]     # an empty list still gets one valid word
    # The copy runs on a side stream so it does not queue behind the work
    # already on the caller's stream (the previous attention launch); only
    # ffa_fwd waits for it, through ``ready``.
    main = torch.cuda.current_stream(device)
    side = _upload_stream(main.device)
    host, slot_done = _staging_slot(main.device, sum(sizes))
    hv = host.numpy()
    off = 0
    for p, n in zip(parts, sizes):
        hv[off:off + p.size] = p
        off += n
    with torch.cuda.stream(side):
        dev = torch.empty(sum(sizes), dtype=torch.int32, device=main.device)
        dev.copy_(host, non_blocking=True)
        ready = torch.cuda.Event()
        ready.record(side)
        slot_done.record(side)
    dev.record_stream(main)
    offs = np.cumsum([0] + sizes)
    views = [dev[offs[i]:offs[i + 1]] for i in range(len(parts))]
    host_arrays = {"slices": slices, "work": work, "tile_slices": ts}
    plan = Plan(nq, nk, hq, hkv, head_dim, code, views[0], views[1], views[2], host_arrays, ready)
    if backward:
        plan.kwork, plan.k_tile_slices, plan.kitem_ext, plan.kreduce = views[3], views[4], views[5], views[6]
        plan.num_slots = nslots
        host_arrays.update(kwork=kwork, k_tile_slices=kts, kitem_ext=kext, kreduce=kred)
    return plan


_UPLOAD_STREAMS = {}
_STAGING = {}
_STAGING_SLOTS = 8  # plan uploads that may be in flight at once per device


def _staging_slot(device, words: int):
    """A pinned int32 staging buffer of at least ``words`` entries from a
    fixed ring per device, and the event that marks its copy as done.

    Allocating pinned memory per upload is slow and, when the host runs far
    ahead of the GPU, turns every plan into a fresh pinned allocation.  The
    ring reuses a slot once the copy that last read it has finished; when all
    slots are still in flight the host waits for the oldest, which bounds how
    far plan building runs ahead of the GPU."""
    idx = torch.device(device).index
    idx = torch.cuda.current_device() if idx is None else idx
    ring = _STAGING.setdefault(idx, {"next": 0, "slots": [None] * _STAGING_SLOTS})
    i = ring["next"]
    ring["next"] = (i + 1) % _STAGING_SLOTS
    slot = ring["slots"][i]
    if slot is not None:
        slot[1].synchronize()   # the copy that last read this slot has finished
    if slot is None or slot[0].numel() < words:
        cap = max(words, 2 * slot[0].numel() if slot is not None else 4096)
        slot = (torch.empty(cap, dtype=torch.int32, pin_memory=True), torch.cuda.Event())
        ring["slots"][i] = slot
    return slot[0][:words], slot[1]


def _upload_stream(device) -> torch.cuda.Stream:
    """One default-priority side stream per device for plan uploads."""
    idx = torch.device(device).index
    idx = torch.cuda.current_device() if idx is None else idx
    s = _UPLOAD_STREAMS.get(idx)
    if s is None:
        s = _UPLOAD_STREAMS[idx] = torch.cuda.Stream(device=idx)
    return s


def plan_for_videos(seqs: Sequence, nq: int, nk: int, hq: int, hkv: int, head_dim: int, dtype,
                    device="cuda", tile_q: int = 0, backward: bool = False) -> Plan:
    """build_slices + schedule (+ schedule_kv) + upload."""
    return make_plan(build_slices(seqs), nq, nk, hq, hkv, head_dim, dtype, device, tile_q, backward)


def _check_3d(name, t, heads, d, any_head_stride=False):
    """[n, heads, d] on the GPU with contiguous channels; the heads of a token
    must be contiguous too unless ``any_head_stride`` (K/V layouts, checked
    for overlap by the library)."""
    if t.dim() != 3 or t.shape[1] != heads or t.shape[2] != d:
        raise ValueError(f"{name}: expected [n, {heads}, {d}], got {list(t.shape)}")
    if t.stride(2) != 1 or (t.stride(1) != d and not any_head_stride):
        raise ValueError(f"{name}: heads and channels must be contiguous (strides {t.stride()})")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


def kv_group_major(nk: int, hkv: int, d: int, dtype, device="cuda") -> torch.Tensor:
    """An empty [nk, hkv, d] K or V tensor stored group-major ([hkv][nk][d]
    underneath): each K/V tile of a group is then one contiguous block, which
    the attention kernels load faster than the token-major layout."""
    return torch.empty((hkv, nk, d), dtype=dtype, device=device).transpose(0, 1)


def qknorm_rope(q: torch.Tensor, k: Optional[torch.Tensor], gain_q: torch.Tensor,
                gain_k: Optional[torch.Tensor], pos_q: torch.Tensor, pos_k: Optional[torch.Tensor],
                rope_base: torch.Tensor, eps: float = 1e-6, q_out: Optional[torch.Tensor] = None,
                k_out: Optional[torch.Tensor] = None, q_scale: float = 1.0, k_scale: float = 1.0,
                k_norm_max: Optional[torch.Tensor] = None, v: Optional[torch.Tensor] = None,
                v_out: Optional[torch.Tensor] = None):
    """magi_qknorm_rope: QK-Norm then 3D RoPE (results times q_scale / k_scale);
    returns (q_out, k_out), or (q_out, k_out, v_out) when ``v`` is given.
    ``k_norm_max`` (float32 [hkv], optional) receives an upper bound on the
    norm of every output key of each head.  ``k_out`` may be any [nk, hkv, d]
    view with contiguous channels, e.g. kv_group_major(); ``v`` (laid out like
    k) is then copied into ``v_out`` (default: a tensor laid out like k_out)."""
    if q is None:   # K (and V) only: Q is normalised elsewhere (ffa_fwd(..., qknorm=...))
        if k is None:
            raise ValueError("nothing to do: q and k are both None")
        d = k.shape[-1]
        if q_out is not None:
            raise ValueError("q_out needs q")
        gain_q = gain_k if gain_q is None else gain_q
    else:
        d = q.shape[-1]
        _check_3d("q", q, q.shape[1], d)
        q_out = torch.empty_like(q) if q_out is None else q_out
        _check_3d("q_out", q_out, q.shape[1], d)
        if q_out.stride(0) != q.stride(0):
            raise ValueError("q and q_out must share the row stride")
    ghs = 0 if gain_q.dim() == 1 else d
    if gain_k is not None and gain_k.dim() != gain_q.dim():
        raise ValueError("gain_q and gain_k must both be shared [d] or both per head [heads, d]")
    nk, hkv, ks = 0, 1, (q.shape[1] * d if q is not None else d)
    kos, kohs = ks, d
    if k is not None:
        _check_3d("k", k, k.shape[1], d)
        k_out = torch.empty_like(k) if k_out is None else k_out
        _check_3d("k_out", k_out, k.shape[1], d, any_head_stride=True)
        if k_out.shape != k.shape:
            raise ValueError("k_out must have k's shape")
        nk, hkv, ks = k.shape[0], k.shape[1], k.stride(0)
        kos, kohs = k_out.stride(0), k_out.stride(1)
    if v is not None:
        if k is None:
            raise ValueError("v needs k")
        _check_3d("v", v, hkv, d)
        if v.shape != k.shape or v.stride() != k.stride() or v.dtype != k.dtype:
            raise ValueError("v must match k in shape, strides and dtype")
        v_out = torch.empty_strided(k_out.shape, k_out.stride(), dtype=v.dtype, device=v.device) \
            if v_out is None else v_out
        if v_out.shape != k_out.shape or v_out.stride() != k_out.stride() or v_out.dtype != v.dtype:
            raise ValueError("v_out must match k_out in shape, strides and dtype")
    elif v_out is not None:
        raise ValueError("v_out needs v")
    if k_norm_max is not None and (k_norm_max.dtype != torch.float32 or k_norm_max.numel() < hkv or
                                   not k_norm_max.is_contiguous() or (k is None or k_norm_max.device != k.device)):
        raise ValueError("k_norm_max must be a contiguous float32 tensor of >= hkv entries on k's device")
    for t in (gain_q, gain_k, rope_base):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("gains and rope_base must be contiguous float32")
    for t in (pos_q, pos_k):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
            raise ValueError("positions must be contiguous int32 [n, 3]")
    nq, hq, qs = (q.shape[0], q.shape[1], q.stride(0)) if q is not None else (0, 1, d)
    dev_t = q if q is not None else k
    check(lib().magi_qknorm_rope(
        _ptr(q), _ptr(q_out), nq, hq, qs,
        _ptr(k), _ptr(k_out), nk, hkv, ks, kos, kohs, _ptr(v), _ptr(v_out), d, dtype_code(dev_t.dtype),
        _ptr(gain_q) if q is not None else None, _ptr(gain_k), ghs, float(eps),
        _ptr(pos_q) if q is not None else None, _ptr(pos_k), _ptr(rope_base),
        float(q_scale), float(k_scale), _ptr(k_norm_max), _stream(dev_t)))
    return (q_out, k_out) if v is None else (q_out, k_out, v_out)


@dataclass
class QNorm:
    """The QK-Norm + 3D RoPE of Q for ffa_fwd(..., qnorm=...): gain [d] or
    [hq, d] (float32), positions int32 [nq, 3], rope base float32 [3]; q_hat
    (optional) receives the normalised, rotated Q."""
    gain: torch.Tensor
    pos: torch.Tensor
    rope_base: torch.Tensor
    eps: float = 1e-6
    scale: float = 1.0
    q_hat: Optional[torch.Tensor] = None


def ffa_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, plan: Plan,
            softmax_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None, return_lse: bool = True,
            k_norm_max: Optional[torch.Tensor] = None, qnorm: Optional[QNorm] = None,
            events: Optional[tuple] = None):
    """magi_ffa_fwd over ``plan``; returns (out [nq, hq, d], lse [nq, hq] fp32 or None).
    ``k_norm_max`` (float32 [hkv], optional) must bound the norm of every key
    row of each group (qknorm_rope writes one).  k and v are [nk, hkv, d]
    views with contiguous channels and one common layout (token-major, or
    group-major as from kv_group_major).  With ``qnorm`` q is the raw Q and
    the kernel applies QK-Norm + 3D RoPE to it (magi_ffa_fwd_qknorm).
    ``events`` (start, stop): torch.cuda.Event objects with timing enabled,
    each recorded once before (so that the HIP event exists); the kernel's
    dispatch records them when it starts and ends (magi_ffa_fwd_timed)."""
    d = q.shape[-1]
    hq, hkv = q.shape[1], k.shape[1]
    _check_3d("q", q, hq, d)
    _check_3d("k", k, hkv, d, any_head_stride=True)
    _check_3d("v", v, hkv, d, any_head_stride=True)
    if k.stride() != v.stride():
        raise ValueError("k and v must share their strides")
    if (plan.nq, plan.nk, plan.hq, plan.hkv, plan.head_dim, plan.dtype) != \
            (q.shape[0], k.shape[0], hq, hkv, d, dtype_code(q.dtype)):
        raise ValueError("plan was made for a different shape or dtype")
    if k_norm_max is not None and (k_norm_max.dtype != torch.float32 or k_norm_max.numel() < hkv or
                                   not k_norm_max.is_contiguous() or k_norm_max.device != q.device):
        raise ValueError("k_norm_max must be a contiguous float32 tensor of >= hkv entries on q's device")
    out = torch.empty_like(q) if out is None else out
    _check_3d("out", out, hq, d)
    if lse is None and return_lse:
        lse = torch.empty((q.shape[0], hq), dtype=torch.float32, device=q.device)
    plan.wait(torch.cuda.current_stream(q.device))
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), q.shape[0], k.shape[0], hq, hkv, d,
            dtype_code(q.dtype), q.stride(0), k.stride(0), k.stride(1), out.stride(0),
            0.0 if softmax_scale is None else float(softmax_scale), _ptr(k_norm_max),
            _ptr(plan.slices), int(plan.host["slices"].shape[0]), _ptr(plan.work), plan.num_work,
            _ptr(plan.tile_slices), int(plan.host["tile_slices"].shape[0]))
    if events is not None:
        if qnorm is not None:
            raise ValueError("events and qnorm cannot be combined")
        handles = [e.cuda_event for e in events]
        if len(handles) != 2 or not all(handles):
            raise ValueError("events must be two torch.cuda.Event objects that have been recorded once")
        check(lib().magi_ffa_fwd_timed(*args, _stream(q), handles[0], handles[1]))
        return out, lse
    if qnorm is None:
        check(lib().magi_ffa_fwd(*args, _stream(q)))
        return out, lse
    g = qnorm
    for t in (g.gain, g.rope_base):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("qnorm gain and rope_base must be contiguous float32")
    if g.pos.dtype != torch.int32 or not g.pos.is_contiguous() or g.pos.shape != (q.shape[0], 3):
        raise ValueError("qnorm positions must be contiguous int32 [nq, 3]")
    if g.q_hat is not None:
        _check_3d("q_hat", g.q_hat, hq, d)
    check(lib().magi_ffa_fwd_qknorm(*args, _ptr(g.gain), 0 if g.gain.dim() == 1 else d, float(g.eps), _ptr(g.pos),
                                    _ptr(g.rope_base), float(g.scale), _ptr(g.q_hat),
                                    g.q_hat.stride(0) if g.q_hat is not None else 0, _stream(q)))
    return out, lse


def _bwd_common(q, k, v, out, dout, lse, plan, dq, dk, dv):
    d = q.shape[-1]
    hq, hkv = q.shape[1], k.shape[1]
    for name, t, heads in (("q", q, hq), ("k", k, hkv), ("v", v, hkv), ("out", out, hq), ("dout", dout, hq)):
        _check_3d(name, t, heads, d, any_head_stride=name in ("k", "v"))
    if k.stride() != v.stride() or out.stride(0) != dout.stride(0):
        raise ValueError("k/v must share their strides and out/dout their row strides")
    if plan.kwork is None:
        raise ValueError("plan has no key-major lists: make it with backward=True")
    if (plan.nq, plan.nk, plan.hq, plan.hkv, plan.head_dim, plan.dtype) != \
            (q.shape[0], k.shape[0], hq, hkv, d, dtype_code(q.dtype)):
        raise ValueError("plan was made for a different shape or dtype")
    if lse.dtype != torch.float32 or lse.shape != (q.shape[0], hq) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [nq, hq]")
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.shape != ref.shape or t.stride() != ref.stride() or t.dtype != ref.dtype:
            raise ValueError(f"{name} must match {name[1:]} in shape, strides and dtype")


def _bwd_list_args(plan):
    H = plan.host
    return (_ptr(plan.slices), int(H["slices"].shape[0]), _ptr(plan.work), plan.num_work,
            _ptr(plan.tile_slices), int(H["tile_slices"].shape[0]),
            _ptr(plan.kwork), int(H["kwork"].shape[0]), _ptr(plan.k_tile_slices), int(H["k_tile_slices"].shape[0]),
            _ptr(plan.kitem_ext), _ptr(plan.kreduce), int(H["kreduce"].shape[0]), plan.num_slots)


def ffa_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, dout: torch.Tensor,
            lse: torch.Tensor, plan: Plan, softmax_scale: Optional[float] = None,
            dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
            dv: Optional[torch.Tensor] = None):
    """magi_ffa_bwd over a backward ``plan`` (make_plan(..., backward=True));
    returns (dq, dk, dv).  q, k, v, out, lse and softmax_scale are the
    forward's; dout has the layout of out."""
    d = q.shape[-1]
    hq = q.shape[1]
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _bwd_common(q, k, v, out, dout, lse, plan, dq, dk, dv)
    delta = torch.empty((q.shape[0], hq), dtype=torch.float32, device=q.device)
    # partial sums of split key tiles: 2 x 128 keys x d fp32 per slot
    nfl = plan.num_slots * 2 * 128 * d
    partial = torch.empty(max(nfl, 4), dtype=torch.float32, device=q.device)
    plan.wait(torch.cuda.current_stream(q.device))
    check(lib().magi_ffa_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(delta),
        q.shape[0], k.shape[0], hq, k.shape[1], d, dtype_code(q.dtype), q.stride(0), k.stride(0), k.stride(1),
        out.stride(0), 0.0 if softmax_scale is None else float(softmax_scale),
        *_bwd_list_args(plan), _ptr(partial), nfl, _stream(q)))
    return dq, dk, dv


def ffa_bwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, dout: torch.Tensor,
                    lse: torch.Tensor, plan: Plan, dq: torch.Tensor, dk: torch.Tensor, dv: torch.Tensor,
                    softmax_scale: Optional[float] = None):
    """magi_ffa_bwd_noalloc: ffa_bwd with its workspace in the library's
    static device scratch; the gradients go into the caller's dq, dk, dv and
    nothing is allocated (the plan must already be on the device)."""
    _bwd_common(q, k, v, out, dout, lse, plan, dq, dk, dv)
    plan.wait(torch.cuda.current_stream(q.device))
    check(lib().magi_ffa_bwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
        q.shape[0], k.shape[0], q.shape[1], k.shape[1], q.shape[-1], dtype_code(q.dtype), q.stride(0), k.stride(0),
        k.stride(1), out.stride(0), 0.0 if softmax_scale is None else float(softmax_scale),
        *_bwd_list_args(plan), _stream(q)))
    return dq, dk, dv

// Device helpers shared by the attention forward and backward kernels
// (gfx950): vector types, the scalar reads of the work and slice lists, the
// walk over the AttnSlices a work item lists, lane-half exchanges and the
// LDS-only workgroup barrier.
#pragma once

#include <hip/hip_runtime.h>

#include "magi_bca.h"

namespace magi {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBufCfg = 0x00020000;  // raw buffer resource word 3 (gfx9 family: 32-bit data format)

__device__ __forceinline__ int32_t uni(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }

// Scalar load of a word that stays constant while the kernel runs (the work
// and slice lists): through the constant address space it becomes a scalar
// memory load, independent of the vector-memory counter.
__device__ __forceinline__ int32_t const_ld(const int32_t* p) {
  return *(__attribute__((address_space(4))) const int32_t*)p;
}

// One work item's fields, read with scalar loads.
__device__ __forceinline__ magi_work_item load_item(const magi_work_item* work, int i) {
  const magi_work_item* wp = work + i;
  magi_work_item w;
  w.q_start = const_ld(&wp->q_start);
  w.q_len = const_ld(&wp->q_len);
  w.slice_begin = const_ld(&wp->slice_begin);
  w.slice_end = const_ld(&wp->slice_end);
  w.kv_group = const_ld(&wp->kv_group);
  w.cost = 0;
  return w;
}

// One slice's fields, read with scalar loads.
__device__ __forceinline__ magi_attn_slice load_slice(const magi_attn_slice* slices, int i) {
  const magi_attn_slice* sp = slices + i;
  magi_attn_slice s;
  s.q_start = const_ld(&sp->q_start);
  s.q_end = const_ld(&sp->q_end);
  s.k_start = const_ld(&sp->k_start);
  s.k_end = const_ld(&sp->k_end);
  s.mask_type = const_ld(&sp->mask_type);
  return s;
}

// Keys [row_key_begin, row_key_end) of row `row` (q_start <= row < q_end)
// under slice s, within [ks, ke).  Bottom-right (causal) bound, type bit 0:
// k - k_end <= row - q_end.  Top-left (inverse causal) bound, type bit 1:
// k - k_start >= row - q_start.
__device__ inline int64_t row_key_end(const magi_attn_slice& s, int64_t ke, int64_t row) {
  if (!(s.mask_type & MAGI_MASK_CAUSAL)) return ke;
  const int64_t e = (int64_t)s.k_end - (int64_t)s.q_end + row + 1;
  return e < ke ? e : ke;
}
__device__ inline int64_t row_key_begin(const magi_attn_slice& s, int64_t ks, int64_t row) {
  if (!(s.mask_type & MAGI_MASK_INVCAUSAL)) return ks;
  const int64_t b = (int64_t)s.k_start - (int64_t)s.q_start + row;
  return b > ks ? b : ks;
}

// The slice lists a kernel walks (device copies of a schedule).
struct SliceLists {
  const magi_attn_slice* slices;
  int32_t num_slices;
  const int32_t* tile_slices;
  int32_t num_tile_slices;
};

// One slice as seen by a query-major work item.  Every field is the same for
// the whole workgroup and lives in scalar registers.  Token and key indices
// fit in 32 bits (the entry points reject nq or nk >= 2^31), so all of it is
// 32-bit scalar arithmetic.
struct SliceGeo {
  int32_t ks;     // first key that any row of the item sees
  int32_t khi;    // one past the last key that any row of the item sees
  int32_t kfull;  // keys below this pass the upper bound of every row of the item
  int32_t klo;    // keys from this on pass the lower bound of every row of the item
  int32_t koff;   // k_end - q_end: under the upper bound row r sees keys below koff + r + 1
  int32_t loff;   // k_start - q_start: under the lower bound row r sees keys from loff + r
  int32_t type;   // mask type: bit 0 = upper (causal) bound, bit 1 = lower bound
  int32_t si;     // position in the tile-slice list
};

// One past the last key row `row` of the item sees: with the upper bound
// min(koff + row + 1, khi), which equals min(koff + row + 1, k_end) for the
// item's rows because khi = min(koff + last row + 1, k_end).
__device__ __forceinline__ int32_t geo_row_end(const SliceGeo& g, int32_t row) {
  const int32_t e = g.koff + row + 1;
  return (g.type & MAGI_MASK_CAUSAL) && e < g.khi ? e : g.khi;
}

// First slice at or after list position si (of the item's [.., slice_end))
// that shows the item's query tokens [first_tok, last_tok] a key.  Returns
// false when the list is exhausted.
__device__ __forceinline__ bool find_slice(const SliceLists& L, int32_t slice_end, int32_t nk, int si,
                                           int32_t first_tok, int32_t last_tok, SliceGeo& g) {
  const int end = slice_end < L.num_tile_slices ? slice_end : L.num_tile_slices;
  for (si = si < 0 ? 0 : si; si < end; ++si) {
    const int sidx = const_ld(L.tile_slices + si);
    if (sidx < 0 || sidx >= L.num_slices) continue;
    const magi_attn_slice s = load_slice(L.slices, sidx);
    const int32_t upper = s.mask_type & MAGI_MASK_CAUSAL, lower = s.mask_type & MAGI_MASK_INVCAUSAL;
    const int32_t ks = s.k_start > 0 ? s.k_start : 0;
    const int32_t ke = s.k_end < nk ? s.k_end : nk;
    // a well-formed schedule only lists slices that cover every row of the
    // item (so qe > last_tok >= first_tok >= qs >= 0, and the host keeps
    // k_start + (q_end - q_start) below 2^31 for a lower bound: no sum below
    // leaves 32 bits)
    if (ks >= ke || first_tok < s.q_start || last_tok >= s.q_end) continue;
    const int32_t koff = s.k_end - s.q_end;
    const int32_t loff = s.k_start - s.q_start;
    const int32_t khi = upper ? (koff + last_tok + 1 < ke ? koff + last_tok + 1 : ke) : ke;
    const int32_t kbeg = lower && loff + first_tok > ks ? loff + first_tok : ks;
    if (khi <= kbeg) continue;
    g.ks = kbeg;
    g.khi = khi;
    g.kfull = upper ? (koff + first_tok + 1 < ke ? koff + first_tok + 1 : ke) : ke;
    g.klo = lower && loff + last_tok > ks ? loff + last_tok : ks;
    g.koff = koff;
    g.loff = loff;
    g.type = s.mask_type & (MAGI_MASK_CAUSAL | MAGI_MASK_INVCAUSAL);
    g.si = si;
    return true;
  }
  return false;
}

// Max of x over the lane pair (l, l ^ 32), and x from the partner lane.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_other(float x, int h) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(h ? r[0] : r[1]);
}

// LDS-only workgroup barrier: LDS stores before it are visible after it,
// while global loads issued earlier stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// V^T (or any row-major tile read as a transposed A operand) for one
// 16-row step: lanes get 8 consecutive rows of one column through the LDS
// transpose read (two 4-row reads).
__device__ __forceinline__ bf16x8 read_tr8(const __attribute__((address_space(3))) __bf16* p, int pitch) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 8 * pitch));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

}  // namespace dev
}  // namespace magi

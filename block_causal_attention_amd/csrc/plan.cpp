// Host half of libmagi_bca: the mask -> AttnSlice builder and the atomic-free
// slice scheduler.  Pure C++17, no HIP calls.
//
// The AttnSlice formulation (a mask as a union of (q range, k range, full or
// causal) rectangles) follows the Flex-Flash-Attention description on the
// MAGI-1 pages (study notes on zhao9797.github.io, "训练 Infra"; 量子位 article
// on dakule.com, "Flex-Flash-Attention").  The work estimate of a piece of the
// mask is its visible area, the measure MagiAttention's dispatch solver
// balances (interview with Zhang Zheng, answer on load balancing).
#include <algorithm>
#include <climits>
#include <cstdint>
#include <numeric>
#include <string>
#include <vector>

#include "status.h"

namespace magi {

std::string& last_error_slot() {
  thread_local std::string msg;
  return msg;
}

namespace {

constexpr int kRowsPerTile = 256;  // query rows (tokens x heads of a group) per work item

// Bit 0 of the mask type: the bottom-right (causal) bound; bit 1: the
// top-left (inverse causal) bound.
inline bool has_upper(const magi_attn_slice& s) { return (s.mask_type & MAGI_MASK_CAUSAL) != 0; }
inline bool has_lower(const magi_attn_slice& s) { return (s.mask_type & MAGI_MASK_INVCAUSAL) != 0; }

// Visible keys of row r (q_start <= r < q_end) under slice s:
// [row_begin, row_end).
inline int64_t row_end(const magi_attn_slice& s, int64_t r) {
  if (!has_upper(s)) return s.k_end;
  int64_t e = (int64_t)s.k_end - (int64_t)s.q_end + r + 1;
  return std::min<int64_t>(s.k_end, e);
}
inline int64_t row_begin(const magi_attn_slice& s, int64_t r) {
  if (!has_lower(s)) return s.k_start;
  return std::max<int64_t>(s.k_start, (int64_t)s.k_start + r - (int64_t)s.q_start);
}

inline int64_t row_count(const magi_attn_slice& s, int64_t r) {
  return std::max<int64_t>(0, row_end(s, r) - row_begin(s, r));
}

// First row of [r0, r1) (rows both slices cover) on which slices a and b
// show a common key, or -1.  Inside a slice's rows each bound is linear in
// the row (slope 1 on a diagonal, 0 otherwise), so the width of the shared
// key range, min(ends) - max(begins), is concave and piecewise linear: its
// maximum lies on an end row or where a diagonal bound crosses the other
// slice's flat one.
int64_t shared_row(const magi_attn_slice& a, const magi_attn_slice& b, int64_t r0, int64_t r1) {
  std::vector<int64_t> cand = {r0, r1 - 1};
  auto add = [&](int64_t r) {
    for (int64_t x = r - 1; x <= r + 1; ++x)
      if (x >= r0 && x < r1) cand.push_back(x);
  };
  if (has_upper(a) != has_upper(b)) {  // k_end - q_end + r + 1 of one meets k_end of the other
    const magi_attn_slice& d = has_upper(a) ? a : b;
    const magi_attn_slice& f = has_upper(a) ? b : a;
    add((int64_t)f.k_end - d.k_end + d.q_end - 1);
  }
  if (has_lower(a) != has_lower(b)) {  // k_start - q_start + r of one meets k_start of the other
    const magi_attn_slice& d = has_lower(a) ? a : b;
    const magi_attn_slice& f = has_lower(a) ? b : a;
    add((int64_t)f.k_start - d.k_start + d.q_start);
  }
  for (int64_t r : cand)
    if (std::max(row_begin(a, r), row_begin(b, r)) < std::min(row_end(a, r), row_end(b, r))) return r;
  return -1;
}

}  // namespace
}  // namespace magi

using namespace magi;

extern "C" const char* magi_version(void) { return "magi_bca 0.1.0 (gfx950)"; }

extern "C" const char* magi_last_error(void) { return last_error_slot().c_str(); }

extern "C" int32_t magi_slices_build(const magi_seq_desc* seqs, int32_t num_seqs,
                                     magi_attn_slice* slices, int32_t slice_cap,
                                     int32_t* num_slices) {
  if (num_slices == nullptr) return fail(MAGI_ERR_INVALID_ARG, "num_slices is NULL");
  if (num_seqs < 0) return fail(MAGI_ERR_INVALID_ARG, "num_seqs < 0");
  if (num_seqs > 0 && seqs == nullptr) return fail(MAGI_ERR_INVALID_ARG, "seqs is NULL");
  if (slice_cap < 0) return fail(MAGI_ERR_INVALID_ARG, "slice_cap < 0");
  if (slices == nullptr && slice_cap != 0) return fail(MAGI_ERR_INVALID_ARG, "slices is NULL but slice_cap > 0");

  struct Span { int64_t a, b; int idx; };
  std::vector<Span> qs, ks;
  int64_t need = 0;
  for (int i = 0; i < num_seqs; ++i) {
    const magi_seq_desc& s = seqs[i];
    if (s.chunk_len < 1) return fail(MAGI_ERR_INVALID_ARG, "seq %d: chunk_len %d < 1", i, s.chunk_len);
    if (s.num_kv_chunks < 1) return fail(MAGI_ERR_INVALID_ARG, "seq %d: num_kv_chunks < 1", i);
    if (s.num_q_chunks < 1 || s.num_q_chunks > s.num_kv_chunks)
      return fail(MAGI_ERR_INVALID_ARG, "seq %d: num_q_chunks %d not in [1, num_kv_chunks]", i, s.num_q_chunks);
    if (s.q_offset < 0 || s.k_offset < 0) return fail(MAGI_ERR_INVALID_ARG, "seq %d: negative offset", i);
    int64_t qe = (int64_t)s.q_offset + (int64_t)s.num_q_chunks * s.chunk_len;
    int64_t ke = (int64_t)s.k_offset + (int64_t)s.num_kv_chunks * s.chunk_len;
    if (qe > INT32_MAX || ke > INT32_MAX) return fail(MAGI_ERR_INVALID_ARG, "seq %d: ranges exceed int32", i);
    bool unlimited = true;
    if (s.kv_range) {
      for (int j = 0; j < s.num_q_chunks; ++j) {
        if (s.kv_range[j] < -1) return fail(MAGI_ERR_INVALID_ARG, "seq %d: kv_range[%d] = %d < -1", i, j, s.kv_range[j]);
        if (s.kv_range[j] >= 0) unlimited = false;
      }
    }
    need += (s.chunk_len == 1 && unlimited) ? 1 : s.num_q_chunks;
    qs.push_back({s.q_offset, qe, i});
    ks.push_back({s.k_offset, ke, i});
  }
  for (auto* v : {&qs, &ks}) {
    std::sort(v->begin(), v->end(), [](const Span& x, const Span& y) { return x.a < y.a; });
    for (size_t j = 1; j < v->size(); ++j)
      if ((*v)[j].a < (*v)[j - 1].b)
        return fail(MAGI_ERR_OVERLAP, "videos %d and %d overlap in the %s index space", (*v)[j - 1].idx,
                    (*v)[j].idx, v == &qs ? "query" : "key");
  }
  if (need > INT32_MAX) return fail(MAGI_ERR_INVALID_ARG, "too many slices");
  *num_slices = (int32_t)need;
  if (slices == nullptr && slice_cap == 0) return ok();
  if (slice_cap < need) return fail(MAGI_ERR_BUFFER_TOO_SMALL, "slice_cap %d < %lld", slice_cap, (long long)need);

  int32_t n = 0;
  for (int i = 0; i < num_seqs; ++i) {
    const magi_seq_desc& s = seqs[i];
    const int32_t C = s.chunk_len;
    const int32_t first = s.num_kv_chunks - s.num_q_chunks;
    bool unlimited = true;
    if (s.kv_range)
      for (int j = 0; j < s.num_q_chunks; ++j) unlimited &= (s.kv_range[j] < 0);
    if (C == 1 && unlimited) {
      // one-token chunks with no KV limit: plain causal attention, which the
      // bottom-right alignment also gives for a streaming query tail
      slices[n++] = {s.q_offset, s.q_offset + s.num_q_chunks, s.k_offset, s.k_offset + s.num_kv_chunks,
                     MAGI_MASK_CAUSAL};
      continue;
    }
    for (int j = 0; j < s.num_q_chunks; ++j) {
      const int32_t c = first + j;
      const int32_t r = s.kv_range ? s.kv_range[j] : -1;
      const int32_t lo = r < 0 ? 0 : std::max(0, c - r);
      slices[n++] = {s.q_offset + j * C, s.q_offset + (j + 1) * C, s.k_offset + lo * C, s.k_offset + (c + 1) * C,
                     MAGI_MASK_FULL};
    }
  }
  return ok();
}

extern "C" int32_t magi_default_tile_q(int32_t hq, int32_t hkv, int32_t head_dim, int32_t dtype) {
  if (hq <= 0 || hkv <= 0) return fail(MAGI_ERR_INVALID_ARG, "hq and hkv must be positive");
  if (hq % hkv) return fail(MAGI_ERR_INVALID_ARG, "hq %% hkv != 0 (hq=%d hkv=%d)", hq, hkv);
  if (dtype != MAGI_DTYPE_BF16 && dtype != MAGI_DTYPE_FP32) return fail(MAGI_ERR_INVALID_ARG, "bad dtype %d", dtype);
  if (head_dim != 24 && head_dim != 48)
    return fail(MAGI_ERR_UNSUPPORTED, "head_dim %d unsupported (24 or 48)", head_dim);
  const int G = hq / hkv;
  if (G > kRowsPerTile) return fail(MAGI_ERR_UNSUPPORTED, "group size %d > %d", G, kRowsPerTile);
  return kRowsPerTile / G;
}

extern "C" int32_t magi_schedule(const magi_attn_slice* slices, int32_t num_slices, int64_t nq, int64_t nk,
                                 int32_t hq, int32_t hkv, int32_t head_dim, int32_t dtype, int32_t tile_q,
                                 magi_work_item* work, int32_t work_cap, int32_t* num_work, int32_t* tile_slices,
                                 int32_t ts_cap, int32_t* num_tile_slices) {
  if (num_work == nullptr || num_tile_slices == nullptr)
    return fail(MAGI_ERR_INVALID_ARG, "num_work / num_tile_slices is NULL");
  if (num_slices < 0) return fail(MAGI_ERR_INVALID_ARG, "num_slices < 0");
  if (num_slices > 0 && slices == nullptr) return fail(MAGI_ERR_INVALID_ARG, "slices is NULL");
  if (nq < 0 || nk < 0 || nq > INT32_MAX || nk > INT32_MAX)
    return fail(MAGI_ERR_INVALID_ARG, "nq/nk must be in [0, 2^31)");
  if (work_cap < 0 || ts_cap < 0) return fail(MAGI_ERR_INVALID_ARG, "negative capacity");
  if ((work == nullptr) != (work_cap == 0) || (tile_slices == nullptr) != (ts_cap == 0))
    return fail(MAGI_ERR_INVALID_ARG, "output array and capacity disagree (NULL needs cap 0)");
  const int32_t dflt = magi_default_tile_q(hq, hkv, head_dim, dtype);
  if (dflt < 0) return dflt;
  if (tile_q < 0 || tile_q > dflt)
    return fail(MAGI_ERR_INVALID_ARG, "tile_q %d not in [0, %d] for this shape", tile_q, dflt);
  if (tile_q == 0) tile_q = dflt;

  // validate slices
  for (int i = 0; i < num_slices; ++i) {
    const magi_attn_slice& s = slices[i];
    if (s.mask_type < MAGI_MASK_FULL || s.mask_type > MAGI_MASK_BICAUSAL)
      return fail(MAGI_ERR_INVALID_ARG, "slice %d: unknown mask type %d", i, s.mask_type);
    if (s.q_start < 0 || s.q_start > s.q_end || s.q_end > nq || s.k_start < 0 || s.k_start > s.k_end ||
        s.k_end > nk)
      return fail(MAGI_ERR_INVALID_ARG, "slice %d: range q[%d,%d) k[%d,%d) outside [0,%lld)x[0,%lld)", i,
                  s.q_start, s.q_end, s.k_start, s.k_end, (long long)nq, (long long)nk);
    // the kernels form k_start + (r - q_start) in 32 bits
    if (has_lower(s) && (int64_t)s.k_start + (s.q_end - s.q_start) > INT32_MAX)
      return fail(MAGI_ERR_INVALID_ARG, "slice %d: k_start + (q_end - q_start) exceeds int32", i);
  }

  // cut the query axis at every slice boundary
  std::vector<int64_t> cuts = {0, nq};
  for (int i = 0; i < num_slices; ++i)
    if (slices[i].q_start < slices[i].q_end && slices[i].k_start < slices[i].k_end) {
      cuts.push_back(slices[i].q_start);
      cuts.push_back(slices[i].q_end);
    }
  std::sort(cuts.begin(), cuts.end());
  cuts.erase(std::unique(cuts.begin(), cuts.end()), cuts.end());
  const size_t nseg = cuts.size() - 1;
  std::vector<std::vector<int32_t>> cover(nseg);
  for (int i = 0; i < num_slices; ++i) {
    const magi_attn_slice& s = slices[i];
    if (s.q_start >= s.q_end || s.k_start >= s.k_end) continue;
    size_t a = std::lower_bound(cuts.begin(), cuts.end(), (int64_t)s.q_start) - cuts.begin();
    for (size_t g = a; g < nseg && cuts[g] < s.q_end; ++g) cover[g].push_back(i);
  }

  // overlap check.  Without a lower bound a slice's key range only grows
  // with the row, so two such slices that share a (q, k) pair anywhere in a
  // segment share one on its last row; a slice with a lower bound is checked
  // against every other slice of the segment (shared_row).
  for (size_t g = 0; g < nseg; ++g) {
    if (cover[g].size() < 2) continue;
    const int64_t r = cuts[g + 1] - 1;
    for (size_t x = 0; x < cover[g].size(); ++x) {
      const magi_attn_slice& a = slices[cover[g][x]];
      if (!has_lower(a)) continue;
      for (size_t y = 0; y < cover[g].size(); ++y) {
        const magi_attn_slice& b = slices[cover[g][y]];
        if (y == x || (has_lower(b) && y < x)) continue;
        const int64_t row = shared_row(a, b, cuts[g], cuts[g + 1]);
        if (row >= 0)
          return fail(MAGI_ERR_OVERLAP, "slices %d and %d overlap at query row %lld", cover[g][x], cover[g][y],
                      (long long)row);
      }
    }
    std::vector<std::pair<int64_t, int64_t>> iv;
    for (int32_t i : cover[g]) {
      if (has_lower(slices[i])) continue;
      int64_t e = row_end(slices[i], r);
      if (e > slices[i].k_start) iv.push_back({slices[i].k_start, e});
    }
    std::vector<size_t> ord(iv.size());
    std::iota(ord.begin(), ord.end(), 0);
    std::sort(ord.begin(), ord.end(), [&](size_t x, size_t y) { return iv[x] < iv[y]; });
    for (size_t j = 1; j < ord.size(); ++j)
      if (iv[ord[j]].first < iv[ord[j - 1]].second)
        return fail(MAGI_ERR_OVERLAP, "slices overlap at query row %lld (key ranges [%lld,%lld) and [%lld,%lld))",
                    (long long)r, (long long)iv[ord[j - 1]].first, (long long)iv[ord[j - 1]].second,
                    (long long)iv[ord[j]].first, (long long)iv[ord[j]].second);
  }
  for (auto& c : cover)
    std::sort(c.begin(), c.end(), [&](int32_t x, int32_t y) {
      return slices[x].k_start != slices[y].k_start ? slices[x].k_start < slices[y].k_start : x < y;
    });

  // tiles
  struct Tile { int64_t q0, len, cost; size_t seg; };
  std::vector<Tile> tiles;
  int64_t ts_total = 0;
  for (size_t g = 0; g < nseg; ++g) {
    for (int64_t t0 = cuts[g]; t0 < cuts[g + 1]; t0 += tile_q) {
      const int64_t len = std::min<int64_t>(tile_q, cuts[g + 1] - t0);
      int64_t cost = 0;
      for (int32_t i : cover[g])
        for (int64_t r = t0; r < t0 + len; ++r) cost += row_count(slices[i], r);
      tiles.push_back({t0, len, cost, g});
      ts_total += (int64_t)cover[g].size();
    }
  }
  const int64_t nwork = (int64_t)tiles.size() * hkv;
  if (nwork > INT32_MAX || ts_total > INT32_MAX) return fail(MAGI_ERR_INVALID_ARG, "work list exceeds int32");
  *num_work = (int32_t)nwork;
  *num_tile_slices = (int32_t)ts_total;
  if (work == nullptr && tile_slices == nullptr) return ok();
  if (work_cap < nwork || ts_cap < ts_total)
    return fail(MAGI_ERR_BUFFER_TOO_SMALL, "need work_cap >= %lld and ts_cap >= %lld", (long long)nwork,
                (long long)ts_total);

  // heaviest tiles first; ties keep query order (deterministic)
  std::vector<size_t> ord(tiles.size());
  std::iota(ord.begin(), ord.end(), 0);
  std::stable_sort(ord.begin(), ord.end(), [&](size_t x, size_t y) { return tiles[x].cost > tiles[y].cost; });
  int32_t ts = 0, w = 0;
  for (size_t rank = 0; rank < ord.size(); ++rank) {
    const Tile& t = tiles[ord[rank]];
    const int32_t sb = ts;
    for (int32_t i : cover[t.seg]) tile_slices[ts++] = i;
    for (int32_t g = 0; g < hkv; ++g)
      work[w++] = {(int32_t)t.q0, (int32_t)t.len, sb, ts, g, (int32_t)std::min<int64_t>(t.cost, INT32_MAX)};
  }
  return ok();
}

namespace magi {
namespace {
constexpr int kKeysPerTile = 128;  // keys of one KV group per backward work item
constexpr int kRowsPerQTile = 64;  // query rows (tokens x heads) per Q/dO tile of the dK/dV pass

// Rows of slice s that see key k (k_start <= k < k_end): [col_first, col_end).
inline int64_t col_first(const magi_attn_slice& s, int64_t k) {
  if (!has_upper(s)) return s.q_start;
  // bottom-right aligned: row r sees k iff k < k_end - q_end + r + 1
  return std::max<int64_t>(s.q_start, k - ((int64_t)s.k_end - (int64_t)s.q_end));
}
inline int64_t col_end(const magi_attn_slice& s, int64_t k) {
  if (!has_lower(s)) return s.q_end;
  // top-left aligned: row r sees k iff k >= k_start + r - q_start
  return std::min<int64_t>(s.q_end, k - (int64_t)s.k_start + (int64_t)s.q_start + 1);
}
inline int64_t col_count(const magi_attn_slice& s, int64_t k) {
  return std::max<int64_t>(0, col_end(s, k) - col_first(s, k));
}
// Whether some row of s sees a key of [k0, k1) (inside s's key range).  The
// row count is concave and piecewise linear in the key, with breaks where a
// diagonal bound reaches the first or last row.
inline bool any_col(const magi_attn_slice& s, int64_t k0, int64_t k1) {
  std::vector<int64_t> cand = {k0, k1 - 1};
  auto add = [&](int64_t k) {
    for (int64_t x = k - 1; x <= k + 1; ++x)
      if (x >= k0 && x < k1) cand.push_back(x);
  };
  if (has_upper(s)) add((int64_t)s.q_start + s.k_end - s.q_end);
  if (has_lower(s)) add((int64_t)s.q_end + s.k_start - s.q_start - 1);
  for (int64_t k : cand)
    if (col_count(s, k) > 0) return true;
  return false;
}
}  // namespace
}  // namespace magi

extern "C" int32_t magi_default_tile_k(int32_t hq, int32_t hkv, int32_t head_dim, int32_t dtype) {
  const int32_t st = magi_default_tile_q(hq, hkv, head_dim, dtype);
  return st < 0 ? st : kKeysPerTile;
}

extern "C" int32_t magi_schedule_kv(const magi_attn_slice* slices, int32_t num_slices, int64_t nq, int64_t nk,
                                    int32_t hq, int32_t hkv, int32_t head_dim, int32_t dtype, int32_t tile_k,
                                    magi_work_item* work, int32_t work_cap, int32_t* num_work,
                                    int32_t* tile_slices, int32_t ts_cap, int32_t* num_tile_slices,
                                    int32_t* item_ext, magi_kv_reduce* reduce, int32_t reduce_cap,
                                    int32_t* num_reduce, int32_t* num_slots) {
  if (num_work == nullptr || num_tile_slices == nullptr || num_reduce == nullptr || num_slots == nullptr)
    return fail(MAGI_ERR_INVALID_ARG, "a count pointer is NULL");
  if (work_cap < 0 || ts_cap < 0 || reduce_cap < 0) return fail(MAGI_ERR_INVALID_ARG, "negative capacity");
  if ((work == nullptr) != (work_cap == 0) || (tile_slices == nullptr) != (ts_cap == 0) ||
      (item_ext == nullptr) != (work_cap == 0) || (reduce == nullptr) != (reduce_cap == 0))
    return fail(MAGI_ERR_INVALID_ARG, "output array and capacity disagree (NULL needs cap 0)");
  // the query-major size query validates the slices (ranges, types, overlap)
  int32_t nw_q = 0, nts_q = 0;
  const int32_t st = magi_schedule(slices, num_slices, nq, nk, hq, hkv, head_dim, dtype, 0, nullptr, 0, &nw_q,
                                   nullptr, 0, &nts_q);
  if (st < 0) return st;
  const int32_t dflt = magi_default_tile_k(hq, hkv, head_dim, dtype);
  if (dflt < 0) return dflt;
  if (tile_k < 0 || tile_k > dflt)
    return fail(MAGI_ERR_INVALID_ARG, "tile_k %d not in [0, %d] for this shape", tile_k, dflt);
  if (tile_k == 0) tile_k = dflt;

  // cut the key axis at every slice boundary
  std::vector<int64_t> cuts = {0, nk};
  for (int i = 0; i < num_slices; ++i)
    if (slices[i].q_start < slices[i].q_end && slices[i].k_start < slices[i].k_end) {
      cuts.push_back(slices[i].k_start);
      cuts.push_back(slices[i].k_end);
    }
  std::sort(cuts.begin(), cuts.end());
  cuts.erase(std::unique(cuts.begin(), cuts.end()), cuts.end());
  const size_t nseg = cuts.size() - 1;
  // slices that show some row a key of the segment, in query order
  std::vector<std::vector<int32_t>> cover(nseg);
  for (int i = 0; i < num_slices; ++i) {
    const magi_attn_slice& s = slices[i];
    if (s.q_start >= s.q_end || s.k_start >= s.k_end) continue;
    size_t a = std::lower_bound(cuts.begin(), cuts.end(), (int64_t)s.k_start) - cuts.begin();
    for (size_t g = a; g < nseg && cuts[g] < s.k_end; ++g)
      if (any_col(s, cuts[g], cuts[g + 1])) cover[g].push_back(i);
  }
  for (auto& c : cover)
    std::sort(c.begin(), c.end(), [&](int32_t x, int32_t y) {
      return slices[x].q_start != slices[y].q_start ? slices[x].q_start < slices[y].q_start : x < y;
    });

  // tiles, with the visible pairs each listed slice contributes
  struct Tile { int64_t k0, len; size_t seg; std::vector<int64_t> pairs; };
  std::vector<Tile> tiles;
  int64_t ts_total = 0, total = 0, largest = 0;
  for (size_t g = 0; g < nseg; ++g) {
    for (int64_t t0 = cuts[g]; t0 < cuts[g + 1]; t0 += tile_k) {
      Tile t{t0, std::min<int64_t>(tile_k, cuts[g + 1] - t0), g, {}};
      for (int32_t i : cover[g]) {
        int64_t c = 0;
        for (int64_t k = t0; k < t0 + t.len; ++k) c += col_count(slices[i], k);
        t.pairs.push_back(c);
        total += c;
        largest = std::max(largest, c);
      }
      ts_total += (int64_t)cover[g].size();
      tiles.push_back(std::move(t));
    }
  }
  // Parts of at most T pairs: runs of consecutive listed slices, or one
  // slice's rows cut into token windows of about equal pairs.  T aims at
  // about 8192 items for the whole list (several workgroups per SIMD over the
  // whole pass), never below 128 x 128 pairs.
  constexpr int64_t kTargetItems = 8192;
  constexpr int64_t kMinPart = 128 * 128;
  const int64_t T = std::max<int64_t>(kMinPart, (total * hkv + kTargetItems - 1) / kTargetItems);
  (void)largest;
  struct Unit { size_t tile; int32_t a, b; int64_t cost; int32_t part, nparts; int32_t lo, hi; };
  std::vector<Unit> units;
  int64_t nslots = 0, nred = 0;
  const int32_t nq32 = (int32_t)nq;
  for (size_t ti = 0; ti < tiles.size(); ++ti) {
    const Tile& t = tiles[ti];
    const std::vector<int32_t>& cv = cover[t.seg];
    const size_t first = units.size();
    int32_t a = 0;
    int64_t acc = 0;
    auto close_run = [&](int32_t b) {
      if (b > a) units.push_back({ti, a, b, acc, 0, 0, 0, nq32});
      a = b;
      acc = 0;
    };
    for (int32_t j = 0; j < (int32_t)t.pairs.size(); ++j) {
      const int64_t c = t.pairs[j];
      if (c > T) {
        // this slice alone, its rows cut into windows of about c / nw pairs
        close_run(j);
        const magi_attn_slice& sl = slices[cv[j]];
        const int64_t nw = (c + T - 1) / T;
        int64_t run = 0, cut = 1;
        const size_t wfirst = units.size();
        const int32_t k_hi = (int32_t)std::min<int64_t>(t.k0 + t.len, sl.k_end);
        const int32_t k_lo = (int32_t)std::max<int64_t>(t.k0, sl.k_start);
        // rows that see a key of the tile, and the keys of the tile row r sees
        int32_t lo = (int32_t)col_first(sl, k_lo);
        const int32_t r_end = (int32_t)col_end(sl, k_hi - 1);
        auto tile_keys = [&](int64_t r) {
          return std::max<int64_t>(0, std::min<int64_t>(k_hi, row_end(sl, r)) -
                                          std::max<int64_t>(k_lo, row_begin(sl, r)));
        };
        // the dK/dV pass walks a window in row tiles of `step` tokens from
        // its first row: windows of whole tiles leave a partial (masked)
        // tile only at the end of the slice's rows
        const int32_t step = std::max<int32_t>(1, kRowsPerQTile / (hq / hkv));
        for (int32_t r = lo; r < r_end; ++r) {
          run += tile_keys(r);
          if (cut < nw && run * nw >= c * cut && (r + 1 - lo) % step == 0) {
            units.push_back({ti, j, j + 1, 0, 0, 0, lo, r + 1});
            lo = r + 1;
            ++cut;
          }
        }
        if (lo < r_end) units.push_back({ti, j, j + 1, 0, 0, 0, lo, r_end});
        // pairs of each window
        for (size_t u = wfirst; u < units.size(); ++u) {
          int64_t pc = 0;
          for (int32_t r = units[u].lo; r < units[u].hi; ++r) pc += tile_keys(r);
          units[u].cost = pc;
        }
        a = j + 1;
        continue;
      }
      if (j > a && acc + c > T) close_run(j);
      acc += c;
    }
    close_run((int32_t)t.pairs.size());
    if (units.size() == first) units.push_back({ti, 0, 0, 0, 0, 0, 0, nq32});  // a tile no row sees
    const int32_t np = (int32_t)(units.size() - first);
    for (int32_t p = 0; p < np; ++p) {
      units[first + p].part = p;
      units[first + p].nparts = np;
    }
    if (np > 1) {
      nslots += (int64_t)np * hkv;
      nred += hkv;
    }
  }
  const int64_t nwork = (int64_t)units.size() * hkv;
  if (nwork > INT32_MAX || ts_total > INT32_MAX || nslots > INT32_MAX)
    return fail(MAGI_ERR_INVALID_ARG, "work list exceeds int32");
  *num_work = (int32_t)nwork;
  *num_tile_slices = (int32_t)ts_total;
  *num_reduce = (int32_t)nred;
  *num_slots = (int32_t)nslots;
  if (work == nullptr && tile_slices == nullptr && reduce == nullptr) return ok();
  if (work_cap < nwork || ts_cap < ts_total || reduce_cap < nred)
    return fail(MAGI_ERR_BUFFER_TOO_SMALL, "need work_cap >= %lld, ts_cap >= %lld and reduce_cap >= %lld",
                (long long)nwork, (long long)ts_total, (long long)nred);

  // tile lists in key order; slots of a split tile: group-major, parts in order
  std::vector<int32_t> tile_sb(tiles.size()), slot0(tiles.size(), -1);
  int32_t ts = 0, slot = 0, r = 0;
  for (size_t ti = 0; ti < tiles.size(); ++ti) {
    tile_sb[ti] = ts;
    for (int32_t i : cover[tiles[ti].seg]) tile_slices[ts++] = i;
  }
  for (const Unit& u : units) {
    if (u.nparts < 2 || u.part != 0) continue;
    const Tile& t = tiles[u.tile];
    slot0[u.tile] = slot;
    for (int32_t g = 0; g < hkv; ++g)
      reduce[r++] = {(int32_t)t.k0, (int32_t)t.len, g, slot + g * u.nparts, u.nparts};
    slot += u.nparts * hkv;
  }
  // heaviest units first.  Ties (most parts of split tiles cost the same)
  // go window by window, key tiles in key order within a window: the units
  // that run side by side then walk the same query rows, so each Q/dO tile
  // is fetched once into the L2 of an XCD (a KV group's items share one XCD)
  // and served from there to the other units.  Deterministic.
  std::vector<size_t> ord(units.size());
  std::iota(ord.begin(), ord.end(), 0);
  std::stable_sort(ord.begin(), ord.end(), [&](size_t x, size_t y) {
    const Unit& ux = units[x];
    const Unit& uy = units[y];
    if (ux.cost != uy.cost) return ux.cost > uy.cost;
    if (ux.lo != uy.lo) return ux.lo < uy.lo;
    return ux.tile < uy.tile;
  });
  int32_t w = 0;
  for (size_t rank = 0; rank < ord.size(); ++rank) {
    const Unit& u = units[ord[rank]];
    const Tile& t = tiles[u.tile];
    for (int32_t g = 0; g < hkv; ++g) {
      item_ext[3 * w] = u.nparts > 1 ? slot0[u.tile] + g * u.nparts + u.part : -1;
      item_ext[3 * w + 1] = u.lo;
      item_ext[3 * w + 2] = u.hi;
      work[w++] = {(int32_t)t.k0, (int32_t)t.len, tile_sb[u.tile] + u.a, tile_sb[u.tile] + u.b, g,
                   (int32_t)std::min<int64_t>(u.cost, INT32_MAX)};
    }
  }
  return ok();
}

extern "C" int32_t magi_slices_cross(const magi_cross_desc* descs, int32_t num_descs, magi_attn_slice* slices,
                                     int32_t slice_cap, int32_t* num_slices) {
  if (num_slices == nullptr) return fail(MAGI_ERR_INVALID_ARG, "num_slices is NULL");
  if (num_descs < 0) return fail(MAGI_ERR_INVALID_ARG, "num_descs < 0");
  if (num_descs > 0 && descs == nullptr) return fail(MAGI_ERR_INVALID_ARG, "descs is NULL");
  if (slice_cap < 0) return fail(MAGI_ERR_INVALID_ARG, "slice_cap < 0");
  if (slices == nullptr && slice_cap != 0) return fail(MAGI_ERR_INVALID_ARG, "slices is NULL but slice_cap > 0");
  struct Span { int64_t a, b; int idx; };
  std::vector<Span> qs;
  int32_t need = 0;
  for (int i = 0; i < num_descs; ++i) {
    const magi_cross_desc& d = descs[i];
    if (d.q_offset < 0 || d.k_offset < 0 || d.q_len < 0 || d.k_len < 0)
      return fail(MAGI_ERR_INVALID_ARG, "sample %d: negative offset or length", i);
    if ((int64_t)d.q_offset + d.q_len > INT32_MAX || (int64_t)d.k_offset + d.k_len > INT32_MAX)
      return fail(MAGI_ERR_INVALID_ARG, "sample %d: ranges exceed int32", i);
    if (d.q_len == 0 || d.k_len == 0) continue;
    qs.push_back({d.q_offset, (int64_t)d.q_offset + d.q_len, i});
    ++need;
  }
  std::sort(qs.begin(), qs.end(), [](const Span& x, const Span& y) { return x.a < y.a; });
  for (size_t j = 1; j < qs.size(); ++j)
    if (qs[j].a < qs[j - 1].b)
      return fail(MAGI_ERR_OVERLAP, "samples %d and %d overlap in the query index space", qs[j - 1].idx, qs[j].idx);
  *num_slices = need;
  if (slices == nullptr && slice_cap == 0) return ok();
  if (slice_cap < need) return fail(MAGI_ERR_BUFFER_TOO_SMALL, "slice_cap %d < %d", slice_cap, need);
  int32_t n = 0;
  for (int i = 0; i < num_descs; ++i) {
    const magi_cross_desc& d = descs[i];
    if (d.q_len == 0 || d.k_len == 0) continue;
    slices[n++] = {d.q_offset, d.q_offset + d.q_len, d.k_offset, d.k_offset + d.k_len, MAGI_MASK_FULL};
  }
  return ok();
}

extern "C" int32_t magi_slices_ring(const magi_ring_desc* d, magi_attn_slice* slices, int32_t slice_cap,
                                    int32_t* num_slices) {
  if (num_slices == nullptr || d == nullptr) return fail(MAGI_ERR_INVALID_ARG, "desc / num_slices is NULL");
  if (slice_cap < 0) return fail(MAGI_ERR_INVALID_ARG, "slice_cap < 0");
  if (slices == nullptr && slice_cap != 0) return fail(MAGI_ERR_INVALID_ARG, "slices is NULL but slice_cap > 0");
  const int64_t C = d->chunk_len, S = d->ring_slots;
  if (C < 1 || S < 1) return fail(MAGI_ERR_INVALID_ARG, "chunk_len and ring_slots must be >= 1");
  if (d->first_chunk < 0) return fail(MAGI_ERR_INVALID_ARG, "first_chunk < 0");
  if (d->num_chunks < 1 || d->num_chunks > S)
    return fail(MAGI_ERR_INVALID_ARG, "num_chunks %d not in [1, ring_slots]", d->num_chunks);
  if (d->num_inflight < 1 || d->num_inflight > d->num_chunks)
    return fail(MAGI_ERR_INVALID_ARG, "num_inflight %d not in [1, num_chunks]", d->num_inflight);
  if (d->q_offset < 0 || d->k_offset < 0) return fail(MAGI_ERR_INVALID_ARG, "negative offset");
  if (d->q_offset + (int64_t)d->num_inflight * C > INT32_MAX || d->k_offset + S * C > INT32_MAX ||
      (int64_t)d->first_chunk + d->num_chunks > INT32_MAX)
    return fail(MAGI_ERR_INVALID_ARG, "ranges exceed int32");
  if (d->kv_range)
    for (int j = 0; j < d->num_inflight; ++j)
      if (d->kv_range[j] < -1) return fail(MAGI_ERR_INVALID_ARG, "kv_range[%d] = %d < -1", j, d->kv_range[j]);
  // chunk c lives in ring slot c mod S; in-flight chunk j is global chunk
  // first_chunk + num_chunks - num_inflight + j and sees the chunks from
  // max(first_chunk, c - r) to c, a run of slots that wraps at most once
  struct Piece { int32_t q0, q1, k0, k1; };
  std::vector<Piece> out;
  const int64_t c_first = (int64_t)d->first_chunk + d->num_chunks - d->num_inflight;
  for (int j = 0; j < d->num_inflight; ++j) {
    const int64_t c = c_first + j;
    const int32_t r = d->kv_range ? d->kv_range[j] : -1;
    const int64_t lo = r < 0 ? d->first_chunk : std::max<int64_t>(d->first_chunk, c - r);
    const int32_t q0 = (int32_t)(d->q_offset + j * C), q1 = (int32_t)(q0 + C);
    const int64_t s_lo = lo % S, s_hi = c % S;
    if (s_lo <= s_hi) {
      out.push_back({q0, q1, (int32_t)(d->k_offset + s_lo * C), (int32_t)(d->k_offset + (s_hi + 1) * C)});
    } else {
      out.push_back({q0, q1, (int32_t)(d->k_offset + s_lo * C), (int32_t)(d->k_offset + S * C)});
      out.push_back({q0, q1, (int32_t)d->k_offset, (int32_t)(d->k_offset + (s_hi + 1) * C)});
    }
  }
  *num_slices = (int32_t)out.size();
  if (slices == nullptr && slice_cap == 0) return ok();
  if (slice_cap < (int32_t)out.size())
    return fail(MAGI_ERR_BUFFER_TOO_SMALL, "slice_cap %d < %d", slice_cap, (int32_t)out.size());
  for (size_t i = 0; i < out.size(); ++i) slices[i] = {out[i].q0, out[i].q1, out[i].k0, out[i].k1, MAGI_MASK_FULL};
  return ok();
}

extern "C" int32_t magi_slices_window(const magi_window_desc* descs, int32_t num_descs, magi_attn_slice* slices,
                                      int32_t slice_cap, int32_t* num_slices) {
  if (num_slices == nullptr) return fail(MAGI_ERR_INVALID_ARG, "num_slices is NULL");
  if (num_descs < 0) return fail(MAGI_ERR_INVALID_ARG, "num_descs < 0");
  if (num_descs > 0 && descs == nullptr) return fail(MAGI_ERR_INVALID_ARG, "descs is NULL");
  if (slice_cap < 0) return fail(MAGI_ERR_INVALID_ARG, "slice_cap < 0");
  if (slices == nullptr && slice_cap != 0) return fail(MAGI_ERR_INVALID_ARG, "slices is NULL but slice_cap > 0");
  struct Span { int64_t a, b; int idx; };
  std::vector<Span> qs, ks;
  int64_t need = 0;
  for (int i = 0; i < num_descs; ++i) {
    const magi_window_desc& d = descs[i];
    if (d.len < 0 || d.q_offset < 0 || d.k_offset < 0)
      return fail(MAGI_ERR_INVALID_ARG, "sequence %d: negative length or offset", i);
    if (d.window < 1) return fail(MAGI_ERR_INVALID_ARG, "sequence %d: window %d < 1", i, d.window);
    if ((int64_t)d.q_offset + d.len > INT32_MAX || (int64_t)d.k_offset + d.len > INT32_MAX)
      return fail(MAGI_ERR_INVALID_ARG, "sequence %d: ranges exceed int32", i);
    if (d.len == 0) continue;
    qs.push_back({d.q_offset, (int64_t)d.q_offset + d.len, i});
    ks.push_back({d.k_offset, (int64_t)d.k_offset + d.len, i});
    need += d.window >= d.len ? 1 : (d.window > 1 ? 2 : 1);
  }
  for (auto* v : {&qs, &ks}) {
    std::sort(v->begin(), v->end(), [](const Span& x, const Span& y) { return x.a < y.a; });
    for (size_t j = 1; j < v->size(); ++j)
      if ((*v)[j].a < (*v)[j - 1].b)
        return fail(MAGI_ERR_OVERLAP, "sequences %d and %d overlap in the %s index space", (*v)[j - 1].idx,
                    (*v)[j].idx, v == &qs ? "query" : "key");
  }
  if (need > INT32_MAX) return fail(MAGI_ERR_INVALID_ARG, "too many slices");
  *num_slices = (int32_t)need;
  if (slices == nullptr && slice_cap == 0) return ok();
  if (slice_cap < need) return fail(MAGI_ERR_BUFFER_TOO_SMALL, "slice_cap %d < %lld", slice_cap, (long long)need);
  int32_t n = 0;
  for (int i = 0; i < num_descs; ++i) {
    const magi_window_desc& d = descs[i];
    if (d.len == 0) continue;
    const int32_t q0 = d.q_offset, k0 = d.k_offset, L = d.len, w = d.window;
    if (w >= L) {
      // the window reaches back to the sequence start for every row
      slices[n++] = {q0, q0 + L, k0, k0 + L, MAGI_MASK_CAUSAL};
      continue;
    }
    // rows 0 .. w-2 see the sequence start: a causal square; the rest see a
    // band of w keys ending at themselves
    if (w > 1) slices[n++] = {q0, q0 + w - 1, k0, k0 + w - 1, MAGI_MASK_CAUSAL};
    slices[n++] = {q0 + w - 1, q0 + L, k0, k0 + L, MAGI_MASK_BICAUSAL};
  }
  return ok();
}

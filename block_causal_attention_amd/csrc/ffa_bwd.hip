// Flex-Flash-Attention backward for gfx950 (MI355X): dQ, dK, dV of the
// forward in ffa_fwd.hip over the same AttnSlices.
//
// The pages use the FFA kernels for training as well (study notes on
// zhao9797.github.io, "训练 Infra"; interview with Zhang Zheng, answer on
// MagiAttention); they give no backward formula, so this is the chain rule
// of softmax attention:
//   P = exp(scale q.k - LSE)           (LSE from the forward)
//   dV_g += P^T dO      dP = dO V_g^T      delta = rowsum(dO * O)
//   dS = P * (dP - delta)
//   dQ = scale dS K_g   dK_g += scale dS^T Q
// with g the KV group of the query head.  No atomics: two passes, each work
// item owning its outputs (the page's FFA uses atomics on Hopper).
//   * dQ pass: the forward's query-major work items (q tile x KV group) walk
//     their K/V tiles and accumulate dQ^T in registers.
//   * dK/dV pass: key-major items (128 keys x KV group, magi_schedule_kv)
//     walk the query rows that see their keys, 64 rows (tokens x heads of
//     the group) at a time, and accumulate dK^T and dV^T in registers; the
//     GQA sum over the group's heads falls out because the heads are rows.
//   * delta = rowsum(dO * O) comes first, from its own small kernel.
//
// MFMA layout (v_mfma_f32_32x32x16_bf16, as in the forward): the dQ pass
// keeps the forward's orientation (keys on M, rows on N, so each lane holds
// 16 keys of one row); the dK/dV pass turns it around (rows on M, keys on N,
// each lane 16 rows of one key).  In both, the elementwise P and dS leave the
// score accumulator already in the B-operand layout of the next product.
// LSE and delta vary per row; they enter the score and dP products as two
// augmented contraction columns: Q' carries -LSE2/c split into a bf16 high
// and low part (exact to about 2^-16) against two ones columns of K, and dO'
// carries -delta likewise against two ones columns of V, so the MFMA returns
// q.k - LSE2/c and dO.v - delta directly.  That needs head_dim + 2 padded to
// a multiple of 16: 24 -> 32 (free), 48 -> 64.
#include <hip/hip_runtime.h>

#include "ffa_common.h"
#include "kernels.h"

namespace magi {
namespace {

using namespace dev;

constexpr int kRows = 256;      // query rows per dQ work item (the forward's items)
constexpr int kKeys = 128;      // keys per dK/dV work item (4 waves x 32)
constexpr int NT = 512;         // threads per workgroup of the bf16 dQ pass
// 32-key blocks per wave of the bf16 dK/dV pass (head_dim 24 / 48).  Two blocks per
// wave at head_dim 24 need 256 VGPRs (2 waves per SIMD) and measured no faster.
constexpr int KB24 = 1, KB48 = 1;
constexpr int TK = 64;          // keys per K/V tile (dQ pass)
constexpr int TQ = 64;          // query rows per Q/dO tile (dK/dV pass)
constexpr int kThreads32 = 256;  // fp32 kernels

template <int D>
struct BCfg {
  static constexpr int DA = (D + 2 + 15) / 16 * 16;  // contraction incl. the two augmented columns
  static constexpr int KS = DA / 16;                 // MFMA k-steps over it
  static constexpr int DM = (D + 31) / 32 * 32;      // rows of the head_dim-major accumulators
  static constexpr int MB = DM / 32;
  // LDS row pitch (elements): 144 bytes puts the 16 rows of a b128 row read
  // in disjoint banks; the transposed reads then see at most 2-way conflicts
  static constexpr int PITCH = 72;
  static constexpr int CH = D / 8;  // 16-byte chunks per row
  static_assert(DA <= PITCH && D % 8 == 0, "layout");
};

// bf16 high and low parts of x (x = hi + lo to about 2^-16 relative)
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = (__bf16)x;
  lo = (__bf16)(x - (float)hi);
}

// ----------------------------------------------------------------- delta

// delta[row][head] = sum_d dO * O, fp32 (one thread per (token, head) vector)
template <int D, typename T>
__global__ __launch_bounds__(256) void bwd_delta(BwdArgs a) {
  const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (v >= a.nq * a.hq) return;
  const int64_t t = v / a.hq;
  const int hh = (int)(v % a.hq);
  const T* o = reinterpret_cast<const T*>(a.out) + t * a.o_stride + (int64_t)hh * D;
  const T* d = reinterpret_cast<const T*>(a.dout) + t * a.o_stride + (int64_t)hh * D;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < D; ++i) s = fmaf((float)o[i], (float)d[i], s);
  a.delta[t * a.hq + hh] = s;
}

// ----------------------------------------------------------------- dQ pass

template <int D, bool PRESCALED>
__global__ __launch_bounds__(NT, 2) void bwd_dq_bf16(BwdArgs a) {
  using C = BCfg<D>;
  constexpr int NCH = (TK * C::CH + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) __bf16 Ks[2][TK * C::PITCH];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[2][TK * C::PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, ln = lane & 31, li = lane & 15;
  const int dgrp = ((lane >> 4) & 1) * 16;
  const magi_work_item wi = load_item(a.qwork, blockIdx.x);
  const int G = a.hq / a.hkv;
  const int cap = kRows / G;
  if (wi.q_start < 0 || wi.q_len <= 0 || (int64_t)wi.q_start + wi.q_len > a.nq || wi.kv_group < 0 ||
      wi.kv_group >= a.hkv)
    return;
  const int qlen = wi.q_len < cap ? wi.q_len : cap;
  const int g = wi.kv_group;
  const float c = a.scale * kLog2e;
  const __bf16* __restrict__ kp = reinterpret_cast<const __bf16*>(a.k);
  const __bf16* __restrict__ vp = reinterpret_cast<const __bf16*>(a.v);

  // padding columns of every K and V buffer: D and D+1 are 1 (they meet the
  // augmented slots), the rest 0; tile stores never touch them
  for (int b = 0; b < 2; ++b)
    for (int i = tid; i < TK * (C::DA - D); i += NT) {
      const int col = D + i % (C::DA - D), row = i / (C::DA - D);
      const __bf16 x = (__bf16)(col < D + 2 ? 1.0f : 0.0f);
      Ks[b][row * C::PITCH + col] = x;
      Vs[b][row * C::PITCH + col] = x;
    }

  // this lane's query row (one 32-row MFMA column block per wave)
  const int n = wave * 32 + ln;
  const int t = n / G, hg = n % G, head = g * G + hg;
  const bool rvalid = t < qlen;
  const int32_t qi = wi.q_start + (rvalid ? t : 0);
  float lse2 = a.lse[(int64_t)qi * a.hq + head] * kLog2e;
  if (!(lse2 > -INFINITY && lse2 < INFINITY)) lse2 = 0.f;  // a row that sees no key
  const float dl = a.delta[(int64_t)qi * a.hq + head];
  __bf16 qa0, qa1, da0, da1;
  split_bf16(-lse2 / c, qa0, qa1);
  split_bf16(-dl, da0, da1);
  bf16x8 qreg[C::KS], dreg[C::KS];
  {
    const __bf16* qrow = reinterpret_cast<const __bf16*>(a.q) + (int64_t)qi * a.q_stride + (int64_t)head * D;
    const __bf16* drow = reinterpret_cast<const __bf16*>(a.dout) + (int64_t)qi * a.o_stride + (int64_t)head * D;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const int d0 = 16 * ks + 8 * h;
      bf16x8 x = {}, y = {};
      if (d0 < D) {
        x = *reinterpret_cast<const bf16x8*>(qrow + d0);
        y = *reinterpret_cast<const bf16x8*>(drow + d0);
      } else if (d0 == D) {
        x[0] = qa0;
        x[1] = qa1;
        y[0] = da0;
        y[1] = da1;
      }
      if (!rvalid) x = y = (bf16x8){};
      qreg[ks] = x;
      dreg[ks] = y;
    }
  }

  // K/V tiles: as in the forward, buffer loads whose range ends at the last
  // visible key (rows past it read as zeros)
  u32x4 kr[NCH], vr[NCH];
  int ch_off[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int ci = tid + j * NT;
    ch_off[j] = (ci / C::CH) * (int)a.kv_stride * 2 + (ci % C::CH) * 16;
  }
  const int32_t kv_row_bytes = (int32_t)a.kv_stride * 2;
  auto load_tile = [&](int32_t kt, int32_t khi) {
    const int64_t elem0 = (int64_t)kt * a.kv_stride + (int64_t)g * a.kv_hstride;
    const int32_t rows = khi - kt < TK ? khi - kt : TK;
    const int nrec = (rows - 1) * kv_row_bytes + D * 2;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kp + elem0), (short)0, nrec, kBufCfg);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vp + elem0), (short)0, nrec, kBufCfg);
#pragma unroll
    for (int j = 0; j < NCH; ++j)
      if (tid + j * NT < TK * C::CH) {
        kr[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, ch_off[j], 0, 0));
        vr[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, ch_off[j], 0, 0));
      }
  };
  auto store_tile = [&](int b) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int ci = tid + j * NT;
      if (ci < TK * C::CH) {
        const int r = ci / C::CH, part = ci % C::CH;
        *reinterpret_cast<u32x4*>(&Ks[b][r * C::PITCH + part * 8]) = kr[j];
        *reinterpret_cast<u32x4*>(&Vs[b][r * C::PITCH + part * 8]) = vr[j];
      }
    }
  };

  const int32_t first_tok = wi.q_start, last_tok = wi.q_start + qlen - 1;
  const SliceLists lists{a.slices, a.num_slices, a.q_tile_slices, a.num_q_tile_slices};
  constexpr auto key_of0 = [](int i) { return 8 * (i / 4) + (i % 4); };

  f32x16 dq[C::MB];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) dq[mb] = (f32x16){};

  SliceGeo cg;
  bool have = find_slice(lists, wi.slice_end, (int32_t)a.nk, wi.slice_begin, first_tok, last_tok, cg);
  int32_t kt = cg.ks;
  if (have) {
    load_tile(kt, cg.khi);
    store_tile(0);
  }
  // drain once: the lane-masked loads and stores above would otherwise make
  // the wait-count bookkeeping serialise every tile on its own prefetch
  __builtin_amdgcn_s_waitcnt(0);
  lds_barrier();
  int buf = 0;
  while (have) {
    SliceGeo ng = cg;
    int32_t nkt = kt + TK;
    bool have_next = true;
    if (nkt >= cg.khi) {
      have_next = find_slice(lists, wi.slice_end, (int32_t)a.nk, cg.si + 1, first_tok, last_tok, ng);
      nkt = ng.ks;
    }
    if (have_next) load_tile(nkt, ng.khi);  // in flight while this tile is computed
    const bool masked = kt < cg.klo || kt + TK > cg.kfull;
    const __bf16* Kb = Ks[buf];
    const __bf16* Vb = Vs[buf];
    const __attribute__((address_space(3))) __bf16* Kt = (const __attribute__((address_space(3))) __bf16*)Ks[buf];
#pragma unroll
    for (int kb = 0; kb < TK / 32; ++kb) {
      // S'^T = K . Q'^T and dP'^T = V . dO'^T (keys on M, rows on N)
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&Kb[(kb * 32 + ln) * C::PITCH + 16 * ks + 8 * h]);
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(&Vb[(kb * 32 + ln) * C::PITCH + 16 * ks + 8 * h]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, dreg[ks], dp, 0, 0, 0);
      }
      if (masked) {
        // keys at block offset >= lim or < lim_lo are hidden from the row
        const int32_t kb0 = kt + kb * 32 + 4 * h;
        const int32_t lim = geo_row_end(cg, qi) - kb0;
        const int32_t lim_lo = (cg.type & MAGI_MASK_INVCAUSAL) ? cg.loff + qi - kb0 : -TK;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (key_of0(i) >= lim || key_of0(i) < lim_lo) s[i] = -INFINITY;
      }
      // dS^T = P^T * dP'^T, rounded to bf16 in the B-operand layout
      bf16x8 dsb[2];
#pragma unroll
      for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = PRESCALED ? s[8 * i2 + e] : s[8 * i2 + e] * c;
          dsb[i2][e] = (__bf16)(__builtin_amdgcn_exp2f(x) * dp[8 * i2 + e]);
        }
      // dQ^T += K^T . dS^T (K^T through the transposed LDS read)
#pragma unroll
      for (int i2 = 0; i2 < 2; ++i2) {
        const int krow = kb * 32 + 16 * i2 + 4 * h + li / 4;
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) {
          const int dcol = mb * 32 + dgrp + 4 * (li % 4);
          const bf16x8 kt8 = read_tr8(Kt + krow * C::PITCH + dcol, C::PITCH);
          dq[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt8, dsb[i2], dq[mb], 0, 0, 0);
        }
      }
    }
    if (have_next) store_tile(buf ^ 1);
    lds_barrier();  // the next tile is in LDS; this buffer is free again
    cg = ng;
    kt = nkt;
    have = have_next;
    buf ^= 1;
  }

  // epilogue: dQ = scale * (dQ^T)^T; lane half h holds d = 8 grp + 4 h + r
  if (rvalid) {
    __bf16* dqp = reinterpret_cast<__bf16*>(a.dq) + (int64_t)qi * a.q_stride + (int64_t)head * D;
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int d = mb * 32 + 8 * grp + 4 * h;
        if (d < D) {
          bf16x4 w;
#pragma unroll
          for (int r = 0; r < 4; ++r) w[r] = (__bf16)(dq[mb][4 * grp + r] * a.scale);
          *reinterpret_cast<bf16x4*>(dqp + d) = w;
        }
      }
  }
}

// ----------------------------------------------------------------- dK/dV pass

// One run of query rows of one slice for a key-major item: tokens [t0, t_end)
// in TQ-row tiles (TQ / G tokens each).
struct QRun {
  int32_t si;      // position in the item's tile-slice list
  int32_t t0;      // first token of the current tile
  int32_t t_end;   // one past the last token of the run
  int32_t ks, ke;  // slice key range (ke clamped to nk)
  int32_t koff;    // k_end - q_end: under the upper bound token t sees keys below koff + t + 1
  int32_t loff;    // k_start - q_start: under the lower bound token t sees keys from loff + t
  int32_t type;    // mask type bits: 1 = upper bound, 2 = lower bound
  int32_t valid;
};

// First slice at or after list position si that shows some row one of the
// item's keys [k0, k1); fills the run of rows that see them.
__device__ __forceinline__ bool find_qrun(const SliceLists& L, int32_t slice_end, int32_t nq, int32_t nk,
                                          int si, int32_t k0, int32_t k1, int32_t w_lo, int32_t w_hi, QRun& r) {
  const int end = slice_end < L.num_tile_slices ? slice_end : L.num_tile_slices;
  for (si = si < 0 ? 0 : si; si < end; ++si) {
    const int sidx = const_ld(L.tile_slices + si);
    if (sidx < 0 || sidx >= L.num_slices) continue;
    const magi_attn_slice s = load_slice(L.slices, sidx);
    const int32_t ks = s.k_start > 0 ? s.k_start : 0;
    const int32_t ke = s.k_end < nk ? s.k_end : nk;
    int32_t qe = s.q_end < nq ? s.q_end : nq;
    if (qe > w_hi) qe = w_hi;  // the item's token window
    if (ks >= ke || s.q_start >= qe || ke <= k0 || ks >= k1) continue;
    const int32_t type = s.mask_type & (MAGI_MASK_CAUSAL | MAGI_MASK_INVCAUSAL);
    const int32_t koff = s.k_end - s.q_end;
    const int32_t loff = s.k_start - s.q_start;
    // rows that see a key of [max(k0, ks), min(k1, ke)): under the upper
    // bound row r sees k iff k < koff + r + 1, under the lower bound iff
    // k >= loff + r
    const int32_t kmin = k0 > ks ? k0 : ks;
    const int32_t kmax = (k1 < ke ? k1 : ke) - 1;
    int32_t t0 = s.q_start;
    if ((type & MAGI_MASK_CAUSAL) && kmin - koff > t0) t0 = kmin - koff;
    if (t0 < w_lo) t0 = w_lo;
    if ((type & MAGI_MASK_INVCAUSAL) && kmax - loff + 1 < qe) qe = kmax - loff + 1;
    if (t0 >= qe) continue;
    r.si = si;
    r.t0 = t0;
    r.t_end = qe;
    r.ks = ks;
    r.ke = ke;
    r.koff = koff;
    r.loff = loff;
    r.type = type;
    r.valid = 1;
    return true;
  }
  r.valid = 0;
  return false;
}

// KB: 32-key blocks per wave.  The item's kKeys keys are spread over
// kKeys / (32 KB) waves; KB = 2 lets one wave's Q'/dO' operand reads (and
// their transposes) serve 64 keys, halving those LDS reads per key.
template <int D, bool PRESCALED, int KB>
__global__ __launch_bounds__(2 * kKeys / KB, 2) void bwd_dkdv_bf16(BwdArgs a) {
  using C = BCfg<D>;
  constexpr int NTK = 2 * kKeys / KB;                // threads per workgroup
  constexpr int NCH = (TQ * C::CH + NTK - 1) / NTK;  // 16-byte chunks per thread per tile (Q and dO each)
  __shared__ __attribute__((aligned(16))) __bf16 Qs[2][TQ * C::PITCH];
  __shared__ __attribute__((aligned(16))) __bf16 Os[2][TQ * C::PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, ln = lane & 31, li = lane & 15;
  const int dgrp = ((lane >> 4) & 1) * 16;
  const magi_work_item wi = load_item(a.kwork, blockIdx.x);
  const int G = a.hq / a.hkv;
  if (wi.q_start < 0 || wi.q_len <= 0 || (int64_t)wi.q_start + wi.q_len > a.nk || wi.kv_group < 0 ||
      wi.kv_group >= a.hkv)
    return;
  const int32_t k0 = wi.q_start;  // key-major item: [k0, k0 + klen) keys of group g
  // partial slot (or -1) and token window of the item
  int32_t slot = -1, w_lo = 0, w_hi = (int32_t)a.nq;
  if (a.kitem_ext != nullptr) {
    slot = const_ld(&a.kitem_ext[3 * blockIdx.x]);
    w_lo = const_ld(&a.kitem_ext[3 * blockIdx.x + 1]);
    w_hi = const_ld(&a.kitem_ext[3 * blockIdx.x + 2]);
  }
  const int32_t klen = wi.q_len < kKeys ? wi.q_len : kKeys;
  const int32_t k1 = k0 + klen;
  const int g = wi.kv_group;
  const float c = a.scale * kLog2e;
  const float cinv = 1.0f / c;
  const int TQT = TQ / G;  // tokens per tile
  // floor(row / G) = (row * ginv) >> 16 for row < 64, G <= 64
  const int32_t ginv = ((1 << 16) + G - 1) / G;
  const int tq_rows = TQT * G;

  // zero padding columns D+2.. of both buffers once; columns D, D+1 are
  // rewritten with each tile's augmented values
  for (int b = 0; b < 2; ++b)
    for (int i = tid; i < TQ * (C::DA - D - 2); i += NTK) {
      const int col = D + 2 + i % (C::DA - D - 2), row = i / (C::DA - D - 2);
      Qs[b][row * C::PITCH + col] = (__bf16)0.0f;
      Os[b][row * C::PITCH + col] = (__bf16)0.0f;
    }

  // this lane's keys (column n of the MFMA, one per key block): K and V
  // rows as B operands with the two ones columns that meet the augmented slots
  int32_t key[KB];
  bool kvalid[KB];
  bf16x8 kreg[KB][C::KS], vreg[KB][C::KS];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    key[kb] = k0 + (wave * KB + kb) * 32 + ln;
    kvalid[kb] = key[kb] < k1;
    const int32_t kk = kvalid[kb] ? key[kb] : k0;
    const __bf16* krow = reinterpret_cast<const __bf16*>(a.k) + (int64_t)kk * a.kv_stride + (int64_t)g * a.kv_hstride;
    const __bf16* vrow = reinterpret_cast<const __bf16*>(a.v) + (int64_t)kk * a.kv_stride + (int64_t)g * a.kv_hstride;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const int d0 = 16 * ks + 8 * h;
      bf16x8 x = {}, y = {};
      if (d0 < D) {
        x = *reinterpret_cast<const bf16x8*>(krow + d0);
        y = *reinterpret_cast<const bf16x8*>(vrow + d0);
      } else if (d0 == D) {
        x[0] = x[1] = y[0] = y[1] = (__bf16)1.0f;
      }
      if (!kvalid[kb]) x = y = (bf16x8){};
      kreg[kb][ks] = x;
      vreg[kb][ks] = y;
    }
  }

  // Q'/dO' tiles: row n of a tile is (token t0 + n / G, head g G + n % G);
  // 16-byte chunks of the rows plus, per row, the augmented pairs
  u32x4 qr[NCH], orr[NCH];
  __bf16 aq0 = 0, aq1 = 0, ao0 = 0, ao1 = 0;  // augmented values of row tid (tid < TQ)
  auto load_tile = [&](const QRun& r) {
    const int32_t ntok = r.t_end - r.t0 < TQT ? r.t_end - r.t0 : TQT;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int ci = tid + j * NTK;
      u32x4 x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
      if (ci < TQ * C::CH) {
        const int row = ci / C::CH, part = ci % C::CH;
        const int tt = row / G, hh = row % G;
        if (row < tq_rows && tt < ntok) {
          const int64_t tok = r.t0 + tt;
          x = *reinterpret_cast<const u32x4*>(reinterpret_cast<const __bf16*>(a.q) + tok * a.q_stride +
                                              (int64_t)(g * G + hh) * D + part * 8);
          y = *reinterpret_cast<const u32x4*>(reinterpret_cast<const __bf16*>(a.dout) + tok * a.o_stride +
                                              (int64_t)(g * G + hh) * D + part * 8);
        }
      }
      qr[j] = x;
      orr[j] = y;
    }
    aq0 = aq1 = ao0 = ao1 = (__bf16)0.0f;
    if (tid < tq_rows && tid / G < ntok) {
      const int64_t tok = r.t0 + tid / G;
      const int64_t idx = tok * a.hq + g * G + tid % G;
      float l2 = a.lse[idx] * kLog2e;
      if (!(l2 > -INFINITY && l2 < INFINITY)) l2 = 0.f;
      split_bf16(-l2 * cinv, aq0, aq1);
      split_bf16(-a.delta[idx], ao0, ao1);
    }
  };
  auto store_tile = [&](int b) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int ci = tid + j * NTK;
      if (ci < TQ * C::CH) {
        const int row = ci / C::CH, part = ci % C::CH;
        *reinterpret_cast<u32x4*>(&Qs[b][row * C::PITCH + part * 8]) = qr[j];
        *reinterpret_cast<u32x4*>(&Os[b][row * C::PITCH + part * 8]) = orr[j];
      }
    }
    if (tid < TQ) {
      Qs[b][tid * C::PITCH + D] = aq0;
      Qs[b][tid * C::PITCH + D + 1] = aq1;
      Os[b][tid * C::PITCH + D] = ao0;
      Os[b][tid * C::PITCH + D + 1] = ao1;
    }
  };
  auto next_run = [&](const QRun& r, QRun& n) {
    n = r;
    n.t0 = r.t0 + TQT;
    if (r.valid && n.t0 >= r.t_end)
      find_qrun(SliceLists{a.slices, a.num_slices, a.k_tile_slices, a.num_k_tile_slices}, wi.slice_end,
                (int32_t)a.nq, (int32_t)a.nk, r.si + 1, k0, k1, w_lo, w_hi, n);
  };

  f32x16 dk[KB][C::MB], dv[KB][C::MB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) dk[kb][mb] = dv[kb][mb] = (f32x16){};

  QRun cur;
  find_qrun(SliceLists{a.slices, a.num_slices, a.k_tile_slices, a.num_k_tile_slices}, wi.slice_end, (int32_t)a.nq,
            (int32_t)a.nk, wi.slice_begin, k0, k1, w_lo, w_hi, cur);
  if (cur.valid) {
    load_tile(cur);
    store_tile(0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  lds_barrier();
  int buf = 0;
  while (cur.valid) {
    QRun nxt;
    next_run(cur, nxt);
    if (nxt.valid) load_tile(nxt);  // in flight while this tile is computed
    const int32_t ntok = cur.t_end - cur.t0 < TQT ? cur.t_end - cur.t0 : TQT;
    // every element visible: the item's keys inside the slice's key range,
    // a whole tile of rows, the tile's first token already seeing the item's
    // last key (upper bound) and its last token still seeing the item's
    // first key (lower bound)
    const bool full = cur.ks <= k0 && k1 <= cur.ke && ntok == TQT && tq_rows == TQ &&
                      (!(cur.type & MAGI_MASK_CAUSAL) || k1 - 1 < cur.koff + cur.t0 + 1) &&
                      (!(cur.type & MAGI_MASK_INVCAUSAL) || k0 >= cur.loff + cur.t0 + TQT - 1);
    const __bf16* Qb = Qs[buf];
    const __bf16* Ob = Os[buf];
    const __attribute__((address_space(3))) __bf16* Qt = (const __attribute__((address_space(3))) __bf16*)Qs[buf];
    const __attribute__((address_space(3))) __bf16* Ot = (const __attribute__((address_space(3))) __bf16*)Os[buf];
#pragma unroll
    for (int rb = 0; rb < TQ / 32; ++rb) {
      // S' = Q' . K^T and dP' = dO' . V^T (rows on M, keys on N); the A
      // operands are read once for all KB key blocks
      f32x16 s[KB], dp[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s[kb] = dp[kb] = (f32x16){};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&Qb[(rb * 32 + ln) * C::PITCH + 16 * ks + 8 * h]);
        const bf16x8 oa = *reinterpret_cast<const bf16x8*>(&Ob[(rb * 32 + ln) * C::PITCH + 16 * ks + 8 * h]);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kreg[kb][ks], s[kb], 0, 0, 0);
          dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vreg[kb][ks], dp[kb], 0, 0, 0);
        }
      }
      if (!full) {
        // Element i holds row 8 (i / 4) + 4 h + i % 4 of this 32-row block,
        // token tt = row / G of the tile.  The key of block kb is seen by
        // tokens lo <= tt < hi: hi = ntok (0 if the key is outside the
        // slice or the item), lowered to key - loff - t0 + 1 under the
        // lower bound (top-left aligned: token t sees k >= loff + t); lo =
        // key - koff - t0 under the upper bound (bottom-right aligned: token
        // t sees k < koff + t + 1).  The hiding mask is built by integer
        // arithmetic and applied with a bit select, so no lane-mask
        // registers are tied up.
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const bool kin = kvalid[kb] && key[kb] >= cur.ks && key[kb] < cur.ke;
          int32_t hi = kin ? ntok : 0;
          if (cur.type & MAGI_MASK_INVCAUSAL) {
            const int32_t e = key[kb] - cur.loff - cur.t0 + 1;
            hi = e < hi ? e : hi;
          }
          const int32_t lo = (cur.type & MAGI_MASK_CAUSAL) ? key[kb] - cur.koff - cur.t0 : -(1 << 30);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = rb * 32 + 8 * (i / 4) + 4 * h + (i % 4);  // < 64
            const int32_t tt = (row * ginv) >> 16;                    // row / G
            const uint32_t hide = (uint32_t)(((tt - lo) | (hi - 1 - tt)) >> 31);
            s[kb][i] = __uint_as_float((__float_as_uint(s[kb][i]) & ~hide) | (0xff800000u & hide));
          }
        }
      }
      // P and dS = P * dP', rounded to bf16 in the B-operand layout
      bf16x8 pb[KB][2], dsb[KB][2];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = PRESCALED ? s[kb][8 * i2 + e] : s[kb][8 * i2 + e] * c;
            const float p = __builtin_amdgcn_exp2f(x);
            pb[kb][i2][e] = (__bf16)p;
            dsb[kb][i2][e] = (__bf16)(p * dp[kb][8 * i2 + e]);
          }
      // dV^T += dO^T . P and dK^T += Q^T . dS (transposed LDS reads, shared
      // by the key blocks)
#pragma unroll
      for (int i2 = 0; i2 < 2; ++i2) {
        const int qrow = rb * 32 + 16 * i2 + 4 * h + li / 4;
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) {
          const int dcol = mb * 32 + dgrp + 4 * (li % 4);
          const bf16x8 ot8 = read_tr8(Ot + qrow * C::PITCH + dcol, C::PITCH);
          const bf16x8 qt8 = read_tr8(Qt + qrow * C::PITCH + dcol, C::PITCH);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            dv[kb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ot8, pb[kb][i2], dv[kb][mb], 0, 0, 0);
            dk[kb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qt8, dsb[kb][i2], dk[kb][mb], 0, 0, 0);
          }
        }
      }
    }
    if (nxt.valid) store_tile(buf ^ 1);
    lds_barrier();
    cur = nxt;
    buf ^= 1;
  }

  // epilogue: lane (key) holds d = mb 32 + 8 grp + 4 h + r of dK^T / dV^T.
  // One part of a split tile stores its fp32 sums (dK unscaled) in its slot;
  // bwd_reduce adds the parts and writes dK, dV.
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    if (kvalid[kb] && slot >= 0 && slot < a.num_slots) {
      float* pk = a.partial + (int64_t)slot * 2 * kKeys * D + (int64_t)(key[kb] - k0) * D;
      float* pv = pk + kKeys * D;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          const int d = mb * 32 + 8 * grp + 4 * h;
          if (d < D) {
            const f32x16& K = dk[kb][mb];
            const f32x16& V = dv[kb][mb];
            *reinterpret_cast<float4*>(pk + d) = make_float4(K[4 * grp], K[4 * grp + 1], K[4 * grp + 2], K[4 * grp + 3]);
            *reinterpret_cast<float4*>(pv + d) = make_float4(V[4 * grp], V[4 * grp + 1], V[4 * grp + 2], V[4 * grp + 3]);
          }
        }
    } else if (kvalid[kb] && slot < 0) {
      __bf16* dkp =
          reinterpret_cast<__bf16*>(a.dk) + (int64_t)key[kb] * a.kv_stride + (int64_t)g * a.kv_hstride;
      __bf16* dvp =
          reinterpret_cast<__bf16*>(a.dv) + (int64_t)key[kb] * a.kv_stride + (int64_t)g * a.kv_hstride;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          const int d = mb * 32 + 8 * grp + 4 * h;
          if (d < D) {
            bf16x4 wk, wv;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              wk[r] = (__bf16)(dk[kb][mb][4 * grp + r] * a.scale);
              wv[r] = (__bf16)dv[kb][mb][4 * grp + r];
            }
            *reinterpret_cast<bf16x4*>(dkp + d) = wk;
            *reinterpret_cast<bf16x4*>(dvp + d) = wv;
          }
        }
    }
  }
}

// ----------------------------------------------------------------- fp32 (small shapes)

// dQ: one thread per query row, keys streamed from global memory
template <int D>
__global__ __launch_bounds__(kThreads32) void bwd_dq_f32(BwdArgs a) {
  const magi_work_item wi = a.qwork[blockIdx.x];
  const int G = a.hq / a.hkv;
  const int cap = kThreads32 / G;
  if (wi.q_start < 0 || wi.q_len <= 0 || (int64_t)wi.q_start + wi.q_len > a.nq || wi.kv_group < 0 ||
      wi.kv_group >= a.hkv)
    return;
  const int qlen = wi.q_len < cap ? wi.q_len : cap;
  const int n = threadIdx.x, t = n / G, g = wi.kv_group, head = g * G + n % G;
  if (t >= qlen) return;
  const int64_t qi = (int64_t)wi.q_start + t;
  const float* qp = reinterpret_cast<const float*>(a.q) + qi * a.q_stride + (int64_t)head * D;
  const float* dop = reinterpret_cast<const float*>(a.dout) + qi * a.o_stride + (int64_t)head * D;
  const float* kp = reinterpret_cast<const float*>(a.k);
  const float* vp = reinterpret_cast<const float*>(a.v);
  const float lse = a.lse[qi * a.hq + head], dl = a.delta[qi * a.hq + head];
  float qv[D], dov[D], acc[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    qv[i] = qp[i];
    dov[i] = dop[i];
    acc[i] = 0.f;
  }
  if (lse > -INFINITY)
    for (int si = wi.slice_begin; si < wi.slice_end; ++si) {
      if (si < 0 || si >= a.num_q_tile_slices) break;
      const int sidx = a.q_tile_slices[si];
      if (sidx < 0 || sidx >= a.num_slices) continue;
      const magi_attn_slice sl = a.slices[sidx];
      if (qi < sl.q_start || qi >= sl.q_end) continue;
      const int64_t ks = sl.k_start > 0 ? sl.k_start : 0;
      const int64_t ke = sl.k_end < a.nk ? sl.k_end : a.nk;
      const int64_t re = row_key_end(sl, ke, qi);
      for (int64_t kk = row_key_begin(sl, ks, qi); kk < re; ++kk) {
        const float* kr = kp + kk * a.kv_stride + (int64_t)g * a.kv_hstride;
        const float* vr = vp + kk * a.kv_stride + (int64_t)g * a.kv_hstride;
        float s = 0.f, dpv = 0.f;
#pragma unroll
        for (int i = 0; i < D; ++i) {
          s = fmaf(qv[i], kr[i], s);
          dpv = fmaf(dov[i], vr[i], dpv);
        }
        const float p = expf(s * a.scale - lse);
        const float ds = p * (dpv - dl);
#pragma unroll
        for (int i = 0; i < D; ++i) acc[i] = fmaf(ds, kr[i], acc[i]);
      }
    }
  float* dqp = reinterpret_cast<float*>(a.dq) + qi * a.q_stride + (int64_t)head * D;
#pragma unroll
  for (int i = 0; i < D; ++i) dqp[i] = acc[i] * a.scale;
}

// dK/dV: one thread per key of the item, rows streamed from global memory
template <int D>
__global__ __launch_bounds__(kThreads32) void bwd_dkdv_f32(BwdArgs a) {
  const magi_work_item wi = a.kwork[blockIdx.x];
  const int G = a.hq / a.hkv;
  if (wi.q_start < 0 || wi.q_len <= 0 || (int64_t)wi.q_start + wi.q_len > a.nk || wi.kv_group < 0 ||
      wi.kv_group >= a.hkv)
    return;
  const int klen = wi.q_len < kThreads32 ? wi.q_len : kThreads32;
  if ((int)threadIdx.x >= klen) return;
  const int64_t key = (int64_t)wi.q_start + threadIdx.x;
  const int g = wi.kv_group;
  int32_t slot = -1, w_lo = 0, w_hi = (int32_t)a.nq;
  if (a.kitem_ext != nullptr) {
    slot = a.kitem_ext[3 * blockIdx.x];
    w_lo = a.kitem_ext[3 * blockIdx.x + 1];
    w_hi = a.kitem_ext[3 * blockIdx.x + 2];
  }
  const float* kr = reinterpret_cast<const float*>(a.k) + key * a.kv_stride + (int64_t)g * a.kv_hstride;
  const float* vr = reinterpret_cast<const float*>(a.v) + key * a.kv_stride + (int64_t)g * a.kv_hstride;
  float kv[D], vv[D], dkacc[D], dvacc[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    kv[i] = kr[i];
    vv[i] = vr[i];
    dkacc[i] = dvacc[i] = 0.f;
  }
  for (int si = wi.slice_begin; si < wi.slice_end; ++si) {
    if (si < 0 || si >= a.num_k_tile_slices) break;
    const int sidx = a.k_tile_slices[si];
    if (sidx < 0 || sidx >= a.num_slices) continue;
    const magi_attn_slice sl = a.slices[sidx];
    const int64_t ke = sl.k_end < a.nk ? sl.k_end : a.nk;
    if (key < sl.k_start || key >= ke) continue;
    int64_t r0 = sl.q_start;
    if (sl.mask_type & MAGI_MASK_CAUSAL) {
      const int64_t f = key - ((int64_t)sl.k_end - sl.q_end);  // first row that sees the key
      r0 = f > r0 ? f : r0;
    }
    if (r0 < w_lo) r0 = w_lo;
    int64_t qe = sl.q_end < a.nq ? sl.q_end : a.nq;
    if (sl.mask_type & MAGI_MASK_INVCAUSAL) {
      const int64_t e = key - ((int64_t)sl.k_start - sl.q_start) + 1;  // one past the last row that sees it
      qe = e < qe ? e : qe;
    }
    if (qe > w_hi) qe = w_hi;
    for (int64_t r = r0; r < qe; ++r)
      for (int hh = 0; hh < G; ++hh) {
        const int head = g * G + hh;
        const float lse = a.lse[r * a.hq + head];
        if (!(lse > -INFINITY)) continue;
        const float* qp = reinterpret_cast<const float*>(a.q) + r * a.q_stride + (int64_t)head * D;
        const float* dop = reinterpret_cast<const float*>(a.dout) + r * a.o_stride + (int64_t)head * D;
        float s = 0.f, dpv = 0.f;
#pragma unroll
        for (int i = 0; i < D; ++i) {
          s = fmaf(qp[i], kv[i], s);
          dpv = fmaf(dop[i], vv[i], dpv);
        }
        const float p = expf(s * a.scale - lse);
        const float ds = p * (dpv - a.delta[r * a.hq + head]);
#pragma unroll
        for (int i = 0; i < D; ++i) {
          dvacc[i] = fmaf(p, dop[i], dvacc[i]);
          dkacc[i] = fmaf(ds, qp[i], dkacc[i]);
        }
      }
  }
  if (slot >= 0) {
    if (slot >= a.num_slots || key - wi.q_start >= kKeys) return;
    float* pk = a.partial + (int64_t)slot * 2 * kKeys * D + (key - wi.q_start) * D;
    float* pv = pk + kKeys * D;
#pragma unroll
    for (int i = 0; i < D; ++i) {
      pk[i] = dkacc[i];
      pv[i] = dvacc[i];
    }
    return;
  }
  float* dkp = reinterpret_cast<float*>(a.dk) + key * a.kv_stride + (int64_t)g * a.kv_hstride;
  float* dvp = reinterpret_cast<float*>(a.dv) + key * a.kv_stride + (int64_t)g * a.kv_hstride;
#pragma unroll
  for (int i = 0; i < D; ++i) {
    dkp[i] = dkacc[i] * a.scale;
    dvp[i] = dvacc[i];
  }
}

// Sums of a split dK/dV pass: one block per reduce entry; each thread owns
// 4 channels of one key of dK or dV and adds the entry's slots in slot
// order (a fixed order, so the result is deterministic), then scales dK.
template <int D, typename T>
__global__ __launch_bounds__(256) void bwd_reduce(BwdArgs a) {
  const magi_kv_reduce r = a.reduce[blockIdx.x];
  if (r.key_len <= 0 || r.key_len > kKeys || r.key_start < 0 || (int64_t)r.key_start + r.key_len > a.nk ||
      r.kv_group < 0 || r.kv_group >= a.hkv || r.slot_begin < 0 || r.slot_count < 1 ||
      (int64_t)r.slot_begin + r.slot_count > a.num_slots)
    return;
  constexpr int Q4 = D / 4;
  const int n = 2 * r.key_len * Q4;  // (dK | dV, key, 4 channels)
  for (int i = threadIdx.x; i < n; i += 256) {
    const int which = i / (r.key_len * Q4), rem = i % (r.key_len * Q4);
    const int kr = rem / Q4, d = 4 * (rem % Q4);
    const float* src = a.partial + (int64_t)r.slot_begin * 2 * kKeys * D + (int64_t)which * kKeys * D +
                       (int64_t)kr * D + d;
    float4 acc = *reinterpret_cast<const float4*>(src);
    for (int sl = 1; sl < r.slot_count; ++sl) {
      const float4 x = *reinterpret_cast<const float4*>(src + (int64_t)sl * 2 * kKeys * D);
      acc.x += x.x;
      acc.y += x.y;
      acc.z += x.z;
      acc.w += x.w;
    }
    if (which == 0) {
      acc.x *= a.scale;
      acc.y *= a.scale;
      acc.z *= a.scale;
      acc.w *= a.scale;
    }
    T* dst = reinterpret_cast<T*>(which == 0 ? a.dk : a.dv) + (int64_t)(r.key_start + kr) * a.kv_stride +
             (int64_t)r.kv_group * a.kv_hstride + d;
    dst[0] = (T)acc.x;
    dst[1] = (T)acc.y;
    dst[2] = (T)acc.z;
    dst[3] = (T)acc.w;
  }
}

template <int D>
hipError_t launch_d(const BwdArgs& a, hipStream_t stream) {
  constexpr int KB = D == 24 ? KB24 : KB48;
  const bool bf = a.dtype == MAGI_DTYPE_BF16;
  const int64_t nvec = a.nq * a.hq;
  if (nvec > 0) {
    const dim3 grid((unsigned)((nvec + 255) / 256));
    if (bf)
      hipLaunchKernelGGL((bwd_delta<D, __bf16>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((bwd_delta<D, float>), grid, dim3(256), 0, stream, a);
  }
  const bool pre = fabsf(a.scale * kLog2e - 1.0f) < 1e-6f;
  if (a.num_qwork > 0) {
    const dim3 grid(a.num_qwork);
    if (!bf)
      hipLaunchKernelGGL((bwd_dq_f32<D>), grid, dim3(kThreads32), 0, stream, a);
    else if (pre)
      hipLaunchKernelGGL((bwd_dq_bf16<D, true>), grid, dim3(NT), 0, stream, a);
    else
      hipLaunchKernelGGL((bwd_dq_bf16<D, false>), grid, dim3(NT), 0, stream, a);
  }
  if (a.num_kwork > 0) {
    const dim3 grid(a.num_kwork);
    if (!bf)
      hipLaunchKernelGGL((bwd_dkdv_f32<D>), grid, dim3(kThreads32), 0, stream, a);
    else if (pre)
      hipLaunchKernelGGL((bwd_dkdv_bf16<D, true, KB>), grid, dim3(2 * kKeys / KB), 0, stream, a);
    else
      hipLaunchKernelGGL((bwd_dkdv_bf16<D, false, KB>), grid, dim3(2 * kKeys / KB), 0, stream, a);
  }
  if (a.num_reduce > 0) {
    const dim3 grid(a.num_reduce);
    if (bf)
      hipLaunchKernelGGL((bwd_reduce<D, __bf16>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((bwd_reduce<D, float>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffa_bwd(const BwdArgs& a, hipStream_t stream) {
  return a.head_dim == 24 ? launch_d<24>(a, stream) : launch_d<48>(a, stream);
}

}  // namespace magi

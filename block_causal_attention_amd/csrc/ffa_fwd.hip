// Flex-Flash-Attention forward for gfx950 (MI355X).
//
// What is computed: softmax attention over the union of AttnSlices listed by
// each work item (the FFA formulation on the MAGI-1 pages: study notes on
// zhao9797.github.io, "训练 Infra"; 量子位 article on dakule.com,
// "Flex-Flash-Attention"), with 128 query heads over 8 KV groups (study notes,
// "模型规格（Table 2）").  The pages' kernel is built on FlashAttention-3 for
// Hopper (TMA, slice-level parallelism, atomics); this one is designed for
// CDNA4 and needs no atomics because every work item owns its output rows.
//
// bf16 kernel layout (one workgroup = one work item = up to 256 query rows):
//  * GQA packing: the 16 query heads of a KV group share K and V, so a query
//    "row" is a (token, head) pair and the item's rows are tile_q tokens x 16
//    heads.  Each of the 4 waves owns 64 rows as two 32-row MFMA column blocks.
//  * Scores are computed transposed, S^T = K . Q^T, with
//    v_mfma_f32_32x32x16_bf16: keys run along the MFMA M axis and rows along
//    N, so every lane holds 16 scores of one row.  The row max needs only
//    in-register max plus one exchange between the two lane halves.
//  * The output is also kept transposed, O^T = V^T . P^T: P^T is exactly the
//    B operand layout of the next MFMA (the score accumulator of one lane
//    half holds keys {4h..4h+3, 8+4h..8+4h+3} of each 16-key step, which is a
//    valid k-slot assignment), so P never leaves registers.  The V^T operand
//    is read from a row-major V tile in LDS with ds_read_b64_tr_b16.
//  * head_dim is padded for the MFMA: the Q.K contraction to a multiple of 16
//    (24 -> 32, 48 stays 48), the V rows to a multiple of 32 (24 -> 32,
//    48 -> 64).  The first padding column of V holds 1.0, so the same MFMA
//    that accumulates P.V also accumulates the softmax denominator sum(P)
//    (of the bf16-rounded P actually used), at no VALU cost.
//  * K/V tiles of 64 keys are staged in LDS once and read by all 4 waves
//    (64 query heads x tokens).  Tiles wholly outside the visible range are
//    never visited; only tiles crossing a range end or a causal diagonal pay
//    for element masking.
//  * Online softmax in fp32 in the log2 domain (scale * log2(e) folded into
//    one multiply), exp via v_exp_f32.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace magi {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kThreads = 256;
constexpr int kRows = 256;  // query rows per work item
constexpr int TK = 64;      // keys per LDS tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1e30f;  // finite "minus infinity" for the running max
constexpr int kBufCfg = 0x00020000;  // raw buffer resource word 3 (gfx9 family: 32-bit data format)
constexpr float kShift = 8.0f;
constexpr float kBoundMargin = 1.0f + 1.0f / 128.0f;  // covers bf16 rounding of k and fp32 sums
constexpr float kBoundMax = 60.0f;                    // log2 units, see the bounded reference
#ifndef MAGI_VROW_MODE
#define MAGI_VROW_MODE 0
#endif
#ifndef MAGI_NB24
#define MAGI_NB24 1
#endif
#ifndef MAGI_NB48
#define MAGI_NB48 1
#endif     // move the softmax reference when a score exceeds it by 2^8

template <int D>
struct Cfg {
  static constexpr int DK = (D + 15) / 16 * 16;       // Q.K contraction length
  static constexpr int KS = DK / 16;                  // MFMA k-steps for Q.K
  static constexpr int DV = (D + 1 + 31) / 32 * 32;   // V columns incl. the ones column
  static constexpr int MB = DV / 32;                  // 32-row blocks of O^T
  static constexpr int KROW = DK + 8;                 // LDS pitch of a K row (elements)
  // LDS pitch of a V row (elements): ds_read_b64_tr_b16 has each group of
  // 16 lanes read 4 consecutive rows x 32 bytes, so the pitch is chosen to
  // put 4 consecutive rows in disjoint bank ranges
  static constexpr int VROW = MAGI_VROW_MODE == 0 ? (DV == 32 ? 32 : DV + 32) : DV + 8;
  static constexpr int CH = D / 8;                    // 16-byte chunks per K/V row
  // position of the denominator (the ones column, V column D) in the O^T
  // accumulator of lane half 0: block D/32, index 4*((D%32)/8) + D%4
  static constexpr int LMB = D / 32;
  static constexpr int LIDX = 4 * ((D % 32) / 8) + (D % 4);
  static_assert(((D % 32) / 4) % 2 == 0, "ones column must fall in lane half 0");
};

__device__ inline int64_t causal_end(const magi_attn_slice& s, int64_t ke, int64_t row) {
  // bottom-right aligned causal: row r sees k with k - k_end <= r - q_end
  const int64_t e = (int64_t)s.k_end - (int64_t)s.q_end + row + 1;
  return e < ke ? e : ke;
}

// One slice as seen by one work item.  Every field is the same for the whole
// workgroup and lives in scalar registers.
struct SliceGeo {
  int64_t ks;     // first key
  int64_t khi;    // one past the last key that any row of the item sees
  int64_t kfull;  // keys below this are visible to every row of the item
  int64_t ke;     // slice key end, clamped to nk
  int64_t koff;   // k_end - q_end: a causal row r sees keys below koff + r + 1
  int32_t causal;
  int32_t si;     // position in the tile-slice list
};

__device__ __forceinline__ int32_t uni(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }

// Largest bf16 value <= x (x finite).
__device__ __forceinline__ __bf16 bf16_floor(float x) {
  __bf16 r = (__bf16)x;
  if ((float)r > x) {
    unsigned short b = __builtin_bit_cast(unsigned short, r);
    b = (b & 0x7fff) == 0 ? 0x8001 : (b & 0x8000 ? b + 1 : b - 1);
    r = __builtin_bit_cast(__bf16, b);
  }
  return r;
}

// First slice at or after list position si that shows this item a key.
// Returns false when the list is exhausted.
__device__ __forceinline__ bool find_slice(const FfaArgs& a, const magi_work_item& wi, int si, int64_t first_tok,
                                           int64_t last_tok, SliceGeo& g) {
  const int end = wi.slice_end < a.num_tile_slices ? wi.slice_end : a.num_tile_slices;
  for (si = si < 0 ? 0 : si; si < end; ++si) {
    const int sidx = uni(a.tile_slices[si]);
    if (sidx < 0 || sidx >= a.num_slices) continue;
    const magi_attn_slice* sp = a.slices + sidx;
    const int64_t qs = uni(sp->q_start), qe = uni(sp->q_end), k0 = uni(sp->k_start), k1 = uni(sp->k_end);
    const int32_t causal = uni(sp->mask_type) == MAGI_MASK_CAUSAL;
    const int64_t ks = k0 > 0 ? k0 : 0;
    const int64_t ke = k1 < a.nk ? k1 : a.nk;
    // a well-formed schedule only lists slices that cover every row of the item
    if (ks >= ke || first_tok < qs || last_tok >= qe) continue;
    const int64_t koff = k1 - qe;
    const int64_t khi = causal ? (koff + last_tok + 1 < ke ? koff + last_tok + 1 : ke) : ke;
    if (khi <= ks) continue;
    g.ks = ks;
    g.khi = khi;
    g.kfull = causal ? (koff + first_tok + 1 < ke ? koff + first_tok + 1 : ke) : ke;
    g.ke = ke;
    g.koff = koff;
    g.causal = causal;
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

// PRESCALED: the caller folded softmax_scale * log2(e) into Q or K, so the
// scores leave the MFMA already in log2 units and need no multiply.
// NB: 32-row column blocks per wave.  The 256 rows of a work item are
// spread over 256 / (32 NB) waves, so NB = 1 doubles the waves per SIMD
// (more latency hiding) at the price of more LDS reads per score.
template <int D, bool PRESCALED, int NB>
__global__ __launch_bounds__(512 / NB, 4 / NB) void ffa_fwd_bf16(FfaArgs a) {
  using C = Cfg<D>;
  constexpr int NT = 512 / NB;  // threads per workgroup
  constexpr int NCH = (TK * C::CH + NT - 1) / NT;  // 16-byte K (and V) chunks per thread per tile
  // 32-key blocks whose scores are held at once: both for d=24, one at a
  // time for d=48 where the larger accumulators leave fewer registers
  constexpr int KG = D <= 32 ? 2 : 1;
  __shared__ __attribute__((aligned(16))) __bf16 Ks[2][TK * C::KROW];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[2][TK * C::VROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, ln = lane & 31;
  magi_work_item wi = a.work[blockIdx.x];
  wi.q_start = uni(wi.q_start);
  wi.q_len = uni(wi.q_len);
  wi.slice_begin = uni(wi.slice_begin);
  wi.slice_end = uni(wi.slice_end);
  wi.kv_group = uni(wi.kv_group);
  const int G = a.hq / a.hkv;
  const int cap = kRows / G;
  if (wi.q_start < 0 || wi.q_len <= 0 || (int64_t)wi.q_start + wi.q_len > a.nq || wi.kv_group < 0 ||
      wi.kv_group >= a.hkv)
    return;
  const int qlen = wi.q_len < cap ? wi.q_len : cap;
  const int g = wi.kv_group;
  const __bf16* __restrict__ qp = reinterpret_cast<const __bf16*>(a.q);
  const __bf16* __restrict__ kp = reinterpret_cast<const __bf16*>(a.k);
  const __bf16* __restrict__ vp = reinterpret_cast<const __bf16*>(a.v);

  // When head_dim leaves padding in the Q.K contraction (24 -> 32), the
  // running max rides in it: K padding column D holds 1 and the matching Q
  // slot holds -m, so the score MFMA itself returns q.k - m.  Otherwise
  // (48) the MFMA accumulator starts at -m instead.
  constexpr bool AUG = C::DK > D;
  // constant padding columns of both LDS buffers: K column D is 1 (AUG),
  // K columns D+1..DK-1 are 0, V column D is 1 (it accumulates the softmax
  // denominator), V columns D+1..DV-1 are 0
  for (int b = 0; b < 2; ++b) {
    if constexpr (AUG)
      for (int i = tid; i < TK * (C::DK - D); i += NT) {
        const int col = D + i % (C::DK - D);
        Ks[b][(i / (C::DK - D)) * C::KROW + col] = (__bf16)(col == D ? 1.0f : 0.0f);
      }
    for (int i = tid; i < TK * (C::DV - D); i += NT) {
      const int col = D + i % (C::DV - D);
      Vs[b][(i / (C::DV - D)) * C::VROW + col] = (__bf16)(col == D ? 1.0f : 0.0f);
    }
  }

  // this lane's two query rows (one per 32-row column block) as MFMA B operands
  int32_t qi[NB];  // query token of the row (< nq < 2^31)
  int hg[NB];
  bool rvalid[NB];
  bf16x8 qreg[NB][C::KS];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = wave * (32 * NB) + nb * 32 + ln;
    const int t = n / G;
    hg[nb] = n % G;
    rvalid[nb] = (t < qlen);
    qi[nb] = wi.q_start + (rvalid[nb] ? t : 0);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const int d0 = 16 * ks + 8 * h;
      bf16x8 x = {};
      if (rvalid[nb] && d0 < D)
        x = *reinterpret_cast<const bf16x8*>(qp + (int64_t)qi[nb] * a.q_stride + (int64_t)(g * G + hg[nb]) * D + d0);
      qreg[nb][ks] = x;
    }
  }

  // Softmax state per row: the reference m (log2 units).  With AUG it is
  // subtracted inside the score MFMA (Q padding slot) and kept exactly
  // representable in bf16; otherwise it is subtracted in the exponent.  m
  // moves only when a row sees its first key or when a score exceeds m by
  // more than kShift, so the common tile needs no rescale (P <= 2^kShift
  // stays finite).
  const float c = a.scale * kLog2e;
  const float cinv = PRESCALED ? 1.0f : 1.0f / c;
  float m[NB];
  bool init[NB];
  f32x16 o[NB][C::MB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m[nb] = 0.f;
    init[nb] = false;
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) o[nb][mb] = (f32x16){};
  }
  // Bounded reference.  When the caller supplies B >= |k| for every key of
  // the group, q.k <= |q| B (Cauchy-Schwarz) bounds every score of a row, so
  // |q| B can be the row's softmax reference from the start: no running
  // max, no rescaling.  A wave uses it when every row's bound keeps the
  // smallest possible score, -|q| B, within 2^-120 of it (bound <= 60 in
  // log2 units: no underflow to zero or denormals); otherwise it keeps the
  // online max.
  bool bounded = false;
  if (a.k_norm_max != nullptr) {
    const float B = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(a.k_norm_max[g])));
    bool ok = B > 0.f;  // also false for NaN
    float mb_row[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float ss = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = (float)qreg[nb][ks][e];
          ss = fmaf(x, x, ss);
        }
      ss += pair_other(ss, h);
      mb_row[nb] = sqrtf(ss) * B * (PRESCALED ? 1.0f : c) * kBoundMargin;
      ok = ok && mb_row[nb] <= kBoundMax;
    }
    bounded = __all(ok);
    if (bounded) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        init[nb] = true;
        if constexpr (AUG) {
          const __bf16 slot = bf16_floor(-mb_row[nb] * cinv);
          m[nb] = PRESCALED ? -(float)slot : -(float)slot * c;
          qreg[nb][C::KS - 1][0] = h ? slot : qreg[nb][C::KS - 1][0];
        } else {
          m[nb] = mb_row[nb];
        }
      }
    }
  }

  const int64_t first_tok = wi.q_start, last_tok = (int64_t)wi.q_start + qlen - 1;
  const int li = lane & 15;
  const int dgrp = ((lane >> 4) & 1) * 16;
  // key offset (within a 32-key block) of accumulator element i of this lane
  auto key_of = [&](int i) { return 8 * (i / 4) + 4 * h + (i % 4); };
  // K/V tiles are fetched with buffer loads whose range ends at the last
  // visible key, so rows past it read as zeros with no per-lane test; each
  // thread's byte offset inside a tile never changes.
  u32x4 kr[NCH], vr[NCH];
  int ch_off[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int ci = tid + j * NT;
    ch_off[j] = (ci / C::CH) * (int)a.kv_stride * 2 + (ci % C::CH) * 16;
  }
  const int64_t kv_row_bytes = a.kv_stride * 2;

  auto load_tile = [&](int64_t kt, int64_t khi) {
    const int64_t elem0 = kt * a.kv_stride + (int64_t)g * D;
    const int64_t valid = (khi - kt - 1) * kv_row_bytes + D * 2;
    const int nrec = valid <= 0 ? 0 : (valid > 0x7fffffff ? 0x7fffffff : (int)valid);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kp + elem0), (short)0, nrec, kBufCfg);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vp + elem0), (short)0, nrec, kBufCfg);
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      if (tid + j * NT < TK * C::CH) {
        kr[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, ch_off[j], 0, 0));
        vr[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, ch_off[j], 0, 0));
      }
    }
  };
  auto store_tile = [&](int b) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int ci = tid + j * NT;
      if (ci < TK * C::CH) {
        const int r = ci / C::CH, part = ci % C::CH;
        *reinterpret_cast<u32x4*>(&Ks[b][r * C::KROW + part * 8]) = kr[j];
        *reinterpret_cast<u32x4*>(&Vs[b][r * C::VROW + part * 8]) = vr[j];
      }
    }
  };

  SliceGeo cg;
  bool have = find_slice(a, wi, wi.slice_begin, first_tok, last_tok, cg);
  int64_t kt = cg.ks;
  if (have) {
    load_tile(kt, cg.khi);
    store_tile(0);
  }
  int buf = 0;
  while (have) {
    // the tile after this one: next in the slice, else the next slice's first
    SliceGeo ng = cg;
    int64_t nkt = kt + TK;
    bool have_next = true;
    if (nkt >= cg.khi) {
      have_next = find_slice(a, wi, cg.si + 1, first_tok, last_tok, ng);
      nkt = ng.ks;
    }
    __syncthreads();  // tile `buf` is in LDS; buffer buf^1 is no longer read
    if (have_next) load_tile(nkt, ng.khi);  // in flight while this tile is computed

    const bool masked = kt + TK > cg.kfull;
    int lim[NB];  // keys at tile offset >= lim[nb] are hidden from the row
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      int64_t re = cg.ke;
      if (cg.causal) {
        const int64_t ce = (int64_t)cg.koff + qi[nb] + 1;
        re = ce < re ? ce : re;
      }
      if (!rvalid[nb]) re = kt;
      const int64_t rel = re - kt;
      lim[nb] = rel < 0 ? 0 : (rel > TK ? TK : (int)rel);
    }
    const __bf16* Kb = Ks[buf];
    __attribute__((address_space(3))) __bf16* Vb = (__attribute__((address_space(3))) __bf16*)Vs[buf];

#pragma unroll
    for (int kb0 = 0; kb0 < 2; kb0 += KG) {
      // S^T = K . Q^T (minus m with AUG) for KG*32 keys x 32 NB rows; a lane
      // holds 16 keys of one row per block
      f32x16 s[KG][NB];
#pragma unroll
      for (int kg = 0; kg < KG; ++kg) {
        const int kb = kb0 + kg;
        bf16x8 kop[C::KS];
#pragma unroll
        for (int ks2 = 0; ks2 < C::KS; ++ks2)
          kop[ks2] = *reinterpret_cast<const bf16x8*>(&Kb[(kb * 32 + ln) * C::KROW + 16 * ks2 + 8 * h]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          f32x16 acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[0], qreg[nb][0], (f32x16){}, 0, 0, 0);
#pragma unroll
          for (int ks2 = 1; ks2 < C::KS; ++ks2)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[ks2], qreg[nb][ks2], acc, 0, 0, 0);
          s[kg][nb] = acc;
        }
      }
      if (masked) {
#pragma unroll
        for (int kg = 0; kg < KG; ++kg)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if ((kb0 + kg) * 32 + key_of(i) >= lim[nb]) s[kg][nb][i] = -INFINITY;
      }
      // row maxima of the shifted scores; move m only where needed (the
      // bounded reference never moves)
      bool sh[NB];
      float delta[NB];
      if (!bounded) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float mx = s[0][nb][0];
#pragma unroll
        for (int kg = 0; kg < KG; ++kg)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kg][nb][i]);
        mx = pair_max(mx);
        const float xm = (PRESCALED ? mx : mx * c) - (AUG ? 0.f : m[nb]);
        sh[nb] = (!init[nb] && xm > -INFINITY) || xm > kShift;
        delta[nb] = sh[nb] ? xm : 0.f;
        init[nb] = init[nb] || xm > -INFINITY;
      }
      bool any_sh = false;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) any_sh |= sh[nb];
      if (__any(any_sh)) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          float mnew = m[nb] + delta[nb];
          __bf16 slot;
          if constexpr (AUG) {
            // the score MFMA subtracts a bf16 copy of m (unscaled units):
            // round it toward larger m so no score can exceed it by more
            // than the rounding step, and track exactly that value
            slot = bf16_floor(-mnew * cinv);
            mnew = PRESCALED ? -(float)slot : -(float)slot * c;
          }
          const float step = mnew - m[nb];
          m[nb] = mnew;
          const float alpha = __builtin_amdgcn_exp2f(-step);
#pragma unroll
          for (int mb = 0; mb < C::MB; ++mb) o[nb][mb] *= alpha;
          if constexpr (AUG) {
            const float dsub = step * cinv;
#pragma unroll
            for (int kg = 0; kg < KG; ++kg)
#pragma unroll
              for (int i = 0; i < 16; ++i) s[kg][nb][i] -= dsub;
            qreg[nb][C::KS - 1][0] = h ? slot : qreg[nb][C::KS - 1][0];
          }
        }
      }
      }
#pragma unroll
      for (int kg = 0; kg < KG; ++kg) {
        const int kb = kb0 + kg;
        // P = 2^(S'), rounded to bf16, already in the B-operand layout of P^T
        bf16x8 pb[2][NB];  // [16-key half][nb]
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float sv = s[kg][nb][8 * i2 + e];
              float x;
              if constexpr (AUG)
                x = PRESCALED ? sv : sv * c;
              else
                x = PRESCALED ? sv - m[nb] : fmaf(sv, c, -m[nb]);
              pb[i2][nb][e] = (__bf16)__builtin_amdgcn_exp2f(x);
            }
        // O^T += V^T . P^T ; the V^T operand comes from the row-major V tile
        // through the LDS transpose read
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2) {
          const int krow = kb * 32 + 16 * i2 + 4 * h + li / 4;
#pragma unroll
          for (int mb = 0; mb < C::MB; ++mb) {
            const int dcol = mb * 32 + dgrp + 4 * (li % 4);
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vb + krow * C::VROW + dcol));
            const s16x4 hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vb + (krow + 8) * C::VROW + dcol));
            const bf16x8 vop =
                __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
              o[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[i2][nb], o[nb][mb], 0, 0, 0);
          }
        }
      }
    }

    if (have_next) store_tile(buf ^ 1);
    cg = ng;
    kt = nkt;
    have = have_next;
    buf ^= 1;
  }

  // epilogue: O = O^T / l, LSE = (m + log2 l) ln 2
  __bf16* __restrict__ op = reinterpret_cast<__bf16*>(a.out);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float mine = o[nb][C::LMB][C::LIDX];
    const float other = pair_other(mine, h);  // all 64 lanes must take part in the swap
    const float l = h == 0 ? mine : other;
    if (!rvalid[nb]) continue;
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    const int64_t obase = (int64_t)qi[nb] * a.o_stride + (int64_t)(g * G + hg[nb]) * D;
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int d = mb * 32 + 8 * grp + 4 * h;
        if (d < D) {
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          bf16x4 w;
#pragma unroll
          for (int r = 0; r < 4; ++r) w[r] = (__bf16)(o[nb][mb][4 * grp + r] * inv);
          *reinterpret_cast<bf16x4*>(op + obase + d) = w;
        }
      }
    if (a.lse != nullptr && h == 0)
      a.lse[(int64_t)qi[nb] * a.hq + g * G + hg[nb]] = l > 0.f ? (m[nb] + __log2f(l)) * kLn2 : -INFINITY;
  }
}
// fp32 path (small shapes): one thread per query row, keys streamed from
// global memory, fp32 online softmax.  Same work list and masking rules.
template <int D>
__global__ __launch_bounds__(kThreads) void ffa_fwd_f32(FfaArgs a) {
  const magi_work_item wi = a.work[blockIdx.x];
  const int G = a.hq / a.hkv;
  const int cap = kRows / G;
  if (wi.q_start < 0 || wi.q_len <= 0 || (int64_t)wi.q_start + wi.q_len > a.nq || wi.kv_group < 0 ||
      wi.kv_group >= a.hkv)
    return;
  const int qlen = wi.q_len < cap ? wi.q_len : cap;
  const int n = threadIdx.x, t = n / G, hgi = n % G, g = wi.kv_group;
  if (t >= qlen) return;
  const int64_t qi = (int64_t)wi.q_start + t;
  const int head = g * G + hgi;
  const float* qp = reinterpret_cast<const float*>(a.q) + qi * a.q_stride + (int64_t)head * D;
  const float* kp = reinterpret_cast<const float*>(a.k);
  const float* vp = reinterpret_cast<const float*>(a.v);
  const float c = a.scale * kLog2e;
  float qv[D], o[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    qv[i] = qp[i];
    o[i] = 0.f;
  }
  float m = kNegBig, l = 0.f;
  for (int si = wi.slice_begin; si < wi.slice_end; ++si) {
    if (si < 0 || si >= a.num_tile_slices) break;
    const int sidx = a.tile_slices[si];
    if (sidx < 0 || sidx >= a.num_slices) continue;
    const magi_attn_slice sl = a.slices[sidx];
    if (qi < sl.q_start || qi >= sl.q_end) continue;
    const int64_t ks = sl.k_start > 0 ? sl.k_start : 0;
    const int64_t ke = sl.k_end < a.nk ? sl.k_end : a.nk;
    const int64_t re = sl.mask_type == MAGI_MASK_CAUSAL ? causal_end(sl, ke, qi) : ke;
    for (int64_t key = ks; key < re; ++key) {
      const float* kr = kp + key * a.kv_stride + (int64_t)g * D;
      const float* vr = vp + key * a.kv_stride + (int64_t)g * D;
      float sdot = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) sdot = fmaf(qv[i], kr[i], sdot);
      const float x = sdot * c;
      const float mnew = fmaxf(m, x);
      const float alpha = exp2f(m - mnew);
      const float p = exp2f(x - mnew);
      l = l * alpha + p;
#pragma unroll
      for (int i = 0; i < D; ++i) o[i] = fmaf(p, vr[i], o[i] * alpha);
      m = mnew;
    }
  }
  float* op = reinterpret_cast<float*>(a.out) + qi * a.o_stride + (int64_t)head * D;
  const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
  for (int i = 0; i < D; ++i) op[i] = o[i] * inv;
  if (a.lse != nullptr) a.lse[qi * a.hq + head] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_ffa_fwd(const FfaArgs& a, hipStream_t stream) {
  if (a.num_work == 0) return hipSuccess;
  const dim3 grid(a.num_work), block(kThreads);
  if (a.dtype == MAGI_DTYPE_BF16) {
    // scores arrive in log2 units when the caller folded scale * log2(e) into Q or K
    const bool pre = fabsf(a.scale * kLog2e - 1.0f) < 1e-6f;
    constexpr int NB24 = MAGI_NB24, NB48 = MAGI_NB48;
    if (a.head_dim == 24) {
      if (pre)
        hipLaunchKernelGGL((ffa_fwd_bf16<24, true, NB24>), grid, dim3(512 / NB24), 0, stream, a);
      else
        hipLaunchKernelGGL((ffa_fwd_bf16<24, false, NB24>), grid, dim3(512 / NB24), 0, stream, a);
    } else {
      if (pre)
        hipLaunchKernelGGL((ffa_fwd_bf16<48, true, NB48>), grid, dim3(512 / NB48), 0, stream, a);
      else
        hipLaunchKernelGGL((ffa_fwd_bf16<48, false, NB48>), grid, dim3(512 / NB48), 0, stream, a);
    }
  } else {
    if (a.head_dim == 24)
      hipLaunchKernelGGL(ffa_fwd_f32<24>, grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL(ffa_fwd_f32<48>, grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace magi

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
//  * GQA packing: the query heads of a KV group share K and V, so a query
//    "row" is a (token, head) pair and the item's rows are tile_q tokens x G
//    heads.  Each wave owns NB 32-row MFMA column blocks (NB = 2 for head_dim
//    24: 4 waves; NB = 1 for 48: 8 waves).
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
//  * K/V tiles of 64 keys are staged in LDS once and read by every wave of
//    the item.  Three LDS buffers rotate: one tile is computed while the next
//    sits in LDS and the one after is in flight from HBM; the K operand of
//    each 32-key block is read one block ahead.  Tiles wholly outside the
//    visible range are never visited; only tiles crossing a range end or a
//    causal diagonal pay for element masking.
//  * Softmax in fp32 in the log2 domain against a fixed per-row reference
//    (a bound from the key norms when the caller supplies one, else an
//    online max that moves only by large steps), exp via v_exp_f32.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <type_traits>

#include "ffa_common.h"
#include "kernels.h"

namespace magi {
namespace {

using namespace dev;

constexpr int kRows = 256;        // query rows per work item
constexpr int kThreads = kRows;   // fp32 kernel: one thread per row
constexpr int TK = 64;  // keys per LDS tile
constexpr float kNegBig = -1e30f;  // finite "minus infinity" for the running max
constexpr float kShift = 8.0f;  // move the softmax reference when a score exceeds it by 2^8
constexpr float kBoundMargin = 1.0f + 1.0f / 128.0f;  // covers bf16 rounding of k and fp32 sums
constexpr float kBoundMax = 60.0f;                    // log2 units, see the bounded reference

template <int D>
struct Cfg {
  static constexpr int DK = (D + 15) / 16 * 16;       // Q.K contraction length
  static constexpr int KS = DK / 16;                  // MFMA k-steps for Q.K
  static constexpr int DV = (D + 1 + 31) / 32 * 32;   // V columns incl. the ones column
  static constexpr int MB = DV / 32;                  // 32-row blocks of O^T
  // K and V tile rows in LDS, so that neither the b128 row reads of K nor
  // the transposed reads of V put two lanes of a pass on one bank: at
  // head_dim 24 64-byte rows with the chunks of K rows permuted by kswz; at
  // 48 padded rows of 112 bytes (K) and 192 bytes (V), which need no
  // permutation (the reads of 4 consecutive V rows x 32 bytes fall in
  // disjoint bank ranges)
  static constexpr int KROW = DK > 32 ? DK + 8 : 32;  // LDS pitch of a K row (elements)
  static constexpr int VROW = DK > 32 ? DV + 32 : DV;  // LDS pitch of a V row (elements)
  static constexpr int CH = D / 8;                    // 16-byte chunks per K/V row
  // position of the denominator (the ones column, V column D) in the O^T
  // accumulator of lane half 0: block D/32, index 4*((D%32)/8) + D%4
  static constexpr int LMB = D / 32;
  static constexpr int LIDX = 4 * ((D % 32) / 8) + (D % 4);
  static_assert(((D % 32) / 4) % 2 == 0, "ones column must fall in lane half 0");
};

// Slot of chunk c in row r of a K or V tile: c ^ swizzle(r).  The 64-byte
// K rows of head_dim 24 move chunks by bits 2-3 of r, so that 16
// consecutive rows of one chunk cover all 16 four-bank groups; V there (4
// consecutive rows x 4 chunks are 16 consecutive slots) and both tiles at
// 48 (padded rows) keep their order.
template <int D>
__device__ __forceinline__ int kswz(int r) {
  return D > 32 ? 0 : (r >> 2) & 3;
}
template <int D>
__device__ __forceinline__ int vswz(int) {
  return 0;
}

// Buffer load of 16 bytes per lane straight into LDS: lane l's bytes land
// at dst + 16 l (dst wave-uniform); lanes past the resource's range write
// zeros, inactive lanes write nothing.  Counted by vmcnt like other loads.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, __bf16* dst, int32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 0);
}

// Transposed read of an 8-row step whose 4-row halves sit at their own
// addresses.  Restrict-qualified sources (both only read) give the inlined
// reads alias-scope metadata, so the compiler's wait-count pass does not
// drain the direct tile loads in flight before them; the tile they read
// was completed before the barrier that precedes its use.
__device__ __forceinline__ bf16x8 read_tr_pair(const __attribute__((address_space(3))) __bf16* __restrict__ lo,
                                               const __attribute__((address_space(3))) __bf16* __restrict__ hi) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)lo);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)hi);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

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

// PRESCALED: the caller folded softmax_scale * log2(e) into Q or K, so the
// scores leave the MFMA already in log2 units and need no multiply.
// NB: 32-row column blocks per wave.  The 256 rows of a work item are
// spread over 256 / (32 NB) waves, so NB = 1 doubles the waves of a
// workgroup at the price of more LDS reads per score.  Both run 4 waves
// per SIMD (NB = 2 fits 128 VGPRs once no registers stage the tiles).
// QN: q holds the raw queries; each lane applies QK-Norm and the 3D RoPE to
// its rows after loading them (as the prologue kernel does for K).
template <int D, bool PRESCALED, int NB, bool QN>
__global__ __launch_bounds__(2 * kRows / NB, 4) void ffa_fwd_bf16(FfaArgs a) {
  using C = Cfg<D>;
  constexpr int NT = 2 * kRows / NB;  // threads per workgroup: 32 NB rows per wave
  __shared__ __attribute__((aligned(16))) __bf16 Ks[3][TK * C::KROW];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[3][TK * C::VROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, ln = lane & 31;
  const magi_work_item wi = load_item(a.work, blockIdx.x);
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
  // (the tile loads never write those chunks)
  for (int b = 0; b < 3; ++b) {
    if constexpr (AUG)
      for (int i = tid; i < TK * (C::DK - D); i += NT) {
        const int col = D + i % (C::DK - D), r = i / (C::DK - D);
        Ks[b][r * C::KROW + (((col >> 3) ^ kswz<D>(r)) << 3) + (col & 7)] = (__bf16)(col == D ? 1.0f : 0.0f);
      }
    for (int i = tid; i < TK * (C::DV - D); i += NT) {
      const int col = D + i % (C::DV - D), r = i / (C::DV - D);
      Vs[b][r * C::VROW + (((col >> 3) ^ vswz<D>(r)) << 3) + (col & 7)] = (__bf16)(col == D ? 1.0f : 0.0f);
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
  if constexpr (QN) {
    // Row of 32-row block nb: lane half h holds channels 16 ks + 8 h .. + 7
    // of each k-step ks, i.e. channel pairs 8 ks + 4 h + e (e < 4).  Pair p
    // of axis section p / (D/6) turns by pos_axis * base_axis^(-2 j / (D/3)),
    // j = p mod (D/6).  The RMS needs both lane halves of the row.
    constexpr int PS = D / 6;
    float inv[C::KS][4];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pr = 8 * ks + 4 * h + e;
        inv[ks][e] = 0.f;
        if (2 * pr < D)
          inv[ks][e] = exp2f(-(float)(2 * (pr % PS)) / (float)(D / 3) * log2f(a.qn_base[pr / PS]));
      }
    constexpr float kInv2Pi = 0.15915494309189535f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float x[C::KS][8];
      float ss = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x[ks][e] = (float)qreg[nb][ks][e];
          ss = fmaf(x[ks][e], x[ks][e], ss);
        }
      ss += pair_other(ss, h);
      if (!rvalid[nb]) continue;
      const float r = 1.0f / sqrtf(ss / (float)D + a.qn_eps) * a.qn_scale;
      const float* gp = a.qn_gain + (int64_t)(g * G + hg[nb]) * a.qn_gain_hstride;
      const int32_t* pp = a.qn_pos + (int64_t)qi[nb] * 3;
      const float pos[3] = {(float)pp[0], (float)pp[1], (float)pp[2]};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const int d0 = 16 * ks + 8 * h;
        if (d0 >= D) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int pr = 8 * ks + 4 * h + e;
          const float x0 = x[ks][2 * e] * r * gp[d0 + 2 * e];
          const float x1 = x[ks][2 * e + 1] * r * gp[d0 + 2 * e + 1];
          // angle in turns, reduced to [0, 1) for the hardware sine and cosine
          const float turns = __builtin_amdgcn_fractf(pos[pr / PS] * inv[ks][e] * kInv2Pi);
          const float sn = __builtin_amdgcn_sinf(turns), cs = __builtin_amdgcn_cosf(turns);
          qreg[nb][ks][2 * e] = (__bf16)(x0 * cs - x1 * sn);
          qreg[nb][ks][2 * e + 1] = (__bf16)(x0 * sn + x1 * cs);
        }
        if (a.q_hat != nullptr)
          *reinterpret_cast<bf16x8*>(reinterpret_cast<__bf16*>(a.q_hat) + (int64_t)qi[nb] * a.q_hat_stride +
                                     (int64_t)(g * G + hg[nb]) * D + d0) = qreg[nb][ks];
      }
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
  // Bounded scores.  When the caller supplies B >= |k| for every key of the
  // group, every score of a row lies within +-|q| B (Cauchy-Schwarz).  If
  // that is at most 60 log2 units for every row of the wave, P = 2^s itself
  // stays within [2^-60, 2^60] (normal in fp32 and bf16, sums far from
  // overflow), and a softmax reference would only cancel in
  // O = sum(P v) / sum(P): the wave then uses m = 0 and skips the running
  // max, the rescaling and the subtraction.  Otherwise it keeps the online
  // max.
  bool bounded = false;
  if (a.k_norm_max != nullptr) {
    const uint32_t Bbits = __builtin_amdgcn_readfirstlane(__float_as_uint(a.k_norm_max[g]));
    const float B = __uint_as_float(Bbits);
    // positive and finite, tested on the bits (the device code is compiled
    // assuming no NaN, so a float compare could be folded): 0 < bits < +inf
    bool ok = Bbits - 1u < 0x7f7fffffu;
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
  }

  const int32_t first_tok = wi.q_start, last_tok = wi.q_start + qlen - 1;
  const SliceLists lists{a.slices, a.num_slices, a.tile_slices, a.num_tile_slices};
  const int li = lane & 15;
  const int dgrp = ((lane >> 4) & 1) * 16;
  // Accumulator element i of lane half h holds key 8 (i / 4) + 4 h + i % 4
  // of its 32-key block; the lane-independent part is a compile-time
  // constant, so masking compares against constants.
  constexpr auto key_of0 = [](int i) { return 8 * (i / 4) + (i % 4); };
  // K/V tiles go straight from global memory into LDS (buffer loads with an
  // LDS destination, no staging registers): one load fills 64 consecutive
  // 16-byte slots, so a lane's slot fixes which chunk of which key row it
  // fetches; the first half of the waves fetches K, the second V, LPW loads
  // each per tile.  The loads' range ends at the last visible key, so rows
  // past it read as zeros with no per-lane test; lanes whose slot holds a
  // constant chunk (the ones and zero columns) stay inactive.  A lane's byte
  // offset inside a tile never changes; a tile spans TK rows of kv_stride
  // elements, which the entry point keeps under 2^31 bytes.
  constexpr int NWV = NT / 64;                        // waves
  constexpr int HW = NWV / 2;                         // waves per tensor
  constexpr int KSL = C::KROW / 8, VSL = C::VROW / 8;  // slots per row
  constexpr int NLK = TK * KSL / 64, NLV = TK * VSL / 64;  // loads per tile
  static_assert((TK * KSL) % 64 == 0 && (TK * VSL) % 64 == 0, "whole loads per tile");
  constexpr int LPW = ((NLK > NLV ? NLK : NLV) + HW - 1) / HW;  // loads per wave and tile, at most
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const bool ld_k = wave_u < HW;
  const int ld_n = ld_k ? NLK : NLV;       // loads of this wave's tensor
  const int ld_sl = ld_k ? KSL : VSL;      // its slots per row
  const int32_t kv_row_bytes = (int32_t)a.kv_stride * 2;
  int32_t ld_off[LPW];
  bool ld_on[LPW];
#pragma unroll
  for (int k = 0; k < LPW; ++k) {
    const int sl = 64 * (wave_u % HW + HW * k) + lane;
    const int r = sl / ld_sl;
    const int chunk = (sl % ld_sl) ^ (ld_k ? kswz<D>(r) : vswz<D>(r));
    ld_on[k] = chunk < C::CH;
    ld_off[k] = r * kv_row_bytes + chunk * 16;
  }

  // The item's tiles in visiting order: TK-key steps through one slice's
  // visible key range, then on to the next slice that shows the item a key.
  struct TileRef {
    SliceGeo geo;
    int32_t kt;     // first key of the tile
    int32_t valid;  // 0 once the slice list is exhausted
  };
  auto next_tile = [&](const TileRef& t, TileRef& n) {
    n.geo = t.geo;
    n.kt = t.kt + TK;
    n.valid = t.valid;
    if (t.valid && n.kt >= t.geo.khi) {
      n.valid = find_slice(lists, wi.slice_end, (int32_t)a.nk, t.geo.si + 1, first_tok, last_tok, n.geo);
      n.kt = n.geo.ks;
    }
  };
  auto issue_tile = [&](const TileRef& t, int b) {
    const int64_t elem0 = (int64_t)t.kt * a.kv_stride + (int64_t)g * a.kv_hstride;
    const int32_t rows = t.geo.khi - t.kt < TK ? t.geo.khi - t.kt : TK;  // >= 1
    const int nrec = (rows - 1) * kv_row_bytes + D * 2;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)((ld_k ? kp : vp) + elem0), (short)0, nrec, kBufCfg);
    __bf16* tile = ld_k ? Ks[b] : Vs[b];
#pragma unroll
    for (int k = 0; k < LPW; ++k) {
      const int J = wave_u % HW + HW * k;
      if (J < ld_n && ld_on[k]) load_lds16(rs, tile + J * 64 * 8, ld_off[k]);
    }
  };

  // K operand (A of S^T = K . Q^T) of 32-key block kb of LDS buffer b
  auto read_k = [&](int b, int kb, bf16x8 (&kop)[C::KS]) {
#pragma unroll
    for (int ks2 = 0; ks2 < C::KS; ++ks2)
      kop[ks2] = *reinterpret_cast<const bf16x8*>(
          &Ks[b][(kb * 32 + ln) * C::KROW + (((2 * ks2 + h) ^ kswz<D>(kb * 32 + ln)) << 3)]);
  };

  // Pipeline.  Three LDS buffers hold consecutive tiles.  While a tile is
  // computed, the next one sits in LDS and the one after is in flight from
  // global memory; the K operand of each 32-key block is read from LDS one
  // block ahead, so neither the global nor the LDS latency is on the
  // critical path.  With tile t in buffer t % 3 and one barrier per tile
  // (before its last block):
  //   block NBLK-2 of tile t ends by storing tile t+1 (loads issued one tile
  //   earlier) into buffer (t+1) % 3, whose previous tile t-2 was last read
  //   before the barrier of tile t-1;
  //   after the barrier, the loads of tile t+2 are issued and the K operand
  //   of tile t+1's first block is read.
  constexpr int NBLK = TK / 32;
  static_assert(NBLK >= 2, "the pipeline needs two blocks per tile");
  TileRef T0, T1;
  T0.valid = find_slice(lists, wi.slice_end, (int32_t)a.nk, wi.slice_begin, first_tok, last_tok, T0.geo);
  T0.kt = T0.geo.ks;
  next_tile(T0, T1);
  bf16x8 kcur[C::KS];
  // the first two tiles are fetched together; the barrier's release fence
  // waits for both
  if (T0.valid) issue_tile(T0, 0);
  if (T1.valid) issue_tile(T1, 1);
  __builtin_amdgcn_s_waitcnt(0);
  lds_barrier();
  read_k(0, 0, kcur);  // unused if the item sees no key
  int b0 = 0;  // buffer of T0
  // Whether a slice of the item bounds its keys from below (inverse causal
  // or band): only then do tiles below the diagonal need the second test.
  // The head_dim 24 loop has one instance without that test (it saves 2 %
  // there); head_dim 48 keeps a single instance, which is as fast as the
  // test-free one while a second copy of its loop spills scalar registers.
  bool lower = D == 48;
  if constexpr (D != 48) {
    const int end = wi.slice_end < a.num_tile_slices ? wi.slice_end : a.num_tile_slices;
    for (int si = wi.slice_begin < 0 ? 0 : wi.slice_begin; si < end; ++si) {
      const int sidx = const_ld(a.tile_slices + si);
      if (sidx >= 0 && sidx < a.num_slices) lower |= (const_ld(&a.slices[sidx].mask_type) & MAGI_MASK_INVCAUSAL) != 0;
    }
  }
  // the tile loop, compiled for bounded waves and for waves with an online
  // max, each with and without lower key bounds
  auto tile_loop = [&](auto bounded_tag, auto lower_tag) {
    constexpr bool BOUNDED = decltype(bounded_tag)::value;
    constexpr bool LOWER = decltype(lower_tag)::value;
    while (T0.valid) {
      const int b1 = b0 == 2 ? 0 : b0 + 1;
      const bool masked = (LOWER && T0.kt < T0.geo.klo) || T0.kt + TK > T0.geo.kfull;
      const __bf16* Kb = Ks[b0];
      __attribute__((address_space(3))) __bf16* Vb = (__attribute__((address_space(3))) __bf16*)Vs[b0];
      TileRef T2;
#pragma unroll
      for (int kb = 0; kb < NBLK; ++kb) {
        bf16x8 knext[C::KS];
        if (kb == NBLK - 1) {
          // tile T1 is in buffer b1: the release fence of the barrier waits
          // for this wave's loads of it, the barrier for every wave's
          __builtin_amdgcn_s_waitcnt(0);
          lds_barrier();
          next_tile(T1, T2);
          if (T2.valid) issue_tile(T2, b1 == 2 ? 0 : b1 + 1);  // into the buffer T0's predecessor used
          read_k(b1, 0, knext);  // unused after the last tile
        } else {
          read_k(b0, kb + 1, knext);
        }
        // S^T = K . Q^T (minus m with AUG) for 32 keys x 32 NB rows; a lane
        // holds 16 keys of one row
        f32x16 sc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          f32x16 acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kcur[0], qreg[nb][0], (f32x16){}, 0, 0, 0);
#pragma unroll
          for (int ks2 = 1; ks2 < C::KS; ++ks2)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kcur[ks2], qreg[nb][ks2], acc, 0, 0, 0);
          sc[nb] = acc;
        }
#pragma unroll
        for (int ks2 = 0; ks2 < C::KS; ++ks2) kcur[ks2] = knext[ks2];
        if (masked) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            // keys at block offset >= lim or < lim_lo are hidden from the row
            const int32_t kb0 = T0.kt + kb * 32 + 4 * h;
            const int32_t lim = geo_row_end(T0.geo, qi[nb]) - kb0;
            const int32_t lim_lo = (LOWER && (T0.geo.type & MAGI_MASK_INVCAUSAL)) ? T0.geo.loff + qi[nb] - kb0 : -TK;
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if (key_of0(i) >= lim || (LOWER && key_of0(i) < lim_lo)) sc[nb][i] = -INFINITY;
          }
        }
        // row maxima of the shifted scores; move m only where needed (the
        // bounded reference never moves)
        if constexpr (!BOUNDED) {
          bool sh[NB];
          float delta[NB];
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            float mx = sc[nb][0];
#pragma unroll
            for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc[nb][i]);
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
                for (int i = 0; i < 16; ++i) sc[nb][i] -= dsub;
                qreg[nb][C::KS - 1][0] = h ? slot : qreg[nb][C::KS - 1][0];
              }
            }
          }
        }
        // P = 2^(S'), rounded to bf16, already in the B-operand layout of P^T;
        // O^T += V^T . P^T with the V^T operand read from the row-major V tile
        // through the LDS transpose read
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2) {
          bf16x8 pb[NB];
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float sv = sc[nb][8 * i2 + e];
              float x;
              if constexpr (AUG || BOUNDED)
                x = PRESCALED ? sv : sv * c;
              else
                x = PRESCALED ? sv - m[nb] : fmaf(sv, c, -m[nb]);
              pb[nb][e] = (__bf16)__builtin_amdgcn_exp2f(x);
            }
          const int krow = kb * 32 + 16 * i2 + 4 * h + li / 4;
#pragma unroll
          for (int mb = 0; mb < C::MB; ++mb) {
            const int dcol = mb * 32 + dgrp + 4 * (li % 4);
            const int plo = krow * C::VROW + (((dcol >> 3) ^ vswz<D>(krow)) << 3) + (dcol & 7);
            const int phi = (krow + 8) * C::VROW + (((dcol >> 3) ^ vswz<D>(krow + 8)) << 3) + (dcol & 7);
            const bf16x8 vop = read_tr_pair(Vb + plo, Vb + phi);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
              o[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[nb], o[nb][mb], 0, 0, 0);
          }
        }
      }
      T0 = T1;
      T1 = T2;
      b0 = b1;
    }
  };
  if (bounded) {
    if (lower)
      tile_loop(std::true_type{}, std::true_type{});
    else if constexpr (D != 48)
      tile_loop(std::true_type{}, std::false_type{});
  } else {
    if (lower)
      tile_loop(std::false_type{}, std::true_type{});
    else if constexpr (D != 48)
      tile_loop(std::false_type{}, std::false_type{});
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
    const int64_t re = row_key_end(sl, ke, qi);
    for (int64_t key = row_key_begin(sl, ks, qi); key < re; ++key) {
      const float* kr = kp + key * a.kv_stride + (int64_t)g * a.kv_hstride;
      const float* vr = vp + key * a.kv_stride + (int64_t)g * a.kv_hstride;
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

hipError_t launch_ffa_fwd(const FfaArgs& a, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (a.num_work == 0) return hipSuccess;
  const dim3 grid(a.num_work);
  dim3 block(kThreads);
  void (*kern)(FfaArgs) = nullptr;
  if (a.dtype == MAGI_DTYPE_BF16) {
    // scores arrive in log2 units when the caller folded scale * log2(e) into Q or K
    const bool pre = fabsf(a.scale * kLog2e - 1.0f) < 1e-6f;
    // head_dim 24: 64 rows per wave halve the LDS operand reads per score;
    // head_dim 48: 32 rows per wave
    constexpr int NB24 = 2, NB48 = 1;
    const bool qn = a.qn_gain != nullptr;
    if (a.head_dim == 24) {
      block = dim3(2 * kRows / NB24);
      kern = qn ? (pre ? ffa_fwd_bf16<24, true, NB24, true> : ffa_fwd_bf16<24, false, NB24, true>)
                : (pre ? ffa_fwd_bf16<24, true, NB24, false> : ffa_fwd_bf16<24, false, NB24, false>);
    } else {
      block = dim3(2 * kRows / NB48);
      kern = qn ? (pre ? ffa_fwd_bf16<48, true, NB48, true> : ffa_fwd_bf16<48, false, NB48, true>)
                : (pre ? ffa_fwd_bf16<48, true, NB48, false> : ffa_fwd_bf16<48, false, NB48, false>);
    }
  } else {
    kern = a.head_dim == 24 ? ffa_fwd_f32<24> : ffa_fwd_f32<48>;
  }
  if (start != nullptr || stop != nullptr) {
    FfaArgs arg = a;
    void* args[] = {&arg};
    return hipExtLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, args, 0, stream, start, stop, 0);
  }
  hipLaunchKernelGGL(kern, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace magi

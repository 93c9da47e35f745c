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

#include <mutex>

#include "ffa_common.h"
#include "kernels.h"

namespace magi {
namespace {

using namespace dev;

typedef __attribute__((address_space(3))) void lds_void;

// Buffer load of 16 bytes per lane straight into LDS: lane l's bytes land
// at dst + 16 l (dst wave-uniform); lanes past the resource's range write
// zeros.  Counted by vmcnt like any other load.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, __bf16* dst, int32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, off, 0, 0, 0);
}

// read_tr8 for a tile whose rows are permuted separately: the 4-row halves
// of the 8-row step come from their own addresses.  The restrict-qualified
// sources (both only read) give the inlined reads alias-scope metadata; for
// such a read the compiler's wait-count pass waits only on direct-to-LDS
// loads whose scopes it can match, and the tile loads carry none, so no
// `vmcnt(0)` lands in the middle of a tile (a transposed read without
// scope metadata drains every direct load in flight).  The tiles stay
// correct without that wait: a buffer being filled is read only after the
// tile's explicit vmcnt wait and barrier.
__device__ __forceinline__ bf16x8 read_tr8_pair(const __attribute__((address_space(3))) __bf16* __restrict__ lo,
                                                const __attribute__((address_space(3))) __bf16* __restrict__ hi) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)lo);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)hi);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

constexpr int kRows = 256;      // query rows per dQ work item (the forward's items)
constexpr int kKeys = 128;      // keys per dK/dV work item (4 waves x 32)
constexpr int NT = 512;         // threads per workgroup of the bf16 dQ pass at one row block per wave
// 32-key blocks per wave of the bf16 dK/dV pass (head_dim 24 / 48).  Two blocks per
// wave at head_dim 24 need 256 VGPRs (2 waves per SIMD) and measured no faster.
constexpr int KB24 = 1, KB48 = 1;
// 32-row blocks per wave of the bf16 dQ pass (head_dim 24 / 48): two halve
// the K/V operand reads per score; measured 5 % (24, 3 waves per SIMD at
// 168 VGPRs) and 11 % (48, 2 waves per SIMD) faster than one
constexpr int RBQ24 = 2, RBQ48 = 2;
constexpr int TK = 64;          // keys per K/V tile (dQ pass)
constexpr int TQ = 64;          // query rows per Q/dO tile (dK/dV pass)
constexpr int kThreads32 = 256;  // fp32 kernels

template <int D>
struct BCfg {
  static constexpr int DA = (D + 2 + 15) / 16 * 16;  // contraction incl. the two augmented columns
  static constexpr int KS = DA / 16;                 // MFMA k-steps over it
  static constexpr int DM = (D + 31) / 32 * 32;      // rows of the head_dim-major accumulators
  static constexpr int MB = DM / 32;
  static constexpr int KD = (D + 15) / 16;           // k-steps over the data columns alone (dK/dV pass)
  // LDS row pitch (elements): 144 bytes puts the 16 rows of a b128 row read
  // in disjoint banks; the transposed reads then see at most 2-way conflicts
  static constexpr int PITCH = 72;
  static constexpr int CH = D / 8;  // 16-byte chunks per row
  // Q'/dO' tiles of the dK/dV pass filled by direct loads: 8 16-byte slots
  // per row, the chunks of row r permuted by tile_swizzle(r)
  static constexpr int NC = 8;
  static_assert(DA <= PITCH && D % 8 == 0 && 8 * NC >= DM && D / 8 <= NC, "layout");
};

// Slot of 16-byte chunk c in row r of a direct-loaded dK/dV tile of 128-byte
// rows: c ^ tile_swizzle(r).  With 64 banks of 4 bytes, a b128 row read
// (16 lanes: 16 consecutive rows, one chunk) and a transposed read (32
// lanes: 4 consecutive rows from a multiple of 4, chunks 0-3 or 4-7) then
// each touch every bank once; unswizzled 128-byte rows would put 2 or 4
// lanes on one bank.  The value is 4 * bit 1 of r + bits 2-3 of r.
__device__ __forceinline__ int tile_swizzle(int r) { return ((r >> 1) & 1) * 4 + ((r >> 2) & 3); }

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

// RB: 32-row blocks per wave.  The item's kRows rows are spread over
// kRows / (32 RB) waves; RB = 2 lets one wave's K/V operand reads (and the
// transposed K reads) serve 64 rows, halving those LDS reads per score.
template <int D, bool PRESCALED, int RB>
__global__ __launch_bounds__(NT / RB, RB == 2 && D == 24 ? 3 : 2) void bwd_dq_bf16(BwdArgs a) {
  using C = BCfg<D>;
  constexpr int NTQ = NT / RB;                       // threads per workgroup
  constexpr int NCH = (TK * C::CH + NTQ - 1) / NTQ;  // registers: 16-byte chunks per thread per tile (K and V each)
  // K/V tiles as the dK/dV pass stages its Q'/dO' tiles: at head_dim 48 in
  // three LDS buffers filled by direct loads two tiles ahead, 128-byte rows
  // permuted by tile_swizzle, waves 0-1 loading K and 2-3 V (the padding-only
  // contraction step is built in registers); at 24 in two buffers staged
  // through registers, 144-byte rows.
  constexpr bool DMA = D >= 48;
  constexpr int NC = C::NC;
  constexpr int KP = DMA ? 8 * NC : C::PITCH;  // tile row pitch (elements)
  constexpr int NW = NTQ / 64;                 // waves
  constexpr int LPW = NC / 2;                  // DMA: loads per wave (two waves per tile)
  static_assert(!DMA || (NW == 4 && NC % 2 == 0 && D % 16 == 0), "two waves per tile; no mixed step");
  __shared__ __attribute__((aligned(16))) __bf16 Ks[DMA ? 3 : 2][TK * KP];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[DMA ? 3 : 2][TK * KP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the loads branch per wave
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

  // registers: padding columns of every K and V buffer: D and D+1 are 1
  // (they meet the augmented slots), the rest 0; tile stores never touch them
  if constexpr (!DMA)
    for (int b = 0; b < 2; ++b)
      for (int i = tid; i < TK * (C::DA - D); i += NTQ) {
        const int col = D + i % (C::DA - D), row = i / (C::DA - D);
        const __bf16 x = (__bf16)(col < D + 2 ? 1.0f : 0.0f);
        Ks[b][row * KP + col] = x;
        Vs[b][row * KP + col] = x;
      }

  // this lane's query rows (one per 32-row MFMA column block of the wave)
  int32_t qi[RB];
  bool rvalid[RB];
  int head[RB];
  bf16x8 qreg[RB][C::KS], dreg[RB][C::KS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int n = (wave * RB + rb) * 32 + ln;
    const int t = n / G, hg = n % G;
    head[rb] = g * G + hg;
    rvalid[rb] = t < qlen;
    qi[rb] = wi.q_start + (rvalid[rb] ? t : 0);
    float lse2 = a.lse[(int64_t)qi[rb] * a.hq + head[rb]] * kLog2e;
    // a row that sees no key (LSE = -inf); tested on the bits, which no
    // no-NaN assumption of the device compile can fold: exponent all ones
    if ((__float_as_uint(lse2) & 0x7f800000u) == 0x7f800000u) lse2 = 0.f;
    const float dl = a.delta[(int64_t)qi[rb] * a.hq + head[rb]];
    __bf16 qa0, qa1, da0, da1;
    split_bf16(-lse2 / c, qa0, qa1);
    split_bf16(-dl, da0, da1);
    const __bf16* qrow = reinterpret_cast<const __bf16*>(a.q) + (int64_t)qi[rb] * a.q_stride + (int64_t)head[rb] * D;
    const __bf16* drow = reinterpret_cast<const __bf16*>(a.dout) + (int64_t)qi[rb] * a.o_stride + (int64_t)head[rb] * D;
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
      if (!rvalid[rb]) x = y = (bf16x8){};
      qreg[rb][ks] = x;
      dreg[rb][ks] = y;
    }
  }

  // K/V tiles: as in the forward, buffer loads whose range ends at the last
  // visible key (rows past it read as zeros)
  u32x4 kr[NCH], vr[NCH];
  int ch_off[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int ci = tid + j * NTQ;
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
      if (tid + j * NTQ < TK * C::CH) {
        kr[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, ch_off[j], 0, 0));
        vr[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, ch_off[j], 0, 0));
      }
  };
  auto store_tile = [&](int b) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int ci = tid + j * NTQ;
      if (ci < TK * C::CH) {
        const int r = ci / C::CH, part = ci % C::CH;
        *reinterpret_cast<u32x4*>(&Ks[b][r * KP + part * 8]) = kr[j];
        *reinterpret_cast<u32x4*>(&Vs[b][r * KP + part * 8]) = vr[j];
      }
    }
  };
  // DMA: load k of a wave fills the 64 slots from 64 J, J = (wave & 1) + 2 k,
  // of the K (waves 0-1) or V tile; slot s is key row s / NC, its chunk the
  // one tile_swizzle puts there; chunks >= D / 8 read past the range (zeros)
  constexpr int32_t kPastRange = 0x7ffffff0;
  const bool ldk = wave < 2;
  int32_t ld_off[LPW];
#pragma unroll
  for (int k = 0; k < LPW; ++k) {
    const int sl = 64 * ((wave & 1) + 2 * k) + lane;
    const int row = sl / NC, part = (sl % NC) ^ tile_swizzle(sl / NC);
    ld_off[k] = part < C::CH ? row * kv_row_bytes + part * 16 : kPastRange;
  }
  auto issue_tile = [&](int32_t kt, int32_t khi, int b) {
    const int64_t elem0 = (int64_t)kt * a.kv_stride + (int64_t)g * a.kv_hstride;
    const int32_t rows = khi - kt < TK ? khi - kt : TK;
    const int nrec = (rows - 1) * kv_row_bytes + D * 2;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)((ldk ? kp : vp) + elem0), (short)0, nrec, kBufCfg);
    __bf16* tile = ldk ? Ks[b] : Vs[b];
#pragma unroll
    for (int k = 0; k < LPW; ++k) load_lds16(rs, tile + ((wave & 1) + 2 * k) * 64 * 8, ld_off[k]);
  };
  // DMA: end of a tile, as in the dK/dV pass: this wave's LPW loads of the
  // tile after next may stay in flight, the older ones must have landed
  auto end_tile = [&](bool pending) {
    if (pending)
      __builtin_amdgcn_s_waitcnt(0x70 | LPW);  // vmcnt(LPW), expcnt 7, lgkmcnt(0)
    else
      __builtin_amdgcn_s_waitcnt(0x70);
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
  };

  const int32_t first_tok = wi.q_start, last_tok = wi.q_start + qlen - 1;
  const SliceLists lists{a.slices, a.num_slices, a.q_tile_slices, a.num_q_tile_slices};
  constexpr auto key_of0 = [](int i) { return 8 * (i / 4) + (i % 4); };

  f32x16 dq[RB][C::MB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) dq[rb][mb] = (f32x16){};

  // the tile after (g0, t0): TK keys on in the slice, else the next slice
  // that shows the item a key
  auto next_tile = [&](const SliceGeo& g0, int32_t t0, SliceGeo& g1, int32_t& t1) {
    g1 = g0;
    t1 = t0 + TK;
    bool ok = true;
    if (t1 >= g0.khi) {
      ok = find_slice(lists, wi.slice_end, (int32_t)a.nk, g0.si + 1, first_tok, last_tok, g1);
      t1 = g1.ks;
    }
    return ok;
  };
  SliceGeo cg, ng;
  bool have = find_slice(lists, wi.slice_end, (int32_t)a.nk, wi.slice_begin, first_tok, last_tok, cg);
  int32_t kt = cg.ks, nkt = 0;
  bool have_next = false;
  if constexpr (DMA) {
    if (have) {
      issue_tile(kt, cg.khi, 0);
      have_next = next_tile(cg, kt, ng, nkt);
      if (have_next) issue_tile(nkt, ng.khi, 1);
    }
    end_tile(false);
  } else {
    if (have) {
      load_tile(kt, cg.khi);
      store_tile(0);
    }
    // drain once: the lane-masked loads and stores above would otherwise make
    // the wait-count bookkeeping serialise every tile on its own prefetch
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
  }
  int buf = 0;
  while (have) {
    SliceGeo ng2;
    int32_t nkt2 = 0;
    bool have2 = false;
    if constexpr (DMA) {
      if (have_next) have2 = next_tile(ng, nkt, ng2, nkt2);
      if (have2) issue_tile(nkt2, ng2.khi, buf == 0 ? 2 : buf - 1);  // in flight during this tile and the next
    } else {
      have_next = next_tile(cg, kt, ng, nkt);
      if (have_next) load_tile(nkt, ng.khi);  // in flight while this tile is computed
    }
    const bool masked = kt < cg.klo || kt + TK > cg.kfull;
    const __bf16* Kb = Ks[buf];
    const __bf16* Vb = Vs[buf];
    const __attribute__((address_space(3))) __bf16* Kt = (const __attribute__((address_space(3))) __bf16*)Ks[buf];
#pragma unroll
    for (int kb = 0; kb < TK / 32; ++kb) {
      // S'^T = K . Q'^T and dP'^T = V . dO'^T (keys on M, rows on N); the K
      // and V operands are read once for all RB row blocks
      bf16x8 ka[C::KS], va[C::KS];
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        if (16 * ks >= D) {
          // a step of padding columns only (head_dim 48: 48..63): the two
          // ones columns in lane half 0, zeros elsewhere, as in the buffers
          bf16x8 ones = {};
          ones[0] = ones[1] = (__bf16)1.0f;
          ka[ks] = va[ks] = h ? (bf16x8){} : ones;
        } else {
          const int row = kb * 32 + ln;
          const int col = DMA ? ((2 * ks + h) ^ tile_swizzle(row)) * 8 : 16 * ks + 8 * h;
          ka[ks] = *reinterpret_cast<const bf16x8*>(&Kb[row * KP + col]);
          va[ks] = *reinterpret_cast<const bf16x8*>(&Vb[row * KP + col]);
        }
      }
      // dS^T = P^T * dP'^T, rounded to bf16 in the B-operand layout
      bf16x8 dsb[RB][2];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        f32x16 s = {}, dp = {};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qreg[rb][ks], s, 0, 0, 0);
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[ks], dreg[rb][ks], dp, 0, 0, 0);
        }
        if (masked) {
          // keys at block offset >= lim or < lim_lo are hidden from the row
          const int32_t kb0 = kt + kb * 32 + 4 * h;
          const int32_t lim = geo_row_end(cg, qi[rb]) - kb0;
          const int32_t lim_lo = (cg.type & MAGI_MASK_INVCAUSAL) ? cg.loff + qi[rb] - kb0 : -TK;
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (key_of0(i) >= lim || key_of0(i) < lim_lo) s[i] = -INFINITY;
        }
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = PRESCALED ? s[8 * i2 + e] : s[8 * i2 + e] * c;
            dsb[rb][i2][e] = (__bf16)(__builtin_amdgcn_exp2f(x) * dp[8 * i2 + e]);
          }
      }
      // dQ^T += K^T . dS^T (K^T through the transposed LDS read, shared by
      // the row blocks)
#pragma unroll
      for (int i2 = 0; i2 < 2; ++i2) {
        const int krow = kb * 32 + 16 * i2 + 4 * h + li / 4;
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) {
          const int dcol = mb * 32 + dgrp + 4 * (li % 4);
          bf16x8 kt8;
          if constexpr (DMA) {
            const int lo = krow * KP + (((dcol >> 3) ^ tile_swizzle(krow)) << 3) + (dcol & 7);
            const int hi = (krow + 8) * KP + (((dcol >> 3) ^ tile_swizzle(krow + 8)) << 3) + (dcol & 7);
            kt8 = read_tr8_pair(Kt + lo, Kt + hi);
          } else {
            kt8 = read_tr8(Kt + krow * KP + dcol, KP);
          }
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            dq[rb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt8, dsb[rb][i2], dq[rb][mb], 0, 0, 0);
        }
      }
    }
    if constexpr (DMA) {
      end_tile(have2);
      cg = ng;
      kt = nkt;
      have = have_next;
      ng = ng2;
      nkt = nkt2;
      have_next = have2;
      buf = buf == 2 ? 0 : buf + 1;
    } else {
      if (have_next) store_tile(buf ^ 1);
      lds_barrier();  // the next tile is in LDS; this buffer is free again
      cg = ng;
      kt = nkt;
      have = have_next;
      buf ^= 1;
    }
  }

  // epilogue: dQ = scale * (dQ^T)^T; lane half h holds d = 8 grp + 4 h + r
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (!rvalid[rb]) continue;
    __bf16* dqp = reinterpret_cast<__bf16*>(a.dq) + (int64_t)qi[rb] * a.q_stride + (int64_t)head[rb] * D;
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int d = mb * 32 + 8 * grp + 4 * h;
        if (d < D) {
          bf16x4 w;
#pragma unroll
          for (int r = 0; r < 4; ++r) w[r] = (__bf16)(dq[rb][mb][4 * grp + r] * a.scale);
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
__global__ __launch_bounds__(2 * kKeys / KB, D == 24 ? 4 : 3) void bwd_dkdv_bf16(BwdArgs a) {
  using C = BCfg<D>;
  constexpr int NTK = 2 * kKeys / KB;                // threads per workgroup
  // Two ways to stage the Q'/dO' tiles of TQ rows in LDS:
  //  * head_dim 48 (DMA): three buffers filled straight from global memory
  //    (buffer loads with an LDS destination) two tiles ahead of the tile
  //    being computed, so no registers stage them.  Such a load writes each
  //    lane's 16 bytes to consecutive LDS addresses: a tile row is NC = 8
  //    16-byte slots holding its D / 8 data chunks (and zeros) in the order
  //    tile_swizzle gives, chosen by each lane's source offset, and one load
  //    fills 8 rows.  Waves 0-1 load the Q' tile, waves 2-3 the dO' tile
  //    (one buffer resource per wave and tile).  The data fill whole
  //    k-steps, so the rows' -LSE2 and -delta start the S' and dP'
  //    accumulators (from small fp32 arrays) instead of riding in a
  //    padding step: two MFMAs and eight registers fewer per 32 x 32 block.
  //  * head_dim 24: two buffers, the next tile loaded into registers while
  //    this one is computed and stored at the end, with the rows' -LSE2 and
  //    -delta (each a bf16 high and low part) in padding columns D, D + 1,
  //    which meet ones in K and V inside the last, part-filled k-step (so
  //    they cost no MFMA here).  Direct loads measured 12 % slower at this
  //    size: their longer loop (more scalar work) costs more than it hides.
  constexpr bool DMA = D >= 48;
  constexpr int NC = C::NC;
  constexpr int QP = DMA ? 8 * NC : C::PITCH;  // tile row pitch (elements)
  constexpr int NW = NTK / 64;                 // waves
  constexpr int LPW = NC / 2;                  // DMA: loads per wave (two waves per tile)
  constexpr int NCH = (TQ * C::CH + NTK / 2 - 1) / (NTK / 2);  // registers: 16-byte chunks per thread
  __shared__ __attribute__((aligned(16))) __bf16 Qs[DMA ? 3 : 2][TQ * QP];
  __shared__ __attribute__((aligned(16))) __bf16 Os[DMA ? 3 : 2][TQ * QP];
  // DMA: per row of a tile, -LSE2 (times 1/c unless K is prescaled) and
  // -delta, the initial values of the row's S' and dP' accumulators, so that
  // exp2(S') is P and P dP' is dS without per-score subtractions
  __shared__ __attribute__((aligned(16))) float Qa[DMA ? 3 : 1][DMA ? TQ : 4], Oa[DMA ? 3 : 1][DMA ? TQ : 4];
  constexpr int KQ = DMA ? C::KD : C::KS;  // k-steps of S' and dP'
  // DMA: every wave issues the same LPW loads per tile, so the number in
  // flight is the same in every wave and on every path, and the wait-count
  // bookkeeping stays exact.
  static_assert(!DMA || NC % 2 == 0, "two waves share a tile's loads evenly");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the loads branch per wave
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
  const int tq_rows = TQT * G;

  if constexpr (!DMA) {
    // zero padding columns D+2.. of both buffers once; columns D, D+1 are
    // rewritten with each tile's augmented values
    for (int b = 0; b < 2; ++b)
      for (int i = tid; i < TQ * (C::DA - D - 2); i += NTK) {
        const int col = D + 2 + i % (C::DA - D - 2), row = i / (C::DA - D - 2);
        Qs[b][row * QP + col] = (__bf16)0.0f;
        Os[b][row * QP + col] = (__bf16)0.0f;
      }
  }

  // this lane's keys (column n of the MFMA, one per key block): K and V
  // rows as B operands; the register path adds the two ones columns that
  // meet the augmented slots
  int32_t key[KB];
  bool kvalid[KB];
  bf16x8 kreg[KB][KQ], vreg[KB][KQ];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    key[kb] = k0 + (wave * KB + kb) * 32 + ln;
    kvalid[kb] = key[kb] < k1;
    const int32_t kk = kvalid[kb] ? key[kb] : k0;
    const __bf16* krow = reinterpret_cast<const __bf16*>(a.k) + (int64_t)kk * a.kv_stride + (int64_t)g * a.kv_hstride;
    const __bf16* vrow = reinterpret_cast<const __bf16*>(a.v) + (int64_t)kk * a.kv_stride + (int64_t)g * a.kv_hstride;
#pragma unroll
    for (int ks = 0; ks < KQ; ++ks) {
      const int d0 = 16 * ks + 8 * h;
      bf16x8 x = {}, y = {};
      if (d0 < D) {
        x = *reinterpret_cast<const bf16x8*>(krow + d0);
        y = *reinterpret_cast<const bf16x8*>(vrow + d0);
      } else if (!DMA && d0 == D) {
        x[0] = x[1] = y[0] = y[1] = (__bf16)1.0f;
      }
      if (!kvalid[kb]) x = y = (bf16x8){};
      kreg[kb][ks] = x;
      vreg[kb][ks] = y;
    }
  }

  // Waves 0 and 1 stage the Q' tile, waves 2 and 3 the dO' tile, so a wave
  // builds one buffer resource per tile.  Row n of a tile is (token t0 +
  // n / G, head g G + n % G).  A lane's byte offsets from the tile's first
  // token are fixed (strides below 2^23 elements, checked by the entry
  // point); the loads go through buffer resources whose range ends with the
  // tile's last token, so rows past it read as zeros without per-lane tests.
  const bool ldq = wave < 2;
  const int64_t ld_stride = ldq ? a.q_stride : a.o_stride;
  const __bf16* ld_base = reinterpret_cast<const __bf16*>(ldq ? a.q : a.dout) + (int64_t)g * G * D;
  // registers: chunk ci = tid mod 128 + 128 j of the wave pair's tile; chunks
  // of no row (past tq_rows when G does not divide TQ) stay zero
  u32x4 stg[NCH];
  int32_t st_off[NCH];
  bool st_row[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int ci = (tid & 127) + 128 * j;
    const int row = ci / C::CH, part = ci % C::CH;
    st_row[j] = ci < TQ * C::CH && row < tq_rows;
    st_off[j] = (row / G) * (int32_t)ld_stride * 2 + (row % G) * (D * 2) + part * 16;
    stg[j] = (u32x4){0, 0, 0, 0};
  }
  __bf16 aq0 = 0, aq1 = 0, ao0 = 0, ao1 = 0;  // augmented values of row tid (tid < TQ)
  auto load_tile = [&](const QRun& r) {
    const int32_t ntok = r.t_end - r.t0 < TQT ? r.t_end - r.t0 : TQT;
    const int32_t rec = (ntok - 1) * (int32_t)ld_stride * 2 + G * (D * 2);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(ld_base + (int64_t)r.t0 * ld_stride), (short)0, rec, kBufCfg);
#pragma unroll
    for (int j = 0; j < NCH; ++j)
      if (st_row[j]) stg[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, st_off[j], 0, 0));
    aq0 = aq1 = ao0 = ao1 = (__bf16)0.0f;
    if (tid < tq_rows && tid / G < ntok) {
      const int64_t tok = r.t0 + tid / G;
      const int64_t idx = tok * a.hq + g * G + tid % G;
      float l2 = a.lse[idx] * kLog2e;
      if ((__float_as_uint(l2) & 0x7f800000u) == 0x7f800000u) l2 = 0.f;  // no key: -inf (bit test)
      split_bf16(-l2 * cinv, aq0, aq1);
      split_bf16(-a.delta[idx], ao0, ao1);
    }
  };
  auto store_tile = [&](int b) {
    __bf16* tile = ldq ? Qs[b] : Os[b];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int ci = (tid & 127) + 128 * j;
      if (ci < TQ * C::CH) {
        const int row = ci / C::CH, part = ci % C::CH;
        *reinterpret_cast<u32x4*>(&tile[row * QP + part * 8]) = stg[j];
      }
    }
    if (tid < TQ) {
      Qs[b][tid * QP + D] = aq0;
      Qs[b][tid * QP + D + 1] = aq1;
      Os[b][tid * QP + D] = ao0;
      Os[b][tid * QP + D + 1] = ao1;
    }
  };

  // DMA: load k of a wave fills the 64 slots from 64 J, J = (wave & 1) +
  // 2 k; slot s is row s / NC, and its chunk the one tile_swizzle puts
  // there; slots of no data (chunks >= D / 8, rows past tq_rows when G
  // does not divide TQ) take an offset past any range.
  constexpr int32_t kPastRange = 0x7ffffff0;
  int32_t ld_off[LPW];
#pragma unroll
  for (int k = 0; k < LPW; ++k) {
    const int J = (wave & 1) + 2 * k;
    const int sl = 64 * J + lane;
    const int row = sl / NC, part = (sl % NC) ^ tile_swizzle(sl / NC);
    ld_off[k] = part < C::CH && row < tq_rows
                    ? (row / G) * (int32_t)ld_stride * 2 + (row % G) * (D * 2) + part * 16
                    : kPastRange;
  }
  auto issue_tile = [&](const QRun& r, int b) {
    const int32_t ntok = r.t_end - r.t0 < TQT ? r.t_end - r.t0 : TQT;
    const int32_t rec = (ntok - 1) * (int32_t)ld_stride * 2 + G * (D * 2);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(ld_base + (int64_t)r.t0 * ld_stride), (short)0, rec, kBufCfg);
    __bf16* tile = ldq ? Qs[b] : Os[b];
#pragma unroll
    for (int k = 0; k < LPW; ++k) {
      const int J = (wave & 1) + 2 * k;
      load_lds16(rs, tile + J * 64 * 8, ld_off[k]);
    }
  };
  // accumulator initial values of row tid (tid < TQ) of a tile: loaded when
  // its slots are issued, written to LDS at the end of the tile being computed
  float aug_lse = 0.f, aug_delta = 0.f;
  bool aug_ok = false;
  auto load_aug = [&](const QRun& r) {
    const int32_t ntok = r.t_end - r.t0 < TQT ? r.t_end - r.t0 : TQT;
    aug_ok = tid < tq_rows && tid / G < ntok;
    if (aug_ok) {
      const int64_t idx = ((int64_t)r.t0 + tid / G) * a.hq + g * G + tid % G;
      aug_lse = a.lse[idx];
      aug_delta = a.delta[idx];
    }
  };
  auto store_aug = [&](int b) {
    if (tid < TQ) {
      float q = 0.f, o = 0.f;
      if (aug_ok) {
        float l2 = aug_lse * kLog2e;
        if ((__float_as_uint(l2) & 0x7f800000u) == 0x7f800000u) l2 = 0.f;  // no key: -inf (bit test)
        q = PRESCALED ? -l2 : -l2 * cinv;
        o = -aug_delta;
      }
      Qa[b][tid] = q;
      Oa[b][tid] = o;
    }
  };
  // End of a tile: this wave's LPW loads of the tile after next may stay in
  // flight (issued last, so they are the youngest vmcnt entries), all older
  // ones (the next tile's slots) must have landed; then the barrier makes
  // every wave's slots and augmented values visible.  A plain s_barrier: a
  // release fence would wait for the young loads too.
  auto end_tile = [&](bool pending) {
    // s_waitcnt: vmcnt(n) in bits 3:0, expcnt 7 (no wait), lgkmcnt(0)
    if (pending)
      __builtin_amdgcn_s_waitcnt(0x70 | LPW);
    else
      __builtin_amdgcn_s_waitcnt(0x70);
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
  };
  static_assert(LPW <= 15 && NW == 4, "vmcnt field; two waves per tile");
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

  QRun cur, nxt;
  find_qrun(SliceLists{a.slices, a.num_slices, a.k_tile_slices, a.num_k_tile_slices}, wi.slice_end, (int32_t)a.nq,
            (int32_t)a.nk, wi.slice_begin, k0, k1, w_lo, w_hi, cur);
  if constexpr (DMA) {
    next_run(cur, nxt);
    if (cur.valid) issue_tile(cur, 0);
    if (nxt.valid) issue_tile(nxt, 1);
    if (cur.valid) {
      load_aug(cur);
      store_aug(0);
    }
    if (nxt.valid) {
      load_aug(nxt);
      store_aug(1);
    }
    end_tile(false);
  } else {
    if (cur.valid) {
      load_tile(cur);
      store_tile(0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
  }
  int buf = 0;
  while (cur.valid) {
    QRun nx2;
    int buf2 = 0;
    if constexpr (DMA) {
      next_run(nxt, nx2);
      buf2 = buf == 0 ? 2 : buf - 1;  // (buf + 2) mod 3
      if (nx2.valid) {
        load_aug(nx2);
        issue_tile(nx2, buf2);  // in flight during this tile and the next
      }
    } else {
      next_run(cur, nxt);
      if (nxt.valid) load_tile(nxt);  // in flight while this tile is computed
    }
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
    const float* Qab = Qa[buf];
    const float* Oab = Oa[buf];
    const __attribute__((address_space(3))) __bf16* Qt = (const __attribute__((address_space(3))) __bf16*)Qs[buf];
    const __attribute__((address_space(3))) __bf16* Ot = (const __attribute__((address_space(3))) __bf16*)Os[buf];
#pragma unroll
    for (int rb = 0; rb < TQ / 32; ++rb) {
      // S' = Q' . K^T - LSE2 and dP' = dO' . V^T - delta (rows on M, keys
      // on N); the A operands are read once for all KB key blocks.  DMA: the
      // accumulators start from the rows' values (element i holds row
      // 8 (i / 4) + 4 h + i % 4 of this 32-row block, so 4 b128 reads each);
      // registers: from zero, the values riding in the augmented columns
      f32x16 s[KB], dp[KB];
      if constexpr (!DMA) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) s[kb] = dp[kb] = (f32x16){};
      } else {
        f32x16 s0, d0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 x = *reinterpret_cast<const float4*>(&Qab[rb * 32 + 8 * q + 4 * h]);
          const float4 y = *reinterpret_cast<const float4*>(&Oab[rb * 32 + 8 * q + 4 * h]);
          s0[4 * q] = x.x, s0[4 * q + 1] = x.y, s0[4 * q + 2] = x.z, s0[4 * q + 3] = x.w;
          d0[4 * q] = y.x, d0[4 * q + 1] = y.y, d0[4 * q + 2] = y.z, d0[4 * q + 3] = y.w;
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) s[kb] = s0, dp[kb] = d0;
      }
      static_assert(!DMA || D % 16 == 0, "direct-loaded tiles hold whole k-steps");
#pragma unroll
      for (int ks = 0; ks < KQ; ++ks) {
        // columns 16 ks + 8 h .. + 7: tile data below D; registers: the
        // augmented pair at D, D + 1, zeros above
        const int row = rb * 32 + ln;
        bf16x8 qa, oa;
        if (!DMA) {
          qa = *reinterpret_cast<const bf16x8*>(&Qb[row * QP + 16 * ks + 8 * h]);
          oa = *reinterpret_cast<const bf16x8*>(&Ob[row * QP + 16 * ks + 8 * h]);
        } else {
          const int col = ((2 * ks + h) ^ tile_swizzle(row)) * 8;
          qa = *reinterpret_cast<const bf16x8*>(&Qb[row * QP + col]);
          oa = *reinterpret_cast<const bf16x8*>(&Ob[row * QP + col]);
        }
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
        // t sees k < koff + t + 1).  With both clamped to [0, TQT] that is
        // lo G <= row < hi G, one unsigned compare of row - lo G against
        // (hi - lo) G, with no per-row constants kept across tiles.
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const bool kin = kvalid[kb] && key[kb] >= cur.ks && key[kb] < cur.ke;
          int32_t hi = kin ? ntok : 0;
          if (cur.type & MAGI_MASK_INVCAUSAL) {
            const int32_t e = key[kb] - cur.loff - cur.t0 + 1;
            hi = e < hi ? e : hi;
          }
          int32_t lo = (cur.type & MAGI_MASK_CAUSAL) ? key[kb] - cur.koff - cur.t0 : 0;
          lo = lo < 0 ? 0 : (lo > TQT ? TQT : lo);
          hi = hi < lo ? lo : hi;  // hi <= ntok <= TQT
          const int32_t off = rb * 32 + 4 * h - lo * G;
          const uint32_t span = (uint32_t)((hi - lo) * G);
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if ((uint32_t)(off + 8 * (i / 4) + (i % 4)) >= span) s[kb][i] = -INFINITY;
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
          bf16x8 ot8, qt8;
          if constexpr (DMA) {
            // rows qrow and qrow + 8, each with its own chunk permutation
            const int lo = qrow * QP + (((dcol >> 3) ^ tile_swizzle(qrow)) << 3) + (dcol & 7);
            const int hi = (qrow + 8) * QP + (((dcol >> 3) ^ tile_swizzle(qrow + 8)) << 3) + (dcol & 7);
            ot8 = read_tr8_pair(Ot + lo, Ot + hi);
            qt8 = read_tr8_pair(Qt + lo, Qt + hi);
          } else {
            ot8 = read_tr8(Ot + qrow * QP + dcol, QP);
            qt8 = read_tr8(Qt + qrow * QP + dcol, QP);
          }
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            dv[kb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ot8, pb[kb][i2], dv[kb][mb], 0, 0, 0);
            dk[kb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qt8, dsb[kb][i2], dk[kb][mb], 0, 0, 0);
          }
        }
      }
    }
    if constexpr (DMA) {
      if (nx2.valid) store_aug(buf2);
      end_tile(nx2.valid);
      cur = nxt;
      nxt = nx2;
      buf = buf == 2 ? 0 : buf + 1;
    } else {
      if (nxt.valid) store_tile(buf ^ 1);
      lds_barrier();
      cur = nxt;
      buf ^= 1;
    }
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
  constexpr int64_t kSlot = 2 * kKeys * D;  // floats per slot
  constexpr int kAhead = 8;                 // slot loads in flight per thread
  // one thread per (dK | dV, key, 4 channels) of the tile, spread over
  // gridDim.y blocks; the parts are added in slot order, whatever the
  // batching of the loads
  const int n = 2 * r.key_len * Q4;
  const int i = blockIdx.y * 256 + threadIdx.x;
  if (i >= n) return;
  const int which = i / (r.key_len * Q4), rem = i % (r.key_len * Q4);
  const int kr = rem / Q4, d = 4 * (rem % Q4);
  const float* src = a.partial + (int64_t)r.slot_begin * kSlot + (int64_t)which * kKeys * D + (int64_t)kr * D + d;
  float4 acc = *reinterpret_cast<const float4*>(src);
  int sl = 1;
  for (; sl + kAhead <= r.slot_count; sl += kAhead) {
    float4 x[kAhead];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) x[u] = *reinterpret_cast<const float4*>(src + (int64_t)(sl + u) * kSlot);
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      acc.x += x[u].x;
      acc.y += x[u].y;
      acc.z += x[u].z;
      acc.w += x[u].w;
    }
  }
  for (; sl < r.slot_count; ++sl) {
    const float4 x = *reinterpret_cast<const float4*>(src + (int64_t)sl * kSlot);
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

// The side stream and the two events that fork it from the caller's stream
// and join it back, one set per device, created on first use and kept until
// the process ends.  The lock spans a whole launch sequence, so that each
// wait pairs with the record just before it even when several host threads
// launch backward passes at once.
struct SideStream {
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxDevices = 64;
std::mutex g_side_mu;
SideStream g_side[kMaxDevices];

hipError_t side_stream_for(hipStream_t stream, SideStream** out) {
  int dev = 0;
  hipError_t e = stream != nullptr ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  SideStream& s = g_side[dev];
  if (s.side == nullptr) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    SideStream t;
    e = hipStreamCreateWithFlags(&t.side, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&t.fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&t.join, hipEventDisableTiming);
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (back != hipSuccess) return back;
    s = t;
  }
  *out = &s;
  return hipSuccess;
}

template <int D>
hipError_t launch_d(const BwdArgs& a, hipStream_t stream, bool two_streams) {
  constexpr int KB = D == 24 ? KB24 : KB48;
  constexpr int RBQ = D == 24 ? RBQ24 : RBQ48;
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
  auto dq_pass = [&](hipStream_t s) {
    const dim3 grid(a.num_qwork);
    if (!bf)
      hipLaunchKernelGGL((bwd_dq_f32<D>), grid, dim3(kThreads32), 0, s, a);
    else if (pre)
      hipLaunchKernelGGL((bwd_dq_bf16<D, true, RBQ>), grid, dim3(NT / RBQ), 0, s, a);
    else
      hipLaunchKernelGGL((bwd_dq_bf16<D, false, RBQ>), grid, dim3(NT / RBQ), 0, s, a);
  };
  // the dK/dV pass, then the sums of its split key tiles
  auto dkdv_pass = [&](hipStream_t s) {
    if (a.num_kwork > 0) {
      const dim3 grid(a.num_kwork);
      if (!bf)
        hipLaunchKernelGGL((bwd_dkdv_f32<D>), grid, dim3(kThreads32), 0, s, a);
      else if (pre)
        hipLaunchKernelGGL((bwd_dkdv_bf16<D, true, KB>), grid, dim3(2 * kKeys / KB), 0, s, a);
      else
        hipLaunchKernelGGL((bwd_dkdv_bf16<D, false, KB>), grid, dim3(2 * kKeys / KB), 0, s, a);
    }
    if (a.num_reduce > 0) {
      // gridDim.y covers the 2 x kKeys x D / 4 float4 outputs of a full tile
      const dim3 grid(a.num_reduce, (2 * kKeys * (D / 4) + 255) / 256);
      if (bf)
        hipLaunchKernelGGL((bwd_reduce<D, __bf16>), grid, dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL((bwd_reduce<D, float>), grid, dim3(256), 0, s, a);
    }
  };
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (two_streams && a.num_qwork > 0 && (a.num_kwork > 0 || a.num_reduce > 0)) {
    // The two passes read the same inputs and write disjoint outputs, so
    // they may run at once: the side stream takes the dK/dV pass after
    // delta, and `stream` waits for it after the dQ pass.
    std::lock_guard<std::mutex> lock(g_side_mu);
    SideStream* ss = nullptr;
    if ((e = side_stream_for(stream, &ss)) != hipSuccess) return e;
    if ((e = hipEventRecord(ss->fork, stream)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(ss->side, ss->fork, 0)) != hipSuccess) return e;
    dkdv_pass(ss->side);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = hipEventRecord(ss->join, ss->side)) != hipSuccess) return e;
    dq_pass(stream);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return hipStreamWaitEvent(stream, ss->join, 0);
  }
  if (a.num_qwork > 0) dq_pass(stream);
  dkdv_pass(stream);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffa_bwd(const BwdArgs& a, hipStream_t stream, bool two_streams) {
  return a.head_dim == 24 ? launch_d<24>(a, stream, two_streams) : launch_d<48>(a, stream, two_streams);
}

}  // namespace magi

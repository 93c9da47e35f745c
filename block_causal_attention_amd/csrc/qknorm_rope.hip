// QK-Norm + 3D RoPE prologue for gfx950.
//
// QK-Norm: each (token, head) vector is divided by its RMS over head_dim and
// scaled by a gain (MAGI-1 study notes, zhao9797.github.io, "自回归去噪 DiT",
// QK-Norm + GQA bullet; 量子位 article, "QK-Norm和GQA").  3D RoPE: head_dim is
// split into equal t / h / w sections; adjacent channel pairs of section a
// turn by pos_a * base_a^(-2j/(head_dim/3)), with a learnable base per axis
// (study notes, same section, Block-Causal Attention bullet; 量子位 article,
// "Block-Causal Attention").
//
// An optional output factor lets the caller fold the softmax scale (times
// log2 e) into K once here instead of into every score of the attention.
//
// The kernel is HBM-bound: it reads and writes each element once.  One block
// owns a run of whole tokens; the rotation table (cos, sin per token and
// channel pair) is shared by all heads of a token, so it is built once per
// token in LDS and every head of the token reads it.  Each thread then owns
// one (token, head) vector and moves it with 16-byte loads and stores.
//
// Outputs have a layout of their own: token-major ([n][heads][d]) like the
// inputs, or group-major ([heads][n][d]), where the attention reads each K/V
// tile of a group as one contiguous block.  A third side moves V into K's
// output layout unchanged, in the same launch.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace magi {
namespace {

constexpr int kThreads = 256;

template <typename T>
struct Vec;
template <>
struct Vec<__bf16> {
  static constexpr int kPerChunk = 8;  // elements per 16-byte chunk
};
template <>
struct Vec<float> {
  static constexpr int kPerChunk = 4;
};

__device__ inline float to_f32(__bf16 x) { return (float)x; }
__device__ inline float to_f32(float x) { return x; }
template <typename T>
__device__ inline T from_f32(float x) { return (T)x; }

template <int D, typename T>
__global__ __launch_bounds__(kThreads) void qknorm_rope_kernel(QkArgs a, int end_q, int end_k) {
  constexpr int P = D / 2;   // channel pairs
  constexpr int PS = D / 6;  // pairs per axis section
  constexpr int PC = Vec<T>::kPerChunk;
  constexpr int CHUNKS = D / PC;
  // blocks [0, end_q) take Q, [end_q, end_k) K, the rest V
  const int sidx = blockIdx.x < (unsigned)end_q ? 0 : (blockIdx.x < (unsigned)end_k ? 1 : 2);
  const QkSide& s = a.side[sidx];
  const int b = blockIdx.x - (sidx == 0 ? 0 : (sidx == 1 ? end_q : end_k));
  const int tpb = s.heads >= kThreads ? 1 : kThreads / s.heads;  // tokens per block
  const int64_t tok0 = (int64_t)b * tpb;
  if (tok0 >= s.n) return;
  const int ntok = (int)min<int64_t>(tpb, s.n - tok0);

  // first K block: bound on the norm of every output key of each head.
  // |x / rms(x) * g| <= sqrt(D) max|g| (the RMS step leaves norm sqrt(D)
  // at most, the rotation keeps norms), times |k_scale|, plus a margin for
  // the bf16 rounding of the stored keys.
  if (sidx == 1 && b == 0 && a.k_norm_max != nullptr) {
    for (int hh = threadIdx.x; hh < s.heads; hh += kThreads) {
      const float* gg = s.gain + (int64_t)hh * a.gain_head_stride;
      float gmax = 0.f;
      for (int i = 0; i < D; ++i) gmax = fmaxf(gmax, fabsf(gg[i]));
      a.k_norm_max[hh] = sqrtf((float)D) * gmax * fabsf(s.out_scale) * (1.0f + 1.0f / 128.0f);
    }
  }

  extern __shared__ float2 table[];  // [tpb][P] (cos, sin)
  // Consecutive threads take consecutive heads of a token when the output
  // is token-major, consecutive tokens of a head when it is group-major, so
  // that the stores of a wave cover contiguous memory either way.
  const bool group_out = s.out_head_stride != D;
  auto vec_of = [&](int v, int& t, int& h) {
    if (group_out) {
      t = v % ntok;
      h = v / ntok;
    } else {
      t = v / s.heads;
      h = v % s.heads;
    }
  };

  if (s.gain == nullptr) {
    // V: the same rows, moved into the output layout
    for (int v = threadIdx.x; v < ntok * s.heads; v += kThreads) {
      int t, h;
      vec_of(v, t, h);
      const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(s.in) + (tok0 + t) * s.tok_stride +
                                                        (int64_t)h * D);
      uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<T*>(s.out) + (tok0 + t) * s.out_tok_stride +
                                            (int64_t)h * s.out_head_stride);
#pragma unroll
      for (int c = 0; c < CHUNKS; ++c) dst[c] = src[c];
    }
    return;
  }

  // At d = 48 each thread's first vector is loaded before the rotation
  // table is built, so that its HBM latency overlaps the sin/cos work (a
  // block holds one vector per thread unless a token has more heads than
  // threads): 9 % less time on a 28,800-token layer.  At d = 24 the table is
  // half as long and the early load measured 5 % slower, so it loads late.
  constexpr bool kEarly = D >= 48;
  const int nvec = ntok * s.heads;
  auto load_vec = [&](int v, uint4 (&raw)[CHUNKS]) {
    int t, h;
    vec_of(v, t, h);
    const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(s.in) + (tok0 + t) * s.tok_stride +
                                                      (int64_t)h * D);
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) raw[c] = src[c];
  };
  uint4 cur[CHUNKS];
  if (kEarly && (int)threadIdx.x < nvec) load_vec(threadIdx.x, cur);

  for (int i = threadIdx.x; i < ntok * P; i += kThreads) {
    const int t = i / P, p = i % P;
    const int axis = p / PS, j = p % PS;
    // base^(-2j/(D/3)) = 2^(-(2j/(D/3)) * log2(base))
    const float inv = exp2f(-(float)(2 * j) / (float)(D / 3) * log2f(a.rope_base[axis]));
    const float theta = (float)s.pos[(tok0 + t) * 3 + axis] * inv;
    float sn, cs;
    sincosf(theta, &sn, &cs);
    table[t * P + p] = make_float2(cs, sn);
  }
  __syncthreads();

  for (int v = threadIdx.x; v < nvec; v += kThreads) {
    int t, h;
    vec_of(v, t, h);
    T* dst = reinterpret_cast<T*>(s.out) + (tok0 + t) * s.out_tok_stride + (int64_t)h * s.out_head_stride;
    float x[D];
    auto unpack = [&](const uint4& raw, int c) {
      const T* e = reinterpret_cast<const T*>(&raw);
#pragma unroll
      for (int i = 0; i < PC; ++i) x[c * PC + i] = to_f32(e[i]);
    };
    if constexpr (kEarly) {
      if (v != (int)threadIdx.x) load_vec(v, cur);
#pragma unroll
      for (int c = 0; c < CHUNKS; ++c) unpack(cur[c], c);
    } else {
      const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(s.in) + (tok0 + t) * s.tok_stride +
                                                        (int64_t)h * D);
#pragma unroll
      for (int c = 0; c < CHUNKS; ++c) unpack(src[c], c);
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < D; ++i) ss = fmaf(x[i], x[i], ss);
    const float r = 1.0f / sqrtf(ss / (float)D + a.eps) * s.out_scale;
    const float* g = s.gain + (int64_t)h * a.gain_head_stride;
#pragma unroll
    for (int i = 0; i < D; ++i) x[i] = x[i] * r * g[i];
    const float2* tb = table + t * P;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const float2 cs = tb[p];
      const float x0 = x[2 * p], x1 = x[2 * p + 1];
      x[2 * p] = x0 * cs.x - x1 * cs.y;
      x[2 * p + 1] = x0 * cs.y + x1 * cs.x;
    }
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) {
      uint4 raw;
      T* e = reinterpret_cast<T*>(&raw);
#pragma unroll
      for (int i = 0; i < PC; ++i) e[i] = from_f32<T>(x[c * PC + i]);
      reinterpret_cast<uint4*>(dst)[c] = raw;
    }
  }
}

template <int D, typename T>
hipError_t launch_typed(const QkArgs& a, hipStream_t stream) {
  int blocks[3] = {0, 0, 0};
  int tpb_max = 1;
  for (int i = 0; i < 3; ++i) {
    const QkSide& s = a.side[i];
    if (s.n == 0) continue;
    const int tpb = s.heads >= kThreads ? 1 : kThreads / s.heads;
    tpb_max = tpb > tpb_max ? tpb : tpb_max;
    blocks[i] = (int)((s.n + tpb - 1) / tpb);
  }
  const int total = blocks[0] + blocks[1] + blocks[2];
  if (total == 0) return hipSuccess;
  const size_t lds = (size_t)tpb_max * (D / 2) * sizeof(float2);
  hipLaunchKernelGGL((qknorm_rope_kernel<D, T>), dim3(total), dim3(kThreads), lds, stream, a, blocks[0],
                     blocks[0] + blocks[1]);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qknorm_rope(const QkArgs& a, hipStream_t stream) {
  const bool bf = a.dtype == MAGI_DTYPE_BF16;
  if (a.head_dim == 24) return bf ? launch_typed<24, __bf16>(a, stream) : launch_typed<24, float>(a, stream);
  return bf ? launch_typed<48, __bf16>(a, stream) : launch_typed<48, float>(a, stream);
}

}  // namespace magi

// Launch interfaces of the HIP kernels of libmagi_bca (internal).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "magi_bca.h"

namespace magi {

struct QkSide {
  const void* in;
  void* out;
  int64_t n;           // tokens
  int32_t heads;
  int64_t tok_stride;  // input: elements between consecutive tokens (heads contiguous)
  int64_t out_tok_stride, out_head_stride;  // output layout
  const float* gain;   // nullptr: plain copy into the output layout (V)
  const int32_t* pos;  // [n][3]
  float out_scale;     // factor applied to the result before it is stored
};

struct QkArgs {
  QkSide side[3];  // Q, K, V (n == 0 to skip a side); V is only re-laid out
  float* k_norm_max;  // device [hkv] out: bound on the norm of every output key of a group, or nullptr
  int32_t head_dim;
  int32_t dtype;
  int32_t gain_head_stride;
  float eps;
  const float* rope_base;
};

hipError_t launch_qknorm_rope(const QkArgs& a, hipStream_t stream);

struct FfaArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  int64_t nq, nk;
  int32_t hq, hkv, head_dim, dtype;
  int64_t q_stride, kv_stride, o_stride;
  int64_t kv_hstride;  // elements between consecutive KV heads of K and V
  float scale;
  const float* k_norm_max;  // device [hkv] upper bounds on key norms, or nullptr
  // QK-Norm + 3D RoPE of Q done in the kernel (q is then the raw Q): gain
  // [d] or [hq][d], positions [nq][3], rope base [3]; q_hat (or nullptr)
  // receives the normalised, rotated Q
  const float* qn_gain;  // nullptr: q is used as given
  int32_t qn_gain_hstride;
  float qn_eps, qn_scale;
  const int32_t* qn_pos;
  const float* qn_base;
  void* q_hat;
  int64_t q_hat_stride;
  const magi_attn_slice* slices;
  int32_t num_slices;
  const magi_work_item* work;
  int32_t num_work;
  const int32_t* tile_slices;
  int32_t num_tile_slices;
};

// With start/stop events the dispatch itself records them when the kernel
// starts and when it completes (no marker packets of their own).
hipError_t launch_ffa_fwd(const FfaArgs& a, hipStream_t stream, hipEvent_t start = nullptr,
                          hipEvent_t stop = nullptr);

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // [nq][hq] rowsum(dout * out), written first
  int64_t nq, nk;
  int32_t hq, hkv, head_dim, dtype;
  int64_t q_stride, kv_stride, o_stride;
  int64_t kv_hstride;  // elements between consecutive KV heads of K, V, dK, dV
  float scale;
  const magi_attn_slice* slices;
  int32_t num_slices;
  const magi_work_item* qwork;   // query-major items (magi_schedule)
  int32_t num_qwork;
  const int32_t* q_tile_slices;
  int32_t num_q_tile_slices;
  const magi_work_item* kwork;   // key-major items (magi_schedule_kv)
  int32_t num_kwork;
  const int32_t* k_tile_slices;
  int32_t num_k_tile_slices;
  const int32_t* kitem_ext;      // [num_kwork][3] {partial slot or -1, token window lo, hi} per key-major item
  const magi_kv_reduce* reduce;  // sums of the partial slots
  int32_t num_reduce;
  int32_t num_slots;
  float* partial;                // [num_slots][2][kKeys][head_dim] fp32 (dK, then dV)
};

// With two_streams the dK/dV pass and its reduce run on a side stream of the
// library (one per device, default priority, created on first use) beside
// the dQ pass on `stream`; `stream` waits for them before it returns to the
// caller's later work.  Without, all launches go to `stream` in order.
hipError_t launch_ffa_bwd(const BwdArgs& a, hipStream_t stream, bool two_streams = false);

// The static device workspace of the entry points that allocate nothing:
// kScratchFloats fp32 values (64 MiB) per GPU, held until the process ends.
constexpr int64_t kScratchFloats = (int64_t)16 << 20;

// Device address of the workspace on the device of `stream` (a hipStream_t;
// NULL = the current device), looked up once per device.
hipError_t scratch_for_stream(void* stream, float** out);

}  // namespace magi

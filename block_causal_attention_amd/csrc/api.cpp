// C entry points of the device half of libmagi_bca: argument validation on
// the host (before any HIP call), then one kernel launch on the caller's
// stream.  The library allocates nothing and never synchronises.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "kernels.h"
#include "status.h"

using namespace magi;

namespace {

// Finite test on the bit pattern: no floating-point compile option (the
// device pass of this file assumes no NaN) can fold it away.
inline bool finite_bits(float x) {
  uint32_t u;
  std::memcpy(&u, &x, sizeof u);
  return (u & 0x7f800000u) != 0x7f800000u;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_size(int32_t dtype) { return dtype == MAGI_DTYPE_BF16 ? 2 : 4; }

int32_t check_common(int32_t head_dim, int32_t dtype) {
  if (dtype != MAGI_DTYPE_BF16 && dtype != MAGI_DTYPE_FP32) return fail(MAGI_ERR_INVALID_ARG, "bad dtype %d", dtype);
  if (head_dim != 24 && head_dim != 48)
    return fail(MAGI_ERR_UNSUPPORTED, "head_dim %d unsupported (24 or 48)", head_dim);
  return MAGI_OK;
}

// A tensor of n tokens x heads vectors of head_dim contiguous elements; the
// vector of (token i, head h) starts at element i * tok_stride + h * head_stride.
// Vectors must not overlap: either the heads of a token sit side by side
// (head_stride >= head_dim, tok_stride >= heads * head_stride: token-major)
// or the tokens of a head do (tok_stride >= head_dim, head_stride >=
// n * tok_stride: group-major).
int32_t check_layout(const char* name, const void* p, int64_t n, int32_t heads, int64_t tok_stride,
                     int64_t head_stride, int32_t head_dim, int32_t dtype) {
  if (n < 0 || n > INT32_MAX) return fail(MAGI_ERR_INVALID_ARG, "%s: row count %lld not in [0, 2^31)", name, (long long)n);
  if (heads < 1) return fail(MAGI_ERR_INVALID_ARG, "%s: heads %d < 1", name, heads);
  const bool token_major = head_stride >= head_dim && tok_stride >= (int64_t)heads * head_stride;
  const bool group_major = tok_stride >= head_dim && head_stride >= n * tok_stride;
  if (!token_major && !group_major)
    return fail(MAGI_ERR_INVALID_ARG,
                "%s: strides (token %lld, head %lld) make vectors overlap (need token-major or group-major)", name,
                (long long)tok_stride, (long long)head_stride);
  if ((tok_stride * elem_size(dtype)) % 16 || (head_stride * elem_size(dtype)) % 16)
    return fail(MAGI_ERR_INVALID_ARG, "%s: strides must be multiples of 16 bytes", name);
  if (n > 0 && p == nullptr) return fail(MAGI_ERR_INVALID_ARG, "%s is NULL", name);
  if (n > 0 && !aligned16(p)) return fail(MAGI_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return MAGI_OK;
}

// token-major with the heads of a token contiguous
int32_t check_tensor(const char* name, const void* p, int64_t n, int32_t heads, int64_t stride, int32_t head_dim,
                     int32_t dtype) {
  if (stride < (int64_t)heads * head_dim)
    return fail(MAGI_ERR_INVALID_ARG, "%s: row stride %lld < heads*head_dim = %lld", name, (long long)stride,
                (long long)heads * head_dim);
  return check_layout(name, p, n, heads, stride, head_dim, head_dim, dtype);
}

}  // namespace

extern "C" int32_t magi_qknorm_rope(const void* q_in, void* q_out, int64_t nq, int32_t hq, int64_t q_tok_stride,
                                    const void* k_in, void* k_out, int64_t nk, int32_t hkv, int64_t k_tok_stride,
                                    int64_t k_out_tok_stride, int64_t k_out_head_stride, const void* v_in,
                                    void* v_out, int32_t head_dim, int32_t dtype, const float* gain_q, const float* gain_k,
                                    int32_t gain_head_stride, float eps, const int32_t* pos_q,
                                    const int32_t* pos_k, const float* rope_base, float q_scale, float k_scale,
                                    float* k_norm_max, void* stream) {
  int32_t st;
  if ((st = check_common(head_dim, dtype)) != MAGI_OK) return st;
  if ((st = check_tensor("q_in", q_in, nq, hq, q_tok_stride, head_dim, dtype)) != MAGI_OK) return st;
  if ((st = check_tensor("q_out", q_out, nq, hq, q_tok_stride, head_dim, dtype)) != MAGI_OK) return st;
  if ((v_in == nullptr) != (v_out == nullptr)) return fail(MAGI_ERR_INVALID_ARG, "v_in and v_out go together");
  if (nk > 0) {
    if ((st = check_tensor("k_in", k_in, nk, hkv, k_tok_stride, head_dim, dtype)) != MAGI_OK) return st;
    if ((st = check_layout("k_out", k_out, nk, hkv, k_out_tok_stride, k_out_head_stride, head_dim, dtype)) != MAGI_OK)
      return st;
    if (k_out == k_in && (k_out_tok_stride != k_tok_stride || k_out_head_stride != head_dim))
      return fail(MAGI_ERR_INVALID_ARG, "k_out may alias k_in only with the same layout");
    if (v_in != nullptr) {
      if ((st = check_tensor("v_in", v_in, nk, hkv, k_tok_stride, head_dim, dtype)) != MAGI_OK) return st;
      if ((st = check_layout("v_out", v_out, nk, hkv, k_out_tok_stride, k_out_head_stride, head_dim, dtype)) !=
          MAGI_OK)
        return st;
      if (v_out == v_in) return fail(MAGI_ERR_INVALID_ARG, "v_out must not alias v_in");
    }
    if (gain_k == nullptr || pos_k == nullptr) return fail(MAGI_ERR_INVALID_ARG, "gain_k / pos_k is NULL");
  } else if (nk < 0) {
    return fail(MAGI_ERR_INVALID_ARG, "nk < 0");
  } else if (v_in != nullptr) {
    return fail(MAGI_ERR_INVALID_ARG, "v_in needs K (nk > 0)");
  }
  if (nq > 0 && (gain_q == nullptr || pos_q == nullptr)) return fail(MAGI_ERR_INVALID_ARG, "gain_q / pos_q is NULL");
  if (gain_head_stride != 0 && gain_head_stride != head_dim)
    return fail(MAGI_ERR_INVALID_ARG, "gain_head_stride must be 0 or head_dim");
  if (!(eps >= 0.f) || !finite_bits(eps)) return fail(MAGI_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (rope_base == nullptr) return fail(MAGI_ERR_INVALID_ARG, "rope_base is NULL");
  if (!finite_bits(q_scale) || !finite_bits(k_scale) || q_scale == 0.f || k_scale == 0.f)
    return fail(MAGI_ERR_INVALID_ARG, "q_scale and k_scale must be finite and non-zero");

  QkArgs a{};
  a.side[0] = {q_in, q_out, nq, hq, q_tok_stride, q_tok_stride, head_dim, gain_q, pos_q, q_scale};
  a.side[1] = {k_in, k_out, nk > 0 ? nk : 0, nk > 0 ? hkv : 1, k_tok_stride, k_out_tok_stride, k_out_head_stride,
               gain_k, pos_k, k_scale};
  a.side[2] = {v_in, v_out, nk > 0 && v_in != nullptr ? nk : 0, nk > 0 ? hkv : 1, k_tok_stride, k_out_tok_stride,
               k_out_head_stride, nullptr, nullptr, 1.0f};
  a.head_dim = head_dim;
  a.dtype = dtype;
  a.gain_head_stride = gain_head_stride;
  a.eps = eps;
  a.rope_base = rope_base;
  if (k_norm_max != nullptr && nk == 0)
    return fail(MAGI_ERR_INVALID_ARG, "k_norm_max needs K (nk > 0)");
  if (k_norm_max != nullptr && (reinterpret_cast<uintptr_t>(k_norm_max) & 3u))
    return fail(MAGI_ERR_INVALID_ARG, "k_norm_max is not 4-byte aligned");
  a.k_norm_max = k_norm_max;
  const hipError_t e = launch_qknorm_rope(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MAGI_ERR_HIP, "qknorm_rope launch: %s", hipGetErrorString(e));
  return ok();
}

namespace {

int32_t ffa_fwd_args(FfaArgs& a, const void* q, const void* k, const void* v, void* out, float* lse, int64_t nq,
                                int64_t nk, int32_t hq, int32_t hkv, int32_t head_dim, int32_t dtype,
                                int64_t q_tok_stride, int64_t kv_tok_stride, int64_t kv_head_stride,
                                int64_t o_tok_stride, float softmax_scale, const float* k_norm_max,
                                const magi_attn_slice* slices,
                                int32_t num_slices,
                                const magi_work_item* work, int32_t num_work, const int32_t* tile_slices,
                                int32_t num_tile_slices) {
  int32_t st;
  if ((st = check_common(head_dim, dtype)) != MAGI_OK) return st;
  if (hq < 1 || hkv < 1) return fail(MAGI_ERR_INVALID_ARG, "hq and hkv must be >= 1");
  if (hq % hkv) return fail(MAGI_ERR_INVALID_ARG, "hq %% hkv != 0 (hq=%d hkv=%d)", hq, hkv);
  if (hq / hkv > 256) return fail(MAGI_ERR_UNSUPPORTED, "group size %d > 256", hq / hkv);
  if ((st = check_tensor("q", q, nq, hq, q_tok_stride, head_dim, dtype)) != MAGI_OK) return st;
  if ((st = check_tensor("out", out, nq, hq, o_tok_stride, head_dim, dtype)) != MAGI_OK) return st;
  if ((st = check_layout("k", k, nk, hkv, kv_tok_stride, kv_head_stride, head_dim, dtype)) != MAGI_OK) return st;
  if ((st = check_layout("v", v, nk, hkv, kv_tok_stride, kv_head_stride, head_dim, dtype)) != MAGI_OK) return st;
  // the kernel addresses one K/V tile with 32-bit byte offsets
  if (kv_tok_stride >= (int64_t)1 << 23)
    return fail(MAGI_ERR_UNSUPPORTED, "kv row stride %lld >= 2^23 elements", (long long)kv_tok_stride);
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(MAGI_ERR_INVALID_ARG, "lse is not 4-byte aligned");
  if (!finite_bits(softmax_scale))
    return fail(MAGI_ERR_INVALID_ARG, "softmax_scale must be finite");
  if (k_norm_max != nullptr && (reinterpret_cast<uintptr_t>(k_norm_max) & 3u))
    return fail(MAGI_ERR_INVALID_ARG, "k_norm_max is not 4-byte aligned");
  if (num_slices < 0 || num_work < 0 || num_tile_slices < 0)
    return fail(MAGI_ERR_INVALID_ARG, "negative list length");
  if ((num_slices > 0 && slices == nullptr) || (num_work > 0 && work == nullptr) ||
      (num_tile_slices > 0 && tile_slices == nullptr))
    return fail(MAGI_ERR_INVALID_ARG, "a non-empty list pointer is NULL");
  if (num_work > 0 && nq == 0) return fail(MAGI_ERR_INVALID_ARG, "work items given for an empty query tensor");

  a = FfaArgs{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.nq = nq;
  a.nk = nk;
  a.hq = hq;
  a.hkv = hkv;
  a.head_dim = head_dim;
  a.dtype = dtype;
  a.q_stride = q_tok_stride;
  a.kv_stride = kv_tok_stride;
  a.kv_hstride = kv_head_stride;
  a.o_stride = o_tok_stride;
  a.scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
  a.k_norm_max = dtype == MAGI_DTYPE_BF16 ? k_norm_max : nullptr;
  a.slices = slices;
  a.num_slices = num_slices;
  a.work = work;
  a.num_work = num_work;
  a.tile_slices = tile_slices;
  a.num_tile_slices = num_tile_slices;
  return MAGI_OK;
}

int32_t launch(const FfaArgs& a, void* stream, void* start = nullptr, void* stop = nullptr) {
  const hipError_t e = launch_ffa_fwd(a, reinterpret_cast<hipStream_t>(stream), reinterpret_cast<hipEvent_t>(start),
                                      reinterpret_cast<hipEvent_t>(stop));
  if (e != hipSuccess) return fail(MAGI_ERR_HIP, "ffa_fwd launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" int32_t magi_ffa_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int64_t nq,
                                int64_t nk, int32_t hq, int32_t hkv, int32_t head_dim, int32_t dtype,
                                int64_t q_tok_stride, int64_t kv_tok_stride, int64_t kv_head_stride,
                                int64_t o_tok_stride, float softmax_scale, const float* k_norm_max,
                                const magi_attn_slice* slices, int32_t num_slices, const magi_work_item* work,
                                int32_t num_work, const int32_t* tile_slices, int32_t num_tile_slices,
                                void* stream) {
  FfaArgs a;
  const int32_t st = ffa_fwd_args(a, q, k, v, out, lse, nq, nk, hq, hkv, head_dim, dtype, q_tok_stride,
                                  kv_tok_stride, kv_head_stride, o_tok_stride, softmax_scale, k_norm_max, slices,
                                  num_slices, work, num_work, tile_slices, num_tile_slices);
  if (st != MAGI_OK) return st;
  return launch(a, stream);
}

extern "C" int32_t magi_ffa_fwd_timed(const void* q, const void* k, const void* v, void* out, float* lse,
                                      int64_t nq, int64_t nk, int32_t hq, int32_t hkv, int32_t head_dim,
                                      int32_t dtype, int64_t q_tok_stride, int64_t kv_tok_stride,
                                      int64_t kv_head_stride, int64_t o_tok_stride, float softmax_scale,
                                      const float* k_norm_max, const magi_attn_slice* slices, int32_t num_slices,
                                      const magi_work_item* work, int32_t num_work, const int32_t* tile_slices,
                                      int32_t num_tile_slices, void* stream, void* start_event, void* stop_event) {
  FfaArgs a;
  const int32_t st = ffa_fwd_args(a, q, k, v, out, lse, nq, nk, hq, hkv, head_dim, dtype, q_tok_stride,
                                  kv_tok_stride, kv_head_stride, o_tok_stride, softmax_scale, k_norm_max, slices,
                                  num_slices, work, num_work, tile_slices, num_tile_slices);
  if (st != MAGI_OK) return st;
  return launch(a, stream, start_event, stop_event);
}

extern "C" int32_t magi_ffa_fwd_qknorm(const void* q_raw, const void* k, const void* v, void* out, float* lse,
                                       int64_t nq, int64_t nk, int32_t hq, int32_t hkv, int32_t head_dim,
                                       int32_t dtype, int64_t q_tok_stride, int64_t kv_tok_stride,
                                       int64_t kv_head_stride, int64_t o_tok_stride, float softmax_scale,
                                       const float* k_norm_max, const magi_attn_slice* slices, int32_t num_slices,
                                       const magi_work_item* work, int32_t num_work, const int32_t* tile_slices,
                                       int32_t num_tile_slices, const float* gain_q, int32_t gain_head_stride,
                                       float eps, const int32_t* pos_q, const float* rope_base, float q_scale,
                                       void* q_hat, int64_t q_hat_stride, void* stream) {
  FfaArgs a;
  int32_t st = ffa_fwd_args(a, q_raw, k, v, out, lse, nq, nk, hq, hkv, head_dim, dtype, q_tok_stride,
                            kv_tok_stride, kv_head_stride, o_tok_stride, softmax_scale, k_norm_max, slices,
                            num_slices, work, num_work, tile_slices, num_tile_slices);
  if (st != MAGI_OK) return st;
  if (dtype != MAGI_DTYPE_BF16) return fail(MAGI_ERR_UNSUPPORTED, "the fused Q prologue is bf16 only");
  if (nq > 0 && (gain_q == nullptr || pos_q == nullptr || rope_base == nullptr))
    return fail(MAGI_ERR_INVALID_ARG, "gain_q / pos_q / rope_base is NULL");
  if (gain_head_stride != 0 && gain_head_stride != head_dim)
    return fail(MAGI_ERR_INVALID_ARG, "gain_head_stride must be 0 or head_dim");
  if (!(eps >= 0.f) || !finite_bits(eps)) return fail(MAGI_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (!finite_bits(q_scale) || q_scale == 0.f) return fail(MAGI_ERR_INVALID_ARG, "q_scale must be finite, non-zero");
  if (q_hat != nullptr && (st = check_tensor("q_hat", q_hat, nq, hq, q_hat_stride, head_dim, dtype)) != MAGI_OK)
    return st;
  a.qn_gain = gain_q;
  a.qn_gain_hstride = gain_head_stride;
  a.qn_eps = eps;
  a.qn_scale = q_scale;
  a.qn_pos = pos_q;
  a.qn_base = rope_base;
  a.q_hat = q_hat;
  a.q_hat_stride = q_hat_stride;
  return launch(a, stream);
}

namespace {

// Every check of the backward's arguments except its workspace (delta and
// the partial sums of split key tiles), then the kernel arguments.
int32_t bwd_args(BwdArgs& a, const void* q, const void* k, const void* v, const void* out, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, int64_t nq, int64_t nk, int32_t hq, int32_t hkv,
                 int32_t head_dim, int32_t dtype, int64_t q_tok_stride, int64_t kv_tok_stride,
                 int64_t kv_head_stride, int64_t o_tok_stride, float softmax_scale, const magi_attn_slice* slices,
                 int32_t num_slices, const magi_work_item* qwork, int32_t num_qwork, const int32_t* q_tile_slices,
                 int32_t num_q_tile_slices, const magi_work_item* kwork, int32_t num_kwork,
                 const int32_t* k_tile_slices, int32_t num_k_tile_slices, const int32_t* kitem_ext,
                 const magi_kv_reduce* reduce, int32_t num_reduce, int32_t num_slots) {
  int32_t st;
  if ((st = check_common(head_dim, dtype)) != MAGI_OK) return st;
  if (hq < 1 || hkv < 1) return fail(MAGI_ERR_INVALID_ARG, "hq and hkv must be >= 1");
  if (hq % hkv) return fail(MAGI_ERR_INVALID_ARG, "hq %% hkv != 0 (hq=%d hkv=%d)", hq, hkv);
  if (hq / hkv > 64) return fail(MAGI_ERR_UNSUPPORTED, "group size %d > 64", hq / hkv);
  const struct { const char* name; const void* p; int64_t n; int32_t heads; int64_t stride; } tensors[] = {
      {"q", q, nq, hq, q_tok_stride},        {"dq", dq, nq, hq, q_tok_stride},
      {"out", out, nq, hq, o_tok_stride},    {"dout", dout, nq, hq, o_tok_stride}};
  for (const auto& t : tensors)
    if ((st = check_tensor(t.name, t.p, t.n, t.heads, t.stride, head_dim, dtype)) != MAGI_OK) return st;
  const struct { const char* name; const void* p; } kv[] = {{"k", k}, {"v", v}, {"dk", dk}, {"dv", dv}};
  for (const auto& t : kv)
    if ((st = check_layout(t.name, t.p, nk, hkv, kv_tok_stride, kv_head_stride, head_dim, dtype)) != MAGI_OK) return st;
  if (kv_tok_stride >= (int64_t)1 << 23)
    return fail(MAGI_ERR_UNSUPPORTED, "kv row stride %lld >= 2^23 elements", (long long)kv_tok_stride);
  // the dK/dV pass addresses one Q/dO tile with 32-bit byte offsets
  if (q_tok_stride >= (int64_t)1 << 23 || o_tok_stride >= (int64_t)1 << 23)
    return fail(MAGI_ERR_UNSUPPORTED, "q or out row stride >= 2^23 elements");
  if (nq > 0 && lse == nullptr) return fail(MAGI_ERR_INVALID_ARG, "lse is required");
  if (reinterpret_cast<uintptr_t>(lse) & 3u) return fail(MAGI_ERR_INVALID_ARG, "lse not 4-byte aligned");
  if (!finite_bits(softmax_scale))
    return fail(MAGI_ERR_INVALID_ARG, "softmax_scale must be finite");
  if (num_slices < 0 || num_qwork < 0 || num_q_tile_slices < 0 || num_kwork < 0 || num_k_tile_slices < 0)
    return fail(MAGI_ERR_INVALID_ARG, "negative list length");
  if ((num_slices > 0 && slices == nullptr) || (num_qwork > 0 && qwork == nullptr) ||
      (num_q_tile_slices > 0 && q_tile_slices == nullptr) || (num_kwork > 0 && kwork == nullptr) ||
      (num_k_tile_slices > 0 && k_tile_slices == nullptr))
    return fail(MAGI_ERR_INVALID_ARG, "a non-empty list pointer is NULL");
  if (num_qwork > 0 && nq == 0) return fail(MAGI_ERR_INVALID_ARG, "query work items for an empty query tensor");
  if (num_reduce < 0 || num_slots < 0) return fail(MAGI_ERR_INVALID_ARG, "negative reduce or slot count");
  if ((num_reduce > 0 || num_slots > 0) && (reduce == nullptr || kitem_ext == nullptr))
    return fail(MAGI_ERR_INVALID_ARG, "a split schedule needs kitem_ext and reduce");
  if (num_kwork > 0 && nk == 0) return fail(MAGI_ERR_INVALID_ARG, "key work items for an empty key tensor");

  a = BwdArgs{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.nq = nq;
  a.nk = nk;
  a.hq = hq;
  a.hkv = hkv;
  a.head_dim = head_dim;
  a.dtype = dtype;
  a.q_stride = q_tok_stride;
  a.kv_stride = kv_tok_stride;
  a.kv_hstride = kv_head_stride;
  a.o_stride = o_tok_stride;
  a.scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
  a.slices = slices;
  a.num_slices = num_slices;
  a.qwork = qwork;
  a.num_qwork = num_qwork;
  a.q_tile_slices = q_tile_slices;
  a.num_q_tile_slices = num_q_tile_slices;
  a.kwork = kwork;
  a.num_kwork = num_kwork;
  a.k_tile_slices = k_tile_slices;
  a.num_k_tile_slices = num_k_tile_slices;
  a.kitem_ext = kitem_ext;
  a.reduce = reduce;
  a.num_reduce = num_reduce;
  a.num_slots = num_slots;
  return MAGI_OK;
}

// fp32 values of the partial-sum workspace a schedule with num_slots slots
// needs: 2 (dK, dV) x 128 keys x head_dim per slot, the dK/dV kernel's layout
int64_t partial_need(int32_t num_slots, int32_t head_dim) { return (int64_t)num_slots * 2 * 128 * head_dim; }

int32_t bwd_launch(const BwdArgs& a, void* stream, bool two_streams) {
  const hipError_t e = launch_ffa_bwd(a, reinterpret_cast<hipStream_t>(stream), two_streams);
  if (e != hipSuccess) return fail(MAGI_ERR_HIP, "ffa_bwd launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" int32_t magi_ffa_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                                const float* lse, void* dq, void* dk, void* dv, float* delta, int64_t nq,
                                int64_t nk, int32_t hq, int32_t hkv, int32_t head_dim, int32_t dtype,
                                int64_t q_tok_stride, int64_t kv_tok_stride, int64_t kv_head_stride,
                                int64_t o_tok_stride, float softmax_scale, const magi_attn_slice* slices,
                                int32_t num_slices, const magi_work_item* qwork, int32_t num_qwork,
                                const int32_t* q_tile_slices, int32_t num_q_tile_slices,
                                const magi_work_item* kwork, int32_t num_kwork, const int32_t* k_tile_slices,
                                int32_t num_k_tile_slices, const int32_t* kitem_ext,
                                const magi_kv_reduce* reduce, int32_t num_reduce, int32_t num_slots,
                                float* partial, int64_t partial_floats, void* stream) {
  BwdArgs a;
  int32_t st = bwd_args(a, q, k, v, out, dout, lse, dq, dk, dv, nq, nk, hq, hkv, head_dim, dtype, q_tok_stride,
                        kv_tok_stride, kv_head_stride, o_tok_stride, softmax_scale, slices, num_slices, qwork,
                        num_qwork, q_tile_slices, num_q_tile_slices, kwork, num_kwork, k_tile_slices,
                        num_k_tile_slices, kitem_ext, reduce, num_reduce, num_slots);
  if (st != MAGI_OK) return st;
  if (nq > 0 && delta == nullptr) return fail(MAGI_ERR_INVALID_ARG, "delta is required");
  if (reinterpret_cast<uintptr_t>(delta) & 3u) return fail(MAGI_ERR_INVALID_ARG, "delta not 4-byte aligned");
  if (num_reduce > 0 || num_slots > 0) {
    if (partial == nullptr) return fail(MAGI_ERR_INVALID_ARG, "a split schedule needs partial");
    if (partial_floats < partial_need(num_slots, head_dim))
      return fail(MAGI_ERR_INVALID_ARG, "partial holds %lld floats, %d slots need %lld", (long long)partial_floats,
                  num_slots, (long long)partial_need(num_slots, head_dim));
    if (!aligned16(partial)) return fail(MAGI_ERR_INVALID_ARG, "partial is not 16-byte aligned");
  }
  a.delta = delta;
  a.partial = partial;
  return bwd_launch(a, stream, true);
}

extern "C" int32_t magi_ffa_bwd_noalloc(const void* q, const void* k, const void* v, const void* out,
                                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                        int64_t nq, int64_t nk, int32_t hq, int32_t hkv, int32_t head_dim,
                                        int32_t dtype, int64_t q_tok_stride, int64_t kv_tok_stride,
                                        int64_t kv_head_stride, int64_t o_tok_stride, float softmax_scale,
                                        const magi_attn_slice* slices, int32_t num_slices,
                                        const magi_work_item* qwork, int32_t num_qwork,
                                        const int32_t* q_tile_slices, int32_t num_q_tile_slices,
                                        const magi_work_item* kwork, int32_t num_kwork,
                                        const int32_t* k_tile_slices, int32_t num_k_tile_slices,
                                        const int32_t* kitem_ext, const magi_kv_reduce* reduce,
                                        int32_t num_reduce, int32_t num_slots, void* stream) {
  BwdArgs a;
  int32_t st = bwd_args(a, q, k, v, out, dout, lse, dq, dk, dv, nq, nk, hq, hkv, head_dim, dtype, q_tok_stride,
                        kv_tok_stride, kv_head_stride, o_tok_stride, softmax_scale, slices, num_slices, qwork,
                        num_qwork, q_tile_slices, num_q_tile_slices, kwork, num_kwork, k_tile_slices,
                        num_k_tile_slices, kitem_ext, reduce, num_reduce, num_slots);
  if (st != MAGI_OK) return st;
  // delta first, then the partial sums from a 256-byte boundary
  const int64_t delta_floats = (nq * hq + 63) / 64 * 64;
  const int64_t need = delta_floats + partial_need(num_slots, head_dim);
  if (need > kScratchFloats)
    return fail(MAGI_ERR_UNSUPPORTED,
                "workspace of %lld floats (delta %lld + %d partial slots) exceeds the static %lld-float scratch",
                (long long)need, (long long)(nq * hq), num_slots, (long long)kScratchFloats);
  float* base = nullptr;
  const hipError_t e = scratch_for_stream(stream, &base);
  if (e != hipSuccess) return fail(MAGI_ERR_HIP, "scratch lookup: %s", hipGetErrorString(e));
  a.delta = base;
  a.partial = base + delta_floats;
  return bwd_launch(a, stream, false);
}

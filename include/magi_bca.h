/*
 * magi_bca.h -- block-causal GQA attention forward for AMD MI355X (gfx950).
 *
 * C ABI of libmagi_bca.so.  Plain pointers and sizes only.  Every pointer
 * argument is marked [host] or [device].  Device buffers are always owned by
 * the caller; the library never allocates device memory, never synchronises a
 * stream, and launches its kernels on the caller's hipStream_t (passed as
 * void*; NULL = the default stream).  Every argument is validated on the host
 * before the first HIP call, so argument errors never touch the GPU.
 *
 * Errors: each entry point returns MAGI_OK (0) or a negative magi_status;
 * magi_last_error() then returns a message for the calling thread.
 *
 * The operation is MAGI-1's attention as described on the MAGI-1 pages:
 *   - block-causal attention: full attention inside a chunk, causal across
 *     chunks (MAGI-1 study notes, zhao9797.github.io, "自回归去噪 DiT" and
 *     "整体 pipeline"; 量子位 article on dakule.com, "Block-Causal Attention");
 *   - GQA with 128 query heads over 8 KV groups and QK-Norm (study notes,
 *     "模型规格（Table 2）"; 量子位 article, "QK-Norm和GQA");
 *   - a 3D RoPE over (t, h, w) with a learnable base frequency (study notes,
 *     "自回归去噪 DiT"; 量子位 article, "Block-Causal Attention");
 *   - the mask written as a union of AttnSlices (q range, k range, full or
 *     causal), the Flex-Flash-Attention formulation (study notes, "训练
 *     Infra"; 量子位 article, "Flex-Flash-Attention"; interview with Zhang
 *     Zheng on zhengguannews.cn, answer on q_range / k_range);
 *   - packed videos that must not see each other, and a KV range that limits
 *     a chunk to its most recent predecessors (interview, same answer; study
 *     notes, "推理技巧", KV Cache bullet).
 */
#ifndef MAGI_BCA_H
#define MAGI_BCA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MAGI_OK = 0,
  MAGI_ERR_INVALID_ARG = -1,      /* null pointer, negative size, bad range, bad enum */
  MAGI_ERR_UNSUPPORTED = -2,      /* valid but not implemented (head_dim, group size, dtype) */
  MAGI_ERR_BUFFER_TOO_SMALL = -3, /* a host output array is shorter than needed */
  MAGI_ERR_OVERLAP = -4,          /* two slices list the same (q, k) pair */
  MAGI_ERR_HIP = -5               /* a HIP call failed (message has the HIP error) */
} magi_status;

/* Mask type of a slice.  The pages build every mask from full and causal
 * pieces and name sliding-window attention as the next mask form (interview
 * with Zhang Zheng, answer on FFA's mask types).  A token-level sliding
 * window needs a lower bound on the keys that moves with the row, which no
 * union of full and bottom-right causal rectangles gives; the two types
 * after CAUSAL add it (bit 0 of the type = the upper, bottom-right bound,
 * bit 1 = the lower, top-left bound). */
typedef enum {
  MAGI_MASK_FULL = 0,      /* every (q, k) pair of the rectangle is visible */
  MAGI_MASK_CAUSAL = 1,    /* lower triangle aligned at the bottom-right corner:
                              row r of [q_start, q_end) sees k in [k_start, k_end)
                              with k - k_end <= r - q_end */
  MAGI_MASK_INVCAUSAL = 2, /* upper triangle aligned at the top-left corner:
                              row r sees k in [k_start, k_end) with
                              k - k_start >= r - q_start */
  MAGI_MASK_BICAUSAL = 3   /* both bounds: a band of k_end - k_start - (q_end - q_start) + 1
                              keys per row, e.g. a sliding window */
} magi_mask_type;

typedef enum { MAGI_DTYPE_BF16 = 0, MAGI_DTYPE_FP32 = 1 } magi_dtype;

/* One AttnSlice: half-open token ranges in the packed Q and K index spaces. */
typedef struct {
  int32_t q_start, q_end, k_start, k_end, mask_type;
} magi_attn_slice;

/* One unit of kernel work: a tile of q_len <= tile_q query tokens and one KV
 * group.  It owns those output rows for every query head of the group, so no
 * two items ever write the same output (no atomics).  [slice_begin,
 * slice_end) indexes the tile-slice list, whose entries index the slice
 * array.  cost = visible (q, k) pairs of the tile per head (load estimate). */
typedef struct {
  int32_t q_start, q_len, slice_begin, slice_end, kv_group, cost;
} magi_work_item;

/* One packed video of equal-length chunks. */
typedef struct {
  int32_t chunk_len;       /* tokens per chunk, >= 1 */
  int32_t num_kv_chunks;   /* chunks present in K/V (KV cache + in flight), >= 1 */
  int32_t num_q_chunks;    /* the last num_q_chunks of them carry queries, 1..num_kv_chunks */
  int32_t q_offset;        /* first row of this video in the packed Q index space */
  int32_t k_offset;        /* first row of this video in the packed K index space */
  const int32_t* kv_range; /* [host] [num_q_chunks] or NULL (all unlimited): -1 = unlimited,
                              r >= 0 = the chunk sees itself and its r preceding chunks */
} magi_seq_desc;

/* A KV cache kept as a ring of chunk slots for streaming generation.
 * Global chunk c lives in slot c mod ring_slots, i.e. key rows
 * [k_offset + (c mod ring_slots) * chunk_len, + chunk_len).  The ring holds
 * global chunks [first_chunk, first_chunk + num_chunks); the newest
 * num_inflight of them are being denoised and carry the queries, chunk j of
 * them at query rows [q_offset + j * chunk_len, + chunk_len). */
typedef struct {
  int32_t chunk_len;       /* tokens per chunk, >= 1 */
  int32_t ring_slots;      /* chunks the ring holds, >= num_chunks */
  int32_t first_chunk;     /* global index of the oldest chunk in the ring, >= 0 */
  int32_t num_chunks;      /* chunks present, 1..ring_slots */
  int32_t num_inflight;    /* newest chunks carrying queries, 1..num_chunks */
  int32_t q_offset;        /* first query row of in-flight chunk 0 */
  int32_t k_offset;        /* first key row of slot 0 */
  const int32_t* kv_range; /* [host] [num_inflight] or NULL: -1 = every chunk in the ring up to
                              itself, r >= 0 = itself and its r preceding chunks (clipped to
                              the ring) */
} magi_ring_desc;

/* One packed sample of a cross-attention: its video query rows and its
 * condition (text) key rows. */
typedef struct {
  int32_t q_offset, q_len;  /* video tokens of the sample in the packed Q index space */
  int32_t k_offset, k_len;  /* its condition tokens in the packed K index space */
} magi_cross_desc;

/* One packed sequence under causal sliding-window attention: every token
 * sees itself and the window - 1 tokens before it in its own sequence. */
typedef struct {
  int32_t len;       /* tokens of the sequence (its queries and keys alike), >= 0 */
  int32_t window;    /* keys per row, >= 1 (window >= len is plain causal attention) */
  int32_t q_offset;  /* first row of the sequence in the packed Q index space */
  int32_t k_offset;  /* first row of the sequence in the packed K index space */
} magi_window_desc;

/* Library version string (static storage). */
const char* magi_version(void);

/* Message of the last failed call on this thread ("" if none). */
const char* magi_last_error(void);

/*
 * magi_slices_build -- mask description -> AttnSlices.           [host only]
 *
 * The mask it writes out: block-causal attention, full inside a chunk and
 * causal across chunks (study notes, "整体 pipeline" and "自回归去噪 DiT",
 * Block-Causal Attention bullet); a KV range r that lets a chunk see only
 * itself and its r predecessors (study notes, "推理技巧", KV Cache bullet);
 * several unrelated videos packed into one sequence, invisible to each
 * other (interview with Zhang Zheng, answer on how FFA expresses the mask);
 * each expressed as AttnSlices (q range, k range, mask type), the FFA
 * formulation (study notes, "训练 Infra", Flex-Flash-Attention bullet).
 *
 * For every query chunk c of every video emits one FULL slice
 *   q = [q_offset + j*C, q_offset + (j+1)*C)          (j = c - first query chunk)
 *   k = [k_offset + lo*C, k_offset + (c+1)*C)         (lo = 0, or max(0, c - r) with KV range r)
 * except that a video with chunk_len 1, no KV range limit and queries on all
 * chunks becomes a single CAUSAL slice.  Videos must not overlap each other
 * in either index space (MAGI_ERR_OVERLAP).
 *
 * seqs        [host] num_seqs descriptors (num_seqs >= 0)
 * slices      [host] output array of slice_cap entries, or NULL with slice_cap 0
 * num_slices  [host] out: number of slices needed (always written on OK and on
 *             MAGI_ERR_BUFFER_TOO_SMALL)
 * With slices == NULL and slice_cap == 0 this is a size query and returns MAGI_OK.
 */
int32_t magi_slices_build(const magi_seq_desc* seqs, int32_t num_seqs,
                          magi_attn_slice* slices, int32_t slice_cap, int32_t* num_slices);

/*
 * magi_slices_ring -- streaming step over a ring-buffer KV cache ->
 * AttnSlices.                                                    [host only]
 *
 * The pages cache the keys and values of denoised chunks and reuse them for
 * new chunks, with up to 4 chunks in flight (study notes, "整体 pipeline"), a
 * KV range that bounds the history a chunk sees (constant peak memory), and
 * per-denoising-stage KV ranges for controllable transitions (study notes,
 * "推理技巧", KV Cache bullet; yaliqi.com article, KV Cache and transition
 * items).  A ring of ring_slots chunk
 * slots holds exactly that history: the prologue writes each in-flight
 * chunk's keys (and the caller its values) into the chunk's slot, and a
 * chunk stays there once denoised until the ring wraps over it.  In-flight
 * chunk c sees the chunks max(first_chunk, c - r) .. c: one FULL slice per
 * contiguous run of their slots (two when the run wraps).  Per-stage KV
 * ranges are simply this call's kv_range values.  Output, size query and
 * errors as magi_slices_build.
 */
int32_t magi_slices_ring(const magi_ring_desc* desc, magi_attn_slice* slices, int32_t slice_cap,
                         int32_t* num_slices);

/*
 * magi_slices_cross -- packed cross-attention mask -> AttnSlices.  [host only]
 *
 * The parallel attention block runs a cross-attention from the video tokens
 * to the external condition (text) next to the block-causal self-attention,
 * on the same query projection, with GQA at 128 heads over 8 groups (study
 * notes, "自回归去噪 DiT", Parallel Attention Block bullet; "模型规格（Table 2）",
 * Cross-Attn row).  Every video token of a sample sees every condition
 * token of that sample and nothing else: one FULL slice
 * q = [q_offset, q_offset + q_len), k = [k_offset, k_offset + k_len) per
 * sample with both lengths > 0.  Query ranges must not overlap
 * (MAGI_ERR_OVERLAP); samples may share key ranges.  Output, size query and
 * errors as magi_slices_build; the slices feed magi_schedule / magi_ffa_fwd /
 * magi_ffa_bwd unchanged.
 */
int32_t magi_slices_cross(const magi_cross_desc* descs, int32_t num_descs,
                          magi_attn_slice* slices, int32_t slice_cap, int32_t* num_slices);

/*
 * magi_slices_window -- packed causal sliding-window mask -> AttnSlices.
 *                                                                [host only]
 *
 * Sliding-window attention is the mask form the pages name as the next one
 * for FFA (interview with Zhang Zheng, answer on FFA's mask types); the
 * window here is counted in tokens, row r of a sequence starting at s seeing
 * keys [max(s, r - window + 1), r].  Per sequence of len tokens and window
 * w: one CAUSAL slice when w >= len; otherwise a CAUSAL slice over the first
 * w - 1 rows and keys (when w > 1) and a BICAUSAL slice
 * q = [q_offset + w - 1, q_offset + len), k = [k_offset, k_offset + len),
 * whose band is exactly w keys wide.  Sequences must not overlap each other
 * in either index space (MAGI_ERR_OVERLAP).  Output, size query and errors
 * as magi_slices_build.
 */
int32_t magi_slices_window(const magi_window_desc* descs, int32_t num_descs,
                           magi_attn_slice* slices, int32_t slice_cap, int32_t* num_slices);

/*
 * magi_default_tile_q -- query tokens per work item that magi_ffa_fwd's
 * kernel is built for at this shape (the kernel covers 256 query rows =
 * tile_q tokens x (hq/hkv) heads).  Returns < 0 on unsupported shapes.
 */
int32_t magi_default_tile_q(int32_t hq, int32_t hkv, int32_t head_dim, int32_t dtype);

/*
 * magi_schedule -- AttnSlices -> atomic-free work list.          [host only]
 *
 * Validates the slices (ranges inside [0,nq) x [0,nk), known mask type, no
 * (q, k) pair listed twice, k_start + (q_end - q_start) < 2^31 for a type
 * with the top-left bound), cuts the query axis at every slice boundary,
 * tiles each piece into tiles of at most tile_q tokens (tile_q = 0 picks
 * magi_default_tile_q), and emits one work item per (tile, KV group),
 * including tiles no slice covers (their rows get O = 0, LSE = -inf).
 * Items are ordered heaviest first by visible-pair area (the area measure of
 * MagiAttention's dispatch solver: interview, answer on load balancing;
 * 量子位 article, "计算负载均衡"), with the KV groups interleaved so that
 * consecutive workgroups, which the GPU deals round-robin to its 8 XCDs,
 * keep one KV group per XCD.
 *
 * slices       [host] num_slices slices (num_slices >= 0)
 * work         [host] output, work_cap entries (or NULL with work_cap 0)
 * tile_slices  [host] output, ts_cap int32 slice indices (or NULL with ts_cap 0)
 * num_work, num_tile_slices [host] out: counts needed
 * With both output arrays NULL and both caps 0 this is a size query.
 * The work list is a deterministic function of the arguments.
 */
int32_t magi_schedule(const magi_attn_slice* slices, int32_t num_slices,
                      int64_t nq, int64_t nk, int32_t hq, int32_t hkv,
                      int32_t head_dim, int32_t dtype, int32_t tile_q,
                      magi_work_item* work, int32_t work_cap, int32_t* num_work,
                      int32_t* tile_slices, int32_t ts_cap, int32_t* num_tile_slices);

/*
 * magi_qknorm_rope -- QK-Norm then 3D RoPE on Q and (optionally) K.  [device]
 *
 * The pages normalise Q and K before attention (study notes, "自回归去噪
 * DiT", QK-Norm + GQA bullet; 量子位 article, "QK-Norm和GQA") and encode
 * positions with a 3D RoPE over time and space whose base frequency is
 * learnable (study notes, "自回归去噪 DiT", Block-Causal Attention bullet;
 * 量子位 article, "Block-Causal Attention", 3D RoPE item).  They give no
 * formula; the RMS norm, the equal t/h/w thirds of head_dim and the pairing
 * below are this library's reading.
 *
 * For every token i and head h of X in {Q, K}:
 *   y = x / sqrt(mean_d(x^2) + eps) * gain           (RMS over head_dim)
 *   then for axis a in (t, h, w), channel pair (2j, 2j+1) of section a
 *   (head_dim/3 channels per section), angle = pos[i][a] * base_a^(-2j/(head_dim/3)):
 *   (y0, y1) -> (y0 cos - y1 sin, y0 sin + y1 cos).
 * then y is multiplied by q_scale (Q) or k_scale (K).  Arithmetic is fp32;
 * the result is stored in the input dtype (round-to-nearest-even for bf16).
 * Output may alias input.  Passing k_scale = softmax_scale * log2(e) and then
 * softmax_scale = ln(2) to magi_ffa_fwd folds the softmax scale into K once,
 * which removes one multiply per attention score.
 *
 * q_in, q_out   [device] [nq rows] x [hq heads] x [head_dim], row stride q_tok_stride
 *               elements (>= hq*head_dim), heads contiguous; 16-byte aligned
 * k_in         [device] same for K with hkv heads, row stride k_tok_stride (NULL
 *               and nk = 0 to skip K)
 * k_out        [device] K's output; the vector of (token i, head h) starts at
 *               element i * k_out_tok_stride + h * k_out_head_stride: either
 *               token-major (k_out_head_stride = head_dim, k_out_tok_stride >=
 *               hkv * head_dim) or group-major (k_out_tok_stride = head_dim,
 *               k_out_head_stride >= nk * head_dim), whose K/V tiles
 *               magi_ffa_fwd reads as contiguous blocks (faster).  Strides are
 *               multiples of 16 bytes.  May alias k_in only with k_in's layout.
 * v_in, v_out  [device] optional (both NULL to skip): V, laid out like k_in, is
 *               copied unchanged into k_out's layout (v_out must not alias
 *               v_in), so that K and V reach magi_ffa_fwd in one layout
 * head_dim      24 or 48 (must be divisible by 6)
 * gain_q/gain_k [device] fp32 [head_dim] (gain_head_stride 0) or [heads][head_dim]
 *               (gain_head_stride = head_dim)
 * pos_q, pos_k  [device] int32 [n][3] latent (t, h, w) coordinates
 * rope_base     [device] fp32 [3] base frequency of the t, h, w axes (> 0)
 * q_scale, k_scale  output factors (finite, non-zero; 1 = plain QK-Norm + RoPE)
 * k_norm_max    [device] fp32 [hkv] out, or NULL: an upper bound on the L2
 *               norm of every stored K row of each head, sqrt(head_dim) *
 *               max|gain_k| * |k_scale| * (1 + 2^-7) (the RMS step leaves
 *               norm <= sqrt(head_dim), the rotation keeps norms; the margin
 *               covers bf16 rounding).  Pass it to magi_ffa_fwd.
 */
int32_t magi_qknorm_rope(const void* q_in, void* q_out, int64_t nq, int32_t hq, int64_t q_tok_stride,
                         const void* k_in, void* k_out, int64_t nk, int32_t hkv, int64_t k_tok_stride,
                         int64_t k_out_tok_stride, int64_t k_out_head_stride,
                         const void* v_in, void* v_out,
                         int32_t head_dim, int32_t dtype,
                         const float* gain_q, const float* gain_k, int32_t gain_head_stride,
                         float eps, const int32_t* pos_q, const int32_t* pos_k,
                         const float* rope_base, float q_scale, float k_scale,
                         float* k_norm_max, void* stream);

/*
 * magi_ffa_fwd -- Flex-Flash-Attention forward over a work list.   [device]
 *
 * Softmax attention restricted to the union of AttnSlices, the FFA kernel
 * of the pages (study notes, "训练 Infra", Flex-Flash-Attention bullet;
 * 量子位 article, "Flex-Flash-Attention"), with grouped-query attention at
 * 128 query heads over 8 KV groups (study notes, "模型规格（Table 2）" and
 * "自回归去噪 DiT", QK-Norm + GQA bullet).  The pages' kernel uses atomics;
 * here each work item owns its output rows, so none are needed.
 *
 * For every query row i and head h (KV group g = h / (hq/hkv)):
 *   O[i,h]   = sum_k softmax_k(scale * q[i,h].k[k,g]) v[k,g]   over the visible k
 *   LSE[i,h] = log sum_k exp(scale * q[i,h].k[k,g])             (natural log)
 * where the visible k are the union of the slices listed by the work item
 * that owns row i.  Rows with no visible key get O = 0 and LSE = -inf.
 * bf16: bf16 MFMA products with fp32 accumulation and fp32 online softmax;
 * P is rounded to bf16 for the PV product; O is stored as bf16.
 * fp32: fp32 arithmetic throughout.  The result is bitwise deterministic.
 *
 * q            [device] [nq][hq][head_dim], row stride q_tok_stride elements
 * k, v         [device] nk tokens x hkv heads x head_dim; the vector of (token
 *              i, head h) starts at element i * kv_tok_stride + h *
 *              kv_head_stride: token-major (kv_head_stride = head_dim) or
 *              group-major (kv_tok_stride = head_dim, kv_head_stride >= nk *
 *              head_dim; each K/V tile is then one contiguous block, which
 *              the kernel loads faster), vectors never overlapping
 * out          [device] [nq][hq][head_dim], row stride o_tok_stride elements
 * lse          [device] fp32 [nq][hq] (row stride hq), or NULL
 *              All tensor pointers 16-byte aligned, strides multiples of 8.
 * softmax_scale  <= 0 selects 1/sqrt(head_dim); ln(2) means the scores are
 *              already in log2 units (softmax scale folded into Q or K)
 * k_norm_max   [device] fp32 [hkv] or NULL: an upper bound on the L2 norm of
 *              every K row of each group (as written by magi_qknorm_rope).
 *              With it, each row's softmax reference is |q| * bound
 *              (Cauchy-Schwarz) instead of a running max, which saves the max
 *              and rescaling work; rows whose bound exceeds 60 in log2 units
 *              keep the running max.  A value below the true norms gives wrong
 *              results (possibly inf).  Ignored for fp32.
 * slices, work, tile_slices  [device] copies of magi_schedule's outputs made for
 *              the same nq, nk, hq, hkv, head_dim, dtype (items are clamped to
 *              the tensor bounds on the device, so a mismatched list cannot
 *              read or write out of bounds)
 * Supported: head_dim 24 or 48; hq % hkv == 0; hq/hkv <= 256;
 *              kv_tok_stride < 2^23 elements (MAGI_ERR_UNSUPPORTED otherwise).
 */
int32_t magi_ffa_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                     int64_t nq, int64_t nk, int32_t hq, int32_t hkv, int32_t head_dim, int32_t dtype,
                     int64_t q_tok_stride, int64_t kv_tok_stride, int64_t kv_head_stride,
                     int64_t o_tok_stride, float softmax_scale, const float* k_norm_max,
                     const magi_attn_slice* slices, int32_t num_slices,
                     const magi_work_item* work, int32_t num_work,
                     const int32_t* tile_slices, int32_t num_tile_slices,
                     void* stream);

/*
 * magi_ffa_fwd_timed -- magi_ffa_fwd whose launch also records two HIP
 * events.                                                  [device, async]
 *
 * The same operation as magi_ffa_fwd (study notes, "训练 Infra",
 * Flex-Flash-Attention bullet), for callers that time the kernel: the
 * kernel's dispatch itself records start_event when the kernel starts and
 * stop_event when it completes, so hipEventElapsedTime(start, stop) is the
 * kernel's duration and the stream holds no marker packets of its own
 * around it (recording the events separately adds about 8 us of idle GPU
 * time per launch on the 4.5B-shaped layer).
 *
 * All arguments of magi_ffa_fwd, plus:
 * start_event, stop_event  hipEvent_t created by the caller with timing
 *              enabled, or NULL (no event); both recorded on `stream`.  The
 *              caller keeps ownership.
 * Errors as magi_ffa_fwd; a launch error is MAGI_ERR_HIP.
 */
int32_t magi_ffa_fwd_timed(const void* q, const void* k, const void* v, void* out, float* lse,
                           int64_t nq, int64_t nk, int32_t hq, int32_t hkv, int32_t head_dim, int32_t dtype,
                           int64_t q_tok_stride, int64_t kv_tok_stride, int64_t kv_head_stride,
                           int64_t o_tok_stride, float softmax_scale, const float* k_norm_max,
                           const magi_attn_slice* slices, int32_t num_slices,
                           const magi_work_item* work, int32_t num_work,
                           const int32_t* tile_slices, int32_t num_tile_slices,
                           void* stream, void* start_event, void* stop_event);

/*
 * magi_ffa_fwd_qknorm -- magi_ffa_fwd with the QK-Norm + 3D RoPE of Q done
 * inside the attention kernel.                          [device, async]
 *
 * The same operation as magi_qknorm_rope on Q followed by magi_ffa_fwd (the
 * pages' order: QK-Norm, then RoPE, then attention; study notes "自回归去噪
 * DiT"), with q_raw the un-normalised queries: each work item normalises and
 * rotates its own query rows in registers, so Q is read once and never
 * written back (K still goes through magi_qknorm_rope).  Arithmetic as
 * magi_qknorm_rope (fp32, result rounded to bf16) except that the rotation
 * angles use the hardware sine and cosine of the angle reduced to one turn
 * (absolute error ~1e-6, far below the bf16 rounding of the result).
 *
 * All arguments of magi_ffa_fwd (q replaced by q_raw), plus:
 * gain_q, gain_head_stride, eps, pos_q, rope_base, q_scale
 *              as in magi_qknorm_rope for Q
 * q_hat        [device] out or NULL: receives the normalised, rotated Q
 *              (bf16, [nq][hq][head_dim], row stride q_hat_stride), e.g. for
 *              the backward
 * Supported: bf16 only (MAGI_ERR_UNSUPPORTED for fp32); otherwise as
 * magi_ffa_fwd.
 */
int32_t magi_ffa_fwd_qknorm(const void* q_raw, const void* k, const void* v, void* out, float* lse,
                            int64_t nq, int64_t nk, int32_t hq, int32_t hkv, int32_t head_dim, int32_t dtype,
                            int64_t q_tok_stride, int64_t kv_tok_stride, int64_t kv_head_stride,
                            int64_t o_tok_stride, float softmax_scale, const float* k_norm_max,
                            const magi_attn_slice* slices, int32_t num_slices,
                            const magi_work_item* work, int32_t num_work,
                            const int32_t* tile_slices, int32_t num_tile_slices,
                            const float* gain_q, int32_t gain_head_stride, float eps,
                            const int32_t* pos_q, const float* rope_base, float q_scale,
                            void* q_hat, int64_t q_hat_stride, void* stream);

/*
 * magi_default_tile_k -- keys per key-major work item that magi_ffa_bwd's
 * dK/dV kernel is built for (128).  Returns < 0 on unsupported shapes.
 */
int32_t magi_default_tile_k(int32_t hq, int32_t hkv, int32_t head_dim, int32_t dtype);

/* One sum of the split dK/dV pass: keys [key_start, key_start + key_len) of
 * group kv_group are the sum, in slot order, of the partial results in
 * slots slot_begin .. slot_begin + slot_count - 1. */
typedef struct {
  int32_t key_start, key_len, kv_group, slot_begin, slot_count;
} magi_kv_reduce;

/*
 * magi_schedule_kv -- AttnSlices -> key-major work list for the backward's
 * dK/dV pass.                                                    [host only]
 *
 * The transpose of magi_schedule: validates the slices the same way, cuts
 * the KEY axis at every slice boundary and tiles each piece into tiles of at
 * most tile_k keys (0 = magi_default_tile_k).  tile_slices lists, per tile,
 * the slices that show some row a key of the tile, in query order.
 *
 * A tile whose rows are many (the first chunk of a block-causal video is
 * seen by every later chunk) would make one item far longer than the rest,
 * and a short key list would leave the GPU with too few items, so tiles are
 * split into parts of at most T visible pairs (T = max(128 x 128, total
 * pairs / 8192 items)): runs of consecutive listed slices, or one slice's
 * rows cut into query-token windows of about equal pairs.  A tile of one
 * part gives one item per KV group that writes dK, dV directly (also tiles
 * no row sees: their dK, dV are written as 0).  A tile of P > 1 parts gives
 * P items per group, each writing an fp32 partial result into its own
 * slot, and one reduce entry per group that sums the P slots in order
 * (fixed order: deterministic, no atomics).
 *
 * Items: q_start / q_len hold the first key and the key count;
 * [slice_begin, slice_end) indexes tile_slices (the part's slices); cost =
 * visible pairs of the item per head; heaviest first with the KV groups
 * interleaved.  item_ext (host, 3 x work_cap entries) receives per item
 * {slot or -1 (direct), first query token, one past the last}: the item
 * only takes rows of tokens in that window.  reduce (host, reduce_cap
 * entries) receives the sums; *num_slots the number of slots (each holds 2
 * x tile_k x head_dim fp32 values: dK, then dV).  Size query: all output
 * arrays NULL with caps 0 fills the counts.  Errors as magi_schedule.
 */
int32_t magi_schedule_kv(const magi_attn_slice* slices, int32_t num_slices,
                         int64_t nq, int64_t nk, int32_t hq, int32_t hkv,
                         int32_t head_dim, int32_t dtype, int32_t tile_k,
                         magi_work_item* work, int32_t work_cap, int32_t* num_work,
                         int32_t* tile_slices, int32_t ts_cap, int32_t* num_tile_slices,
                         int32_t* item_ext, magi_kv_reduce* reduce, int32_t reduce_cap,
                         int32_t* num_reduce, int32_t* num_slots);

/*
 * magi_ffa_bwd -- gradients of magi_ffa_fwd.              [device, async]
 *
 * The pages run the FFA kernels for training (study notes, "训练 Infra";
 * interview, answer on MagiAttention) but state no backward; this is the
 * chain rule of the forward's softmax attention over the same slices:
 *   P = exp(scale q.k - LSE),  delta = rowsum(dout * out),
 *   dS = P * (dout v^T - delta),
 *   dq = scale dS k,  dk = scale dS^T q,  dv = P^T dout,
 * with dk and dv summed over the query heads of each KV group.  No atomics
 * and bitwise deterministic: a query-major pass (the forward's work list)
 * writes dq, a key-major pass (magi_schedule_kv's list) writes dk and dv
 * (key tiles split into parts write partial sums that a last launch adds in
 * a fixed order).
 * bf16: bf16 MFMA products with fp32 accumulation; P and dS are rounded to
 * bf16 for their products; the gradients are stored as bf16.  fp32: fp32
 * arithmetic throughout.
 *
 * q, k, v, out, lse, softmax_scale: exactly the forward's inputs and
 *              outputs (a forward run with softmax_scale = ln 2 on prescaled
 *              keys has gradients with respect to those prescaled keys)
 * dout         [device] [nq][hq][head_dim], row stride o_tok_stride
 * dq           [device] out, layout of q (row stride q_tok_stride)
 * dk, dv       [device] out, layout of k / v (kv_tok_stride, kv_head_stride);
 *              rows no query sees are written as 0
 * delta        [device] fp32 [nq][hq] scratch the call fills first (caller
 *              owned, no other contents needed)
 * slices, qwork/q_tile_slices  the forward's schedule (magi_schedule)
 * kwork/k_tile_slices, kitem_ext, reduce/num_reduce, num_slots
 *              [device] magi_schedule_kv's outputs for the same slices
 *              (kitem_ext may be NULL when num_reduce = num_slots = 0: every
 *              item then writes directly and takes all rows)
 * partial      [device] fp32 workspace of partial_floats >= num_slots x 2 x
 *              128 x head_dim values, 16-byte aligned (caller owned, no
 *              contents needed), for the parts of split key tiles; a last
 *              launch sums them into dk, dv
 * stream       the caller's stream.  delta and the dq pass run on it; the
 *              dk/dv pass and its sums run at the same time on a side stream
 *              of the library (one per device, default priority, created
 *              with two events on the first call and kept until the process
 *              ends), forked from `stream` after delta and joined back before
 *              the call returns, so later work on `stream` sees dq, dk, dv.
 *              Calls from several host threads are serialised around the
 *              fork and join.
 * Supported: head_dim 24 or 48; hq % hkv == 0; hq/hkv <= 64;
 * kv_tok_stride, q_tok_stride and o_tok_stride < 2^23 (MAGI_ERR_UNSUPPORTED
 * otherwise).  Errors as magi_ffa_fwd.
 */
int32_t magi_ffa_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv, float* delta,
                     int64_t nq, int64_t nk, int32_t hq, int32_t hkv, int32_t head_dim, int32_t dtype,
                     int64_t q_tok_stride, int64_t kv_tok_stride, int64_t kv_head_stride,
                     int64_t o_tok_stride, float softmax_scale, const magi_attn_slice* slices,
                     int32_t num_slices, const magi_work_item* qwork, int32_t num_qwork,
                     const int32_t* q_tile_slices, int32_t num_q_tile_slices,
                     const magi_work_item* kwork, int32_t num_kwork,
                     const int32_t* k_tile_slices, int32_t num_k_tile_slices,
                     const int32_t* kitem_ext, const magi_kv_reduce* reduce, int32_t num_reduce,
                     int32_t num_slots, float* partial, int64_t partial_floats,
                     void* stream);

/*
 * magi_ffa_bwd_noalloc -- magi_ffa_bwd with its workspace taken from the
 * library's static device scratch instead of caller buffers.  [device, async]
 *
 * For callers that cannot allocate device memory or be handed a workspace:
 * code under HIP graph capture, tight serving or training loops, harnesses
 * that forbid hipMalloc.  The call allocates nothing (no hipMalloc, no
 * hipFree, no allocating library routine); the caller still passes every
 * input and output.
 *
 * Arguments, results and errors as magi_ffa_bwd without delta, partial and
 * partial_floats.  The workspace -- delta (nq x hq fp32, rounded up to 64)
 * followed by the partial sums of split key tiles (num_slots x 2 x 128 x
 * head_dim fp32) -- lives in a file-scope device array of 16 Mi fp32 values
 * (64 MiB) that every GPU the library runs on holds until the process ends;
 * a call needing more returns MAGI_ERR_UNSUPPORTED before any HIP call.
 * Nothing in it needs to start at zero (every value is written before it is
 * read within the call).  Every call on one GPU uses that GPU's single copy:
 * calls that overlap on one GPU (other streams, other host threads) race and
 * give wrong results; calls serialised on one stream are safe.
 */
int32_t magi_ffa_bwd_noalloc(const void* q, const void* k, const void* v, const void* out, const void* dout,
                             const float* lse, void* dq, void* dk, void* dv,
                             int64_t nq, int64_t nk, int32_t hq, int32_t hkv, int32_t head_dim, int32_t dtype,
                             int64_t q_tok_stride, int64_t kv_tok_stride, int64_t kv_head_stride,
                             int64_t o_tok_stride, float softmax_scale, const magi_attn_slice* slices,
                             int32_t num_slices, const magi_work_item* qwork, int32_t num_qwork,
                             const int32_t* q_tile_slices, int32_t num_q_tile_slices,
                             const magi_work_item* kwork, int32_t num_kwork,
                             const int32_t* k_tile_slices, int32_t num_k_tile_slices,
                             const int32_t* kitem_ext, const magi_kv_reduce* reduce, int32_t num_reduce,
                             int32_t num_slots, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MAGI_BCA_H */

/*
 * moeq.h -- C ABI of libmoeq: NF4 / row-wise int8 quantization of fused MoE
 * expert tensors and the routed experts forward straight from the packed
 * storage, on AMD Instinct MI355X (gfx950).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every data pointer is a DEVICE pointer to caller-owned memory.  The
 *   library allocates nothing and keeps no state between calls.
 * - Calls are asynchronous on `stream` (a hipStream_t; NULL is the default
 *   stream).  MOEQ_OK means validation passed and every kernel was enqueued;
 *   a HIP launch error maps to MOEQ_EDEVICE.  No call synchronises the host.
 * - All validation happens on the host before any HIP call, so a rejected
 *   call has no side effect.  No call ever no-ops silently on bad input: the
 *   pages describe expert tensors silently left unquantized, and a packed
 *   uint8 tensor silently reaching a float kernel, as the failures to avoid
 *   (bitsandbytes issue #1849, comment thread; unsloth-zoo issue #850).
 * - Tensors are row-major and contiguous.  An expert tensor is
 *   [E][rows][cols] with each [e] slice an [out_features, in_features]
 *   weight: gate_up_proj is [E][2I][H] and down_proj is [E][H][I]
 *   (bitsandbytes issue #1849, Description code and maintainer thread).
 * - bf16 values travel as their uint16_t bit patterns.
 */
#ifndef MOEQ_H
#define MOEQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOEQ_ABI_VERSION 3
#define MOEQ_NF4_BLOCKSIZE 64
#define MOEQ_DQ_GROUP 256 /* NF4 blocks per double-quantization group */
#define MOEQ_MAX_EXPERTS 1024

typedef int32_t moeq_status;
enum {
  MOEQ_OK = 0,
  MOEQ_EINVAL = -1,     /* null pointer, a dimension <= 0, K < 1, T < 0, scale_codes
                           set for a format without them (or missing for NF4_DQ)   */
  MOEQ_ESHAPE = -2,     /* gate_up / down / hidden dimensions inconsistent          */
  MOEQ_EBLOCK = -3,     /* NF4: blocksize != 64 or cols % 64 != 0; int8: blocksize != cols */
  MOEQ_EFORMAT = -4,    /* format tag not what the call needs, or gate_up and down differ */
  MOEQ_EALIGN = -5,     /* a pointer is not 16-byte aligned                          */
  MOEQ_EWORKSPACE = -6, /* workspace null or smaller than moeq_experts_forward_workspace_bytes */
  MOEQ_EDEVICE = -7     /* a HIP call failed                                         */
};

enum { MOEQ_FMT_NF4 = 1, MOEQ_FMT_INT8_ROWWISE = 2, MOEQ_FMT_NF4_DQ = 3 };

/*
 * A quantized expert tensor [E][rows][cols] in caller-owned device memory.
 *
 * NF4 (format MOEQ_FMT_NF4, blocksize 64; "MoE Expert Quantization",
 * Implementation details: 4-bit mode is NF4; bitsandbytes issue #1849,
 * maintainer thread: plain packed storage plus a module-owned absmax
 * [num_experts, blocks_per_expert], in_features divisible by the blocksize):
 *   qdata  uint8 [E][rows][cols/2]; column 2m in the high nibble of byte m,
 *          column 2m+1 in the low nibble.
 *   scales fp32 [E][rows*cols/64]: the absmax of each 64-element block along
 *          a row, blocks in row order.
 * int8 row-wise (format MOEQ_FMT_INT8_ROWWISE, blocksize == cols;
 * "MoE Expert Quantization", Implementation details: 8-bit mode is a
 * row-wise int8 parametrization):
 *   qdata  int8 [E][rows][cols], codes in [-127, 127].
 *   scales fp32 [E][rows]: absmax(row) / 127.
 * NF4 with double-quantized absmax (format MOEQ_FMT_NF4_DQ, blocksize 64;
 * bitsandbytes issue #1849, Reproduction: the 4-bit config turns double
 * quantization on; maintainer thread: per-expert compress_statistics, the
 * absmax itself quantized, deferred from the first version; the pages fix
 * no format, this one is the library's own):
 *   qdata        as for NF4.
 *   scale_codes  uint8 [E][nb], nb = rows*cols/64: absmax code c of each
 *                block, c = round_half_even(fp32(fp32(255 a) / m)).
 *   scales       fp32 [E][ceil(nb/256)]: group scale s2 = fp32(m / 255),
 *                m the largest absmax of the group (groups of MOEQ_DQ_GROUP
 *                consecutive blocks of one expert, the last one possibly
 *                shorter; an all-zero group stores s2 = 0 and codes 0).
 *   The weights decode with absmax' = fp32(c * s2).
 * Since blocks and groups never straddle an expert, &qdata[e] / &scales[e]
 * (and &scale_codes[e]) with num_experts = 1 describe expert e alone.
 * scale_codes must be NULL for the other formats.
 */
typedef struct moeq_qweight {
  int32_t format;
  int32_t num_experts;
  int32_t rows;
  int32_t cols;
  int32_t blocksize;
  void *qdata;
  float *scales;
  uint8_t *scale_codes;
} moeq_qweight;

/* Version of this ABI (MOEQ_ABI_VERSION). */
int32_t moeq_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char *moeq_status_string(moeq_status status);

/*
 * Host copy of the 16 NF4 levels the kernels use (ascending, fp32), written
 * to out[0..15].  The pages name the NF4 format without printing it; the
 * levels are the QLoRA NormalFloat construction (evenly spaced standard-
 * normal quantiles, zero exactly representable, extremes -1 and +1).
 * Host-only; makes no HIP call.  MOEQ_EINVAL if out is NULL.
 */
moeq_status moeq_nf4_codebook(float *out);

/*
 * Quantize-on-load, 4-bit ("MoE Expert Quantization", intro and
 * Implementation details; bitsandbytes issue #1849, maintainer thread).
 * w_bf16: bf16 [E][rows][cols] (16-byte aligned); dst describes the output
 * and must have format MOEQ_FMT_NF4 or MOEQ_FMT_NF4_DQ, blocksize 64,
 * cols % 64 == 0, and 16-byte aligned qdata/scales/scale_codes.  For each
 * 64-block: absmax = max |w|; n = fp32(w / absmax) (IEEE division); code =
 * nearest NF4 level, an exact tie to the lower index; an all-zero block
 * stores absmax 0 and code 7.  With MOEQ_FMT_NF4_DQ the absmax is then
 * double-quantized in the same pass (as moeq_compress_absmax would); the
 * 4-bit codes are those of the plain format.
 * The source may be freed (stream-ordered) as soon as the call returns.
 * Preconditions not checked on device: finite weights.
 */
moeq_status moeq_quantize_nf4(const uint16_t *w_bf16, const moeq_qweight *dst, void *stream);

/*
 * Measurement reference, not part of the method: the launch shape, loads and
 * stores of moeq_quantize_nf4 on a plain NF4 tensor (every bf16 element read
 * once with the same 16-byte loads, 0.5 B of codes and 4/64 B of absmax
 * written per element) with the NF4 decision replaced by an XOR fold, so its
 * rate is the bandwidth attainable with the quantize kernel's byte mix and
 * access pattern.  Same arguments and checks as moeq_quantize_nf4 (format
 * MOEQ_FMT_NF4 only); the bytes it writes into dst are meaningless.
 */
moeq_status moeq_stream_reference(const uint16_t *w_bf16, const moeq_qweight *dst, void *stream);

/*
 * Quantize-on-load, 8-bit ("MoE Expert Quantization", Implementation
 * details: row-wise int8 parametrization).  dst: format
 * MOEQ_FMT_INT8_ROWWISE, blocksize == cols, cols % 8 == 0.  Per row:
 * absmax = max |w|; scale = fp32(absmax / 127); q = round-half-even of
 * fp32(fp32(127 w) / absmax); a zero row gives scale 0 and q 0.
 * Preconditions not checked on device: finite weights, |w| < 2^120.
 */
moeq_status moeq_quantize_int8_rowwise(const uint16_t *w_bf16, const moeq_qweight *dst, void *stream);

/*
 * Double-quantize the absmax of an NF4 tensor (bitsandbytes issue #1849,
 * Reproduction and maintainer thread: double quantization, the absmax
 * itself quantized).  src: MOEQ_FMT_NF4; dst: MOEQ_FMT_NF4_DQ of the same
 * shape.  dst->qdata may be src->qdata (the 4-bit codes are shared) or
 * another buffer (they are copied).  Codes and group scales as described
 * at moeq_qweight.  Preconditions not checked on device: finite absmax >= 0.
 */
moeq_status moeq_compress_absmax(const moeq_qweight *src, const moeq_qweight *dst, void *stream);

/*
 * Dequantize (bitsandbytes issue #1849, maintainer thread: the
 * correctness-first path dequantizes the experts; "MoE Expert
 * Quantization", Implementation details: int8 is dequantized for the
 * forward).  out_bf16: bf16 [E][rows][cols], 16-byte aligned.
 * NF4: out = bf16_rne(fp32(level[code] * absmax)); int8: out =
 * bf16_rne(fp32(q * scale)) -- the fp32 product first, then round to bf16.
 * NF4 with double-quantized absmax: as NF4 with absmax' = fp32(c * s2).
 */
moeq_status moeq_dequantize(const moeq_qweight *src, uint16_t *out_bf16, void *stream);

/*
 * Device workspace moeq_experts_forward needs for T tokens and top-K routing
 * over these weights (an upper bound independent of the routing); 0 if the
 * arguments are invalid.  Host-only.
 */
size_t moeq_experts_forward_workspace_bytes(int32_t T, int32_t K, const moeq_qweight *gate_up,
                                            const moeq_qweight *down);

/*
 * Routed experts forward from packed storage (unsloth-zoo issue #850,
 * Suggested fix: the (hidden_states, top_k_index, top_k_weights) interface
 * is uniform across fused-expert architectures; bitsandbytes issue #1849,
 * Description: gate_up_proj [E, 2I, H], down_proj [E, H, I], act_fn).
 *   hidden_bf16   bf16 [T][H]
 *   top_k_index   int32 [T][K]; entries outside [0, E) are not routed and
 *                 contribute nothing; a repeated expert counts per occurrence
 *   top_k_weights fp32 [T][K], used as given
 *   gate_up       [E][2I][H]: rows 0..I-1 are the gate, rows I..2I-1 the up
 *                 projection; down [E][H][I]; both of one format (NF4,
 *                 NF4 with double-quantized absmax, or int8)
 *   out_bf16      bf16 [T][H]:
 *                 out[t] = sum_k w[t,k] * down[e] @ (silu(gate[e] x_t) * up[e] x_t)
 *                 with the k terms added in order k = 0..K-1 in fp32
 *                 (deterministic, bit-identical run to run); above 512
 *                 assignments each weighted term is first rounded to bf16.
 *   workspace     device memory of at least
 *                 moeq_experts_forward_workspace_bytes(T, K, gate_up, down).
 * Weights are dequantized tile by tile inside the kernels (bf16 operands,
 * fp32 accumulation); no dequantized tensor is materialised.  T == 0 is a
 * valid no-op.  MOEQ_ESHAPE unless H and I are multiples of 64, T*K <= 2^24
 * and hidden_states is smaller than 4 GiB.
 */
moeq_status moeq_experts_forward(const uint16_t *hidden_bf16, const int32_t *top_k_index,
                                 const float *top_k_weights, int32_t T, int32_t K,
                                 const moeq_qweight *gate_up, const moeq_qweight *down,
                                 uint16_t *out_bf16, void *workspace, size_t workspace_bytes,
                                 void *stream);

/*
 * moeq_experts_forward with stage timing: stage_events is NULL or an array of
 * 5 hipEvent_t (created by the caller) recorded on `stream` before routing,
 * after routing, after the gate_up GEMM, after the down GEMM and after the
 * combine, so the caller can time each stage with hipEventElapsedTime.
 * Otherwise identical to moeq_experts_forward.
 */
moeq_status moeq_experts_forward_timed(const uint16_t *hidden_bf16, const int32_t *top_k_index,
                                       const float *top_k_weights, int32_t T, int32_t K,
                                       const moeq_qweight *gate_up, const moeq_qweight *down,
                                       uint16_t *out_bf16, void *workspace, size_t workspace_bytes,
                                       void *stream, void *const *stage_events);

/*
 * moeq_experts_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, kernels and results, without the
 * workspace argument.  The workspace is a device array inside the library of
 * MOEQ_NOALLOC_SCRATCH_BYTES (64 MiB), which each GPU the library runs on
 * holds until the process ends; its address on the current device is looked
 * up on the first call there (the stream must belong to the current device).
 * The call allocates nothing.  MOEQ_EWORKSPACE when
 * moeq_experts_forward_workspace_bytes(T, K, gate_up, down) exceeds the array
 * (the largest batches that fit: 818 tokens of an OLMoE-shaped layer at
 * top-8, 744 of a Mixtral-shaped one at top-2; every few-assignment batch
 * fits).  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (different
 * streams, or threads) race and must be serialised by the caller.  Nothing
 * in the array needs clearing between calls (every byte the forward reads is
 * written earlier in the same call).
 */
#define MOEQ_NOALLOC_SCRATCH_BYTES (64u << 20)
moeq_status moeq_experts_forward_noalloc(const uint16_t *hidden_bf16, const int32_t *top_k_index,
                                         const float *top_k_weights, int32_t T, int32_t K,
                                         const moeq_qweight *gate_up, const moeq_qweight *down,
                                         uint16_t *out_bf16, void *stream);

/*
 * Gradients of the routed experts block with respect to its inputs, the
 * packed weights frozen: the workload the quantized experts serve is adapter
 * training over frozen 4-bit/8-bit experts ("MoE Expert Quantization",
 * Axolotl docs, intro and Expert LoRA targeting; Axolotl issue #3787, Use
 * case).  With out = moeq_experts_forward(...) and the incoming gradient
 * grad_out = dL/dout (bf16 [T][H]):
 *   grad_hidden_bf16   bf16 [T][H]: dL/dhidden = sum_k (gate^T dg + up^T du),
 *                      added in k order, with dh = w * down^T grad_out_t,
 *                      dg = dh u s (1 + g (1 - s)), du = dh g s,
 *                      s = sigmoid(g), g / u the gate / up projections
 *   grad_weights       fp32 [T][K]: dL/dw[t,k] = grad_out_t . (down h),
 *                      formed as (down^T grad_out_t) . h from the down^T
 *                      product that dh needs; 0 for an unrouted assignment
 * Same arguments and rules as moeq_experts_forward otherwise; the forward's
 * gate_up GEMM is recomputed inside (g, u and h are not taken from a previous
 * call).  Roundings: h and dg/du feed bf16 MFMA operands; every sum is fp32;
 * deterministic (no float atomics).  workspace: at least
 * moeq_experts_backward_workspace_bytes(T, K, gate_up, down) bytes.
 * MOEQ_ESHAPE additionally unless T*K*2I*2 bytes < 4 GiB.
 */
size_t moeq_experts_backward_workspace_bytes(int32_t T, int32_t K, const moeq_qweight *gate_up,
                                             const moeq_qweight *down);
moeq_status moeq_experts_backward(const uint16_t *hidden_bf16, const int32_t *top_k_index,
                                  const float *top_k_weights, int32_t T, int32_t K,
                                  const moeq_qweight *gate_up, const moeq_qweight *down,
                                  const uint16_t *grad_out_bf16, uint16_t *grad_hidden_bf16,
                                  float *grad_weights, void *workspace, size_t workspace_bytes,
                                  void *stream);

/*
 * Training pair without the backward's recompute of the gate_up GEMM, for
 * adapter training over frozen quantized experts ("MoE Expert Quantization",
 * Axolotl docs, Expert LoRA targeting; Axolotl issue #3787, Use case) when
 * the memory for the pre-activations is there.  moeq_experts_forward_save is
 * moeq_experts_forward that also writes, for every routed assignment, the
 * fp32 g = gate[e] x_t and u = up[e] x_t; moeq_experts_backward_saved takes
 * them in place of its recompute.  The chain rule, roundings and order are
 * moeq_experts_backward's, and both calls group the assignments in the same
 * deterministic order, so the gradients equal moeq_experts_backward's bit
 * for bit.
 *   gu_saved  fp32 [T*K][2I], caller-owned, 16-byte aligned: row p holds g
 *             (columns 0..I-1) then u (I..2I-1) of the p-th assignment in
 *             the expert-major stable order of moeq_route_buckets' perm;
 *             rows past the routed count are not written.  It must come from
 *             moeq_experts_forward_save with the same top_k_index, hidden
 *             states and gate_up (not checked).
 * moeq_experts_forward_save takes the tiled path for every batch size (for
 * T*K <= 512 moeq_experts_forward takes the few-assignment path, whose
 * output then agrees within rounding, not bit for bit); its workspace is
 * moeq_experts_forward_workspace_bytes.  The backward needs no hidden
 * states; its workspace, moeq_experts_backward_saved_workspace_bytes, has
 * no g|u region.  Both return MOEQ_ESHAPE where moeq_experts_backward does.
 */
moeq_status moeq_experts_forward_save(const uint16_t *hidden_bf16, const int32_t *top_k_index,
                                      const float *top_k_weights, int32_t T, int32_t K,
                                      const moeq_qweight *gate_up, const moeq_qweight *down, uint16_t *out_bf16,
                                      float *gu_saved, void *workspace, size_t workspace_bytes, void *stream);
size_t moeq_experts_backward_saved_workspace_bytes(int32_t T, int32_t K, const moeq_qweight *gate_up,
                                                   const moeq_qweight *down);
moeq_status moeq_experts_backward_saved(const int32_t *top_k_index, const float *top_k_weights, int32_t T,
                                        int32_t K, const moeq_qweight *gate_up, const moeq_qweight *down,
                                        const float *gu_saved, const uint16_t *grad_out_bf16,
                                        uint16_t *grad_hidden_bf16, float *grad_weights, void *workspace,
                                        size_t workspace_bytes, void *stream);

/*
 * Router front-end producing the experts' (top_k_index, top_k_weights): the
 * gate weight mlp.gate.weight stays bf16 beside the quantized experts
 * ("MoE Expert Quantization", Axolotl docs, Expert LoRA targeting;
 * bitsandbytes issue #1849, maintainer thread: router-only training over
 * NF4 experts) and feeds the uniform experts interface (unsloth-zoo issue
 * #850, Suggested fix).
 *   hidden_bf16    bf16 [T][H], 16-byte aligned
 *   gate_bf16      bf16 [E][H] (one row per expert), 16-byte aligned
 *   logits         gate @ x_t: bf16 operands, fp32 accumulation
 *   top_k_index    int32 [T][K]: the K largest logits, largest first, equal
 *                  logits to the lower expert index
 *   top_k_weights  fp32 [T][K]: softmax over all E of the selected logits;
 *                  with renormalize != 0 divided by their sum (a softmax
 *                  over the K selected logits)
 * Deterministic.  MOEQ_ESHAPE unless H % 64 == 0 and 1 <= K <= E <=
 * MOEQ_MAX_EXPERTS; T == 0 is a valid no-op.
 */
moeq_status moeq_router_topk(const uint16_t *hidden_bf16, const uint16_t *gate_bf16, int32_t T, int32_t H,
                             int32_t E, int32_t K, int32_t renormalize, int32_t *top_k_index,
                             float *top_k_weights, void *stream);

/*
 * Router front-end fused with the routing stage: the same logits, top-K and
 * weights as moeq_router_topk, and from the same selections the grouping of
 * the T*K assignments a = t*K + k by expert that moeq_route_buckets computes
 * (unsloth-zoo issue #850, Suggested fix: one generic routing behind the
 * uniform (hidden_states, top_k_index, top_k_weights) interface; "MoE Expert
 * Quantization", Axolotl docs, Expert LoRA targeting: the router
 * mlp.gate.weight beside the quantized experts).  The router's workgroups
 * rank their own selections (stable, by assignment order) as they make them,
 * so top_k_index is not read back; a per-expert scan and a scatter follow.
 *   top_k_index, top_k_weights  as for moeq_router_topk ([T][K])
 *   counts  int32 [E], offsets int32 [E+1], perm int32 [T*K], slot int32 [T*K]:
 *           as for moeq_route_buckets (every selection is routed, so perm is
 *           a full permutation and no slot is -1)
 *   workspace  device memory of moeq_router_route_workspace_bytes(T, H, E, K)
 * Bit-identical to moeq_router_topk followed by moeq_route_buckets.
 * MOEQ_ESHAPE unless H % 64 == 0, 1 <= K <= min(E, 64), E <= MOEQ_MAX_EXPERTS
 * and T*K <= 2^24; T == 0 writes zero counts and offsets.
 */
size_t moeq_router_route_workspace_bytes(int32_t T, int32_t H, int32_t E, int32_t K);
moeq_status moeq_router_route(const uint16_t *hidden_bf16, const uint16_t *gate_bf16, int32_t T, int32_t H,
                              int32_t E, int32_t K, int32_t renormalize, int32_t *top_k_index,
                              float *top_k_weights, int32_t *counts, int32_t *offsets, int32_t *perm,
                              int32_t *slot, void *workspace, size_t workspace_bytes, void *stream);

/*
 * moeq_experts_forward with the routing already done: offsets, perm and slot
 * are the grouping of this top_k_index by expert (as moeq_router_route or
 * moeq_route_buckets wrote it), so the routing stage is skipped.  Same
 * arguments, workspace, rules and results as moeq_experts_forward (the
 * output is bit-identical).  Preconditions not checked on device: the
 * routing buffers belong to this top_k_index.
 */
moeq_status moeq_experts_forward_routed(const uint16_t *hidden_bf16, const int32_t *top_k_index,
                                        const float *top_k_weights, int32_t T, int32_t K,
                                        const moeq_qweight *gate_up, const moeq_qweight *down,
                                        const int32_t *offsets, const int32_t *perm, const int32_t *slot,
                                        uint16_t *out_bf16, void *workspace, size_t workspace_bytes,
                                        void *stream);

/*
 * Asynchronous copy of one packed expert tensor (codes and scales) between
 * host and device memory, in either direction, on `stream`: the building
 * block of expert-granularity offload, where every layer's packed experts
 * live in pinned host memory, one layer is resident and layer N+1 is
 * prefetched on a side stream during layer N (Axolotl issue #3787, Proposed
 * shape; Evidence: the forward is bit-identical with offload on or off).
 * src and dst must describe the same format and shape (codes, scales and,
 * for MOEQ_FMT_NF4_DQ, absmax codes are copied); their pointers may be
 * pinned host memory (allocated pinned, e.g. hipHostMalloc) or device
 * memory.  The copy is ordered on `stream` like any other call; the caller
 * makes the compute stream wait (an event) before using dst.
 */
moeq_status moeq_qweight_copy_async(const moeq_qweight *src, const moeq_qweight *dst, void *stream);

/*
 * The routing stage of moeq_experts_forward on its own (same kernels):
 * groups the T*K assignments a = t*K + k by expert (unsloth-zoo issue #850,
 * Suggested fix: one generic routing for every architecture).
 *   counts  int32 [E]    assignments per expert
 *   offsets int32 [E+1]  exclusive prefix sum of counts
 *   perm    int32 [T*K]  assignments sorted by expert, ascending a within an
 *                        expert; entries past offsets[E] are left untouched
 *   slot    int32 [T*K]  position of a in perm, -1 for an unrouted a
 * Needs T*K <= 2^24 and E <= MOEQ_MAX_EXPERTS; workspace as for the forward
 * (moeq_experts_forward_workspace_bytes with any weights of E experts) or
 * moeq_route_workspace_bytes(T, K, E).
 */
size_t moeq_route_workspace_bytes(int32_t T, int32_t K, int32_t E);
moeq_status moeq_route_buckets(const int32_t *top_k_index, int32_t T, int32_t K, int32_t E,
                               int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *slot,
                               void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOEQ_H */

/*
 * moe.h -- C ABI of libmoe: an MI355X (gfx950) implementation of a sparse
 * MoE block with an int8 router, int4 affine group-64 SwiGLU experts carrying
 * an unmerged LoRA delta, a weighted combine, and a Prerouter head.
 *
 * Sources (page title, section):
 *   [P1] "Edge0开源框架实现35BMoE模型在Mac上流式推理，峰值内存仅2.9GiB"
 *        (tech.news18a.com): Recover-LoRA paragraph; Prerouter paragraph
 *        (prediction, expert loading and LoRA delta as separate native parts).
 *   [P2] "SSD 专家卸载 · Prerouter 路由预测" (autoark.ai): tier table (E, K,
 *        layers); prefill/decode paragraph; expert-pool and double-shift
 *        paragraphs.
 *   [P3] "iPhone、Mac、Android、Windows 实测横评：Edge0 五大平台谁最能打"
 *        (2kiu.com): model-structure paragraph (256 experts, K=4, hidden
 *        2048); "三件套" bullets (affine 4-bit, group_size 64; unmerged
 *        LoRA; prediction heads); quality section (8-bit router gate and
 *        shared-expert gate).
 *
 * Conventions for every entry point:
 *   - Tensors are row-major.  bf16 values travel as uint16_t bit patterns.
 *   - "device" pointers must be HIP device memory (or device-visible pinned
 *     host memory where stated); "host" pointers are ordinary host memory.
 *   - The caller owns every buffer.  No call allocates or frees device
 *     memory; scratch comes from the caller's workspace (`ws`, sized by
 *     moe_workspace_bytes).  Workspace contents need no initialisation.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work on it; nothing synchronises with the host, so every call
 *     can be captured in a HIP graph.
 *   - Errors: arguments are validated before anything is enqueued.  A bad
 *     argument returns MOE_EINVAL, a shape the kernels are not built for
 *     returns MOE_EUNSUPPORTED, a too-small workspace returns MOE_EWORKSPACE,
 *     a failed launch returns MOE_EHIP.  moe_last_error() then describes the
 *     failure (thread-local).  Device faults surface at the caller's next
 *     synchronisation.  No C++ exception crosses this ABI.
 *   - Shapes supported by the kernels: H and I in {64, 128, 256, 512, 1024,
 *     2048, 4096}, 1 <= K <= E <= 1024, K <= 16, 0 <= r <= 16, n_shared in
 *     {0, 1}; the shared expert has the same shape (H, I, r) as the routed
 *     ones.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,
  MOE_EUNSUPPORTED = 2,
  MOE_EHIP = 3,
  MOE_EWORKSPACE = 4
} moe_status_t;

/* Description of the last failure on this thread ("" if none). */
MOE_API const char* moe_last_error(void);

/* Block dimensions.  [P2] tier table, [P3] model-structure paragraph.
 *   H  hidden size            E  routed experts     K  experts per token
 *   I  expert intermediate    r  LoRA rank (0 = no LoRA)
 *   lora_scale  lambda = alpha / r of the unmerged delta lambda * B (A v)
 *   n_shared    0 or 1 shared expert gated by sigmoid(shared-gate logit)
 *   norm_topk   1: weights = softmax over the K selected logits (a full
 *               softmax renormalised over the selection); 0: plain full-
 *               softmax entries of the selection. */
typedef struct {
  int32_t H, I, E, K, r, n_shared, norm_topk;
  float lora_scale;
} moe_dims_t;

/* ---------------------------------------------------------------------------
 * Expert blobs.  One expert = one contiguous, fixed-stride blob holding
 * {gate, up, down} x {int4 codes, bf16 scale, bf16 bias} and the LoRA
 * factors {A, B} x {gate, up, down}; [P3] "三件套" bullets give the affine
 * 4-bit group-64 format and the unmerged LoRA.  One blob is one expert-pool
 * slot.  The byte layout inside a blob is private to this library: build
 * blobs only with moe_pack_expert.
 * ------------------------------------------------------------------------- */

/* Bytes of one expert blob (a multiple of 256). */
MOE_API size_t moe_expert_blob_bytes(int32_t H, int32_t I, int32_t r);

/* Host-only.  Pack one expert's logical tensors into `blob_out` (host, at
 * least moe_expert_blob_bytes bytes).  For p in gate, up (out = I, in = H)
 * and down (out = H, in = I):
 *   q_p  uint8  [out, in]     codes 0..15 (values above 15 -> MOE_EINVAL)
 *   s_p  bf16   [out, in/64]  scale, b_p bf16 [out, in/64] bias:
 *        w[j, i] = s[j, i/64] * q[j, i] + b[j, i/64]
 *        The prefill GEMMs dequantise to fp16, so every group must satisfy
 *        |s|, |b|, |15 s + b| <= 65504 (fp16's largest finite value), all
 *        finite; otherwise MOE_EUNSUPPORTED.  Scales below fp16's normal
 *        range (2^-14) keep 2^-24 absolute resolution there.
 *   A_p  bf16   [r, in],  B_p bf16 [out, r]  (may be NULL when r == 0)  */
MOE_API moe_status_t moe_pack_expert(int32_t H, int32_t I, int32_t r,
                             const uint8_t* q_gate, const uint16_t* s_gate, const uint16_t* b_gate,
                             const uint16_t* A_gate, const uint16_t* B_gate,
                             const uint8_t* q_up, const uint16_t* s_up, const uint16_t* b_up,
                             const uint16_t* A_up, const uint16_t* B_up,
                             const uint8_t* q_down, const uint16_t* s_down, const uint16_t* b_down,
                             const uint16_t* A_down, const uint16_t* B_down,
                             void* blob_out, size_t blob_bytes);

/* Where the routed experts of one layer live.  [P2] expert-pool paragraph:
 * a pool caches recently used experts and prefetched ones; here the pool is a
 * set of HBM slots addressed through a device table.
 *   slots           device, n_slots blobs of moe_expert_blob_bytes each.
 *   expert_to_slot  device int32 [E]: slot holding expert e, or -1 if not
 *                   resident.  NULL means slots holds all E experts in
 *                   expert order (n_slots == E).
 *   host_blobs      device-visible pointer to pinned, mapped host memory
 *                   with all E blobs in expert order; a non-resident expert
 *                   is read from here over PCIe.  Required when
 *                   expert_to_slot is not NULL.
 *   counters        device uint64 [2] or NULL: counters[0] += lookups served
 *                   from a slot, counters[1] += all lookups.
 *   read_delay_ns   modeled storage latency of the host copy ([P2] Prerouter
 *                   and SSD paragraphs: the benefit of early loads grows with
 *                   storage latency): in moe_block_decode(_exec), a
 *                   workgroup that reads non-resident experts first waits
 *                   this long, once however many of its experts missed (a
 *                   bounded wall-clock wait; its reads are issued together).
 *                   0: none; at most
 *                   MOE_MAX_READ_DELAY_NS (else MOE_EINVAL).  The other
 *                   calls ignore it. */
#define MOE_MAX_READ_DELAY_NS 1000000u
typedef struct {
  const void* slots;
  int32_t n_slots;
  const int32_t* expert_to_slot;
  const void* host_blobs;
  unsigned long long* counters;
  uint32_t read_delay_ns;
} moe_experts_t;

/* Workspace bytes needed by moe_route + moe_expert_forward (+ prefill
 * grouping when `prefill` != 0) for T tokens.  One workspace may be reused by
 * consecutive calls on the same stream. */
MOE_API size_t moe_workspace_bytes(const moe_dims_t* d, int32_t T, int32_t prefill);

/* ---------------------------------------------------------------------------
 * moe_route: router logits, top-K selection, routing weights, shared gate,
 * and (optionally) grouping of the (token, k) pairs by expert for prefill.
 * [P2] tier table / [P3] model-structure paragraph: top-K of E experts per
 * token; [P3] quality section: 8-bit router gate and shared-expert gate;
 * [P2] prefill/decode paragraph: prefill batches tokens per expert.
 *   gate_q  device int8 [E, H], gate_s device fp32 [E, H/64]:
 *           logit[t, e] = sum_i gate_s[e, i/64] * gate_q[e, i] * x[t, i]
 *                         (+ logit_bias[e])
 *   sgate_q device int8 [H], sgate_s fp32 [H/64]: shared-gate projection;
 *           required iff n_shared == 1.
 *   x       device bf16 [T, H].      logit_bias  device fp32 [E] or NULL.
 *   topk_idx  device int32 [T, K]: experts ordered by (-logit, index), so
 *             equal logits go to the lower index.
 *   topk_w    device fp32 [T, K]: routing weights (see norm_topk).
 *   shared_w  device fp32 [T] (n_shared == 1, else may be NULL):
 *             sigmoid(shared-gate logit).
 *   logits    device fp32 [T, E] or NULL: the biased logits.
 *   counts    device int32 [E], offsets int32 [E+1], perm int32 [T*K]: all
 *             NULL, or all set to group the pairs p = t*K + k by expert
 *             (offsets exclusive prefix of counts; perm lists each expert's
 *             pairs in ascending p).  Requires a workspace sized with
 *             prefill != 0.
 * T == 0 is valid and enqueues nothing. */
MOE_API moe_status_t moe_route(const moe_dims_t* d, const int8_t* gate_q, const float* gate_s,
                       const int8_t* sgate_q, const float* sgate_s, const uint16_t* x,
                       int32_t T, const float* logit_bias, int32_t* topk_idx, float* topk_w,
                       float* shared_w, float* logits, int32_t* counts, int32_t* offsets,
                       int32_t* perm, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * moe_expert_forward: every selected expert's SwiGLU FFN with its unmerged
 * LoRA delta, plus the shared expert.  [P1] Recover-LoRA paragraph, [P3]
 * "三件套" bullets: frozen int4 base plus an unmerged LoRA added on the fly.
 *   a_p = deq(Q_p) v + lora_scale * B_p (A_p v) for p in gate, up, down;
 *   h = silu(a_gate(x)) * a_up(x);  y = a_down(h).  h enters the down
 *   projection as fp16 scaled by a power of two (one exponent per row on the
 *   prefill path, per 32-column slice on the decode path), not as bf16.
 *   routed       where the routed experts live (see moe_experts_t).
 *   shared_blob  device blob of the shared expert (n_shared == 1) or NULL.
 *   x            device bf16 [T, H];  topk_idx device int32 [T, K] (the decode
 *                path clamps an entry outside [0, E) into range: that slot's
 *                output is then undefined, but no address leaves the experts).
 *                counts/offsets/perm must be moe_route's grouping outputs for
 *                the same T, K and E.
 *   counts, offsets, perm: NULL -> decode path (weight-streaming GEMV, one
 *                pass over each selected expert per token); the outputs of
 *                moe_route's grouping -> prefill path (grouped MFMA GEMM
 *                over each expert's tokens).
 *   y            device fp32 [T, K + n_shared, H]: y[t, k] is the output of
 *                expert topk_idx[t, k] on token t; y[t, K] the shared one.
 */
MOE_API moe_status_t moe_expert_forward(const moe_dims_t* d, const moe_experts_t* routed,
                                const void* shared_blob, const uint16_t* x, int32_t T,
                                const int32_t* topk_idx, const int32_t* counts,
                                const int32_t* offsets, const int32_t* perm, float* y,
                                void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * moe_combine: out[t] = bf16( sum_k topk_w[t,k] y[t,k] + shared_w[t] y[t,K]
 *                             (+ residual[t]) ).
 * With `norm_out` set it also writes bf16(RMSNorm(out[t])) (unit gain, eps)
 * -- the next layer's input in a residual + RMSNorm stack.
 *   y device fp32 [T, K+n_shared, H]; topk_w fp32 [T, K]; shared_w fp32 [T]
 *   (n_shared == 1); residual bf16 [T, H] or NULL; out bf16 [T, H];
 *   norm_out bf16 [T, H] or NULL. */
MOE_API moe_status_t moe_combine(const moe_dims_t* d, const float* y, const float* topk_w,
                         const float* shared_w, int32_t T, const uint16_t* residual,
                         uint16_t* out, uint16_t* norm_out, float eps, void* stream);

/* ---------------------------------------------------------------------------
 * moe_block_prefill: the whole block for a batch of prefill tokens in one
 * call -- moe_route with grouping, moe_expert_forward on the grouped path,
 * moe_combine -- with the same arithmetic except for where the expert
 * outputs are kept: in the workspace, as fp16(y * 2^-e) with one power-of-two
 * exponent e per (token, slot) row instead of fp32, which halves the bytes the
 * down GEMM writes and the combine reads.  e comes from a bound on the down
 * projection's outputs that moe_pack_expert stores in each blob, so no value
 * can overflow, and each y keeps fp16's 11-bit significand (relative rounding
 * 2^-11; values below 2^-29 of the bound lose precision as subnormals).
 * [P2] "SSD 专家卸载 · Prerouter 路由预测", prefill/decode paragraph: prefill
 * batches the whole layer's computation.
 *   gate_q .. logit_bias, x, T: as in moe_route (logit_bias may be NULL).
 *   routed, shared_blob: as in moe_expert_forward.
 *   residual, out, norm_out, eps: as in moe_combine.
 *   topk_idx device int32 [T, K], topk_w fp32 [T, K]: the routing (outputs).
 *   ws     moe_block_prefill_workspace_bytes(d, T) bytes; calls that share
 *          one must be ordered on one stream.
 * T == 0 is valid and enqueues nothing. */
MOE_API size_t moe_block_prefill_workspace_bytes(const moe_dims_t* d, int32_t T);
MOE_API moe_status_t moe_block_prefill(const moe_dims_t* d, const int8_t* gate_q,
                                       const float* gate_s, const int8_t* sgate_q,
                                       const float* sgate_s, const float* logit_bias,
                                       const moe_experts_t* routed, const void* shared_blob,
                                       const uint16_t* x, int32_t T, const uint16_t* residual,
                                       int32_t* topk_idx, float* topk_w, uint16_t* out,
                                       uint16_t* norm_out, float eps, void* ws, size_t ws_bytes,
                                       void* stream);

/* moe_rmsnorm: out[t] = bf16(h[t] / sqrt(mean(h[t]^2) + eps)), unit gain.
 * h, out device bf16 [T, H] (may alias). */
MOE_API moe_status_t moe_rmsnorm(const uint16_t* h, int32_t T, int32_t H, float eps, uint16_t* out,
                         void* stream);

/* ---------------------------------------------------------------------------
 * moe_block_decode: the whole block for a few decode tokens in ONE kernel
 * launch -- router, top-K, every selected expert and the shared expert with
 * their LoRA deltas, the weighted combine -- with the same arithmetic as
 * moe_route + moe_expert_forward + moe_combine.  [P2] decode paragraph: decode
 * is the latency-critical path (route, fetch the chosen experts, compute).
 *   flags  MOE_DECODE_NORM_INPUT: x = bf16(RMSNorm(h_in)) (unit gain, eps),
 *          else x = h_in;  MOE_DECODE_RESIDUAL: out = bf16(h_in + block(x)),
 *          else out = bf16(block(x)).
 *   h_in   device bf16 [T, H];  out device bf16 [T, H] (must not alias h_in).
 *   topk_idx int32 [T, K], topk_w fp32 [T, K]: optional copies of the
 *          routing (NULL to skip).
 *   ws     moe_block_decode_workspace_bytes(d, T) bytes, zeroed once with
 *          moe_workspace_init before the first call (the library then keeps
 *          its control words consistent from call to call).  Calls sharing a
 *          workspace must be ordered (same stream); concurrent calls need
 *          separate workspaces.
 *   Supported: T <= 4 and T * (K + n_shared) <= 8; H in {256, ..., 2048},
 *   I in {128, ..., 2048}; r <= H / 32 and r <= I / 32.  A wait that exceeds its bound (~0.2 s) sets the
 *   sticky int32 at byte MOE_DECODE_ERR_OFFSET of ws to 1 and the call
 *   completes with undefined output. */
#define MOE_DECODE_NORM_INPUT 1
#define MOE_DECODE_RESIDUAL 2
#define MOE_DECODE_SYNC_BYTES 768
#define MOE_DECODE_ERR_OFFSET 512
MOE_API size_t moe_block_decode_workspace_bytes(const moe_dims_t* d, int32_t T);
/* Zero a fused-decode workspace (a kernel, so it can be captured in a graph). */
MOE_API moe_status_t moe_workspace_init(void* ws, size_t ws_bytes, void* stream);
MOE_API moe_status_t moe_block_decode(const moe_dims_t* d, const int8_t* gate_q,
                                      const float* gate_s, const int8_t* sgate_q,
                                      const float* sgate_s, const moe_experts_t* routed,
                                      const void* shared_blob, const uint16_t* h_in, int32_t T,
                                      int32_t flags, float eps, int32_t* topk_idx, float* topk_w,
                                      uint16_t* out, void* ws, size_t ws_bytes, void* stream);

/* moe_block_decode_exec: moe_block_decode with the routed experts given
 * instead of selected (prediction-as-routing).  [P3] "三件套" Prerouter
 * bullet: the predicted route is used as the route, so expert loads can
 * overlap the forward pass; [P2] Prerouter paragraph: predicted routes take
 * part in the actual execution.
 *   exec_idx  device int32 [T, K]: the experts token t executes, in this
 *             order (typically the previous token's Prerouter prediction for
 *             this layer).  The router still runs: the weights are the
 *             softmax of its logits over the given experts (renormalised
 *             when d->norm_topk, else their full-softmax entries), and the
 *             shared gate is unchanged.  topk_idx / topk_w (optional) get
 *             the executed experts and their weights.
 *   An entry outside [0, E) sets the sticky error word (as a wait that
 *   exceeds its bound does) and is executed as expert 0.  Other arguments,
 *   limits and the workspace are those of moe_block_decode (the same
 *   workspace may serve both calls, in stream order). */
MOE_API moe_status_t moe_block_decode_exec(const moe_dims_t* d, const int8_t* gate_q,
                                           const float* gate_s, const int8_t* sgate_q,
                                           const float* sgate_s, const moe_experts_t* routed,
                                           const void* shared_blob, const uint16_t* h_in,
                                           int32_t T, int32_t flags, float eps,
                                           const int32_t* exec_idx, int32_t* topk_idx,
                                           float* topk_w, uint16_t* out, void* ws,
                                           size_t ws_bytes, void* stream);

/* moe_block_decode_noalloc: moe_block_decode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The same kernel and the same results as
 * moe_block_decode; the workspace is a library-owned device array of
 * MOE_NOALLOC_SCRATCH_BYTES per GPU instead of a caller buffer, and this call
 * never allocates or frees memory.
 *   Arguments, limits and outputs are moe_block_decode's (no ws, ws_bytes).
 *   error_out  device int32 or NULL: receives this call's timeout flag (1 if
 *              a wait exceeded its bound, else 0); the flag is then cleared.
 *   Scratch: the first call on a device looks up that device's array and
 *   zeroes it with a kernel on `stream`; each later call finds the array as
 *   the previous call on that device left it (its control words consistent).
 *   Shapes whose workspace layout exceeds MOE_NOALLOC_SCRATCH_BYTES return
 *   MOE_EUNSUPPORTED before any device work.  Every call on one GPU shares
 *   that GPU's array: calls that overlap in time on one GPU (different
 *   streams or threads without ordering) race and give undefined results. */
#define MOE_NOALLOC_SCRATCH_BYTES 1048576
MOE_API moe_status_t moe_block_decode_noalloc(const moe_dims_t* d, const int8_t* gate_q,
                                              const float* gate_s, const int8_t* sgate_q,
                                              const float* sgate_s, const moe_experts_t* routed,
                                              const void* shared_blob, const uint16_t* h_in,
                                              int32_t T, int32_t flags, float eps,
                                              int32_t* topk_idx, float* topk_w, uint16_t* out,
                                              int32_t* error_out, void* stream);

/* ---------------------------------------------------------------------------
 * prerouter_predict: the Prerouter head.  [P1] Prerouter paragraph and [P2]
 * double-shift paragraph: a light MLP after layer N predicts layer N+1's
 * top-K (for the next token) so expert loads can start early.
 *   z = W2 silu(W1 h), pred = top-K of z ordered by (-z, index).
 *   W1 device bf16 [D, H], W2 bf16 [E, D], h bf16 [T, H];
 *   pred_idx int32 [T, K]; pred_logits fp32 [T, E] or NULL.
 *   One kernel launch per call: workgroups of W1 rows hand partial logits to
 *   one workgroup per token, which adds them in a fixed order and selects.
 *   ws: device, at least prerouter_workspace_bytes(D, E, T) bytes, ZEROED
 *   ONCE before its first use (it holds the launch epoch and an arrival
 *   counter); later calls find it as the previous call left it.  Calls that
 *   share a workspace must not overlap (issue them on one stream).  Should a
 *   bounded in-kernel wait run out (a launch that cannot make progress), the
 *   token's pred_idx entries are -1.
 *   Supported: H as above, D a multiple of 64 up to 4096, 1 <= K <= 16,
 *   K <= E <= 1024, T <= 65535. */
MOE_API size_t prerouter_workspace_bytes(int32_t D, int32_t E, int32_t T);
MOE_API moe_status_t prerouter_predict(const uint16_t* W1, const uint16_t* W2, int32_t H, int32_t D,
                               int32_t E, int32_t K, const uint16_t* h, int32_t T,
                               int32_t* pred_idx, float* pred_logits, void* ws, size_t ws_bytes,
                               void* stream);

/* prerouter_predict_feat: the Prerouter head with routing features.  [P1]
 * Prerouter paragraph (the head also sees the sequence of experts already
 * executed) and [P2] Prerouter paragraph (routing features as input): the
 * input is h with the one-hot of the experts the layer executed appended,
 *   z = W2 silu(W1 [h; onehot(prev)]), pred = top-K of z ordered by (-z, index).
 *   W1 device bf16 [D, H + E] (columns H + e weight expert e); prev_idx
 *   device int32 [T, Kp] (ids outside [0, E) are ignored, so -1 pads; a
 *   repeated id counts once: the one-hot is an indicator vector);
 *   everything else as prerouter_predict.  Supported: 0 <= Kp <= 16, and
 *   H + E a multiple of 8 (16-byte W1 rows), else MOE_EUNSUPPORTED. */
MOE_API moe_status_t prerouter_predict_feat(const uint16_t* W1, const uint16_t* W2, int32_t H,
                                            int32_t D, int32_t E, int32_t K, const uint16_t* h,
                                            const int32_t* prev_idx, int32_t Kp, int32_t T,
                                            int32_t* pred_idx, float* pred_logits, void* ws,
                                            size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Expert pool.  [P2] "SSD 专家卸载 · Prerouter 路由预测", expert-pool and
 * Prerouter paragraphs: a streaming pool caches recently used experts and
 * loads the experts the Prerouter predicts; layer N's prediction on the
 * current token is for layer N+1 of the next token and is committed at the
 * step boundary, so loads overlap the next step's compute.
 *
 * Here every layer has n_slots HBM slots; the master copy of all experts is
 * pinned host memory; kernels find expert e of a layer through the device
 * slot table (moe_experts_t.expert_to_slot) and read a non-resident expert
 * from the host copy directly, so results do not depend on the pool state.
 *
 * moe_lru_*: the host-only planner (no device work, usable without a GPU).
 * A plan step takes, per layer, the K experts executed in the step just
 * finished and Kp predicted experts (entries < 0: none), and returns fills:
 *   - executed and predicted experts that are resident become most recent;
 *   - fill candidates are the predicted experts that are not resident, then
 *     the executed ones that missed, each once, at most max_fills per layer
 *     (max_fills < 0: no limit);
 *   - a fill takes a free slot, else the least recently used slot whose
 *     expert was neither executed nor predicted in this step (ties: lowest
 *     slot); with no such slot the layer's remaining candidates are skipped.
 * fills[] are ordered by layer, then candidate order.
 */
typedef struct moe_lru moe_lru_t;
typedef struct {
  int32_t layer, expert, slot, evicted; /* evicted: expert that left the slot, or -1 */
} moe_pool_fill_t;

MOE_API moe_status_t moe_lru_create(int32_t n_layers, int32_t E, int32_t n_slots, moe_lru_t** out);
MOE_API void moe_lru_destroy(moe_lru_t* l);
/* executed: host int32 [n_layers][K]; predicted: host int32 [n_layers][Kp]
 * or NULL with Kp = 0.  fills: host array of max_out entries; *n_out gets
 * the number of fills (MOE_EINVAL if it exceeds max_out; the plan is still
 * applied to the planner state). */
MOE_API moe_status_t moe_lru_plan(moe_lru_t* l, const int32_t* executed, int32_t K,
                                  const int32_t* predicted, int32_t Kp, int32_t max_fills,
                                  moe_pool_fill_t* fills, int32_t max_out, int32_t* n_out);
/* The planner's current slot of every expert of `layer` (host int32 [E]). */
MOE_API moe_status_t moe_lru_table(const moe_lru_t* l, int32_t layer, int32_t* expert_to_slot);
MOE_API moe_status_t moe_lru_stats(const moe_lru_t* l, unsigned long long* fills,
                                   unsigned long long* evictions);

/* moe_pool_*: the planner plus the device side.  The caller owns
 *   device_slots  device [n_layers][n_slots][blob_bytes],
 *   device_table  device int32 [n_layers][E] (set to -1 here, synchronously
 *                 on `stream`),
 *   host_blobs    pinned host [n_layers][E][blob_bytes], device-visible
 *                 (checked with hipHostGetDevicePointer: MOE_EINVAL if not);
 * the pool owns pinned staging rows and one event per layer.  Not
 * thread-safe; one pool per stream pair. */
typedef struct moe_pool moe_pool_t;
MOE_API moe_status_t moe_pool_create(int32_t n_layers, int32_t E, int32_t n_slots, size_t blob_bytes,
                                     void* device_slots, int32_t* device_table,
                                     const void* host_blobs, void* stream, moe_pool_t** out);
MOE_API void moe_pool_destroy(moe_pool_t* p);
/* Modeled storage latency of the master copy (0: none, at most
 * MOE_MAX_READ_DELAY_NS, else MOE_EINVAL).  Each moe_pool_update whose plan
 * has fills starts them with one wait of this length on side_stream (the
 * step's reads are issued together and complete after one latency), and
 * moe_pool_layer reports it as read_delay_ns, so kernels that read a
 * non-resident expert on demand pay it too. */
MOE_API moe_status_t moe_pool_set_read_delay(moe_pool_t* p, uint32_t ns);
/* The moe_experts_t of one layer (counters may be NULL). */
MOE_API moe_status_t moe_pool_layer(const moe_pool_t* p, int32_t layer, unsigned long long* counters,
                                    moe_experts_t* out);
/* Plan one step (as moe_lru_plan) and enqueue it on side_stream: per layer
 * with fills, the table row without the evicted experts, event inv[layer],
 * the blob copies, then the table row with the new slots.  Waits (host) for
 * side_stream's previous work first.  Call it only after every kernel of the
 * step that produced `executed` has completed. */
MOE_API moe_status_t moe_pool_update(moe_pool_t* p, const int32_t* executed, int32_t K,
                                     const int32_t* predicted, int32_t Kp, int32_t max_fills,
                                     void* side_stream, int32_t* n_fills);
/* Make `stream` wait for the last update's invalidation of `layer` (no-op if
 * the layer had no fills since the last wait).  Call before a kernel that
 * reads the layer's table. */
MOE_API moe_status_t moe_pool_wait_layer(moe_pool_t* p, int32_t layer, void* stream);
/* Make `stream` wait until the last update's fills of `layer` are complete
 * and its table row is final (no-op if the layer had no fills since the last
 * wait): every expert the update filled for the layer is then read from its
 * slot.  Used when the next step executes the predicted experts. */
MOE_API moe_status_t moe_pool_wait_layer_filled(moe_pool_t* p, int32_t layer, void* stream);
/* Host wait for all enqueued fills. */
MOE_API moe_status_t moe_pool_sync(moe_pool_t* p, void* side_stream);
/* The pool's planner (for moe_lru_table / moe_lru_stats). */
MOE_API const moe_lru_t* moe_pool_lru(const moe_pool_t* p);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */

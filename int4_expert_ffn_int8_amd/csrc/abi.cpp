// C ABI entry points: argument validation, workspace layout, launches.
#include <math.h>
#include <string.h>

#include "launch.h"
#include "moe_internal.h"
#include "fused.h"
#include "prefill.h"
#include "status.h"
#include "workspace.h"

using namespace moe;

extern "C" const char* moe_last_error(void) { return last_error_buffer(); }

namespace {

moe_status_t check_dims(const moe_dims_t* d, const char* fn) {
  if (!d) return fail(MOE_EINVAL, "%s: dims is NULL", fn);
  if (d->H <= 0 || d->I <= 0 || d->H % kGroup || d->I % kGroup)
    return fail(MOE_EINVAL, "%s: H=%d and I=%d must be positive multiples of 64", fn, d->H, d->I);
  if (!width_supported(d->H) || !width_supported(d->I))
    return fail(MOE_EUNSUPPORTED, "%s: H=%d / I=%d not in {64,...,4096} powers of two", fn, d->H,
                d->I);
  if (d->E < 1 || d->E > kMaxE)
    return fail(MOE_EUNSUPPORTED, "%s: E=%d outside [1, %d]", fn, d->E, kMaxE);
  if (d->K < 1 || d->K > d->E) return fail(MOE_EINVAL, "%s: K=%d outside [1, E=%d]", fn, d->K, d->E);
  if (d->K > kMaxK) return fail(MOE_EUNSUPPORTED, "%s: K=%d above %d", fn, d->K, kMaxK);
  if (d->r < 0 || d->r > kMaxR)
    return fail(MOE_EUNSUPPORTED, "%s: LoRA rank r=%d outside [0, %d]", fn, d->r, kMaxR);
  if (d->n_shared != 0 && d->n_shared != 1)
    return fail(MOE_EINVAL, "%s: n_shared=%d must be 0 or 1", fn, d->n_shared);
  if (d->norm_topk != 0 && d->norm_topk != 1)
    return fail(MOE_EINVAL, "%s: norm_topk=%d must be 0 or 1", fn, d->norm_topk);
  if (!isfinite(d->lora_scale)) return fail(MOE_EINVAL, "%s: lora_scale is not finite", fn);
  return MOE_OK;
}

moe_status_t hip_status(hipError_t e, const char* fn) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_EHIP, "%s: %s", fn, hipGetErrorString(e));
}

}  // namespace

extern "C" size_t moe_workspace_bytes(const moe_dims_t* d, int32_t T, int32_t prefill) {
  if (check_dims(d, "moe_workspace_bytes") != MOE_OK || T < 0) return 0;
  return ws_layout(*d, T, prefill != 0).total;
}

extern "C" moe_status_t moe_route(const moe_dims_t* d, const int8_t* gate_q, const float* gate_s,
                                  const int8_t* sgate_q, const float* sgate_s, const uint16_t* x,
                                  int32_t T, const float* logit_bias, int32_t* topk_idx,
                                  float* topk_w, float* shared_w, float* logits, int32_t* counts,
                                  int32_t* offsets, int32_t* perm, void* ws, size_t ws_bytes,
                                  void* stream) {
  const char* fn = "moe_route";
  moe_status_t st = check_dims(d, fn);
  if (st != MOE_OK) return st;
  if (T < 0) return fail(MOE_EINVAL, "%s: T=%d is negative", fn, T);
  const int ngroup = (counts != nullptr) + (offsets != nullptr) + (perm != nullptr);
  if (ngroup != 0 && ngroup != 3)
    return fail(MOE_EINVAL, "%s: counts, offsets and perm must be all NULL or all set", fn);
  const bool group = ngroup == 3;
  if (T == 0) return MOE_OK;
  if (!gate_q || !gate_s || !x || !topk_idx || !topk_w)
    return fail(MOE_EINVAL, "%s: null gate, x or output pointer", fn);
  if (d->n_shared && (!sgate_q || !sgate_s || !shared_w))
    return fail(MOE_EINVAL, "%s: n_shared=1 needs sgate_q, sgate_s and shared_w", fn);
  const WsLayout W = ws_layout(*d, T, group);
  if (!ws || ws_bytes < W.total)
    return fail(MOE_EWORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, W.total);
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  float* lg = logits ? logits : reinterpret_cast<float*>(wsb + W.logits);
  float* sg = reinterpret_cast<float*>(wsb + W.sg);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* plog = nullptr;  // K-split partial logits, summed by the top-K kernel
  // grouping: per-chunk expert histograms, zeroed by the router kernel and
  // filled by the top-K kernel
  int32_t* hist = group ? reinterpret_cast<int32_t*>(wsb + W.chunk_hist) : nullptr;
  const int nhist = group ? ((T * d->K + kGroupChunk - 1) / kGroupChunk) * d->E : 0;
  if (T >= kRouterGemmMinT) {
    // many tokens: MFMA GEMM over int8 codes (exact in bf16), fp32 group
    // scale applied per 64-column chunk
    GemmArgs g = {};
    g.T = T;
    g.K = d->K;
    g.S = d->n_shared;
    g.E = d->E;
    g.H = d->H;
    g.I = d->I;
    g.x = x;
    g.rq = gate_q;
    g.rs = gate_s;
    g.sq = sgate_q;
    g.ss = sgate_s;
    g.bias = logit_bias;
    g.logits = lg;
    g.sg_logit = sg;
    g.plog = plog = reinterpret_cast<float*>(wsb + W.plog);
    g.zero = hist;
    g.nzero = nhist;
    st = hip_status(launch_router_gemm(g, s), fn);
  } else {
    st = hip_status(launch_router_logits(d->H, gate_q, gate_s, sgate_q, sgate_s, x, logit_bias,
                                         d->E, d->n_shared, T, lg, sg, s, hist, nhist),
                    fn);
  }
  if (st != MOE_OK) return st;
  st = hip_status(launch_topk(lg, sg, T, d->E, d->K, d->n_shared, d->norm_topk, topk_idx, topk_w,
                              shared_w, s, plog, plog ? kRouterSplit : 0, logit_bias, hist),
                  fn);
  if (st != MOE_OK || !group) return st;
  return hip_status(launch_group(topk_idx, T, d->K, d->E, counts, offsets, perm, hist, s),
                    fn);
}

namespace {

// moe_expert_forward; with y16/ey set (prefill path only) the down GEMM
// writes the compact expert outputs of moe_block_prefill instead of y.
moe_status_t expert_forward(const moe_dims_t* d, const moe_experts_t* routed,
                            const void* shared_blob, const uint16_t* x, int32_t T,
                            const int32_t* topk_idx, const int32_t* counts, const int32_t* offsets,
                            const int32_t* perm, float* y, uint16_t* y16, int32_t* ey, void* ws,
                            size_t ws_bytes, void* stream, const char* fn) {
  moe_status_t st = check_dims(d, fn);
  if (st != MOE_OK) return st;
  if (T < 0) return fail(MOE_EINVAL, "%s: T=%d is negative", fn, T);
  const int ngroup = (counts != nullptr) + (offsets != nullptr) + (perm != nullptr);
  if (ngroup != 0 && ngroup != 3)
    return fail(MOE_EINVAL, "%s: counts, offsets and perm must be all NULL or all set", fn);
  const bool group = ngroup == 3;
  if (!routed || !routed->slots) return fail(MOE_EINVAL, "%s: routed experts missing", fn);
  if (routed->expert_to_slot == nullptr && routed->n_slots < d->E)
    return fail(MOE_EINVAL, "%s: without a slot table n_slots=%d must cover E=%d experts", fn,
                routed->n_slots, d->E);
  if (routed->expert_to_slot != nullptr && routed->host_blobs == nullptr)
    return fail(MOE_EINVAL, "%s: a slot table needs host_blobs for non-resident experts", fn);
  if (routed->n_slots < 1) return fail(MOE_EINVAL, "%s: n_slots=%d", fn, routed->n_slots);
  if (d->n_shared && !shared_blob) return fail(MOE_EINVAL, "%s: n_shared=1 needs shared_blob", fn);
  if (T == 0) return MOE_OK;
  if (!x || !topk_idx || !(y || y16)) return fail(MOE_EINVAL, "%s: null x, topk_idx or y", fn);
  const WsLayout W = ws_layout(*d, T, group);
  if (!ws || ws_bytes < W.total)
    return fail(MOE_EWORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, W.total);
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  const BlobLayout L = blob_layout(d->H, d->I, d->r);
  ExpertSource src;
  src.slots = static_cast<const uint8_t*>(routed->slots);
  src.expert_to_slot = routed->expert_to_slot;
  src.host_blobs = static_cast<const uint8_t*>(routed->host_blobs);
  src.counters = routed->counters;
  src.stride = L.total;
  if (group) {
    GemmArgs g = {};
    g.T = T;
    g.K = d->K;
    g.S = d->n_shared;
    g.E = d->E;
    g.H = d->H;
    g.I = d->I;
    g.r = d->r;
    g.lam = d->lora_scale;
    g.perm = perm;
    g.offsets = offsets;
    g.gstart = reinterpret_cast<const int32_t*>(wsb + W.gstart);
    g.tstart = reinterpret_cast<const int32_t*>(wsb + W.tstart);
    g.gblob = reinterpret_cast<const unsigned long long*>(wsb + W.gblob);
    g.L = L;
    g.x = x;
    uint16_t* x16 = reinterpret_cast<uint16_t*>(wsb + W.x16);
    int32_t* ex = reinterpret_cast<int32_t*>(wsb + W.ex);
    uint16_t* hs16 = reinterpret_cast<uint16_t*>(wsb + W.hs16);
    int32_t* eh = reinterpret_cast<int32_t*>(wsb + W.eh);
    g.x16 = x16;
    g.ex = ex;
    g.hl = reinterpret_cast<uint16_t*>(wsb + W.hl);
    g.hbe = reinterpret_cast<int8_t*>(wsb + W.hbe);
    g.hmax = reinterpret_cast<uint32_t*>(wsb + W.hmax);
    g.hs = hs16;
    g.eh = eh;
    g.ud = g.ud_out = reinterpret_cast<uint16_t*>(wsb + W.pud);
    g.upart = reinterpret_cast<float*>(wsb + W.upart);
    g.y = y;
    g.y16 = y16;
    g.ey = ey;
    return hip_status(launch_prefill_experts(g, counts, src,
                                             static_cast<const uint8_t*>(shared_blob), x16, ex,
                                             hs16, eh, static_cast<hipStream_t>(stream)),
                      fn);
  }
  DecodeArgs a;
  a.x = x;
  a.topk_idx = topk_idx;
  a.T = T;
  a.H = d->H;
  a.I = d->I;
  a.K = d->K;
  a.E = d->E;
  a.S = d->n_shared;
  a.r = d->r;
  a.lam = d->lora_scale;
  a.L = L;
  a.src = src;
  a.shared_blob = static_cast<const uint8_t*>(shared_blob);
  a.blobptr = reinterpret_cast<unsigned long long*>(wsb + W.blobptr);
  a.u = reinterpret_cast<float*>(wsb + W.u);
  a.h = reinterpret_cast<float*>(wsb + W.h);
  a.vpart = reinterpret_cast<float*>(wsb + W.vpart);
  a.y = y;
  return hip_status(launch_decode(a, static_cast<hipStream_t>(stream)), fn);
}

}  // namespace

extern "C" moe_status_t moe_expert_forward(const moe_dims_t* d, const moe_experts_t* routed,
                                           const void* shared_blob, const uint16_t* x, int32_t T,
                                           const int32_t* topk_idx, const int32_t* counts,
                                           const int32_t* offsets, const int32_t* perm, float* y,
                                           void* ws, size_t ws_bytes, void* stream) {
  return expert_forward(d, routed, shared_blob, x, T, topk_idx, counts, offsets, perm, y, nullptr,
                        nullptr, ws, ws_bytes, stream, "moe_expert_forward");
}

extern "C" moe_status_t moe_combine(const moe_dims_t* d, const float* y, const float* topk_w,
                                    const float* shared_w, int32_t T, const uint16_t* residual,
                                    uint16_t* out, uint16_t* norm_out, float eps, void* stream) {
  const char* fn = "moe_combine";
  moe_status_t st = check_dims(d, fn);
  if (st != MOE_OK) return st;
  if (T < 0) return fail(MOE_EINVAL, "%s: T=%d is negative", fn, T);
  if (T == 0) return MOE_OK;
  if (!y || !topk_w || !out) return fail(MOE_EINVAL, "%s: null y, topk_w or out", fn);
  if (d->n_shared && !shared_w) return fail(MOE_EINVAL, "%s: n_shared=1 needs shared_w", fn);
  if (norm_out && !(eps >= 0.f && isfinite(eps)))
    return fail(MOE_EINVAL, "%s: eps must be finite and >= 0", fn);
  return hip_status(launch_combine(y, topk_w, shared_w, T, d->K, d->n_shared, d->H, residual, out,
                                   norm_out, eps, static_cast<hipStream_t>(stream)),
                    fn);
}

extern "C" moe_status_t moe_rmsnorm(const uint16_t* h, int32_t T, int32_t H, float eps,
                                    uint16_t* out, void* stream) {
  const char* fn = "moe_rmsnorm";
  if (T < 0 || H <= 0) return fail(MOE_EINVAL, "%s: T=%d, H=%d", fn, T, H);
  if (!(eps >= 0.f && isfinite(eps))) return fail(MOE_EINVAL, "%s: eps must be finite and >= 0", fn);
  if (T == 0) return MOE_OK;
  if (!h || !out) return fail(MOE_EINVAL, "%s: null pointer", fn);
  return hip_status(launch_rmsnorm(h, T, H, eps, out, static_cast<hipStream_t>(stream)), fn);
}

// ---------------------------------------------------------------------------
// one-call prefill block
// ---------------------------------------------------------------------------
extern "C" size_t moe_block_prefill_workspace_bytes(const moe_dims_t* d, int32_t T) {
  if (check_dims(d, "moe_block_prefill_workspace_bytes") != MOE_OK || T < 0) return 0;
  return block_prefill_layout(*d, T).total;
}

extern "C" moe_status_t moe_block_prefill(const moe_dims_t* d, const int8_t* gate_q,
                                          const float* gate_s, const int8_t* sgate_q,
                                          const float* sgate_s, const float* logit_bias,
                                          const moe_experts_t* routed, const void* shared_blob,
                                          const uint16_t* x, int32_t T, const uint16_t* residual,
                                          int32_t* topk_idx, float* topk_w, uint16_t* out,
                                          uint16_t* norm_out, float eps, void* ws, size_t ws_bytes,
                                          void* stream) {
  const char* fn = "moe_block_prefill";
  moe_status_t st = check_dims(d, fn);
  if (st != MOE_OK) return st;
  if (T < 0) return fail(MOE_EINVAL, "%s: T=%d is negative", fn, T);
  if (T == 0) return MOE_OK;
  if (!x || !topk_idx || !topk_w || !out) return fail(MOE_EINVAL, "%s: null x or output pointer", fn);
  if (norm_out && !(eps >= 0.f && isfinite(eps)))
    return fail(MOE_EINVAL, "%s: eps must be finite and >= 0", fn);
  const BlockPrefillLayout P = block_prefill_layout(*d, T);
  if (!ws || ws_bytes < P.total)
    return fail(MOE_EWORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, P.total);
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  int32_t* counts = reinterpret_cast<int32_t*>(wsb + P.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(wsb + P.offsets);
  int32_t* perm = reinterpret_cast<int32_t*>(wsb + P.perm);
  float* shared_w = d->n_shared ? reinterpret_cast<float*>(wsb + P.shared_w) : nullptr;
  uint16_t* y16 = reinterpret_cast<uint16_t*>(wsb + P.y16);
  int32_t* ey = reinterpret_cast<int32_t*>(wsb + P.ey);
  st = moe_route(d, gate_q, gate_s, sgate_q, sgate_s, x, T, logit_bias, topk_idx, topk_w, shared_w,
                 nullptr, counts, offsets, perm, ws, P.W.total, stream);
  if (st != MOE_OK) return st;
  st = expert_forward(d, routed, shared_blob, x, T, topk_idx, counts, offsets, perm, nullptr, y16,
                      ey, ws, P.W.total, stream, fn);
  if (st != MOE_OK) return st;
  return hip_status(launch_combine16(y16, ey, topk_w, shared_w, T, d->K, d->n_shared, d->H,
                                     residual, out, norm_out, eps, static_cast<hipStream_t>(stream)),
                    fn);
}

// ---------------------------------------------------------------------------
// fused single-launch decode block
// ---------------------------------------------------------------------------
extern "C" size_t moe_block_decode_workspace_bytes(const moe_dims_t* d, int32_t T) {
  if (check_dims(d, "moe_block_decode_workspace_bytes") != MOE_OK || T < 0) return 0;
  return fused_ws_layout(T, d->E, d->K, d->n_shared, d->I, d->r).total;
}

extern "C" moe_status_t moe_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "moe_workspace_init";
  if (!ws || ws_bytes < kSyncBytes || ws_bytes % 4)
    return fail(MOE_EINVAL, "%s: workspace must hold at least %zu bytes (a multiple of 4)", fn,
                kSyncBytes);
  return hip_status(launch_zero_ints(static_cast<int*>(ws), int(ws_bytes / 4),
                                     static_cast<hipStream_t>(stream)),
                    fn);
}

namespace moe {

uint32_t wall_ticks(uint32_t ns) {
  if (ns == 0) return 0;
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0) {
    (void)hipGetLastError();
    khz = 100000;  // the 100 MHz constant-rate clock of CDNA parts
  }
  const uint64_t t = (uint64_t(ns) * uint64_t(khz) + 999999u) / 1000000u;
  return uint32_t(t > 0xFFFFFFFFull ? 0xFFFFFFFFull : t);
}

}  // namespace moe

namespace moe {

moe_status_t block_decode_check(const char* fn, const moe_dims_t* d, const int8_t* gate_q,
                                const float* gate_s, const int8_t* sgate_q, const float* sgate_s,
                                const moe_experts_t* routed, const void* shared_blob,
                                const uint16_t* h_in, int32_t T, int32_t flags, float eps,
                                uint16_t* out) {
  moe_status_t st = check_dims(d, fn);
  if (st != MOE_OK) return st;
  if (T < 0) return fail(MOE_EINVAL, "%s: T=%d is negative", fn, T);
  if (flags & ~(MOE_DECODE_NORM_INPUT | MOE_DECODE_RESIDUAL))
    return fail(MOE_EINVAL, "%s: unknown flags 0x%x", fn, flags);
  if (!fused_shape_supported(d->H, d->I, d->r))
    return fail(MOE_EUNSUPPORTED,
                "%s: H=%d, I=%d, r=%d (H in 256..2048, I in 128..2048, r <= H/32 and I/32)", fn,
                d->H, d->I, d->r);
  if (T > kFusedMaxT || T * (d->K + d->n_shared) > kFusedMaxP)
    return fail(MOE_EUNSUPPORTED, "%s: T=%d with K+shared=%d exceeds %d tokens / %d pairs", fn,
                T, d->K + d->n_shared, kFusedMaxT, kFusedMaxP);
  if (!routed || !routed->slots) return fail(MOE_EINVAL, "%s: routed experts missing", fn);
  if (routed->expert_to_slot == nullptr && routed->n_slots < d->E)
    return fail(MOE_EINVAL, "%s: without a slot table n_slots=%d must cover E=%d experts", fn,
                routed->n_slots, d->E);
  if (routed->expert_to_slot != nullptr && routed->host_blobs == nullptr)
    return fail(MOE_EINVAL, "%s: a slot table needs host_blobs for non-resident experts", fn);
  if (d->n_shared && (!shared_blob || !sgate_q || !sgate_s))
    return fail(MOE_EINVAL, "%s: n_shared=1 needs shared_blob, sgate_q and sgate_s", fn);
  if ((flags & MOE_DECODE_NORM_INPUT) && !(eps >= 0.f && isfinite(eps)))
    return fail(MOE_EINVAL, "%s: eps must be finite and >= 0", fn);
  if (routed->read_delay_ns > MOE_MAX_READ_DELAY_NS)
    return fail(MOE_EINVAL, "%s: read_delay_ns=%u exceeds %u", fn, routed->read_delay_ns,
                MOE_MAX_READ_DELAY_NS);
  if (T == 0) return MOE_OK;
  if (!gate_q || !gate_s || !h_in || !out) return fail(MOE_EINVAL, "%s: null pointer", fn);
  return MOE_OK;
}

moe_status_t block_decode_launch(const char* fn, const moe_dims_t* d, const int8_t* gate_q,
                                 const float* gate_s, const int8_t* sgate_q, const float* sgate_s,
                                 const moe_experts_t* routed, const void* shared_blob,
                                 const uint16_t* h_in, int32_t T, int32_t flags, float eps,
                                 const int32_t* exec_idx, int32_t* topk_idx, float* topk_w,
                                 uint16_t* out, void* ws, size_t ws_bytes, int32_t* err_out,
                                 void* stream) {
  const FusedWs W = fused_ws_layout(T, d->E, d->K, d->n_shared, d->I, d->r);
  if (!ws || ws_bytes < W.total)
    return fail(MOE_EWORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, W.total);
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  FusedArgs a = {};
  a.T = T;
  a.E = d->E;
  a.K = d->K;
  a.S = d->n_shared;
  a.r = d->r;
  a.H = d->H;
  a.I = d->I;
  a.norm_topk = d->norm_topk;
  a.lam = d->lora_scale;
  a.eps = eps;
  a.norm_input = (flags & MOE_DECODE_NORM_INPUT) != 0;
  a.residual = (flags & MOE_DECODE_RESIDUAL) != 0;
  a.rq = gate_q;
  a.rs = gate_s;
  a.sq = sgate_q;
  a.ss = sgate_s;
  a.L = blob_layout(d->H, d->I, d->r);
  a.src.slots = static_cast<const uint8_t*>(routed->slots);
  a.src.expert_to_slot = routed->expert_to_slot;
  a.src.host_blobs = static_cast<const uint8_t*>(routed->host_blobs);
  a.src.counters = routed->counters;
  a.src.stride = a.L.total;
  a.src.delay_ticks = routed->expert_to_slot ? wall_ticks(routed->read_delay_ns) : 0;
  a.shared_blob = static_cast<const uint8_t*>(shared_blob);
  a.h_in = h_in;
  a.out = out;
  a.user_idx = topk_idx;
  a.user_w = topk_w;
  a.exec_idx = exec_idx;
  a.err_out = err_out;
  a.sync = reinterpret_cast<int*>(wsb + W.sync);
  a.logits = reinterpret_cast<tword_t*>(wsb + W.logits);
  a.route = reinterpret_cast<tword_t*>(wsb + W.route);
  a.wts = reinterpret_cast<tword_t*>(wsb + W.wts);
  a.u = reinterpret_cast<tword_t*>(wsb + W.u);
  a.h = reinterpret_cast<tword_t*>(wsb + W.h);
  a.hexp = reinterpret_cast<tword_t*>(wsb + W.hexp);
  a.vpart = reinterpret_cast<tword_t*>(wsb + W.vpart);
  a.v = reinterpret_cast<tword_t*>(wsb + W.v);
  return hip_status(launch_fused(a, static_cast<hipStream_t>(stream)), fn);
}

}  // namespace moe

namespace {

moe_status_t block_decode(const char* fn, const moe_dims_t* d, const int8_t* gate_q,
                          const float* gate_s, const int8_t* sgate_q, const float* sgate_s,
                          const moe_experts_t* routed, const void* shared_blob,
                          const uint16_t* h_in, int32_t T, int32_t flags, float eps,
                          const int32_t* exec_idx, int32_t* topk_idx, float* topk_w,
                          uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = block_decode_check(fn, d, gate_q, gate_s, sgate_q, sgate_s, routed,
                                       shared_blob, h_in, T, flags, eps, out);
  if (st != MOE_OK || T == 0) return st;
  return block_decode_launch(fn, d, gate_q, gate_s, sgate_q, sgate_s, routed, shared_blob, h_in, T,
                             flags, eps, exec_idx, topk_idx, topk_w, out, ws, ws_bytes, nullptr,
                             stream);
}

}  // namespace

extern "C" moe_status_t moe_block_decode(const moe_dims_t* d, const int8_t* gate_q,
                                         const float* gate_s, const int8_t* sgate_q,
                                         const float* sgate_s, const moe_experts_t* routed,
                                         const void* shared_blob, const uint16_t* h_in, int32_t T,
                                         int32_t flags, float eps, int32_t* topk_idx,
                                         float* topk_w, uint16_t* out, void* ws, size_t ws_bytes,
                                         void* stream) {
  return block_decode("moe_block_decode", d, gate_q, gate_s, sgate_q, sgate_s, routed,
                      shared_blob, h_in, T, flags, eps, nullptr, topk_idx, topk_w, out, ws,
                      ws_bytes, stream);
}

extern "C" moe_status_t moe_block_decode_exec(const moe_dims_t* d, const int8_t* gate_q,
                                              const float* gate_s, const int8_t* sgate_q,
                                              const float* sgate_s, const moe_experts_t* routed,
                                              const void* shared_blob, const uint16_t* h_in,
                                              int32_t T, int32_t flags, float eps,
                                              const int32_t* exec_idx, int32_t* topk_idx,
                                              float* topk_w, uint16_t* out, void* ws,
                                              size_t ws_bytes, void* stream) {
  if (T > 0 && exec_idx == nullptr)
    return fail(MOE_EINVAL, "moe_block_decode_exec: exec_idx is NULL");
  return block_decode("moe_block_decode_exec", d, gate_q, gate_s, sgate_q, sgate_s, routed,
                      shared_blob, h_in, T, flags, eps, exec_idx, topk_idx, topk_w, out, ws,
                      ws_bytes, stream);
}

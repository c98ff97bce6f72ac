// Prerouter head: z = W2 silu(W1 h), prediction = top-K of z.
//
// [P1] "Edge0开源框架实现35BMoE模型在Mac上流式推理…", Prerouter paragraph: a
// light MLP head predicts the next layer's top-K experts so that loading can
// overlap compute.  [P2] "SSD 专家卸载 · Prerouter 路由预测", double-shift
// paragraph: the head after layer N predicts layer N+1 for the next token.
#include <math.h>

#include "device_utils.h"
#include "launch.h"
#include "moe_internal.h"
#include "status.h"

namespace moe {

// a[t, d] = silu(sum_i W1[d, i] h[t, i] + sum_k W1[d, H + prev[t, k]]).
// W1 rows are ldw >= H wide; the second sum (the one-hot of the experts the
// layer executed, appended to h) is empty when prev is NULL.
// grid (ceil(D / (4 RPL)), T).
template <int H>
__global__ void __launch_bounds__(256) k_prerouter_l1(const uint16_t* __restrict__ W1, int ldw,
                                                       const uint16_t* __restrict__ h, int D,
                                                       const int32_t* __restrict__ prev, int Kp,
                                                       int E, float* __restrict__ a) {
  using G = Geo<H>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, sub = lane % G::LPR;
  const int t = blockIdx.y;
  const int row = (blockIdx.x * 4 + wave) * G::RPL + lane / G::LPR;
  float acc = 0.f;
  if (row < D) {
#pragma unroll
    for (int c = 0; c < G::SL; ++c) {
      const int col0 = 32 * sub + 2048 * c;
      const uint4* wp = reinterpret_cast<const uint4*>(W1 + size_t(row) * ldw + col0);
      const uint4* hp = reinterpret_cast<const uint4*>(h + size_t(t) * H + col0);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint4 wv = wp[k], hv = hp[k];
        acc = dot2_bf16(wv.x, hv.x, acc);
        acc = dot2_bf16(wv.y, hv.y, acc);
        acc = dot2_bf16(wv.z, hv.z, acc);
        acc = dot2_bf16(wv.w, hv.w, acc);
      }
    }
  }
  acc = group_sum<G::LPR>(acc);
  if (row < D && sub == 0) {
    for (int k = 0; k < Kp; ++k) {  // one-hot features: column H + expert id
      const int e = prev[size_t(t) * Kp + k];
      if (e >= 0 && e < E) acc += bf16_to_f32(W1[size_t(row) * ldw + H + e]);
    }
    a[size_t(t) * D + row] = silu_f(acc);
  }
}

// z[t, e] = sum_d W2[e, d] a[t, d] (a kept in fp32).  grid (ceil(E / (4 RPL)), T).
template <int D>
__global__ void __launch_bounds__(256) k_prerouter_l2(const uint16_t* __restrict__ W2,
                                                       const float* __restrict__ a, int E,
                                                       float* __restrict__ z) {
  using G = Geo<D>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, sub = lane % G::LPR;
  const int t = blockIdx.y;
  const int row = (blockIdx.x * 4 + wave) * G::RPL + lane / G::LPR;
  float acc = 0.f;
  if (row < E) {
#pragma unroll
    for (int c = 0; c < G::SL; ++c) {
      const int col0 = 32 * sub + 2048 * c;
      const uint4* wp = reinterpret_cast<const uint4*>(W2 + size_t(row) * D + col0);
      const float4* ap = reinterpret_cast<const float4*>(a + size_t(t) * D + col0);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint4 wv = wp[k];
        const float4 a0 = ap[2 * k], a1 = ap[2 * k + 1];
        acc = fmaf(bf16_lo(wv.x), a0.x, acc);
        acc = fmaf(bf16_hi(wv.x), a0.y, acc);
        acc = fmaf(bf16_lo(wv.y), a0.z, acc);
        acc = fmaf(bf16_hi(wv.y), a0.w, acc);
        acc = fmaf(bf16_lo(wv.z), a1.x, acc);
        acc = fmaf(bf16_hi(wv.z), a1.y, acc);
        acc = fmaf(bf16_lo(wv.w), a1.z, acc);
        acc = fmaf(bf16_hi(wv.w), a1.w, acc);
      }
    }
  }
  acc = group_sum<G::LPR>(acc);
  if (row < E && sub == 0) z[size_t(t) * E + row] = acc;
}

template <int H>
static void launch_l1(const uint16_t* W1, int ldw, const uint16_t* h, int D, const int32_t* prev,
                      int Kp, int E, int T, float* a, hipStream_t st) {
  using G = Geo<H>;
  hipLaunchKernelGGL(k_prerouter_l1<H>, dim3((D + 4 * G::RPL - 1) / (4 * G::RPL), T), dim3(256),
                     0, st, W1, ldw, h, D, prev, Kp, E, a);
}

template <int D>
static void launch_l2(const uint16_t* W2, const float* a, int E, int T, float* z,
                      hipStream_t st) {
  using G = Geo<D>;
  hipLaunchKernelGGL(k_prerouter_l2<D>, dim3((E + 4 * G::RPL - 1) / (4 * G::RPL), T), dim3(256),
                     0, st, W2, a, E, z);
}

}  // namespace moe

using namespace moe;

extern "C" size_t prerouter_workspace_bytes(int32_t D, int32_t E, int32_t T) {
  if (D <= 0 || E <= 0 || T < 0) return 0;
  return align256(size_t(T) * D * 4) + align256(size_t(T) * E * 4) +
         align256(size_t(T) * kMaxK * 4) + 256;
}

static moe_status_t prerouter_run(const char* fn, const uint16_t* W1, int ldw, const uint16_t* W2,
                                  int32_t H, int32_t D, int32_t E, int32_t K, const uint16_t* h,
                                  const int32_t* prev, int32_t Kp, int32_t T, int32_t* pred_idx,
                                  float* pred_logits, void* ws, size_t ws_bytes, void* stream) {
  if (H <= 0 || D <= 0 || H % kGroup || D % kGroup)
    return fail(MOE_EINVAL, "%s: H=%d, D=%d must be positive multiples of 64", fn, H, D);
  if (!width_supported(H) || !width_supported(D))
    return fail(MOE_EUNSUPPORTED, "%s: H=%d / D=%d not in {64,...,4096} powers of two", fn, H, D);
  if (E < 1 || E > kMaxE) return fail(MOE_EUNSUPPORTED, "%s: E=%d outside [1, %d]", fn, E, kMaxE);
  if (K < 1 || K > E || K > kMaxK)
    return fail(MOE_EINVAL, "%s: K=%d outside [1, min(E, %d)]", fn, K, kMaxK);
  if (Kp < 0 || Kp > kMaxK) return fail(MOE_EINVAL, "%s: Kp=%d outside [0, %d]", fn, Kp, kMaxK);
  if (T < 0) return fail(MOE_EINVAL, "%s: T=%d is negative", fn, T);
  if (T == 0) return MOE_OK;
  if (!W1 || !W2 || !h || !pred_idx || (Kp > 0 && !prev)) return fail(MOE_EINVAL, "%s: null pointer", fn);
  const size_t need = prerouter_workspace_bytes(D, E, T);
  if (!ws || ws_bytes < need)
    return fail(MOE_EWORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  float* a = reinterpret_cast<float*>(wsb);
  float* z = pred_logits ? pred_logits : reinterpret_cast<float*>(wsb + align256(size_t(T) * D * 4));
  float* wts = reinterpret_cast<float*>(wsb + align256(size_t(T) * D * 4) + align256(size_t(T) * E * 4));
  hipStream_t st = static_cast<hipStream_t>(stream);
#define MOE_CASE(V)                                               \
  case V:                                                         \
    launch_l1<V>(W1, ldw, h, D, prev, Kp, E, T, a, st);           \
    break;
  switch (H) { MOE_FOR_EACH_WIDTH(MOE_CASE) }
#undef MOE_CASE
#define MOE_CASE(V)                        \
  case V:                                  \
    launch_l2<V>(W2, a, E, T, z, st);      \
    break;
  switch (D) { MOE_FOR_EACH_WIDTH(MOE_CASE) }
#undef MOE_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MOE_EHIP, "%s: %s", fn, hipGetErrorString(e));
  // ranking only: weights go to scratch, no shared gate
  e = launch_topk(z, nullptr, T, E, K, 0, 1, pred_idx, wts, nullptr, st);
  if (e != hipSuccess) return fail(MOE_EHIP, "%s: %s", fn, hipGetErrorString(e));
  return MOE_OK;
}

extern "C" moe_status_t prerouter_predict(const uint16_t* W1, const uint16_t* W2, int32_t H,
                                          int32_t D, int32_t E, int32_t K, const uint16_t* h,
                                          int32_t T, int32_t* pred_idx, float* pred_logits,
                                          void* ws, size_t ws_bytes, void* stream) {
  return prerouter_run("prerouter_predict", W1, H, W2, H, D, E, K, h, nullptr, 0, T, pred_idx,
                       pred_logits, ws, ws_bytes, stream);
}

extern "C" moe_status_t prerouter_predict_feat(const uint16_t* W1, const uint16_t* W2, int32_t H,
                                               int32_t D, int32_t E, int32_t K, const uint16_t* h,
                                               const int32_t* prev_idx, int32_t Kp, int32_t T,
                                               int32_t* pred_idx, float* pred_logits, void* ws,
                                               size_t ws_bytes, void* stream) {
  return prerouter_run("prerouter_predict_feat", W1, H + E, W2, H, D, E, K, h, prev_idx, Kp, T,
                       pred_idx, pred_logits, ws, ws_bytes, stream);
}

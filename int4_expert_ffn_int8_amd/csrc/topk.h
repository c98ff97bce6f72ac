// Wave-level top-K expert selection for one token.
//
// [P2] "SSD 专家卸载 · Prerouter 路由预测", tier table: each token keeps K of
// the E routed experts, those with the largest gate logits.  Here lane l of a
// wave holds the logits of experts l, l + 64, ...; experts are taken in order
// of logit (descending), equal logits by expert index (ascending), which makes
// the selection unique.  A NaN logit ranks as -infinity, so every selection
// is K distinct experts in [0, E) whatever the input.
#pragma once

#include "device_utils.h"

namespace moe {

constexpr uint32_t kNoExpert = 0xFFFFFFFFu;

// (va, ea) ranks before (vb, eb): larger logit, then smaller index
__device__ __forceinline__ bool topk_before(float va, uint32_t ea, float vb, uint32_t eb) {
  return va > vb || (va == vb && ea < eb);
}

// For MP <= 4 logits per lane: each lane sorts its own entries once; a round
// is then one wave max over the lanes' heads, one wave min over the indices
// that reach it, and a shift in the winning lane.  emit(k, logit, expert) is
// called with wave-uniform arguments for k = 0 .. K-1.
template <int MP, typename Emit>
__device__ __forceinline__ void topk_wave_sorted(const float* vin, int E, int K, int lane, Emit&& emit) {
  static_assert(MP >= 1 && MP <= 4, "sorted top-K holds at most 4 logits per lane");
  float v[MP];
  uint32_t e[MP];
#pragma unroll
  for (int m = 0; m < MP; ++m) {
    const uint32_t idx = uint32_t(lane + 64 * m);
    const bool ok = idx < uint32_t(E);
    v[m] = (ok && !isnan(vin[m])) ? vin[m] : -INFINITY;
    e[m] = ok ? idx : kNoExpert;
  }
#pragma unroll
  for (int i = 1; i < MP; ++i)
#pragma unroll
    for (int j = i; j > 0; --j) {
      const bool sw = topk_before(v[j], e[j], v[j - 1], e[j - 1]);
      const float tv = v[j];
      const uint32_t te = e[j];
      v[j] = sw ? v[j - 1] : v[j];
      e[j] = sw ? e[j - 1] : e[j];
      v[j - 1] = sw ? tv : v[j - 1];
      e[j - 1] = sw ? te : e[j - 1];
    }
  for (int k = 0; k < K; ++k) {
    const float mx = wave_max(v[0]);
    const uint32_t sel = wave_min_u32(v[0] == mx ? e[0] : kNoExpert);
    if (e[0] == sel) {
#pragma unroll
      for (int m = 0; m + 1 < MP; ++m) {
        v[m] = v[m + 1];
        e[m] = e[m + 1];
      }
      v[MP - 1] = -INFINITY;
      e[MP - 1] = kNoExpert;
    }
    emit(k, mx, sel);
  }
}

// Any MP: K rounds of a lane-local scan over the entries not yet taken.
template <int MP, typename Emit>
__device__ __forceinline__ void topk_wave_scan(const float* vin, int E, int K, int lane, Emit&& emit) {
  uint32_t alive = 0;
#pragma unroll
  for (int m = 0; m < MP; ++m)
    if (lane + 64 * m < E) alive |= 1u << m;
  for (int k = 0; k < K; ++k) {
    float bv = -INFINITY;
    uint32_t be = kNoExpert;
#pragma unroll
    for (int m = 0; m < MP; ++m) {  // ascending index keeps the lowest among equal logits
      const float x = isnan(vin[m]) ? -INFINITY : vin[m];
      if (64 * m < E && ((alive >> m) & 1) && (be == kNoExpert || x > bv)) {
        bv = x;
        be = uint32_t(lane + 64 * m);
      }
    }
    const float mx = wave_max(bv);
    const uint32_t sel = wave_min_u32((be != kNoExpert && bv == mx) ? be : kNoExpert);
    if ((sel & 63) == uint32_t(lane)) alive &= ~(1u << (sel >> 6));
    emit(k, mx, sel);
  }
}

// Dispatch on E: vin holds MPMAX entries per lane (only ceil(E/64) are read).
template <int MPMAX, typename Emit>
__device__ __forceinline__ void topk_wave(const float (&vin)[MPMAX], int E, int K, int lane, Emit&& emit) {
  if (E <= 64)
    topk_wave_sorted<1>(vin, E, K, lane, emit);
  else if (E <= 128)
    topk_wave_sorted<2>(vin, E, K, lane, emit);
  else if (E <= 256)
    topk_wave_sorted<4>(vin, E, K, lane, emit);
  else
    topk_wave_scan<MPMAX>(vin, E, K, lane, emit);
}

}  // namespace moe

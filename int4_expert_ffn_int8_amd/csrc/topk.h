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

// For MP <= 4 logits per lane.  Each entry becomes one unsigned key that
// orders like its logit (NaN as -infinity; 0, below every logit, marks an
// empty entry), and each lane sorts its entries once by (key desc, index
// asc).  A round is then one wave max over the lanes' head keys; the winner
// is the only lane holding that key (read from a ballot) or, when several
// lanes tie, the one with the lowest index; the winning lane shifts its list.
// emit(k, logit, expert) is called with wave-uniform arguments for
// k = 0 .. K-1.
template <int MP, typename Emit>
__device__ __forceinline__ void topk_wave_sorted(const float* vin, int E, int K, int lane, Emit&& emit) {
  static_assert(MP >= 1 && MP <= 4, "sorted top-K holds at most 4 logits per lane");
  uint32_t key[MP];
  uint32_t e[MP];
  constexpr uint32_t kNegInfKey = 0x007FFFFFu;  // f32_order_key(-infinity)
#pragma unroll
  for (int m = 0; m < MP; ++m) {
    const uint32_t idx = uint32_t(lane + 64 * m);
    const bool ok = idx < uint32_t(E);
    // -0 + 0 is +0, so -0 and +0 give one key (a tie, as compared); a NaN
    // stays a NaN and ranks as -infinity (selects, no branches)
    const float x = vin[m] + 0.0f;
    const uint32_t kx = f32_order_key(x);
    key[m] = ok ? (x != x ? kNegInfKey : kx) : 0u;
    e[m] = ok ? idx : kNoExpert;
  }
  // lane-local insertion sort; entries of a lane have ascending indices, so a
  // strict key comparison keeps equal keys in index order
#pragma unroll
  for (int i = 1; i < MP; ++i)
#pragma unroll
    for (int j = i; j > 0; --j) {
      const bool sw = key[j] > key[j - 1];
      const uint32_t tk = key[j], te = e[j];
      key[j] = sw ? key[j - 1] : key[j];
      e[j] = sw ? e[j - 1] : e[j];
      key[j - 1] = sw ? tk : key[j - 1];
      e[j - 1] = sw ? te : e[j - 1];
    }
  for (int k = 0; k < K; ++k) {
    const uint32_t kmax = wave_max_u32(key[0]);
    const unsigned long long m = __ballot(key[0] == kmax);
    const uint32_t sel = ((m & (m - 1)) == 0)  // one lane holds it (m != 0)
                             ? uint32_t(__builtin_amdgcn_readlane(int(e[0]), __builtin_ctzll(m)))
                             : wave_min_u32(key[0] == kmax ? e[0] : kNoExpert);
    if (e[0] == sel) {
#pragma unroll
      for (int j = 0; j + 1 < MP; ++j) {
        key[j] = key[j + 1];
        e[j] = e[j + 1];
      }
      key[MP - 1] = 0u;
      e[MP - 1] = kNoExpert;
    }
    emit(k, f32_from_order_key(kmax), sel);
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

// Dispatch on E: vin holds MPMAX entries per lane (only ceil(E/64) are read;
// E <= 64 MPMAX).
template <int MPMAX, typename Emit>
__device__ __forceinline__ void topk_wave(const float (&vin)[MPMAX], int E, int K, int lane, Emit&& emit) {
  static_assert(MPMAX >= 4, "room for the sorted lists of E <= 256");
  if constexpr (MPMAX > 4) {
    if (E > 256) {
      topk_wave_scan<MPMAX>(vin, E, K, lane, emit);
      return;
    }
  }
  if (E <= 64)
    topk_wave_sorted<1>(vin, E, K, lane, emit);
  else if (E <= 128)
    topk_wave_sorted<2>(vin, E, K, lane, emit);
  else
    topk_wave_sorted<4>(vin, E, K, lane, emit);
}

}  // namespace moe

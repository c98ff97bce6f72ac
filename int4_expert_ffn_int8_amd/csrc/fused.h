// Fused single-launch decode block: arguments, workspace and hand-off words.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"
#include "moe_internal.h"

namespace moe {

constexpr int kFusedMaxT = 4;    // tokens per fused call
constexpr int kFusedMaxP = 8;    // (token, slot) pairs per fused call
constexpr int kFusedJW = 32;     // gate/up outputs per workgroup
constexpr unsigned kFusedSpinLimit = 1u << 20;  // bounded waits (~0.2 s)

// Control words at the start of the fused workspace, one 256-byte slot each.
// The launch epoch is bumped by the last workgroup of every launch; all
// hand-off data is tagged with (epoch + 1), so words left by earlier launches
// never look valid and nothing needs clearing between launches.
constexpr int kSlotInts = 64;
constexpr int kSlotEpoch = 0;
constexpr int kSlotDone = 1;
constexpr int kSlotErr = 2;  // sticky: 1 after a timed-out wait
constexpr int kNumSlots = 3;
constexpr size_t kSyncBytes = size_t(kNumSlots) * kSlotInts * 4;
static_assert(kSyncBytes == MOE_DECODE_SYNC_BYTES, "header constant");
static_assert(kSlotErr * kSlotInts * 4 == MOE_DECODE_ERR_OFFSET, "header constant");

// A hand-off word: tag in the high 32 bits, payload bits in the low 32.
typedef unsigned long long tword_t;

struct FusedArgs {
  int T, E, K, S, r, H, I, norm_topk;
  float lam, eps;
  int norm_input, residual;
  const int8_t* rq;
  const float* rs;
  const int8_t* sq;
  const float* ss;
  ExpertSource src;
  const uint8_t* shared_blob;
  BlobLayout L;
  const uint16_t* h_in;  // [T][H] bf16
  uint16_t* out;         // [T][H] bf16
  int32_t* user_idx;     // [T][K] or null
  float* user_w;         // [T][K] or null
  const int32_t* exec_idx;  // [T][K] experts to execute (prediction-as-routing) or null
  // workspace
  int* sync;
  tword_t* logits;  // [T][E + 1]   router logits; column E: shared-gate logit
  tword_t* route;   // [T][K]       expert ids
  tword_t* wts;     // [T][K + 1]   routing weights; column K: shared gate
  tword_t* u;       // [P][2r]      A_gate x, A_up x
  tword_t* h;       // [P][I / 2]   fp16 pairs of h * 2^-e
  tword_t* hexp;    // [P][I / 32]  e of each 32-column block of h
  tword_t* vpart;   // [P][I / kFusedJW][r]
  // grid layout (filled by the launcher)
  int nR, nWA, nBG, nD, base_la, base_gu, base_dn, total;
};

struct FusedWs {
  size_t sync, logits, route, wts, u, h, hexp, vpart, total;
};

inline FusedWs fused_ws_layout(int T, int E, int K, int S, int I, int r) {
  FusedWs W;
  const size_t P = size_t(T) * (K + S);
  size_t o = 0;
  W.sync = o;   o = align256(o + kSyncBytes);
  W.logits = o; o = align256(o + size_t(T) * (E + 1) * 8);
  W.route = o;  o = align256(o + size_t(T) * K * 8);
  W.wts = o;    o = align256(o + size_t(T) * (K + 1) * 8);
  W.u = o;      o = align256(o + P * 2 * r * 8);
  W.h = o;      o = align256(o + P * (I / 2) * 8);
  W.hexp = o;   o = align256(o + P * (I / 32) * 8);
  W.vpart = o;  o = align256(o + P * (I / kFusedJW) * r * 8);
  W.total = o;
  return W;
}

bool fused_shape_supported(int H, int I, int r);
hipError_t launch_fused(const FusedArgs& a, hipStream_t st);
hipError_t launch_zero_ints(int* p, int n, hipStream_t st);

}  // namespace moe

// Fused single-launch decode block: arguments, workspace and hand-off words.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"
#include "handoff.h"
#include "moe_internal.h"

namespace moe {

constexpr int kFusedMaxT = 4;    // tokens per fused call
constexpr int kFusedMaxP = 8;    // (token, slot) pairs per fused call
constexpr int kFusedJW = 16;     // gate/up outputs per workgroup = columns per h exponent
constexpr int kCopies = 8;       // copies of each broadcast hand-off word (one per XCD)
constexpr unsigned kFusedSpinLimit = 1u << 20;  // bounded waits (~0.2 s)
// routed gate/up code bytes of a launch (T K I H) from which the down
// workgroups defer their routed rows
constexpr uint64_t kDeferDownBytes = uint64_t(1) << 21;

// Control words at the start of the fused workspace, one 256-byte slot each:
// the 64-bit launch counter that tags all hand-off data (words left by earlier
// launches never look valid, so nothing needs clearing between launches), the
// arrival count of launches that report their error word, the error word.
constexpr int kSlotInts = 64;
constexpr int kSlotEpoch = 0;
constexpr int kSlotDone = 1;
constexpr int kSlotErr = 2;  // sticky: 1 after a timed-out wait
constexpr int kNumSlots = 3;
constexpr size_t kSyncBytes = size_t(kNumSlots) * kSlotInts * 4;
static_assert(kSyncBytes == MOE_DECODE_SYNC_BYTES, "header constant");
static_assert(kSlotErr * kSlotInts * 4 == MOE_DECODE_ERR_OFFSET, "header constant");


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
  int32_t* err_out;         // device int32 or null: the last workgroup moves the sticky
                            // error word here and clears it
  // workspace; words that many workgroups read are written in kCopies copies
  // and each reader takes the copy of its XCD (blockIdx % 8)
  int* sync;
  tword_t* logits;  // [T][E + 1]                router logits; column E: shared-gate logit
  tword_t* route;   // [kCopies][T][K]           expert ids
  tword_t* wts;     // [kCopies][T][K + 1]       routing weights; column K: shared gate
  tword_t* u;       // [kCopies][P][2r]          A_gate x, A_up x
  tword_t* h;       // [kCopies][P][I / 2]       fp16 pairs of h * 2^-e
  tword_t* hexp;    // [kCopies][P][I / JW]      e of each JW-column block of h
  tword_t* vpart;   // [P][I / JW][r]            per-block partials of A_down h
  tword_t* v;       // [kCopies][P][r]           A_down h
  // grid layout (filled by the launcher)
  int nR, nWA, nBG, nV, nD, base_la, base_gu, base_v, base_dn, total;
  int defer_down;  // the down workgroups wait before fetching their routed rows
};

struct FusedWs {
  size_t sync, logits, route, wts, u, h, hexp, vpart, v, total;
};

inline FusedWs fused_ws_layout(int T, int E, int K, int S, int I, int r) {
  FusedWs W;
  const size_t P = size_t(T) * (K + S);
  const size_t C = kCopies;
  size_t o = 0;
  W.sync = o;   o = align256(o + kSyncBytes);
  W.logits = o; o = align256(o + size_t(T) * (E + 1) * 8);
  W.route = o;  o = align256(o + C * T * K * 8);
  W.wts = o;    o = align256(o + C * T * (K + 1) * 8);
  W.u = o;      o = align256(o + C * P * 2 * r * 8);
  W.h = o;      o = align256(o + C * P * (I / 2) * 8);
  W.hexp = o;   o = align256(o + C * P * (I / kFusedJW) * 8);
  W.vpart = o;  o = align256(o + P * (I / kFusedJW) * r * 8);
  W.v = o;      o = align256(o + C * P * r * 8);
  W.total = o;
  return W;
}

bool fused_shape_supported(int H, int I, int r);
hipError_t launch_fused(const FusedArgs& a, hipStream_t st);
hipError_t launch_zero_ints(int* p, int n, hipStream_t st);

// Argument checks of moe_block_decode(_exec) (no device work), and the launch
// on a caller-chosen workspace base (ws_bytes is checked against the layout).
moe_status_t block_decode_check(const char* fn, const moe_dims_t* d, const int8_t* gate_q,
                                const float* gate_s, const int8_t* sgate_q, const float* sgate_s,
                                const moe_experts_t* routed, const void* shared_blob,
                                const uint16_t* h_in, int32_t T, int32_t flags, float eps,
                                uint16_t* out);
moe_status_t block_decode_launch(const char* fn, const moe_dims_t* d, const int8_t* gate_q,
                                 const float* gate_s, const int8_t* sgate_q, const float* sgate_s,
                                 const moe_experts_t* routed, const void* shared_blob,
                                 const uint16_t* h_in, int32_t T, int32_t flags, float eps,
                                 const int32_t* exec_idx, int32_t* topk_idx, float* topk_w,
                                 uint16_t* out, void* ws, size_t ws_bytes, int32_t* err_out,
                                 void* stream);

}  // namespace moe

// Workspace layout shared by moe_route and moe_expert_forward.
#pragma once

#include "../../include/moe.h"
#include "launch.h"
#include "moe_internal.h"

namespace moe {

struct WsLayout {
  // routing
  size_t logits;   // fp32 [T, E] (used when the caller passes no logits buffer)
  size_t sg;       // fp32 [T]    shared-gate logits
  // decode expert path
  size_t blobptr;  // u64 [NP]    resolved blob address per (token, slot)
  size_t u;        // fp32 [NP, 2r]
  size_t h;        // bf16 [NP, I]
  size_t vpart;    // fp32 [NP, I/JW, r]
  size_t total;
};

inline WsLayout ws_layout(const moe_dims_t& d, int T, bool prefill) {
  (void)prefill;
  WsLayout W;
  const size_t NP = size_t(T) * (d.K + d.n_shared);
  const int jw = decode_gateup_block_j(d.H);
  const size_t nb = jw ? size_t(d.I / jw) : 0;
  size_t o = 0;
  W.logits = o;  o = align256(o + size_t(T) * d.E * 4);
  W.sg = o;      o = align256(o + size_t(T) * 4);
  W.blobptr = o; o = align256(o + NP * 8);
  W.u = o;       o = align256(o + NP * 2 * d.r * 4);
  W.h = o;       o = align256(o + NP * d.I * 2);
  W.vpart = o;   o = align256(o + NP * nb * d.r * 4);
  W.total = o;
  return W;
}

}  // namespace moe

// Workspace layout shared by moe_route and moe_expert_forward.
#pragma once

#include "../../include/moe.h"
#include "launch.h"
#include "moe_internal.h"
#include "prefill.h"

namespace moe {

struct WsLayout {
  // routing
  size_t logits;   // fp32 [T, E] (used when the caller passes no logits buffer)
  size_t sg;       // fp32 [T]    shared-gate logits
  size_t plog;     // fp32 [kRouterSplit, T, E + S] router GEMM partials (T >= kRouterGemmMinT)
  // decode expert path
  size_t blobptr;  // u64 [NP]    resolved blob address per (token, slot)
  size_t u;        // fp32 [NP, 2r]
  size_t h;        // fp32 [NP, I]
  size_t vpart;    // fp32 [NP, I/JW, r]
  // prefill grouping and grouped GEMMs (NR = T*K + n_shared*T sorted rows)
  size_t chunk_hist;  // int32 [nch, E]
  size_t gstart;      // int32 [E+2]
  size_t tstart;      // int32 [E+2]
  size_t gblob;       // u64 [E+1]
  size_t pud;         // bf16 [NR, 64]  lambda * LoRA-A of down (hi/lo pairs)
  size_t upart;       // fp32 [kLoraSplit, NR, 32] K-split partials of the gate/up LoRA-A
  size_t x16;         // fp16 [T, H]    x * 2^-ex (prefill)
  size_t ex;          // int32 [T]
  size_t hl;          // fp16 [NR, I]   h in sorted rows, scaled per 16-column block
  size_t hbe;         // int8 [NR, I/16] the blocks' exponents
  size_t hmax;        // u32 [NR]       max |h| per row
  size_t hs16;        // fp16 [NR, I]   h * 2^-eh
  size_t eh;          // int32 [NR]
  size_t total;
};

inline WsLayout ws_layout(const moe_dims_t& d, int T, bool prefill) {
  WsLayout W;
  const size_t NP = size_t(T) * (d.K + d.n_shared);
  const int jw = decode_gateup_block_j(d.H);
  const size_t nb = jw ? size_t(d.I / jw) : 0;
  size_t o = 0;
  W.logits = o;  o = align256(o + size_t(T) * d.E * 4);
  W.sg = o;      o = align256(o + size_t(T) * 4);
  W.plog = o;    o = align256(o + (T >= kRouterGemmMinT ? size_t(kRouterSplit) * T * (d.E + d.n_shared) * 4 : 0));
  W.blobptr = o; o = align256(o + NP * 8);
  W.u = o;       o = align256(o + NP * 2 * d.r * 4);
  W.h = o;       o = align256(o + NP * d.I * 4);
  W.vpart = o;   o = align256(o + NP * nb * d.r * 4);
  const size_t TK = size_t(T) * d.K;
  const size_t nch = prefill ? (TK + kGroupChunk - 1) / kGroupChunk : 0;
  const size_t NR = prefill ? TK + size_t(d.n_shared) * T : 0;
  const size_t E = prefill ? d.E : 0;
  W.chunk_hist = o; o = align256(o + nch * E * 4);
  W.gstart = o;     o = align256(o + (prefill ? (E + 2) * 4 : 0));
  W.tstart = o;     o = align256(o + (prefill ? (E + 2) * 4 : 0));
  W.gblob = o;      o = align256(o + (prefill ? (E + 1) * 8 : 0));
  W.pud = o;        o = align256(o + NR * kLoraK * 2);
  W.upart = o;      o = align256(o + size_t(kLoraSplit) * NR * 32 * 4);
  const size_t TP = prefill ? size_t(T) : 0;
  W.x16 = o;        o = align256(o + TP * d.H * 2);
  W.ex = o;         o = align256(o + TP * 4);
  W.hl = o;         o = align256(o + NR * d.I * 2);
  W.hbe = o;        o = align256(o + NR * (d.I / 16));
  W.hmax = o;       o = align256(o + NR * 4);
  W.hs16 = o;       o = align256(o + NR * d.I * 2);
  W.eh = o;         o = align256(o + NR * 4);
  W.total = o;
  return W;
}

// Workspace of moe_block_prefill: the route + expert workspace, the routing
// outputs the caller does not receive, and the compact expert outputs.
struct BlockPrefillLayout {
  WsLayout W;       // at offset 0
  size_t counts;    // int32 [E]
  size_t offsets;   // int32 [E+1]
  size_t perm;      // int32 [T*K]
  size_t shared_w;  // fp32 [T]
  size_t y16;       // fp16 [T, K+S, H]
  size_t ey;        // int32 [T, K+S]
  size_t total;
};

inline BlockPrefillLayout block_prefill_layout(const moe_dims_t& d, int T) {
  BlockPrefillLayout P;
  P.W = ws_layout(d, T, true);
  const size_t NP = size_t(T) * (d.K + d.n_shared);
  size_t o = P.W.total;
  P.counts = o;   o = align256(o + size_t(d.E) * 4);
  P.offsets = o;  o = align256(o + size_t(d.E + 1) * 4);
  P.perm = o;     o = align256(o + size_t(T) * d.K * 4);
  P.shared_w = o; o = align256(o + size_t(T) * 4);
  P.y16 = o;      o = align256(o + NP * d.H * 2);
  P.ey = o;       o = align256(o + NP * 4);
  P.total = o;
  return P;
}

}  // namespace moe

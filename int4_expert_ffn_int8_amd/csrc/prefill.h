// Prefill path: arguments of the grouped GEMM kernels and their launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_internal.h"

namespace moe {

constexpr int kGroupChunk = 1024;  // pairs per grouping workgroup
constexpr int kPrefillBM = 128;    // rows (pairs/tokens) per expert-GEMM tile
constexpr int kRouterGemmMinT = 64;  // tokens from which the router uses MFMA
constexpr int kRouterSplit = 4;      // K splits of the router GEMM
constexpr int kLoraSplit = 4;        // K splits of the gate/up LoRA-A GEMM

// expert GEMM modes (values shared with the grouped GEMM kernel's modes)
constexpr int kGemmGateUp = 2;
constexpr int kGemmDown = 4;

struct GemmArgs {
  int T, K, S, E, H, I, r;
  float lam;
  // sorted row space
  const int32_t* perm;        // [T*K]
  const int32_t* offsets;     // [E+1]
  const int32_t* gstart;      // [E+2] group row starts (last = T*K + S*T)
  const int32_t* tstart;      // [E+2] group m-tile starts (last = total tiles)
  const unsigned long long* gblob;  // [E+1] blob address per group
  BlobLayout L;
  // activations
  const uint16_t* x;          // [T][H] bf16
  const uint16_t* x16;        // [T][H] fp16 x * 2^-ex[t]
  const int32_t* ex;          // [T]
  uint16_t* hl;               // [NR][I] SwiGLU output h as fp16(h * 2^-hbe) in sorted rows,
  int8_t* hbe;                //   one exponent per 16-column block: hbe [NR][I/16]
  uint32_t* hmax;             // [NR] float bits of max |h| per row (zeroed by the setup)
  const uint16_t* hs;         // [NR][I] fp16 h * 2^-eh[s]
  const int32_t* eh;          // [NR]
  uint16_t* hs_out;           // where the LoRA-A GEMM of down writes hs (and eh_out eh)
  int32_t* eh_out;
  const uint16_t* ud;         // [NR][64] lambda * (A_d h) * 2^-eh as bf16 hi/lo pairs
  uint16_t* ud_out;
  // router GEMM
  const int8_t* rq;
  const float* rs;
  const int8_t* sq;
  const float* ss;
  const float* bias;
  float* logits;
  float* sg_logit;
  float* plog;  // [kRouterSplit][T][E + S] partial logits of the K splits, or null (no split)
  float* upart;  // [kLoraSplit][NR][32] partial LoRA-A of gate/up over the K splits
  int32_t* zero;  // router GEMM: nzero ints its first workgroup sets to 0 (grouping histogram)
  int nzero;
  // down output, [T][K+S][H]: fp32 y, or (y16 set) fp16 y * 2^-ey with one
  // exponent per (token, slot) row, ey [T][K+S]
  float* y;
  uint16_t* y16;
  int32_t* ey;
};

hipError_t launch_group(const int32_t* idx, int T, int K, int E, int32_t* counts,
                        int32_t* offsets, int32_t* perm, const int32_t* chunk_hist,
                        hipStream_t st);
hipError_t launch_router_gemm(const GemmArgs& a, hipStream_t st);
int prefill_max_mtiles(int T, int K, int E, int S);
hipError_t launch_prefill_experts(const GemmArgs& a, const int32_t* counts, ExpertSource src,
                                  const uint8_t* shared_blob, uint16_t* x16, int32_t* ex,
                                  uint16_t* hs16, int32_t* eh, hipStream_t st);
// expert_gemm.hip
// x to fp16 with a row exponent, zeros of the gate/up row maxima, and the
// expert-GEMM setup (group row starts, tile starts, blob addresses), in one launch
struct X16SetupArgs {
  const uint16_t* x;  // [T][H] bf16
  int T, H, E, K, S;
  uint16_t* x16;      // [T][H]
  int32_t* ex;        // [T]
  uint32_t* hmax;     // [T * (K + S)]
  const int32_t* counts;   // [E]
  const int32_t* offsets;  // [E + 1]
  ExpertSource src;
  const uint8_t* shared_blob;
  int32_t* gstart;           // [E + 2]
  int32_t* tstart;           // [E + 2]
  unsigned long long* gblob; // [E + 1]
};
hipError_t launch_x16_setup(const X16SetupArgs& a, hipStream_t st);
hipError_t launch_h16(const uint16_t* hl, const int8_t* hbe, const uint32_t* hmax, const int32_t* nrows,
                      int NR, int I, uint16_t* hs16, int32_t* eh, hipStream_t st);
hipError_t launch_expert_gemm(int mode, const GemmArgs& a, int mtiles, hipStream_t st);

}  // namespace moe

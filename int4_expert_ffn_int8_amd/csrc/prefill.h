// Prefill path: arguments of the grouped GEMM kernels and their launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_internal.h"

namespace moe {

constexpr int kGroupChunk = 1024;  // pairs per grouping workgroup
constexpr int kPrefillBM = 128;    // rows (pairs/tokens) per expert-GEMM tile
constexpr int kRouterGemmMinT = 64;  // tokens from which the router uses MFMA

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
  const uint16_t* x;          // [T][H]
  const uint16_t* hs;         // [NR][I] h (fp16) in sorted rows
  uint16_t* hs_out;
  const uint16_t* u;          // [NR][64] lambda * A_g x, A_u x as bf16 hi/lo pairs
  uint16_t* u_out;
  const uint16_t* ud;         // [NR][64] lambda * A_d h as fp16 hi/lo pairs
  uint16_t* ud_out;
  // router GEMM
  const int8_t* rq;
  const float* rs;
  const int8_t* sq;
  const float* ss;
  const float* bias;
  float* logits;
  float* sg_logit;
  // down output, [T][K+S][H]
  float* y;
};

hipError_t launch_group(const int32_t* idx, int T, int K, int E, int32_t* counts,
                        int32_t* offsets, int32_t* perm, int32_t* chunk_hist, int32_t* base,
                        hipStream_t st);
hipError_t launch_router_gemm(const GemmArgs& a, hipStream_t st);
int prefill_max_mtiles(int T, int K, int E, int S);
hipError_t launch_prefill_experts(const GemmArgs& a, const int32_t* counts, ExpertSource src,
                                  const uint8_t* shared_blob, hipStream_t st);

}  // namespace moe

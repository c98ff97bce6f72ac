// Host-side launchers of the gfx950 kernels (declarations).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_internal.h"

// Input widths (H or I) the streaming kernels are instantiated for.
#define MOE_FOR_EACH_WIDTH(X) X(64) X(128) X(256) X(512) X(1024) X(2048) X(4096)

namespace moe {

inline bool width_supported(int v) {
  return v == 64 || v == 128 || v == 256 || v == 512 || v == 1024 || v == 2048 || v == 4096;
}

// router
hipError_t launch_router_logits(int H, const int8_t* q, const float* s, const int8_t* sq,
                                const float* ss, const uint16_t* x, const float* bias, int E,
                                int n_shared, int T, float* logits, float* sg_logit,
                                hipStream_t st, int32_t* zero = nullptr, int nzero = 0);
// Top-K, routing weights and shared gate, one wave per token.  With `plog`
// ([nks][T][E + n_shared] partial logits of a K-split router GEMM) the wave
// first sums the partials in split order, adds `bias` and stores the logits
// (`logits`, `sg_logit`); otherwise it reads them.  With `hist` (zeroed
// [ceil(T K / 1024)][E]) it also counts each (token, slot) pair in its
// chunk's expert histogram for the grouping.
hipError_t launch_topk(float* logits, float* sg_logit, int T, int E, int K, int n_shared,
                       int norm, int32_t* idx, float* w, float* sw, hipStream_t st,
                       const float* plog = nullptr, int nks = 0, const float* bias = nullptr,
                       int32_t* hist = nullptr);

// decode expert path
struct DecodeArgs {
  const uint16_t* x;       // [T, H]
  const int32_t* topk_idx; // [T, K]; entries are clamped into [0, E)
  int T, H, I, K, S, r, E;
  float lam;
  ExpertSource src;
  const uint8_t* shared_blob;
  BlobLayout L;
  // workspace
  unsigned long long* blobptr;  // [NP]
  float* u;                     // [NP, 2r]
  float* h;                     // [NP, I]
  float* vpart;                 // [NP, I/JW, r]
  float* y;                     // [NP, H]
};
int decode_gateup_block_j(int H);  // output units (j) per gate/up workgroup
hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);

// combine / norm
hipError_t launch_combine(const float* y, const float* w, const float* sw, int T, int K, int S,
                          int H, const uint16_t* residual, uint16_t* out, uint16_t* norm_out,
                          float eps, hipStream_t st);
hipError_t launch_combine16(const uint16_t* y16, const int32_t* ey, const float* w, const float* sw,
                            int T, int K, int S, int H, const uint16_t* residual, uint16_t* out,
                            uint16_t* norm_out, float eps, hipStream_t st);
hipError_t launch_rmsnorm(const uint16_t* h, int T, int H, float eps, uint16_t* out,
                          hipStream_t st);

}  // namespace moe

// Internal definitions shared by the host ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kGroup = 64;   // quantisation group along the input dimension
constexpr int kMaxK = 16;    // experts per token supported by the top-K kernel
constexpr int kMaxE = 1024;  // routed experts supported
constexpr int kMaxR = 16;    // LoRA rank supported
constexpr int kLoraK = 64;   // width of the LoRA chunk appended to a GEMM's K

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// ---------------------------------------------------------------------------
// Expert blob layout (one expert = one pool slot).
//
// gate/up rows are interleaved in blocks of 16: blob row 32*b + i is gate row
// 16*b + i and blob row 32*b + 16 + i is up row 16*b + i (i < 16).  A GEMM
// tile of 32 blob rows therefore holds gate and up for the same 16 outputs,
// and the SwiGLU epilogue needs no data exchange.
//
// Codes: each 32-bit word covers 8 consecutive columns c0..c7 of one row;
// code c_{2s} sits in bits [4s, 4s+4) and c_{2s+1} in bits [16+4s, 16+4s+4)
// (s = 0..3).  (w >> 4s) & 0x000F000F then holds columns (2s, 2s+1) in the
// low and high halves, ready to become a bf16 pair.
//
// Scale/bias: one 32-bit word per (row, group): bf16 scale in the low half,
// bf16 bias in the high half.
// ---------------------------------------------------------------------------
struct BlobLayout {
  size_t gu_codes;  // uint8 [2I][H/2]   gate/up codes, interleaved rows
  size_t gu_sb;     // uint32 [2I][H/64] gate/up scale|bias
  size_t dn_codes;  // uint8 [H][I/2]    down codes
  size_t dn_sb;     // uint32 [H][I/64]  down scale|bias
  size_t a_gu;      // bf16 [2][r][H]    LoRA A of gate, then of up
  size_t b_gu;      // bf16 [2I][r]      LoRA B of gate/up, interleaved rows
  size_t a_dn;      // bf16 [r][I]       LoRA A of down
  size_t b_dn;      // bf16 [H][r]       LoRA B of down
  size_t meta;      // fp32 [2]          bounds of the down projection (see kMetaDown*)
  size_t total;
};
// Meta words written by the packer: the largest absolute row sum of the
// dequantised down weights, max_i sum_j |s q + b|, and a bound on that of the
// down LoRA product B A, max_i sum_r |B[i, r]| sum_j |A[r, j]|.  With
// |h| <= M, every down output obeys |y_i| <= (W + |lambda| L) M.
constexpr int kMetaDownW = 0, kMetaDownL = 1;

inline BlobLayout blob_layout(int H, int I, int r) {
  BlobLayout L;
  size_t o = 0;
  L.gu_codes = o; o = align256(o + size_t(2) * I * (H / 2));
  L.gu_sb = o;    o = align256(o + size_t(2) * I * (H / kGroup) * 4);
  L.dn_codes = o; o = align256(o + size_t(H) * (I / 2));
  L.dn_sb = o;    o = align256(o + size_t(H) * (I / kGroup) * 4);
  L.a_gu = o;     o = align256(o + size_t(2) * r * H * 2);
  L.b_gu = o;     o = align256(o + size_t(2) * I * r * 2);
  L.a_dn = o;     o = align256(o + size_t(r) * I * 2);
  L.b_dn = o;     o = align256(o + size_t(H) * r * 2);
  L.meta = o;     o = align256(o + 2 * 4);
  L.total = o;
  return L;
}

// blob row of gate output j / up output j
__host__ __device__ inline int gu_row_gate(int j) { return ((j >> 4) << 5) | (j & 15); }
__host__ __device__ inline int gu_row_up(int j) { return gu_row_gate(j) | 16; }

// Where a layer's routed experts live (device-side copy of moe_experts_t).
struct ExpertSource {
  const uint8_t* slots;
  const int32_t* expert_to_slot;  // nullptr: identity
  const uint8_t* host_blobs;
  unsigned long long* counters;
  size_t stride;
  uint32_t delay_ticks = 0;  // modeled storage latency of a host read, wall-clock ticks
};

// Host: ns -> ticks of the device's constant-rate wall clock (current device).
uint32_t wall_ticks(uint32_t ns);
// One wait of `ticks` wall-clock ticks on stream st (a single-lane kernel).
hipError_t launch_storage_delay(uint32_t ticks, hipStream_t st);

}  // namespace moe

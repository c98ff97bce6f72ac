// Device helpers for the gfx950 kernels (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// fp16 <-> fp32
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return float(__builtin_bit_cast(f16x2_t, w)[0]);
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return float(__builtin_bit_cast(f16x2_t, w)[1]);
}
__device__ __forceinline__ float f16_to_f32(uint16_t b) {
  return float(__builtin_bit_cast(_Float16, b));
}
// float -> fp16 bits, round to nearest even, saturated to the finite range
__device__ __forceinline__ uint16_t f32_to_f16_sat(float f) {
  f = fminf(fmaxf(f, -65504.0f), 65504.0f);
  return __builtin_bit_cast(uint16_t, _Float16(f));
}
// bf16 pair -> fp16 pair (exact for normal-range fp16 values)
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  f16x2_t v = {_Float16(bf16_lo(w)), _Float16(bf16_hi(w))};
  return __builtin_bit_cast(uint32_t, v);
}

// acc + a.lo*b.lo + a.hi*b.hi on fp16 pairs (v_dot2c_f32_f16)
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b),
                                acc, false);
}

// acc + a.lo*b.lo + a.hi*b.hi on bf16 pairs (v_dot2c_f32_bf16)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                          __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// Two int4 codes (bits [0,4) and [16,20) of w after the shift) as the bf16
// pair (128 + c_lo, 128 + c_hi): 0x4300 is bf16 128.0 and codes 0..15 fill
// its low mantissa bits exactly.
__device__ __forceinline__ uint32_t codes_to_bf16x2_biased(uint32_t w, int s) {
  return ((w >> (4 * s)) & 0x000F000Fu) | 0x43004300u;
}

// The same two codes as the fp16 pair (128 + c_lo, 128 + c_hi): 0x5800 is
// fp16 128.0, whose mantissa step is 1/8, so each code moves to bits [3, 7).
__device__ __forceinline__ uint32_t codes_to_f16x2_biased(uint32_t w, int s) {
  const uint32_t t = (s == 0) ? (w << 3) : (w >> (4 * s - 3));
  return (t & 0x00780078u) | 0x58005800u;
}

// Cross-lane moves without LDS round trips (gfx9 DPP).  Row permutations
// (quad_perm [1,0,3,2] / [2,3,0,1], row_half_mirror, row_mirror) exchange
// within 16-lane rows; row_bcast:15 adds lane 15 of rows 0 and 2 into rows 1
// and 3, row_bcast:31 adds lane 31 into rows 2 and 3 (other rows get the
// `old` operand, 0 here).
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- 7 - i within 8
constexpr int kDppMirror = 0x140;      // lane i <- 15 - i within 16
constexpr int kDppBcast15 = 0x142;
constexpr int kDppBcast31 = 0x143;

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v, uint32_t old = 0) {
  return uint32_t(__builtin_amdgcn_update_dpp(int(old), int(v), CTRL, ROWS, 0xF, false));
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_f(float v, float old = 0.f) {
  return __uint_as_float(dpp_u<CTRL, ROWS>(__float_as_uint(v), __float_as_uint(old)));
}
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Sum over groups of `width` consecutive lanes (width a power of two <= 64);
// every lane of a group ends with the group's sum.  The pairing is the fixed
// butterfly (partners 1, 2, 4, 8, 16, 32 lanes apart): every lane of a group
// holds the bit-identical sum and results are run-to-run identical.
template <int width>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (width >= 2) v += dpp_f<kDppXor1>(v);
  if constexpr (width >= 4) v += dpp_f<kDppXor2>(v);
  if constexpr (width >= 8) v += dpp_f<kDppHalfMirror>(v);
  if constexpr (width >= 16) v += dpp_f<kDppMirror>(v);
  if constexpr (width >= 32) v += dpp_f<kDppBcast15, 0xA>(v);  // lanes 31, 63: 32-lane sums
  if constexpr (width == 32) {
    const float lo = readlane_f(v, 31), hi = readlane_f(v, 63);
    v = (__lane_id() < 32) ? lo : hi;
  }
  if constexpr (width == 64) {
    v += dpp_f<kDppBcast31, 0xC>(v);  // lane 63: the wave sum
    v = readlane_f(v, 63);
  }
  return v;
}

// Wave-wide max / min; the result is wave-uniform.  The float max runs on
// order-preserving unsigned keys (sign bit set for x >= +0, all bits flipped
// for negatives), an exact integer max that folds into the DPP instructions;
// it returns the largest element's bits (+0 over -0; a NaN ranks above
// +infinity, so callers map NaN first where that matters).
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return u ^ (uint32_t(int32_t(u) >> 31) | 0x80000000u);
}
__device__ __forceinline__ float f32_from_order_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
__device__ __forceinline__ float wave_max(float f) {
  uint32_t v = f32_order_key(f);
  v = max(v, dpp_u<kDppXor1>(v));
  v = max(v, dpp_u<kDppXor2>(v));
  v = max(v, dpp_u<kDppHalfMirror>(v));
  v = max(v, dpp_u<kDppMirror>(v));
  v = max(v, dpp_u<kDppBcast15, 0xA>(v, v));
  v = max(v, dpp_u<kDppBcast31, 0xC>(v, v));
  return f32_from_order_key(uint32_t(__builtin_amdgcn_readlane(int(v), 63)));
}
// Wave max of unsigned keys.  Lanes outside a row broadcast's row mask read
// 0, the identity of max, so each step is one fused DPP instruction.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u<kDppXor1>(v));
  v = max(v, dpp_u<kDppXor2>(v));
  v = max(v, dpp_u<kDppHalfMirror>(v));
  v = max(v, dpp_u<kDppMirror>(v));
  v = max(v, dpp_u<kDppBcast15, 0xA>(v));
  v = max(v, dpp_u<kDppBcast31, 0xC>(v));
  return uint32_t(__builtin_amdgcn_readlane(int(v), 63));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u<kDppXor1>(v));
  v = min(v, dpp_u<kDppXor2>(v));
  v = min(v, dpp_u<kDppHalfMirror>(v));
  v = min(v, dpp_u<kDppMirror>(v));
  v = min(v, dpp_u<kDppBcast15, 0xA>(v, v));
  v = min(v, dpp_u<kDppBcast31, 0xC>(v, v));
  return uint32_t(__builtin_amdgcn_readlane(int(v), 63));
}

// Geometry of a row-streaming GEMV over an input of IN columns: each lane
// owns 32 consecutive columns (per slice); LPR lanes cover one row and a wave
// covers RPL rows per load; inputs wider than 2048 give each lane SL slices
// 2048 columns apart.
template <int IN>
struct Geo {
  static_assert(IN % 64 == 0 && IN >= 64 && IN <= 4096, "unsupported input width");
  static constexpr int LPR = (IN / 32) < 64 ? (IN / 32) : 64;
  static constexpr int RPL = 64 / LPR;
  static constexpr int SL = (IN / 32) > 64 ? (IN / 2048) : 1;
};

// Exponent e >= 0 of a block of activations stored as fp16(v * 2^-e): the
// smallest shift that keeps the block's largest magnitude m below 2^15, so
// fp16 (largest finite 65504) never saturates; e = 0 when m < 2^15.
__device__ __forceinline__ int h_block_exp(float m) {
  if (!(m >= 32768.0f)) return 0;
  return min(ilogbf(m) - 14, 126);
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }
__device__ __forceinline__ float sigmoid_f(float z) { return 1.0f / (1.0f + expf(-z)); }

// Load through a global-address-space pointer (addresses read from memory
// would otherwise be flat).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
template <typename T>
__device__ __forceinline__ T gload(const void* p) {
  return *reinterpret_cast<const __attribute__((address_space(1))) T*>(reinterpret_cast<uintptr_t>(p));
}
__device__ __forceinline__ uint4 gload16(const void* p) {
  const u32x4_t v = gload<u32x4_t>(p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Wait `ticks` periods of the constant-rate wall clock.  The bound is the
// argument itself, so the loop always ends.
__device__ __forceinline__ void wall_wait(uint32_t ticks) {
  const uint64_t t0 = uint64_t(wall_clock64());
  while (uint64_t(wall_clock64()) - t0 < ticks) __builtin_amdgcn_s_sleep(8);
}

// Row exponent: the largest magnitude m of a row is scaled into [2^14, 2^15)
// (e may be negative); rows of zeros keep e = 0.
__device__ __forceinline__ int row_exp(float m) {
  if (!(m > 0.f)) return 0;
  return max(min(ilogbf(m) - 14, 126), -100);
}

}  // namespace moe

// Weighted combine of the expert outputs (+ residual), and RMSNorm.
//
// The block output is the routing-weighted sum of the selected experts'
// outputs plus the gated shared expert ([P3] "iPhone、Mac、Android、Windows
// 实测横评…", quality section: a shared expert with its own 8-bit gate).  In
// the stacked workloads layers are joined by a residual add and a unit-gain
// RMSNorm only; the norm of the next layer's input is fused here.
#include "device_utils.h"
#include "launch.h"

namespace moe {

__device__ __forceinline__ float block_sum_256(float v, float* red) {
  v = group_sum<64>(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// grid T, block 256.  Each thread takes 8 consecutive columns (two 16-byte
// loads per expert row, issued four rows at a time); the expert order of the
// sum is fixed (k = 0..K-1, then shared).
__global__ void __launch_bounds__(256) k_combine(const float* __restrict__ y,
                                                  const float* __restrict__ w,
                                                  const float* __restrict__ sw, int K, int S, int H,
                                                  const uint16_t* __restrict__ residual,
                                                  uint16_t* __restrict__ out,
                                                  uint16_t* __restrict__ norm_out, float eps) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const int KS = K + S;
  const float g = S ? sw[t] : 0.f;
  const float* yt = y + size_t(t) * KS * H;
  float ss = 0.f;
  for (int c = threadIdx.x; c < H / 8; c += 256) {
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < KS; k0 += 4) {
      float4 v[4][2];
#pragma unroll
      for (int u = 0; u < 4; ++u) {  // rows past KS re-read the last row (not summed)
        const float4* src = reinterpret_cast<const float4*>(yt + size_t(min(k0 + u, KS - 1)) * H) + 2 * c;
        v[u][0] = src[0];
        v[u][1] = src[1];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int k = k0 + u;
        if (k >= KS) break;
        const float coef = (k < K) ? w[size_t(t) * K + k] : g;
        const float e[8] = {v[u][0].x, v[u][0].y, v[u][0].z, v[u][0].w, v[u][1].x, v[u][1].y, v[u][1].z, v[u][1].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = fmaf(coef, e[i], o[i]);
      }
    }
    if (residual) {
      const uint4 rv = *reinterpret_cast<const uint4*>(residual + size_t(t) * H + 8 * c);
      const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[2 * i] += bf16_lo(rw[i]);
        o[2 * i + 1] += bf16_hi(rw[i]);
      }
    }
    uint32_t ow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint16_t lo = f32_to_bf16(o[2 * i]), hi = f32_to_bf16(o[2 * i + 1]);
      ow[i] = uint32_t(lo) | (uint32_t(hi) << 16);
      const float a0 = bf16_to_f32(lo), a1 = bf16_to_f32(hi);
      ss = fmaf(a0, a0, ss);
      ss = fmaf(a1, a1, ss);
    }
    *reinterpret_cast<uint4*>(out + size_t(t) * H + 8 * c) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
  }
  if (!norm_out) return;
  const float tot = block_sum_256(ss, red);
  const float inv = 1.0f / sqrtf(tot / float(H) + eps);
  for (int c = threadIdx.x; c < H / 8; c += 256) {  // the columns this thread wrote
    const uint4 ov = *reinterpret_cast<const uint4*>(out + size_t(t) * H + 8 * c);
    const uint32_t iw[4] = {ov.x, ov.y, ov.z, ov.w};
    uint32_t nw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      nw[i] = uint32_t(f32_to_bf16(bf16_lo(iw[i]) * inv)) | (uint32_t(f32_to_bf16(bf16_hi(iw[i]) * inv)) << 16);
    *reinterpret_cast<uint4*>(norm_out + size_t(t) * H + 8 * c) = make_uint4(nw[0], nw[1], nw[2], nw[3]);
  }
}

// k_combine over compact expert outputs: y16 [T][K+S][H] fp16 holding
// y * 2^-ey with one exponent per (token, slot) row (ey [T][K+S]).  The same
// sum as k_combine; each power of two is folded into the row's coefficient
// exactly.
__global__ void __launch_bounds__(256) k_combine16(const uint16_t* __restrict__ y16,
                                                    const int32_t* __restrict__ ey,
                                                    const float* __restrict__ w,
                                                    const float* __restrict__ sw, int K, int S, int H,
                                                    const uint16_t* __restrict__ residual,
                                                    uint16_t* __restrict__ out,
                                                    uint16_t* __restrict__ norm_out, float eps) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const int KS = K + S;
  const float g = S ? sw[t] : 0.f;
  const uint16_t* yt = y16 + size_t(t) * KS * H;
  float ss = 0.f;
  for (int c = threadIdx.x; c < H / 8; c += 256) {
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < KS; k0 += 4) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)  // rows past KS re-read the last row (not summed)
        v[u] = *reinterpret_cast<const uint4*>(yt + size_t(min(k0 + u, KS - 1)) * H + 8 * c);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int k = k0 + u;
        if (k >= KS) break;
        const float cf = ldexpf((k < K) ? w[size_t(t) * K + k] : g, ey[size_t(t) * KS + k]);
        const f16x2_t p[4] = {__builtin_bit_cast(f16x2_t, v[u].x), __builtin_bit_cast(f16x2_t, v[u].y),
                              __builtin_bit_cast(f16x2_t, v[u].z), __builtin_bit_cast(f16x2_t, v[u].w)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[2 * i] = fmaf(cf, float(p[i][0]), o[2 * i]);
          o[2 * i + 1] = fmaf(cf, float(p[i][1]), o[2 * i + 1]);
        }
      }
    }
    if (residual) {
      const uint4 rv = *reinterpret_cast<const uint4*>(residual + size_t(t) * H + 8 * c);
      const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[2 * i] += bf16_lo(rw[i]);
        o[2 * i + 1] += bf16_hi(rw[i]);
      }
    }
    uint32_t ow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint16_t lo = f32_to_bf16(o[2 * i]), hi = f32_to_bf16(o[2 * i + 1]);
      ow[i] = uint32_t(lo) | (uint32_t(hi) << 16);
      const float a0 = bf16_to_f32(lo), a1 = bf16_to_f32(hi);
      ss = fmaf(a0, a0, ss);
      ss = fmaf(a1, a1, ss);
    }
    *reinterpret_cast<uint4*>(out + size_t(t) * H + 8 * c) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
  }
  if (!norm_out) return;
  const float tot = block_sum_256(ss, red);
  const float inv = 1.0f / sqrtf(tot / float(H) + eps);
  for (int c = threadIdx.x; c < H / 8; c += 256) {  // the columns this thread wrote
    const uint4 ov = *reinterpret_cast<const uint4*>(out + size_t(t) * H + 8 * c);
    const uint32_t iw[4] = {ov.x, ov.y, ov.z, ov.w};
    uint32_t nw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      nw[i] = uint32_t(f32_to_bf16(bf16_lo(iw[i]) * inv)) | (uint32_t(f32_to_bf16(bf16_hi(iw[i]) * inv)) << 16);
    *reinterpret_cast<uint4*>(norm_out + size_t(t) * H + 8 * c) = make_uint4(nw[0], nw[1], nw[2], nw[3]);
  }
}

// grid T, block 256
__global__ void __launch_bounds__(256) k_rmsnorm(const uint16_t* __restrict__ h, int H, float eps,
                                                  uint16_t* __restrict__ out) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  float ss = 0.f;
  for (int i = threadIdx.x; i < H; i += 256) {
    const float v = bf16_to_f32(h[size_t(t) * H + i]);
    ss = fmaf(v, v, ss);
  }
  const float tot = block_sum_256(ss, red);
  const float inv = 1.0f / sqrtf(tot / float(H) + eps);
  for (int i = threadIdx.x; i < H; i += 256)
    out[size_t(t) * H + i] = f32_to_bf16(bf16_to_f32(h[size_t(t) * H + i]) * inv);
}

hipError_t launch_combine(const float* y, const float* w, const float* sw, int T, int K, int S,
                          int H, const uint16_t* residual, uint16_t* out, uint16_t* norm_out,
                          float eps, hipStream_t st) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(k_combine, dim3(T), dim3(256), 0, st, y, w, sw, K, S, H, residual, out,
                     norm_out, eps);
  return hipGetLastError();
}

hipError_t launch_combine16(const uint16_t* y16, const int32_t* ey, const float* w, const float* sw,
                            int T, int K, int S, int H, const uint16_t* residual, uint16_t* out,
                            uint16_t* norm_out, float eps, hipStream_t st) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(k_combine16, dim3(T), dim3(256), 0, st, y16, ey, w, sw, K, S, H, residual,
                     out, norm_out, eps);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const uint16_t* h, int T, int H, float eps, uint16_t* out,
                          hipStream_t st) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(k_rmsnorm, dim3(T), dim3(256), 0, st, h, H, eps, out);
  return hipGetLastError();
}

}  // namespace moe

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

// grid T, block 256.  Each thread walks columns tid, tid+256, ... so loads are
// coalesced; the expert order of the sum is fixed (k = 0..K-1, then shared).
__global__ void __launch_bounds__(256) k_combine(const float* __restrict__ y,
                                                  const float* __restrict__ w,
                                                  const float* __restrict__ sw, int K, int S, int H,
                                                  const uint16_t* __restrict__ residual,
                                                  uint16_t* __restrict__ out,
                                                  uint16_t* __restrict__ norm_out, float eps) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const int KS = K + S;
  float wk[kMaxK + 1];
#pragma unroll
  for (int k = 0; k < kMaxK; ++k) wk[k] = (k < K) ? w[size_t(t) * K + k] : 0.f;
  const float g = S ? sw[t] : 0.f;
  const float* yt = y + size_t(t) * KS * H;
  float ss = 0.f;
  for (int i = threadIdx.x; i < H; i += 256) {
    float o = 0.f;
    for (int k = 0; k < K; ++k) o = fmaf(wk[k], yt[size_t(k) * H + i], o);
    if (S) o = fmaf(g, yt[size_t(K) * H + i], o);
    if (residual) o += bf16_to_f32(residual[size_t(t) * H + i]);
    const uint16_t ob = f32_to_bf16(o);
    out[size_t(t) * H + i] = ob;
    const float ov = bf16_to_f32(ob);
    ss = fmaf(ov, ov, ss);
  }
  if (!norm_out) return;
  const float tot = block_sum_256(ss, red);
  const float inv = 1.0f / sqrtf(tot / float(H) + eps);
  for (int i = threadIdx.x; i < H; i += 256)
    norm_out[size_t(t) * H + i] = f32_to_bf16(bf16_to_f32(out[size_t(t) * H + i]) * inv);
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

hipError_t launch_rmsnorm(const uint16_t* h, int T, int H, float eps, uint16_t* out,
                          hipStream_t st) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(k_rmsnorm, dim3(T), dim3(256), 0, st, h, H, eps, out);
  return hipGetLastError();
}

}  // namespace moe

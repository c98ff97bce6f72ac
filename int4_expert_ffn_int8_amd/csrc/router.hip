// Router: int8 group-64 gate GEMV, wavefront top-K with lowest-index ties,
// softmax weights and the sigmoid shared-expert gate.
//
// [P2] "SSD 专家卸载 · Prerouter 路由预测", tier table: K of E routed experts
// per token.  [P3] "iPhone、Mac、Android、Windows 实测横评…", quality
// section: the router gate and the shared-expert gate are 8-bit projections.
#include "device_utils.h"
#include "launch.h"
#include "moe_internal.h"
#include "prefill.h"
#include "topk.h"

namespace moe {


// logits[t, e] = sum_i s[e, i/64] q[e, i] x[t, i] (+ bias[e]); the row after
// the last expert is the shared-expert gate (its logit goes to sg_logit[t]).
// grid (ceil(rows / (4 RPL)), T), block 256.
template <int H>
__global__ void __launch_bounds__(256) k_router_logits(const int8_t* __restrict__ q,
                                                        const float* __restrict__ s,
                                                        const int8_t* __restrict__ sq,
                                                        const float* __restrict__ ss,
                                                        const uint16_t* __restrict__ x,
                                                        const float* __restrict__ bias, int E,
                                                        int n_shared, float* __restrict__ logits,
                                                        float* __restrict__ sg_logit,
                                                        int32_t* __restrict__ zero, int nzero) {
  using G = Geo<H>;
  if (zero && blockIdx.x == 0 && blockIdx.y == 0)  // the grouping histogram
    for (int i = threadIdx.x; i < nzero; i += 256) zero[i] = 0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % G::LPR;
  const int t = blockIdx.y;
  const int row = (blockIdx.x * 4 + wave) * G::RPL + lane / G::LPR;
  const int rows = E + n_shared;
  const bool valid = row < rows;
  const int8_t* qrow = (row < E) ? q + size_t(row) * H : sq;
  const float* srow = (row < E) ? s + size_t(row) * (H / 64) : ss;
  float acc = 0.f;
  if (valid) {
#pragma unroll
    for (int c = 0; c < G::SL; ++c) {
      const int col0 = 32 * sub + 2048 * c;
      const uint4 w0 = *reinterpret_cast<const uint4*>(qrow + col0);
      const uint4 w1 = *reinterpret_cast<const uint4*>(qrow + col0 + 16);
      const uint4* xp = reinterpret_cast<const uint4*>(x + size_t(t) * H + col0);
      uint32_t xw[16];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint4 v = xp[k];
        xw[4 * k] = v.x; xw[4 * k + 1] = v.y; xw[4 * k + 2] = v.z; xw[4 * k + 3] = v.w;
      }
      const uint32_t qw[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      float part = 0.f;
#pragma unroll
      for (int d = 0; d < 8; ++d) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int col = 4 * d + b;  // column within the lane's 32
          const float qv = float(int8_t((qw[d] >> (8 * b)) & 0xFF));
          const uint32_t xpair = xw[col >> 1];
          const float xv = (col & 1) ? bf16_hi(xpair) : bf16_lo(xpair);
          part = fmaf(qv, xv, part);
        }
      }
      acc = fmaf(srow[col0 / 64], part, acc);
    }
  }
  acc = group_sum<G::LPR>(acc);
  if (valid && sub == 0) {
    if (row < E)
      logits[size_t(t) * E + row] = acc + (bias ? bias[row] : 0.f);
    else
      sg_logit[t] = acc;
  }
}

constexpr int kMaxTopkSplits = kRouterSplit;  // K splits of the router GEMM summed by k_topk

constexpr int kTopkTokens = 16;  // tokens (waves) per top-K workgroup

// One wave per token: K rounds of wave argmax over (logit desc, index asc),
// then the routing weights and the shared gate.  With plog the logits are
// first summed from the K splits of the router GEMM (split order, then the
// bias) and stored.  MP logits per lane (E <= 64 MP).  With hist, the
// workgroup counts its (token, slot) pairs per chunk and expert in LDS first
// and adds each nonzero count to the chunk histogram once: under a skewed
// routing one expert takes a large share of the pairs, and one global add
// per pair made those adds queue on a few addresses.  grid
// ceil(T / kTopkTokens), block 64 kTopkTokens.
template <int MP>
__device__ __forceinline__ void topk_token(float* __restrict__ logits,
                                           float* __restrict__ sg_logit, int t, int T, int E,
                                           int K, int n_shared, int norm,
                                           int32_t* __restrict__ idx, float* __restrict__ w,
                                           float* __restrict__ sw,
                                           const float* __restrict__ plog, int nks,
                                           const float* __restrict__ bias, int* lhist, int c0) {
  const int lane = threadIdx.x & 63;
  float* l = logits + size_t(t) * E;
  float v[MP];
#pragma unroll
  for (int m = 0; m < MP; ++m) v[m] = 0.f;
  float sgl = 0.f;  // shared-gate logit
  if (plog) {
    const int N = E + n_shared;
    // the sum of column n over the splits: every split's load first (clamped,
    // unconditional), then the sum in split order
    auto split_sum = [&](int n) {
      float pv[kMaxTopkSplits];
#pragma unroll
      for (int k = 0; k < kMaxTopkSplits; ++k)
        pv[k] = plog[(size_t(min(k, nks - 1)) * T + t) * N + min(n, N - 1)];
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < kMaxTopkSplits; ++k)
        if (k < nks) acc += pv[k];
      return acc;
    };
#pragma unroll
    for (int m = 0; m < MP; ++m) {
      if (64 * m >= E) break;
      const int n = lane + 64 * m;
      const float acc = split_sum(n);
      if (n < E) {
        v[m] = acc + (bias ? bias[n] : 0.f);
        l[n] = v[m];
      }  // entries >= E are not read
    }
    if (n_shared) {  // column E: the shared-gate logit (every lane sums it)
      sgl = split_sum(E);
      if (lane == 0) sg_logit[t] = sgl;
    }
  } else {
#pragma unroll
    for (int m = 0; m < MP; ++m) v[m] = l[min(lane + 64 * m, E - 1)];  // entries >= E are not read
    if (n_shared) sgl = sg_logit[t];
  }
  // softmax weights over the selection (norm) or full-softmax entries
  float first = 0.f, denom = 0.f, mine = 0.f;
  int mine_e = 0;
  topk_wave(v, E, K, lane, [&](int k, float mx, uint32_t sel) {
    if (k == 0) first = mx;
    const float ev = expf(mx - first);
    denom += ev;
    if (k == lane) {
      mine = ev;
      mine_e = int(sel);
    }
  });
  if (!norm) {
    float part = 0.f;
#pragma unroll
    for (int m = 0; m < MP; ++m)
      if (lane + 64 * m < E) part += expf(v[m] - first);
    denom = group_sum<64>(part);
  }
  if (lane < K) {
    idx[size_t(t) * K + lane] = mine_e;
    w[size_t(t) * K + lane] = mine / denom;
    // per-chunk expert histogram of the (token, slot) pairs for the grouping
    // (integer adds: the counts do not depend on their order)
    if (lhist) atomicAdd(&lhist[((t * K + lane) / kGroupChunk - c0) * E + mine_e], 1);
  }
  if (n_shared && lane == 0) sw[t] = sigmoid_f(sgl);
}

template <int MP>
__global__ void __launch_bounds__(64 * kTopkTokens) k_topk(float* __restrict__ logits,
                                                            float* __restrict__ sg_logit, int T,
                                                            int E, int K, int n_shared, int norm,
                                                            int32_t* __restrict__ idx,
                                                            float* __restrict__ w,
                                                            float* __restrict__ sw,
                                                            const float* __restrict__ plog,
                                                            int nks, const float* __restrict__ bias,
                                                            int32_t* __restrict__ hist) {
  // the workgroup's pairs lie in at most two chunks (kTopkTokens K <= kGroupChunk)
  __shared__ int lhist[2 * kMaxE];
  const int t0 = blockIdx.x * kTopkTokens, t = t0 + (threadIdx.x >> 6);
  const int c0 = (t0 * K) / kGroupChunk;
  if (hist) {
    for (int i = threadIdx.x; i < 2 * E; i += 64 * kTopkTokens) lhist[i] = 0;
    __syncthreads();
  }
  if (t < T)
    topk_token<MP>(logits, sg_logit, t, T, E, K, n_shared, norm, idx, w, sw, plog, nks, bias,
                   hist ? lhist : nullptr, c0);
  if (hist) {
    __syncthreads();
    const int nch = (T * K + kGroupChunk - 1) / kGroupChunk;
    for (int i = threadIdx.x; i < 2 * E; i += 64 * kTopkTokens) {
      const int v = lhist[i], c = c0 + i / E;
      if (v && c < nch) atomicAdd(&hist[size_t(c) * E + i % E], v);
    }
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
template <int H>
static hipError_t launch_router_logits_t(const int8_t* q, const float* s, const int8_t* sq,
                                         const float* ss, const uint16_t* x, const float* bias,
                                         int E, int n_shared, int T, float* logits,
                                         float* sg_logit, hipStream_t st, int32_t* zero,
                                         int nzero) {
  using G = Geo<H>;
  const int rows = E + n_shared;
  dim3 grid((rows + 4 * G::RPL - 1) / (4 * G::RPL), T);
  hipLaunchKernelGGL(k_router_logits<H>, grid, dim3(256), 0, st, q, s, sq, ss, x, bias, E,
                     n_shared, logits, sg_logit, zero, nzero);
  return hipGetLastError();
}

hipError_t launch_router_logits(int H, const int8_t* q, const float* s, const int8_t* sq,
                                const float* ss, const uint16_t* x, const float* bias, int E,
                                int n_shared, int T, float* logits, float* sg_logit,
                                hipStream_t st, int32_t* zero, int nzero) {
#define MOE_CASE(V) \
  case V:           \
    return launch_router_logits_t<V>(q, s, sq, ss, x, bias, E, n_shared, T, logits, sg_logit, st, \
                                     zero, nzero);
  switch (H) {
    MOE_FOR_EACH_WIDTH(MOE_CASE)
    default:
      return hipErrorInvalidValue;
  }
#undef MOE_CASE
}

hipError_t launch_topk(float* logits, float* sg_logit, int T, int E, int K, int n_shared,
                       int norm, int32_t* idx, float* w, float* sw, hipStream_t st,
                       const float* plog, int nks, const float* bias, int32_t* hist) {
  if (plog && (nks < 1 || nks > kMaxTopkSplits)) return hipErrorInvalidValue;
  static_assert(kTopkTokens * kMaxK <= kGroupChunk, "a workgroup's pairs span at most two chunks");
  const dim3 grid((T + kTopkTokens - 1) / kTopkTokens), block(64 * kTopkTokens);
  if (E <= 256)  // four logits per lane
    hipLaunchKernelGGL(k_topk<4>, grid, block, 0, st, logits, sg_logit, T, E, K, n_shared, norm,
                       idx, w, sw, plog, nks, bias, hist);
  else
    hipLaunchKernelGGL(k_topk<kMaxE / 64>, grid, block, 0, st, logits, sg_logit, T, E, K,
                       n_shared, norm, idx, w, sw, plog, nks, bias, hist);
  return hipGetLastError();
}

}  // namespace moe

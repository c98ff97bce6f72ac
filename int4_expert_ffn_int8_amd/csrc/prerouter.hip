// Prerouter head: z = W2 silu(W1 h), prediction = top-K of z.
//
// [P1] "Edge0开源框架实现35BMoE模型在Mac上流式推理…", Prerouter paragraph: a
// light MLP head predicts the next layer's top-K experts so that loading can
// overlap compute.  [P2] "SSD 专家卸载 · Prerouter 路由预测", double-shift
// paragraph: the head after layer N predicts layer N+1 for the next token.
#include <math.h>

#include "device_utils.h"
#include "handoff.h"
#include "launch.h"
#include "moe_internal.h"
#include "status.h"
#include "topk.h"

// Timeline marks: a timing build of this file defines PR_MARK(k) to record
// the wall clock of a workgroup's phases; here they are empty.
#ifndef PR_MARK
#define PR_MARK(k)
#endif

namespace moe {

constexpr unsigned kPrSpinLimit = 1u << 20;  // bounded wait of the gathering workgroup (~0.2 s)
constexpr int kPrSyncBytes = 256;            // the 64-bit launch counter at byte 0
constexpr int kPrMinRows = 8;                // smallest row block: the workspace holds
                                             // ceil(D / 8) partial-logit blocks per token
constexpr int kPrGatherWords = 32;           // partial-logit words a gathering thread loads per round

struct PrArgs {
  const uint16_t* W1;  // [D][ldw] bf16
  int ldw;
  const uint16_t* W2;  // [E][D] bf16
  const uint16_t* h;   // [T][H] bf16
  const int32_t* prev; // [T][Kp] or null
  int Kp, D, E, K, T, nB;
  int32_t* pred_idx;   // [T][K]
  float* pred_logits;  // [T][E] or null
  unsigned long long* ctr;
  tword_t* zp;         // [T][nB][E] tagged partial logits
};

// W1 rows of one workgroup: each wave takes RW rows, RPL per row load of the
// lane layout (a lane owns 32 consecutive columns of h).  Blocks of 8 rows
// (for H >= 1024) measured fastest for a 256 x 2048 W1: more, smaller blocks
// shorten the W1 phase by more than the larger gather costs.
template <int H>
struct PrGeo {
  static constexpr int RPL = Geo<H>::RPL;
  static constexpr int RW = RPL > 2 ? RPL : 2;  // rows per wave
  static constexpr int NL = RW / RPL;            // row loads per lane
  static constexpr int DB = 4 * RW;              // rows per workgroup
  static constexpr int NQ = DB / 8;              // 16-byte W2 chunks per expert row
  static constexpr int NK = (kMaxK + Geo<H>::LPR - 1) / Geo<H>::LPR;  // features per lane
  static_assert(DB % kPrMinRows == 0, "row blocks are whole 8-row W2 chunks");
};

// One launch per head, grid (nB, T), block 256.  Workgroup (b, t):
//   a[d] = silu(sum_i W1[d, i] h[t, i] + sum_e W1[d, H + e])
// for its DB rows d, the second sum over the distinct ids e in [0, E) of
// prev[t, :] (the one-hot of the experts the layer executed, appended to h;
// empty when prev is NULL), then its block's partial of the expert logits,
// zp[b][e] = sum over its rows of W2[e, d] a[d], handed over as tagged words.
// Workgroup (nB - 1, t), the last of the token's to start, adds its own
// partial to the others in block order and runs the wave top-K.  It waits
// only on workgroups with lower ids.  a stays in fp32 throughout.
template <int H>
__global__ void __launch_bounds__(256) k_prerouter(PrArgs a) {
  using G = Geo<H>;
  using P = PrGeo<H>;
  constexpr int NE = kMaxE / 256;  // experts per thread
  __shared__ float lds_a[P::DB];
  __shared__ float lds_z[kMaxE];
  __shared__ unsigned s_tag;
  PR_MARK(0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, sub = lane % G::LPR;
  const int b = blockIdx.x, t = blockIdx.y;
  const int d0 = b * P::DB;
  const int ne = (a.E + 255) / 256;
  const bool gather = b == a.nB - 1;
  unsigned long long c0 = 0;
  if (tid == 0) c0 = counter_read(a.ctr);

  // loads first: executed-expert ids, W1 rows (clamped to row D - 1), h, the
  // one-hot columns of W1, then the W2 block
  int pv[P::NK];  // the lane's ids, -1 where out of range or repeated (the one-hot is an indicator)
  {
    int pu[kMaxK];  // the token's whole list
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) pu[k] = k < a.Kp ? a.prev[size_t(t) * a.Kp + k] : -1;
#pragma unroll
    for (int k = 0; k < P::NK; ++k) {
      const int kk = sub + k * G::LPR;
      const int id = kk < a.Kp ? a.prev[size_t(t) * a.Kp + kk] : -1;
      bool first = id >= 0 && id < a.E;
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) first &= !(j < kk && pu[j] == id);
      pv[k] = first ? id : -1;
    }
  }
  uint4 q[P::NL][G::SL][4];
  int rows[P::NL];
#pragma unroll
  for (int i = 0; i < P::NL; ++i) {
    rows[i] = d0 + wave * P::RW + i * G::RPL + lane / G::LPR;
    const int rc = min(rows[i], a.D - 1);
#pragma unroll
    for (int c = 0; c < G::SL; ++c)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        q[i][c][k] = reinterpret_cast<const uint4*>(a.W1 + size_t(rc) * a.ldw + 32 * sub + 2048 * c)[k];
  }
  uint32_t xw[G::SL][16];
#pragma unroll
  for (int c = 0; c < G::SL; ++c)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint4 v = reinterpret_cast<const uint4*>(a.h + size_t(t) * H + 32 * sub + 2048 * c)[k];
      xw[c][4 * k] = v.x; xw[c][4 * k + 1] = v.y; xw[c][4 * k + 2] = v.z; xw[c][4 * k + 3] = v.w;
    }
  float fw[P::NL][P::NK];
#pragma unroll
  for (int i = 0; i < P::NL; ++i)
#pragma unroll
    for (int k = 0; k < P::NK; ++k) {
      const int rc = min(rows[i], a.D - 1);
      fw[i][k] = pv[k] >= 0 ? bf16_to_f32(a.W1[size_t(rc) * a.ldw + H + pv[k]]) : 0.f;
    }
  constexpr int PQ = P::NQ * NE <= 8 ? P::NQ : 1;  // W2 chunks held per expert row
  uint4 w2[NE][PQ];
  if (P::NQ * NE <= 8) {
#pragma unroll
    for (int j = 0; j < NE; ++j)
      if (j < ne) {
        const int e = min(tid + 256 * j, a.E - 1);
#pragma unroll
        for (int qq = 0; qq < PQ; ++qq)
          w2[j][qq] = d0 + 8 * qq < a.D
                          ? reinterpret_cast<const uint4*>(a.W2 + size_t(e) * a.D + d0)[qq]
                          : make_uint4(0, 0, 0, 0);
      }
  }
  if (tid == 0) {  // the launch's tag, handed to the workgroup at the barrier below
    s_tag = counter_tag(c0);
    counter_arrive(a.ctr, c0, t * a.nB + b, a.nB * a.T);
  }

  // a for the block's rows
#pragma unroll
  for (int i = 0; i < P::NL; ++i) {
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < G::SL; ++c)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc = dot2_bf16(q[i][c][k].x, xw[c][4 * k], acc);
        acc = dot2_bf16(q[i][c][k].y, xw[c][4 * k + 1], acc);
        acc = dot2_bf16(q[i][c][k].z, xw[c][4 * k + 2], acc);
        acc = dot2_bf16(q[i][c][k].w, xw[c][4 * k + 3], acc);
      }
#pragma unroll
    for (int k = 0; k < P::NK; ++k)
      if (pv[k] >= 0) acc += fw[i][k];
    acc = group_sum<G::LPR>(acc);
    if (sub == 0) lds_a[rows[i] - d0] = rows[i] < a.D ? silu_f(acc) : 0.f;
  }
  PR_MARK(1);
  __syncthreads();
  const unsigned tag = s_tag;

  // the block's partial logits
  float zown[NE];
#pragma unroll
  for (int j = 0; j < NE; ++j) {
    zown[j] = 0.f;
    if (j >= ne) continue;
    const int e = tid + 256 * j;
    const int ec = min(e, a.E - 1);
    float acc = 0.f;
#pragma unroll
    for (int qq = 0; qq < P::NQ; ++qq) {
      if (d0 + 8 * qq >= a.D) break;
      const uint4 w = P::NQ * NE <= 8 ? w2[j][qq % PQ]
                                       : reinterpret_cast<const uint4*>(a.W2 + size_t(ec) * a.D + d0)[qq];
      const float* av = lds_a + 8 * qq;
      acc = fmaf(bf16_lo(w.x), av[0], acc);
      acc = fmaf(bf16_hi(w.x), av[1], acc);
      acc = fmaf(bf16_lo(w.y), av[2], acc);
      acc = fmaf(bf16_hi(w.y), av[3], acc);
      acc = fmaf(bf16_lo(w.z), av[4], acc);
      acc = fmaf(bf16_hi(w.z), av[5], acc);
      acc = fmaf(bf16_lo(w.w), av[6], acc);
      acc = fmaf(bf16_hi(w.w), av[7], acc);
    }
    zown[j] = acc;
    if (!gather && e < a.E) st_dev(&a.zp[(size_t(t) * a.nB + b) * a.E + e], twf(tag, acc));
  }
  PR_MARK(2);
  if (!gather) return;

  // wait for blocks 0 .. nB-2 of this token, kPrGatherWords at a time, and
  // add them in block order; a wait that runs out leaves -1 in the token's
  // predictions
  bool timed_out = false;
#pragma unroll
  for (int j = 0; j < NE; ++j) {
    if (j >= ne) continue;
    const int e = tid + 256 * j;
    const int ec = min(e, a.E - 1);
    float s = 0.f;
    for (int b0 = 0; b0 < a.nB - 1; b0 += kPrGatherWords) {
      tword_t w[kPrGatherWords];
      for (unsigned it = 0;; ++it) {
#pragma unroll
        for (int kk = 0; kk < kPrGatherWords; ++kk)
          w[kk] = ld_dev(&a.zp[(size_t(t) * a.nB + min(b0 + kk, a.nB - 2)) * a.E + ec]);
        bool ok = true;
#pragma unroll
        for (int kk = 0; kk < kPrGatherWords; ++kk)
          ok &= (b0 + kk >= a.nB - 1) || has_tag(w[kk], tag);
        if (__syncthreads_and(ok)) break;
        if (timed_out || it >= kPrSpinLimit) {  // one bounded wait per launch
          timed_out = true;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
#pragma unroll
      for (int kk = 0; kk < kPrGatherWords; ++kk)
        if (b0 + kk < a.nB - 1) s += wf(w[kk]);
    }
    s += zown[j];
    if (e < a.E) {
      lds_z[e] = s;
      if (a.pred_logits) a.pred_logits[size_t(t) * a.E + e] = s;
    }
  }
  __syncthreads();
  PR_MARK(3);
  if (wave == 0) {
    float vin[kMaxE / 64];
#pragma unroll
    for (int m = 0; m < kMaxE / 64; ++m) vin[m] = lds_z[min(lane + 64 * m, a.E - 1)];
    int32_t* out = a.pred_idx + size_t(t) * a.K;
    topk_wave<kMaxE / 64>(vin, a.E, a.K, lane, [&](int k, float, uint32_t e) {
      if (lane == 0) out[k] = timed_out ? -1 : int32_t(e);
    });
    PR_MARK(4);
  }
}

template <int H>
static hipError_t launch_prerouter_t(PrArgs a, hipStream_t st) {
  a.nB = (a.D + PrGeo<H>::DB - 1) / PrGeo<H>::DB;
  hipLaunchKernelGGL(k_prerouter<H>, dim3(a.nB, a.T), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe

using namespace moe;

extern "C" size_t prerouter_workspace_bytes(int32_t D, int32_t E, int32_t T) {
  if (D <= 0 || E <= 0 || T < 0) return 0;
  // launch counter, partial logits of at most ceil(D / 8) row blocks per token
  return kPrSyncBytes + align256(size_t(T) * ((D + kPrMinRows - 1) / kPrMinRows) * E * 8);
}

static moe_status_t prerouter_run(const char* fn, const uint16_t* W1, int ldw, const uint16_t* W2,
                                  int32_t H, int32_t D, int32_t E, int32_t K, const uint16_t* h,
                                  const int32_t* prev, int32_t Kp, int32_t T, int32_t* pred_idx,
                                  float* pred_logits, void* ws, size_t ws_bytes, void* stream) {
  if (H <= 0 || D <= 0 || H % kGroup || D % kGroup)
    return fail(MOE_EINVAL, "%s: H=%d, D=%d must be positive multiples of 64", fn, H, D);
  if (!width_supported(H))
    return fail(MOE_EUNSUPPORTED, "%s: H=%d not in {64,...,4096} powers of two", fn, H);
  if (D > 4096) return fail(MOE_EUNSUPPORTED, "%s: D=%d above 4096", fn, D);
  if (E < 1 || E > kMaxE) return fail(MOE_EUNSUPPORTED, "%s: E=%d outside [1, %d]", fn, E, kMaxE);
  if (ldw % 8)
    return fail(MOE_EUNSUPPORTED, "%s: W1 rows of %d columns: H + E must be a multiple of 8", fn, ldw);
  if (K < 1 || K > E || K > kMaxK)
    return fail(MOE_EINVAL, "%s: K=%d outside [1, min(E, %d)]", fn, K, kMaxK);
  if (Kp < 0 || Kp > kMaxK) return fail(MOE_EINVAL, "%s: Kp=%d outside [0, %d]", fn, Kp, kMaxK);
  if (T < 0) return fail(MOE_EINVAL, "%s: T=%d is negative", fn, T);
  if (T > 65535) return fail(MOE_EUNSUPPORTED, "%s: T=%d above 65535 tokens per call", fn, T);
  if (T == 0) return MOE_OK;
  if (!W1 || !W2 || !h || !pred_idx || (Kp > 0 && !prev)) return fail(MOE_EINVAL, "%s: null pointer", fn);
  const size_t need = prerouter_workspace_bytes(D, E, T);
  if (!ws || ws_bytes < need)
    return fail(MOE_EWORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  PrArgs a;
  a.W1 = W1; a.ldw = ldw; a.W2 = W2; a.h = h; a.prev = Kp > 0 ? prev : nullptr;
  a.Kp = Kp; a.D = D; a.E = E; a.K = K; a.T = T; a.nB = 0;
  a.pred_idx = pred_idx; a.pred_logits = pred_logits;
  a.ctr = reinterpret_cast<unsigned long long*>(wsb);
  a.zp = reinterpret_cast<tword_t*>(wsb + kPrSyncBytes);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipErrorInvalidValue;
#define MOE_CASE(V)                            \
  case V:                                      \
    e = launch_prerouter_t<V>(a, st);          \
    break;
  switch (H) { MOE_FOR_EACH_WIDTH(MOE_CASE) }
#undef MOE_CASE
  if (e != hipSuccess) return fail(MOE_EHIP, "%s: %s", fn, hipGetErrorString(e));
  return MOE_OK;
}

extern "C" moe_status_t prerouter_predict(const uint16_t* W1, const uint16_t* W2, int32_t H,
                                          int32_t D, int32_t E, int32_t K, const uint16_t* h,
                                          int32_t T, int32_t* pred_idx, float* pred_logits,
                                          void* ws, size_t ws_bytes, void* stream) {
  return prerouter_run("prerouter_predict", W1, H, W2, H, D, E, K, h, nullptr, 0, T, pred_idx,
                       pred_logits, ws, ws_bytes, stream);
}

extern "C" moe_status_t prerouter_predict_feat(const uint16_t* W1, const uint16_t* W2, int32_t H,
                                               int32_t D, int32_t E, int32_t K, const uint16_t* h,
                                               const int32_t* prev_idx, int32_t Kp, int32_t T,
                                               int32_t* pred_idx, float* pred_logits, void* ws,
                                               size_t ws_bytes, void* stream) {
  return prerouter_run("prerouter_predict_feat", W1, H + E, W2, H, D, E, K, h, prev_idx, Kp, T,
                       pred_idx, pred_logits, ws, ws_bytes, stream);
}

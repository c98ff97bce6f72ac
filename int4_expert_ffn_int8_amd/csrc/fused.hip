// Fused decode: one launch runs a whole MoE block for a few tokens.
//
// [P2] "SSD 专家卸载 · Prerouter 路由预测", decode paragraph: route, then
// stream the chosen experts, then compute.  On MI355X a decode block moves
// ~10 MB, which HBM delivers in ~1.3 us, while each kernel boundary costs
// over a microsecond; so the block is one kernel whose workgroups take roles
// and hand results to each other through device memory:
//
//   router    logits of its gate rows (x = optional RMSNorm of h_in, done
//             redundantly and identically in every workgroup); the last
//             router workgroup also waits for every logit and runs the
//             wavefront top-K, publishing ids, weights and the shared gate.
//             With given experts (prediction-as-routing, [P3] "三件套"
//             Prerouter bullet) it publishes those instead, weighted by the
//             softmax of their logits.
//   lora_a    u = [A_gate; A_up] x for one (token, slot) pair.
//   gate_up   16 gate/up outputs of one pair (+ lambda B u), SwiGLU -> h
//             (fp16 with one power-of-two exponent per 16 columns), and that
//             block's partial of v = A_down h.
//   vred      v = sum of a pair's partials, in block order.
//   down      a few output rows for every pair: y = deq(Q_down) h +
//             lambda B_down v, then the weighted combine (+ residual) -> out.
//
// Weight loads are issued before the waits they do not depend on (shared
// expert from the start, routed experts as soon as their ids arrive).  An
// expert that is not resident in the pool is read from the pinned host copy,
// after an optional modeled storage latency (a bounded wall-clock wait, once
// per workgroup).  A role waits only on roles with lower workgroup ids, which
// the dispatcher starts first, and every wait is bounded: on timeout the
// kernel records an error and still runs to completion.
//
// Hand-off protocol.  The 8 XCDs have separate L2 caches, and a device-scope
// release/acquire fence writes back / invalidates a whole L2, which at one
// fence per workgroup costs far more than the block itself.  So every value
// one workgroup hands to another is a 64-bit word -- payload in the low half,
// the launch's tag in the high half -- written and read with device-scope
// relaxed atomics (loads and stores that bypass the XCD L2s).  A producer just
// stores; a consumer loads every word it needs and repeats the loads until all
// of them carry this launch's tag.  The tag is the launch epoch + 1; the last
// workgroup to finish bumps the epoch, so stale words of earlier launches
// never match and nothing needs clearing.  Weights and inputs, read-only in
// the kernel, use ordinary cached loads.
//
// Such loads are served at the memory side, so hundreds of workgroups
// re-reading one word serialise there.  Words read by many workgroups
// (routes, weights, u, h and its exponents, v) are therefore written in 8
// copies and each reader takes the copy of its XCD; the down role first waits
// for one word per h block from a single wave, then reads its h words once,
// instead of polling all of them from every thread.
//
// Load discipline.  Vector loads complete in order, so a load whose value is
// used inside a divergent branch makes the wave wait for every load issued
// before it.  Every batch of loads here is therefore issued unconditionally
// (indices clamped to valid elements), and guards, tag checks and arithmetic
// run in a second pass.
#include "device_utils.h"
#include "fused.h"
#include "handoff.h"
#include "launch.h"
#include "moe_internal.h"
#include "topk.h"

// Timeline marks: a timing build of this file defines FUSED_MARK(k) to record
// the wall clock of a workgroup's phases; here they are empty.
#ifndef FUSED_MARK
#define FUSED_MARK(k)
#endif

namespace moe {

__device__ __forceinline__ int* slot(const FusedArgs& a, int s) { return a.sync + s * kSlotInts; }

__device__ __forceinline__ unsigned long long* launch_counter(const FusedArgs& a) {
  return reinterpret_cast<unsigned long long*>(slot(a, kSlotEpoch));
}
// this launch's tag (never 0); every thread may read it until its workgroup
// arrives at the kernel's end
__device__ __forceinline__ unsigned launch_tag(const FusedArgs& a) {
  return counter_tag(counter_read(launch_counter(a)));
}

// the copy of broadcast words this workgroup reads: its XCD's (workgroups
// are spread over the 8 XCDs round-robin by id)
__device__ __forceinline__ int xcd_copy() { return int(blockIdx.x) & (kCopies - 1); }

__device__ __forceinline__ void set_err(const FusedArgs& a) { st_dev(slot(a, kSlotErr), 1); }

// one thread waits (bounded, with sleeps) until *w carries `tag`
__device__ __forceinline__ tword_t poll_word(const FusedArgs& a, const tword_t* w, unsigned tag) {
  unsigned n = 0;
  tword_t v;
  while (!has_tag(v = ld_dev(w), tag)) {
    __builtin_amdgcn_s_sleep(2);
    if (++n > kFusedSpinLimit) {
      set_err(a);
      break;
    }
  }
  return v;
}

// Workgroup-wide retry of a load round: true once every thread's words were
// valid; sleeps between rounds and gives up (recording the error) after the
// spin limit.
__device__ __forceinline__ bool round_done(const FusedArgs& a, bool ok, unsigned& n) {
  if (__syncthreads_and(ok)) return true;
  if (++n > kFusedSpinLimit) {
    if (threadIdx.x == 0) set_err(a);
    return true;
  }
  __builtin_amdgcn_s_sleep(2);
  return false;
}

// pair index of work unit q: shared-expert pairs first (they need no routing)
__device__ __forceinline__ int pair_of_unit(const FusedArgs& a, int q) {
  const int KS = a.K + a.S;
  if (q < a.S * a.T) return q * KS + a.K;
  q -= a.S * a.T;
  return (q / a.K) * KS + q % a.K;
}

// blob of routed expert e (pool lookup); `miss` is set when the blob is the
// pinned host copy (the expert is not resident in a slot)
__device__ __forceinline__ const uint8_t* expert_blob_at(const FusedArgs& a, int e, bool count,
                                                         bool& miss) {
  if (a.src.expert_to_slot == nullptr) return a.src.slots + size_t(e) * a.src.stride;
  const int s = a.src.expert_to_slot[e];
  if (count && a.src.counters) {
    atomicAdd(&a.src.counters[1], 1ull);
    if (s >= 0) atomicAdd(&a.src.counters[0], 1ull);
  }
  if (s >= 0) return a.src.slots + size_t(s) * a.src.stride;
  miss = true;
  return a.src.host_blobs + size_t(e) * a.src.stride;
}

// The modeled storage latency of the host reads a workgroup is about to
// issue: one wait however many of its blobs missed (the reads are issued
// together, so they wait in parallel).
__device__ __forceinline__ void storage_latency(const FusedArgs& a, bool miss) {
  if (miss && a.src.delay_ticks) wall_wait(a.src.delay_ticks);
}

__device__ __forceinline__ const uint8_t* expert_blob(const FusedArgs& a, int e, bool count) {
  bool miss = false;
  const uint8_t* b = expert_blob_at(a, e, count, miss);
  storage_latency(a, miss);
  return b;
}

// Expert id of routed pair p, published by the top-K (workgroup-uniform).
__device__ __forceinline__ int wait_expert(const FusedArgs& a, int p, unsigned tag, int* lds_int) {
  const int KS = a.K + a.S;
  if (threadIdx.x == 0)
    *lds_int = int(uint32_t(poll_word(
        a, &a.route[(xcd_copy() * a.T + p / KS) * a.K + p % KS], tag)));
  __syncthreads();
  return *lds_int;
}

// The lane's 32 columns of the token input x (bf16 pairs) and their sum.
// With norm, x = bf16(h * rsqrt(mean(h^2) + eps)); the lanes of one row group
// cover all H columns, so the mean needs no cross-wave step and every
// workgroup computes bit-identical x.
template <int H>
__device__ __forceinline__ void token_slice(const FusedArgs& a, int t, int sub, uint32_t (&xw)[16],
                                            float& xs) {
  using G = Geo<H>;
  const uint4* hp = reinterpret_cast<const uint4*>(a.h_in + size_t(t) * H + 32 * sub);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint4 v = hp[k];
    xw[4 * k] = v.x; xw[4 * k + 1] = v.y; xw[4 * k + 2] = v.z; xw[4 * k + 3] = v.w;
  }
  if (a.norm_input) {
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float lo = bf16_lo(xw[k]), hi = bf16_hi(xw[k]);
      ss = fmaf(lo, lo, ss);
      ss = fmaf(hi, hi, ss);
    }
    ss = group_sum<G::LPR>(ss);
    const float inv = 1.0f / sqrtf(ss / float(H) + a.eps);
#pragma unroll
    for (int k = 0; k < 16; ++k) xw[k] = pack_bf16x2(bf16_lo(xw[k]) * inv, bf16_hi(xw[k]) * inv);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) s += bf16_lo(xw[k]) + bf16_hi(xw[k]);
  xs = s;
}

// (s*q + b) . x over the lane's 32 columns of bf16 x
__device__ __forceinline__ float slice_dot_bf16(const uint4 q, uint32_t sbw, const uint32_t* xw,
                                                float xs) {
  const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
  float acc = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = dot2_bf16(codes_to_bf16x2_biased(qw[d], s), xw[4 * d + s], acc);
  const float sc = bf16_lo(sbw), bi = bf16_hi(sbw);
  return fmaf(sc, acc, (bi - 128.0f * sc) * xs);
}

// ---------------------------------------------------------------------------
// One wave routes token t: waits for all its logits (and the shared-gate
// logit), selects (or takes the given experts), publishes ids and weights.
// MP logits per lane (experts lane + 64 m).
template <int MP>
__device__ void route_token(const FusedArgs& a, int t, int lane, unsigned tag) {
  const tword_t* l = a.logits + t * (a.E + 1);
  float v[MP];
  float sgl = 0.f;
  for (unsigned n = 0;; ++n) {
    tword_t w[MP];
#pragma unroll
    for (int m = 0; m < MP; ++m) w[m] = ld_dev(&l[min(lane + 64 * m, a.E - 1)]);
    const tword_t ws = ld_dev(&l[a.E]);  // shared-gate logit (unused without S)
    unsigned bad = unsigned(a.S != 0) & unsigned(!has_tag(ws, tag));
#pragma unroll
    for (int m = 0; m < MP; ++m) {
      bad |= unsigned(lane + 64 * m < a.E) & unsigned(!has_tag(w[m], tag));
      v[m] = wf(w[m]);
    }
    sgl = wf(ws);
    if (__all(bad == 0)) break;
    if (++n > kFusedSpinLimit) {
      if (lane == 0) set_err(a);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  if (t == 0) FUSED_MARK(2);
  // Lane l holds slot k = l % 8 of the selection (K <= 8 here): every group
  // of 8 lanes computes the weights, and group c publishes copy c.
  const int kk = lane & 7;
  float first = 0.f, mine_l = -INFINITY;
  int mine_e = 0;
  if (a.exec_idx == nullptr) {
    auto emit = [&](int k, float mx, uint32_t sel) {
      if (k == 0) first = mx;  // the largest logit
      if (k == kk) {
        mine_l = mx;
        mine_e = int(sel);
      }
    };
    if constexpr (MP > 4)  // E > 256
      topk_wave_scan<MP>(v, a.E, a.K, lane, emit);
    else
      topk_wave(v, a.E, a.K, lane, emit);
  } else {
    // given experts: slot k takes expert exec_idx[t][k] and fetches its logit
    // from the lane that holds it
    if (kk < a.K) {
      mine_e = a.exec_idx[t * a.K + kk];
      if (uint32_t(mine_e) >= uint32_t(a.E)) {
        set_err(a);
        mine_e = 0;
      }
    }
    float gl = 0.f;
#pragma unroll
    for (int m = 0; m < MP; ++m) {
      if (64 * m >= a.E) break;
      const float c = __shfl(v[m], mine_e & 63);
      if ((mine_e >> 6) == m) gl = c;
    }
    mine_l = kk < a.K ? gl : -INFINITY;
    first = wave_max(mine_l);
  }
  // the ids first: the expert roles wait on them, the weights only the combine
  const int c = lane >> 3;
  if (kk < a.K) st_dev(&a.route[(c * a.T + t) * a.K + kk], tw(tag, uint32_t(mine_e)));
  float mine = kk < a.K ? expf(mine_l - first) : 0.f;
  float denom;
  if (a.norm_topk) {
    denom = group_sum<8>(mine);  // fixed pairing: the same bits on every path
  } else {  // full-softmax entries: denominator over all E, from the largest logit
    float mx = -INFINITY;
#pragma unroll
    for (int m = 0; m < MP; ++m)
      if (lane + 64 * m < a.E) mx = fmaxf(mx, v[m]);
    const float top = wave_max(mx);
    mine = kk < a.K ? expf(mine_l - top) : 0.f;
    float part = 0.f;
#pragma unroll
    for (int m = 0; m < MP; ++m)
      if (lane + 64 * m < a.E) part += expf(v[m] - top);
    denom = group_sum<64>(part);
  }
  const float wv = mine / denom;
  if (lane < a.K) {
    if (a.user_idx) a.user_idx[t * a.K + lane] = mine_e;
    if (a.user_w) a.user_w[t * a.K + lane] = wv;
  }
  if (kk < a.K) st_dev(&a.wts[(c * a.T + t) * (a.K + 1) + kk], twf(tag, wv));
  if (a.S && kk == 0) st_dev(&a.wts[(c * a.T + t) * (a.K + 1) + a.K], twf(tag, sigmoid_f(sgl)));
  if (t == 0) FUSED_MARK(3);
}

template <int H>
__device__ void role_router(const FusedArgs& a, int b) {
  using G = Geo<H>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, sub = lane % G::LPR;
  const int row = (b * 4 + wave) * G::RPL + lane / G::LPR;
  const int rows = a.E + a.S;
  const bool valid = row < rows;
  uint4 w0 = make_uint4(0, 0, 0, 0), w1 = w0;
  float sc = 0.f;
  if (valid) {
    const int8_t* q = (row < a.E) ? a.rq + size_t(row) * H : a.sq;
    const float* s = (row < a.E) ? a.rs + size_t(row) * (H / 64) : a.ss;
    w0 = *reinterpret_cast<const uint4*>(q + 32 * sub);
    w1 = *reinterpret_cast<const uint4*>(q + 32 * sub + 16);
    sc = s[sub >> 1];
  }
  const unsigned tag = launch_tag(a);
  const uint32_t qw[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  for (int t = 0; t < a.T; ++t) {
    uint32_t xw[16];
    float xs;
    token_slice<H>(a, t, sub, xw, xs);
    float part = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d)
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int col = 4 * d + bb;
        const float qv = float(int8_t((qw[d] >> (8 * bb)) & 0xFF));
        part = fmaf(qv, (col & 1) ? bf16_hi(xw[col >> 1]) : bf16_lo(xw[col >> 1]), part);
      }
    part = group_sum<G::LPR>(sc * part);
    // column E of the logits row holds the shared-gate logit
    if (valid && sub == 0) st_dev(&a.logits[t * (a.E + 1) + row], twf(tag, part));
  }
  FUSED_MARK(1);
  if (b != a.nR - 1) return;
  // The last router workgroup: wait for every logit of its token (one wave
  // per token), then K rounds of wave argmax by (logit desc, index asc).
  for (int t = wave; t < a.T; t += 4) {
    if (a.E <= 256)  // four logits per lane: no loads beyond the experts
      route_token<4>(a, t, lane, tag);
    else
      route_token<kMaxE / 64>(a, t, lane, tag);
  }
}

// ---------------------------------------------------------------------------
template <int H>
__device__ void role_lora_a(const FusedArgs& a, int unit, int part, int* lds_int) {
  using G = Geo<H>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, sub = lane % G::LPR;
  const int p = pair_of_unit(a, unit);
  const int KS = a.K + a.S;
  const int P = a.T * KS;
  const int t = p / KS;
  const bool routed = (p % KS) < a.K;
  const unsigned tag = launch_tag(a);
  uint32_t xw[16];
  float xs;
  token_slice<H>(a, t, sub, xw, xs);
  const uint8_t* blob = a.shared_blob;
  if (routed) blob = expert_blob(a, wait_expert(a, p, tag, lds_int), false);
  FUSED_MARK(1);
  const uint16_t* A = reinterpret_cast<const uint16_t*>(blob + a.L.a_gu);
  const int rows = 2 * a.r;
  const int rw = part * 4 * G::RPL + wave * G::RPL + lane / G::LPR;  // 4 waves x RPL rows
  uint4 q[4];
  const uint4* ap = reinterpret_cast<const uint4*>(A + size_t(min(rw, rows - 1)) * H + 32 * sub);
#pragma unroll
  for (int k = 0; k < 4; ++k) q[k] = ap[k];
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    acc = dot2_bf16(q[k].x, xw[4 * k], acc);
    acc = dot2_bf16(q[k].y, xw[4 * k + 1], acc);
    acc = dot2_bf16(q[k].z, xw[4 * k + 2], acc);
    acc = dot2_bf16(q[k].w, xw[4 * k + 3], acc);
  }
  acc = group_sum<G::LPR>(acc);  // every lane of the row group holds the sum
  static_assert(Geo<256>::LPR >= kCopies, "one lane per copy");
  if (rw < rows && sub < kCopies) st_dev(&a.u[(sub * P + p) * rows + rw], twf(tag, acc));
  FUSED_MARK(2);
}

// ---------------------------------------------------------------------------
template <int H>
__device__ void role_gate_up(const FusedArgs& a, int unit, int blk, float* lds, int* lds_int) {
  using G = Geo<H>;
  constexpr int RPL = G::RPL;
  constexpr int JW = kFusedJW, JPW = JW / 4;  // outputs per workgroup / wave
  constexpr int NR = 2 * JPW, NL = NR / RPL;  // gate + up rows per wave, loads per lane
  static_assert(NR % RPL == 0, "rows per wave");
  static_assert(JW * kMaxR == 256, "one (rank, column) product of v per thread");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, sub = lane % G::LPR;
  const int tid = threadIdx.x;
  const int p = pair_of_unit(a, unit);
  const int KS = a.K + a.S;
  const int P = a.T * KS;
  const int NB = a.I / JW;
  const int t = p / KS;
  const bool routed = (p % KS) < a.K;
  const int j0 = blk * JW + wave * JPW;
  const int r = a.r;
  const unsigned tag = launch_tag(a);
  // the token's input (and its norm) while the route is not yet known
  uint32_t xw[16];
  float xs;
  token_slice<H>(a, t, sub, xw, xs);
  const uint8_t* blob = a.shared_blob;
  if (routed) blob = expert_blob(a, wait_expert(a, p, tag, lds_int), false);
  FUSED_MARK(1);
  // every weight this workgroup needs, before anything waits on data
  const uint8_t* codes = blob + a.L.gu_codes;
  const uint32_t* sb = reinterpret_cast<const uint32_t*>(blob + a.L.gu_sb);
  const uint16_t* Bgu = reinterpret_cast<const uint16_t*>(blob + a.L.b_gu);
  const uint16_t* Ad = reinterpret_cast<const uint16_t*>(blob + a.L.a_dn);
  uint4 q[NL];
  uint32_t sbw[NL];
  int brow[NL];
  uint16_t braw[NL];  // B[row][sub] (one LoRA rank per lane; r <= LPR)
  uint16_t adraw = 0; // A_down[rank tid / JW][column blk * JW + tid % JW]
  const int rc = max(r - 1, 0);
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int ri = i * RPL + lane / G::LPR;
    const int j = j0 + (ri >> 1);
    brow[i] = (ri & 1) ? gu_row_up(j) : gu_row_gate(j);
    q[i] = *reinterpret_cast<const uint4*>(codes + size_t(brow[i]) * (H / 2) + 16 * sub);
    sbw[i] = sb[size_t(brow[i]) * (H / 64) + (sub >> 1)];
  }
  if (r > 0) {
#pragma unroll
    for (int i = 0; i < NL; ++i) braw[i] = Bgu[size_t(brow[i]) * r + min(sub, rc)];
    adraw = Ad[size_t(min(tid / JW, rc)) * a.I + blk * JW + tid % JW];
  }
  float part[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) part[i] = slice_dot_bf16(q[i], sbw[i], xw, xs);
  FUSED_MARK(2);
  float* lds_a = lds;           // [4][NR]
  float* lds_h = lds + 4 * NR;  // [JW]
  float* lds_hraw = lds_h + JW; // [JW]
  if (r > 0) {  // u = A x of this pair (from its lora_a workgroups)
    const tword_t* up = a.u + (size_t(xcd_copy()) * P + p) * 2 * r;
    float uv[2] = {0.f, 0.f};  // lane's rank `sub` of A_gate x and A_up x
    for (unsigned n = 0;; ++n) {
      const tword_t g = ld_dev(&up[min(sub, rc)]);
      const tword_t uu = ld_dev(&up[r + min(sub, rc)]);
      const bool ok = has_tag(g, tag) && has_tag(uu, tag);
      uv[0] = wf(g);
      uv[1] = wf(uu);
      if (round_done(a, ok, n)) break;
    }
    FUSED_MARK(3);
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int ri = i * RPL + lane / G::LPR;
      const float bl = (sub < r) ? a.lam * bf16_to_f32(braw[i]) : 0.f;
      part[i] = fmaf(bl, uv[ri & 1], part[i]);
    }
  }
  // all sums first (independent chains interleave), then the stores
#pragma unroll
  for (int i = 0; i < NL; ++i) part[i] = group_sum<G::LPR>(part[i]);
  int hexp;
  if constexpr (RPL == 1) {
    // each wave holds all rows of its JPW outputs in every lane: SwiGLU in
    // registers, one barrier to share the raw h and the wave maxima
    float hv[JPW], wmax = 0.f;
#pragma unroll
    for (int jl = 0; jl < JPW; ++jl) {
      hv[jl] = silu_f(part[2 * jl]) * part[2 * jl + 1];
      wmax = fmaxf(wmax, fabsf(hv[jl]));
    }
    if (lane < JPW) {
      float hl = hv[0];
#pragma unroll
      for (int jl = 1; jl < JPW; ++jl)
        if (lane == jl) hl = hv[jl];
      lds_hraw[wave * JPW + lane] = hl;
    }
    if (lane == 0) lds_a[wave] = wmax;
    __syncthreads();
    // this block of h is one 16-column slice of the down rows: it is stored
    // as fp16(h * 2^-e) with one exponent e per block (e = 0 unless |h| >= 2^15)
    hexp = h_block_exp(fmaxf(fmaxf(lds_a[0], lds_a[1]), fmaxf(lds_a[2], lds_a[3])));
    // every copy: lanes 2c + i of wave w store word 2w + i (outputs 4w + 2i,
    // 4w + 2i + 1) of copy c
    if (lane < 2 * kCopies) {
      const int i = lane & 1, c = lane >> 1;
      const float h0 = i ? hv[2] : hv[0], h1 = i ? hv[3] : hv[1];
      const f16x2_t pr = {_Float16(f16_to_f32(f32_to_f16_sat(ldexpf(h0, -hexp)))),
                          _Float16(f16_to_f32(f32_to_f16_sat(ldexpf(h1, -hexp))))};
      st_dev(&a.h[(size_t(c) * P + p) * (a.I / 2) + blk * (JW / 2) + 2 * wave + i],
             tw(tag, __builtin_bit_cast(uint32_t, pr)));
    } else if (wave == 0 && lane >= 32 && lane < 32 + kCopies) {
      st_dev(&a.hexp[(size_t(lane - 32) * P + p) * NB + blk], tw(tag, uint32_t(hexp)));
    }
    // the block's h as the down rows will see it, for the v partial
    if (tid < JW)
      lds_h[tid] = ldexpf(f16_to_f32(f32_to_f16_sat(ldexpf(lds_hraw[tid], -hexp))), hexp);
    __syncthreads();
  } else {
    if (sub == 0) {
#pragma unroll
      for (int i = 0; i < NL; ++i) lds_a[wave * NR + i * RPL + lane / G::LPR] = part[i];
    }
    __syncthreads();
    if (tid < JW) {
      const int w = tid / JPW, jl = tid % JPW;
      lds_hraw[tid] = silu_f(lds_a[w * NR + 2 * jl]) * lds_a[w * NR + 2 * jl + 1];
    }
    __syncthreads();
    // this block of h is one 16-column slice of the down rows: it is stored as
    // fp16(h * 2^-e) with one exponent e per block (e = 0 unless |h| >= 2^15)
    float hmax = 0.f;
#pragma unroll
    for (int j = 0; j < JW; ++j) hmax = fmaxf(hmax, fabsf(lds_hraw[j]));
    hexp = h_block_exp(hmax);
    if (tid < JW) lds_h[tid] = ldexpf(f16_to_f32(f32_to_f16_sat(ldexpf(lds_hraw[tid], -hexp))), hexp);
    __syncthreads();
    // every copy: fp16 pairs of h * 2^-e (one tagged word per pair), then e
    if (tid < kCopies * (JW / 2)) {
      const int c = tid / (JW / 2), i = tid % (JW / 2);
      const f16x2_t pr = {_Float16(ldexpf(lds_h[2 * i], -hexp)), _Float16(ldexpf(lds_h[2 * i + 1], -hexp))};
      st_dev(&a.h[(size_t(c) * P + p) * (a.I / 2) + blk * (JW / 2) + i],
             tw(tag, __builtin_bit_cast(uint32_t, pr)));
    } else if (tid >= 64 && tid < 64 + kCopies) {
      st_dev(&a.hexp[(size_t(tid - 64) * P + p) * NB + blk], tw(tag, uint32_t(hexp)));
    }
  }
  FUSED_MARK(4);
  if (r > 0) {  // this block's partial of v = A_down h: thread (rank, column)
    const int rr = tid / JW, jj = tid % JW;
    const float ad = (rr < r) ? bf16_to_f32(adraw) : 0.f;
    const float prod = group_sum<JW>(ad * lds_h[jj]);
    if (jj == 0 && rr < r) st_dev(&a.vpart[(size_t(p) * NB + blk) * r + rr], twf(tag, prod));
  }
}

// ---------------------------------------------------------------------------
// v of one pair: its NB blocks' partials of A_down h.  Thread (rank tid % 16,
// group tid / 16) adds blocks group, group + 16, ... in order; the 16 group
// sums of a rank are then added in group order (a fixed order: the same bits
// every launch).
template <int I>
__device__ void role_vred(const FusedArgs& a, int unit, float* lds) {
  constexpr int NB = I / kFusedJW;
  constexpr int NBG = (NB + 15) / 16;  // blocks per thread
  static_assert(kMaxR == 16, "one rank per lane of a 16-lane group");
  const int tid = threadIdx.x;
  const int rr = tid & 15, bg = tid >> 4;
  const int p = pair_of_unit(a, unit);
  const int P = a.T * (a.K + a.S);
  const int r = a.r;
  const unsigned tag = launch_tag(a);
  const tword_t* vp = a.vpart + size_t(p) * NB * r;
  const int rc = min(rr, r - 1);
  tword_t w[NBG];
  for (unsigned it = 0;; ++it) {
#pragma unroll
    for (int k = 0; k < NBG; ++k) w[k] = ld_dev(&vp[min(bg + 16 * k, NB - 1) * r + rc]);
    bool ok = true;
#pragma unroll
    for (int k = 0; k < NBG; ++k) ok &= (bg + 16 * k >= NB) || (rr >= r) || has_tag(w[k], tag);
    if (round_done(a, ok, it)) break;
  }
  FUSED_MARK(1);
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < NBG; ++k)
    if (bg + 16 * k < NB) sum += wf(w[k]);
  lds[bg * 16 + rr] = sum;
  __syncthreads();
  if (tid < r * kCopies) {
    const int c = tid / r, k = tid % r;
    float v = 0.f;
#pragma unroll
    for (int g = 0; g < 16; ++g) v += lds[g * 16 + k];  // groups past NB hold 0
    st_dev(&a.v[(size_t(c) * P + p) * r + k], twf(tag, v));
  }
  FUSED_MARK(2);
}

// ---------------------------------------------------------------------------
// Down rows: each lane owns SL slices of kFusedJW (16) columns of its row,
// i.e. whole h exponent blocks.
template <int I>
struct DGeo {
  static constexpr int NS = I / kFusedJW;           // slices per row
  static constexpr int LPR = NS < 64 ? NS : 64;     // lanes per row
  static constexpr int RPL = 64 / LPR;              // rows per wave
  static constexpr int SL = NS / LPR;               // slices per lane
  static_assert(NS % LPR == 0 && SL >= 1, "down geometry");
};

constexpr int kDownDeferSleep = 110;  // x 64 shader clocks

template <int H, int I>
__device__ void role_down(const FusedArgs& a, int d, uint16_t* lds_hh, float* lds_hs, int* lds_he,
                          float* lds_v, float* lds_wt, int* lds_idx) {
  using D = DGeo<I>;
  constexpr int LPR = D::LPR, SL = D::SL;
  constexpr int NB = I / kFusedJW;                      // h blocks per pair
  constexpr int MAXH = (kFusedMaxP * I / 2 + 255) / 256;  // h words per thread
  constexpr int MAXE = (kFusedMaxP * NB + 255) / 256;     // exponents per thread
  constexpr int MAXCAN = (kFusedMaxP * NB + 63) / 64;     // exponents per lane of the canary wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, sub = lane % LPR;
  const int tid = threadIdx.x;
  const int row = d * 4 * D::RPL + wave * D::RPL + lane / LPR;
  const bool valid = row < H;
  const int KS = a.K + a.S;
  const int P = a.T * KS;
  const int r = a.r;
  const int c = xcd_copy();
  const unsigned tag = launch_tag(a);
  // Prefetch this lane's down-row slices of every pair into registers: the
  // shared expert at once, routed experts as soon as their ids arrive.
  uint2 q[kFusedMaxP][SL];
  uint32_t sbw[kFusedMaxP][SL];
  uint16_t bdraw[kFusedMaxP];  // B_down[row][sub]
  const uint8_t* bl[kFusedMaxP];
  const int rowc = min(row, H - 1), subr = min(sub, max(r - 1, 0));
  auto fetch = [&](int p) {  // p is workgroup-uniform: no divergent guard
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      const int sl = sub + LPR * s;
      q[p][s] = *reinterpret_cast<const uint2*>(bl[p] + a.L.dn_codes + size_t(rowc) * (I / 2) + 8 * sl);
      sbw[p][s] = reinterpret_cast<const uint32_t*>(bl[p] + a.L.dn_sb)[size_t(rowc) * (I / 64) + sl / 4];
    }
    if (r > 0)
      bdraw[p] = reinterpret_cast<const uint16_t*>(bl[p] + a.L.b_dn)[size_t(rowc) * r + subr];
  };
#pragma unroll
  for (int p = 0; p < kFusedMaxP; ++p) {
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      q[p][s] = make_uint2(0, 0);
      sbw[p][s] = 0;
    }
    bdraw[p] = 0;
    bl[p] = a.shared_blob;
    if (p < P && (p % KS) >= a.K) fetch(p);
  }
  float resid[kFusedMaxT];  // residual input of this lane's row, read early
#pragma unroll
  for (int t = 0; t < kFusedMaxT; ++t)
    resid[t] = bf16_to_f32(a.h_in[size_t(min(t, a.T - 1)) * H + rowc]);
  // routed expert ids: one polling thread per pair
  if (tid < P) {
    const int t = tid / KS, k = tid % KS;
    lds_idx[tid] =
        (k < a.K) ? int(uint32_t(poll_word(a, &a.route[(c * a.T + t) * a.K + k], tag))) : -1;
  }
  __syncthreads();
  FUSED_MARK(1);
  // With many routed gate/up rows in flight (the large blocks: defer_down),
  // this role waits ~3 us before it fetches its rows and starts polling for
  // h: h cannot be complete earlier, and the fetch would only take HBM
  // bandwidth from the gate/up rows that the step is waiting for.
  if (a.defer_down) __builtin_amdgcn_s_sleep(kDownDeferSleep);
  // resident blobs are fetched at once; if any blob is the host copy, one
  // modeled latency precedes all of this thread's host reads
  uint32_t missed = 0;
#pragma unroll
  for (int p = 0; p < kFusedMaxP; ++p) {
    if (p < P && (p % KS) < a.K) {
      bool m = false;
      bl[p] = expert_blob_at(a, lds_idx[p], d == 0 && tid == 0, m);  // one count per lookup
      if (m)
        missed |= 1u << p;
      else
        fetch(p);
    }
  }
  if (missed) {
    storage_latency(a, true);
#pragma unroll
    for (int p = 0; p < kFusedMaxP; ++p)
      if ((missed >> p) & 1u) fetch(p);
  }
  // One wave waits until every h block of every pair has published its
  // exponent (each block writes it with its h words)...
  const int nblk = P * NB;
  const tword_t* hexp_c = a.hexp + size_t(c) * P * NB;
  if (wave == 0) {
    for (unsigned n = 0;; ++n) {
      tword_t cw[MAXCAN];
#pragma unroll
      for (int k = 0; k < MAXCAN; ++k) cw[k] = ld_dev(&hexp_c[min(lane + 64 * k, nblk - 1)]);
      bool ok = true;
#pragma unroll
      for (int k = 0; k < MAXCAN; ++k) ok &= (lane + 64 * k >= nblk) || has_tag(cw[k], tag);
      if (__all(ok)) break;
      if (++n > kFusedSpinLimit) {
        if (lane == 0) set_err(a);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
  FUSED_MARK(2);
  // ...then the workgroup reads h, the exponents and the routing weights,
  // repeating the reads until every word carries this launch's tag
  const tword_t* h_c = a.h + size_t(c) * P * (I / 2);
  const int nh = P * (I / 2);
  tword_t hv[MAXH], hev[MAXE];
  float wtv = 0.f;
  const int tw_t = min(tid, P - 1) / KS, tw_k = min(tid, P - 1) % KS;
  const int tw_i = (c * a.T + tw_t) * (a.K + 1) + (tw_k < a.K ? tw_k : a.K);
  for (unsigned n = 0;; ++n) {
#pragma unroll
    for (int k = 0; k < MAXH; ++k) hv[k] = ld_dev(&h_c[min(tid + 256 * k, nh - 1)]);
#pragma unroll
    for (int k = 0; k < MAXE; ++k) hev[k] = ld_dev(&hexp_c[min(tid + 256 * k, nblk - 1)]);
    const tword_t w = ld_dev(&a.wts[tw_i]);
    unsigned bad = unsigned(tid < P) & unsigned(!has_tag(w, tag));
    wtv = wf(w);
#pragma unroll
    for (int k = 0; k < MAXH; ++k) bad |= unsigned(tid + 256 * k < nh) & unsigned(!has_tag(hv[k], tag));
#pragma unroll
    for (int k = 0; k < MAXE; ++k)
      bad |= unsigned(tid + 256 * k < nblk) & unsigned(!has_tag(hev[k], tag));
    if (round_done(a, bad == 0, n)) break;
  }
  FUSED_MARK(3);
  // v of every pair (copy c): loaded now, so its latency overlaps the work
  // below; checked (and reloaded if not yet published) before its use
  const int nv = P * r;
  const tword_t* v_c = a.v + size_t(c) * P * r;
  // (without LoRA the second read below takes a logit word instead, unused)
  const tword_t* vsrc = r > 0 ? v_c + min(tid, nv - 1) : a.logits;
  tword_t vw = 0, vw2 = 0;
  if (r > 0) vw = ld_dev(vsrc);
  {
    // h words to LDS, and the sum of each 16-column block (8 consecutive
    // words, held by 8 consecutive threads) for the affine term
    uint32_t* dst = reinterpret_cast<uint32_t*>(lds_hh);
#pragma unroll
    for (int k = 0; k < MAXH; ++k) {
      const int i = tid + 256 * k;
      const uint32_t hw = uint32_t(hv[k]);
      const float ss = group_sum<8>(f16_lo(hw) + f16_hi(hw));
      if (i < nh) {
        dst[i] = hw;
        if ((i & 7) == 0) lds_hs[i >> 3] = ss;
      }
    }
  }
  if (tid < P) lds_wt[tid] = wtv;
#pragma unroll
  for (int k = 0; k < MAXE; ++k)
    if (tid + 256 * k < nblk) lds_he[tid + 256 * k] = int(uint32_t(hev[k]));
  __syncthreads();
  // this lane's part of every pair's output row; the LDS operands of pair
  // p + 1 are read before pair p is computed (reads past P are harmless)
  struct HB { uint4 h0, h1; float hs; int he; };
  HB cur[SL], nxt[SL];
  auto ldh = [&](int p, HB (&dst)[SL]) {
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      const int sl = sub + LPR * s;  // block of 16 columns
      const uint4* hp = reinterpret_cast<const uint4*>(lds_hh + p * I + 16 * sl);
      dst[s].h0 = hp[0];
      dst[s].h1 = hp[1];
      dst[s].hs = lds_hs[p * NB + sl];
      dst[s].he = lds_he[p * NB + sl];
    }
  };
  ldh(0, cur);
  float y[kFusedMaxP];
#pragma unroll
  for (int p = 0; p < kFusedMaxP; ++p) {
    y[p] = 0.f;
    if (p >= P) continue;
    if (p + 1 < kFusedMaxP) ldh(p + 1, nxt);
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      const uint32_t hw[8] = {cur[s].h0.x, cur[s].h0.y, cur[s].h0.z, cur[s].h0.w,
                              cur[s].h1.x, cur[s].h1.y, cur[s].h1.z, cur[s].h1.w};
      const uint32_t qw[2] = {q[p][s].x, q[p][s].y};
      float acc = 0.f;
#pragma unroll
      for (int dd = 0; dd < 2; ++dd)
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) acc = dot2_f16(codes_to_f16x2_biased(qw[dd], s4), hw[4 * dd + s4], acc);
      const float sc = bf16_lo(sbw[p][s]), bi = bf16_hi(sbw[p][s]);
      y[p] += ldexpf(fmaf(sc, acc, (bi - 128.0f * sc) * cur[s].hs), cur[s].he);
    }
    if (p + 1 < kFusedMaxP) {
#pragma unroll
      for (int s = 0; s < SL; ++s) cur[s] = nxt[s];
    }
    if (p == 1) {
      // a second read of v part way through the rows (the first often comes
      // back before v is published), so that a valid copy returns about when
      // the rows are done rather than one memory round trip after them
      __builtin_amdgcn_sched_barrier(0);
      vw2 = ld_dev(vsrc);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  FUSED_MARK(4);
  if (r > 0) {  // lambda B_down v
    vw = has_tag(vw, tag) ? vw : vw2;
    for (unsigned n = 0;; ++n) {
      if (round_done(a, tid >= nv || has_tag(vw, tag), n)) break;
      vw = ld_dev(vsrc);
    }
    if (tid < nv) lds_v[(tid / r) * kMaxR + tid % r] = wf(vw);
    __syncthreads();
#pragma unroll
    for (int p = 0; p < kFusedMaxP; ++p)
      if (p < P && sub < r) y[p] = fmaf(a.lam * bf16_to_f32(bdraw[p]), lds_v[p * kMaxR + sub], y[p]);
  }
  FUSED_MARK(5);
  float o[kFusedMaxT];
#pragma unroll
  for (int t = 0; t < kFusedMaxT; ++t) o[t] = 0.f;
#pragma unroll
  for (int p = 0; p < kFusedMaxP; ++p) {
    if (p >= P) continue;
    const float yp = group_sum<LPR>(y[p]);
    const int t = p / KS;
    const float wk = lds_wt[p];
#pragma unroll
    for (int tt = 0; tt < kFusedMaxT; ++tt)
      if (tt == t) o[tt] = fmaf(wk, yp, o[tt]);
  }
  if (valid && sub == 0) {
#pragma unroll
    for (int t = 0; t < kFusedMaxT; ++t) {
      if (t >= a.T) break;
      float v = o[t];
      if (a.residual) v += resid[t];
      a.out[size_t(t) * H + row] = f32_to_bf16(v);
    }
  }
}

// ---------------------------------------------------------------------------
template <int H, int I>
__global__ void __launch_bounds__(256) k_fused_decode(FusedArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_hh[kFusedMaxP * I];
  __shared__ float lds_hs[kFusedMaxP * I / kFusedJW];
  __shared__ int lds_he[kFusedMaxP * I / kFusedJW];
  __shared__ __attribute__((aligned(16))) float lds_f[kFusedMaxP * kMaxR + 64];
  __shared__ float lds_wt[kFusedMaxP];
  __shared__ int lds_i[kFusedMaxP];
  static_assert(4 * (2 * kFusedJW / 4) + 2 * kFusedJW <= kFusedMaxP * kMaxR + 64, "gate/up LDS");
  static_assert(16 * kMaxR <= kFusedMaxP * I / 2, "v reducer LDS");
  static_assert(kFusedMaxP <= 8, "one selection slot per lane of an 8-lane group");
  const int b = blockIdx.x;
  FUSED_MARK(0);
  if (b < a.nR) {
    role_router<H>(a, b);
  } else if (b < a.base_gu) {
    const int i = b - a.base_la;
    role_lora_a<H>(a, i / a.nWA, i % a.nWA, lds_i);
  } else if (b < a.base_v) {
    const int i = b - a.base_gu;
    role_gate_up<H>(a, i / a.nBG, i % a.nBG, lds_f, lds_i);
  } else if (b < a.base_dn) {
    role_vred<I>(a, b - a.base_v, reinterpret_cast<float*>(lds_hh));
  } else {
    role_down<H, I>(a, b - a.base_dn, lds_hh, lds_hs, lds_he, lds_f, lds_wt, lds_i);
  }
  // the workgroup's share of the launch counter (every read of it is done);
  // with err_out, the last workgroup out also moves the error word there
  FUSED_MARK(7);
  __syncthreads();
  if (threadIdx.x == 0) counter_arrive(launch_counter(a), 0, b, a.total);
  if (a.err_out && last_to_arrive(slot(a, kSlotDone), a.total)) {
    // every other workgroup has finished: the error word is final
    *a.err_out = ld_dev(slot(a, kSlotErr));
    st_dev(slot(a, kSlotErr), 0);
  }
}

// ---------------------------------------------------------------------------
template <int H, int I>
static hipError_t launch_fused_t(FusedArgs a, hipStream_t st) {
  constexpr int RPL_H = Geo<H>::RPL;
  const int P = a.T * (a.K + a.S);
  a.nR = (a.E + a.S + 4 * RPL_H - 1) / (4 * RPL_H);
  a.nWA = a.r > 0 ? (2 * a.r + 4 * RPL_H - 1) / (4 * RPL_H) : 0;
  a.nBG = a.I / kFusedJW;
  a.nV = a.r > 0 ? 1 : 0;
  a.nD = (H + 4 * DGeo<I>::RPL - 1) / (4 * DGeo<I>::RPL);
  a.base_la = a.nR;
  a.base_gu = a.base_la + P * a.nWA;
  a.base_v = a.base_gu + P * a.nBG;
  a.base_dn = a.base_v + P * a.nV;
  a.total = a.base_dn + a.nD;
  a.defer_down = uint64_t(a.T) * a.K * uint64_t(a.I) * a.H >= kDeferDownBytes;
  hipLaunchKernelGGL((k_fused_decode<H, I>), dim3(a.total), dim3(256), 0, st, a);
  return hipGetLastError();
}

bool fused_shape_supported(int H, int I, int r) {
  // one LoRA rank per lane of a row group: r <= H / 32 and r <= I / 32
  return (H == 256 || H == 512 || H == 1024 || H == 2048) &&
         (I == 128 || I == 256 || I == 512 || I == 1024 || I == 2048) && r <= H / 32 &&
         r <= I / 32;
}

hipError_t launch_fused(const FusedArgs& a, hipStream_t st) {
  // every workspace region the roles address must be set
  if (!a.sync || !a.logits || !a.route || !a.wts || !a.u || !a.h || !a.hexp || !a.vpart || !a.v)
    return hipErrorInvalidValue;
#define MOE_CASE_I(HV, IV) \
  case IV:                 \
    return launch_fused_t<HV, IV>(a, st);
#define MOE_CASE_H(HV)                                                                        \
  case HV:                                                                                    \
    switch (a.I) {                                                                            \
      MOE_CASE_I(HV, 128) MOE_CASE_I(HV, 256) MOE_CASE_I(HV, 512) MOE_CASE_I(HV, 1024)        \
      MOE_CASE_I(HV, 2048) default : return hipErrorInvalidValue;                             \
    }
  switch (a.H) {
    MOE_CASE_H(256) MOE_CASE_H(512) MOE_CASE_H(1024) MOE_CASE_H(2048)
    default:
      return hipErrorInvalidValue;
  }
#undef MOE_CASE_H
#undef MOE_CASE_I
}

__global__ void k_zero_ints(int* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

__global__ void k_storage_delay(uint32_t ticks) { wall_wait(ticks); }

hipError_t launch_storage_delay(uint32_t ticks, hipStream_t st) {
  hipLaunchKernelGGL(k_storage_delay, dim3(1), dim3(1), 0, st, ticks);
  return hipGetLastError();
}

hipError_t launch_zero_ints(int* p, int n, hipStream_t st) {
  hipLaunchKernelGGL(k_zero_ints, dim3(1), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace moe

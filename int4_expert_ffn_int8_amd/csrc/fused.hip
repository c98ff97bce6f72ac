// Fused decode: one launch runs a whole MoE block for a few tokens.
//
// [P2] "SSD 专家卸载 · Prerouter 路由预测", decode paragraph: route, then
// stream the chosen experts, then compute.  On MI355X a decode block moves
// ~10 MB, which HBM delivers in ~1.3 us, while each kernel boundary costs
// several microseconds; so the block is one kernel whose workgroups take
// roles and hand results to each other through device memory:
//
//   router    logits of its gate rows (x = optional RMSNorm of h_in, done
//             redundantly and identically in every workgroup); the last
//             router workgroup also waits for every logit and runs the
//             wavefront top-K, publishing ids, weights and the shared gate.
//             With given experts (prediction-as-routing, [P3] "三件套"
//             Prerouter bullet) it publishes those instead, weighted by the
//             softmax of their logits.
//   lora_a    u = [A_gate; A_up] x for one (token, slot) pair.
//   gate_up   32 gate/up outputs of one pair (+ lambda B u), SwiGLU -> h
//             (fp16), and that block's partial of v = A_down h.
//   down      a block of output rows for every pair: v = sum of the pair's
//             partials (fixed order), y = deq(Q_down) h + lambda B_down v,
//             then the weighted combine (+ residual) -> out.
//
// Weight loads are issued before the waits they do not depend on (shared
// expert from the start, routed experts as soon as their ids arrive).  An
// expert that is not resident in the pool is read from the pinned host copy,
// after an optional modeled storage latency (a bounded wall-clock wait).  A role
// waits only on roles with lower workgroup ids, which the dispatcher starts
// first, and every wait is bounded: on timeout the kernel records an error
// and still runs to completion.
//
// Hand-off protocol.  The 8 XCDs have separate L2 caches, and a device-scope
// release/acquire fence writes back / invalidates a whole L2, which at one
// fence per workgroup costs far more than the block itself.  So every value
// one workgroup hands to another is a 64-bit word -- payload in the low half,
// the launch's tag in the high half -- written and read with device-scope
// relaxed atomics (sc1 stores and loads that the XCD L2s do not hold
// incoherently).  A producer just stores; a consumer polls one word (from one
// thread, with sleeps, so waiting costs little bandwidth), then loads every
// word it needs and repeats the loads until all of them carry this launch's
// tag.  The tag is the launch epoch + 1; the last workgroup to finish bumps
// the epoch, so stale words of earlier launches never match and nothing needs
// clearing.  Weights and inputs, read-only in the kernel, use ordinary cached
// loads.
//
// Load discipline.  Vector loads complete in order, so a load whose value is
// used inside a divergent branch makes the wave wait for every load issued
// before it.  Every batch of loads here is therefore issued unconditionally
// (indices clamped to valid elements), and guards, tag checks and arithmetic
// run in a second pass.
#include "device_utils.h"
#include "fused.h"
#include "launch.h"
#include "moe_internal.h"
#include "topk.h"

namespace moe {

template <typename T>
__device__ __forceinline__ T ld_dev(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int add_dev(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int* slot(const FusedArgs& a, int s) { return a.sync + s * kSlotInts; }

// this launch's tag (epoch + 1, never 0)
__device__ __forceinline__ unsigned launch_tag(const FusedArgs& a) {
  return (unsigned(ld_dev(slot(a, kSlotEpoch))) % 0x7FFFFFFFu) + 1u;
}
__device__ __forceinline__ tword_t tw(unsigned tag, uint32_t bits) {
  return (tword_t(tag) << 32) | bits;
}
__device__ __forceinline__ tword_t twf(unsigned tag, float v) { return tw(tag, __float_as_uint(v)); }
__device__ __forceinline__ bool has_tag(tword_t w, unsigned tag) { return unsigned(w >> 32) == tag; }
__device__ __forceinline__ float wf(tword_t w) { return __uint_as_float(uint32_t(w)); }

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

// blob of routed expert e (pool lookup)
__device__ __forceinline__ const uint8_t* expert_blob(const FusedArgs& a, int e, bool count) {
  if (a.src.expert_to_slot == nullptr) return a.src.slots + size_t(e) * a.src.stride;
  const int s = a.src.expert_to_slot[e];
  if (count && a.src.counters) {
    atomicAdd(&a.src.counters[1], 1ull);
    if (s >= 0) atomicAdd(&a.src.counters[0], 1ull);
  }
  if (s >= 0) return a.src.slots + size_t(s) * a.src.stride;
  if (a.src.delay_ticks) wall_wait(a.src.delay_ticks);  // modeled storage latency
  return a.src.host_blobs + size_t(e) * a.src.stride;
}

// Expert id of routed pair p, published by the top-K (workgroup-uniform).
__device__ __forceinline__ int wait_expert(const FusedArgs& a, int p, unsigned tag, int* lds_int) {
  const int KS = a.K + a.S;
  if (threadIdx.x == 0)
    *lds_int = int(uint32_t(poll_word(a, &a.route[(p / KS) * a.K + p % KS], tag)));
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

// (s*q + b) . v over the lane's 32 columns; v is bf16 (F16 false) or fp16
template <bool F16>
__device__ __forceinline__ float slice_dot(const uint4 q, uint32_t sbw, const uint32_t* xw,
                                           float xs) {
  const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
  float acc = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      acc = F16 ? dot2_f16(codes_to_f16x2_biased(qw[d], s), xw[4 * d + s], acc)
                : dot2_bf16(codes_to_bf16x2_biased(qw[d], s), xw[4 * d + s], acc);
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
  float first = 0.f, denom = 0.f, mine = 0.f;
  int mine_e = 0;
  if (a.exec_idx == nullptr) {
    topk_wave(v, a.E, a.K, lane, [&](int k, float mx, uint32_t sel) {
      if (k == 0) first = mx;
      const float ev = expf(mx - first);
      denom += ev;
      if (k == lane) {
        mine = ev;
        mine_e = int(sel);
      }
    });
  } else {
    // given experts: lane k < K takes expert exec_idx[t][k] and fetches its
    // logit from the lane that holds it
    if (lane < a.K) {
      mine_e = a.exec_idx[t * a.K + lane];
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
    first = wave_max(lane < a.K ? gl : -INFINITY);
    mine = lane < a.K ? expf(gl - first) : 0.f;
    // summed in k order, as the selection path does: given experts equal
    // to the router's top-K reproduce its weights bit for bit
    for (int k = 0; k < a.K; ++k) denom += __shfl(mine, k);
    if (!a.norm_topk) {  // the full-softmax form below subtracts the largest logit
      float mx = -INFINITY;
#pragma unroll
      for (int m = 0; m < MP; ++m)
        if (lane + 64 * m < a.E) mx = fmaxf(mx, v[m]);
      const float top = wave_max(mx);
      mine = lane < a.K ? expf(gl - top) : 0.f;
      first = top;
    }
  }
  if (!a.norm_topk) {  // full-softmax entries: denominator over all E
    float part = 0.f;
#pragma unroll
    for (int m = 0; m < MP; ++m)
      if (lane + 64 * m < a.E) part += expf(v[m] - first);
    denom = group_sum<64>(part);
  }
  if (lane < a.K) {
    const float wv = mine / denom;
    st_dev(&a.route[t * a.K + lane], tw(tag, uint32_t(mine_e)));
    st_dev(&a.wts[t * (a.K + 1) + lane], twf(tag, wv));
    if (a.user_idx) a.user_idx[t * a.K + lane] = mine_e;
    if (a.user_w) a.user_w[t * a.K + lane] = wv;
  }
  if (a.S && lane == 0) st_dev(&a.wts[t * (a.K + 1) + a.K], twf(tag, sigmoid_f(sgl)));
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
  const int t = p / KS;
  const bool routed = (p % KS) < a.K;
  const unsigned tag = launch_tag(a);
  uint32_t xw[16];
  float xs;
  token_slice<H>(a, t, sub, xw, xs);
  const uint8_t* blob = a.shared_blob;
  if (routed) blob = expert_blob(a, wait_expert(a, p, tag, lds_int), false);
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
  acc = group_sum<G::LPR>(acc);
  if (rw < rows && sub == 0) st_dev(&a.u[p * rows + rw], twf(tag, acc));
}

// ---------------------------------------------------------------------------
template <int H>
__device__ void role_gate_up(const FusedArgs& a, int unit, int blk, float* lds, int* lds_int) {
  using G = Geo<H>;
  constexpr int RPL = G::RPL;
  constexpr int JW = kFusedJW, JPW = JW / 4;  // outputs per workgroup / wave
  constexpr int NR = 2 * JPW, NL = NR / RPL;  // gate + up rows per wave, loads per lane
  static_assert(NR % RPL == 0, "rows per wave");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, sub = lane % G::LPR;
  const int tid = threadIdx.x;
  const int p = pair_of_unit(a, unit);
  const int KS = a.K + a.S;
  const int t = p / KS;
  const bool routed = (p % KS) < a.K;
  const int j0 = blk * JW + wave * JPW;
  const int r = a.r;
  const unsigned tag = launch_tag(a);
  const uint8_t* blob = a.shared_blob;
  if (routed) blob = expert_blob(a, wait_expert(a, p, tag, lds_int), false);
  // every weight this workgroup needs, before anything waits on data
  const uint8_t* codes = blob + a.L.gu_codes;
  const uint32_t* sb = reinterpret_cast<const uint32_t*>(blob + a.L.gu_sb);
  const uint16_t* Bgu = reinterpret_cast<const uint16_t*>(blob + a.L.b_gu);
  const uint16_t* Ad = reinterpret_cast<const uint16_t*>(blob + a.L.a_dn);
  uint4 q[NL];
  uint32_t sbw[NL];
  int brow[NL];
  uint16_t braw[NL];  // B[row][sub] (one LoRA rank per lane; r <= LPR)
  uint16_t adraw[2];  // A_down entries of this block's partial of v
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
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int id = c * 256 + tid, rr = min(id / JW, rc), jj = id % JW;
      adraw[c] = Ad[size_t(rr) * a.I + blk * JW + jj];
    }
  }
  uint32_t xw[16];
  float xs;
  token_slice<H>(a, t, sub, xw, xs);
  float part[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) part[i] = slice_dot<false>(q[i], sbw[i], xw, xs);
  float* lds_a = lds;           // [4][NR]
  float* lds_h = lds + 4 * NR;  // [JW]
  if (r > 0) {  // u = A x of this pair (from its lora_a workgroups)
    float uv[2] = {0.f, 0.f};  // lane's rank `sub` of A_gate x and A_up x
    for (unsigned n = 0;; ++n) {
      const tword_t g = ld_dev(&a.u[p * 2 * r + min(sub, rc)]);
      const tword_t uu = ld_dev(&a.u[p * 2 * r + r + min(sub, rc)]);
      const bool ok = has_tag(g, tag) && has_tag(uu, tag);
      uv[0] = wf(g);
      uv[1] = wf(uu);
      if (round_done(a, ok, n)) break;
    }
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
  if (sub == 0) {
#pragma unroll
    for (int i = 0; i < NL; ++i) lds_a[wave * NR + i * RPL + lane / G::LPR] = part[i];
  }
  __syncthreads();
  float* lds_hraw = lds_h + JW;  // [JW]
  if (tid < JW) {
    const int w = tid / JPW, jl = tid % JPW;
    lds_hraw[tid] = silu_f(lds_a[w * NR + 2 * jl]) * lds_a[w * NR + 2 * jl + 1];
  }
  __syncthreads();
  // this block of h is one 32-column slice of the down rows: it is stored as
  // fp16(h * 2^-e) with one exponent e per block (e = 0 unless |h| >= 2^15)
  float hmax = 0.f;
  for (int j = 0; j < JW; ++j) hmax = fmaxf(hmax, fabsf(lds_hraw[j]));
  const int hexp = h_block_exp(hmax);
  if (tid < JW) lds_h[tid] = ldexpf(f16_to_f32(f32_to_f16_sat(ldexpf(lds_hraw[tid], -hexp))), hexp);
  __syncthreads();
  if (tid < JW / 2) {  // fp16 pairs of h * 2^-e, one tagged word per pair
    f16x2_t pr = {_Float16(ldexpf(lds_h[2 * tid], -hexp)), _Float16(ldexpf(lds_h[2 * tid + 1], -hexp))};
    st_dev(&a.h[p * (a.I / 2) + blk * (JW / 2) + tid], tw(tag, __builtin_bit_cast(uint32_t, pr)));
  } else if (tid == JW / 2) {
    st_dev(&a.hexp[p * (a.I / JW) + blk], tw(tag, uint32_t(hexp)));
  }
  if (r > 0) {  // this block's partial of v = A_down h
    const int NB = a.I / JW;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int id = c * 256 + tid, rr = id / JW, jj = id % JW;
      const float ad = (rr < r) ? bf16_to_f32(adraw[c]) : 0.f;
      const float prod = group_sum<JW>(ad * lds_h[jj]);
      if (jj == 0 && rr < r) st_dev(&a.vpart[(p * NB + blk) * r + rr], twf(tag, prod));
    }
  }
}

// ---------------------------------------------------------------------------
template <int H, int I>
__device__ void role_down(const FusedArgs& a, int d, uint16_t* lds_hh, float* lds_hs, int* lds_he,
                          float* lds_v,
                          float* lds_wt, int* lds_idx) {
  using G = Geo<I>;
  constexpr int RPL = G::RPL;
  constexpr int NB = I / kFusedJW;  // partials of A_down h per pair
  constexpr int MAXH = (kFusedMaxP * I / 2 + 255) / 256;
  constexpr int MAXC = (kFusedMaxP * kMaxR * 16 + 255) / 256;
  constexpr int MAXE = (kFusedMaxP * I / 32 + 255) / 256;
  static_assert(kFusedJW == 32, "one h exponent per 32-column slice of a down row");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, sub = lane % G::LPR;
  const int tid = threadIdx.x;
  const int row = d * 4 * RPL + wave * RPL + lane / G::LPR;
  const bool valid = row < H;
  const int KS = a.K + a.S;
  const int P = a.T * KS;
  const int r = a.r;
  const unsigned tag = launch_tag(a);
  // Prefetch this lane's down-row slice of every pair into registers: the
  // shared expert at once, routed experts as soon as their ids arrive.
  uint4 q[kFusedMaxP];
  uint32_t sbw[kFusedMaxP];
  uint16_t bdraw[kFusedMaxP];  // B_down[row][sub]
  const uint8_t* bl[kFusedMaxP];
  const int rowc = min(row, H - 1), subr = min(sub, max(r - 1, 0));
  auto fetch = [&](int p) {  // p is workgroup-uniform: no divergent guard
    q[p] = *reinterpret_cast<const uint4*>(bl[p] + a.L.dn_codes + size_t(rowc) * (I / 2) + 16 * sub);
    sbw[p] = reinterpret_cast<const uint32_t*>(bl[p] + a.L.dn_sb)[size_t(rowc) * (I / 64) + (sub >> 1)];
    if (r > 0)
      bdraw[p] = reinterpret_cast<const uint16_t*>(bl[p] + a.L.b_dn)[size_t(rowc) * r + subr];
  };
#pragma unroll
  for (int p = 0; p < kFusedMaxP; ++p) {
    q[p] = make_uint4(0, 0, 0, 0);
    sbw[p] = 0;
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
    lds_idx[tid] = (k < a.K) ? int(uint32_t(poll_word(a, &a.route[t * a.K + k], tag))) : -1;
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < kFusedMaxP; ++p) {
    if (p < P && (p % KS) < a.K) {
      bl[p] = expert_blob(a, lds_idx[p], d == 0 && tid == 0);  // one count per lookup
      fetch(p);
    }
  }
  // wait for the last h word, then load every pair's h, v partials and
  // routing weights until all carry this launch's tag
  if (tid == 0) poll_word(a, &a.h[P * (I / 2) - 1], tag);
  __syncthreads();
  tword_t hv[MAXH], vp[MAXC];
  float wtv = 0.f;
  const int nh = P * (I / 2);
  const int ne = P * (I / 32);
  tword_t hev[MAXE];
  const int tw_t = min(tid, P - 1) / KS, tw_k = min(tid, P - 1) % KS;
  const int tw_i = tw_t * (a.K + 1) + (tw_k < a.K ? tw_k : a.K);
  // partial of v read by slot c of this thread: (pair, rank, block < 16);
  // without LoRA every slot reads a valid dummy word and is not checked
  const tword_t* vsrc = (r > 0) ? a.vpart : a.wts;
  int vidx[MAXC];
  uint32_t vneed = 0;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int id = c * 256 + tid;
    const int pr = id >> 4, q16 = id & 15;
    const int p = (r > 0) ? pr / r : P, rr = (r > 0) ? pr % r : 0;
    const bool need = p < P && q16 < NB;  // NB <= 16 here; larger NB is summed below
    vidx[c] = need ? (p * NB + q16) * r + rr : 0;
    vneed |= uint32_t(need) << c;
  }
  for (unsigned n = 0;; ++n) {
    // every load of the round first (fixed count, clamped indices), then the checks
#pragma unroll
    for (int k = 0; k < MAXH; ++k) hv[k] = ld_dev(&a.h[min(tid + 256 * k, nh - 1)]);
#pragma unroll
    for (int k = 0; k < MAXE; ++k) hev[k] = ld_dev(&a.hexp[min(tid + 256 * k, ne - 1)]);
#pragma unroll
    for (int c = 0; c < MAXC; ++c) vp[c] = ld_dev(&vsrc[vidx[c]]);
    const tword_t w = ld_dev(&a.wts[tw_i]);
    unsigned bad = unsigned(tid < P) & unsigned(!has_tag(w, tag));
    wtv = wf(w);
#pragma unroll
    for (int k = 0; k < MAXH; ++k) bad |= unsigned(tid + 256 * k < nh) & unsigned(!has_tag(hv[k], tag));
#pragma unroll
    for (int k = 0; k < MAXE; ++k) bad |= unsigned(tid + 256 * k < ne) & unsigned(!has_tag(hev[k], tag));
#pragma unroll
    for (int c = 0; c < MAXC; ++c) bad |= ((vneed >> c) & 1u) & unsigned(!has_tag(vp[c], tag));
    if (round_done(a, bad == 0, n)) break;
  }
  // partial blocks beyond the first 16 (I > 512): summed after the round
  float vs[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int id = c * 256 + tid;
    const int pr = id >> 4, q16 = id & 15;
    const int p = (r > 0) ? pr / r : P, rr = (r > 0) ? pr % r : 0;
    float s = ((vneed >> c) & 1u) ? wf(vp[c]) : 0.f;
    if (p < P)
      for (int bb = q16 + 16; bb < NB; bb += 16) {
        const tword_t w = poll_word(a, &a.vpart[(p * NB + bb) * r + rr], tag);
        s += wf(w);
      }
    vs[c] = s;
  }
  {
    // h words to LDS, and the sum of each 32-column slice (16 consecutive
    // words, held by 16 consecutive threads) for the affine term
    uint32_t* dst = reinterpret_cast<uint32_t*>(lds_hh);
#pragma unroll
    for (int k = 0; k < MAXH; ++k) {
      const int i = tid + 256 * k;
      const uint32_t hw = uint32_t(hv[k]);
      const float ss = group_sum<16>(f16_lo(hw) + f16_hi(hw));
      if (i < nh) {
        dst[i] = hw;
        if ((i & 15) == 0) lds_hs[i >> 4] = ss;
      }
    }
  }
  if (r > 0) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int id = c * 256 + tid;
      const int pr = id >> 4, q16 = id & 15;
      const int p = pr / r, rr = pr % r;
      const float s = group_sum<16>(vs[c]);
      if (q16 == 0 && p < P) lds_v[p * kMaxR + rr] = s;
    }
  }
  if (tid < P) lds_wt[tid] = wtv;
#pragma unroll
  for (int k = 0; k < MAXE; ++k)
    if (tid + 256 * k < ne) lds_he[tid + 256 * k] = int(uint32_t(hev[k]));
  __syncthreads();
  float o[kFusedMaxT];
#pragma unroll
  for (int t = 0; t < kFusedMaxT; ++t) o[t] = 0.f;
#pragma unroll
  for (int p = 0; p < kFusedMaxP; ++p) {
    if (p >= P) continue;
    uint32_t hw[16];
    const uint4* hp = reinterpret_cast<const uint4*>(lds_hh + p * I + 32 * sub);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint4 v = hp[k];
      hw[4 * k] = v.x; hw[4 * k + 1] = v.y; hw[4 * k + 2] = v.z; hw[4 * k + 3] = v.w;
    }
    float y = slice_dot<true>(q[p], sbw[p], hw, lds_hs[p * (I / 32) + sub]);
    y = ldexpf(y, lds_he[p * (I / 32) + sub]);
    if (sub < r) y = fmaf(a.lam * bf16_to_f32(bdraw[p]), lds_v[p * kMaxR + sub], y);
    y = group_sum<G::LPR>(y);
    const int t = p / KS;
    const float wk = lds_wt[p];
#pragma unroll
    for (int tt = 0; tt < kFusedMaxT; ++tt)
      if (tt == t) o[tt] = fmaf(wk, y, o[tt]);
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
  __shared__ float lds_hs[kFusedMaxP * I / 32];
  __shared__ int lds_he[kFusedMaxP * I / 32];
  __shared__ __attribute__((aligned(16))) float lds_f[kFusedMaxP * kMaxR + 160];
  __shared__ float lds_wt[kFusedMaxP];
  __shared__ int lds_i[kFusedMaxP];
  const int b = blockIdx.x;
  if (b < a.nR) {
    role_router<H>(a, b);
  } else if (b < a.base_gu) {
    const int i = b - a.base_la;
    role_lora_a<H>(a, i / a.nWA, i % a.nWA, lds_i);
  } else if (b < a.base_dn) {
    const int i = b - a.base_gu;
    role_gate_up<H>(a, i / a.nBG, i % a.nBG, lds_f, lds_i);
  } else {
    role_down<H, I>(a, b - a.base_dn, lds_hh, lds_hs, lds_he, lds_f, lds_wt, lds_i);
  }
  // the last workgroup out starts the next epoch
  __syncthreads();
  if (threadIdx.x == 0 && add_dev(slot(a, kSlotDone), 1) == a.total - 1) {
    const int e = ld_dev(slot(a, kSlotEpoch));
    st_dev(slot(a, kSlotDone), 0);
    st_dev(slot(a, kSlotEpoch), e + 1);
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
  a.nD = (H + 4 * Geo<I>::RPL - 1) / (4 * Geo<I>::RPL);
  a.base_la = a.nR;
  a.base_gu = a.base_la + P * a.nWA;
  a.base_dn = a.base_gu + P * a.nBG;
  a.total = a.base_dn + a.nD;
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

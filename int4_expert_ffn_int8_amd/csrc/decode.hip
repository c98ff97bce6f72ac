// Decode expert path: weight-streaming GEMV over the selected experts.
//
// [P1] "Edge0开源框架实现35BMoE模型在Mac上流式推理…", Recover-LoRA and
// Prerouter paragraphs: the int4 base is frozen and an unmerged LoRA delta is
// added at inference.  [P3] "iPhone、Mac、Android、Windows 实测横评…",
// "三件套" bullets: affine 4-bit codes with group_size 64.  [P2] "SSD 专家卸载
// · Prerouter 路由预测", prefill/decode paragraph: decode streams each
// selected expert once per token.
//
// Per (token, slot) pair p -- slot k < K is the k-th routed expert, slot K
// the shared expert -- three kernels run:
//   k_lora_a_decode   resolve the expert's blob through the pool table, and
//                     u = [A_gate; A_up] x  (2r dot products over H, a few
//                     rows per workgroup)
//   k_gateup_decode   a_g, a_u rows (+ lambda B u), h = silu(a_g) * a_u (fp16),
//                     and per-workgroup partials of v = A_down h
//   k_down_decode     y = deq(Q_down) h + lambda B_down v
// Each lane owns 32 consecutive input columns: one 16-byte load of int4 codes
// per row, turned in registers into exact (128 + code) pairs -- bf16 against
// the bf16 token x, fp16 against the fp16 hidden h -- and reduced with
// v_dot2c_f32_{bf16,f16}; the +128 offset and the affine map are applied per
// half-group in fp32 with the lane's sum of the input.  h is kept in fp16
// (11-bit significand): with bf16 the down projection's partial cancellation
// turns the rounding of h into errors near 1% of the output's RMS.  No
// floating-point atomics: every sum has a fixed order.
#include "device_utils.h"
#include "launch.h"
#include "moe_internal.h"

namespace moe {


template <int H>
struct GateUpGeo {
  static constexpr int RPL = Geo<H>::RPL;
  static constexpr int JPW = (RPL / 2) > 2 ? (RPL / 2) : 2;  // outputs j per wave
  static constexpr int NR = 2 * JPW;                          // gate + up rows per wave
  static constexpr int NL = NR / RPL;                         // row loads per lane
  static constexpr int JW = 4 * JPW;                          // outputs j per workgroup
};

template <int I>
struct DownGeo {
  static constexpr int RPL = Geo<I>::RPL;
  static constexpr int NR = RPL > 8 ? RPL : 8;  // rows per wave
  static constexpr int NL = NR / RPL;
  static constexpr int RW = 4 * NR;             // rows per workgroup
};

__device__ __forceinline__ const uint8_t* resolve_blob(const DecodeArgs& a, int p, bool count) {
  const int KS = a.K + a.S;
  const int t = p / KS, k = p % KS;
  if (k >= a.K) return a.shared_blob;
  // a caller-supplied id outside [0, E) is clamped: never an address past the experts
  const int e = min(max(a.topk_idx[size_t(t) * a.K + k], 0), a.E - 1);
  if (a.src.expert_to_slot == nullptr) return a.src.slots + size_t(e) * a.src.stride;
  const int slot = a.src.expert_to_slot[e];
  if (count && a.src.counters) {
    atomicAdd(&a.src.counters[1], 1ull);
    if (slot >= 0) atomicAdd(&a.src.counters[0], 1ull);
  }
  return slot >= 0 ? a.src.slots + size_t(slot) * a.src.stride
                   : a.src.host_blobs + size_t(e) * a.src.stride;
}

// Load the lane's 32-column slices of a bf16 (or fp16) vector as 16 pairs
// each, plus their sums.
template <int IN, bool F16 = false>
__device__ __forceinline__ void load_vec_slices(const uint16_t* v, int sub,
                                                uint32_t (&xw)[Geo<IN>::SL][16],
                                                float (&xs)[Geo<IN>::SL]) {
#pragma unroll
  for (int c = 0; c < Geo<IN>::SL; ++c) {
    const uint4* xp = reinterpret_cast<const uint4*>(v + 32 * sub + 2048 * c);
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint4 q = xp[k];
      xw[c][4 * k] = q.x; xw[c][4 * k + 1] = q.y; xw[c][4 * k + 2] = q.z; xw[c][4 * k + 3] = q.w;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k)
      sum += F16 ? f16_lo(xw[c][k]) + f16_hi(xw[c][k]) : bf16_lo(xw[c][k]) + bf16_hi(xw[c][k]);
    xs[c] = sum;
  }
}

// sum over the lane's 32 columns of (s*q + b) * x for one row slice; x holds
// bf16 pairs (F16 = false) or fp16 pairs (F16 = true)
template <bool F16 = false>
__device__ __forceinline__ float int4_slice_dot(const uint4 q, uint32_t sbw, const uint32_t* xw,
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
// u = [A_gate; A_up] x, RPL rows per wave and 4 RPL rows per workgroup;
// workgroup (p, 0) also records the pair's blob (and counts the pool lookup).
// grid (NP, lora_a_blocks), block 256.
template <int H>
constexpr int lora_a_rows_per_block() { return 4 * Geo<H>::RPL; }

template <int H>
__global__ void __launch_bounds__(256) k_lora_a_decode(DecodeArgs a) {
  using G = Geo<H>;
  const int p = blockIdx.x;
  const uint8_t* blob = resolve_blob(a, p, blockIdx.y == 0);
  if (blockIdx.y == 0 && threadIdx.x == 0)
    a.blobptr[p] = reinterpret_cast<unsigned long long>(blob);
  if (a.r == 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, sub = lane % G::LPR;
  const int t = p / (a.K + a.S);
  const int rows = 2 * a.r;
  const int row = (blockIdx.y * 4 + wave) * G::RPL + lane / G::LPR;
  const uint16_t* A = reinterpret_cast<const uint16_t*>(blob + a.L.a_gu);
  // the row's loads first (clamped to a valid row), then the token
  const int rc = min(row, rows - 1);
  uint4 q[G::SL][4];
#pragma unroll
  for (int c = 0; c < G::SL; ++c)
#pragma unroll
    for (int k = 0; k < 4; ++k)
      q[c][k] = reinterpret_cast<const uint4*>(A + size_t(rc) * H + 32 * sub + 2048 * c)[k];
  uint32_t xw[G::SL][16];
  float xs[G::SL];
  load_vec_slices<H>(a.x + size_t(t) * H, sub, xw, xs);
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < G::SL; ++c)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc = dot2_bf16(q[c][k].x, xw[c][4 * k], acc);
      acc = dot2_bf16(q[c][k].y, xw[c][4 * k + 1], acc);
      acc = dot2_bf16(q[c][k].z, xw[c][4 * k + 2], acc);
      acc = dot2_bf16(q[c][k].w, xw[c][4 * k + 3], acc);
    }
  acc = group_sum<G::LPR>(acc);
  if (row < rows && sub == 0) a.u[size_t(p) * rows + row] = acc;
}

// ---------------------------------------------------------------------------
// gate/up rows, SwiGLU, h (fp16) and partials of A_down h.
// grid (NP, I / JW), block 256.
template <int H>
__global__ void __launch_bounds__(256) k_gateup_decode(DecodeArgs a) {
  using G = Geo<H>;
  using U = GateUpGeo<H>;
  __shared__ float lds_a[4][U::NR];
  __shared__ float lds_h[U::JW];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, sub = lane % G::LPR;
  const int p = blockIdx.x, blk = blockIdx.y;
  const int t = p / (a.K + a.S);
  const int j0 = blk * U::JW + wave * U::JPW;
  const uint8_t* blob = reinterpret_cast<const uint8_t*>(a.blobptr[p]);
  const uint8_t* codes = blob + a.L.gu_codes;
  const uint32_t* sb = reinterpret_cast<const uint32_t*>(blob + a.L.gu_sb);

  // issue every weight load of this lane first
  uint4 q[U::NL][G::SL];
  uint32_t sbw[U::NL][G::SL];
  int brow[U::NL];
#pragma unroll
  for (int i = 0; i < U::NL; ++i) {
    const int ri = i * G::RPL + lane / G::LPR;
    const int j = j0 + (ri >> 1);
    brow[i] = (ri & 1) ? gu_row_up(j) : gu_row_gate(j);
#pragma unroll
    for (int c = 0; c < G::SL; ++c) {
      const int col0 = 32 * sub + 2048 * c;
      q[i][c] = *reinterpret_cast<const uint4*>(codes + size_t(brow[i]) * (H / 2) + col0 / 2);
      sbw[i][c] = sb[size_t(brow[i]) * (H / 64) + col0 / 64];
    }
  }
  uint32_t xw[G::SL][16];
  float xs[G::SL];
  load_vec_slices<H>(a.x + size_t(t) * H, sub, xw, xs);

  const int r = a.r;
  const uint16_t* Bgu = reinterpret_cast<const uint16_t*>(blob + a.L.b_gu);
  const float* u = a.u + size_t(p) * 2 * r;
#pragma unroll
  for (int i = 0; i < U::NL; ++i) {
    const int ri = i * G::RPL + lane / G::LPR;
    float part = 0.f;
#pragma unroll
    for (int c = 0; c < G::SL; ++c) part += int4_slice_dot(q[i][c], sbw[i][c], xw[c], xs[c]);
    const float* uu = u + ((ri & 1) ? r : 0);
    for (int rr = sub; rr < r; rr += G::LPR)
      part = fmaf(a.lam * bf16_to_f32(Bgu[size_t(brow[i]) * r + rr]), uu[rr], part);
    part = group_sum<G::LPR>(part);
    if (sub == 0) lds_a[wave][ri] = part;
  }
  __syncthreads();
  const int tid = threadIdx.x;
  if (tid < U::JW) {
    const int w = tid / U::JPW, jl = tid % U::JPW;
    const float hv = silu_f(lds_a[w][2 * jl]) * lds_a[w][2 * jl + 1];
    a.h[size_t(p) * a.I + blk * U::JW + tid] = hv;
    lds_h[tid] = hv;
  }
  __syncthreads();
  if (r == 0) return;
  const uint16_t* Ad = reinterpret_cast<const uint16_t*>(blob + a.L.a_dn);
  const int NB = a.I / U::JW;
  for (int base = 0; base < r * U::JW; base += 256) {
    const int id = base + tid;
    const int rr = id / U::JW, jj = id % U::JW;
    float prod = 0.f;
    if (rr < r) prod = bf16_to_f32(Ad[size_t(rr) * a.I + blk * U::JW + jj]) * lds_h[jj];
    prod = group_sum<U::JW>(prod);
    if (jj == 0 && rr < r) a.vpart[(size_t(p) * NB + blk) * r + rr] = prod;
  }
}

// ---------------------------------------------------------------------------
// y = deq(Q_down) h + lambda B_down v.  grid (NP, ceil(H / RW)), block 256.
template <int I>
__global__ void __launch_bounds__(256) k_down_decode(DecodeArgs a, int NB) {
  using G = Geo<I>;
  using D = DownGeo<I>;
  __shared__ float vs[kMaxR];
  __shared__ float vg[16][kMaxR];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, sub = lane % G::LPR;
  const int p = blockIdx.x;
  const int H = a.H, r = a.r;
  const int row0 = blockIdx.y * D::RW + wave * D::NR;
  const uint8_t* blob = reinterpret_cast<const uint8_t*>(a.blobptr[p]);
  const uint8_t* codes = blob + a.L.dn_codes;
  const uint32_t* sb = reinterpret_cast<const uint32_t*>(blob + a.L.dn_sb);
  uint4 q[D::NL][G::SL];
  uint32_t sbw[D::NL][G::SL];
#pragma unroll
  for (int i = 0; i < D::NL; ++i) {
    const int row = row0 + i * G::RPL + lane / G::LPR;
#pragma unroll
    for (int c = 0; c < G::SL; ++c) {
      const int col0 = 32 * sub + 2048 * c;
      if (row < H) {
        q[i][c] = *reinterpret_cast<const uint4*>(codes + size_t(row) * (I / 2) + col0 / 2);
        sbw[i][c] = sb[size_t(row) * (I / 64) + col0 / 64];
      } else {
        q[i][c] = make_uint4(0, 0, 0, 0);
        sbw[i][c] = 0;
      }
    }
  }
  // v = sum of the NB <= I / 8 partials: thread (rank tid % 16, group tid / 16)
  // adds blocks group, group + 16, ... (all its loads issued at once), and the
  // 16 group sums of a rank are added in group order below.
  constexpr int NBG = (I / 8 + 15) / 16;
  static_assert(kMaxR == 16, "one rank per lane of a 16-lane group");
  if (r > 0) {
    const int rr = threadIdx.x & 15, bg = threadIdx.x >> 4;
    const float* vp = a.vpart + size_t(p) * NB * r + min(rr, r - 1);
    float w[NBG];
#pragma unroll
    for (int k = 0; k < NBG; ++k) w[k] = vp[size_t(min(bg + 16 * k, NB - 1)) * r];
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < NBG; ++k)
      if (bg + 16 * k < NB) s += w[k];
    vg[bg][rr] = s;
  }
  // h slices as fp16(h * 2^-e), one exponent per 32-column slice
  uint32_t xw[G::SL][16];
  float xs[G::SL];
  int xe[G::SL];
#pragma unroll
  for (int c = 0; c < G::SL; ++c) {
    const float4* hp = reinterpret_cast<const float4*>(a.h + size_t(p) * I + 32 * sub + 2048 * c);
    float hv[32];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float4 v = hp[k];
      hv[4 * k] = v.x; hv[4 * k + 1] = v.y; hv[4 * k + 2] = v.z; hv[4 * k + 3] = v.w;
    }
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < 32; ++k) m = fmaxf(m, fabsf(hv[k]));
    xe[c] = h_block_exp(m);
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      f16x2_t pr = {_Float16(ldexpf(hv[2 * k], -xe[c])), _Float16(ldexpf(hv[2 * k + 1], -xe[c]))};
      xw[c][k] = __builtin_bit_cast(uint32_t, pr);
      sum += float(pr[0]) + float(pr[1]);
    }
    xs[c] = sum;
  }
  __syncthreads();
  if (threadIdx.x < r) {
    float v = 0.f;
#pragma unroll
    for (int g = 0; g < 16; ++g) v += vg[g][threadIdx.x];
    vs[threadIdx.x] = v;
  }
  __syncthreads();
  const uint16_t* Bd = reinterpret_cast<const uint16_t*>(blob + a.L.b_dn);
#pragma unroll
  for (int i = 0; i < D::NL; ++i) {
    const int row = row0 + i * G::RPL + lane / G::LPR;
    float part = 0.f;
#pragma unroll
    for (int c = 0; c < G::SL; ++c)
      part += ldexpf(int4_slice_dot<true>(q[i][c], sbw[i][c], xw[c], xs[c]), xe[c]);
    if (row < H)
      for (int rr = sub; rr < r; rr += G::LPR)
        part = fmaf(a.lam * bf16_to_f32(Bd[size_t(row) * r + rr]), vs[rr], part);
    part = group_sum<G::LPR>(part);
    if (sub == 0 && row < H) a.y[size_t(p) * H + row] = part;
  }
}

// ---------------------------------------------------------------------------
template <int H>
static int jw_of() { return GateUpGeo<H>::JW; }

int decode_gateup_block_j(int H) {
#define MOE_CASE(V) \
  case V:           \
    return jw_of<V>();
  switch (H) {
    MOE_FOR_EACH_WIDTH(MOE_CASE)
    default:
      return 0;
  }
#undef MOE_CASE
}

template <int H>
static hipError_t launch_front(const DecodeArgs& a, int NP, hipStream_t st) {
  const int ra = lora_a_rows_per_block<H>();
  const int ny = a.r > 0 ? (2 * a.r + ra - 1) / ra : 1;
  hipLaunchKernelGGL(k_lora_a_decode<H>, dim3(NP, ny), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_gateup_decode<H>, dim3(NP, a.I / GateUpGeo<H>::JW), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int I>
static hipError_t launch_back(const DecodeArgs& a, int NP, int NB, hipStream_t st) {
  const int rw = DownGeo<I>::RW;
  hipLaunchKernelGGL(k_down_decode<I>, dim3(NP, (a.H + rw - 1) / rw), dim3(256), 0, st, a, NB);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  const int NP = a.T * (a.K + a.S);
  if (NP == 0) return hipSuccess;
  hipError_t e = hipErrorInvalidValue;
#define MOE_CASE(V)                    \
  case V:                              \
    e = launch_front<V>(a, NP, st);    \
    break;
  switch (a.H) {
    MOE_FOR_EACH_WIDTH(MOE_CASE)
    default:
      return hipErrorInvalidValue;
  }
#undef MOE_CASE
  if (e != hipSuccess) return e;
  const int NB = a.I / decode_gateup_block_j(a.H);
  if (NB < 1 || 8 * NB > a.I) return hipErrorInvalidValue;  // k_down_decode sums <= I / 8 partials
#define MOE_CASE(V)                      \
  case V:                                \
    return launch_back<V>(a, NP, NB, st);
  switch (a.I) {
    MOE_FOR_EACH_WIDTH(MOE_CASE)
    default:
      return hipErrorInvalidValue;
  }
#undef MOE_CASE
}

}  // namespace moe

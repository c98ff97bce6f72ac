// Prefill path: group (token, k) pairs by expert, then grouped MFMA GEMMs.
//
// [P2] "SSD 专家卸载 · Prerouter 路由预测", prefill/decode paragraph: prefill
// loads whole layers and computes in batches, decode relies on caching and
// prefetch.  Here prefill groups each expert's tokens and runs one dense
// contraction per expert: int4 codes are dequantised to bf16 in LDS (affine,
// group 64: [P3] "iPhone、Mac、Android、Windows 实测横评…", "三件套" bullets)
// and fed to v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  The unmerged
// LoRA delta ([P1] Recover-LoRA paragraph) is one extra 64-wide K chunk: the
// activation side holds lambda * (A v) as a hi + lo pair (computed by a skinny
// GEMM first), the weight side holds B twice.
//
// Codes enter the MFMA exactly, as the values 128 + q; the affine map of each
// 64-column group is applied in fp32 after the MFMA: acc += s * P + (b - 128 s)
// * (row sum of the activations over the group).  Gate/up run in bf16 (x is
// bf16); the SwiGLU output h is stored in fp16 and the down side (LoRA-A of
// down, down projection) runs fp16 MFMA: rounding h to bf16 would cost up to
// 1% of the output's RMS through the down projection's cancellation.
//
// Row space of the expert GEMMs ("sorted rows"): s in [0, T*K) are the routed
// pairs in perm order (expert by expert, ascending pair id), s in [T*K,
// T*K + T) are the tokens of the shared expert.  Group g < E is routed expert
// g, group E the shared expert.
#include "device_utils.h"
#include "launch.h"
#include "moe_internal.h"
#include "prefill.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ===========================================================================
// grouping
// ===========================================================================

// Lanes of this wave whose key equals the calling lane's key (bit-sliced
// ballots; `nbits` covers the key range).
__device__ __forceinline__ unsigned long long same_key_mask(int key, int nbits, bool valid) {
  unsigned long long m = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1;
    const unsigned long long bm = __ballot(valid && bit);
    m &= bit ? bm : ~bm;
  }
  return m;
}

// Per chunk of kGroupChunk pairs: histogram of experts.  grid nch, block 1024.
__global__ void __launch_bounds__(1024) k_group_hist(const int32_t* __restrict__ idx, int TK, int E,
                                                      int32_t* __restrict__ chunk_hist) {
  __shared__ int h[kMaxE];
  const int tid = threadIdx.x, c = blockIdx.x;
  for (int e = tid; e < E; e += 1024) h[e] = 0;
  __syncthreads();
  const int p = c * kGroupChunk + tid;
  if (p < TK) atomicAdd(&h[idx[p]], 1);
  __syncthreads();
  for (int e = tid; e < E; e += 1024) chunk_hist[size_t(c) * E + e] = h[e];
}

// Block-wide exclusive scan of one int per thread (1024 threads); returns the
// exclusive prefix, `total` receives the sum.
__device__ __forceinline__ int block_exclusive_scan_1024(int v, int* lds16, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  __syncthreads();
  if (lane == 63) lds16[wave] = inc;
  __syncthreads();
  int wbase = 0, tot = 0;
  for (int w = 0; w < 16; ++w) {
    const int c = lds16[w];
    if (w < wave) wbase += c;
    tot += c;
  }
  total = tot;
  return wbase + inc - v;
}

// One workgroup: per-expert counts, exclusive offsets and per-chunk bases.
__global__ void __launch_bounds__(1024) k_group_scan(const int32_t* __restrict__ chunk_hist,
                                                      int nch, int E, int TK,
                                                      int32_t* __restrict__ counts,
                                                      int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ base) {
  __shared__ int lds16[16];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int c = 0; c < nch; ++c) {
      const int v = chunk_hist[size_t(c) * E + e];
      base[size_t(c) * E + e] = run;
      run += v;
    }
  }
  int total;
  const int off = block_exclusive_scan_1024(e < E ? run : 0, lds16, total);
  if (e < E) {
    counts[e] = run;
    offsets[e] = off;
  }
  if (e == 0) offsets[E] = TK;
}

// Stable scatter: pair p goes to offsets[e] + (earlier pairs of expert e).
// grid nch, block 1024, dynamic LDS 16 * E ints.
__global__ void __launch_bounds__(1024) k_group_scatter(const int32_t* __restrict__ idx, int TK,
                                                         int E, int nbits,
                                                         const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ base,
                                                         int32_t* __restrict__ perm) {
  extern __shared__ int wcnt[];  // [16][E]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c = blockIdx.x;
  for (int i = tid; i < 16 * E; i += 1024) wcnt[i] = 0;
  __syncthreads();
  const int p = c * kGroupChunk + tid;
  const bool valid = p < TK;
  const int e = valid ? idx[p] : 0;
  const unsigned long long m = same_key_mask(e, nbits, valid);
  const int rank = __popcll(m & ((1ull << lane) - 1ull));
  if (valid && rank == 0) wcnt[wave * E + e] = __popcll(m);
  __syncthreads();
  if (valid) {
    int pre = 0;
    for (int w = 0; w < wave; ++w) pre += wcnt[w * E + e];
    perm[offsets[e] + base[size_t(c) * E + e] + pre + rank] = p;
  }
}

// Expert-GEMM setup (one workgroup): group row starts, m-tile starts for
// tiles of kPrefillBM rows, and each group's blob address (pool lookup for
// routed experts with at least one token).
__global__ void __launch_bounds__(1024) k_prefill_setup(const int32_t* __restrict__ counts,
                                                         const int32_t* __restrict__ offsets,
                                                         int E, int T, int K, int S,
                                                         ExpertSource src,
                                                         const uint8_t* shared_blob,
                                                         int32_t* __restrict__ gstart,
                                                         int32_t* __restrict__ tstart,
                                                         unsigned long long* __restrict__ gblob) {
  __shared__ int lds16[16];
  const int e = threadIdx.x;
  const int n = (e < E) ? counts[e] : 0;
  const int tiles = (n + kPrefillBM - 1) / kPrefillBM;
  int total;
  const int ts = block_exclusive_scan_1024(tiles, lds16, total);
  if (e < E) {
    gstart[e] = offsets[e];
    tstart[e] = ts;
    const uint8_t* b;
    if (src.expert_to_slot == nullptr) {
      b = src.slots + size_t(e) * src.stride;
    } else {
      const int slot = src.expert_to_slot[e];
      if (n > 0 && src.counters) {
        atomicAdd(&src.counters[1], 1ull);
        if (slot >= 0) atomicAdd(&src.counters[0], 1ull);
      }
      b = slot >= 0 ? src.slots + size_t(slot) * src.stride : src.host_blobs + size_t(e) * src.stride;
    }
    gblob[e] = reinterpret_cast<unsigned long long>(b);
  }
  if (e == 0) {
    const int TK = T * K;
    gstart[E] = TK;
    gstart[E + 1] = TK + S * T;
    tstart[E] = total;
    tstart[E + 1] = total + S * ((T + kPrefillBM - 1) / kPrefillBM);
    gblob[E] = reinterpret_cast<unsigned long long>(shared_blob);
  }
}

// ===========================================================================
// grouped GEMM
// ===========================================================================
enum GemmMode { kRouter = 0, kLoraGU = 1, kGateUp = 2, kLoraD = 3, kDown = 4 };

constexpr int BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // bf16 elements; 144-byte rows avoid bank conflicts

template <int BM, int BN, int WM, int WN>
struct TileCfg {
  static_assert(WM * WN == 4, "4 waves");
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int MB = WTM / 16, NB = WTN / 16;
  static constexpr int A_SEGS = BM * 8 / 256;  // 16-byte A segments per thread per chunk
};

// token of sorted row s
__device__ __forceinline__ int token_of(const GemmArgs& a, int s) {
  const int TK = a.T * a.K;
  return s < TK ? a.perm[s] / a.K : s - TK;
}

// find group g with tstart[g] <= mt < tstart[g+1] (g in [0, E])
__device__ __forceinline__ int group_of_tile(const int32_t* tstart, int G, int mt) {
  int lo = 0, hi = G;  // invariant: tstart[lo] <= mt < tstart[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tstart[mid] <= mt) lo = mid; else hi = mid;
  }
  return lo;
}

// 16 int8 codes -> 16 bf16 (exact)
__device__ __forceinline__ void int8x16_to_bf16(const uint4 q, uint4& lo, uint4& hi) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  uint32_t o[8];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float c0 = float(int8_t((w[d] >> (16 * h)) & 0xFF));
      const float c1 = float(int8_t((w[d] >> (16 * h + 8)) & 0xFF));
      o[2 * d + h] = (__float_as_uint(c0) >> 16) | (__float_as_uint(c1) & 0xFFFF0000u);
    }
  }
  lo = make_uint4(o[0], o[1], o[2], o[3]);
  hi = make_uint4(o[4], o[5], o[6], o[7]);
}

template <int MODE, int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(256) k_gemm(GemmArgs a) {
  using C = TileCfg<BM, BN, WM, WN>;
  constexpr bool kF16 = (MODE == kLoraD || MODE == kDown);  // fp16 operands
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDS_STRIDE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave / WN) * C::WTM, wn0 = (wave % WN) * C::WTN;

  // ---- which tile ---------------------------------------------------------
  int ntn, Kdim, Nrows;
  if (MODE == kRouter) { Kdim = a.H; Nrows = a.E + a.S; }
  else if (MODE == kLoraGU) { Kdim = a.H; Nrows = 64; }
  else if (MODE == kGateUp) { Kdim = a.H; Nrows = 2 * a.I; }
  else if (MODE == kLoraD) { Kdim = a.I; Nrows = 64; }
  else { Kdim = a.I; Nrows = a.H; }
  ntn = (Nrows + BN - 1) / BN;
  const int mt = blockIdx.x / ntn, nt = blockIdx.x % ntn;
  const int n0 = nt * BN;
  int row0, row_end, g = 0;
  const uint8_t* blob = nullptr;
  if (MODE == kRouter) {
    row0 = mt * BM;
    if (row0 >= a.T) return;
    row_end = min(a.T, row0 + BM);
  } else {
    const int G = a.E + 1;
    if (mt >= a.tstart[G]) return;
    g = group_of_tile(a.tstart, G, mt);
    row0 = a.gstart[g] + (mt - a.tstart[g]) * BM;
    row_end = min(a.gstart[g + 1], row0 + BM);
    blob = reinterpret_cast<const uint8_t*>(a.gblob[g]);
  }

  // ---- per-thread A row sources ------------------------------------------
  const uint16_t* arow[C::A_SEGS];
  int aseg[C::A_SEGS];
#pragma unroll
  for (int i = 0; i < C::A_SEGS; ++i) {
    const int sidx = tid + 256 * i;
    const int m = sidx >> 3;
    aseg[i] = sidx & 7;
    const int s = row0 + m;
    if (s >= row_end) { arow[i] = nullptr; continue; }
    if (MODE == kRouter) arow[i] = a.x + size_t(s) * a.H;
    else if (MODE == kLoraGU || MODE == kGateUp) arow[i] = a.x + size_t(token_of(a, s)) * a.H;
    else arow[i] = a.hs + size_t(s) * a.I;
  }

  const int nchunks = Kdim / BK;
  const bool lora_chunk = (MODE == kGateUp || MODE == kDown) && a.r > 0;
  const int total_chunks = nchunks + (lora_chunk ? 1 : 0);

  f32x4_t acc[C::MB][C::NB];
#pragma unroll
  for (int i = 0; i < C::MB; ++i)
#pragma unroll
    for (int j = 0; j < C::NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // register staging of one chunk
  uint4 ra[C::A_SEGS];
  // B staging: int4 -> 16B codes + scale/bias; int8 -> 16B codes; bf16 -> 16B
  constexpr int B_SEGS_INT4 = (BN * 2 + 255) / 256;   // 16B = 32 codes = half a row-chunk
  constexpr int B_SEGS_INT8 = (BN * 4 + 255) / 256;   // 16B = 16 codes
  constexpr int B_SEGS_BF16 = (BN * 8 + 255) / 256;   // 16B = 8 bf16
  constexpr int B_SEGS = (MODE == kRouter) ? B_SEGS_INT8
                         : (MODE == kLoraGU || MODE == kLoraD) ? B_SEGS_BF16 : B_SEGS_INT4;
  uint4 rb[B_SEGS > B_SEGS_BF16 ? B_SEGS : B_SEGS_BF16];
  uint32_t rsb[B_SEGS];

  auto load_chunk = [&](int c) {
    const bool is_lora = lora_chunk && c == nchunks;
    const int k0 = c * BK;
    // A side
#pragma unroll
    for (int i = 0; i < C::A_SEGS; ++i) {
      const int m = (tid + 256 * i) >> 3;
      const uint16_t* src = arow[i];
      if (is_lora) {
        src = nullptr;
        const int s = row0 + m;
        if (s < row_end) src = (MODE == kGateUp ? a.u : a.ud) + size_t(s) * kLoraK;
        ra[i] = src ? *reinterpret_cast<const uint4*>(src + 8 * aseg[i]) : make_uint4(0, 0, 0, 0);
      } else {
        ra[i] = src ? *reinterpret_cast<const uint4*>(src + k0 + 8 * aseg[i]) : make_uint4(0, 0, 0, 0);
      }
    }
    // B side
    if (is_lora) {
      // rows of B_lora [rows][r] bf16, repeated at the hi and lo positions of
      // the activation side: gate/up k = [g_hi 0..15 | g_lo 16..31 | u_hi 32..47
      // | u_lo 48..63], down k = [hi 0..31 | lo 32..63]
#pragma unroll
      for (int i = 0; i < B_SEGS_BF16; ++i) {
        const int sidx = tid + 256 * i;
        const int n = sidx >> 3, seg = sidx & 7;
        uint32_t v[4] = {0, 0, 0, 0};
        const int R = n0 + n;
        if (n < BN && R < Nrows) {
          const uint16_t* Bl = reinterpret_cast<const uint16_t*>(
              blob + (MODE == kGateUp ? a.L.b_gu : a.L.b_dn));
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t pair[2] = {0u, 0u};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int k = 8 * seg + 2 * q + h;
              bool ok;
              int rr;
              if (MODE == kGateUp) {
                ok = ((k >> 5) == ((R >> 4) & 1));  // gate rows take k < 32, up rows k >= 32
                rr = k & 15;
              } else {
                ok = true;
                rr = k & 31;
              }
              if (ok && rr < a.r) pair[h] = Bl[size_t(R) * a.r + rr];
            }
            v[q] = pair[0] | (pair[1] << 16);
          }
        }
        rb[i] = make_uint4(v[0], v[1], v[2], v[3]);
      }
      return;
    }
    if (MODE == kRouter) {
#pragma unroll
      for (int i = 0; i < B_SEGS_INT8; ++i) {
        const int sidx = tid + 256 * i;
        const int n = sidx >> 2, seg = sidx & 3;
        const int R = n0 + n;
        const int8_t* q = nullptr;
        if (n < BN && R < Nrows) q = (R < a.E) ? a.rq + size_t(R) * a.H : a.sq;
        rb[i] = q ? *reinterpret_cast<const uint4*>(q + k0 + 16 * seg) : make_uint4(0, 0, 0, 0);
      }
    } else if (MODE == kLoraGU || MODE == kLoraD) {
#pragma unroll
      for (int i = 0; i < B_SEGS_BF16; ++i) {
        const int sidx = tid + 256 * i;
        const int n = sidx >> 3, seg = sidx & 7;
        const uint16_t* src = nullptr;
        if (n < BN) {
          // output column n computes row (n & 15) of A_gate (n < 32) or A_up
          // (n >= 32) for gate/up, row (n & 31) of A_down for down; each row
          // appears twice so the epilogue can store a hi and a lo bf16 part
          if (MODE == kLoraGU) {
            const int rr = n & 15;
            if (rr < a.r)
              src = reinterpret_cast<const uint16_t*>(blob + a.L.a_gu) +
                    (size_t(n >= 32 ? a.r : 0) + rr) * a.H;
          } else if ((n & 31) < a.r) {
            src = reinterpret_cast<const uint16_t*>(blob + a.L.a_dn) + size_t(n & 31) * a.I;
          }
        }
        rb[i] = src ? *reinterpret_cast<const uint4*>(src + k0 + 8 * seg) : make_uint4(0, 0, 0, 0);
      }
    } else {
      const size_t off_c = (MODE == kGateUp) ? a.L.gu_codes : a.L.dn_codes;
      const size_t off_s = (MODE == kGateUp) ? a.L.gu_sb : a.L.dn_sb;
#pragma unroll
      for (int i = 0; i < B_SEGS_INT4; ++i) {
        const int sidx = tid + 256 * i;
        const int n = sidx >> 1, half = sidx & 1;
        const int R = n0 + n;
        if (n < BN && R < Nrows) {
          rb[i] = *reinterpret_cast<const uint4*>(blob + off_c + size_t(R) * (Kdim / 2) + k0 / 2 +
                                                  16 * half);
          rsb[i] = reinterpret_cast<const uint32_t*>(blob + off_s)[size_t(R) * (Kdim / 64) + c];
        } else {
          rb[i] = make_uint4(0, 0, 0, 0);
          rsb[i] = 0;
        }
      }
    }
  };

  // router: fp32 group scale per output column, applied per chunk (never
  // rounded into the bf16 operand)
  auto router_scale = [&](int n, int c) -> float {
    const int R = n0 + n;
    if (R < a.E) return a.rs[size_t(R) * (a.H / 64) + c];
    if (R < Nrows) return a.ss[c];
    return 0.f;
  };

  // Per-chunk fp32 affine terms of the post-scaled modes: column scale, column
  // offset (b - 128 s) and the row sums of the activations over the chunk.
  __shared__ __attribute__((aligned(16))) float Ssc[BN];
  __shared__ __attribute__((aligned(16))) float Sbp[BN];
  __shared__ __attribute__((aligned(16))) float Xs[BM];
  constexpr bool kPost = (MODE == kRouter || MODE == kGateUp || MODE == kDown);

  auto store_chunk = [&](int c) {
    const bool is_lora = lora_chunk && c == nchunks;
#pragma unroll
    for (int i = 0; i < C::A_SEGS; ++i) {
      const int sidx = tid + 256 * i;
      *reinterpret_cast<uint4*>(&As[(sidx >> 3) * LDS_STRIDE + 8 * (sidx & 7)]) = ra[i];
      if ((MODE == kGateUp || MODE == kDown) && !is_lora) {
        // row sum over the 64 columns of this chunk: 8 lanes hold one row
        const uint32_t w4[4] = {ra[i].x, ra[i].y, ra[i].z, ra[i].w};
        float sum = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          sum += kF16 ? f16_lo(w4[k]) + f16_hi(w4[k]) : bf16_lo(w4[k]) + bf16_hi(w4[k]);
        sum = group_sum<8>(sum);
        if ((sidx & 7) == 0) Xs[sidx >> 3] = sum;
      }
    }
    if (is_lora || MODE == kLoraGU || MODE == kLoraD) {
#pragma unroll
      for (int i = 0; i < B_SEGS_BF16; ++i) {
        const int sidx = tid + 256 * i;
        if ((sidx >> 3) < BN) {
          uint4 v = rb[i];
          if (kF16)  // bf16 LoRA factors -> fp16 operands
            v = make_uint4(bf16x2_to_f16x2(v.x), bf16x2_to_f16x2(v.y), bf16x2_to_f16x2(v.z),
                           bf16x2_to_f16x2(v.w));
          *reinterpret_cast<uint4*>(&Bs[(sidx >> 3) * LDS_STRIDE + 8 * (sidx & 7)]) = v;
        }
      }
    } else if (MODE == kRouter) {
#pragma unroll
      for (int i = 0; i < B_SEGS_INT8; ++i) {
        const int sidx = tid + 256 * i;
        const int n = sidx >> 2;
        if (n < BN) {
          uint4 lo, hi;
          int8x16_to_bf16(rb[i], lo, hi);
          uint16_t* dst = &Bs[n * LDS_STRIDE + 16 * (sidx & 3)];
          *reinterpret_cast<uint4*>(dst) = lo;
          *reinterpret_cast<uint4*>(dst + 8) = hi;
          if ((sidx & 3) == 0) {
            Ssc[n] = router_scale(n, c);
            Sbp[n] = 0.f;
          }
        }
      }
    } else {
      // int4: exact codes as the bf16 values 128 + q; the affine map is applied
      // in fp32 after the MFMA (s * P + (b - 128 s) * rowsum)
#pragma unroll
      for (int i = 0; i < B_SEGS_INT4; ++i) {
        const int sidx = tid + 256 * i;
        const int n = sidx >> 1;
        if (n < BN) {
          uint16_t* dst = &Bs[n * LDS_STRIDE + 32 * (sidx & 1)];
          const uint32_t w[4] = {rb[i].x, rb[i].y, rb[i].z, rb[i].w};
#pragma unroll
          for (int d = 0; d < 4; ++d)
            *reinterpret_cast<uint4*>(dst + 8 * d) =
                kF16 ? make_uint4(codes_to_f16x2_biased(w[d], 0), codes_to_f16x2_biased(w[d], 1),
                                  codes_to_f16x2_biased(w[d], 2), codes_to_f16x2_biased(w[d], 3))
                     : make_uint4(codes_to_bf16x2_biased(w[d], 0), codes_to_bf16x2_biased(w[d], 1),
                                  codes_to_bf16x2_biased(w[d], 2), codes_to_bf16x2_biased(w[d], 3));
          if ((sidx & 1) == 0) {
            const float sc = bf16_lo(rsb[i]);
            Ssc[n] = sc;
            Sbp[n] = fmaf(-128.0f, sc, bf16_hi(rsb[i]));
          }
        }
      }
    }
  };

  load_chunk(0);
  for (int c = 0; c < total_chunks; ++c) {
    __syncthreads();
    store_chunk(c);
    __syncthreads();
    if (c + 1 < total_chunks) load_chunk(c + 1);
    const bool post = kPost && !(lora_chunk && c == nchunks);
    f32x4_t part[C::MB][C::NB];
#pragma unroll
    for (int i = 0; i < C::MB; ++i)
#pragma unroll
      for (int j = 0; j < C::NB; ++j) part[i][j] = post ? f32x4_t{0.f, 0.f, 0.f, 0.f} : acc[i][j];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 af[C::MB], bfr[C::NB];
#pragma unroll
      for (int i = 0; i < C::MB; ++i)
        af[i] = *reinterpret_cast<const uint4*>(
            &As[(wm0 + 16 * i + (lane & 15)) * LDS_STRIDE + 32 * ks + 8 * (lane >> 4)]);
#pragma unroll
      for (int j = 0; j < C::NB; ++j)
        bfr[j] = *reinterpret_cast<const uint4*>(
            &Bs[(wn0 + 16 * j + (lane & 15)) * LDS_STRIDE + 32 * ks + 8 * (lane >> 4)]);
#pragma unroll
      for (int i = 0; i < C::MB; ++i)
#pragma unroll
        for (int j = 0; j < C::NB; ++j) {
          if (kF16)
            part[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                __builtin_bit_cast(f16x8_t, af[i]), __builtin_bit_cast(f16x8_t, bfr[j]),
                part[i][j], 0, 0, 0);
          else
            part[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, af[i]), __builtin_bit_cast(bf16x8_t, bfr[j]),
                part[i][j], 0, 0, 0);
        }
    }
    if (post) {
      float xg[C::MB][4];
#pragma unroll
      for (int i = 0; i < C::MB; ++i) {
        if (MODE == kRouter) {
          xg[i][0] = xg[i][1] = xg[i][2] = xg[i][3] = 0.f;
        } else {
          const float4 v = *reinterpret_cast<const float4*>(&Xs[wm0 + 16 * i + 4 * (lane >> 4)]);
          xg[i][0] = v.x; xg[i][1] = v.y; xg[i][2] = v.z; xg[i][3] = v.w;
        }
      }
#pragma unroll
      for (int j = 0; j < C::NB; ++j) {
        const float sc = Ssc[wn0 + 16 * j + (lane & 15)];
        const float bp = Sbp[wn0 + 16 * j + (lane & 15)];
#pragma unroll
        for (int i = 0; i < C::MB; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[i][j][q] = fmaf(sc, part[i][j][q], fmaf(bp, xg[i][q], acc[i][j][q]));
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::MB; ++i)
#pragma unroll
        for (int j = 0; j < C::NB; ++j) acc[i][j] = part[i][j];
    }
  }

  // ---- epilogue ----------------------------------------------------------
#pragma unroll
  for (int i = 0; i < C::MB; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = wm0 + 16 * i + 4 * (lane >> 4) + q;
      const int s = row0 + m;
      if (s >= row_end) continue;
      if (MODE == kGateUp) {
#pragma unroll
        for (int j = 0; j < C::NB; j += 2) {
          const int R = n0 + wn0 + 16 * j + (lane & 15);  // gate blob row
          const int jj = ((R >> 5) << 4) | (R & 15);
          const float hv = silu_f(acc[i][j][q]) * acc[i][j + 1][q];
          a.hs_out[size_t(s) * a.I + jj] = f32_to_f16_sat(hv);
        }
      } else {
#pragma unroll
        for (int j = 0; j < C::NB; ++j) {
          const int n = n0 + wn0 + 16 * j + (lane & 15);
          const float v = acc[i][j][q];
          if (MODE == kRouter) {
            if (n < a.E) a.logits[size_t(s) * a.E + n] = v + (a.bias ? a.bias[n] : 0.f);
            else if (n < Nrows) a.sg_logit[s] = v;
          } else if (MODE == kLoraGU || MODE == kLoraD) {
            // lambda * (A v) as a hi + lo pair: bf16 for gate/up (about 16
            // significant bits), fp16 for down (about 22)
            const float lv = a.lam * v;
            const bool lo_col = (MODE == kLoraGU) ? (n & 16) : (n & 32);
            uint16_t out;
            if (kF16) {
              const uint16_t hi = f32_to_f16_sat(lv);
              out = lo_col ? f32_to_f16_sat(lv - f16_to_f32(hi)) : hi;
            } else {
              const uint16_t hi = f32_to_bf16(lv);
              out = lo_col ? f32_to_bf16(lv - bf16_to_f32(hi)) : hi;
            }
            if (n < kLoraK) (MODE == kLoraGU ? a.u_out : a.ud_out)[size_t(s) * kLoraK + n] = out;
          } else {  // kDown
            if (n < Nrows) {
              const int TK = a.T * a.K, KS = a.K + a.S;
              size_t dest;
              if (s < TK) {
                const int pr = a.perm[s];
                dest = size_t(pr / a.K) * KS + pr % a.K;
              } else {
                dest = size_t(s - TK) * KS + a.K;
              }
              a.y[dest * a.H + n] = v;
            }
          }
        }
      }
    }
  }
}

// ===========================================================================
// host launchers
// ===========================================================================
hipError_t launch_group(const int32_t* idx, int T, int K, int E, int32_t* counts,
                        int32_t* offsets, int32_t* perm, int32_t* chunk_hist, int32_t* base,
                        hipStream_t st) {
  const int TK = T * K;
  const int nch = (TK + kGroupChunk - 1) / kGroupChunk;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  if (nch > 0) hipLaunchKernelGGL(k_group_hist, dim3(nch), dim3(1024), 0, st, idx, TK, E, chunk_hist);
  hipLaunchKernelGGL(k_group_scan, dim3(1), dim3(1024), 0, st, chunk_hist, nch, E, TK, counts,
                     offsets, base);
  if (nch > 0)
    hipLaunchKernelGGL(k_group_scatter, dim3(nch), dim3(1024), 16 * E * sizeof(int), st, idx, TK,
                       E, nbits, offsets, base, perm);
  return hipGetLastError();
}

hipError_t launch_router_gemm(const GemmArgs& a, hipStream_t st) {
  constexpr int BM = 64, BN = 64;
  const int mtn = (a.T + BM - 1) / BM, ntn = (a.E + a.S + BN - 1) / BN;
  hipLaunchKernelGGL((k_gemm<kRouter, BM, BN, 2, 2>), dim3(mtn * ntn), dim3(256), 0, st, a);
  return hipGetLastError();
}

int prefill_max_mtiles(int T, int K, int E, int S) {
  const int TK = T * K;
  return (TK + kPrefillBM - 1) / kPrefillBM + (TK < E ? TK : E) +
         S * ((T + kPrefillBM - 1) / kPrefillBM);
}

hipError_t launch_prefill_experts(const GemmArgs& a, const int32_t* counts, ExpertSource src,
                                  const uint8_t* shared_blob, hipStream_t st) {
  hipLaunchKernelGGL(k_prefill_setup, dim3(1), dim3(1024), 0, st, counts, a.offsets, a.E, a.T,
                     a.K, a.S, src, shared_blob, const_cast<int32_t*>(a.gstart),
                     const_cast<int32_t*>(a.tstart), const_cast<unsigned long long*>(a.gblob));
  const int mt = prefill_max_mtiles(a.T, a.K, a.E, a.S);
  if (a.r > 0)
    hipLaunchKernelGGL((k_gemm<kLoraGU, kPrefillBM, 64, 2, 2>), dim3(mt), dim3(256), 0, st, a);
  hipLaunchKernelGGL((k_gemm<kGateUp, kPrefillBM, 128, 2, 2>), dim3(mt * ((2 * a.I + 127) / 128)),
                     dim3(256), 0, st, a);
  if (a.r > 0)
    hipLaunchKernelGGL((k_gemm<kLoraD, kPrefillBM, 64, 2, 2>), dim3(mt), dim3(256), 0, st, a);
  hipLaunchKernelGGL((k_gemm<kDown, kPrefillBM, 128, 2, 2>), dim3(mt * ((a.H + 127) / 128)),
                     dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe

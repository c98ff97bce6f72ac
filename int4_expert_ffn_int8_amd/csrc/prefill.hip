// Prefill path: group (token, k) pairs by expert; router and LoRA-A GEMMs.
//
// [P2] "SSD 专家卸载 · Prerouter 路由预测", prefill/decode paragraph: prefill
// loads whole layers and computes in batches, decode relies on caching and
// prefetch.  Here prefill groups each expert's tokens (stable, by expert) and
// runs one dense contraction per expert (the expert GEMMs are in
// expert_gemm.hip).  This file holds the stable scatter of the grouping (the
// per-chunk histograms are filled by the top-K kernel), and k_gemm for the
// router GEMM (int8 codes exact in bf16, fp32
// scale per 64-column chunk) and the two skinny LoRA-A GEMMs of the unmerged
// delta ([P1] Recover-LoRA paragraph), whose outputs lambda * (A v) are
// stored as bf16 hi + lo pairs in the row-scaled domain of the expert GEMMs.
// The LoRA-A GEMM of down also converts h (fp32, from the gate/up epilogue)
// into the fp16 rows with row exponents that the down GEMM reads.
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

// Stable scatter: pair p of chunk c goes to offsets[e] + (pairs of expert e in
// chunks before c) + (earlier pairs of e in chunk c).  Every workgroup first
// scans the per-chunk histograms (filled by the top-K kernel) for its own
// bases and the offsets; workgroup 0 also writes counts and offsets.
// grid nch, block 1024, dynamic LDS 16 * E ints.
__global__ void __launch_bounds__(1024) k_group_scatter(const int32_t* __restrict__ idx, int TK,
                                                         int E, int nbits, int nch,
                                                         const int32_t* __restrict__ chunk_hist,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ perm) {
  extern __shared__ int wcnt[];  // [16][E]
  __shared__ int lds16[16];
  __shared__ int lds_start[kMaxE];  // offsets[e] + pairs of e in earlier chunks
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c = blockIdx.x;
  // bases of this chunk and the totals, for expert tid
  int before = 0, tot = 0;
  if (tid < E) {
    for (int cc = 0; cc < nch; ++cc) {
      const int v = chunk_hist[size_t(cc) * E + tid];
      before += (cc < c) ? v : 0;
      tot += v;
    }
  }
  int total;
  const int off = block_exclusive_scan_1024(tid < E ? tot : 0, lds16, total);
  if (tid < E) {
    lds_start[tid] = off + before;
    if (c == 0) {
      counts[tid] = tot;
      offsets[tid] = off;
    }
  }
  if (c == 0 && tid == 0) offsets[E] = TK;
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
    perm[lds_start[e] + pre + rank] = p;
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

// v, or zeros when !keep (bit operations, no branch)
__device__ __forceinline__ uint4 and_mask(uint4 v, bool keep) {
  const uint32_t m = keep ? ~0u : 0u;
  return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
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
  static_assert(MODE == kRouter || MODE == kLoraGU || MODE == kLoraD,
                "k_gemm: router and LoRA-A GEMMs (the expert GEMMs are k_expert_gemm)");
  using C = TileCfg<BM, BN, WM, WN>;
  constexpr bool kF16 = (MODE == kLoraD);  // fp16 operands (h * 2^-eh and A_down)
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDS_STRIDE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave / WN) * C::WTM, wn0 = (wave % WN) * C::WTN;
  if (MODE == kRouter && a.zero && blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = tid; i < a.nzero; i += 256) a.zero[i] = 0;

  // ---- which tile ---------------------------------------------------------
  int ntn, Kdim, Nrows;
  if (MODE == kRouter) { Kdim = a.H; Nrows = a.E + a.S; }
  else if (MODE == kLoraGU) { Kdim = a.H; Nrows = 32; }  // A_gate rows 0..15, A_up rows 16..31
  else { Kdim = a.I; Nrows = 64; }
  ntn = (Nrows + BN - 1) / BN;
  // LoRA-A tiles may be narrower than the 128-row group tiles: each group
  // tile then takes kPrefillBM / BM consecutive workgroups
  constexpr int kSub = (MODE == kRouter) ? 1 : kPrefillBM / BM;
  static_assert(MODE == kRouter || kPrefillBM % BM == 0, "LoRA-A tiles divide the group tiles");
  int mt, nt, sub, ks, nks;
  if (MODE == kRouter) {
    // 1-D grid, workgroup b on XCD b % 8: each XCD takes a contiguous run of
    // (row tile, K split) units, and the column tiles of a unit, which read
    // the same slice of x, run on that XCD one after another (its L2 serves
    // all but the first read of the slice)
    nks = a.plog ? kRouterSplit : 1;
    const int units = ((a.T + BM - 1) / BM) * nks, per = (units + 7) / 8;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int unit = xcd * per + slot / ntn;
    if (slot / ntn >= per || unit >= units) return;
    mt = unit / nks;
    ks = unit % nks;
    nt = slot % ntn;
    sub = 0;
  } else {
    mt = blockIdx.x / ntn / kSub;
    nt = blockIdx.x % ntn;
    sub = (blockIdx.x / ntn) % kSub;
    ks = blockIdx.y;  // split-K over blockIdx.y (partial sums of disjoint chunk ranges)
    nks = gridDim.y;
  }
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
    row0 = a.gstart[g] + (mt - a.tstart[g]) * kPrefillBM + sub * BM;
    if (row0 >= a.gstart[g + 1]) return;
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
    else if (MODE == kLoraGU) arow[i] = a.x + size_t(token_of(a, s)) * a.H;
    else arow[i] = a.hs + size_t(s) * a.I;
  }
  // LoRA-A of down reads h in fp32 and converts each row to fp16(h * 2^-e)
  // itself (e from the row maximum of the gate/up epilogue), writing the
  // converted rows and exponents for the down GEMM as it goes: every row of
  // the sorted row space is read by exactly one workgroup, once.
  constexpr bool kH16 = (MODE == kLoraD);
  int hexp[C::A_SEGS], hrs[C::A_SEGS];
#pragma unroll
  for (int i = 0; i < C::A_SEGS; ++i) {
    const int s = row0 + ((tid + 256 * i) >> 3);
    const bool ok = kH16 && s < row_end;
    hrs[i] = ok ? s : -1;
    hexp[i] = ok ? row_exp(__uint_as_float(a.hmax[s])) : 0;
  }

  const int nchunks = Kdim / BK;

  f32x4_t acc[C::MB][C::NB];
#pragma unroll
  for (int i = 0; i < C::MB; ++i)
#pragma unroll
    for (int j = 0; j < C::NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // register staging of a chunk, two chunks in flight (stages 0 and 1)
  constexpr int H_SEGS = kH16 ? C::A_SEGS : 1;  // h segments with their block exponents (LoRA-A of down)
  // B staging: int4 -> 16B codes + scale/bias; int8 -> 16B codes; bf16 -> 16B
  constexpr int B_SEGS_INT8 = (BN * 4 + 255) / 256;   // 16B = 16 codes
  constexpr int B_SEGS_BF16 = (BN * 8 + 255) / 256;   // 16B = 8 bf16
  constexpr int B_SEGS = (MODE == kRouter) ? B_SEGS_INT8 : B_SEGS_BF16;
  struct Stage {
    uint4 ra[C::A_SEGS];
    uint4 rh[H_SEGS];
    int rhe[H_SEGS];
    uint4 rb[B_SEGS];
    float rs[B_SEGS];  // router: the fp32 group scale of the column
  };
  Stage st0, st1;

  // whether B staging column n holds a LoRA-A row (else it is zeroed)
  auto lora_b_ok = [&](int n) {
    return n < BN && (MODE == kLoraGU ? (n & 15) : (n & 31)) < a.r;
  };
  // Every load is issued unconditionally (operands outside the tile read
  // valid memory of the same array; store_chunk zeroes them), so that the
  // waits before a chunk's use cover only that chunk's loads.
  auto load_chunk = [&](Stage& st, int c) {
    uint4(&ra)[C::A_SEGS] = st.ra;
    uint4(&rh)[H_SEGS] = st.rh;
    int(&rhe)[H_SEGS] = st.rhe;
    uint4(&rb)[B_SEGS] = st.rb;
    const int k0 = c * BK;
    if constexpr (kH16) {
#pragma unroll
      for (int i = 0; i < C::A_SEGS; ++i) {
        const int s = hrs[i] >= 0 ? hrs[i] : 0;  // rows past the tile read row 0 (zeroed when stored)
        const int col = k0 + 8 * aseg[i];        // 8 columns inside one 16-column block
        rh[i] = *reinterpret_cast<const uint4*>(a.hl + size_t(s) * a.I + col);
        rhe[i] = a.hbe[size_t(s) * (a.I / 16) + col / 16];
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::A_SEGS; ++i) {
        ra[i] = *reinterpret_cast<const uint4*>((arow[i] ? arow[i] : a.x) + k0 + 8 * aseg[i]);
      }
    }
    if (MODE == kRouter) {
#pragma unroll
      for (int i = 0; i < B_SEGS_INT8; ++i) {
        const int sidx = tid + 256 * i;
        const int n = sidx >> 2, seg = sidx & 3;
        const int R = n0 + n;
        const int8_t* q = !(n < BN && R < Nrows) ? a.rq : (R < a.E) ? a.rq + size_t(R) * a.H : a.sq;
        rb[i] = *reinterpret_cast<const uint4*>(q + k0 + 16 * seg);
        // the column's scale for this chunk (rows past the tile read row 0's)
        const float* sp = (R < a.E && n < BN) ? a.rs + size_t(R) * (a.H / 64)
                                              : (R < Nrows && n < BN ? a.ss : a.rs);
        st.rs[i] = sp[c];
      }
    } else {
      // (no LoRA-A launch without LoRA: r >= 1, so row 0 of each factor exists)
      const uint16_t* base = reinterpret_cast<const uint16_t*>(blob + (MODE == kLoraGU ? a.L.a_gu : a.L.a_dn));
#pragma unroll
      for (int i = 0; i < B_SEGS_BF16; ++i) {
        const int sidx = tid + 256 * i;
        const int n = sidx >> 3, seg = sidx & 7;
        // gate/up: output column n computes row (n & 15) of A_gate (n < 16)
        // or A_up (n >= 16), summed over K splits and split into hi/lo bf16
        // parts as the gate/up GEMM stages its LoRA chunk; down: row (n & 31) of A_down, each row
        // appearing twice so the epilogue can store a hi and a lo part
        const size_t row = (MODE == kLoraGU) ? size_t(n >= 16 ? a.r : 0) + (n & 15) : size_t(n & 31);
        const size_t ld = (MODE == kLoraGU) ? size_t(a.H) : size_t(a.I);
        // (through the global address space: the blob address is read from
        // memory and would otherwise load through flat instructions)
        rb[i] = gload16(base + (lora_b_ok(n) ? row * ld : 0) + k0 + 8 * seg);
      }
    }
  };

  // router: fp32 scale of each output column for the current chunk (the
  // int8 codes enter the MFMA exactly; the scale is applied per chunk)
  __shared__ __attribute__((aligned(16))) float Ssc[BN];
  constexpr bool kPost = (MODE == kRouter);

  auto store_chunk = [&](Stage& st, int c) {
    uint4(&ra)[C::A_SEGS] = st.ra;
    uint4(&rh)[H_SEGS] = st.rh;
    int(&rhe)[H_SEGS] = st.rhe;
    uint4(&rb)[B_SEGS] = st.rb;
    if constexpr (kH16) {  // fp16(h * 2^-e), as the down GEMM reads it: a power-of-two rescale
#pragma unroll
      for (int i = 0; i < C::A_SEGS; ++i) {
        const int dd = rhe[i] - hexp[i];
        const uint32_t hw[4] = {rh[i].x, rh[i].y, rh[i].z, rh[i].w};
        uint32_t ow[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const f16x2_t p = __builtin_bit_cast(f16x2_t, hw[k]);
          const f16x2_t r = {_Float16(ldexpf(float(p[0]), dd)), _Float16(ldexpf(float(p[1]), dd))};
          ow[k] = __builtin_bit_cast(uint32_t, r);
        }
        ra[i] = make_uint4(ow[0], ow[1], ow[2], ow[3]);
        ra[i] = and_mask(ra[i], hrs[i] >= 0);  // a row past the tile is zero
        if (hrs[i] >= 0) {
          *reinterpret_cast<uint4*>(a.hs_out + size_t(hrs[i]) * a.I + c * BK + 8 * aseg[i]) = ra[i];
          if (c == 0 && aseg[i] == 0) a.eh_out[hrs[i]] = hexp[i];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < C::A_SEGS; ++i) {
      const int sidx = tid + 256 * i;
      const bool ok = kH16 || arow[i] != nullptr;  // rows past the tile are zero
      *reinterpret_cast<uint4*>(&As[(sidx >> 3) * LDS_STRIDE + 8 * (sidx & 7)]) = and_mask(ra[i], ok);
    }
    if (MODE == kLoraGU || MODE == kLoraD) {
#pragma unroll
      for (int i = 0; i < B_SEGS_BF16; ++i) {
        const int sidx = tid + 256 * i;
        if ((sidx >> 3) < BN) {
          uint4 v = and_mask(rb[i], lora_b_ok(sidx >> 3));
          if (kF16)  // bf16 LoRA factors -> fp16 operands
            v = make_uint4(bf16x2_to_f16x2(v.x), bf16x2_to_f16x2(v.y), bf16x2_to_f16x2(v.z),
                           bf16x2_to_f16x2(v.w));
          *reinterpret_cast<uint4*>(&Bs[(sidx >> 3) * LDS_STRIDE + 8 * (sidx & 7)]) = v;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < B_SEGS_INT8; ++i) {
        const int sidx = tid + 256 * i;
        const int n = sidx >> 2;
        if (n < BN) {
          const bool ok = n0 + n < Nrows;  // columns past the router rows are zero
          uint4 lo, hi;
          int8x16_to_bf16(and_mask(rb[i], ok), lo, hi);
          uint16_t* dst = &Bs[n * LDS_STRIDE + 16 * (sidx & 3)];
          *reinterpret_cast<uint4*>(dst) = lo;
          *reinterpret_cast<uint4*>(dst + 8) = hi;
          // (the column's four threads write the same value)
          Ssc[n] = __uint_as_float(__float_as_uint(st.rs[i]) & (ok ? ~0u : 0u));
        }
      }
    }
  };

  const int c0 = ks * nchunks / nks, c1 = (ks + 1) * nchunks / nks;
  const int clast = max(c1 - 1, c0);  // prefetches past the range reload its last chunk (unused)
  auto compute = [&]() {
    const bool post = kPost;
    f32x4_t part[C::MB][C::NB];
#pragma unroll
    for (int i = 0; i < C::MB; ++i)
#pragma unroll
      for (int j = 0; j < C::NB; ++j) part[i][j] = post ? f32x4_t{0.f, 0.f, 0.f, 0.f} : acc[i][j];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint4 af[C::MB], bfr[C::NB];
#pragma unroll
      for (int i = 0; i < C::MB; ++i)
        af[i] = *reinterpret_cast<const uint4*>(
            &As[(wm0 + 16 * i + (lane & 15)) * LDS_STRIDE + 32 * kk + 8 * (lane >> 4)]);
#pragma unroll
      for (int j = 0; j < C::NB; ++j)
        bfr[j] = *reinterpret_cast<const uint4*>(
            &Bs[(wn0 + 16 * j + (lane & 15)) * LDS_STRIDE + 32 * kk + 8 * (lane >> 4)]);
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
#pragma unroll
      for (int j = 0; j < C::NB; ++j) {
        const float sc = Ssc[wn0 + 16 * j + (lane & 15)];
#pragma unroll
        for (int i = 0; i < C::MB; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[i][j][q] = fmaf(sc, part[i][j][q], acc[i][j][q]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::MB; ++i)
#pragma unroll
        for (int j = 0; j < C::NB; ++j) acc[i][j] = part[i][j];
    }
  };
  // chunk c from a stage to LDS, the stage's next chunk (two ahead) into its
  // registers, then the MFMAs of chunk c; the other stage's loads stay in flight
  load_chunk(st0, c0);
  load_chunk(st1, min(c0 + 1, clast));
  for (int c = c0; c < c1; c += 2) {
    __syncthreads();
    store_chunk(st0, c);
    __syncthreads();
    load_chunk(st0, min(c + 2, clast));
    compute();
    if (c + 1 < c1) {
      __syncthreads();
      store_chunk(st1, c + 1);
      __syncthreads();
      load_chunk(st1, min(c + 3, clast));
      compute();
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
      {
#pragma unroll
        for (int j = 0; j < C::NB; ++j) {
          const int n = n0 + wn0 + 16 * j + (lane & 15);
          const float v = acc[i][j][q];
          if (MODE == kRouter) {
            if (a.plog) {  // partial of this K split; summed (and biased) by the top-K kernel
              if (n < Nrows) a.plog[(size_t(ks) * a.T + s) * Nrows + n] = v;
            } else if (n < a.E) {
              a.logits[size_t(s) * a.E + n] = v + (a.bias ? a.bias[n] : 0.f);
            } else if (n < Nrows) {
              a.sg_logit[s] = v;
            }
          } else if (MODE == kLoraGU) {  // partial of this K split
            if (n < Nrows) a.upart[(size_t(ks) * a.gstart[a.E + 1] + s) * Nrows + n] = v;
          } else if (MODE == kLoraD) {
            // lambda * (A v), in the row's scaled domain of the expert GEMM
            // (x rows enter as x * 2^-ex[token]; the down side's A operand is
            // already h * 2^-eh), as a bf16 hi + lo pair (about 16 significant bits)
            const float lv = a.lam * v;
            const bool lo_col = n & 32;
            const uint16_t hi = f32_to_bf16(lv);
            const uint16_t out = lo_col ? f32_to_bf16(lv - bf16_to_f32(hi)) : hi;
            if (n < kLoraK) a.ud_out[size_t(s) * kLoraK + n] = out;
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
                        int32_t* offsets, int32_t* perm, const int32_t* chunk_hist,
                        hipStream_t st) {
  const int TK = T * K;
  const int nch = (TK + kGroupChunk - 1) / kGroupChunk;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  if (nch > 0)
    hipLaunchKernelGGL(k_group_scatter, dim3(nch), dim3(1024), 16 * E * sizeof(int), st, idx, TK,
                       E, nbits, nch, chunk_hist, counts, offsets, perm);
  return hipGetLastError();
}

constexpr int kLoraBM = 64;  // rows per LoRA-A workgroup (two per group tile)

hipError_t launch_router_gemm(const GemmArgs& a, hipStream_t st) {
  constexpr int BM = 64, BN = 64;
  const int mtn = (a.T + BM - 1) / BM, ntn = (a.E + a.S + BN - 1) / BN;
  // split K so a few thousand tokens give about 1000 workgroups with short
  // chunk loops; the partial sums are reduced in a fixed order
  const int nks = a.plog ? kRouterSplit : 1;
  // (the top-K kernel sums the splits); one 1-D slot per (row tile, split,
  // column tile), padded so that every XCD has the same number of slots
  const int units = mtn * nks;
  hipLaunchKernelGGL((k_gemm<kRouter, BM, BN, 2, 2>), dim3(8 * ((units + 7) / 8) * ntn), dim3(256), 0, st, a);
  return hipGetLastError();
}

int prefill_max_mtiles(int T, int K, int E, int S) {
  const int TK = T * K;
  return (TK + kPrefillBM - 1) / kPrefillBM + (TK < E ? TK : E) +
         S * ((T + kPrefillBM - 1) / kPrefillBM);
}

hipError_t launch_prefill_experts(const GemmArgs& a, const int32_t* counts, ExpertSource src,
                                  const uint8_t* shared_blob, uint16_t* x16, int32_t* ex,
                                  uint16_t* hs16, int32_t* eh, hipStream_t st) {
  const int NR = a.T * a.K + a.S * a.T;
  X16SetupArgs xs;
  xs.x = a.x;
  xs.T = a.T;
  xs.H = a.H;
  xs.E = a.E;
  xs.K = a.K;
  xs.S = a.S;
  xs.x16 = x16;
  xs.ex = ex;
  xs.hmax = a.hmax;
  xs.counts = counts;
  xs.offsets = a.offsets;
  xs.src = src;
  xs.shared_blob = shared_blob;
  xs.gstart = const_cast<int32_t*>(a.gstart);
  xs.tstart = const_cast<int32_t*>(a.tstart);
  xs.gblob = const_cast<unsigned long long*>(a.gblob);
  hipError_t e = launch_x16_setup(xs, st);
  if (e != hipSuccess) return e;
  const int mt = prefill_max_mtiles(a.T, a.K, a.E, a.S);
  if (a.r > 0)  // LoRA-A of gate/up: K split in kLoraSplit; the gate/up GEMM sums the partials in order
    hipLaunchKernelGGL((k_gemm<kLoraGU, kLoraBM, 32, 2, 2>), dim3(mt * (kPrefillBM / kLoraBM), kLoraSplit),
                       dim3(256), 0, st, a);
  e = launch_expert_gemm(kGemmGateUp, a, mt, st);
  if (e != hipSuccess) return e;
  if (a.r > 0) {  // LoRA-A of down, which also writes h as fp16 rows with their exponents
    GemmArgs ad = a;
    ad.hs_out = hs16;
    ad.eh_out = eh;
    hipLaunchKernelGGL((k_gemm<kLoraD, kLoraBM, 64, 2, 2>), dim3(mt * (kPrefillBM / kLoraBM)), dim3(256), 0, st, ad);
  } else {
    e = launch_h16(a.hl, a.hbe, a.hmax, a.gstart + a.E + 1, NR, a.I, hs16, eh, st);
    if (e != hipSuccess) return e;
  }
  return launch_expert_gemm(kGemmDown, a, mt, st);
}

}  // namespace moe

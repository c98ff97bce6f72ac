// Prefill expert GEMMs (gate/up + SwiGLU, down) over each expert's rows.
//
// [P2] "SSD 专家卸载 · Prerouter 路由预测", prefill/decode paragraph: prefill
// computes in batches over whole layers.  Per expert group the contraction is
// dense, so it runs on v_mfma_f32_16x16x32_f16 with fp32 accumulation:
//
//   * weights: int4 codes are dequantised into LDS as fp16 w = s*q + b
//     (affine, group 64: [P3] "iPhone、Mac、Android、Windows 实测横评…",
//     "三件套" bullets), one rounding of the exact value (2^-11 relative),
//     so no per-group work remains after the MFMA;
//   * activations: each row enters as fp16(v * 2^-e) with a power-of-two
//     exponent per row chosen so the row's largest magnitude lies in
//     [2^14, 2^15); the epilogue multiplies the row by 2^e.  Rows of x are
//     converted once per token (k_x16), rows of the SwiGLU output h once per
//     row after the gate/up GEMM (k_h16, from an fp32 h and its row maximum);
//   * the unmerged LoRA delta ([P1] Recover-LoRA paragraph) is one extra
//     64-wide K chunk on bf16 MFMA: the activation side holds
//     lambda * (A v) * 2^-e as a bf16 hi + lo pair, the weight side holds B
//     twice.
//
// Tiles of 128 rows x 128 columns, 4 waves of 64 x 64, K chunks of 64 (one
// quantisation group), LDS double-buffered with one barrier per chunk.
// Workgroups are renumbered so that the column tiles of one row tile (which
// share activation rows) and neighbouring row tiles of one expert (which
// share weights) run on the same XCD and its L2.
#include "device_utils.h"
#include "launch.h"
#include "moe_internal.h"
#include "prefill.h"

namespace moe {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Row exponent: the largest magnitude m of a row is scaled into [2^14, 2^15)
// (e may be negative); rows of zeros keep e = 0.
__device__ __forceinline__ int row_exp(float m) {
  if (!(m > 0.f)) return 0;
  return max(min(ilogbf(m) - 14, 126), -100);
}

// ---------------------------------------------------------------------------
// x [T][H] bf16 -> x16 [T][H] fp16 scaled by 2^-ex[t].  One wave per token.
// grid ceil(T / 4), block 256.
__global__ void __launch_bounds__(256) k_x16(const uint16_t* __restrict__ x, int T, int H,
                                             uint16_t* __restrict__ x16, int32_t* __restrict__ ex) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const uint4* src = reinterpret_cast<const uint4*>(x + size_t(t) * H);
  float m = 0.f;
  for (int i = lane; i < H / 8; i += 64) {
    const uint4 v = src[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) m = fmaxf(m, fmaxf(fabsf(bf16_lo(w[k])), fabsf(bf16_hi(w[k]))));
  }
  m = wave_max(m);
  const int e = row_exp(m);
  uint4* dst = reinterpret_cast<uint4*>(x16 + size_t(t) * H);
  for (int i = lane; i < H / 8; i += 64) {
    const uint4 v = src[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f16x2_t p = {_Float16(ldexpf(bf16_lo(w[k]), -e)), _Float16(ldexpf(bf16_hi(w[k]), -e))};
      o[k] = __builtin_bit_cast(uint32_t, p);
    }
    dst[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
  if (lane == 0) ex[t] = e;
}

// h [NR][I] fp32 -> hs16 [NR][I] fp16 scaled by 2^-eh[s], with the row maxima
// hmax[s] (float bits of max |h|) from the gate/up epilogue.  One wave per
// row, grid ceil(NR / 4), block 256.  Rows past `rows` (tiles that were not
// computed) are skipped.
__global__ void __launch_bounds__(256) k_h16(const float* __restrict__ h, const uint32_t* __restrict__ hmax,
                                             const int32_t* __restrict__ nrows, int I,
                                             uint16_t* __restrict__ hs16, int32_t* __restrict__ eh) {
  const int lane = threadIdx.x & 63;
  const int s = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (s >= *nrows) return;
  const int e = row_exp(__uint_as_float(hmax[s]));
  const float4* src = reinterpret_cast<const float4*>(h + size_t(s) * I);
  uint2* dst = reinterpret_cast<uint2*>(hs16 + size_t(s) * I);
  for (int i = lane; i < I / 4; i += 64) {
    const float4 v = src[i];
    f16x2_t a = {_Float16(ldexpf(v.x, -e)), _Float16(ldexpf(v.y, -e))};
    f16x2_t b = {_Float16(ldexpf(v.z, -e)), _Float16(ldexpf(v.w, -e))};
    dst[i] = make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
  }
  if (lane == 0) eh[s] = e;
}

// ---------------------------------------------------------------------------
constexpr int EBM = 128, EBN = 128, EBK = 64;
constexpr int ELDS = EBK + 8;  // fp16 elements per LDS row (144 bytes)

// token of sorted row s
__device__ __forceinline__ int etoken_of(const GemmArgs& a, int s) {
  const int TK = a.T * a.K;
  return s < TK ? a.perm[s] / a.K : s - TK;
}

__device__ __forceinline__ int egroup_of_tile(const int32_t* tstart, int G, int mt) {
  int lo = 0, hi = G;  // tstart[lo] <= mt < tstart[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tstart[mid] <= mt) lo = mid; else hi = mid;
  }
  return lo;
}

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

// Workgroups are dispatched to the 8 XCDs round-robin (XCD = id % 8).  Each
// XCD takes a contiguous run of the active row tiles (a run of experts, so an
// expert's weights stay in one L2), with all column tiles of a row tile
// together (they share the activation rows).  Returns false for workgroups
// past the XCD's run.
__device__ __forceinline__ bool xcd_tile(int bid, int active_mt, int ntn, int& mt, int& nt) {
  const int xcd = bid & 7, slot = bid >> 3;
  const int run = (active_mt + 7) >> 3;
  mt = xcd * run + slot / ntn;
  nt = slot % ntn;
  return slot / ntn < run && mt < active_mt;
}

// Eight int4 codes of one 32-bit word (columns 2s and 2s+1 in the bits
// [4s, 4s+4) and [16+4s, 20+4s)) -> fp16 s*q + b, two per output word.
__device__ __forceinline__ void dequant8_f16(uint32_t w, f16x2_t sc, f16x2_t bi, uint32_t (&o)[4]) {
  const f16x2_t off = {_Float16(1024.0f), _Float16(1024.0f)};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    // 0x6400 is fp16 1024 with a zero mantissa: the code fills the low bits
    const uint32_t c = ((w >> (4 * s)) & 0x000F000Fu) | 0x64006400u;
    const f16x2_t q = __builtin_bit_cast(f16x2_t, c) - off;  // exact
    o[s] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, sc, bi));
  }
}

template <int MODE>
__global__ void __launch_bounds__(256, 2) k_expert_gemm(GemmArgs a, int nblk) {
  static_assert(MODE == kGemmGateUp || MODE == kGemmDown, "expert GEMM modes");
  __shared__ __attribute__((aligned(16))) uint16_t As[2][EBM * ELDS];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][EBN * ELDS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave >> 1) * 64, wn0 = (wave & 1) * 64;

  const int Kdim = (MODE == kGemmGateUp) ? a.H : a.I;
  const int Nrows = (MODE == kGemmGateUp) ? 2 * a.I : a.H;
  const int ntn = (Nrows + EBN - 1) / EBN;
  const int G = a.E + 1;
  int mt, nt;
  if (!xcd_tile(blockIdx.x, a.tstart[G], ntn, mt, nt)) return;
  const int g = egroup_of_tile(a.tstart, G, mt);
  const int row0 = a.gstart[g] + (mt - a.tstart[g]) * EBM;
  const int row_end = min(a.gstart[g + 1], row0 + EBM);
  const int n0 = nt * EBN;
  const uint8_t* blob = reinterpret_cast<const uint8_t*>(a.gblob[g]);

  // Per-row facts of the tile, resolved once (dependent loads of perm and the
  // exponents) into LDS: the activation row (token for gate/up), the output
  // row of y (down) and the row exponent.  Rows past the group end are
  // clamped to its last row: they are computed, not stored.
  __shared__ int row_src[EBM], row_dst[EBM], row_e[EBM];
  if (tid < EBM) {
    const int s = min(row0 + tid, row_end - 1);
    if (MODE == kGemmGateUp) {
      const int t = etoken_of(a, s);
      row_src[tid] = t;
      row_e[tid] = a.ex[t];
    } else {
      const int TK = a.T * a.K, KS = a.K + a.S;
      int dest;
      if (s < TK) {
        const int pr = a.perm[s];
        dest = (pr / a.K) * KS + pr % a.K;
      } else {
        dest = (s - TK) * KS + a.K;
      }
      row_src[tid] = s;
      row_dst[tid] = dest;
      row_e[tid] = a.eh[s];
    }
  }
  __syncthreads();
  // A: 4 segments of 8 elements per thread per chunk (row sidx>>3, seg sidx&7)
  const uint16_t* arow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = row_src[(tid + 256 * i) >> 3];
    arow[i] = (MODE == kGemmGateUp) ? a.x16 + size_t(r) * a.H : a.hs + size_t(r) * a.I;
  }
  const int nchunks = Kdim / EBK;
  const bool lora = a.r > 0;

  // B: one weight row half (32 codes) per thread: row n = tid >> 1, half = tid & 1
  const int bn = tid >> 1, bhalf = tid & 1;
  const int R = min(n0 + bn, Nrows - 1);  // columns past Nrows are computed, not stored
  const uint8_t* bcodes = blob + (MODE == kGemmGateUp ? a.L.gu_codes : a.L.dn_codes) +
                          size_t(R) * (Kdim / 2) + 16 * bhalf;
  const uint32_t* bsb = reinterpret_cast<const uint32_t*>(
      blob + (MODE == kGemmGateUp ? a.L.gu_sb : a.L.dn_sb)) + size_t(R) * (Kdim / 64);

  // The LoRA chunk's operands, loaded first (used after the main loop):
  // A = lambda * (A v) * 2^-e hi/lo pairs of the tile's rows, B = this thread's
  // 32 k values of B row R (gate/up: k = [gate hi 0..15 | gate lo 16..31 | up
  // hi 32..47 | up lo 48..63], a gate row (R & 16 == 0) takes k < 32, an up
  // row k >= 32; down: k = [hi 0..31 | lo 32..63]).
  uint4 la[4], lb[4];
  if (lora) {
    const uint16_t* src = (MODE == kGemmGateUp) ? a.u : a.ud;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = min(row0 + ((tid + 256 * i) >> 3), row_end - 1);
      la[i] = gload16(src + size_t(s) * kLoraK + 8 * ((tid + 256 * i) & 7));
    }
    const uint16_t* Bl = reinterpret_cast<const uint16_t*>(
        blob + (MODE == kGemmGateUp ? a.L.b_gu : a.L.b_dn)) + size_t(R) * a.r;
    uint32_t bv[kMaxR];  // B[R][rr], every load issued (index clamped), selected below
#pragma unroll
    for (int rr = 0; rr < kMaxR; ++rr) bv[rr] = gload<uint16_t>(Bl + min(rr, a.r - 1));
    uint32_t v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      uint32_t pair[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = 32 * bhalf + 2 * q + h;  // compile-time within each bhalf
        const bool ok = (MODE == kGemmGateUp) ? ((k >> 5) == ((R >> 4) & 1)) : true;
        const int rr = (MODE == kGemmGateUp) ? (k & 15) : (k & 31);
        pair[h] = (ok && rr < a.r && rr < kMaxR) ? bv[rr & (kMaxR - 1)] : 0u;
      }
      v[q] = pair[0] | (pair[1] << 16);
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) lb[d] = make_uint4(v[4 * d], v[4 * d + 1], v[4 * d + 2], v[4 * d + 3]);
  }

  // one K chunk of a thread's global data: 4 A segments, 32 codes and the
  // group's scale/bias word; two sets (chunks are fetched two ahead)
  struct Stage {
    uint4 a0, a1, a2, a3, b;
    uint32_t sb;
  };
  Stage st0, st1;
  const int aoff = 8 * (tid & 7);  // (tid + 256 i) & 7 == tid & 7
  auto load = [&](Stage& r, int c) {
    r.a0 = gload16(arow[0] + c * EBK + aoff);
    r.a1 = gload16(arow[1] + c * EBK + aoff);
    r.a2 = gload16(arow[2] + c * EBK + aoff);
    r.a3 = gload16(arow[3] + c * EBK + aoff);
    r.b = gload16(bcodes + c * (EBK / 2));
    r.sb = gload<uint32_t>(bsb + c);
  };
  // A rows of a thread's four segments: (tid >> 3) + 32 i, column 8 (tid & 7)
  const int alds = (tid >> 3) * ELDS + aoff;
  auto store = [&](const Stage& r, int buf) {
    uint16_t* as = As[buf];
    *reinterpret_cast<uint4*>(&as[alds]) = r.a0;
    *reinterpret_cast<uint4*>(&as[alds + 32 * ELDS]) = r.a1;
    *reinterpret_cast<uint4*>(&as[alds + 64 * ELDS]) = r.a2;
    *reinterpret_cast<uint4*>(&as[alds + 96 * ELDS]) = r.a3;
    uint16_t* dst = &Bs[buf][bn * ELDS + 32 * bhalf];
    const f16x2_t sc = {_Float16(bf16_lo(r.sb)), _Float16(bf16_lo(r.sb))};
    const f16x2_t bi = {_Float16(bf16_hi(r.sb)), _Float16(bf16_hi(r.sb))};
    const uint32_t w[4] = {r.b.x, r.b.y, r.b.z, r.b.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t o[4];
      dequant8_f16(w[d], sc, bi, o);
      *reinterpret_cast<uint4*>(dst + 8 * d) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // one 64-wide K chunk from LDS buffer `buf` (fp16, or bf16 for the LoRA chunk)
  auto compute = [&](int buf, bool bf) {
    const uint16_t* as = As[buf];
    const uint16_t* bs = Bs[buf];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const uint4*>(&as[(wm0 + 16 * i + (lane & 15)) * ELDS + 32 * ks + 8 * (lane >> 4)]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *reinterpret_cast<const uint4*>(&bs[(wn0 + 16 * j + (lane & 15)) * ELDS + 32 * ks + 8 * (lane >> 4)]);
      if (!bf) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                __builtin_bit_cast(f16x8_t, af[i]), __builtin_bit_cast(f16x8_t, bfr[j]), acc[i][j], 0, 0, 0);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, af[i]), __builtin_bit_cast(bf16x8_t, bfr[j]), acc[i][j], 0, 0, 0);
      }
    }
  };

  // Pipeline: chunk c is computed from LDS buffer c & 1 while chunk c + 1
  // (fetched during chunk c - 1) is dequantised into the other buffer and
  // chunk c + 2 is fetched into the register set chunk c has freed.
  load(st0, 0);
  if (nchunks > 1) load(st1, 1);
  store(st0, 0);
  __syncthreads();
  for (int c = 0; c < nchunks; c += 2) {
    if (c + 2 < nchunks) load(st0, c + 2);
    compute(0, false);
    if (c + 1 < nchunks) store(st1, 1);
    __syncthreads();
    if (c + 1 >= nchunks) break;
    if (c + 3 < nchunks) load(st1, c + 3);
    compute(1, false);
    if (c + 2 < nchunks) store(st0, 0);
    __syncthreads();
  }
  if (lora) {  // the LoRA chunk (every buffer is free after the last barrier)
    const int buf = 0;
    uint16_t* as = As[buf];
    *reinterpret_cast<uint4*>(&as[alds]) = la[0];
    *reinterpret_cast<uint4*>(&as[alds + 32 * ELDS]) = la[1];
    *reinterpret_cast<uint4*>(&as[alds + 64 * ELDS]) = la[2];
    *reinterpret_cast<uint4*>(&as[alds + 96 * ELDS]) = la[3];
    uint16_t* dst = &Bs[buf][bn * ELDS + 32 * bhalf];
#pragma unroll
    for (int d = 0; d < 4; ++d) *reinterpret_cast<uint4*>(dst + 8 * d) = lb[d];
    __syncthreads();
    compute(buf, true);
  }

  // ---- epilogue: row scale 2^e, then SwiGLU (gate/up) or the y rows (down)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = wm0 + 16 * i + 4 * (lane >> 4) + q;
      const int s = row0 + m;
      const bool valid = s < row_end;
      const int e = row_e[m];
      if (MODE == kGemmGateUp) {
        float hm = 0.f;
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
          const int Rg = n0 + wn0 + 16 * j + (lane & 15);  // gate blob row
          const int jj = ((Rg >> 5) << 4) | (Rg & 15);
          const float g = ldexpf(acc[i][j][q], e);
          // SiLU with the hardware exp and reciprocal (about 1e-6 relative);
          // g -> -inf gives g * 0 = -0
          const float hv = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * ldexpf(acc[i][j + 1][q], e);
          if (valid) a.hf[size_t(s) * a.I + jj] = hv;
          hm = fmaxf(hm, fabsf(hv));
        }
        // the 16 lanes of one row group hold the same row: one atomic per row
        hm = fmaxf(hm, dpp_f<kDppXor1>(hm));
        hm = fmaxf(hm, dpp_f<kDppXor2>(hm));
        hm = fmaxf(hm, dpp_f<kDppHalfMirror>(hm));
        hm = fmaxf(hm, dpp_f<kDppMirror>(hm));
        if (valid && (lane & 15) == 0) atomicMax(&a.hmax[s], __float_as_uint(hm));
      } else {
        const size_t dest = size_t(row_dst[m]);
        if (valid) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int n = n0 + wn0 + 16 * j + (lane & 15);
            if (n < Nrows) a.y[dest * a.H + n] = ldexpf(acc[i][j][q], e);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// enough workgroups for every XCD to take ceil(mtiles / 8) row tiles
int expert_gemm_blocks(int mtiles, int nrows) {
  return 8 * ((mtiles + 7) / 8) * ((nrows + EBN - 1) / EBN);
}

hipError_t launch_x16(const uint16_t* x, int T, int H, uint16_t* x16, int32_t* ex, hipStream_t st) {
  if (T > 0) hipLaunchKernelGGL(k_x16, dim3((T + 3) / 4), dim3(256), 0, st, x, T, H, x16, ex);
  return hipGetLastError();
}

hipError_t launch_h16(const float* h, const uint32_t* hmax, const int32_t* nrows, int NR, int I,
                      uint16_t* hs16, int32_t* eh, hipStream_t st) {
  if (NR > 0) hipLaunchKernelGGL(k_h16, dim3((NR + 3) / 4), dim3(256), 0, st, h, hmax, nrows, I, hs16, eh);
  return hipGetLastError();
}

hipError_t launch_expert_gemm(int mode, const GemmArgs& a, int mtiles, hipStream_t st) {
  const int nrows = (mode == kGemmGateUp) ? 2 * a.I : a.H;
  const int nblk = expert_gemm_blocks(mtiles, nrows);
  if (nblk <= 0) return hipSuccess;
  if (mode == kGemmGateUp)
    hipLaunchKernelGGL(k_expert_gemm<kGemmGateUp>, dim3(nblk), dim3(256), 0, st, a, nblk);
  else
    hipLaunchKernelGGL(k_expert_gemm<kGemmDown>, dim3(nblk), dim3(256), 0, st, a, nblk);
  return hipGetLastError();
}

}  // namespace moe

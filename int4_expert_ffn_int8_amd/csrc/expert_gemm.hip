// Prefill expert GEMMs (gate/up + SwiGLU, down) over each expert's rows.
//
// [P2] "SSD 专家卸载 · Prerouter 路由预测", prefill/decode paragraph: prefill
// computes in batches over whole layers.  Per expert group the contraction is
// dense, so it runs on v_mfma_f32_16x16x32_f16 with fp32 accumulation:
//
//   * weights: the int4 codes and the group scale/bias go through LDS; each
//     wave dequantises its own columns in registers to fp16 w = s*q + b
//     (affine, group 64: [P3] "iPhone、Mac、Android、Windows 实测横评…",
//     "三件套" bullets), one rounding of the exact value (2^-11 relative);
//   * activations: each row enters as fp16(v * 2^-e) with a power-of-two
//     exponent per row chosen so the row's largest magnitude lies in
//     [2^14, 2^15); the epilogue multiplies the row by 2^e.  Rows of x are
//     converted once per token (k_x16_setup, whose last workgroup also does
//     the per-group setup), rows of the SwiGLU output h once per row after
//     the gate/up GEMM, from h stored by the gate/up epilogue as fp16 with
//     one exponent per 16-column block and from its row maximum (by the
//     LoRA-A GEMM of down, which reads every row of h anyway; by k_h16
//     without LoRA): a power-of-two rescale of each block;
//   * the unmerged LoRA delta ([P1] Recover-LoRA paragraph) is one extra
//     64-wide K chunk on bf16 MFMA: the activation side holds
//     lambda * (A v) * 2^-e as a bf16 hi + lo pair, the weight side holds B
//     twice.
//
// Tiles of 128 rows x 256 columns per workgroup of 8 waves (each wave all 128
// rows and 32 columns), K chunks of 64 (one quantisation group) through a
// ring of three LDS stages filled by LDS DMA two chunks ahead; two
// workgroups per CU.  Workgroups are renumbered so that the column tiles of
// one row tile (which share activation rows) and neighbouring row tiles of
// one expert (which share weights) run on the same XCD and its L2.
#include "device_utils.h"
#include "launch.h"
#include "moe_internal.h"
#include "prefill.h"

namespace moe {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));


// ---------------------------------------------------------------------------
// Expert-GEMM setup for the 256 threads of one workgroup: group row starts,
// m-tile starts for tiles of kPrefillBM rows (exclusive scan over the experts
// in order, 4 experts per thread), and each group's blob address (pool lookup
// for routed experts with at least one token; one hit/lookup count each).
__device__ __forceinline__ void expert_setup_block(const X16SetupArgs& a) {
  __shared__ int wsum[4];
  constexpr int EPT = kMaxE / 256;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int tiles[EPT], cnt[EPT], local = 0;
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int e = tid * EPT + k;
    cnt[k] = (e < a.E) ? a.counts[e] : 0;
    tiles[k] = (cnt[k] + kPrefillBM - 1) / kPrefillBM;
    local += tiles[k];
  }
  int inc = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int run = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (w < wave) run += wsum[w];
    total += wsum[w];
  }
  run += inc - local;
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int e = tid * EPT + k;
    if (e < a.E) {
      a.gstart[e] = a.offsets[e];
      a.tstart[e] = run;
      const ExpertSource& src = a.src;
      const uint8_t* b;
      if (src.expert_to_slot == nullptr) {
        b = src.slots + size_t(e) * src.stride;
      } else {
        const int slot = src.expert_to_slot[e];
        if (cnt[k] > 0 && src.counters) {
          atomicAdd(&src.counters[1], 1ull);
          if (slot >= 0) atomicAdd(&src.counters[0], 1ull);
        }
        b = slot >= 0 ? src.slots + size_t(slot) * src.stride : src.host_blobs + size_t(e) * src.stride;
      }
      a.gblob[e] = reinterpret_cast<unsigned long long>(b);
    }
    run += tiles[k];
  }
  if (tid == 0) {
    const int TK = a.T * a.K;
    a.gstart[a.E] = TK;
    a.gstart[a.E + 1] = TK + a.S * a.T;
    a.tstart[a.E] = total;
    a.tstart[a.E + 1] = total + a.S * ((a.T + kPrefillBM - 1) / kPrefillBM);
    a.gblob[a.E] = reinterpret_cast<unsigned long long>(a.shared_blob);
  }
}

// Blocks 0 .. ceil(T/4) - 1: x [T][H] bf16 -> x16 [T][H] fp16 scaled by
// 2^-ex[t], one wave per token, and zeros of the gate/up row maxima of their
// tokens' rows; the last block: the expert-GEMM setup.  block 256.
__global__ void __launch_bounds__(256) k_x16_setup(X16SetupArgs a) {
  const int nx = (a.T + 3) / 4;
  if (int(blockIdx.x) == nx) {
    expert_setup_block(a);
    return;
  }
  const int KS = a.K + a.S, NR = a.T * KS;
  for (int i = threadIdx.x; i < 4 * KS; i += 256) {
    const int r = blockIdx.x * 4 * KS + i;
    if (r < NR) a.hmax[r] = 0u;
  }
  const int H = a.H;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const uint4* src = reinterpret_cast<const uint4*>(a.x + size_t(t) * H);
  float m = 0.f;
  for (int i = lane; i < H / 8; i += 64) {
    const uint4 v = src[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) m = fmaxf(m, fmaxf(fabsf(bf16_lo(w[k])), fabsf(bf16_hi(w[k]))));
  }
  m = wave_max(m);
  const int e = row_exp(m);
  uint4* dst = reinterpret_cast<uint4*>(a.x16 + size_t(t) * H);
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
  if (lane == 0) a.ex[t] = e;
}

// h [NR][I] as fp16(h * 2^-hbe) per 16-column block -> hs16 [NR][I] fp16
// scaled by 2^-eh[s] for the whole row, eh[s] from the row maxima hmax[s]
// (float bits of max |h|) of the gate/up epilogue: a power-of-two rescale of
// each block, exact unless a value becomes subnormal.  One wave per row,
// grid ceil(NR / 4), block 256.  Rows past `rows` (tiles that were not
// computed) are skipped.
__global__ void __launch_bounds__(256) k_h16(const uint16_t* __restrict__ hl, const int8_t* __restrict__ hbe,
                                             const uint32_t* __restrict__ hmax,
                                             const int32_t* __restrict__ nrows, int I,
                                             uint16_t* __restrict__ hs16, int32_t* __restrict__ eh) {
  const int lane = threadIdx.x & 63;
  const int s = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (s >= *nrows) return;
  const int e = row_exp(__uint_as_float(hmax[s]));
  const uint4* src = reinterpret_cast<const uint4*>(hl + size_t(s) * I);
  uint4* dst = reinterpret_cast<uint4*>(hs16 + size_t(s) * I);
  for (int i = lane; i < I / 8; i += 64) {  // 8 columns, within one 16-column block
    const uint4 v = src[i];
    const int d = int(hbe[size_t(s) * (I / 16) + i / 2]) - e;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f16x2_t p = __builtin_bit_cast(f16x2_t, w[k]);
      const f16x2_t r = {_Float16(ldexpf(float(p[0]), d)), _Float16(ldexpf(float(p[1]), d))};
      o[k] = __builtin_bit_cast(uint32_t, r);
    }
    dst[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
  if (lane == 0) eh[s] = e;
}

// ---------------------------------------------------------------------------
constexpr int EBM = 128, EBN = 256, EKC = 64;  // tile rows, tile columns, K per chunk

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

// Buffer resource over [p, p + bytes) in scalar registers (raw buffer:
// stride 0, 32-bit offsets); reads at or past `bytes` return zero.
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t buffer_rsrc(const void* p, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(p);
  return i32x4_t{__builtin_amdgcn_readfirstlane(int32_t(uint32_t(b))),
                 __builtin_amdgcn_readfirstlane(int32_t(uint32_t(b >> 32) & 0xFFFFu)),
                 __builtin_amdgcn_readfirstlane(int32_t(bytes)), 0x00020000};
}
constexpr uint32_t kOobOffset = 0x80000000u;  // an offset past every buffer (sizes < 2^31): reads zero

// 16 / 4 bytes per lane from global memory straight into LDS: lane L of the
// wave writes lds + 16 L (resp. 4 L); completion is counted by vmcnt.  The
// instruction is written out here (M0 saved and restored around it) because
// the compiler's own tracking of such fetches waits for all of them before
// any LDS read; the kernels below wait for them explicitly instead.
__device__ __forceinline__ void dma16(i32x4_t r, const void* lds, uint32_t voff, uint32_t soff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(lds)))), "v"(voff), "s"(r),
        "s"(soff)
      : "memory");
}
__device__ __forceinline__ void dma4(i32x4_t r, const void* lds, uint32_t voff, uint32_t soff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(lds)))), "v"(voff), "s"(r),
        "s"(soff)
      : "memory");
}

// (x & mask) | magic in one VALU op (mask in a VGPR: one scalar operand)
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t vmask, uint32_t magic) {
  uint32_t d;
  asm volatile("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(x), "v"(vmask), "s"(magic));
  return d;
}

// Eight int4 codes of one 32-bit word (columns 2s and 2s+1 in the bits
// [4s, 4s+4) and [16+4s, 20+4s)) -> fp16 s*q + b, two per output word.  A
// code in bits 0..3 of a half fills the low mantissa bits of fp16 1024
// (0x6400, unit 1); a code in bits 4..7 those of fp16 64 (0x5400, unit 1/16),
// so one shift by 8 serves all four positions.  The offset (1024 or 64) is
// subtracted exactly and one fused multiply-add applies the group's scale and
// bias.  m0 = 0x000F000F and m1 = 0x00F000F0 (in VGPRs).
__device__ __forceinline__ f16x8_t dequant8_fast(uint32_t w, uint32_t m0, uint32_t m1, f16x2_t sc,
                                                 f16x2_t bi) {
  const f16x2_t off0 = {_Float16(1024.0f), _Float16(1024.0f)};
  const f16x2_t off1 = {_Float16(64.0f), _Float16(64.0f)};
  const uint32_t w8 = w >> 8;
  const uint32_t c[4] = {and_or(w, m0, 0x64006400u), and_or(w, m1, 0x54005400u),
                         and_or(w8, m0, 0x64006400u), and_or(w8, m1, 0x54005400u)};
  u32x4_t o;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const f16x2_t q = __builtin_bit_cast(f16x2_t, c[s]) - ((s & 1) ? off1 : off0);  // exact
    o[s] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, sc, bi));
  }
  return __builtin_bit_cast(f16x8_t, o);
}

// LDS stage of the ring, one K chunk of 64 (one quantisation group):
//   A      [128 rows][128 B]: 16-byte slot p of row r holds k-segment
//          p ^ ((r >> 1) & 7) (8 fp16 each);
//   codes  [256 rows][32 B]:  8-byte unit p of row r holds the 16 codes
//          k = 16 (p ^ 2 ((r >> 3) & 1)) + 0..15;
//   scale/bias [256 rows] words.
// The XOR swizzles make the MFMA operand reads of every 16 lanes hit
// distinct LDS banks.
constexpr int kStA = 0, kStB = EBM * 128, kStS = kStB + EBN * 32, kStage = kStS + EBN * 4;

// Grouped expert GEMM, one 128-row x 256-column tile per workgroup of 8
// waves; wave w owns all 128 rows and columns 32 w .. 32 w + 31 (8 x 2
// blocks of 16 x 16), so each weight is dequantised once per tile.  Two
// workgroups share a CU (four waves per SIMD) to cover LDS and barrier
// latency with the other waves' MFMAs.
template <int MODE>
__global__ void __launch_bounds__(512, 4) k_expert_gemm(GemmArgs a, int nblk) {
  static_assert(MODE == kGemmGateUp || MODE == kGemmDown, "expert GEMM modes");
  constexpr int IM = EBM / 16;      // 16-row blocks per wave
  constexpr int JN = EBN / 8 / 16;  // 16-column blocks per wave
  __shared__ __attribute__((aligned(1024))) uint8_t S0[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t S1[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t S2[kStage];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 15, lq = lane >> 4;
  const int wn0 = wave * (EBN / 8);

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

  // Per-row facts of the tile, resolved once into LDS: the activation row
  // (token for gate/up), the output row of y (down) and the row exponent.
  // Rows past the group end are clamped to its last row: computed, not stored.
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

  __syncthreads();  // row tables

  // ---- global -> LDS fetch of one K chunk: A 2 and codes 1 DMA instruction
  // per thread, scale/bias 1 per thread of waves 0..3; each wave instruction
  // writes 1 KB (256 B) of contiguous LDS.
  const i32x4_t ra = buffer_rsrc(
      (MODE == kGemmGateUp) ? (const void*)a.x16 : (const void*)a.hs,
      uint32_t((MODE == kGemmGateUp) ? size_t(a.T) * a.H * 2 : size_t(a.gstart[G]) * a.I * 2));
  const i32x4_t rb = buffer_rsrc(blob, uint32_t(a.L.total));
  uint32_t aoff[2], boff, soff;
#pragma unroll
  for (int u = 0; u < 2; ++u) {  // A: LDS slot (8 u + wave) * 64 + lane
    const int idx = (8 * u + wave) * 64 + lane, r = idx >> 3;
    const int seg = (idx & 7) ^ ((r >> 1) & 7);
    aoff[u] = uint32_t(row_src[r]) * uint32_t(Kdim) * 2u + 16u * seg;
  }
  {  // codes: LDS 16-byte slot wave * 64 + lane = row r, half h (units 2h, 2h + 1)
    const int idx = wave * 64 + lane, r = idx >> 1, h = idx & 1;
    const int R = min(n0 + r, Nrows - 1);  // columns past Nrows: computed, not stored
    boff = uint32_t(((MODE == kGemmGateUp) ? a.L.gu_codes : a.L.dn_codes) + size_t(R) * (Kdim / 2)) +
           16u * (h ^ ((r >> 3) & 1));
  }
  {  // scale/bias: LDS word wave * 64 + lane = row r (waves 0..3)
    const int R = min(n0 + (wave & 3) * 64 + lane, Nrows - 1);
    soff = uint32_t(((MODE == kGemmGateUp) ? a.L.gu_sb : a.L.dn_sb) + size_t(R) * (Kdim / 64) * 4);
  }
  const int nchunks = Kdim / EKC;
  const int clast = nchunks - 1;
  auto fetch = [&](uint8_t* st, int c) {
    dma16(ra, st + kStA + wave * 1024, aoff[0], c * (EKC * 2));
    dma16(ra, st + kStA + (8 + wave) * 1024, aoff[1], c * (EKC * 2));
    dma16(rb, st + kStB + wave * 1024, boff, c * (EKC / 2));
    if (wave < 4) dma4(rb, st + kStS + wave * 256, soff, c * 4);
  };
  // wait for this wave's fetches of the chunk before the newest one
  auto wait_prev = [&]() {
    if (wave < 4)
      __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
    else
      __builtin_amdgcn_s_waitcnt(0x0F73);  // vmcnt(3)
  };

  f32x4_t acc[IM][JN];
#pragma unroll
  for (int i = 0; i < IM; ++i)
#pragma unroll
    for (int j = 0; j < JN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const uint32_t m0 = 0x000F000Fu, m1 = 0x00F000F0u;
  // one chunk from stage st: 2 MFMA steps of 32 k.  Lane (ln, lq) takes the
  // codes k = 16 lq + 0..15 of its columns, step t their codes 8 t .. 8 t + 7;
  // the activation side reads the same k (segment 2 lq + t).
  const int bslot = 8 * (lq ^ (2 * (ln >> 3)));
  const int abase = ln * 128;
  const int aswz = (ln >> 1) & 7;
  auto compute = [&](const uint8_t* st) {
    uint2 q[JN];
    f16x2_t sc[JN], bi[JN];
#pragma unroll
    for (int j = 0; j < JN; ++j) {
      const int r = wn0 + 16 * j + ln;
      q[j] = *reinterpret_cast<const uint2*>(st + kStB + r * 32 + bslot);
      const uint32_t sw = *reinterpret_cast<const uint32_t*>(st + kStS + r * 4);
      sc[j] = f16x2_t{_Float16(bf16_lo(sw)), _Float16(bf16_lo(sw))};
      bi[j] = f16x2_t{_Float16(bf16_hi(sw)), _Float16(bf16_hi(sw))};
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f16x8_t bf[JN];
#pragma unroll
      for (int j = 0; j < JN; ++j) bf[j] = dequant8_fast(t ? q[j].y : q[j].x, m0, m1, sc[j], bi[j]);
      const uint8_t* as = st + kStA + abase + 16 * ((2 * lq + t) ^ aswz);
#pragma unroll
      for (int i = 0; i < IM; ++i) {
        const f16x8_t af = *reinterpret_cast<const f16x8_t*>(as + i * 16 * 128);
#pragma unroll
        for (int j = 0; j < JN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[j], acc[i][j], 0, 0, 0);
      }
    }
  };

  // Pipeline over a ring of three LDS stages: chunk c lives in stage c % 3.
  // Each step waits for its own fetches of chunk c (those of chunk c + 1 stay
  // in flight), meets the other waves at the barrier (after which chunk c is
  // complete in LDS and stage (c + 2) % 3 is no longer read), starts the
  // fetch of chunk c + 2 into that stage and computes chunk c.  The loop body
  // covers three chunks so each stage is a distinct array; fetch indices are
  // clamped and a step past the end skips its MFMAs, so the body has no exit.
  fetch(S0, 0);
  fetch(S1, min(1, clast));
#define MOE_STEP(CUR, NXT, I)                 \
  wait_prev();                                \
  __syncthreads();                            \
  fetch(NXT, min(c + (I) + 2, clast));        \
  if (c + (I) < nchunks) compute(CUR);
  for (int c = 0; c < nchunks; c += 3) {
    MOE_STEP(S0, S2, 0)
    MOE_STEP(S1, S0, 1)
    MOE_STEP(S2, S1, 2)
  }
#undef MOE_STEP
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no fetch still writes LDS
  __syncthreads();

  if (a.r > 0) {  // the LoRA chunk, in stage 0's A layout
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 512 * i, m = idx >> 3, sg = idx & 7;
      const int s = min(row0 + m, row_end - 1);
      u32x4_t seg;
      if (MODE == kGemmGateUp) {
        // lambda * (A v) * 2^-ex from the LoRA-A GEMM's K-split partials,
        // summed in split order: segment sg holds [gate hi | gate lo | up hi
        // | up lo] entries 8 (sg & 1) .. + 7 of its quarter
        const int NR = a.gstart[a.E + 1];
        const int j0 = (sg >= 4 ? 16 : 0) + 8 * (sg & 1);
        float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int k = 0; k < kLoraSplit; ++k) {
          const f32x4_t* src = reinterpret_cast<const f32x4_t*>(a.upart + (size_t(k) * NR + s) * 32 + j0);
          const f32x4_t p0 = gload<f32x4_t>(src), p1 = gload<f32x4_t>(src + 1);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v[q] += p0[q];
            v[4 + q] += p1[q];
          }
        }
        const bool lo_part = (sg >> 1) & 1;
        uint32_t hb[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float lv = (8 * (sg & 1) + q < a.r) ? ldexpf(a.lam * v[q], -row_e[m]) : 0.f;
          const uint16_t hi = f32_to_bf16(lv);
          hb[q] = lo_part ? f32_to_bf16(lv - bf16_to_f32(hi)) : hi;
        }
        seg = u32x4_t{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16), hb[4] | (hb[5] << 16), hb[6] | (hb[7] << 16)};
      } else {
        seg = gload<u32x4_t>(a.ud + size_t(s) * kLoraK + 8 * sg);
      }
      *reinterpret_cast<u32x4_t*>(S0 + kStA + m * 128 + 16 * (sg ^ ((m >> 1) & 7))) = seg;
    }
    __syncthreads();
    // Weight side: B[R][rr] as bf16 for the k the lane covers.  Activation
    // side u: gate/up k = [gate hi 0..15 | gate lo 16..31 | up hi 32..47 |
    // up lo 48..63], so a gate column block (j even) meets step 0 only and an
    // up block (j odd) step 1 only, with rank rr = 8 (lq & 1) + e; down
    // k = [hi 0..31 | lo 32..63], both steps, rr = 8 lq + e.
    const uint16_t* Bl = reinterpret_cast<const uint16_t*>(
        blob + (MODE == kGemmGateUp ? a.L.b_gu : a.L.b_dn));
    const int rr0 = (MODE == kGemmGateUp) ? 8 * (lq & 1) : 8 * lq;
    bf16x8_t bw[JN];
#pragma unroll
    for (int j = 0; j < JN; ++j) {
      const int R = min(n0 + wn0 + 16 * j + ln, Nrows - 1);
      u32x4_t bw4;
      if (a.r == kMaxR) {  // whole rows of 16: one 16-byte load (zero past the rank)
        const u32x4_t v = gload<u32x4_t>(Bl + size_t(R) * kMaxR + min(rr0, kMaxR - 8));
        bw4 = (rr0 < kMaxR) ? v : u32x4_t{0u, 0u, 0u, 0u};
      } else {
        uint32_t v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = gload<uint16_t>(Bl + size_t(R) * a.r + min(rr0 + e, a.r - 1));
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const uint32_t lo = (rr0 + e < a.r) ? v[e] : 0u;
          const uint32_t hi = (rr0 + e + 1 < a.r) ? v[e + 1] : 0u;
          bw4[e >> 1] = lo | (hi << 16);
        }
      }
      bw[j] = __builtin_bit_cast(bf16x8_t, bw4);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint8_t* as = S0 + kStA + abase + 16 * ((4 * t + lq) ^ aswz);
#pragma unroll
      for (int i = 0; i < IM; ++i) {
        const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(as + i * 16 * 128);
#pragma unroll
        for (int j = 0; j < JN; ++j) {
          if (MODE == kGemmGateUp && (j & 1) != t) continue;
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bw[j], acc[i][j], 0, 0, 0);
        }
      }
    }
  }

  // Compact y (down): fp16(acc * 2^-yc), with yc from the blob's bound on the
  // down outputs: |acc| <= (W + |lambda| L) 2^15 since every row of h enters
  // scaled to |h| <= 2^15, so acc * 2^-yc stays below 2^15 whatever the data.
  float yscale = 1.0f;
  int yc = 0;
  if (MODE == kGemmDown && a.y16 != nullptr) {
    const float* meta = reinterpret_cast<const float*>(blob + a.L.meta);
    const float bound = gload<float>(meta + kMetaDownW) + fabsf(a.lam) * gload<float>(meta + kMetaDownL);
    // (c >= -126 keeps 2^-c finite; a smaller bound still gives |acc| 2^-c < 2^15)
    yc = !(bound > 0.f) ? 0 : (bound <= 3.0e38f ? max(min(ilogbf(bound) + 1, 127), -126) : 127);
    yscale = ldexpf(1.0f, -yc);
  }

  // ---- epilogue: row scale 2^e, then SwiGLU (gate/up) or the y rows (down)
#pragma unroll
  for (int i = 0; i < IM; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = 16 * i + 4 * lq + q;
      const int s = row0 + m;
      const bool valid = s < row_end;
      const int e = row_e[m];
      if (MODE == kGemmGateUp) {
        // the wave's gate/up columns 0..15 / 16..31 give the 16 h columns
        // of one block (lane ln: column jj), stored as fp16(h * 2^-eb) with
        // eb from the block's largest |h|; the row maximum over all blocks
        // (an atomic per row) sets the exponent the down GEMM uses
        static_assert(JN == 2, "one gate and one up column block per wave");
        const int Rg = n0 + wn0 + ln;  // gate blob row
        const int jj = ((Rg >> 5) << 4) | (Rg & 15);
        const float gv = ldexpf(acc[i][0][q], e);
        // SiLU with the hardware exp and reciprocal (about 1e-6 relative);
        // g -> -inf gives g * 0 = -0
        const float hv = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * ldexpf(acc[i][1][q], e);
        float hm = Rg < Nrows ? fabsf(hv) : 0.f;
        // the 16 lanes of one row group hold the same row
        hm = fmaxf(hm, dpp_f<kDppXor1>(hm));
        hm = fmaxf(hm, dpp_f<kDppXor2>(hm));
        hm = fmaxf(hm, dpp_f<kDppHalfMirror>(hm));
        hm = fmaxf(hm, dpp_f<kDppMirror>(hm));
        const int eb = row_exp(hm);
        if (valid && Rg < Nrows) {
          a.hl[size_t(s) * a.I + jj] = __builtin_bit_cast(uint16_t, _Float16(ldexpf(hv, -eb)));
          if (ln == 0) {
            a.hbe[size_t(s) * (a.I / 16) + (jj >> 4)] = int8_t(eb);
            atomicMax(&a.hmax[s], __float_as_uint(hm));
          }
        }
      } else if (a.y16 == nullptr) {
        const size_t dest = size_t(row_dst[m]);
        if (valid) {
#pragma unroll
          for (int j = 0; j < JN; ++j) {
            const int n = n0 + wn0 + 16 * j + ln;
            if (n < Nrows) a.y[dest * a.H + n] = ldexpf(acc[i][j][q], e);
          }
        }
      } else {
        // Lane ln holds columns ln (j = 0) and 16 + ln (j = 1) of its row;
        // neighbouring lanes swap one value so that an even lane stores
        // columns ln, ln + 1 and an odd lane columns 15 + ln, 16 + ln: one
        // 4-byte store per lane, 64 contiguous bytes per row.
        static_assert(JN == 2, "the pairing below covers two 16-column blocks");
        const size_t dest = size_t(row_dst[m]);
        const float v0 = acc[i][0][q] * yscale, v1 = acc[i][1][q] * yscale;
        const float o0 = dpp_f<kDppXor1>(v0), o1 = dpp_f<kDppXor1>(v1);
        const bool odd = ln & 1;
        const f16x2_t pv = {_Float16(odd ? o1 : v0), _Float16(odd ? v1 : o0)};
        const int n = n0 + wn0 + (odd ? 15 + ln : ln);
        if (valid && n < Nrows)  // n is even and Nrows a multiple of 64: n + 1 < Nrows too
          *reinterpret_cast<uint32_t*>(a.y16 + dest * a.H + n) = __builtin_bit_cast(uint32_t, pv);
        if (valid && nt == 0 && wave == 0 && ln == 0) a.ey[dest] = e + yc;  // one writer per row
      }
    }
  }
}

// ---------------------------------------------------------------------------
// enough workgroups for every XCD to take ceil(mtiles / 8) row tiles
int expert_gemm_blocks(int mtiles, int nrows) {
  return 8 * ((mtiles + 7) / 8) * ((nrows + EBN - 1) / EBN);
}

hipError_t launch_x16_setup(const X16SetupArgs& a, hipStream_t st) {
  if (a.E > kMaxE) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_x16_setup, dim3((a.T + 3) / 4 + 1), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_h16(const uint16_t* hl, const int8_t* hbe, const uint32_t* hmax, const int32_t* nrows,
                      int NR, int I, uint16_t* hs16, int32_t* eh, hipStream_t st) {
  if (NR > 0)
    hipLaunchKernelGGL(k_h16, dim3((NR + 3) / 4), dim3(256), 0, st, hl, hbe, hmax, nrows, I, hs16, eh);
  return hipGetLastError();
}

hipError_t launch_expert_gemm(int mode, const GemmArgs& a, int mtiles, hipStream_t st) {
  const int nrows = (mode == kGemmGateUp) ? 2 * a.I : a.H;
  const int nblk = expert_gemm_blocks(mtiles, nrows);
  if (nblk <= 0) return hipSuccess;
  // buffer offsets are 32-bit: activations, weights of one expert
  const size_t NR = size_t(a.T) * (a.K + a.S);
  if (size_t(a.T) * a.H * 2 > 0x7FFFFFFFu || NR * a.I * 2 > 0x7FFFFFFFu || a.L.total > 0x7FFFFFFFu)
    return hipErrorInvalidValue;
  if (mode == kGemmGateUp)
    hipLaunchKernelGGL(k_expert_gemm<kGemmGateUp>, dim3(nblk), dim3(512), 0, st, a, nblk);
  else
    hipLaunchKernelGGL(k_expert_gemm<kGemmDown>, dim3(nblk), dim3(512), 0, st, a, nblk);
  return hipGetLastError();
}

}  // namespace moe

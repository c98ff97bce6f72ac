// Host-side packer: logical expert tensors -> one fixed-stride expert blob.
//
// [P5] "iPhone 也能跑 35B 大模型？…" (sheratonhq.com), iPhone section: the
// release layout needed several scattered reads per expert and was repacked
// so one expert is one sequential read.  The blob below is that idea for HBM:
// one contiguous block per expert, which is also one expert-pool slot.
#include <math.h>
#include <string.h>

#include "moe_internal.h"
#include "status.h"

using namespace moe;

namespace {

// Pack one row of `n` codes into n/8 little-endian words with the nibble
// order described in moe_internal.h.
bool pack_code_row(const uint8_t* q, int n, uint8_t* dst) {
  for (int w = 0; w < n / 8; ++w) {
    uint32_t word = 0;
    for (int s = 0; s < 4; ++s) {
      uint32_t c0 = q[8 * w + 2 * s], c1 = q[8 * w + 2 * s + 1];
      if (c0 > 15 || c1 > 15) return false;
      word |= c0 << (4 * s);
      word |= c1 << (16 + 4 * s);
    }
    memcpy(dst + 4 * size_t(w), &word, 4);
  }
  return true;
}

float bf16_value(uint16_t v) {
  const uint32_t u = uint32_t(v) << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

// The prefill GEMMs dequantise in fp16 (w = fp16(s q + b)), so every weight a
// group can hold, and its scale and bias, must lie within fp16's finite range.
constexpr float kF16Max = 65504.0f;
bool group_fits_f16(uint16_t s, uint16_t b) {
  const double sv = bf16_value(s), bv = bf16_value(b);
  const double far = fabs(15.0 * sv + bv);
  return fabs(sv) <= kF16Max && fabs(bv) <= kF16Max && far <= kF16Max;  // false for NaN / inf
}

bool pack_sb_row(const uint16_t* s, const uint16_t* b, int groups, uint8_t* dst) {
  for (int g = 0; g < groups; ++g) {
    if (!group_fits_f16(s[g], b[g])) return false;
    uint32_t word = uint32_t(s[g]) | (uint32_t(b[g]) << 16);
    memcpy(dst + 4 * size_t(g), &word, 4);
  }
  return true;
}

}  // namespace

extern "C" size_t moe_expert_blob_bytes(int32_t H, int32_t I, int32_t r) {
  if (H <= 0 || I <= 0 || r < 0 || H % kGroup || I % kGroup) return 0;
  return blob_layout(H, I, r).total;
}

extern "C" moe_status_t moe_pack_expert(
    int32_t H, int32_t I, int32_t r, const uint8_t* q_gate, const uint16_t* s_gate,
    const uint16_t* b_gate, const uint16_t* A_gate, const uint16_t* B_gate, const uint8_t* q_up,
    const uint16_t* s_up, const uint16_t* b_up, const uint16_t* A_up, const uint16_t* B_up,
    const uint8_t* q_down, const uint16_t* s_down, const uint16_t* b_down, const uint16_t* A_down,
    const uint16_t* B_down, void* blob_out, size_t blob_bytes) {
  if (H <= 0 || I <= 0 || H % kGroup || I % kGroup)
    return fail(MOE_EINVAL, "moe_pack_expert: H=%d, I=%d must be positive multiples of 64", H, I);
  if (r < 0 || r > kMaxR) return fail(MOE_EINVAL, "moe_pack_expert: r=%d outside [0, %d]", r, kMaxR);
  if (!q_gate || !s_gate || !b_gate || !q_up || !s_up || !b_up || !q_down || !s_down || !b_down ||
      !blob_out)
    return fail(MOE_EINVAL, "moe_pack_expert: null code/scale/bias/output pointer");
  if (r > 0 && (!A_gate || !B_gate || !A_up || !B_up || !A_down || !B_down))
    return fail(MOE_EINVAL, "moe_pack_expert: r=%d needs all six LoRA factors", r);
  const BlobLayout L = blob_layout(H, I, r);
  if (blob_bytes < L.total)
    return fail(MOE_EINVAL, "moe_pack_expert: blob_bytes=%zu < %zu", blob_bytes, L.total);
  uint8_t* out = static_cast<uint8_t*>(blob_out);
  memset(out, 0, L.total);
  const int Gh = H / kGroup, Gi = I / kGroup;
  for (int j = 0; j < I; ++j) {
    const int rg = gu_row_gate(j), ru = gu_row_up(j);
    if (!pack_code_row(q_gate + size_t(j) * H, H, out + L.gu_codes + size_t(rg) * (H / 2)) ||
        !pack_code_row(q_up + size_t(j) * H, H, out + L.gu_codes + size_t(ru) * (H / 2)))
      return fail(MOE_EINVAL, "moe_pack_expert: gate/up code above 15 in output row %d", j);
    if (!pack_sb_row(s_gate + size_t(j) * Gh, b_gate + size_t(j) * Gh, Gh,
                     out + L.gu_sb + size_t(rg) * Gh * 4) ||
        !pack_sb_row(s_up + size_t(j) * Gh, b_up + size_t(j) * Gh, Gh,
                     out + L.gu_sb + size_t(ru) * Gh * 4))
      return fail(MOE_EUNSUPPORTED, "moe_pack_expert: gate/up output row %d has a group whose "
                  "scale, bias or 15 * scale + bias is outside the fp16 range (or not finite)", j);
    if (r > 0) {
      memcpy(out + L.b_gu + size_t(rg) * r * 2, B_gate + size_t(j) * r, size_t(r) * 2);
      memcpy(out + L.b_gu + size_t(ru) * r * 2, B_up + size_t(j) * r, size_t(r) * 2);
    }
  }
  for (int i = 0; i < H; ++i) {
    if (!pack_code_row(q_down + size_t(i) * I, I, out + L.dn_codes + size_t(i) * (I / 2)))
      return fail(MOE_EINVAL, "moe_pack_expert: down code above 15 in output row %d", i);
    if (!pack_sb_row(s_down + size_t(i) * Gi, b_down + size_t(i) * Gi, Gi,
                     out + L.dn_sb + size_t(i) * Gi * 4))
      return fail(MOE_EUNSUPPORTED, "moe_pack_expert: down output row %d has a group whose "
                  "scale, bias or 15 * scale + bias is outside the fp16 range (or not finite)", i);
  }
  if (r > 0) {
    memcpy(out + L.a_gu, A_gate, size_t(r) * H * 2);
    memcpy(out + L.a_gu + size_t(r) * H * 2, A_up, size_t(r) * H * 2);
    memcpy(out + L.a_dn, A_down, size_t(r) * I * 2);
    memcpy(out + L.b_dn, B_down, size_t(H) * r * 2);
  }
  // bounds of the down projection's output (moe_internal.h, kMetaDown*)
  double wmax = 0.0, lmax = 0.0;
  for (int i = 0; i < H; ++i) {
    double sum = 0.0;
    for (int j = 0; j < I; ++j) {
      const size_t gidx = size_t(i) * Gi + j / kGroup;
      sum += fabs(bf16_value(s_down[gidx]) * double(q_down[size_t(i) * I + j]) + bf16_value(b_down[gidx]));
    }
    wmax = fmax(wmax, sum);
  }
  if (r > 0) {
    double arow[kMaxR];
    for (int k = 0; k < r; ++k) {
      arow[k] = 0.0;
      for (int j = 0; j < I; ++j) arow[k] += fabs(double(bf16_value(A_down[size_t(k) * I + j])));
    }
    for (int i = 0; i < H; ++i) {
      double sum = 0.0;
      for (int k = 0; k < r; ++k) sum += fabs(double(bf16_value(B_down[size_t(i) * r + k]))) * arow[k];
      lmax = fmax(lmax, sum);
    }
  }
  const float meta[2] = {float(wmax) * (1.0f + 1e-6f), float(lmax) * (1.0f + 1e-6f)};
  memcpy(out + L.meta, meta, sizeof(meta));
  return MOE_OK;
}

// moe_block_decode_noalloc: the fused decode block with a library-owned
// workspace, for callers that cannot allocate device memory.
//
// The workspace is a file-scope device array.  In host code its name is only
// a host-side stand-in, so its device address is looked up once per device
// (with that device current) and kept; kernels and the zeroing launch get
// that address, never the name.
#include <mutex>

#include "../../include/moe.h"
#include "fused.h"
#include "status.h"

namespace moe {
namespace {

constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's scratch; on the first call for a
// device it is looked up and the array is zeroed on `st` (a kernel, so a
// captured first call stays valid: every hand-off word reads as stale).
moe_status_t device_scratch(const char* fn, void** out, hipStream_t st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_EHIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_EUNSUPPORTED, "%s: device %d beyond %d", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(MOE_EHIP, "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(e));
    e = launch_zero_ints(static_cast<int*>(p), int(kScratchBytes / 4), st);
    if (e != hipSuccess)
      return fail(MOE_EHIP, "%s: zeroing the scratch: %s", fn, hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" moe_status_t moe_block_decode_noalloc(const moe_dims_t* d, const int8_t* gate_q,
                                                 const float* gate_s, const int8_t* sgate_q,
                                                 const float* sgate_s,
                                                 const moe_experts_t* routed,
                                                 const void* shared_blob, const uint16_t* h_in,
                                                 int32_t T, int32_t flags, float eps,
                                                 int32_t* topk_idx, float* topk_w, uint16_t* out,
                                                 int32_t* error_out, void* stream) {
  using namespace moe;
  const char* fn = "moe_block_decode_noalloc";
  moe_status_t st = block_decode_check(fn, d, gate_q, gate_s, sgate_q, sgate_s, routed,
                                       shared_blob, h_in, T, flags, eps, out);
  if (st != MOE_OK || T == 0) return st;
  const FusedWs W = fused_ws_layout(T, d->E, d->K, d->n_shared, d->I, d->r);
  if (W.total > kScratchBytes)
    return fail(MOE_EUNSUPPORTED, "%s: workspace of %zu bytes exceeds the %zu-byte scratch", fn,
                W.total, kScratchBytes);
  void* ws = nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = device_scratch(fn, &ws, s);
  if (st != MOE_OK) return st;
  return block_decode_launch(fn, d, gate_q, gate_s, sgate_q, sgate_s, routed, shared_blob, h_in, T,
                             flags, eps, nullptr, topk_idx, topk_w, out, ws, kScratchBytes,
                             error_out, stream);
}

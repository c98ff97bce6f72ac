// Cross-workgroup hand-off words for single-launch kernels.
//
// The 8 XCDs of the chip have separate L2 caches, and a device-scope
// release/acquire fence writes back / invalidates a whole L2.  Values one
// workgroup hands to another inside a launch are therefore 64-bit words --
// payload bits in the low half, the launch's tag in the high half -- written
// and read with device-scope relaxed atomics, which are served at the memory
// side and bypass the XCD L2s.  A producer just stores; a consumer loads the
// words it needs and repeats the loads until all of them carry this launch's
// tag.  The tag is a per-workspace launch epoch + 1 that the last workgroup of
// every launch bumps, so words left by earlier launches never look valid and
// nothing needs clearing between launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// tag in the high 32 bits, payload bits in the low 32
typedef unsigned long long tword_t;

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

// the tag of the launch that reads epoch word *ep (epoch + 1, never 0)
__device__ __forceinline__ unsigned epoch_tag(const int* ep) {
  return (unsigned(ld_dev(ep)) % 0x7FFFFFFFu) + 1u;
}
__device__ __forceinline__ tword_t tw(unsigned tag, uint32_t bits) {
  return (tword_t(tag) << 32) | bits;
}
__device__ __forceinline__ tword_t twf(unsigned tag, float v) { return tw(tag, __float_as_uint(v)); }
__device__ __forceinline__ bool has_tag(tword_t w, unsigned tag) { return unsigned(w >> 32) == tag; }
__device__ __forceinline__ float wf(tword_t w) { return __uint_as_float(uint32_t(w)); }

// Launch counter without a returning atomic.  *ctr (64-bit, zero before the
// first launch) grows by exactly 2^32 per launch: one thread of each of the
// launch's `total` workgroups reads it once (counter_read) and then adds the
// workgroup's share (counter_arrive).  A workgroup reads before its own add,
// so every read of a launch returns a value in [n 2^32, (n + 1) 2^32) and the
// whole launch derives the same tag from n (counter_tag), whatever the order
// in which its workgroups run; launches of different grid sizes may share the
// counter.  The adds are fire-and-forget: no workgroup waits for them.  A
// second read after the add could see the next launch's epoch, so the reading
// thread hands the tag to the rest of its workgroup (through LDS).
__device__ __forceinline__ unsigned long long counter_read(const unsigned long long* ctr) {
  return ld_dev(ctr);
}
__device__ __forceinline__ unsigned counter_tag(unsigned long long c) {
  return unsigned((c >> 32) % 0x7FFFFFFFull) + 1u;
}
__device__ __forceinline__ void counter_arrive(unsigned long long* ctr, unsigned long long c, int wg,
                                               int total) {
  const unsigned long long q = (1ull << 32) / unsigned(total);
  unsigned long long share = wg == 0 ? (1ull << 32) - q * unsigned(total - 1) : q;
  // c never reaches 2^64 - 1, so this changes nothing but makes the add wait
  // for the read's value: the read is performed first
  share ^= (unsigned long long)(c == ~0ull);
  __hip_atomic_fetch_add(ctr, share, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// End of a workgroup's part of the launch (call after its last hand-off store,
// from every thread): the last of `total` workgroups to arrive resets the
// arrival counter *done and starts the next epoch *ep.  Returns true in thread
// 0 of that last workgroup, whose caller may then act on state every other
// workgroup has finished with.
__device__ __forceinline__ bool finish_launch(int* ep, int* done, int total) {
  __syncthreads();
  if (threadIdx.x == 0 && add_dev(done, 1) == total - 1) {
    const int e = ld_dev(ep);
    st_dev(done, 0);
    st_dev(ep, e + 1);
    return true;
  }
  return false;
}

}  // namespace moe

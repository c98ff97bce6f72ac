// Cross-workgroup hand-off words for single-launch kernels.
//
// The 8 XCDs of the chip have separate L2 caches, and a device-scope
// release/acquire fence writes back / invalidates a whole L2.  Values one
// workgroup hands to another inside a launch are therefore 64-bit words --
// payload bits in the low half, the launch's tag in the high half -- written
// and read with device-scope relaxed atomics, which are served at the memory
// side and bypass the XCD L2s.  A producer just stores; a consumer loads the
// words it needs and repeats the loads until all of them carry this launch's
// tag.  The tag comes from a per-workspace launch counter (below) that grows
// by a fixed amount per launch, so words left by earlier launches never look
// valid and nothing needs clearing between launches.
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

__device__ __forceinline__ tword_t tw(unsigned tag, uint32_t bits) {
  return (tword_t(tag) << 32) | bits;
}
__device__ __forceinline__ tword_t twf(unsigned tag, float v) { return tw(tag, __float_as_uint(v)); }
__device__ __forceinline__ bool has_tag(tword_t w, unsigned tag) { return unsigned(w >> 32) == tag; }
__device__ __forceinline__ float wf(tword_t w) { return __uint_as_float(uint32_t(w)); }

// Launch counter without a returning atomic.  *ctr (64-bit, zero before the
// first launch) grows by exactly 2^32 per launch: each of the launch's `total`
// workgroups adds its share once (counter_arrive), after the last read of the
// counter by any of its threads.  Every read of a launch then returns a value
// in [n 2^32, (n + 1) 2^32) -- the other workgroups' shares sum to less than
// 2^32 -- and the whole launch derives the same tag from n (counter_tag),
// whatever the order in which its workgroups run; launches of different grid
// sizes may share the counter.  The adds are fire-and-forget: no workgroup
// waits for them.
__device__ __forceinline__ unsigned long long counter_read(const unsigned long long* ctr) {
  return ld_dev(ctr);
}
__device__ __forceinline__ unsigned counter_tag(unsigned long long c) {
  return unsigned((c >> 32) % 0x7FFFFFFFull) + 1u;
}
// `c`: a value this thread read from the counter; the add waits for it, so a
// workgroup whose only reader is this thread may add right after its read.
__device__ __forceinline__ void counter_arrive(unsigned long long* ctr, unsigned long long c, int wg,
                                               int total) {
  const unsigned long long q = (1ull << 32) / unsigned(total);
  unsigned long long share = wg == 0 ? (1ull << 32) - q * unsigned(total - 1) : q;
  // c never reaches 2^64 - 1, so this changes nothing but makes the add wait
  // for the read's value: the read is performed first
  share ^= (unsigned long long)(c == ~0ull);
  __hip_atomic_fetch_add(ctr, share, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Arrival count (call from every thread at the end of a workgroup's part of
// the launch): true in thread 0 of the last of `total` workgroups to arrive,
// which also resets *done for the next launch.  A returning atomic: use it
// only where some workgroup must act after all the others.
__device__ __forceinline__ bool last_to_arrive(int* done, int total) {
  __syncthreads();
  if (threadIdx.x == 0 && add_dev(done, 1) == total - 1) {
    st_dev(done, 0);
    return true;
  }
  return false;
}

}  // namespace moe

// Hand-off of partial results between workgroups of one launch.
//
// A producer workgroup writes its payload with device-coherent (sc1) stores,
// which reach the level shared by all XCDs without a write-back of its own L2,
// waits for them, and then publishes a 64-bit tag of the launch with one
// device-scope store.  A consumer polls the tag with device-scope loads
// (sleeping between polls) and reads the payload with device-coherent loads,
// so that no stale line of its own L2 is used.  The tag identifies the launch
// (queue and packet), so a workspace needs no clearing between calls: what an
// earlier launch left in it never matches.  A consumer only waits for
// workgroups that were dispatched before it (lower workgroup ids), so every
// wait ends, whatever the number of workgroups resident at once.
#pragma once

#include "common.h"

namespace qlora {

__device__ uint64_t hsa_dispatch_id() __asm("llvm.amdgcn.dispatch.id");

// cache policy of a buffer load or store (gfx950): sc1, the device-coherent level
constexpr int kCoherent = 1 << 4;
// polls of one tag before a consumer gives up (and marks its outputs NaN)
constexpr int kSpinLimit = 1 << 22;

// splitmix64 finalizer (Steele, Lea and Flood, "Fast splittable pseudorandom
// number generators", 2014): a bijective 64-bit mix.
__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// Tag of this launch: unique per (queue, packet), identical in every workgroup.
__device__ __forceinline__ uint64_t launch_tag() {
    const uint64_t q = (uint64_t)reinterpret_cast<uintptr_t>(__builtin_amdgcn_queue_ptr());
    return mix64(hsa_dispatch_id() ^ mix64(q));
}

// Producer side, after every wave's payload stores were issued with kCoherent:
// once they have completed in every wave, thread 0 publishes the tag.  Each
// wave waits for its own stores (s_waitcnt with every count at 0) before the
// barrier.  A workgroup-scope fence would not wait (within one CU the waves
// need no such wait), so the tag could overtake the data; a device-scope
// release fence would wait too, but it also writes back the whole L2 of the
// XCD, which costs about a microsecond per workgroup and is not needed: every
// payload store already goes to the device-coherent level.
__device__ __forceinline__ void publish_tag(uint64_t* flag, uint64_t tag) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(flag, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Consumer side, one wave: lane p polls flags[p] for p < n (n may exceed 64).
// Returns true (in every lane) if some flag never showed the tag.  The payload
// loads that follow stay behind the polls.
__device__ __forceinline__ bool wait_tags(const uint64_t* flags, int n, uint64_t tag) {
    const int lane = threadIdx.x & 63;
    bool fail = false;
    for (int p = lane; p < n; p += 64) {
        int spins = 0;
        while (__hip_atomic_load(flags + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != tag) {
            if (++spins > kSpinLimit) {
                fail = true;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    return __builtin_amdgcn_ballot_w64(fail) != 0;
}

}  // namespace qlora

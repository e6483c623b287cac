// Blocks of one launch that hand data to each other.
//
// A block stores the data another block will read with agent-coherent
// stores (sc1), waits until they have completed (s_waitcnt vmcnt(0)), then
// stores its 64-bit flag word; a reader that has seen every flag it needs
// equal to the launch's token loads the data with agent-coherent loads. On
// this multi-XCD part an agent-scope release is compiled to a write-back of
// the XCD's L2 (buffer_wbl2) and an acquire to an invalidate, each paid by
// every block that executes it; the protocol needs neither. Flags are never
// cleared: the token is unique to the launch (launch_token), so a stale or
// uninitialised word cannot hold it. Waits are bounded (the caller says what
// happens when one gives up), so no launch can hang on a flag.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace md_sync {

// every vector-memory operation of this wave has completed
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <typename X>
__device__ __forceinline__ void put(X* p, X v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename X>
__device__ __forceinline__ X get(const X* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The calling block's flag: thread 0 stores the token once the block's data
// stores have completed (every thread waits for its own, then the barrier).
__device__ __forceinline__ void raise_flag(uint64_t* flag, uint64_t token) {
    wait_vm();
    __syncthreads();
    if (threadIdx.x == 0) put(flag, token);
}

// Every one of flags[0, n) holds the token (block-wide, NT threads; polled
// at most `limit` times).
template <int NT>
__device__ __forceinline__ bool all_flags(const uint64_t* __restrict__ flags, int n, uint64_t token, int limit) {
    for (int it = 0; it < limit; ++it) {
        int mine = 1;
        for (int b = threadIdx.x; b < n; b += NT) mine &= get(flags + b) == token;
        if (__syncthreads_and(mine)) return true;
        __builtin_amdgcn_s_sleep(8);
    }
    return false;
}

}  // namespace md_sync

// Hand-off of a state between two blocks of one launch (the "relay" that splits a work
// unit in time, part 1 continuing from part 0's final state).  Workgroups are dispatched
// in index order, so a waiting block's predecessor always has a smaller index and already
// holds a slot; the wait is bounded all the same.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mambascan {

// Bounded wait for a relay flag (one thread of the block).  Polls with relaxed
// device-scope loads (no cache invalidation per poll, which would disturb every other
// wave on the XCD) and long sleeps, then acquires once; gives up after 2^20 polls (a few
// seconds), so a missing hand-off can never hang the device.
__device__ __forceinline__ void relay_wait(uint32_t *flag)
{
    for (uint32_t i = 0; i < (1u << 20); ++i) {
        if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u)
            break;
        __builtin_amdgcn_s_sleep(127);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Publish the state every thread of the block has stored: release its stores at device
// scope, then one thread raises the flag.
__device__ __forceinline__ void relay_signal(uint32_t *flag)
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (threadIdx.x == 0)
        __hip_atomic_store(flag, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// The waiting side: thread 0 waits, the block joins it, and every thread acquires before
// reading the state.
__device__ __forceinline__ void relay_receive(uint32_t *flag)
{
    if (threadIdx.x == 0)
        relay_wait(flag);
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

} // namespace mambascan
